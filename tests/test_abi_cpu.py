"""The C-ABI library loads, exports every symbol include/mtp.h declares, and
rejects invalid arguments on the host (no GPU needed: these paths return
before any launch)."""
import ctypes as C
import os
import re

import pytest

from deepseek_sequential_mtp_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mtp.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mtp_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libmtp.so not built (run __graft_entry__.build())")
    return _lib.load()


def test_header_declares_the_three_entry_points():
    decl = _declared_functions()
    for name in ("mtp_chain_forward", "mtp_head_ce_fwd_bwd", "mtp_verify"):
        assert name in decl
    assert set(decl) == set(_lib.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.mtp_abi_version() == 2
    assert lib.mtp_strerror(0) == b"ok"
    assert lib.mtp_strerror(-3) == b"depth must be positive"


def _chain_args(**kw):
    a = _lib.ChainArgs()
    a.B, a.T, a.d, a.n_heads, a.head_dim, a.ffn, a.V, a.D = 2, 16, 64, 4, 16, 172, 512, 1
    a.dtype, a.eps, a.rope_theta = _lib.MTP_F32, 1e-6, 1e4
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_chain_host_errors(lib):
    run = lambda a: lib.mtp_chain_forward(C.byref(a), None)
    assert lib.mtp_chain_forward(None, None) == -1                   # MTP_ERR_NULL
    assert run(_chain_args(D=0)) == -3                               # depth must be positive
    assert run(_chain_args(dtype=7)) == -4
    assert run(_chain_args(d=0)) == -2
    assert run(_chain_args(d=66)) == -2                              # not a chunk multiple
    assert run(_chain_args(head_dim=15)) == -2
    assert run(_chain_args(head_dim=48)) == -8                       # unsupported head width
    assert run(_chain_args(dtype=_lib.MTP_BF16, ffn=176, head_dim=16)) == -8
    assert run(_chain_args(dtype=_lib.MTP_BF16)) == -2                # ffn 172 not a multiple of 8
    assert run(_chain_args(eps=-1.0)) == -6
    assert run(_chain_args()) == -1                                  # pointers missing
    assert lib.mtp_chain_workspace_size(C.byref(_chain_args(D=0))) == 0
    ws = lib.mtp_chain_workspace_size(C.byref(_chain_args()))
    assert ws > 0
    # workspace grows with the sizes
    assert lib.mtp_chain_workspace_size(C.byref(_chain_args(T=32))) > ws


def test_ce_host_errors(lib):
    def args(**kw):
        a = _lib.CeArgs()
        a.B, a.T, a.d, a.V, a.D = 2, 16, 64, 512, 1
        a.dtype, a.eps, a.lambda_, a.reduce, a.denom = _lib.MTP_F32, 1e-6, 0.1, 0, 0.0
        for k, v in kw.items():
            setattr(a, k, v)
        return a
    run = lambda a: lib.mtp_head_ce_fwd_bwd(C.byref(a), None)
    assert run(args(D=0)) == -3
    assert run(args(reduce=5)) == -6
    assert run(args(denom=-1.0)) == -6
    assert run(args(V=510)) == -2
    assert run(args(V=1 << 21)) == -2       # a 256-row logit tile must span < 2 GiB
    assert run(args(V=(1 << 21) - 4)) == -1  # shape accepted; fails on the null pointers
    assert run(args()) == -1
    assert lib.mtp_ce_workspace_size(C.byref(args())) > 0


def test_verify_host_errors(lib):
    def args(**kw):
        a = _lib.VerifyArgs()
        a.R, a.gamma, a.V, a.temperature, a.logits_dtype = 4, 2, 100, 1.0, _lib.MTP_BF16
        for k, v in kw.items():
            setattr(a, k, v)
        return a
    run = lambda a: lib.mtp_verify(C.byref(a), None)
    assert run(args(gamma=0)) == -2
    assert run(args(temperature=0.0)) == -6
    assert run(args(logits_dtype=3)) == -4
    assert run(args()) == -1
    # row log-sum-exps (2 doubles per row), 16-byte test outcomes, one
    # double per chunk of emission weights (chunks of 8 bf16 logits when V
    # is a multiple of 8, single logits otherwise) and per tile of 256 chunks
    assert lib.mtp_verify_workspace_size(C.byref(args())) == 4 * 5 * 2 * 8 + 4 * 16 + 4 * (100 + 1) * 8
    assert lib.mtp_verify_workspace_size(C.byref(args(V=128))) == 4 * 5 * 2 * 8 + 4 * 16 + 4 * (16 + 1) * 8
