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


def _header_abi_version():
    m = re.search(r"#define\s+MTP_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert m, "MTP_ABI_VERSION missing from the header"
    return int(m.group(1))


def test_header_declares_the_entry_points():
    decl = _declared_functions()
    for name in ("mtp_chain_forward", "mtp_head_ce_fwd_bwd", "mtp_verify", "mtp_propose_step",
                 "mtp_round_commit"):
        assert name in decl
    assert set(decl) == set(_lib.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.mtp_abi_version() == _lib.ABI_VERSION == _header_abi_version()
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
    # one batch row's [q | k | v] must span < 2 GiB: 65536 x 3 x 16384 bf16 does not,
    # 32768 x 3 x 8192 x 2 bytes (1.5 GiB) does
    big = dict(dtype=_lib.MTP_BF16, d=1024, ffn=2816, n_heads=128, head_dim=128, B=1)
    assert run(_chain_args(T=65536, **big)) == -8
    assert run(_chain_args(T=32768, **dict(big, n_heads=64))) == -1
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
    # top-1 accuracy adds the slab's row maxima, one argmax per row and a hit
    # count per depth (32 + 32 + 1 four-byte values here, plus alignment)
    base = lib.mtp_ce_workspace_size(C.byref(args()))
    for name in ("pred", "correct", "accuracy"):
        a = args()
        setattr(a, name, 0x7f0000000000)
        extra = lib.mtp_ce_workspace_size(C.byref(a)) - base
        assert 65 * 4 <= extra <= 65 * 4 + 3 * 256, (name, extra)


def test_verify_host_errors(lib):
    def args(**kw):
        a = _lib.VerifyArgs()
        a.R, a.gamma, a.V, a.temperature, a.logits_dtype = 4, 2, 100, 1.0, _lib.MTP_BF16
        for k, v in kw.items():
            setattr(a, k, v)
        return a
    run = lambda a: lib.mtp_verify(C.byref(a), None)
    assert run(args(gamma=0)) == -2
    assert run(args(R=65536)) == -8        # more requests than one grid dimension holds
    assert run(args(R=65535)) == -1        # accepted; fails on the null pointers
    assert run(args(temperature=0.0)) == -6
    assert run(args(logits_dtype=3)) == -4
    assert run(args()) == -1
    # row log-sum-exps (2 doubles per row), 16-byte test outcomes, one
    # double per chunk of emission weights (chunks of 8 bf16 logits when V
    # is a multiple of 8, single logits otherwise) and per tile of 256 chunks
    assert lib.mtp_verify_workspace_size(C.byref(args())) == 4 * 5 * 2 * 8 + 4 * 16 + 4 * (100 + 1) * 8
    assert lib.mtp_verify_workspace_size(C.byref(args(V=128))) == 4 * 5 * 2 * 8 + 4 * 16 + 4 * (16 + 1) * 8


def test_propose_host_errors(lib):
    def args(**kw):
        a = _lib.ProposeArgs()
        a.R, a.L_max, a.d, a.n_heads, a.head_dim, a.ffn, a.V = 4, 32, 64, 4, 16, 172, 512
        a.dtype, a.eps, a.rope_theta, a.temperature = _lib.MTP_F32, 1e-6, 1e4, 1.0
        for k, v in kw.items():
            setattr(a, k, v)
        return a
    run = lambda a: lib.mtp_propose_step(C.byref(a), None)
    assert lib.mtp_propose_step(None, None) == -1
    assert run(args(dtype=5)) == -4
    assert run(args(R=0)) == -2
    assert run(args(L_max=0)) == -2
    assert run(args(L_max=(1 << 20) + 1)) == -2
    assert run(args(V=510)) == -2
    assert run(args(head_dim=48)) == -8
    assert run(args(R=65536)) == -8
    assert run(args(temperature=0.0)) == -6
    assert run(args(temperature=float("inf"))) == -6
    assert run(args()) == -1                      # pointers missing
    ws = lib.mtp_propose_workspace_size(C.byref(args()))
    assert ws > 0 and lib.mtp_propose_workspace_size(C.byref(args(R=8))) > ws
    assert lib.mtp_propose_workspace_size(C.byref(args(R=0))) == 0


def test_round_commit_host_errors(lib):
    run = lambda a: lib.mtp_round_commit(C.byref(a), None)
    assert lib.mtp_round_commit(None, None) == -1
    a = _lib.RoundArgs()
    a.R, a.gamma, a.eos = 4, 0, -1
    assert run(a) == -2
    a.gamma, a.R = 4, 0
    assert run(a) == -2
    a.R = 4
    assert run(a) == -1                          # pointers missing
    fake = 0x7f0000001000
    names = ("draft_tokens", "accepted_len", "next_token", "status", "remaining", "new_tokens", "n_new",
             "rows_to_keep", "pending_frontier", "stopped")
    for i, n in enumerate(names):
        setattr(a, n, fake + 0x1000 * i)
    a.stopped = fake + 0x1000 * 9 + 4            # misaligned: rejected before any launch
    assert run(a) == -6


def test_misaligned_pointers_are_rejected_before_any_launch(lib):
    """Device pointers must be 16-byte aligned; the checks run on the host and
    return before anything is launched (the fake addresses are never used:
    with no workspace the call stops at MTP_ERR_WORKSPACE)."""
    fake = 0x7f0000001000
    names = ("target_logits", "draft_logits", "draft_tokens", "u_accept", "u_sample", "accepted_len",
             "next_token", "status")

    def vargs(bad=None, off=8):
        a = _lib.VerifyArgs()
        a.R, a.gamma, a.V, a.temperature, a.logits_dtype = 4, 2, 128, 1.0, _lib.MTP_BF16
        for i, n in enumerate(names):
            setattr(a, n, fake + 0x10000 * i + (off if n == bad else 0))
        return a
    run = lambda a: lib.mtp_verify(C.byref(a), None)
    assert run(vargs()) == -5                    # aligned: stops at the missing workspace
    for n in names:
        assert run(vargs(n)) == -6, n
    a = vargs()
    a.margin = fake + 4                          # optional output, still checked
    assert run(a) == -6

    D = 2
    hs = (C.c_void_p * D)(fake, fake + 0x100000)
    dhs = (C.c_void_p * D)(fake + 0x200000, fake + 0x300000)
    ce_names = ("labels", "W_out", "g_out", "loss_sum", "counts", "loss", "loss_mtp", "dW_out", "dg_out",
                "pred", "correct", "accuracy")

    def cargs(bad=None):
        a = _lib.CeArgs()
        a.B, a.T, a.d, a.V, a.D = 2, 16, 64, 512, D
        a.dtype, a.eps, a.lambda_, a.reduce, a.denom = _lib.MTP_BF16, 1e-6, 0.1, 0, 0.0
        a.h = C.cast(hs, C.POINTER(C.c_void_p))
        a.dh = C.cast(dhs, C.POINTER(C.c_void_p))
        for i, n in enumerate(ce_names):
            setattr(a, n, fake + 0x400000 + 0x10000 * i + (2 if n == bad else 0))
        return a
    runc = lambda a: lib.mtp_head_ce_fwd_bwd(C.byref(a), None)
    assert runc(cargs()) == -5
    for n in ce_names:
        assert runc(cargs(n)) == -6, n
    hs[1] = fake + 0x100000 + 4
    assert runc(cargs()) == -6


def _c_name(field):
    return "lambda" if field == "lambda_" else field


@pytest.mark.skipif(__import__("shutil").which("gcc") is None, reason="gcc not available")
def test_ctypes_struct_layouts_match_the_header(tmp_path):
    """Every ctypes mirror of an argument struct has the header's field
    offsets and size: a C program compiled against include/mtp.h prints
    offsetof/sizeof for each field the binding declares."""
    structs = {name: cls for name, cls in vars(_lib).items()
               if isinstance(cls, type) and issubclass(cls, C.Structure) and cls is not C.Structure}
    c_types = {"DepthWeights": "mtp_depth_weights", "ChainArgs": "mtp_chain_args", "CeArgs": "mtp_ce_args",
               "VerifyArgs": "mtp_verify_args", "ProposeArgs": "mtp_propose_args",
               "RoundArgs": "mtp_round_args"}
    for name in structs:
        assert name in c_types or name in getattr(_lib, "C_STRUCT_NAMES", {}), f"unmapped struct {name}"
    c_types.update(getattr(_lib, "C_STRUCT_NAMES", {}))
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void) {"]
    for name, cls in structs.items():
        ct = c_types[name]
        lines.append(f'  printf("{name} sizeof %zu\\n", sizeof({ct}));')
        for f, _ in cls._fields_:
            lines.append(f'  printf("{name} {f} %zu\\n", offsetof({ct}, {_c_name(f)}));')
        # the header has no field the binding lacks: the last field ends the struct
    lines.append("  return 0;\n}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    import subprocess
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-o", str(exe), str(src)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {}
    for line in out:
        if line:
            s, f, v = line.split()
            got[(s, f)] = int(v)
    for name, cls in structs.items():
        assert got[(name, "sizeof")] == C.sizeof(cls), name
        for f, _ in cls._fields_:
            assert got[(name, f)] == getattr(cls, f).offset, (name, f)


def test_verify_noalloc_refuses_beyond_its_scratch_on_the_host(lib):
    # a request needing more than the static scratch returns MTP_ERR_TOO_LARGE
    # before any launch (the pointers are never dereferenced)
    fake = C.c_void_p(1 << 20)
    a = _lib.VerifyArgs(600, 4, 129280, 1.0, _lib.MTP_BF16, fake, fake, fake, fake, fake, fake, fake, fake,
                        None, None, 0)
    assert lib.mtp_verify_workspace_size(C.byref(a)) > (64 << 20)
    assert lib.mtp_verify_noalloc(C.byref(a), None) == -9
    assert lib.mtp_verify_noalloc(None, None) == -1
    a.R = 0
    assert lib.mtp_verify_noalloc(C.byref(a), None) == -2


FAKE = 0x7f0000000000          # 16-byte aligned, never dereferenced: these calls return before any launch


def _bwd_args(**kw):
    a = _lib.ChainBwdArgs()
    a.B, a.T, a.d, a.n_heads, a.head_dim, a.ffn, a.V, a.D = 2, 64, 256, 2, 128, 688, 1000, 2
    a.dtype, a.eps, a.rope_theta = _lib.MTP_BF16, 1e-6, 1e4
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _fill_bwd_pointers(a, D):
    w = (_lib.DepthWeights * D)()
    g = (_lib.DepthGrads * D)()
    for k in range(D):
        for name, _ in _lib.DepthWeights._fields_:
            setattr(w[k], name, FAKE)
        for name, _ in _lib.DepthGrads._fields_:
            setattr(g[k], name, FAKE)
    h = (C.c_void_p * D)(*([FAKE] * D))
    dh = (C.c_void_p * D)(*([FAKE] * D))
    for name in ("tokens", "segment_ids", "h0", "embed", "dh0", "dE"):
        setattr(a, name, FAKE)
    a.w, a.dw, a.h, a.dh = w, g, h, dh
    return (w, g, h, dh)                    # keep the arrays alive


def test_chain_backward_host_errors(lib):
    run = lambda a: lib.mtp_chain_backward(C.byref(a), None)
    assert lib.mtp_chain_backward(None, None) == -1
    assert run(_bwd_args(D=0)) == -3
    assert run(_bwd_args(dtype=_lib.MTP_F32, ffn=172, d=64, head_dim=16, n_heads=4)) == -8   # bf16 only
    assert run(_bwd_args(head_dim=32, n_heads=8)) == -8                                     # head width 64 or 128
    assert run(_bwd_args(d=8200, ffn=688)) == -8                                            # rows up to 8192
    assert run(_bwd_args(eps=-1.0)) == -6
    assert run(_bwd_args()) == -1                                                           # pointers missing
    a = _bwd_args()
    keep = _fill_bwd_pointers(a, a.D)
    a.dh[0] = None                                # the head's gradient of depth 1 is required
    assert run(a) == -1
    a.dh[0] = FAKE
    a.w[1].Wo = FAKE + 8                          # misaligned weight
    assert run(a) == -6
    a.w[1].Wo = FAKE
    need = lib.mtp_chain_backward_workspace_size(C.byref(a))
    assert need > 0
    a.workspace, a.workspace_bytes = FAKE, need - 1
    assert run(a) == -5                           # workspace too small
    a.workspace = None
    assert run(a) == -5
    del keep
    # the workspace grows with the rows and does not depend on the pointers
    assert lib.mtp_chain_backward_workspace_size(C.byref(_bwd_args(T=128))) > need
    assert lib.mtp_chain_backward_workspace_size(C.byref(_bwd_args(D=0))) == 0


def test_horizon_heads_host_errors(lib):
    def args(**kw):
        a = _lib.HorizonArgs()
        a.B, a.T, a.d, a.n_heads, a.head_dim, a.ffn, a.V, a.K = 2, 64, 256, 2, 128, 688, 1000, 2
        a.dtype, a.eps, a.rope_theta, a.lambda_ = _lib.MTP_BF16, 1e-6, 1e4, 0.1
        for k, v in kw.items():
            setattr(a, k, v)
        return a
    run = lambda a: lib.mtp_horizon_heads(C.byref(a), None)
    assert lib.mtp_horizon_heads(None, None) == -1
    assert run(args(K=0)) == -3
    assert run(args(V=1004)) == -2                       # V a multiple of 8
    assert run(args(head_dim=32, n_heads=8)) == -8
    assert run(args(lambda_=float("nan"))) == -6
    assert run(args()) == -1
    a = args()
    w = (_lib.BlockWeights * 2)()
    g = (_lib.BlockGrads * 2)()
    for k in range(2):
        for name, _ in _lib.BlockWeights._fields_:
            setattr(w[k], name, FAKE)
        for name, _ in _lib.BlockGrads._fields_:
            setattr(g[k], name, FAKE)
    for name in ("tokens", "segment_ids", "h", "W_out", "g_out", "loss", "counts", "loss_total", "dh", "dW_out",
                 "dg_out"):
        setattr(a, name, FAKE)
    a.w, a.dw = w, g
    a.dw[1].Wgate = None
    assert run(a) == -1
    a.dw[1].Wgate = FAKE + 4
    assert run(a) == -6
    a.dw[1].Wgate = FAKE
    need = lib.mtp_horizon_heads_workspace_size(C.byref(a))
    assert need > 0
    a.workspace, a.workspace_bytes = FAKE, need - 1
    assert run(a) == -5


def test_saved_activation_sizes_and_errors(lib):
    a = _chain_args(dtype=_lib.MTP_BF16, d=256, ffn=688, n_heads=2, head_dim=128, V=1000, T=64, D=2)
    per = lib.mtp_chain_saved_bytes(C.byref(a)) // 2
    N, d, A, H, f = 2 * 64, 256, 256, 2, 688
    # c, u, x_a, q|k|v, o, (lse2, D) pairs, a, y, gate|up (f32): each region 256-byte aligned
    exact = N * (2 * d * 2 + d * 4 + d * 2 + 3 * A * 2 + A * 2 + H * 8 + d * 4 + d * 2 + 2 * f * 4)
    assert exact <= per < exact + 9 * 256
    assert lib.mtp_chain_saved_bytes(C.byref(_chain_args())) == 0            # f32: no saving
    assert lib.mtp_chain_saved_bytes(C.byref(_chain_args(D=0))) == 0
    # forward: every pointer set (never dereferenced), workspace large enough
    ws = lib.mtp_chain_workspace_size(C.byref(a))
    w = (_lib.DepthWeights * 2)()
    for k in range(2):
        for name, _ in _lib.DepthWeights._fields_:
            setattr(w[k], name, FAKE)
    hout = (C.c_void_p * 2)(FAKE, FAKE)
    for name in ("tokens", "segment_ids", "h0", "embed", "state_mask", "loss_mask", "labels", "counts",
                 "device_error"):
        setattr(a, name, FAKE)
    a.w, a.h_out, a.workspace, a.workspace_bytes = w, hout, FAKE, ws
    run = lambda x: lib.mtp_chain_forward(C.byref(x), None)
    a.saved, a.saved_bytes = FAKE, 2 * per - 1
    assert run(a) == -5                                                      # saved buffer too small
    a.saved, a.saved_bytes = FAKE + 8, 2 * per
    assert run(a) == -6                                                      # misaligned
    f = _chain_args()
    for name in ("tokens", "segment_ids", "h0", "embed", "state_mask", "loss_mask", "labels", "counts",
                 "device_error"):
        setattr(f, name, FAKE)
    wf = (_lib.DepthWeights * 1)()
    for name, _ in _lib.DepthWeights._fields_:
        setattr(wf[0], name, FAKE)
    hf = (C.c_void_p * 1)(FAKE)
    f.w, f.h_out, f.workspace = wf, hf, FAKE
    f.workspace_bytes = lib.mtp_chain_workspace_size(C.byref(f))
    f.saved, f.saved_bytes = FAKE, 1 << 30
    assert run(f) == -8                                                      # f32 chain keeps nothing
    # backward: a saved buffer smaller than the forward's is refused
    b = _bwd_args()
    keep = _fill_bwd_pointers(b, b.D)
    b.workspace, b.workspace_bytes = FAKE, lib.mtp_chain_backward_workspace_size(C.byref(b))
    b.saved, b.saved_bytes = FAKE, 1024
    assert lib.mtp_chain_backward(C.byref(b), None) == -5
    b.saved = FAKE + 4
    assert lib.mtp_chain_backward(C.byref(b), None) == -6
    del keep
