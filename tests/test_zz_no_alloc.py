"""mtp_verify_noalloc (the verify entry point that uses the library's static
scratch instead of a caller workspace) against mtp_verify on the same
inputs: accepted length, token, status and margin identical, on two calls in
a row whose second is smaller (the scratch keeps the first call's contents),
and a request larger than the scratch refused on the host with outputs
untouched."""
import pytest
import torch

from deepseek_sequential_mtp_amd import _lib

pytestmark = pytest.mark.gpu


def _inputs(R, G, V, dtype, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    zt = (2.0 * torch.randn((R, G + 1, V), generator=g, device="cuda")).to(dtype)
    zd = (zt[:, :G].float() + 0.5 * torch.randn((R, G, V), generator=g, device="cuda")).to(dtype)
    # draft tokens: the draft's argmax or a random id, so that both
    # acceptances and rejections occur
    y = torch.where(torch.rand((R, G), generator=g, device="cuda") < 0.7, zd.float().argmax(-1),
                    torch.randint(0, V, (R, G), generator=g, device="cuda")).to(torch.int32)
    ua = torch.rand((R, G), generator=g, device="cuda")
    us = torch.rand((R, G + 1), generator=g, device="cuda")
    return zt.contiguous(), zd.contiguous(), y.contiguous(), ua, us


def _outs(R):
    return dict(accepted_len=torch.full((R,), -7, dtype=torch.int32, device="cuda"),
                next_token=torch.full((R,), -7, dtype=torch.int32, device="cuda"),
                status=torch.full((R,), -7, dtype=torch.int32, device="cuda"),
                margin=torch.full((R,), -7.0, dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_verify_on_two_calls(dtype):
    for (R, G, V, seed) in ((256, 4, 129280, 1), (40, 2, 1000, 2)):
        print(f"[noalloc] {dtype} R={R} gamma={G} V={V}", flush=True)
        zt, zd, y, ua, us = _inputs(R, G, V, dtype, seed)
        ref = _lib.verify(zt, zd, y, ua, us)
        got = _lib.verify_noalloc(zt, zd, y, ua, us, out=_outs(R))
        torch.cuda.synchronize()
        for k in ("accepted_len", "next_token", "status", "margin"):
            assert torch.equal(got[k], ref[k]), k
        A = got["accepted_len"]
        assert (got["status"] == 0).all()
        assert ((A >= 0) & (A <= G)).all() and (A < G).any() and (A > 0).any()


def test_noalloc_refuses_a_request_beyond_the_scratch():
    R, G, V = 600, 4, 129280        # needs about 78 MB of scratch, more than the 64 MiB held
    zt = torch.zeros((R, G + 1, V), dtype=torch.bfloat16, device="cuda")
    zd = torch.zeros((R, G, V), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((R, G), dtype=torch.int32, device="cuda")
    ua = torch.zeros((R, G), device="cuda")
    us = torch.zeros((R, G + 1), device="cuda")
    out = _outs(R)
    with pytest.raises(_lib.MtpError) as e:
        _lib.verify_noalloc(zt, zd, y, ua, us, out=out)
    assert e.value.status == -9
    torch.cuda.synchronize()
    assert (out["accepted_len"] == -7).all() and (out["status"] == -7).all()
