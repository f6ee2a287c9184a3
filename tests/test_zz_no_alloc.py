"""instant_backward_static (the entry point for callers that cannot allocate: its
intermediates live in a static device array of the library) against instant_backward, bit
for bit, on two calls in a row, the second with a smaller batch; and the size limit. Runs
both alone in a fresh process and after the other tests.

Notes "INSTANT: Compressing Gradients and Activations for Resource-Efficient Training",
关键设计 3 (the low-rank backward)."""
import zlib

import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [
    # dtype, B_max, smaller B, L, Cx, Cy, Rx, Ry
    ("bf16", 32, 5, 512, 768, 768, 8, 8),       # fused g_x + g_w tail
    ("bf16", 8, 3, 512, 768, 3072, 14, 14),     # g_w GEMM, g_hat_x GEMM, expansion
    ("bf16", 3, 2, 70, 1544, 11008, 19, 23),    # g_hat_x over K slices: float32 partials in the scratch
    ("fp32", 4, 1, 64, 64, 64, 10, 10),
]


def _bits(t, dtype):
    return t.view(torch.int16) if dtype == "bf16" else t.view(torch.int32)


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-B{c[1]}.{c[2]}-L{c[3]}-{c[4]}x{c[5]}" for c in CASES])
def test_static_scratch_backward_matches_workspace_backward(case):
    import rank_compressed_backprop_amd as rcb
    from gpu_util import empty, to_dev
    dtype, B_max, B2, L, Cx, Cy, Rx, Ry = case
    print(f"[no-alloc] {case}", flush=True)
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    lay = rcb.InstantLayer(rcb.make_config(L, Cx, Cy, B_max, R_max=64, p=0, dtype=dtype))
    P = torch.from_numpy((rng.standard_normal((Rx, L)) / np.sqrt(L)).astype(np.float32)).cuda()
    Q = torch.from_numpy((rng.standard_normal((Ry, L)) / np.sqrt(L)).astype(np.float32)).cuda()
    lay.set_projections(P, Rx, Q, Ry)
    w = to_dev(W.to_io(0.05 * rng.standard_normal((Cy, Cx)), dtype), dtype)
    for B in (B_max, B2):
        x = to_dev(W.to_io(rng.standard_normal((B, L, Cx)), dtype), dtype)
        gy = to_dev(W.to_io(rng.standard_normal((B, L, Cy)), dtype), dtype)
        xhat = empty((B, Rx, Cx), dtype)
        lay.compress_fwd(x, B, xhat)
        gw_r, gx_r = empty((Cy, Cx), dtype), empty((B, L, Cx), dtype)
        gw_s, gx_s = empty((Cy, Cx), dtype), empty((B, L, Cx), dtype)
        gw_s.fill_(3.0)
        gx_s.fill_(3.0)
        lay.backward(xhat, gy, w, B, gw_r, gx_r)
        s = rcb.instant_backward_static(lay.h, xhat, gy, w, B, gw_s, gx_s)
        assert s == rcb.INSTANT_OK, rcb.instant_status_str(s)
        torch.cuda.synchronize()
        assert torch.equal(_bits(gw_s, dtype), _bits(gw_r, dtype)), f"B={B}: g_w differs"
        assert torch.equal(_bits(gx_s, dtype), _bits(gx_r, dtype)), f"B={B}: g_x differs"
        print(f"  B={B}: g_w and g_x bit-identical to instant_backward", flush=True)


def test_static_scratch_size_limit():
    """A call whose intermediates exceed the static array is refused on the host."""
    import rank_compressed_backprop_amd as rcb
    from gpu_util import empty
    B, L, Cx, Cy, R = 64, 64, 64, 8192, 64
    # P g_y and Q g_y alone: 2 * 64 * 64 * 8192 * 2 bytes = 128 MiB > 64 MiB
    assert 2 * B * R * Cy * 2 > rcb.INSTANT_STATIC_SCRATCH_BYTES
    lay = rcb.InstantLayer(rcb.make_config(L, Cx, Cy, B, R_max=64, p=0, dtype="bf16"))
    P = torch.eye(L, device="cuda")[:R].contiguous()
    lay.set_projections(P, R, P, R)
    xhat, gy, w = empty((B, R, Cx), "bf16"), empty((B, L, Cy), "bf16"), empty((Cy, Cx), "bf16")
    gw, gx = empty((Cy, Cx), "bf16"), empty((B, L, Cx), "bf16")
    assert rcb.instant_backward_static(lay.h, xhat, gy, w, B, gw, gx) == rcb.INSTANT_E_SHAPE
    # the same layer within the limit at a smaller batch (16 * 64 * 8192 * 2 * 2 = 32 MiB)
    assert rcb.instant_backward_static(lay.h, xhat, gy, w, 16, gw, gx) == rcb.INSTANT_OK
    torch.cuda.synchronize()
