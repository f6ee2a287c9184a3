"""instant_backward captured into a HIP graph (how bench.py times it): every replay must
reproduce the eager call bit for bit, with the program's own eager work and
synchronisations between the replays. Covers the fused g_x path (w resident in L2), the
unfused path (GEMM + expansion) and the path that reads a large w once over K slices.

Notes "INSTANT: Compressing Gradients and Activations for Resource-Efficient Training",
关键设计 3 (the low-rank backward)."""
import zlib

import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [
    # dtype, B, L, Cx, Cy, Rx, Ry
    ("bf16", 8, 512, 768, 768, 8, 8),       # fused g_x + g_w tail
    ("bf16", 4, 512, 768, 3072, 14, 14),    # g_w GEMM, g_hat_x GEMM, expansion
    ("bf16", 3, 70, 1544, 11008, 19, 23),   # g_hat_x over K slices with a second reduction launch
    ("fp32", 2, 64, 64, 64, 10, 10),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-B{c[1]}-L{c[2]}-{c[3]}x{c[4]}" for c in CASES])
def test_graph_replays_match_eager(case):
    import rank_compressed_backprop_amd as rcb
    from gpu_util import empty, to_dev
    dtype, B, L, Cx, Cy, Rx, Ry = case
    print(f"[graph] {case}", flush=True)
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    lay = rcb.InstantLayer(rcb.make_config(L, Cx, Cy, B, R_max=64, p=0, dtype=dtype))
    P = torch.from_numpy((rng.standard_normal((Rx, L)) / np.sqrt(L)).astype(np.float32)).cuda()
    Q = torch.from_numpy((rng.standard_normal((Ry, L)) / np.sqrt(L)).astype(np.float32)).cuda()
    lay.set_projections(P, Rx, Q, Ry)
    x = to_dev(W.to_io(rng.standard_normal((B, L, Cx)), dtype), dtype)
    gy = to_dev(W.to_io(rng.standard_normal((B, L, Cy)), dtype), dtype)
    w = to_dev(W.to_io(0.05 * rng.standard_normal((Cy, Cx)), dtype), dtype)
    xhat = empty((B, Rx, Cx), dtype)
    lay.compress_fwd(x, B, xhat)
    gw_e, gx_e = empty((Cy, Cx), dtype), empty((B, L, Cx), dtype)
    lay.backward(xhat, gy, w, B, gw_e, gx_e)
    torch.cuda.synchronize()

    gw_g, gx_g = empty((Cy, Cx), dtype), empty((B, L, Cx), dtype)
    gw_o, gx_o = empty((Cy, Cx), dtype), empty((B, L, Cx), dtype)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        rcb.instant_backward(lay.h, xhat, gy, w, B, gw_g, gx_g)
    torch.cuda.synchronize()

    def bits(t):
        return t.view(torch.int16) if dtype == "bf16" else t.view(torch.int32)

    for r in range(4):
        gw_g.fill_(7.0)  # stale values a replay must overwrite
        gx_g.fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(gw_g), bits(gw_e)), f"replay {r}: g_w differs"
        assert torch.equal(bits(gx_g), bits(gx_e)), f"replay {r}: g_x differs"
        # eager work on the same handle between replays (other outputs, same workspace)
        lay.backward(xhat, gy, w, B, gw_o, gx_o)
        torch.cuda.synchronize()
        assert torch.equal(bits(gx_o), bits(gx_e))
    print(f"[graph] {case}: 4 replays bit-identical to the eager call", flush=True)
    del g
