"""Run-to-run determinism of the paths whose float32 partial sums are folded across blocks or
launches (split-K slices of g_hat_x added by the expansion, K slices of the LDS-tiled g_w, the
statistics' slices in 128 x 128 and 256 x 128 blocks): every fold adds in a fixed order, so two
calls on the same inputs give the same bits. The values themselves are checked against the
oracle in the parity tests."""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


# dtype, B, L, Cx, Cy, Rx, Ry: the read-w-once g_hat_x whose slices the expansion adds
# (w 34 MB), and the EfficientFormer-shaped path with the K-split LDS-tiled g_w
CASES = [("bf16", 3, 70, 1544, 11008, 19, 23), ("bf16", 64, 49, 448, 1792, 29, 29)]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[1]}-L{c[2]}-{c[3]}x{c[4]}" for c in CASES])
def test_backward_is_bitwise_repeatable(case):
    import rank_compressed_backprop_amd as rcb
    from gpu_util import empty, to_dev
    dtype, B, L, Cx, Cy, Rx, Ry = case
    print(f"[determinism] backward {case}", flush=True)
    rng = np.random.default_rng(41)
    lay = rcb.InstantLayer(rcb.make_config(L, Cx, Cy, B, R_max=64, p=0, dtype=dtype))
    P = torch.from_numpy((rng.standard_normal((Rx, L)) / np.sqrt(L)).astype(np.float32)).cuda()
    Q = torch.from_numpy((rng.standard_normal((Ry, L)) / np.sqrt(L)).astype(np.float32)).cuda()
    lay.set_projections(P, Rx, Q, Ry)
    w = to_dev(W.to_io(0.05 * rng.standard_normal((Cy, Cx)), dtype), dtype)
    x = to_dev(W.to_io(rng.standard_normal((B, L, Cx)), dtype), dtype)
    gy = to_dev(W.to_io(rng.standard_normal((B, L, Cy)), dtype), dtype)
    xhat = empty((B, Rx, Cx), dtype)
    lay.compress_fwd(x, B, xhat)
    outs = []
    for _ in range(2):
        gw, gx = empty((Cy, Cx), dtype), empty((B, L, Cx), dtype)
        lay.backward(xhat, gy, w, B, gw, gx)
        outs.append((gw, gx))
    torch.cuda.synchronize()
    assert torch.equal(_bits(outs[0][0]), _bits(outs[1][0])), "g_w differs between two calls"
    assert torch.equal(_bits(outs[0][1]), _bits(outs[1][1])), "g_x differs between two calls"


@pytest.mark.parametrize("L", [512, 2000])
def test_statistics_are_bitwise_repeatable(L):
    """Two layers accumulating the same batches hold the same float64 sums, bit for bit
    (L = 512: 128 x 128 blocks, 24 slices a side; L = 2000: 256 x 128 blocks)."""
    import rank_compressed_backprop_amd as rcb
    from gpu_util import to_dev
    B, Cx, Cy = (32, 768, 768) if L == 512 else (3, 136, 264)
    print(f"[determinism] statistics L={L} B={B} C={Cx}/{Cy}", flush=True)
    rng = np.random.default_rng(43)
    batches = [(to_dev(W.to_io(rng.standard_normal((B, L, Cx)), "bf16"), "bf16"),
                to_dev(W.to_io(rng.standard_normal((B, L, Cy)), "bf16"), "bf16")) for _ in range(2)]
    stats = []
    for _ in range(2):
        lay = rcb.InstantLayer(rcb.make_config(L, Cx, Cy, B, R_max=64, p=0, eps=0.9, dtype="bf16"))
        for x, gy in batches:
            assert lay.calibrate(x, gy, B, finalize=False) == rcb.INSTANT_OK
        CX = torch.empty((L, L), dtype=torch.float64, device="cuda")
        CG = torch.empty((L, L), dtype=torch.float64, device="cuda")
        lay.get_statistics(CX, CG)
        torch.cuda.synchronize()
        stats.append((CX, CG))
        del lay
    assert torch.equal(stats[0][0].view(torch.int64), stats[1][0].view(torch.int64)), "C_X differs"
    assert torch.equal(stats[0][1].view(torch.int64), stats[1][1].view(torch.int64)), "C_G differs"
