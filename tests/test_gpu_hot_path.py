"""GPU parity of the per-step path (forward compression and low-rank backward) against
the CPU oracle, with projections injected so the kernels are checked on their own.

Every call goes through the C ABI (ctypes binding of libinstant.so)."""
import zlib

import numpy as np
import pytest

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

FULL_CASES = [("tiny", "main"), ("bert_attn", "main"), ("bert_ffn", "up"), ("bert_ffn", "down"),
              ("effformer", "up"), ("effformer", "down")]


def _run(dtype, L, Cx, Cy, B, P, Q, x_io, gy_io, w_io, B_max=None):
    import rank_compressed_backprop_amd as rcb
    from gpu_util import empty, to_dev
    lay = rcb.InstantLayer(rcb.make_config(L, Cx, Cy, B_max or B, R_max=64, p=0, dtype=dtype))
    Rx, Ry = P.shape[0], Q.shape[0]
    lay.set_projections(torch.from_numpy(P.astype(np.float32)).cuda(), Rx,
                        torch.from_numpy(Q.astype(np.float32)).cuda(), Ry)
    x, gy, w = to_dev(x_io, dtype), to_dev(gy_io, dtype), to_dev(w_io, dtype)
    xhat = empty((B, Rx, Cx), dtype)
    gw = empty((Cy, Cx), dtype)
    gx = empty((B, L, Cx), dtype)
    lay.compress_fwd(x, B, xhat)
    lay.backward(xhat, gy, w, B, gw, gx)
    torch.cuda.synchronize()
    return lay, (x, gy, w, xhat, gw, gx)


def _oracle(P, Q, x64, gy64, w64):
    """The oracle's x_hat and backward under the installed (float32) projections, and the
    magnitudes of their terms (the scale of the per-element bound)."""
    from gpu_util import oracle_magnitudes
    P64 = P.astype(np.float32).astype(np.float64)
    Q64 = Q.astype(np.float32).astype(np.float64)
    xh = O.compress(P64, x64)
    return xh, O.backward(P64, Q64, xh, gy64, w64), oracle_magnitudes(O, P64, Q64, x64, gy64, w64)


@pytest.mark.parametrize("name,layer", FULL_CASES)
def test_hot_path_full_size(name, layer):
    from gpu_util import check_close, from_dev
    wl = W.get_workload(name)
    ly = wl.layer(layer)
    print(f"[hot path] {name}/{layer} B={wl.B} L={wl.L} Cx={ly.Cx} Cy={ly.Cy} {wl.dtype}", flush=True)
    c0 = W.make_layer_batch(wl, layer, 0)
    cal = O.calibrate([c0["x64"]], [c0["gy64"]], wl.eps, wl.p, O.COMP_PAPER)
    P, Q = cal["x"]["P"], cal["g"]["P"]
    d = W.make_layer_batch(wl, layer, wl.n_cal, with_w=True)
    _, (x, gy, w, xhat, gw, gx) = _run(wl.dtype, wl.L, ly.Cx, ly.Cy, wl.B, P, Q, d["x"], d["gy"], d["w"])
    xh_o, out, (xh_m, out_m) = _oracle(P, Q, d["x64"], d["gy64"], d["w64"])
    dt = wl.dtype
    msg = [check_close("xhat", from_dev(xhat, dt), xh_o, dt, xh_m),
           check_close("gw", from_dev(gw, dt), out["gw"], dt, out_m["gw"]),
           check_close("gx", from_dev(gx, dt), out["gx"], dt, out_m["gx"])]
    print("  rel err Frobenius/per-element: " + ", ".join(msg), flush=True)


# small shapes that still span several tiles and ragged tails in every dimension
RAGGED = [
    # dtype, B, L, Cx, Cy, Rx, Ry
    ("fp32", 3, 17, 24, 40, 1, 3),
    ("fp32", 2, 100, 136, 264, 13, 7),
    ("bf16", 1, 33, 8, 16, 2, 1),
    ("bf16", 5, 70, 264, 136, 17, 29),
    ("bf16", 3, 130, 392, 520, 64, 64),
    ("fp32", 2, 64, 64, 64, 64, 64),
    ("bf16", 7, 49, 448, 1792, 33, 31),
    # more g_w tiles than the compute units the g_x strips leave free (256 of them): some
    # blocks take two tiles, an odd count of them
    ("bf16", 40, 33, 264, 2952, 5, 9),
    # w (1544 x 11008, 34 MB) too large for L2: g_hat_x reads it once over K slices, with a
    # partial last column strip and a row count (3 * 23) that fills no whole tile
    ("bf16", 3, 70, 1544, 11008, 19, 23),
    # the same w with 7 * 23 = 161 rows of Q g_y (the middle row-group size of that kernel) and
    # a token count that leaves a partial last stage of P g_y
    ("bf16", 7, 40, 1544, 11008, 19, 23),
    # LDS-tiled g_w with K split in two slices (K = 960) and ragged M (1800) and N (1000)
    ("bf16", 32, 40, 1000, 1800, 30, 30),
    # LDS-tiled g_hat_x (270 tiles) with ragged M (40 * 29), N (3400) and a partial last stage
    # (K = 1032); LDS-tiled g_w unsplit with a ragged K (520)
    ("bf16", 40, 40, 3400, 1032, 13, 29),
    # fused g_x with two samples stacked per block (2 * Ry <= 16) and an odd batch: the last
    # group holds one sample
    ("bf16", 5, 64, 136, 264, 7, 7),
    ("fp32", 3, 40, 72, 48, 5, 8),
]


@pytest.mark.parametrize("case", RAGGED, ids=[f"{c[0]}-B{c[1]}-L{c[2]}-{c[3]}x{c[4]}-R{c[5]}.{c[6]}" for c in RAGGED])
def test_hot_path_ragged(case):
    from gpu_util import check_close, from_dev
    dtype, B, L, Cx, Cy, Rx, Ry = case
    print(f"[hot path ragged] {case}", flush=True)
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    P = rng.standard_normal((Rx, L)) / np.sqrt(L)
    Q = rng.standard_normal((Ry, L)) / np.sqrt(L)
    x = W.to_io(rng.standard_normal((B, L, Cx)), dtype)
    gy = W.to_io(rng.standard_normal((B, L, Cy)), dtype)
    w = W.to_io(0.05 * rng.standard_normal((Cy, Cx)), dtype)
    _, (_, _, _, xhat, gw, gx) = _run(dtype, L, Cx, Cy, B, P, Q, x, gy, w, B_max=B + 1)
    xh_o, out, (xh_m, out_m) = _oracle(P, Q, W.io_to_f64(x, dtype), W.io_to_f64(gy, dtype),
                                       W.io_to_f64(w, dtype))
    msg = [check_close("xhat", from_dev(xhat, dtype), xh_o, dtype, xh_m),
           check_close("gw", from_dev(gw, dtype), out["gw"], dtype, out_m["gw"]),
           check_close("gx", from_dev(gx, dtype), out["gx"], dtype, out_m["gx"])]
    print("  rel err Frobenius/per-element: " + ", ".join(msg), flush=True)


def test_backward_is_bitwise_deterministic():
    from gpu_util import empty
    wl = W.get_workload("bert_attn")
    ly = wl.layer(0)
    rng = np.random.default_rng(3)
    P = rng.standard_normal((8, wl.L)) / np.sqrt(wl.L)
    Q = rng.standard_normal((8, wl.L)) / np.sqrt(wl.L)
    d = W.make_layer_batch(wl, 0, 1, with_w=True)
    lay, (x, gy, w, xhat, gw, gx) = _run(wl.dtype, wl.L, ly.Cx, ly.Cy, wl.B, P, Q, d["x"], d["gy"], d["w"])
    gw2, gx2 = empty(gw.shape, wl.dtype), empty(gx.shape, wl.dtype)
    for _ in range(3):
        lay.backward(xhat, gy, w, wl.B, gw2, gx2)
        torch.cuda.synchronize()
        assert torch.equal(gw.view(torch.int16), gw2.view(torch.int16))
        assert torch.equal(gx.view(torch.int16), gx2.view(torch.int16))


def test_smaller_batch_than_bmax():
    from gpu_util import check_close, from_dev
    wl = W.get_workload("bert_attn")
    ly = wl.layer(0)
    rng = np.random.default_rng(4)
    P = rng.standard_normal((8, wl.L)) / np.sqrt(wl.L)
    Q = rng.standard_normal((10, wl.L)) / np.sqrt(wl.L)
    d = W.make_layer_batch(wl, 0, 2, with_w=True)
    B = 5
    _, (_, _, _, xhat, gw, gx) = _run(wl.dtype, wl.L, ly.Cx, ly.Cy, B, P, Q, d["x"][:B], d["gy"][:B], d["w"],
                                      B_max=wl.B)
    xh_o, out, (_, out_m) = _oracle(P, Q, d["x64"][:B], d["gy64"][:B], d["w64"])
    check_close("gw", from_dev(gw, wl.dtype), out["gw"], wl.dtype, out_m["gw"])
    check_close("gx", from_dev(gx, wl.dtype), out["gx"], wl.dtype, out_m["gx"])


def test_state_and_shape_errors():
    import rank_compressed_backprop_amd as rcb
    from gpu_util import empty
    lay = rcb.InstantLayer(rcb.make_config(64, 64, 64, 2, dtype="fp32"))
    x = empty((2, 64, 64), "fp32")
    xh = empty((2, 64, 64), "fp32")
    assert rcb.instant_compress_fwd(lay.h, x, 2, xh) == rcb.INSTANT_E_STATE
    assert rcb.instant_backward(lay.h, xh, x, x, 2, x, x) == rcb.INSTANT_E_STATE
    assert rcb.instant_compress_fwd(lay.h, x, 3, xh) == rcb.INSTANT_E_SHAPE
    P = torch.zeros((65, 64), device="cuda")
    assert rcb.instant_set_projections(lay.h, P, 65, P, 4) == rcb.INSTANT_E_SHAPE
    assert rcb.instant_set_projections(lay.h, P, 0, P, 4) == rcb.INSTANT_E_SHAPE
    assert rcb.instant_calibrate(lay.h, None, None, 0, 1) == rcb.INSTANT_E_STATE
