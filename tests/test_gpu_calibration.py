"""GPU parity of the calibration (statistics, Jacobi eigen-decomposition, truncation,
compensation) and of the end-to-end path against the CPU oracle, through the C ABI."""
import numpy as np
import pytest

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

COMP = {"paper": O.COMP_PAPER, "none": O.COMP_NONE, "ratio": O.COMP_RATIO}


def _calibrate_both(wl, layer, comp="paper", R_max=64, n_cal=None, max_sweeps=30):
    import rank_compressed_backprop_amd as rcb
    from gpu_util import to_dev
    ly = wl.layer(layer)
    n_cal = n_cal or wl.n_cal
    lay = rcb.InstantLayer(rcb.make_config(wl.L, ly.Cx, ly.Cy, wl.B, R_max=R_max, p=wl.p, eps=wl.eps,
                                           dtype=wl.dtype, comp=comp, max_sweeps=max_sweeps))
    xa, ga = O.Accumulator(wl.L), O.Accumulator(wl.L)
    for t in range(n_cal):
        d = W.make_layer_batch(wl, layer, t)
        xa.add(d["x64"])
        ga.add(d["gy64"])
        assert lay.calibrate(to_dev(d["x"], wl.dtype), to_dev(d["gy"], wl.dtype), wl.B, finalize=False) == 0
    CX = torch.empty((wl.L, wl.L), dtype=torch.float64, device="cuda")
    CG = torch.empty((wl.L, wl.L), dtype=torch.float64, device="cuda")
    lay.get_statistics(CX, CG)
    torch.cuda.synchronize()
    status = lay.calibrate(None, None, 0, finalize=True)
    return lay, status, (xa, ga), (CX.cpu().numpy(), CG.cpu().numpy())


CAL_CASES = [("tiny", "main", "paper"), ("tiny", "main", "ratio"), ("bert_attn", "main", "paper"),
             ("bert_attn", "main", "none"), ("effformer", "up", "paper"), ("effformer", "down", "paper"),
             ("bert_ffn", "up", "paper"), ("bert_ffn", "down", "paper"), ("bert_ffn", "up", "ratio"),
             ("bert_ffn", "down", "none")]


@pytest.mark.parametrize("name,layer,comp", CAL_CASES)
def test_calibration_and_end_to_end(name, layer, comp):
    import rank_compressed_backprop_amd as rcb
    from gpu_util import check_close, empty, from_dev, oracle_magnitudes, rel, to_dev
    wl = W.get_workload(name)
    ly = wl.layer(layer)
    print(f"[calibration] {name}/{layer} comp={comp} L={wl.L}", flush=True)
    lay, status, (xa, ga), (CX_g, CG_g) = _calibrate_both(wl, layer, comp)
    assert status == rcb.INSTANT_OK, rcb.instant_status_str(status)

    # statistics: float32 tile sums of exact products, float64 across slices and batches
    e_cx, e_cg = rel(CX_g, xa.mean()), rel(CG_g, ga.mean())
    print(f"  stats rel err C_X {e_cx:.2e} C_G {e_cg:.2e}", flush=True)
    assert e_cx < 1e-5 and e_cg < 1e-5

    ox = O.calibrate_side(xa.mean(), wl.eps, wl.p, COMP[comp], 64)
    og = O.calibrate_side(ga.mean(), wl.eps, wl.p, COMP[comp], 64)
    assert ox["status"] == O.OK and og["status"] == O.OK
    # the integer decisions are well defined only with a margin at the threshold
    assert ox["margin"] >= 1e-4 and og["margin"] >= 1e-4
    s, info = lay.query()
    print(f"  gpu k/R x {info.kx}/{info.Rx} g {info.ky}/{info.Ry} sweeps {info.sweeps_x}/{info.sweeps_g}; "
          f"oracle x {ox['k']}/{ox['R']} g {og['k']}/{og['R']}", flush=True)
    assert (info.kx, info.Rx, info.ky, info.Ry) == (ox["k"], ox["R"], og["k"], og["R"])

    Rx, Ry = info.Rx, info.Ry
    P_g = torch.empty((Rx, wl.L), device="cuda")
    Q_g = torch.empty((Ry, wl.L), device="cuda")
    sx = torch.empty(wl.L, device="cuda")
    sg = torch.empty(wl.L, device="cuda")
    lay.get_projections(P_g, Q_g, sx, sg)
    torch.cuda.synchronize()
    P_g, Q_g = P_g.cpu().numpy().astype(np.float64), Q_g.cpu().numpy().astype(np.float64)
    sx, sg = sx.cpu().numpy().astype(np.float64), sg.cpu().numpy().astype(np.float64)
    # singular values: the kept ones and the total energy
    for sgpu, o in ((sx, ox), (sg, og)):
        R = o["R"]
        e_sig = np.max(np.abs(sgpu[:R] - o["sigma"][:R]) / o["sigma"][0])
        e_E = abs(np.sum(sgpu ** 2) - o["E"]) / o["E"]
        print(f"  sigma max err {e_sig:.2e} (of sigma_0), energy rel err {e_E:.2e}", flush=True)
        # float32 columns: each of the ~sweeps*(L/8) rotations of a column rounds it at 2^-24,
        # a random walk of about sqrt(#rotations) * 2^-24 <= 1e-5 here; 1e-4 leaves room and
        # is still ten times under the margin the integer decision is required to have
        assert e_sig < 1e-4 and e_E < 1e-4
    # compensation scalars and the projectors (gauge-invariant)
    assert abs(info.cP - ox["c"]) <= 1e-5 * ox["c"]
    assert abs(info.cQ - og["c"]) <= 1e-5 * og["c"]
    for Pg, o in ((P_g, ox), (Q_g, og)):
        Po = o["P"]
        d = rel(Pg.T @ Pg, Po.T @ Po)
        print(f"  projector distance {d:.2e} (gap {o['gap']:.1e})", flush=True)
        assert d < 1e-3
        # with canonical signs on both sides the rows themselves agree
        assert rel(Pg, Po) < 2e-3

    # end to end on a fresh batch: the GPU's own projections against the oracle's
    d = W.make_layer_batch(wl, layer, wl.n_cal, with_w=True)
    x, gy, w = to_dev(d["x"], wl.dtype), to_dev(d["gy"], wl.dtype), to_dev(d["w"], wl.dtype)
    xhat = empty((wl.B, Rx, ly.Cx), wl.dtype)
    gw = empty((ly.Cy, ly.Cx), wl.dtype)
    gx = empty((wl.B, wl.L, ly.Cx), wl.dtype)
    lay.compress_fwd(x, wl.B, xhat)
    lay.backward(xhat, gy, w, wl.B, gw, gx)
    torch.cuda.synchronize()
    xh_o = O.compress(ox["P"], d["x64"])
    out = O.backward(ox["P"], og["P"], xh_o, d["gy64"], d["w64"])
    xh_m, out_m = oracle_magnitudes(O, ox["P"], og["P"], d["x64"], d["gy64"], d["w64"])
    dt = wl.dtype
    msg = [check_close("xhat", from_dev(xhat, dt), xh_o, dt, xh_m),
           check_close("gw", from_dev(gw, dt), out["gw"], dt, out_m["gw"]),
           check_close("gx", from_dev(gx, dt), out["gx"], dt, out_m["gx"])]
    print("  end-to-end rel err Frobenius/per-element: " + ", ".join(msg), flush=True)


def test_full_rank_identity_on_gpu():
    """R = L with uncompensated projections: P^T P = I, so the low-rank gradients are
    the exact g_w = sum gy^T x and g_x = gy w (fp32, L = 64)."""
    import rank_compressed_backprop_amd as rcb
    from gpu_util import empty, from_dev, rel, to_dev
    rng = np.random.default_rng(11)
    B, L, C = 4, 64, 64
    lay = rcb.InstantLayer(rcb.make_config(L, C, C, B, R_max=64, p=64, eps=0.95, dtype="fp32", comp="none"))
    x = rng.standard_normal((B, L, C)).astype(np.float32)
    gy = rng.standard_normal((B, L, C)).astype(np.float32)
    w = (0.1 * rng.standard_normal((C, C))).astype(np.float32)
    assert lay.calibrate(to_dev(x, "fp32"), to_dev(gy, "fp32"), B, finalize=True) == 0
    s, info = lay.query()
    assert info.Rx == L and info.Ry == L
    xh, gw, gx = empty((B, L, C), "fp32"), empty((C, C), "fp32"), empty((B, L, C), "fp32")
    xd, gyd, wd = to_dev(x, "fp32"), to_dev(gy, "fp32"), to_dev(w, "fp32")
    lay.compress_fwd(xd, B, xh)
    lay.backward(xh, gyd, wd, B, gw, gx)
    torch.cuda.synchronize()
    ex = O.exact_backward(x, gy, w)
    e_gw, e_gx = rel(from_dev(gw, "fp32"), ex["gw"]), rel(from_dev(gx, "fp32"), ex["gx"])
    print(f"  full-rank identity rel err gw {e_gw:.2e} gx {e_gx:.2e}", flush=True)
    assert e_gw < 1e-4 and e_gx < 1e-4


def test_eps_one_keeps_every_direction():
    """eps = 1 (关键设计 2: the whole energy): k is the last index whose sigma^2 still adds to
    the prefix sum, i.e. every direction of full-rank statistics, so k = R = L; with the
    compensation off P^T P = I and the low-rank gradients are the exact ones."""
    import rank_compressed_backprop_amd as rcb
    from gpu_util import check_close, empty, from_dev, to_dev
    rng = np.random.default_rng(21)
    B, L, C = 4, 64, 64
    x = rng.standard_normal((B, L, C)).astype(np.float32)
    gy = rng.standard_normal((B, L, C)).astype(np.float32)
    w = (0.1 * rng.standard_normal((C, C))).astype(np.float32)
    lay = rcb.InstantLayer(rcb.make_config(L, C, C, B, R_max=64, p=0, eps=1.0, dtype="fp32", comp="none"))
    assert lay.calibrate(to_dev(x, "fp32"), to_dev(gy, "fp32"), B, finalize=True) == rcb.INSTANT_OK
    _, info = lay.query()
    acc_x, acc_g = O.Accumulator(L), O.Accumulator(L)
    acc_x.add(x)
    acc_g.add(gy)
    for acc, k_gpu, R_gpu in ((acc_x, info.kx, info.Rx), (acc_g, info.ky, info.Ry)):
        o = O.calibrate_side(acc.mean(), 1.0, 0, O.COMP_NONE, 64)
        # the decision is well defined: the last direction's share is far above rounding
        assert o["sigma"][-1] ** 2 / o["E"] > 1e-6
        print(f"[eps=1] gpu k/R {k_gpu}/{R_gpu}, oracle {o['k']}/{o['R']}", flush=True)
        assert (k_gpu, R_gpu) == (o["k"], o["R"]) == (L, L)
    xh, gw, gx = empty((B, L, C), "fp32"), empty((C, C), "fp32"), empty((B, L, C), "fp32")
    xd, gyd, wd = to_dev(x, "fp32"), to_dev(gy, "fp32"), to_dev(w, "fp32")
    lay.compress_fwd(xd, B, xh)
    lay.backward(xh, gyd, wd, B, gw, gx)
    torch.cuda.synchronize()
    ex = O.exact_backward(x, gy, w)
    mag = O.exact_backward(np.abs(x), np.abs(gy), np.abs(w))
    print("  " + check_close("gw", from_dev(gw, "fp32"), ex["gw"], "fp32", mag["gw"]) + ", "
          + check_close("gx", from_dev(gx, "fp32"), ex["gx"], "fp32", mag["gx"]), flush=True)


def test_statistics_long_ragged_token_axis():
    """Statistics (关键设计 1: S = sum over samples of x_b x_b^T, accumulated over batches) on a
    long ragged token axis, L = 2000 (16 tiles of 128 rows, the last one partly padded), with
    channel counts that are not multiples of a stage (136, 264), over two batches (the second
    adds to the first): the float64 means against the oracle's, entry by entry. At this length
    the SYRK runs in 256 x 128 blocks."""
    import rank_compressed_backprop_amd as rcb
    from gpu_util import rel, to_dev
    rng = np.random.default_rng(33)
    B, L, Cx, Cy = 3, 2000, 136, 264
    lay = rcb.InstantLayer(rcb.make_config(L, Cx, Cy, B, R_max=64, p=0, eps=0.9, dtype="bf16"))
    acc = {"C_X": O.Accumulator(L), "C_G": O.Accumulator(L)}
    mag = {"C_X": O.Accumulator(L), "C_G": O.Accumulator(L)}
    for t in range(2):
        x = W.to_io(rng.standard_normal((B, L, Cx)), "bf16")
        gy = W.to_io(rng.standard_normal((B, L, Cy)), "bf16")
        for k, v in (("C_X", x), ("C_G", gy)):
            v64 = W.io_to_f64(v, "bf16")
            acc[k].add(v64)
            mag[k].add(np.abs(v64))
        assert lay.calibrate(to_dev(x, "bf16"), to_dev(gy, "bf16"), B, finalize=False) == rcb.INSTANT_OK
    CX = torch.empty((L, L), dtype=torch.float64, device="cuda")
    CG = torch.empty((L, L), dtype=torch.float64, device="cuda")
    lay.get_statistics(CX, CG)
    torch.cuda.synchronize()
    for name, got in (("C_X", CX.cpu().numpy()), ("C_G", CG.cpu().numpy())):
        ref, m = acc[name].mean(), mag[name].mean()
        # bf16 products are exact in float32; a float32 partial sums at most B * 2 * C of them,
        # whose rounding error is at most that count times 2^-24 times the sum of |terms| (m),
        # before the float64 sums
        bound = 2.0 ** -24 * B * 2 * (Cy if name == "C_G" else Cx) * m
        worst = float(np.max(np.abs(got - ref) - bound))
        print(f"[stats L={L}] {name}: rel err {rel(got, ref):.2e}, max |err| - bound {worst:.2e}", flush=True)
        assert np.array_equal(got, got.T), name
        assert rel(got, ref) < 1e-5 and worst <= 0.0, name


def _fresh_layer(dtype="fp32", L=32, C=16, B=2, **kw):
    import rank_compressed_backprop_amd as rcb
    return rcb.InstantLayer(rcb.make_config(L, C, C, B, dtype=dtype, **kw))


def test_zero_energy_is_reported_and_keeps_old_projections():
    import rank_compressed_backprop_amd as rcb
    from gpu_util import empty, to_dev
    lay = _fresh_layer()
    P = torch.eye(32, device="cuda")[:3].contiguous()
    lay.set_projections(P, 3, P, 3)
    z = to_dev(np.zeros((2, 32, 16), np.float32), "fp32")
    g = to_dev(np.random.default_rng(1).standard_normal((2, 32, 16)).astype(np.float32), "fp32")
    assert lay.calibrate(z, g, 2, finalize=True) == rcb.INSTANT_E_ENERGY
    s, info = lay.query()
    assert s == rcb.INSTANT_E_ENERGY and info.Rx == 3
    xh = empty((2, 3, 16), "fp32")
    lay.compress_fwd(g, 2, xh)  # the old projections are still active
    torch.cuda.synchronize()


def test_rank_overflow_is_reported():
    import rank_compressed_backprop_amd as rcb
    from gpu_util import to_dev
    wl = W.get_workload("bert_attn")
    lay = rcb.InstantLayer(rcb.make_config(wl.L, 768, 768, wl.B, R_max=4, p=wl.p, dtype="bf16"))
    d = W.make_layer_batch(wl, 0, 0)
    assert lay.calibrate(to_dev(d["x"], "bf16"), to_dev(d["gy"], "bf16"), wl.B, finalize=True) == rcb.INSTANT_E_RANK


def test_nonfinite_statistics_are_reported():
    import rank_compressed_backprop_amd as rcb
    from gpu_util import to_dev
    lay = _fresh_layer()
    x = np.random.default_rng(2).standard_normal((2, 32, 16)).astype(np.float32)
    x[1, 5, 3] = np.nan
    assert lay.calibrate(to_dev(x, "fp32"), to_dev(np.abs(x[::-1]).copy(), "fp32"), 2,
                         finalize=True) == rcb.INSTANT_E_NONFINITE


def test_no_convergence_is_reported():
    import rank_compressed_backprop_amd as rcb
    from gpu_util import to_dev
    lay = _fresh_layer(L=64, C=64, max_sweeps=1)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 64, 64)).astype(np.float32)
    assert lay.calibrate(to_dev(x, "fp32"), to_dev(x, "fp32"), 2, finalize=True) == rcb.INSTANT_E_NOCONV


def test_hand_built_spectrum_through_gpu_eigensolver():
    """C = H diag(lam) H^T with a normalised Hadamard H: the GPU must recover lam and
    pick the brute-force k; statistics are fed as samples t_b = H diag(sqrt(lam)) (scaled)."""
    import rank_compressed_backprop_amd as rcb
    from gpu_util import to_dev
    from pins import brute_force_k, hadamard
    L = 64
    H = hadamard(L)
    lam = 0.7 ** np.arange(L)
    eps, p = 0.9, 3
    # one sample whose t t^T equals L * C when its L channels are H diag(sqrt(lam)) * sqrt(L)
    t = (H * np.sqrt(lam)[None, :]).astype(np.float32)[None]  # [1, L, L]: t t^T = H diag(lam) H^T
    lay = rcb.InstantLayer(rcb.make_config(L, L, L, 1, p=p, eps=eps, dtype="fp32", comp="none"))
    assert lay.calibrate(to_dev(t, "fp32"), to_dev(t, "fp32"), 1, finalize=True) == 0
    s, info = lay.query()
    kb = brute_force_k(lam, eps)
    assert info.kx == kb and info.Rx == min(kb + p, L)
    sx = torch.empty(L, device="cuda")
    lay.get_projections(None, None, sx, None)
    torch.cuda.synchronize()
    got = sx.cpu().numpy().astype(np.float64)
    R = info.Rx
    # kept values to float32 resolution
    assert np.max(np.abs(got[:R] - lam[:R]) / lam[:R]) < 1e-5
    # every value to 1e-4 of ||C||_F, a bound stated apart from the solver's internals: a
    # backward-stable float32 eigensolver at L = 64 is accurate to about L * 2^-24 * ||C||_F
    # (4e-6 of it); 1e-4 leaves room for the small tail it may leave unrotated
    assert np.max(np.abs(got - lam)) < 1e-4 * np.sqrt(np.sum(lam ** 2))
    # and what the truncation needs (关键设计 2): the measured errors move the prefix sums of
    # sigma^2 by less than the margin that decides k on the exact spectrum
    st, k, _, prefix = O.truncate(lam, O.eps_as_f32(eps), p)
    assert st == O.OK and k == kb
    assert np.sum(np.abs(got ** 2 - lam ** 2)) < O.margin(prefix, k, O.eps_as_f32(eps)) * prefix[-1]


@pytest.mark.parametrize("name", ["tiny", "bert_attn", "effformer"])
def test_warm_started_recalibration(name):
    """The second finalize starts from the first one's accumulated rotation; it must
    reproduce the oracle on its own statistics (and needs fewer sweeps)."""
    import rank_compressed_backprop_amd as rcb
    from gpu_util import rel, to_dev
    wl = W.get_workload(name)
    ly = wl.layer(0)
    lay = rcb.InstantLayer(rcb.make_config(wl.L, ly.Cx, ly.Cy, wl.B, R_max=64, p=wl.p, eps=wl.eps,
                                           dtype=wl.dtype, comp="paper"))
    half = max(wl.n_cal // 2, 1)
    sweeps = []
    for window in (range(0, half), range(half, 2 * half)):
        xa, ga = O.Accumulator(wl.L), O.Accumulator(wl.L)
        for j, t in enumerate(window):
            d = W.make_layer_batch(wl, 0, t)
            xa.add(d["x64"])
            ga.add(d["gy64"])
            s = lay.calibrate(to_dev(d["x"], wl.dtype), to_dev(d["gy"], wl.dtype), wl.B,
                              finalize=(j == len(window) - 1))
            assert s in (0,), rcb.instant_status_str(s)
        _, info = lay.query()
        sweeps.append((info.sweeps_x, info.sweeps_g))
        ox = O.calibrate_side(xa.mean(), wl.eps, wl.p, O.COMP_PAPER, 64)
        og = O.calibrate_side(ga.mean(), wl.eps, wl.p, O.COMP_PAPER, 64)
        assert (info.kx, info.Rx, info.ky, info.Ry) == (ox["k"], ox["R"], og["k"], og["R"])
        P_g = torch.empty((info.Rx, wl.L), device="cuda")
        Q_g = torch.empty((info.Ry, wl.L), device="cuda")
        lay.get_projections(P_g, Q_g)
        torch.cuda.synchronize()
        for Pg, o in ((P_g, ox), (Q_g, og)):
            Pg = Pg.cpu().numpy().astype(np.float64)
            assert rel(Pg.T @ Pg, o["P"].T @ o["P"]) < 1e-3
    print(f"  sweeps cold {sweeps[0]} warm {sweeps[1]}", flush=True)
