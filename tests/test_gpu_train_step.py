"""GPU tests of the training-step integration (rank_compressed_backprop_amd.linear): the
calibration schedule of each N_t window, exact gradients on calibration steps, the
library's low-rank gradients (against the oracle) on the others, what the forward keeps
for the backward, and the gradient error against the exact gradient as p varies.

Notes "INSTANT: Compressing Gradients and Activations for Resource-Efficient Training":
整体框架 (calibrate every N_t steps, compress in between), 关键设计 2 (p), 关键设计 3."""
import numpy as np
import pytest

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _step(mod, x_dev, gy_dev):
    """One training step of the layer: forward, then backward of y with incoming gradient gy."""
    x = x_dev.clone().requires_grad_(True)
    mod.weight.grad = None
    y = mod(x)
    y.backward(gy_dev)
    return x.grad, mod.weight.grad


def test_schedule_and_gradients_fp32():
    """Two windows of N_t = 5 steps with N_cal = 2 on the tiny fp32 workload."""
    from gpu_util import from_dev, rel, to_dev
    from rank_compressed_backprop_amd.linear import InstantLinear
    wl = W.get_workload("tiny")
    ly = wl.layer(0)
    B, L = wl.B, wl.L
    N_t, N_cal, R_max = 5, 2, 32
    d0 = W.make_layer_batch(wl, 0, 0, with_w=True)
    w = to_dev(d0["w"], "fp32")
    mod = InstantLinear(L, ly.Cx, ly.Cy, B, N_t=N_t, N_cal=N_cal, p=wl.p, eps=wl.eps, dtype="fp32",
                        R_max=R_max, weight=w)
    w64 = d0["w64"]
    # before the first finalize the steps after the calibration ones have no projections
    assert [mod.mode_of_step(s) for s in range(N_t)] == ["calibrate", "finalize", "exact", "exact", "exact"]
    modes = []

    batches = [W.make_layer_batch(wl, 0, t) for t in range(2 * N_t)]
    for s in range(2 * N_t):
        d = batches[s]
        mode = mod.mode_of_step(s)
        modes.append(mode)
        print(f"[train step] step {s} mode {mode}", flush=True)
        gx, gw = _step(mod, to_dev(d["x"], "fp32"), to_dev(d["gy"], "fp32"))
        gx, gw = from_dev(gx, "fp32"), from_dev(gw, "fp32")
        if mode in ("calibrate", "finalize"):
            ex = O.exact_backward(d["x64"], d["gy64"], w64)
            e = (rel(gw, ex["gw"]), rel(gx, ex["gx"]))
            print(f"  exact step: rel err gw {e[0]:.2e} gx {e[1]:.2e}", flush=True)
            assert max(e) <= 1e-5
        else:
            P = torch.empty((mod.Rx, L), dtype=torch.float32, device="cuda")
            Q = torch.empty((mod.Ry, L), dtype=torch.float32, device="cuda")
            mod.layer.get_projections(P, Q)
            P64 = P.cpu().numpy().astype(np.float64)
            Q64 = Q.cpu().numpy().astype(np.float64)
            out = O.backward(P64, Q64, O.compress(P64, d["x64"]), d["gy64"], w64)
            e = (rel(gw, out["gw"]), rel(gx, out["gx"]))
            print(f"  low-rank step: rel err gw {e[0]:.2e} gx {e[1]:.2e}", flush=True)
            assert max(e) <= 1e-4
        if mode == "finalize":
            # the window's projections come from its own calibration steps only
            w0 = s - (N_cal - 1)
            # (the layer's default compensation is the ratio reading)
            cal = O.calibrate([batches[t]["x64"] for t in range(w0, s + 1)],
                              [batches[t]["gy64"] for t in range(w0, s + 1)], wl.eps, wl.p, O.COMP_RATIO, R_max)
            assert mod.last_status == 0, mod.status()
            assert (mod.Rx, mod.Ry) == (cal["x"]["R"], cal["g"]["R"])
            P = torch.empty((mod.Rx, L), dtype=torch.float32, device="cuda")
            Q = torch.empty((mod.Ry, L), dtype=torch.float32, device="cuda")
            mod.layer.get_projections(P, Q)
            for Pg, o in ((P.cpu().numpy().astype(np.float64), cal["x"]), (Q.cpu().numpy().astype(np.float64), cal["g"])):
                dist = rel(Pg.T @ Pg, o["P"].T @ o["P"])
                print(f"  window projections: R {o['R']} projector distance {dist:.2e}", flush=True)
                assert dist < 1e-3
    assert modes == ["calibrate", "finalize", "compress", "compress", "compress"] * 2
    assert mod.generation == 2 and mod.step == 2 * N_t


def test_compressed_step_keeps_only_xhat():
    """What a compressed step's forward saves: x_hat [B, Rx, Cx] (and w), not x."""
    from gpu_util import to_dev
    from rank_compressed_backprop_amd.linear import InstantLinear
    wl = W.get_workload("tiny")
    ly = wl.layer(0)
    B, L = wl.B, wl.L
    mod = InstantLinear(L, ly.Cx, ly.Cy, B, N_t=3, N_cal=1, p=wl.p, eps=wl.eps, dtype="fp32", R_max=32)
    d = W.make_layer_batch(wl, 0, 0)
    x, gy = to_dev(d["x"], "fp32"), to_dev(d["gy"], "fp32")
    _step(mod, x, gy)  # calibration step: finalizes
    assert mod.generation == 1 and mod.Rx < L
    saved = []
    with torch.autograd.graph.saved_tensors_hooks(lambda t: (saved.append(tuple(t.shape)), t)[1], lambda t: t):
        xr = x.clone().requires_grad_(True)
        y = mod(xr)
    assert mod.mode_of_step(mod.step - 1) == "compress"
    assert (B, mod.Rx, ly.Cx) in saved and (B, L, ly.Cx) not in saved
    y.backward(gy)
    # memory the step keeps for its backward, against the exact backward's x
    print(f"[train step] saved {saved}: activation kept {mod.Rx}/{L} of x", flush=True)


@pytest.mark.timeout(300)
def test_gradient_error_against_exact_as_p_varies():
    """BERT-base attention projection (B=32, L=512, 768 -> 768, bf16): relative error of the
    low-rank gradients against the exact gradients of the same steps, for p = 0, 2, 8
    (N_cal = 4 calibration steps, then 4 compressed steps), and the drift of the projection
    subspace between two windows at p = 2.

    The error is measured with the compensation off (P = U_R^T, an orthogonal projector)
    and with the ratio reading (the layer's default): the printed compensation scales
    g_w by c_P^2 and g_x by c_Q^2 with c = S_R^(-1/2), a scalar with units that makes the
    raw error against the exact gradient meaningless. With the compensation off, more
    oversampling keeps more of the spectrum, so the error may not grow with p."""
    from gpu_util import to_dev
    from rank_compressed_backprop_amd.linear import InstantLinear
    wl = W.get_workload("bert_attn")
    ly = wl.layer(0)
    B, L = wl.B, wl.L
    N_cal, N_t = 4, 8
    print("[train step] generating 2 windows of BERT-size batches", flush=True)
    dw = W.make_layer_batch(wl, 0, 0, with_w=True)
    w = to_dev(dw["w"], "bf16")
    data = []
    for t in range(2 * N_t):
        d = W.make_layer_batch(wl, 0, 100 + t)
        data.append((to_dev(d["x"], "bf16"), to_dev(d["gy"], "bf16")))
        del d
    w32 = w.float()
    errs = {}
    proj = []
    for comp in ("none", "ratio"):
        for p in (0, 2, 8):
            mod = InstantLinear(L, ly.Cx, ly.Cy, B, N_t=N_t, N_cal=N_cal, p=p, eps=wl.eps, dtype="bf16",
                                comp=comp, weight=w)
            e_w, e_x = [], []
            nwin = 2 if (comp, p) == ("none", 2) else 1
            for s in range(nwin * N_t):
                x, gy = data[s]
                gx, gw = _step(mod, x, gy)
                if mod.mode_of_step(s) == "compress":
                    # exact gradient of the same step in float32
                    xf, gf = x.float().reshape(-1, ly.Cx), gy.float().reshape(-1, ly.Cy)
                    gw_ex = gf.t().contiguous() @ xf
                    gx_ex = gf @ w32
                    e_w.append(float(torch.linalg.norm(gw.float() - gw_ex) / torch.linalg.norm(gw_ex)))
                    e_x.append(float(torch.linalg.norm(gx.float().reshape(-1, ly.Cx) - gx_ex)
                                     / torch.linalg.norm(gx_ex)))
                if mod.mode_of_step(s) == "finalize" and nwin == 2:
                    P = torch.empty((mod.Rx, L), dtype=torch.float32, device="cuda")
                    mod.layer.get_projections(P, None)
                    proj.append(P.double().cpu().numpy())
            errs[(comp, p)] = (float(np.mean(e_w)), float(np.mean(e_x)), mod.Rx, mod.Ry)
            print(f"  comp {comp} p={p}: Rx {mod.Rx} Ry {mod.Ry}; mean rel err vs exact over 4 steps: "
                  f"g_w {errs[(comp, p)][0]:.3e} g_x {errs[(comp, p)][1]:.3e}", flush=True)
            del mod
    for a, b in ((0, 2), (2, 8)):
        ea, eb = errs[("none", a)], errs[("none", b)]
        assert eb[2] >= ea[2]
        assert eb[0] <= ea[0] * 1.02 and eb[1] <= ea[1] * 1.02
    # the layer's default compensation keeps a compressed step's gradients on the scale of the
    # exact gradients of the same step (the printed factor would shrink them by c^2 ~ 1e-11)
    import rank_compressed_backprop_amd as rcb
    mod = InstantLinear(L, ly.Cx, ly.Cy, B, N_t=N_t, N_cal=N_cal, p=2, eps=wl.eps, dtype="bf16", weight=w)
    assert mod.layer.cfg.comp == rcb.INSTANT_COMP_RATIO
    for s in range(N_t):
        x, gy = data[s]
        gx, gw = _step(mod, x, gy)
        if mod.mode_of_step(s) == "compress":
            xf, gf = x.float().reshape(-1, ly.Cx), gy.float().reshape(-1, ly.Cy)
            r_w = float(torch.linalg.norm(gw.float()) / torch.linalg.norm(gf.t().contiguous() @ xf))
            r_x = float(torch.linalg.norm(gx.float()) / torch.linalg.norm(gf @ w32))
            print(f"  default compensation, step {s}: |g_w| / |g_w exact| {r_w:.3f}, "
                  f"|g_x| / |g_x exact| {r_x:.3f}", flush=True)
            assert 0.5 <= r_w <= 2.0 and 0.5 <= r_x <= 2.0
    mod.layer.close()

    P1, P2 = proj
    k = min(P1.shape[0], P2.shape[0])
    U1 = np.linalg.qr(P1[:k].T)[0]
    U2 = np.linalg.qr(P2[:k].T)[0]
    drift = float(np.linalg.norm(U1 @ U1.T - U2 @ U2.T) / np.sqrt(2 * k))
    print(f"  comp none p=2: subspace drift between the two windows' P (rank {k}): {drift:.3e}", flush=True)
    assert 0.0 <= drift <= 1.0
