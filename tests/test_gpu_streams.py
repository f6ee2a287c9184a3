"""GPU test of the one overlap the C ABI allows: statistics calls on a second stream while
the forward compression and the low-rank backward run on another. Every kernel is
deterministic, so the overlapped run must reproduce the serial one bit for bit.

Notes "INSTANT: Compressing Gradients and Activations for Resource-Efficient Training":
整体框架 (statistics on calibration steps, compression and backward on every step)."""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _run(two_streams: bool, xs, gys, w, P0, Q0, L, Cx, Cy, B):
    import rank_compressed_backprop_amd as rcb
    from gpu_util import empty
    lay = rcb.InstantLayer(rcb.make_config(L, Cx, Cy, B, R_max=64, p=2, dtype="bf16"))
    lay.set_projections(P0, P0.shape[0], Q0, Q0.shape[0])
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream() if two_streams else main
    ready = torch.cuda.Event()
    ready.record(main)  # inputs and projections are in place on the main stream
    side.wait_event(ready)
    outs = []
    n = len(xs)
    Rx = P0.shape[0]  # every step runs under the installed projections; the finalize comes last
    for t in range(n):
        xhat = empty((B, 64, Cx), "bf16")
        gw, gx = empty((Cy, Cx), "bf16"), empty((B, L, Cx), "bf16")
        lay.compress_fwd(xs[t], B, xhat)
        lay.backward(xhat, gys[t], w, B, gw, gx)
        fin = t == n - 1
        if fin and two_streams:
            # the finalize rewrites the inactive projection buffer: after the main stream's calls
            ev = torch.cuda.Event()
            ev.record(main)
            side.wait_event(ev)
        s = lay.calibrate(xs[t], gys[t], B, finalize=fin, stream=side)
        assert s == rcb.INSTANT_OK, rcb.instant_status_str(s)
        # x_hat is packed [B, Rx, Cx] at the start of the R_max-sized buffer
        outs.append((gw, gx, xhat.view(-1)[:B * Rx * Cx].view(B, Rx, Cx)))
    torch.cuda.synchronize()
    _, info = lay.query()
    P = torch.empty((info.Rx, L), device="cuda")
    Q = torch.empty((info.Ry, L), device="cuda")
    lay.get_projections(P, Q)
    torch.cuda.synchronize()
    return outs, P, Q, info


def test_statistics_on_a_second_stream_match_serial():
    wl = W.get_workload("bert_attn")
    ly = wl.layer(0)
    B, L, Cx, Cy = 8, wl.L, ly.Cx, ly.Cy
    from gpu_util import to_dev
    xs, gys = [], []
    for t in range(4):
        d = W.make_layer_batch(wl, 0, 300 + t)
        xs.append(to_dev(d["x"][:B], "bf16"))
        gys.append(to_dev(d["gy"][:B], "bf16"))
    w = to_dev(W.make_layer_batch(wl, 0, 0, with_w=True)["w"], "bf16")
    rng = np.random.default_rng(11)
    P0 = torch.from_numpy((rng.standard_normal((8, L)) / np.sqrt(L)).astype(np.float32)).cuda()
    Q0 = torch.from_numpy((rng.standard_normal((8, L)) / np.sqrt(L)).astype(np.float32)).cuda()
    print("[streams] serial run, then statistics on a side stream", flush=True)
    ref = _run(False, xs, gys, w, P0, Q0, L, Cx, Cy, B)
    got = _run(True, xs, gys, w, P0, Q0, L, Cx, Cy, B)
    for (a, b) in zip(ref[0], got[0]):
        for ta, tb in zip(a, b):
            assert torch.equal(ta.view(torch.int16), tb.view(torch.int16))
    assert torch.equal(ref[1], got[1]) and torch.equal(ref[2], got[2])
    assert (ref[3].Rx, ref[3].Ry, ref[3].kx, ref[3].ky) == (got[3].Rx, got[3].Ry, got[3].kx, got[3].ky)
    print(f"[streams] identical: Rx {got[3].Rx} Ry {got[3].Ry}", flush=True)


def test_async_finalize_matches_sync_and_switches_at_a_forward():
    """An asynchronous finalize (queued on a side stream, no host wait) publishes the same
    projections bit for bit as a synchronous one; they take effect at the first forward
    compression after the device has finished the finalize, and instant_query waits for it."""
    import rank_compressed_backprop_amd as rcb
    from gpu_util import empty, to_dev
    wl = W.get_workload("bert_attn")
    ly = wl.layer(0)
    B, L, Cx, Cy = 8, wl.L, ly.Cx, ly.Cy
    batches = []
    for t in range(8):
        d = W.make_layer_batch(wl, 0, 400 + t)
        batches.append((to_dev(d["x"][:B], "bf16"), to_dev(d["gy"][:B], "bf16")))
    cfg = dict(R_max=64, p=2, dtype="bf16")
    ref = rcb.InstantLayer(rcb.make_config(L, Cx, Cy, B, **cfg))
    lay = rcb.InstantLayer(rcb.make_config(L, Cx, Cy, B, **cfg))
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()

    def window(ws):
        for x, g in ws[:-1]:
            assert ref.calibrate(x, g, B) == 0
            assert lay.calibrate(x, g, B, stream=side) == 0
        x, g = ws[-1]
        s = ref.calibrate(x, g, B, finalize=True)
        assert s == rcb.INSTANT_OK, rcb.instant_status_str(s)
        side.wait_stream(main)
        assert lay.calibrate(x, g, B, finalize="async", stream=side) == rcb.INSTANT_OK

    def proj(l, info):
        P = torch.empty((info.Rx, L), device="cuda")
        Q = torch.empty((info.Ry, L), device="cuda")
        l.get_projections(P, Q)
        torch.cuda.synchronize()
        return P, Q

    # first window: query waits for the asynchronous outcome
    window(batches[:4])
    side.wait_stream(main)
    s, info = lay.query()
    _, info_r = ref.query()
    assert s == rcb.INSTANT_OK and info.generation == 1
    assert (info.kx, info.Rx, info.ky, info.Ry) == (info_r.kx, info_r.Rx, info_r.ky, info_r.Ry)
    for a, b in zip(proj(lay, info), proj(ref, info_r)):
        assert torch.equal(a, b)

    # second window: once the device has finished, the next forward uses the new projections
    window(batches[4:])
    torch.cuda.synchronize()
    x = batches[0][0]
    xh_l, xh_r = empty((B, 64, Cx), "bf16"), empty((B, 64, Cx), "bf16")
    lay.compress_fwd(x, B, xh_l)  # raises on an error status
    ref.compress_fwd(x, B, xh_r)
    torch.cuda.synchronize()
    _, info = lay.query()
    _, info_r = ref.query()
    assert info.generation == 2 and info_r.generation == 2
    n = B * info.Rx * Cx
    assert torch.equal(xh_l.view(-1)[:n].view(torch.int16), xh_r.view(-1)[:n].view(torch.int16))
    print(f"[streams] asynchronous finalize identical: Rx {info.Rx} Ry {info.Ry}", flush=True)
