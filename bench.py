"""Throughput of the INSTANT low-rank backward on one MI355X.

Workload: BERT-base attention-projection-shaped linear y = x w^T, bf16 I/O with
float32 accumulation, B=32 sequences of L=512 tokens, Cx=Cy=768, eps=0.95, p=2,
statistics over N_cal=16 batches, recalibration every N_t=100 steps (shapes of the
BERT layers the INSTANT notes evaluate; synthetic token-low-rank data, see
workloads/).

The metric (`value`) is the low-rank backward's throughput: tokens/s = B * L / t_bwd,
where t_bwd is the median time of one instant_backward (the stacked projection of g_y,
g_w, g_hat_x and the expansion; notes section 关键设计 3). It is measured with HIP events
on the launch stream around runs of 8 consecutive instant_backward calls, 200 timed runs
after 20 untimed ones, each call on its own resident batch (g_y, x_hat, g_x rotate over
the resident set, beyond the 256 MB last-level cache); p10 and p90 of the per-call time
are reported beside it, and the same runs replayed from a HIP graph for comparison.

The `--steps K --warmup W` steps are whole passes of the path on the notes'
schedule (section 整体框架): every step compresses x (x_hat = P x) and runs the low-rank
backward; the first N_cal steps of every N_t-step window also accumulate the statistics,
and the last of them finalizes (eigen-decomposition, truncation, new P and Q). Their wall
time gives `ms_per_step`. Because K is usually less than a window, the schedule's own rate
is measured separately over two whole N_t windows (`parts.schedule_*`), so it does not
depend on K.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores
MFMA_FP32_PEAK_TFLOPS = 157.3   # MI355X dense fp32
WORKLOAD_NAMES = {"tiny": "tiny fp32", "bert_attn": "BERT-base attention projection",
                  "bert_ffn": "BERT-base FFN", "effformer": "EfficientFormer-L1 last-stage",
                  "llm_mlp": "LLM MLP"}
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "backward_bert_attn_traffic.json")
CALLS_PER_RUN = 8
TIMED_RUNS = 200
WARM_RUNS = 20


def measured_traffic(workload):
    """HBM bytes per instant_backward from the recorded rocprofv3 counters (FETCH_SIZE and
    WRITE_SIZE of the backward's kernels, scaled by a copy kernel of known size), or None
    when the record is for another workload or the kernel sources changed since."""
    import hashlib
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
        if rec.get("workload") != workload:
            return None
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["sources_sha256"]:
            return None
        return rec["traffic_bytes_per_backward"]
    except (OSError, KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="timed steps of the whole path (K)")
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps before them")
    ap.add_argument("--workload", default="bert_attn",
                    help="bert_attn (the headline line); bert_block (every linear layer of a BERT-base "
                         "encoder layer: its low-rank backward against the exact one); or one layer of "
                         "tiny, bert_ffn, effformer, llm_mlp run through the same measurement")
    ap.add_argument("--layer", default="0", help="layer of a two-layer workload (up or down)")
    ap.add_argument("--batches", type=int, default=None,
                    help="distinct resident batches cycled through (default 32: more than N_cal, so "
                         "consecutive calibration windows see different statistics; N_cal for llm_mlp, "
                         "whose batches take seconds each to generate)")
    ap.add_argument("--windows", type=int, default=2, help="whole N_t windows timed for the schedule rate")
    ap.add_argument("--runs", type=int, default=TIMED_RUNS,
                    help=f"timed runs of {CALLS_PER_RUN} consecutive instant_backward calls (the metric's samples)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--one-stream", action="store_true",
                    help="run the statistics on the main stream too (no overlap with the hot path)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before the timed region, copy a buffer of this many MiB three times (a plain "
                         "copy kernel of known size that scales the profiler's byte counters)")
    ap.add_argument("--cpu-sample", type=int, default=8, help="samples of a batch the oracle times")
    ap.add_argument("--solver", default="subspace", choices=("jacobi", "subspace"),
                    help="eigensolver of the finalize: the top-m subspace iteration (stops once its "
                         "Ritz residuals pass), or the full Jacobi decomposition")
    ap.add_argument("--sub-iters", type=int, default=6, help="most subspace steps per finalize")
    ap.add_argument("--sync-finalize", action="store_true",
                    help="finalize synchronously (the host waits for the outcome) instead of queueing it "
                         "and letting the next forward compression after it pick up the new projections")
    return ap.parse_args()


def quantile(v, q):
    v = sorted(v)
    if not v:
        return None
    pos = q * (len(v) - 1)
    lo = int(pos)
    hi = min(lo + 1, len(v) - 1)
    return v[lo] + (v[hi] - v[lo]) * (pos - lo)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the multi-GPU data-parallel path is a design, not built "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.workload == "bert_block":
        bench_block(args)
        return

    import numpy as np
    import torch

    import rank_compressed_backprop_amd as rcb
    import workloads as W

    wl = W.get_workload(args.workload)
    layer = int(args.layer) if args.layer.isdigit() else args.layer
    ly = wl.layer(layer)
    li = wl.layers.index(ly)
    B, L, Cx, Cy = wl.B, wl.L, ly.Cx, ly.Cy
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32

    def up(a):
        if wl.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    # resident synthetic batches (distinct, so the 256 MB last-level cache cannot hold a step's data)
    nb = args.batches if args.batches is not None else (wl.n_cal if L * (Cx + Cy) * B > 1 << 27 else 32)
    nb = max(nb, wl.n_cal)
    print(f"[bench] {wl.name}/{ly.name}: B={B} L={L} Cx={Cx} Cy={Cy} {wl.dtype}; generating {nb} resident "
          "batches", file=sys.stderr, flush=True)
    xs, gys = [], []
    for t in range(nb):
        d = W.make_layer_batch(wl, li, t)
        xs.append(up(d["x"]))
        gys.append(up(d["gy"]))
        if nb * B * L * (Cx + Cy) > 1 << 30:
            print(f"[bench] generated resident batch {t + 1}/{nb}", file=sys.stderr, flush=True)
    w = up(W.to_io(W.make_w(wl, li), wl.dtype))
    del d

    R_max = 64
    lay = rcb.InstantLayer(rcb.make_config(L, Cx, Cy, B, R_max=R_max, p=wl.p, N_t=wl.n_t, eps=wl.eps,
                                           dtype=wl.dtype, comp="paper", solver=args.solver,
                                           sub_iters=args.sub_iters), device=dev)
    # the library takes the full decomposition when the subspace basis (R_max + 16 columns,
    # rounded up to 16, R_max clamped to L) would not be narrower than L
    m_sub = (min(R_max, L) + 16 + 15) // 16 * 16
    if args.solver == "jacobi":
        solver_used = "jacobi"
    elif m_sub < L:
        solver_used = f"subspace (at most {args.sub_iters} steps)"
    else:
        solver_used = f"jacobi (a subspace basis of {m_sub} columns is not narrower than L = {L})"
    xhat = torch.empty((B, R_max, Cx), dtype=tdt, device=dev)
    gw = torch.empty((Cy, Cx), dtype=tdt, device=dev)
    gx = torch.empty((B, L, Cx), dtype=tdt, device=dev)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # initial calibration (set-up; the cold finalize is timed on its own)
    for t in range(wl.n_cal):
        if t == wl.n_cal - 1:
            torch.cuda.synchronize()
            tc0 = time.perf_counter()
        s = lay.calibrate(xs[t], gys[t], B, finalize=(t == wl.n_cal - 1))
        assert s == rcb.INSTANT_OK, rcb.instant_status_str(s)
    t_cold = time.perf_counter() - tc0

    # The statistics run on a side stream, overlapping the compression and backward on the
    # main one (the overlap the C ABI allows: they use disjoint parts of the workspace; the
    # resident inputs are ready on both streams). A finalizing call first waits for the
    # main stream's calls, since it rewrites the projection buffer they may still read.
    # The finalizing calls of the schedule windows are bracketed by HIP events on the side
    # stream (one pair per window; the span includes that step's statistics batch and the
    # host round trip of the finalize).
    finalize_mode = True if args.sync_finalize else "async"
    main_st = torch.cuda.current_stream()
    side_st = torch.cuda.Stream() if not args.one_stream else main_st
    fin_events = []

    def step(i, timed=False):
        t = i % nb
        ph = i % wl.n_t
        lay.compress_fwd(xs[t], B, xhat)
        lay.backward(xhat, gys[t], w, B, gw, gx)
        if ph < wl.n_cal:
            fin = ph == wl.n_cal - 1
            if fin:
                side_st.wait_stream(main_st)
            if fin and timed:
                ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                ev[0].record(side_st)
            s = lay.calibrate(xs[t], gys[t], B, finalize=(fin and finalize_mode), stream=side_st)
            if fin and timed:
                ev[1].record(side_st)
                fin_events.append(ev)
            if s != rcb.INSTANT_OK:
                raise RuntimeError("calibration failed: " + rcb.instant_status_str(s))

    side_st.wait_stream(main_st)  # the resident batches and the set-up's projections
    # ---- the --steps / --warmup passes: W untimed, then exactly K timed passes of the whole path
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, args.warmup + args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"[bench] {args.steps} timed steps of the whole path: {wall / args.steps * 1e3:.4f} ms a step",
          file=sys.stderr, flush=True)

    # ---- the schedule's rate over whole N_t windows (independent of K): from the next
    # window boundary, `windows` full windows, statistics and finalize included
    i0 = (args.warmup + args.steps + wl.n_t - 1) // wl.n_t * wl.n_t
    for i in range(args.warmup + args.steps, i0):
        step(i)
    torch.cuda.synchronize()
    gen0 = lay.query()[1].generation
    fin_events.clear()
    n_sched = args.windows * wl.n_t
    ts0 = time.perf_counter()
    for i in range(i0, i0 + n_sched):
        step(i, timed=True)
    torch.cuda.synchronize()
    wall_sched = time.perf_counter() - ts0
    fin_loop = [a.elapsed_time(b) * 1e-3 for a, b in fin_events]
    _, info = lay.query()
    published = info.generation - gen0
    if published != len(fin_events):
        print(f"warning: {len(fin_events) - published} of {len(fin_events)} finalizes in the schedule windows "
              "published no projections", file=sys.stderr)
    Rx, Ry = info.Rx, info.Ry
    print(f"[bench] {args.windows} schedule windows: {wall_sched / n_sched * 1e6:.2f} us a step; Rx {Rx} Ry {Ry}",
          file=sys.stderr, flush=True)

    # ---- the metric: one instant_backward. Each call has its own resident batch (g_y), the
    # compressed activation of that batch (under the projections now active) and its own g_x
    # output, so consecutive calls stream different memory. A timed sample is a run of
    # CALLS_PER_RUN consecutive calls on the launch stream between two HIP events (a pair of
    # events around a single call would add the markers' dispatch latency to it); the
    # per-call time of a sample is the run's time over CALLS_PER_RUN.
    st = torch.cuda.current_stream()
    xhats = [torch.empty((B, Rx, Cx), dtype=tdt, device=dev) for _ in range(nb)]
    for t in range(nb):
        lay.compress_fwd(xs[t], B, xhats[t])
    gxs = [torch.empty((B, L, Cx), dtype=tdt, device=dev) for _ in range(nb)]
    torch.cuda.synchronize()

    def run(r):
        for j in range(CALLS_PER_RUN):
            t = (r * CALLS_PER_RUN + j) % nb
            lay.backward(xhats[t], gys[t], w, B, gw, gxs[t])

    for r in range(WARM_RUNS):
        run(r)
    torch.cuda.synchronize()
    runs = max(args.runs, 1)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(runs)]
    for r in range(runs):
        evs[r][0].record(st)
        run(r)
        evs[r][1].record(st)
    torch.cuda.synchronize()
    per_call = [a.elapsed_time(b) * 1e-3 / CALLS_PER_RUN for a, b in evs]  # seconds
    t_bwd = quantile(per_call, 0.5)
    t_bwd_p10, t_bwd_p90 = quantile(per_call, 0.1), quantile(per_call, 0.9)
    t_bwd_mean = sum(per_call) / len(per_call)
    print(f"[bench] instant_backward: median {t_bwd * 1e6:.2f} us (p10 {t_bwd_p10 * 1e6:.2f}, "
          f"p90 {t_bwd_p90 * 1e6:.2f})", file=sys.stderr, flush=True)

    # the same calls captured in a HIP graph and replayed (for comparison)
    cap = torch.cuda.Stream()
    cap.wait_stream(st)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        run(0)
    torch.cuda.synchronize()
    for _ in range(5):
        g.replay()
    gevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(50)]
    for a, b in gevs:
        a.record(st)
        g.replay()
        b.record(st)
    torch.cuda.synchronize()
    t_bwd_graph = quantile([a.elapsed_time(b) * 1e-3 / CALLS_PER_RUN for a, b in gevs], 0.5)
    del g

    # ---- the other parts with HIP events on the launch stream over runs of consecutive
    # launches (a pair of events around one launch would add the markers' dispatch latency)
    def ev_time(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn(0)
        torch.cuda.synchronize()
        e0.record(st)
        for r in range(reps):
            fn(r)
        e1.record(st)
        e1.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3  # seconds

    t_fwd = ev_time(lambda r: lay.compress_fwd(xs[r % nb], B, xhats[r % nb]), 200)
    t_acc = ev_time(lambda r: lay.calibrate(xs[r % nb], gys[r % nb], B, finalize=False), 50)
    # one full finalize (eigen-decomposition of both statistics, truncation, publish)
    torch.cuda.synchronize()
    tf0 = time.perf_counter()
    s = lay.calibrate(None, None, 0, finalize=True)
    torch.cuda.synchronize()
    t_fin = time.perf_counter() - tf0
    _, info2 = lay.query()

    es = 2 if wl.dtype == "bf16" else 4
    bytes_fwd = es * (B * L * Cx + B * Rx * Cx)
    # read g_y once, read x_hat and w, write g_w and g_x
    bytes_bwd = es * (B * L * Cy + B * Rx * Cx + 2 * Cx * Cy + B * L * Cx)
    flops_bwd = B * (2 * (Rx + Ry) * L * Cy + 2 * (Rx + Ry) * Cx * Cy + 2 * Ry * L * Cx)
    # statistics: the upper triangle of both L x L sums per batch (the mirror earns no credit)
    flops_acc = L * (L + 1) * B * (Cx + Cy)
    gbs_bwd = bytes_bwd / t_bwd / 1e9
    gbs_bwd_mean = bytes_bwd / t_bwd_mean / 1e9

    headline = wl.name == "bert_attn"
    wname = f"{WORKLOAD_NAMES.get(wl.name, wl.name)} linear{'' if len(wl.layers) == 1 else ' (' + ly.name + ')'}"
    out = {
        "metric": ("low-rank backward tokens/s + achieved HBM GB/s (% peak), BERT-base linear" if headline else
                   f"low-rank backward tokens/s + achieved HBM GB/s (% peak), {wl.name} linear"),
        "value": B * L / t_bwd,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"{wname}, B={B} L={L} Cx={Cx} Cy={Cy}, "
                               f"eps={wl.eps} p={wl.p} N_cal={wl.n_cal} N_t={wl.n_t}",
                   "global_batch": B, "seq_len": L, "parallelism": "single GPU",
                   "value": "B*L / median time of one instant_backward (a5-a8): HIP events around runs of "
                            f"{CALLS_PER_RUN} consecutive calls on rotating resident batches, {runs} timed "
                            "runs after 20 untimed ones",
                   "step": "ms_per_step: compress + low-rank backward every step; statistics on the first N_cal "
                           "steps of each N_t window; eigen-decomposition + truncation once per window",
                   "streams": "statistics and finalize on a side stream" if not args.one_stream else "one stream",
                   "finalize": "synchronous" if args.sync_finalize else
                               "asynchronous (new projections from the first forward after it completes)",
                   "Rx": Rx, "Ry": Ry, "kx": info.kx, "ky": info.ky},
        "parts": {
            "backward_us_median": t_bwd * 1e6, "backward_us_p10": t_bwd_p10 * 1e6,
            "backward_us_p90": t_bwd_p90 * 1e6, "backward_us_mean": t_bwd_mean * 1e6,
            "backward_GBs": gbs_bwd, "backward_pct_hbm_peak": 100.0 * gbs_bwd / HBM_PEAK_GBS,
            "backward_tokens_per_s_p10_p90": [B * L / t_bwd_p90, B * L / t_bwd_p10],
            "backward_TFLOPs": flops_bwd / t_bwd / 1e12,
            "backward_algorithmic_bytes": bytes_bwd,
            "backward_us_graph_replay_median": t_bwd_graph * 1e6,
            "compress_fwd_us": t_fwd * 1e6, "compress_fwd_GBs": bytes_fwd / t_fwd / 1e9,
            "compress_fwd_pct_hbm_peak": 100.0 * bytes_fwd / t_fwd / 1e9 / HBM_PEAK_GBS,
            "statistics_per_batch_us": t_acc * 1e6,
            "statistics_TFLOPs": flops_acc / t_acc / 1e12,
            "statistics_pct_mfma_bf16_peak" if wl.dtype == "bf16" else "statistics_pct_mfma_fp32_peak":
                100.0 * flops_acc / t_acc / 1e12 / (MFMA_BF16_PEAK_TFLOPS if wl.dtype == "bf16" else
                                                    MFMA_FP32_PEAK_TFLOPS),
            "statistics_GBs": es * B * L * (Cx + Cy) / t_acc / 1e9,
            "schedule_tokens_per_s": n_sched * B * L / wall_sched,
            "schedule_us_per_step": wall_sched / n_sched * 1e6,
            "schedule_windows": args.windows,
            "eigensolver": solver_used,
            "cold_finalize_ms": t_cold * 1e3,
            "finalize_ms": t_fin * 1e3,
            "finalize_in_window_ms": (sum(fin_loop) / len(fin_loop) * 1e3) if fin_loop else None,
            "finalizes_published": f"{published}/{len(fin_events)}",
            "jacobi_sweeps": [info2.sweeps_x, info2.sweeps_g],
            "finalize_status": rcb.instant_status_str(s),
        },
        "roofline": {"kernel": "instant_backward: stacked projection [P;Q] g_y + the g_w / g_hat_x / expansion "
                               "kernels, one call", "bound": "hbm",
                     "achieved": gbs_bwd_mean, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs_bwd_mean / HBM_PEAK_GBS, "traffic": measured_traffic(wl.name + "/" + ly.name),
                     "launch_us_mean": t_bwd_mean * 1e6, "calls_timed": runs * CALLS_PER_RUN,
                     "algorithmic_bytes_per_call": bytes_bwd},
    }

    if not args.no_cpu_baseline and headline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample)
    print(json.dumps(out), flush=True)
    torch.cuda.synchronize()
    lay.close()


# The linear layers of one BERT-base encoder layer (B=32, L=512, bf16): the four attention
# projections (Q, K, V and the output projection, 768 -> 768 each; a fused QKV is the first
# three side by side) and the FFN (768 -> 3072 -> 768), each with its own P and Q.
BLOCK_LAYERS = (("q", "bert_attn", 0, 0), ("k", "bert_attn", 0, 1), ("v", "bert_attn", 0, 2),
                ("o", "bert_attn", 0, 3), ("ffn_up", "bert_ffn", "up", 0), ("ffn_down", "bert_ffn", "down", 0))


def bench_block(args):
    """Per training step of a BERT-base encoder layer's linear layers: the INSTANT path
    (forward compression + low-rank backward of every layer) against the exact backward
    (g_x = g_y w and g_w = g_y^T x by PyTorch/hipBLASLt GEMMs), with the formula FLOP ratio
    and the activation memory ratio of notes 关键设计 3 (vanilla backward 4 L Cx Cy per sample;
    low-rank 2 (Rx + Ry)(Cx Cy + L Cx + L Cy), the compression included; kept activation
    x [L, Cx] against x_hat [Rx, Cx]). Calibration is set-up here, on 4 batches per layer."""
    import numpy as np
    import torch

    import rank_compressed_backprop_amd as rcb
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    n_setup, layers = 4, []
    for name, wname, lname, k in BLOCK_LAYERS:
        wl = W.get_workload(wname)
        ly = wl.layer(lname)
        B, L = wl.B, wl.L
        lay = rcb.InstantLayer(rcb.make_config(L, ly.Cx, ly.Cy, B, R_max=64, p=wl.p, N_t=wl.n_t, eps=wl.eps,
                                               dtype="bf16", comp="paper"), device=dev)
        for t in range(n_setup):
            d = W.make_layer_batch(wl, lname, 200 * k + t)
            s = lay.calibrate(up(d["x"]), up(d["gy"]), B, finalize=(t == n_setup - 1))
            if s != rcb.INSTANT_OK:
                raise RuntimeError(f"{name}: calibration failed: " + rcb.instant_status_str(s))
        d = W.make_layer_batch(wl, lname, 200 * k + n_setup)
        _, info = lay.query()
        layers.append({"name": name, "lay": lay, "B": B, "L": L, "Cx": ly.Cx, "Cy": ly.Cy,
                       "Rx": info.Rx, "Ry": info.Ry, "x": up(d["x"]), "gy": up(d["gy"]),
                       "w": up(W.to_io(W.make_w(wl, lname), "bf16")),
                       "xhat": torch.empty((B, info.Rx, ly.Cx), dtype=torch.bfloat16, device=dev),
                       "gw": torch.empty((ly.Cy, ly.Cx), dtype=torch.bfloat16, device=dev),
                       "gx": torch.empty((B, L, ly.Cx), dtype=torch.bfloat16, device=dev)})
        del d
    st = torch.cuda.current_stream()

    def ev_time(fn, reps=50):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0.record(st)
        for _ in range(reps):
            fn()
        e1.record(st)
        e1.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3  # us

    def instant(c):
        c["lay"].compress_fwd(c["x"], c["B"], c["xhat"])
        c["lay"].backward(c["xhat"], c["gy"], c["w"], c["B"], c["gw"], c["gx"])

    def exact(c):
        gy2 = c["gy"].view(-1, c["Cy"])
        torch.mm(gy2, c["w"], out=c["gx"].view(-1, c["Cx"]))
        torch.mm(gy2.t(), c["x"].view(-1, c["Cx"]), out=c["gw"])

    out_layers, tot = [], {"instant_us": 0.0, "exact_us": 0.0, "flops_vanilla": 0, "flops_lowrank": 0,
                           "act_bytes_exact": 0, "act_bytes_instant": 0}
    for c in layers:
        ti, te = ev_time(lambda: instant(c)), ev_time(lambda: exact(c))
        B, L, Cx, Cy, Rx, Ry = c["B"], c["L"], c["Cx"], c["Cy"], c["Rx"], c["Ry"]
        fv = B * 4 * L * Cx * Cy
        fl = B * 2 * (Rx + Ry) * (Cx * Cy + L * Cx + L * Cy)
        ax, ah = 2 * B * L * Cx, 2 * B * Rx * Cx
        out_layers.append({"layer": c["name"], "Cx": Cx, "Cy": Cy, "Rx": Rx, "Ry": Ry, "instant_us": ti,
                           "exact_us": te, "speedup": te / ti, "flop_ratio": fv / fl, "activation_ratio": ax / ah})
        for key, v in (("instant_us", ti), ("exact_us", te), ("flops_vanilla", fv), ("flops_lowrank", fl),
                       ("act_bytes_exact", ax), ("act_bytes_instant", ah)):
            tot[key] += v
    both = lambda: [instant(c) for c in layers]  # noqa: E731
    t_block = ev_time(both)
    B, L = layers[0]["B"], layers[0]["L"]
    res = {"metric": "BERT-base encoder layer, all linear layers: low-rank backward time (compression "
                     "included) against the exact backward",
           "value": B * L / (t_block * 1e-6), "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "BERT-base encoder layer linears Q, K, V, O (768->768), FFN up (768->3072), "
                                  "down (3072->768); B=32 L=512; calibrated on 4 synthetic batches per layer",
                      "global_batch": B, "seq_len": L},
           "block": {"instant_us": t_block, "instant_us_sum_of_layers": tot["instant_us"],
                     "exact_us": tot["exact_us"], "speedup": tot["exact_us"] / t_block,
                     "flop_ratio_formula": tot["flops_vanilla"] / tot["flops_lowrank"],
                     "activation_memory_ratio": tot["act_bytes_exact"] / tot["act_bytes_instant"]},
           "layers": out_layers}
    print(json.dumps(res), flush=True)
    torch.cuda.synchronize()
    for c in layers:
        c["lay"].close()


def cpu_baseline(wl, nsample):
    """The CPU oracle (float64 numpy), as it stands, timed on a bounded sample of the same
    workload: its low-rank backward (a5-a8, the metric's work) on `nsample` samples of one
    batch, scaled to tokens/s; and, for context, its whole per-step schedule."""
    import numpy as np  # noqa: F401

    import oracle as O
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    d = W.make_layer_batch(wl, 0, 0, with_w=True)
    xs, gys, w = d["x64"][:nsample], d["gy64"][:nsample], d["w64"]
    cal = O.calibrate([d["x64"]], [d["gy64"]], wl.eps, wl.p, O.COMP_PAPER)
    P, Q = cal["x"]["P"], cal["g"]["P"]
    xh = O.compress(P, xs)
    t0 = time.perf_counter()
    O.backward(P, Q, xh, gys, w)
    t_bwd = (time.perf_counter() - t0) / nsample           # per sample
    t0 = time.perf_counter()
    O.compress(P, xs)
    t_cmp = (time.perf_counter() - t0) / nsample           # per sample
    t0 = time.perf_counter()
    acc = O.Accumulator(wl.L)
    acc.add(xs)
    acc.add(gys)
    t_acc = (time.perf_counter() - t0) / nsample            # per sample, both tensors
    t0 = time.perf_counter()
    O.calibrate_side(cal["C_X"], wl.eps, wl.p, O.COMP_PAPER, wl.L)
    O.calibrate_side(cal["C_G"], wl.eps, wl.p, O.COMP_PAPER, wl.L)
    t_fin = time.perf_counter() - t0                        # per finalize
    per_step = wl.B * (t_cmp + t_bwd) + (wl.n_cal / wl.n_t) * wl.B * t_acc + t_fin / wl.n_t
    return {"value": wl.L / t_bwd, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"the oracle's low-rank backward (P g_y, Q g_y, g_w, g_hat_x, expansion) on {nsample} of "
                      f"{wl.B} samples of one batch: tokens/s = {nsample}*L / time",
            "schedule_tokens_per_s": wl.B * wl.L / per_step,
            "schedule_sample": f"per step B*t_sample(compress + backward) + (N_cal/N_t)*B*t_sample(statistics) "
                               f"+ t_finalize/N_t, with one full finalize (eigh of both {wl.L}x{wl.L} statistics)"}


if __name__ == "__main__":
    main()
