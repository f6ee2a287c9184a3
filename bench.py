"""Throughput of the INSTANT low-rank backward on one MI355X.

Workload: BERT-base attention-projection-shaped linear y = x w^T, bf16 I/O with
float32 accumulation, B=32 sequences of L=512 tokens, Cx=Cy=768, eps=0.95, p=2,
statistics over N_cal=16 batches, recalibration every N_t=100 steps (shapes of the
BERT layers the INSTANT notes evaluate; synthetic token-low-rank data, see
workloads/).

One step is one training step's share of the method on one batch, on the notes'
schedule (section 整体框架): every step compresses x (x_hat = P x) and runs the
low-rank backward (g_w, g_x); the first N_cal steps of every N_t-step window also
accumulate the statistics, and the last of them finalizes (eigen-decomposition,
truncation, new P and Q). So every kernel of the path runs inside the timed region,
with the calibration amortised exactly as the schedule amortises it.

Prints one JSON line; `value` is tokens/s = steps * B * L / wall time.
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
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "proj_bert_attn_traffic.json")


def measured_traffic():
    """HBM bytes per forward-compression launch from the recorded rocprofv3 counters
    (FETCH_SIZE and WRITE_SIZE scaled by a copy kernel of known size), or None when the
    kernel sources changed since the counters were taken."""
    import hashlib
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["sources_sha256"]:
            return None
        return rec["traffic_bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="bert_attn",
                    help="bert_attn (the headline line); bert_block (every linear layer of a BERT-base "
                         "encoder layer: its low-rank backward against the exact one); or one layer of "
                         "tiny, bert_ffn, effformer, llm_mlp run through the same step loop")
    ap.add_argument("--layer", default="0", help="layer of a two-layer workload (up or down)")
    ap.add_argument("--batches", type=int, default=None,
                    help="distinct resident batches cycled through (default 32: more than N_cal, so "
                         "consecutive calibration windows see different statistics; N_cal for llm_mlp, "
                         "whose batches take seconds each to generate)")
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
    # The finalizing calls inside the timed loop are bracketed by HIP events on the side
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
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # every successful finalize publishes one new generation of projections; an asynchronous
    # one that fails is only seen here (the old projections stay in use)
    gen0 = lay.query()[1].generation
    t0 = time.perf_counter()
    for i in range(args.warmup, args.warmup + args.steps):
        step(i, timed=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fin_loop = [a.elapsed_time(b) * 1e-3 for a, b in fin_events]
    _, info = lay.query()
    published = info.generation - gen0
    if published != len(fin_events):
        print(f"warning: {len(fin_events) - published} of {len(fin_events)} finalizes in the timed loop "
              "published no projections", file=sys.stderr)
    Rx, Ry = info.Rx, info.Ry

    # ---- per-part timing with HIP events on the launch stream, right after the timed loop.
    # A pair of events around one launch inside the loop would add the markers' dispatch
    # latency (about 3.5 us) to a 7.5 us kernel, so each part is timed over a run of
    # consecutive launches on the same stream and resident batches.
    st = torch.cuda.current_stream()

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

    reps = 200
    t_fwd = ev_time(lambda r: lay.compress_fwd(xs[r % nb], B, xhat), reps)
    t_bwd = ev_time(lambda r: lay.backward(xhat, gys[r % nb], w, B, gw, gx), reps)
    t_acc = ev_time(lambda r: lay.calibrate(xs[r % nb], gys[r % nb], B, finalize=False), 50)
    # host cost of enqueueing one plain step (compress + backward), measured from a drained
    # queue: when it exceeds the GPU time of a step, the loop above is bound by the host
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    for r in range(50):
        lay.compress_fwd(xs[r % nb], B, xhat)
        lay.backward(xhat, gys[r % nb], w, B, gw, gx)
    t_issue = (time.perf_counter() - h0) / 50
    # one full finalize (eigen-decomposition of both statistics, truncation, publish)
    torch.cuda.synchronize()
    tf0 = time.perf_counter()
    s = lay.calibrate(None, None, 0, finalize=True)
    torch.cuda.synchronize()
    t_fin = time.perf_counter() - tf0
    _, info2 = lay.query()

    es = 2 if wl.dtype == "bf16" else 4
    bytes_fwd = es * (B * L * Cx + B * Rx * Cx)
    bytes_bwd = es * (B * L * Cy + B * Rx * Cx + 2 * Cx * Cy + B * L * Cx)
    flops_bwd = B * (2 * (Rx + Ry) * L * Cy + 2 * (Rx + Ry) * Cx * Cy + 2 * Ry * L * Cx)
    # statistics: the upper triangle of both L x L sums per batch (the mirror earns no credit)
    flops_acc = L * (L + 1) * B * (Cx + Cy)
    gbs_fwd = bytes_fwd / t_fwd / 1e9

    headline = wl.name == "bert_attn"
    ms_per_step = wall / args.steps * 1e3
    tokens = args.steps * B * L
    value = tokens / wall

    out = {
        "metric": ("low-rank backward tokens/s + achieved HBM GB/s (% peak), BERT-base linear" if headline else
                   f"low-rank backward tokens/s + achieved HBM GB/s (% peak), {wl.name} linear"),
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"{WORKLOAD_NAMES.get(wl.name, wl.name)} linear{'' if len(wl.layers) == 1 else ' (' + ly.name + ')'}, "
                               f"B={B} L={L} Cx={Cx} Cy={Cy}, "
                               f"eps={wl.eps} p={wl.p} N_cal={wl.n_cal} N_t={wl.n_t}",
                   "global_batch": B, "seq_len": L, "parallelism": "single GPU",
                   "step": "compress + low-rank backward every step; statistics on the first N_cal steps of "
                           "each N_t window; eigen-decomposition + truncation once per window",
                   "streams": "statistics and finalize on a side stream" if not args.one_stream else "one stream",
                   "finalize": "synchronous" if args.sync_finalize else
                               "asynchronous (new projections from the first forward after it completes)",
                   "Rx": Rx, "Ry": Ry, "kx": info.kx, "ky": info.ky},
        "parts": {
            "compress_fwd_us": t_fwd * 1e6, "compress_fwd_GBs": gbs_fwd,
            "backward_us": t_bwd * 1e6, "backward_GBs": bytes_bwd / t_bwd / 1e9,
            "backward_pct_hbm_peak": 100.0 * bytes_bwd / t_bwd / 1e9 / HBM_PEAK_GBS,
            "backward_tokens_per_s": B * L / t_bwd, "backward_TFLOPs": flops_bwd / t_bwd / 1e12,
            "statistics_per_batch_us": t_acc * 1e6,
            "statistics_TFLOPs": flops_acc / t_acc / 1e12,
            "statistics_pct_mfma_bf16_peak" if wl.dtype == "bf16" else "statistics_pct_mfma_fp32_peak":
                100.0 * flops_acc / t_acc / 1e12 / (MFMA_BF16_PEAK_TFLOPS if wl.dtype == "bf16" else
                                                    MFMA_FP32_PEAK_TFLOPS),
            "statistics_GBs": es * B * L * (Cx + Cy) / t_acc / 1e9,
            "eigensolver": solver_used,
            "cold_finalize_ms": t_cold * 1e3,
            "finalize_ms": t_fin * 1e3,
            "finalize_in_loop_ms": (sum(fin_loop) / len(fin_loop) * 1e3) if fin_loop else None,
            "finalizes_in_loop": len(fin_loop), "host_enqueue_us_per_plain_step": t_issue * 1e6, "jacobi_sweeps": [info2.sweeps_x, info2.sweeps_g],
            "finalize_status": rcb.instant_status_str(s),
            "finalizes_published": f"{published}/{len(fin_events)}",
        },
        "roofline": {"kernel": "proj (forward compression x_hat = P x)", "bound": "hbm",
                     "achieved": gbs_fwd, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs_fwd / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "launch_us": t_fwd * 1e6, "launches_timed": reps,
                     "algorithmic_bytes_per_launch": bytes_fwd},
    }

    if not args.no_cpu_baseline and headline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample)
    print(json.dumps(out), flush=True)


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


def cpu_baseline(wl, nsample):
    """The CPU oracle (float64 numpy) timed on a bounded sample of the same step."""
    import numpy as np

    import oracle as O
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    ly = wl.layer(0)
    d = W.make_layer_batch(wl, 0, 0, with_w=True)
    xs, gys, w = d["x64"][:nsample], d["gy64"][:nsample], d["w64"]
    cal = O.calibrate([d["x64"]], [d["gy64"]], wl.eps, wl.p, O.COMP_PAPER)
    P, Q = cal["x"]["P"], cal["g"]["P"]
    t0 = time.perf_counter()
    xh = O.compress(P, xs)
    O.backward(P, Q, xh, gys, w)
    t_cb = (time.perf_counter() - t0) / nsample            # per sample
    t0 = time.perf_counter()
    acc = O.Accumulator(wl.L)
    acc.add(xs)
    acc.add(gys)
    t_acc = (time.perf_counter() - t0) / nsample            # per sample, both tensors
    t0 = time.perf_counter()
    O.calibrate_side(cal["C_X"], wl.eps, wl.p, O.COMP_PAPER, wl.L)
    O.calibrate_side(cal["C_G"], wl.eps, wl.p, O.COMP_PAPER, wl.L)
    t_fin = time.perf_counter() - t0                        # per finalize
    per_step = wl.B * t_cb + (wl.n_cal / wl.n_t) * wl.B * t_acc + t_fin / wl.n_t
    return {"value": wl.B * wl.L / per_step, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{nsample} of {wl.B} samples of one batch for compress+backward and the statistics, "
                      f"one full finalize (eigh of both {wl.L}x{wl.L} statistics); per-step time = "
                      f"B*t_sample(compress+backward) + (N_cal/N_t)*B*t_sample(statistics) + t_finalize/N_t",
            "seconds_per_step": per_step}


if __name__ == "__main__":
    main()
