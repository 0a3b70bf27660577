"""Bench of the quantized routed-expert MoE layer on one MI355X.

Headline (one JSON line on stdout): decode tokens/s of one MoE layer at the pages'
routing shape (d_model 2048, 512 routed experts, top-10 + 1 shared, expert FFN width
512, int4 group-32 weights, one token per call).  A step is the whole hot path for one
token: router + top-k, shared expert, grouping, routed experts, combine.  Inputs are
resident in HBM before timing; the step sequence is captured in a HIP graph and replayed.
To keep the 256 MB Infinity Cache from serving the weights, steps rotate over
``--copies`` distinct copies of the layer (a different token per copy).

Also reported in the same line:
  roofline      the routed expert FFN call of a decode step (the HBM-bound hot spot):
                algorithmic bytes (selected experts' packed weights + scales, activations
                in, pair rows out) / its event-timed average duration vs 8 TB/s
  cpu_baseline  the CPU oracle on a bounded sample of the same workload
  prefill       8192-token prefill through one layer (Zipf routing): tokens/s and the
                grouped GEMM's MFMA utilisation (useful flops / time / 2.5 PFLOP/s)
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=640)
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--copies", type=int, default=32,
                   help="distinct layer copies rotated through (defeats the 256 MB MALL)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--eager", action="store_true", help="no graph capture (for profilers)")
    return p.parse_args()


def clone_layer(lay):
    import copy
    c = copy.copy(lay)
    c.router = copy.copy(lay.router)
    c.router.w = lay.router.w.clone()
    c.router.scale = None if lay.router.scale is None else lay.router.scale.clone()
    c.router.bias = None if lay.router.bias is None else lay.router.bias.clone()
    for name in ("routed", "shared"):
        ex = copy.copy(getattr(lay, name))
        for a in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down"):
            setattr(ex, a, getattr(ex, a).clone())
        setattr(c, name, ex)
    return c


def expert_bytes(ex):
    return ex.nbytes() // ex.E


def time_graph(fn, reps, warm=2):
    """Capture fn() in a graph, replay; returns ms per replay (HIP events)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                  # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / reps, g


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only (--gpus %d requested); the layer "
              "shards by tokens with no communication, see DESIGN.md" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import quantized_sparse_moe_router_amd as moe
    import synth

    torch.cuda.set_device(0)
    w = synth.WORKLOADS["decode_d2048_e512_top10_t1"]
    L = max(1, args.copies)
    base = synth.make_layer(w, seed=0, device="cuda")
    copies = [base] + [clone_layer(base) for _ in range(L - 1)]
    toks = synth.make_tokens(w, T=L, seed=0, device="cuda")
    xs = [toks[i:i + 1] for i in range(L)]
    layers = [moe.MoeLayer(c.router, c.routed, c.shared, w.k, 1) for c in copies]
    torch.cuda.synchronize()

    def step_all():
        for i in range(L):
            layers[i].forward(xs[i])

    # eager pass: fills every layer's buffers and checks for device errors
    step_all()
    torch.cuda.synchronize()
    moe.moe_check_device_error()

    reps = max(1, -(-args.steps // L))
    warm = max(1, -(-args.warmup // L))
    steps = reps * L
    if args.eager:
        for _ in range(warm):
            step_all()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            step_all()
        t1.record()
        torch.cuda.synchronize()
        ms_replay = t0.elapsed_time(t1) / reps
    else:
        ms_replay, _ = time_graph(step_all, reps, warm)
    ms_step = ms_replay / L
    tok_s = 1000.0 / ms_step

    # ---- roofline: the routed expert FFN call (selected experts' weights streamed once)
    E_b = expert_bytes(base.routed)
    alg_bytes_ffn = w.k * E_b + w.d * 2 + w.k * w.d * 2

    def ffn_all():
        for i in range(L):
            lay = layers[i]
            moe.moe_expert_ffn(lay.routed, xs[i], 1, w.k, lay.ids, lay.offsets,
                               lay.sorted_pairs, lay.y_pairs, lay.ws_ffn)

    ffn_reps = max(4, reps // 2)
    ms_ffn = time_graph(ffn_all, ffn_reps)[0] / L if not args.eager else None
    if ms_ffn is None:
        ffn_all()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(ffn_reps):
            ffn_all()
        t1.record()
        torch.cuda.synchronize()
        ms_ffn = t0.elapsed_time(t1) / (ffn_reps * L)
    achieved = alg_bytes_ffn / (ms_ffn * 1e-3) / 1e9
    alg_bytes_step = (base.router.w.numel() * base.router.w.element_size()
                      + (w.k + 1) * E_b + 2 * w.d * 2)

    line = {
        "metric": "moe_layer_decode_tokens_per_s",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm * L,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4-weights/bf16-act/fp32-acc",
        "data": "synthetic (seeded N(0,0.02) weights quantised int4 g32, N(0,1) bf16 tokens)",
        "config": {"workload": "decode_d2048_e512_top10_t1", "d_model": w.d, "experts": w.E,
                   "top_k": w.k, "shared_experts": 1, "d_ff": w.F, "tokens_per_step": 1,
                   "layer_copies_rotated": L, "graph": not args.eager,
                   "step_weight_stream_GBps": round(alg_bytes_step / (ms_step * 1e-3) / 1e9, 1),
                   "alg_bytes_per_step": alg_bytes_step},
        "roofline": {"bound": "hbm", "kernel": "routed expert FFN call (gate/up+SwiGLU, down)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "alg_bytes_per_launch": alg_bytes_ffn,
                     "avg_launch_us": round(ms_ffn * 1e3, 3)},
    }

    # ---- prefill: 8192 tokens, Zipf routing, one layer
    if not args.no_prefill:
        line["prefill"] = prefill_bench(moe, synth, np, torch)

    # ---- CPU oracle on a bounded sample of the decode workload
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(base, toks, w, args.cpu_seconds)

    print(json.dumps(line), flush=True)


def prefill_bench(moe, synth, np, torch):
    w = synth.WORKLOADS["prefill_8192_zipf"]
    lay = synth.make_layer(w, seed=0, device="cuda")
    x = synth.make_tokens(w, seed=0, device="cuda")
    layer = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, w.T)
    layer.forward(x)
    torch.cuda.synchronize()
    moe.moe_check_device_error()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    reps = 10
    t0, t1 = ev(), ev()
    t0.record()
    for _ in range(reps):
        layer.forward(x)
    t1.record()
    torch.cuda.synchronize()
    ms_layer = t0.elapsed_time(t1) / reps
    # grouped GEMM (routed experts): useful flops 6 * pairs * d * F
    P = w.T * w.k
    t0, t1 = ev(), ev()
    t0.record()
    for _ in range(reps):
        moe.moe_expert_ffn(layer.routed, x, w.T, w.k, layer.ids, layer.offsets,
                           layer.sorted_pairs, layer.y_pairs, layer.ws_ffn)
    t1.record()
    torch.cuda.synchronize()
    ms_gemm = t0.elapsed_time(t1) / reps
    flops = 6.0 * P * w.d * w.F
    counts = np.diff(layer.offsets.cpu().numpy())
    return {"workload": "prefill_8192_zipf", "tokens": w.T,
            "tokens_per_s": round(w.T / (ms_layer * 1e-3), 1),
            "ms_layer": round(ms_layer, 4), "ms_routed_grouped_gemm": round(ms_gemm, 4),
            "routed_gemm_tflops": round(flops / (ms_gemm * 1e-3) / 1e12, 1),
            "mfma_util": round(flops / (ms_gemm * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "active_experts": int((counts > 0).sum()), "max_rows_per_expert": int(counts.max())}


def cpu_baseline(base, toks, w, seconds):
    import numpy as np

    import oracle
    from synth import inputs as si
    r_h, ex_h, sh_h = base.router.host(), base.routed.host(), base.shared.host()
    x_h = si.bits16(toks)
    n_tok = x_h.shape[0]
    # calibrate on a few tokens, then run a sample sized for ~`seconds`
    threads = oracle.num_threads()
    n_cal = max(1, min(threads, n_tok))
    t = time.perf_counter()
    oracle.layer_tokens(r_h, ex_h, sh_h, x_h, np.arange(n_cal, dtype=np.int32), w.k)
    per = (time.perf_counter() - t) / n_cal
    n = int(max(8, min(4096, seconds / max(per, 1e-6))))
    tok_idx = (np.arange(n) % n_tok).astype(np.int32)
    t = time.perf_counter()
    oracle.layer_tokens(r_h, ex_h, sh_h, x_h, tok_idx, w.k)
    dt = time.perf_counter() - t
    return {"value": round(n / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d single-token decode calls of the same layer (fp64 oracle, OpenMP "
                      "over tokens), %.1f s" % (n, dt)}


if __name__ == "__main__":
    main()
