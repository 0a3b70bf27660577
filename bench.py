"""Bench of the quantized routed-expert MoE layer on one MI355X.

Headline (one JSON line on stdout): decode tokens/s of one MoE layer at the pages'
routing shape (d_model 2048, 512 routed experts, top-10 + 1 shared, expert FFN width
512, int4 group-32 weights, one token per call).  A step is the whole hot path for one
token: router + top-k, shared expert, routed experts, combine -- moe_layer_decode, which
is checked bit for bit against the four-call composition before timing (whose time per
step is reported too).  Inputs are resident in HBM before timing; the step sequence is
captured in a HIP graph and replayed.
To keep the 256 MB Infinity Cache from serving the weights, steps rotate over
``--copies`` distinct copies of the layer (a different token per copy).  Before the warm-up
a graph of the timed region's shape is replayed once on other copies (the process's first
replay of such a graph costs ~24 us more, once), then every copy is read again.

Also reported in the same line:
  roofline        the expert kernels of a decode step (moe_experts_decode: gate/up kernel then
                  down + combine kernel): algorithmic bytes (10 routed + 1 shared expert's
                  packed weights and scales, activations in and out) / their event-timed
                  average duration vs 8 TB/s
  decode_batches  1..128 tokens per call (several decode slots, or drafts verified together)
  decode_batches_zipf  16..128 tokens per call with Zipf-skewed routing (hot experts)
  decode_low_bit  the decode layer with int4 / int3 / int2 experts at 1, 16 and 64 tokens
  mall_residency  what the 256 MB cache in front of HBM gives: stream reads cold and warm,
                  a Zipf-routed decode cycling over 1..32 layer copies
  decode_sweep    48 distinct normed, gated blocks chained, 1 and 4 tokens per step
  prefill         8192-token prefill through one layer (Zipf routing), and 32768 tokens with
                  mixed formats: tokens/s and the grouped GEMM's MFMA utilisation
  achievable      measured ceilings of this GPU (stream read, MFMA loop, vendor GEMM)
  cpu_baseline    the CPU oracle on a bounded sample of the same workload
"""
import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0

# Counter-measured memory traffic of moe_experts_decode, taken by two rocprofv3 --pmc runs
# (FETCH_SIZE, WRITE_SIZE) and scaled by the same counters on a copy of known size; the
# summary records a digest of the kernel sources it was measured on.
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "decode_experts_traffic.md")
TRAFFIC_SOURCES = ["decode.hip", "gemv_common.h", "topk_common.h", "combine_common.h",
                   "moe_common.h"]


def kernel_source_digest():
    """Digest of the kernel sources with comments and whitespace removed, so that only a
    change of the code itself marks the counter summary as stale."""
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "quantized_sparse_moe_router_amd", "csrc", f)) as fh:
            code = fh.read()
        code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """Bytes per moe_experts_decode call from the committed counter summary, or None when
    it is missing or was taken on other kernel sources."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    vals = dict(re.findall(r"^(traffic_bytes_per_launch|source_digest): *(\S+)$", text, re.M))
    if vals.get("source_digest") != kernel_source_digest():
        return None
    return int(vals["traffic_bytes_per_launch"])


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=640)
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--reps", type=int, default=20,
                   help="repetitions (at least 20) of each timed region for median and min")
    p.add_argument("--copies", type=int, default=32,
                   help="distinct layer copies rotated through (defeats the 256 MB MALL)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-sweep", action="store_true", help="skip the 48-layer decode sweep")
    p.add_argument("--no-mall", action="store_true",
                   help="skip the cache residency leg (stream reads, Zipf decode over copies)")
    p.add_argument("--no-low-bit", action="store_true",
                   help="skip the int3 / int2 expert decode leg")
    p.add_argument("--no-batches", action="store_true",
                   help="skip the decode batch sizes 1..128")
    p.add_argument("--batch-sizes", default="1,4,6,8,16,32,64,96,128",
                   help="tokens per call of the decode-batches leg (comma-separated)")
    p.add_argument("--zipf-batch-sizes", default="16,32,64,96,128",
                   help="tokens per call of the Zipf-routed decode-batches leg "
                        "(comma-separated; empty skips the leg)")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--eager", action="store_true", help="no graph capture (for profilers)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only copy 256 MiB device to device 8 times (calibrates the memory "
                        "traffic counters against a transfer of known size), then exit")
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


def capture(fn, eager=True):
    """Capture fn() into a HIP graph (after one eager pass on a side stream, unless the
    calls have run eagerly before)."""
    import torch
    if eager:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def timed_replay(g, lead_cycles=2_000_000):
    """GPU time (ms) of one replay of g between two events on the current stream.  A GPU
    sleep is queued ahead of the first event so that the host has enqueued the replay
    before the GPU reaches it: the events then bracket GPU work only."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(lead_cycles)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def time_graph(fn, reps, warm=2):
    """Capture fn() in a graph; returns (median ms per replay over `reps` replays, each
    timed on its own, min, graph)."""
    import statistics
    g = capture(fn)
    for _ in range(warm):
        g.replay()
    ts = [timed_replay(g) for _ in range(reps)]
    return statistics.median(ts), min(ts), g


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU (--gpus %d requested): the layer shards by tokens "
              "with no communication between GPUs, so one GPU's throughput is the measure"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_calibration:
        torch.cuda.set_device(0)
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel(), "copies": 8}), flush=True)
        return

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
            layers[i].decode(xs[i])

    def step_all_calls():
        for i in range(L):
            layers[i].forward(xs[i])

    K, W = max(1, args.steps), max(0, args.warmup)
    REPS = max(20, args.reps)

    # eager passes: fill every layer's buffers, check for device errors, and check that the
    # two-launch layer equals the four-call composition bit for bit
    step_all_calls()
    ref = [lay.out[:1].clone() for lay in layers]
    step_all()
    torch.cuda.synchronize()
    moe.moe_check_device_error()
    for i in range(L):
        if not torch.equal(layers[i].out[:1].view(torch.int16), ref[i].view(torch.int16)):
            raise SystemExit("bench.py: moe_layer_decode differs from the four calls")


    def steps_fn(first, n, call):
        def fn():
            for i in range(first, first + n):
                call(i % L)
        return fn

    # The first replay of a graph of K steps in a process carries a one-time cost of the
    # graph runtime (measured 24 us at K = 20 in fresh processes, whichever copies it reads;
    # not a matter of clocks: a 10 ms GPU sleep ahead of the timed region leaves it).  A
    # graph of the same shape on the copies after the timed ones is replayed once here (and
    # kept until the timing is done), then every copy is read again (760 MB, three times the
    # 256 MB cache), so the timed copies are as cold as before.
    g_pre = None
    if not args.eager:
        g_pre = capture(steps_fn(W + K, K, lambda i: layers[i].decode(xs[i])), eager=False)
        g_pre.replay()
        torch.cuda.synchronize()
        step_all()
        torch.cuda.synchronize()

    if args.eager:
        def run_region(first, n, call):
            import statistics
            steps_fn(first, n, call)()
            torch.cuda.synchronize()
            ts = []
            for _ in range(REPS):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                steps_fn(first, n, call)()
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b))
            return statistics.median(ts), min(ts)
    else:
        def run_region(first, n, call):
            med, mn, _ = time_graph(steps_fn(first, n, call), REPS)
            return med, mn

    decode_call = lambda i: layers[i].decode(xs[i])          # noqa: E731
    # the headline: W untimed warm-up steps (one graph), then exactly K timed steps (one
    # graph, its first replay), continuing the rotation over the copies.  Every copy ran
    # eagerly above, so the graphs are captured without another eager pass: the timed
    # steps' copies were last read before the warm-up and the checks' later copies, more
    # than the 256 MB cache holds.
    if args.eager:
        steps_fn(0, W, decode_call)()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(2_000_000)
        a.record()
        steps_fn(W, K, decode_call)()
        b.record()
        torch.cuda.synchronize()
        ms_region = a.elapsed_time(b)
        g_k = None
    else:
        g_w = capture(steps_fn(0, W, decode_call), eager=False) if W > 0 else None
        g_k = capture(steps_fn(W, K, decode_call), eager=False)
        torch.cuda.synchronize()
        if g_w is not None:
            g_w.replay()
        ms_region = timed_replay(g_k)
    ms_step = ms_region / K
    tok_s = 1000.0 / ms_step
    # the same K-step region repeated REPS times, each replay timed on its own
    if g_k is not None:
        import statistics
        rep_ms = [timed_replay(g_k) / K for _ in range(REPS)]
        ms_med, ms_min = statistics.median(rep_ms), min(rep_ms)
    else:
        ms_med, ms_min = run_region(W, K, decode_call)
        ms_med, ms_min = ms_med / K, ms_min / K
    ms_calls, _ = run_region(0, L, lambda i: layers[i].forward(xs[i]))
    ms_step_calls = ms_calls / L

    # ---- roofline: the expert kernels of the decode step (moe_experts_decode: the routed
    # experts and the shared one streamed once, SwiGLU, combine) -- two launches per call
    E_b = expert_bytes(base.routed)
    alg_bytes_exp = (w.k + 1) * E_b + 2 * w.d * 2
    ms_exp_med, ms_exp_min = run_region(0, L, lambda i: layers[i].experts_decode(xs[i]))
    ms_exp = ms_exp_med / L
    achieved = alg_bytes_exp / (ms_exp * 1e-3) / 1e9
    alg_bytes_step = (base.router.w.numel() * base.router.w.element_size()
                      + (w.k + 1) * E_b + 2 * w.d * 2)
    # per-leg split of the step, event-timed: the router alone (moe_route at one token:
    # logits and selection in one launch) and the expert side (moe_experts_decode)
    ms_route, _ = run_region(0, L, lambda i: layers[i].route_only(xs[i]))
    ms_route /= L

    line = {
        "metric": "moe_layer_decode_tokens_per_s",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4-weights/bf16-act/fp32-acc",
        "data": "synthetic (seeded N(0,0.02) weights quantised int4 g32, N(0,1) bf16 tokens)",
        "config": {"workload": "decode_d2048_e512_top10_t1", "d_model": w.d, "experts": w.E,
                   "top_k": w.k, "shared_experts": 1, "d_ff": w.F, "tokens_per_step": 1,
                   "layer_copies_rotated": L, "graph": not args.eager,
                   "entry_point": "moe_layer_decode",
                   "step_weight_stream_GBps": round(alg_bytes_step / (ms_step * 1e-3) / 1e9, 1),
                   "alg_bytes_per_step": alg_bytes_step,
                   "ms_per_step_median": round(ms_med, 5), "ms_per_step_min": round(ms_min, 5),
                   "repetitions": REPS,
                   "ms_per_step_four_calls": round(ms_step_calls, 5),
                   "step_split_us": {
                       "moe_route_one_launch": round(ms_route * 1e3, 3),
                       "moe_experts_decode": round(ms_exp * 1e3, 3),
                       "step": round(ms_med * 1e3, 3)}},
        "roofline": {"bound": "hbm",
                     "kernel": "decode_gateup_kernel + decode_down_kernel (moe_experts_decode:"
                               " 10 routed + 1 shared expert FFN and combine)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "alg_bytes_per_launch": alg_bytes_exp,
                     "avg_launch_us": round(ms_exp * 1e3, 3),
                     "min_launch_us": round(ms_exp_min / L * 1e3, 3)},
    }

    # ---- decode batches: 1 .. 128 tokens per call through the layer (several decode slots
    # or drafts verified together), on the same rotated copies
    if not args.no_batches:
        line["decode_batches"] = decode_batches(
            moe, synth, np, torch, copies, w, args,
            Ts=tuple(int(t) for t in args.batch_sizes.split(",") if t.strip()))
        torch.cuda.empty_cache()
        # the same with the router's bias skewing the routing (Zipf, s = 1.1): fewer distinct
        # experts, some chosen by many of the call's tokens
        zts = tuple(int(t) for t in args.zipf_batch_sizes.split(",") if t.strip())
        if zts:
            zbase = synth.make_layer(w, seed=0, device="cuda", bias="zipf")
            zcopies = [zbase] + [clone_layer(zbase) for _ in range(L - 1)]
            line["decode_batches_zipf"] = decode_batches(
                moe, synth, np, torch, zcopies, w, args, Ts=zts)
            line["decode_batches_zipf"]["routing"] = "zipf s=1.1 (router bias)"
            del zbase, zcopies
            torch.cuda.empty_cache()

    # ---- lower-bit expert codecs: the same decode step with every expert at 3 or 2 bits
    if not args.no_low_bit:
        line["decode_low_bit"] = decode_low_bit(moe, synth, np, torch, copies, w, args)
        torch.cuda.empty_cache()

    # ---- what the 256 MB cache in front of HBM gives the decode step under Zipf routing
    if not args.no_mall:
        line["mall_residency"] = mall_residency(moe, synth, np, torch, args)
        torch.cuda.empty_cache()

    # ---- 48 chained layers, 1 and 4 tokens per step
    if not args.no_sweep:
        line["decode_sweep"] = decode_sweep(moe, synth, np, torch, args)
        torch.cuda.empty_cache()

    # ---- prefill: 8192 tokens Zipf; 32768 tokens mixed precision, Zipf and uniform
    if not args.no_prefill:
        line["prefill"] = prefill_bench(moe, synth, np, torch, "prefill_8192_zipf", None)
        torch.cuda.empty_cache()
        line["prefill_32k"] = [prefill_bench(moe, synth, np, torch, "prefill_32768_mixed", b)
                               for b in ("zipf", "none")]

    # ---- what this chip reaches on plain work, next to the spec peaks: the rates above as
    # fractions of the measured stream read and MFMA loop too
    ach = achievable_peaks(torch)
    line["achievable"] = ach
    line["roofline"]["frac_of_measured_stream"] = round(
        line["roofline"]["achieved"] / ach["hbm_read_GBps_stream_kernel"], 4)
    for p in ([line["prefill"]] + line["prefill_32k"]) if "prefill" in line else []:
        p["mfma_util_of_measured_loop"] = round(
            p["routed_gemm_tflops"] / ach["mfma_bf16_tflops_loop"], 4)

    # ---- CPU oracle on a bounded sample of the decode workload
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(base, toks, w, args.cpu_seconds)

    print(json.dumps(line), flush=True)


def decode_low_bit(moe, synth, np, torch, copies4, w4, args, Ts=(1, 16, 64)):
    """The decode layer (d 2048, 512 experts, top-10 + shared) with every expert in the int4,
    int3 or int2 group-32 codec, T = 1 (moe_layer_decode, two launches after the router)
    and T = 16, 64 (the four calls: GEMV in sorted mode), each format on its own rotated
    layer copies.  Weight-stream bytes: router + (distinct routed experts + shared) x the
    expert bytes of the format + activations; layer_weight_bytes = what one layer holds."""
    out = {"workload": "decode_d2048_e512_top10, experts int4 / int3 / int2 g32",
           "copies_rotated": len(copies4)}
    for name in ("decode_d2048_e512_top10_t1", "int3_d2048_e512_top10",
                 "int2_d2048_e512_top10"):
        w = synth.WORKLOADS[name]
        if name == "decode_d2048_e512_top10_t1":
            copies = copies4
        else:
            base = synth.make_layer(w, seed=0, device="cuda")
            copies = [base] + [clone_layer(base) for _ in range(len(copies4) - 1)]
        n_cp = len(copies)
        c0 = copies[0]
        E_b = expert_bytes(c0.routed)
        r_b = c0.router.w.numel() * c0.router.w.element_size()
        row = {"expert_bytes": int(E_b),
               "layer_weight_bytes": int(c0.routed.nbytes() + c0.shared.nbytes() + r_b)}
        for T in Ts:
            mls = [moe.MoeLayer(c.router, c.routed, c.shared, w.k, T) for c in copies]
            xs = [synth.make_tokens(w, T=T, seed=200 + i, device="cuda") for i in range(n_cp)]
            dec = T * w.k <= 64
            for i in range(n_cp):
                ref = mls[i].forward(xs[i]).clone()
                if dec and not torch.equal(mls[i].decode(xs[i]).view(torch.int16),
                                           ref.view(torch.int16)):
                    raise SystemExit("bench.py: %s decode differs from the four calls" % name)
            torch.cuda.synchronize()
            moe.moe_check_device_error()
            U = [int(np.unique(m.ids[:T].cpu().numpy()).size) for m in mls]
            bytes_step = float(np.mean([r_b + (u + 1) * E_b + 2 * T * w.d * 2 for u in U]))

            def run():
                for i in range(n_cp):
                    if dec:
                        mls[i].decode(xs[i])
                    else:
                        mls[i].forward(xs[i])
            ms, _, _ = time_graph(run, max(20, args.reps), 2)
            us = ms * 1e3 / n_cp
            row["T%d" % T] = {"entry": "moe_layer_decode" if dec else "four calls",
                              "us_per_step": round(us, 2),
                              "alg_bytes_per_step": int(bytes_step),
                              "weight_stream_GBps": round(bytes_step / (us * 1e-6) / 1e9, 1),
                              "tokens_per_s": round(T / (us * 1e-6), 1)}
            del mls, xs
        out[w.routed_fmt] = row
        del copies
        torch.cuda.empty_cache()
    return out


def mall_residency(moe, synth, np, torch, args):
    """What the 256 MB Infinity Cache (MALL) in front of HBM gives the decode step.

    read: our stream-read kernel over a working set of S MB, cold (after 1 GiB of other
    reads) and warm (the same S MB read again at once): the effective GB/s of data the cache
    holds against data it does not.
    decode_zipf: one token per step through moe_layer_decode (d 2048, 512 experts, top-10 +
    shared, Zipf router bias), 64 distinct tokens per replay, cycling over n_copies distinct
    copies of the layer: one copy's hot experts (most of the Zipf traffic) stay cached, 32
    copies touch more than the cache holds between reuses.  touched_MB = router rows and
    distinct experts the 64 steps read, summed over the copies."""
    import ctypes
    import statistics
    out = {}
    P = ctypes.CDLL(os.path.join(ROOT, "quantized_sparse_moe_router_amd", "libmoe_peaks.so"))
    P.moe_peaks_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                        ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sink = torch.empty(P.moe_peaks_stream_blocks(), dtype=torch.int32, device="cuda")
    flush = torch.ones((1 << 30) // 4, dtype=torch.int32, device="cuda")
    big = torch.ones((512 << 20) // 4, dtype=torch.int32, device="cuda")

    def read(t, n):
        assert P.moe_peaks_stream_read(t.data_ptr(), n, sink.data_ptr(), stream) == 0

    def timed(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b)
    rows = {}
    for mb in (16, 64, 128, 192, 256, 384, 512):
        n = mb << 20
        cold, warm = [], []
        for _ in range(7):
            read(flush, flush.numel() * 4)
            torch.cuda.synchronize()
            cold.append(timed(lambda: read(big, n)))
            warm.append(timed(lambda: read(big, n)))
        rows["%dMB" % mb] = {"cold_GBps": round(n / (statistics.median(cold) * 1e6), 1),
                             "warm_GBps": round(n / (statistics.median(warm) * 1e6), 1)}
    out["read"] = rows
    del flush, big, sink
    torch.cuda.empty_cache()

    w = synth.WORKLOADS["decode_d2048_e512_top10_t1"]
    base = synth.make_layer(w, seed=0, device="cuda", bias="zipf")
    copies = [base] + [clone_layer(base) for _ in range(31)]
    E_b = expert_bytes(base.routed)
    r_b = base.router.w.numel() * base.router.w.element_size()
    n_steps = 64
    toks = synth.make_tokens(w, T=n_steps, seed=7, device="cuda")
    xs = [toks[i:i + 1] for i in range(n_steps)]
    dz = {}
    for n_cp in (1, 2, 4, 8, 16, 32):
        mls = [moe.MoeLayer(c.router, c.routed, c.shared, w.k, 1) for c in copies[:n_cp]]
        seen = [set() for _ in range(n_cp)]
        for s_ in range(n_steps):
            m = mls[s_ % n_cp]
            m.decode(xs[s_])
            seen[s_ % n_cp].update(m.ids[:1].cpu().numpy().ravel().tolist())
        torch.cuda.synchronize()
        moe.moe_check_device_error()
        touched = sum(r_b + (len(z) + 1) * E_b for z in seen)

        def run():
            for s_ in range(n_steps):
                mls[s_ % n_cp].decode(xs[s_])
        ms, ms_min, _ = time_graph(run, max(20, args.reps), 2)
        dz["copies%d" % n_cp] = {"us_per_step": round(ms * 1e3 / n_steps, 3),
                                 "us_per_step_min": round(ms_min * 1e3 / n_steps, 3),
                                 "touched_MB": round(touched / 2 ** 20, 1),
                                 "distinct_experts_per_copy": round(
                                     float(np.mean([len(z) for z in seen])), 1)}
        del mls
    out["decode_zipf"] = dz
    del copies, base
    torch.cuda.empty_cache()
    return out


def decode_batches(moe, synth, np, torch, copies, w, args, Ts=(1, 4, 6, 8, 16, 32, 64, 96, 128)):
    """T tokens per call through the decode layer (d 2048, 512 experts, top-10 + shared),
    T = 1 .. 128: the four calls (forward) and, while T*k <= 64, moe_layer_decode; each step
    on the next of the rotated layer copies (more than the 256 MB cache holds for T >= 2).
    The routed experts run the weight-streaming GEMV (sorted mode past 24 pairs; from 640
    pairs the experts with many pairs on the grouped MFMA GEMM); the router computes its
    logits by GEMV up to 512 tokens.  Weight-stream bytes: router + (distinct routed experts + shared) x 1.77 MB."""
    E_b = expert_bytes(copies[0].routed)
    r_b = copies[0].router.w.numel() * copies[0].router.w.element_size()
    n_cp = len(copies)
    out = {"workload": "decode_d2048_e512_top10", "copies_rotated": n_cp}
    for T in Ts:
        mls = [moe.MoeLayer(c.router, c.routed, c.shared, w.k, T) for c in copies]
        xs = [synth.make_tokens(w, T=T, seed=100 + i, device="cuda") for i in range(n_cp)]
        for i in range(n_cp):
            mls[i].forward(xs[i])
        torch.cuda.synchronize()
        moe.moe_check_device_error()
        U = [int(np.unique(m.ids[:T].cpu().numpy()).size) for m in mls]
        bytes_step = float(np.mean([r_b + (u + 1) * E_b + 2 * T * w.d * 2 for u in U]))
        row = {"distinct_experts_mean": round(float(np.mean(U)), 2),
               "alg_bytes_per_step": int(bytes_step)}

        def fwd():
            for i in range(n_cp):
                mls[i].forward(xs[i])
        ms, _, _ = time_graph(fwd, max(20, args.reps), 2)
        ms /= n_cp
        row["four_calls_us"] = round(ms * 1e3, 2)
        row["four_calls_GBps"] = round(bytes_step / (ms * 1e-3) / 1e9, 1)
        row["four_calls_tokens_per_s"] = round(T / (ms * 1e-3), 1)
        if T * w.k <= 64:
            def dec():
                for i in range(n_cp):
                    mls[i].decode(xs[i])
            ms, _, _ = time_graph(dec, max(20, args.reps), 2)
            ms /= n_cp
            row["layer_decode_us"] = round(ms * 1e3, 2)
            row["layer_decode_GBps"] = round(bytes_step / (ms * 1e-3) / 1e9, 1)
        out["T%d" % T] = row
        del mls, xs
    return out


def decode_sweep(moe, synth, np, torch, args):
    """48 distinct blocks chained: each is the pre-layer RMS norm, the MoE layer and the
    gated residual, x_{l+1} = bf16(x_l + bf16(sigmoid(z_l) * out_l)) (moe_block_decode: the
    norm and the gate fused into the layer's three launches), one token and four tokens (one
    real + three drafts) per step; the whole 48-block step is one graph.  Weights: 48 x 0.91
    GB resident, so no cache holds them between steps.  (Without the norm the stream grows
    like x + c x^2 through the quadratic SwiGLU and overflows bf16 within ~30 layers.)"""
    w = synth.WORKLOADS["decode_sweep_48_layers"]
    lays = [synth.make_layer(w, seed=0, layer=l, device="cuda") for l in range(w.layers)]
    nrms = [synth.make_norm(w, seed=0, layer=l, device="cuda") for l in range(w.layers)]
    E_b = expert_bytes(lays[0].routed)
    r_b = lays[0].router.w.numel() * lays[0].router.w.element_size()
    n_b = 2 * w.d * 4                                 # gamma and the gate row, fp32
    out = {"workload": "decode_sweep_48_layers", "layers": w.layers, "router_bias": "zipf",
           "block": "rmsnorm -> moe layer -> gated residual (moe_block_decode)"}
    for T in (1, 4):
        mls = [moe.MoeLayer(L.router, L.routed, L.shared, w.k, T, norm=N)
               for L, N in zip(lays, nrms)]
        xs = [synth.make_tokens(w, T=T, seed=0, device="cuda")]
        xs += [torch.empty_like(xs[0]) for _ in range(w.layers)]

        def step():
            for l in range(w.layers):
                mls[l].block_decode(xs[l], out=xs[l + 1])

        step()
        torch.cuda.synchronize()
        moe.moe_check_device_error()
        rms_out = float(xs[-1].float().pow(2).mean().sqrt())
        if not np.isfinite(rms_out):
            raise SystemExit("bench.py: the 48-block stream is not finite")
        # distinct routed experts per layer (the bytes a step must stream)
        U = [int(np.unique(m.ids[:T].cpu().numpy()).size) for m in mls]
        ms, ms_min, _ = time_graph(step, max(20, args.reps), 2)
        bytes_step = sum(r_b + n_b + (u + 1) * E_b + 2 * T * w.d * 2 for u in U)
        out["T%d" % T] = {"tokens_per_s": round(T / (ms * 1e-3), 1),
                          "ms_per_step": round(ms, 4), "ms_per_step_min": round(ms_min, 4),
                          "us_per_layer": round(ms * 1e3 / w.layers, 3),
                          "distinct_experts_per_layer_mean": round(float(np.mean(U)), 2),
                          "alg_bytes_per_step": bytes_step,
                          "weight_stream_GBps": round(bytes_step / (ms * 1e-3) / 1e9, 1),
                          "rms_x_after_48_blocks": round(rms_out, 3)}
        del mls, xs
    del lays, nrms
    return out


def prefill_bench(moe, synth, np, torch, name, bias):
    w = synth.WORKLOADS[name]
    lay = synth.make_layer(w, seed=0, device="cuda", bias=bias)
    x = synth.make_tokens(w, seed=0, device="cuda")
    layer = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, w.T)
    layer.forward(x)
    torch.cuda.synchronize()
    moe.moe_check_device_error()
    import statistics

    def each(fn, reps=20):
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            torch.cuda._sleep(2_000_000)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return statistics.median(ts), min(ts)
    ms_layer, ms_layer_min = each(lambda: layer.forward(x))
    # grouped GEMM (routed experts): useful flops 6 * pairs * d * F
    P = w.T * w.k
    ms_gemm, ms_gemm_min = each(lambda: moe.moe_expert_ffn(
        layer.routed, x, w.T, w.k, layer.ids, layer.offsets, layer.sorted_pairs,
        layer.y_pairs, layer.ws_ffn))
    flops = 6.0 * P * w.d * w.F
    counts = np.diff(layer.offsets.cpu().numpy())
    del layer, lay
    return {"workload": name, "router_bias": bias or w.bias, "tokens": w.T,
            "tokens_per_s": round(w.T / (ms_layer * 1e-3), 1),
            "ms_layer": round(ms_layer, 4), "ms_layer_min": round(ms_layer_min, 4),
            # the routed moe_expert_ffn call: the grouped GEMM for experts with 4 or more
            # pairs, the GEMV for the others
            "routed_call": "moe_expert_ffn (grouped MFMA GEMM; GEMV for experts with < 4 pairs)",
            "ms_routed_grouped_gemm": round(ms_gemm, 4),
            "ms_routed_grouped_gemm_min": round(ms_gemm_min, 4),
            "routed_gemm_tflops": round(flops / (ms_gemm * 1e-3) / 1e12, 1),
            "mfma_util": round(flops / (ms_gemm * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "active_experts": int((counts > 0).sum()), "max_rows_per_expert": int(counts.max())}


def achievable_peaks(torch):
    """Measured ceilings on this GPU, next to the spec peaks: our stream-read kernel over
    4 GiB of HBM and our loop of bf16 MFMAs (libmoe_peaks.so, with the shader clock it runs
    at), plus torch's dense bf16 matmul (the vendor GEMM library) at the routed GEMMs'
    shapes for 8192 tokens (81920 pair rows; gate+up K=2048/N=1024, down K=512/N=2048)."""
    import ctypes

    def timed_ms(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps
    out = {}
    P = ctypes.CDLL(os.path.join(ROOT, "quantized_sparse_moe_router_amd", "libmoe_peaks.so"))
    P.moe_peaks_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                        ctypes.c_void_p]
    P.moe_peaks_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(P.moe_peaks_stream_blocks(), dtype=torch.int32, device="cuda")

    def stream_read():
        assert P.moe_peaks_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), stream) == 0
    out["hbm_read_GBps_stream_kernel"] = round(nbytes / (timed_ms(stream_read) * 1e6), 1)
    del buf, sink
    blocks, iters = 2048, 20000
    fsink = torch.empty(blocks * 4, dtype=torch.float32, device="cuda")
    clk = torch.empty(blocks * 2, dtype=torch.int64, device="cuda")

    def mfma_loop():
        assert P.moe_peaks_mfma_loop(blocks, iters, fsink.data_ptr(), clk.data_ptr(),
                                     stream) == 0
    ms = timed_ms(mfma_loop, reps=5)
    flops = blocks * 4.0 * iters * 8 * 32768
    out["mfma_bf16_tflops_loop"] = round(flops / (ms * 1e9), 1)
    c = clk.view(blocks, 2).double()
    out["sclk_mhz_mfma_loop"] = round(float((c[:, 0] / c[:, 1]).mean()) * 100.0, 0)
    x = torch.ones(1 << 29, dtype=torch.float32, device="cuda")
    out["hbm_read_GBps_torch_sum"] = round(x.numel() * 4 / (timed_ms(lambda: x.sum()) * 1e6), 1)
    del x
    for name, (M, K, N) in (("gateup", (81920, 2048, 1024)), ("down", (81920, 512, 2048))):
        g = torch.Generator(device="cuda").manual_seed(0)
        a = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
        b = torch.randn((K, N), generator=g, device="cuda").to(torch.bfloat16)
        ms = timed_ms(lambda: a @ b)
        out["dense_bf16_matmul_tflops_%s" % name] = round(2.0 * M * K * N / (ms * 1e9), 1)
        del a, b
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(base, toks, w, seconds, prefill_every=64):
    import numpy as np

    import oracle
    import synth
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
    out = {"value": round(n / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "cpu_model": cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0)),
           "sample": "%d single-token decode calls of the same layer (fp64 oracle, OpenMP "
                     "over tokens), %.1f s" % (n, dt)}
    # one thread on every `prefill_every`-th token of the 8192-token prefill, extrapolated
    pw = synth.WORKLOADS["prefill_8192_zipf"]
    lay = synth.make_layer(pw, seed=0, device="cuda")
    xp = si.bits16(synth.make_tokens(pw, seed=0, device="cuda"))
    # the router's fp32 audit: tokens whose top-k set another valid fp32 summation order
    # could change (exact logits within twice / once the rigorous rounding bound across the
    # cut), and tokens whose fixed-order selection differs from the exact one
    t = time.perf_counter()
    audit = {}
    for name, rr, xx, kk in (("decode_tokens", r_h, x_h, w.k),
                             ("prefill_8192_zipf", lay.router.host(), xp, pw.k)):
        a2 = oracle.router_tie_audit(rr, xx, kk, factor=2.0)
        a1 = oracle.router_tie_audit(rr, xx, kk, factor=1.0)
        audit[name] = {"tokens": int(xx.shape[0]), "within_2x_bound": a2["count"],
                       "within_1x_bound": a1["count"],
                       "fp32_selection_differs_from_exact": a1["differs"]}
    audit["seconds"] = round(time.perf_counter() - t, 1)
    out["router_tie_audit"] = audit
    sel = np.arange(0, pw.T, prefill_every, dtype=np.int32)
    oracle.set_num_threads(1)
    try:
        t = time.perf_counter()
        oracle.layer_tokens(lay.router.host(), lay.routed.host(), lay.shared.host(), xp, sel,
                            pw.k)
        dt1 = time.perf_counter() - t
    finally:
        oracle.set_num_threads(threads)
    del lay, xp
    out["prefill_8192_single_thread_extrapolated"] = {
        "tokens_per_s": round(sel.size / dt1, 3),
        "seconds_for_8192_tokens": round(dt1 * pw.T / sel.size, 1),
        "sample": "every %dth token (%d tokens) of the 8192-token Zipf prefill on 1 thread, "
                  "%.1f s, extrapolated to 8192 tokens (label: extrapolated)"
                  % (prefill_every, sel.size, dt1)}
    return out


if __name__ == "__main__":
    main()
