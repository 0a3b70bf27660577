"""Bench of the quantized routed-expert MoE layer on one MI355X.

Headline (one JSON line on stdout): decode tokens/s of one MoE layer at the pages'
routing shape (d_model 2048, 512 routed experts, top-10 + 1 shared, expert FFN width
512, int4 group-32 weights, one token per call).  A step is the whole hot path for one
token: router + top-k, shared expert, routed experts, combine -- moe_layer_decode, which
is checked bit for bit against the four-call composition before timing (whose time per
step is reported too).  Inputs are resident in HBM before timing; the step sequence is
captured in a HIP graph and replayed.
To keep the 256 MB Infinity Cache from serving the weights, steps rotate over
``--copies`` distinct copies of the layer (a different token per copy).

Also reported in the same line:
  roofline      the expert kernels of a decode step (moe_experts_decode: gate/up kernel then
                down + combine kernel): algorithmic bytes (10 routed + 1 shared expert's
                packed weights and scales, activations in and out) / their event-timed
                average duration vs 8 TB/s
  cpu_baseline  the CPU oracle on a bounded sample of the same workload
  prefill       8192-token prefill through one layer (Zipf routing): tokens/s and the
                grouped GEMM's MFMA utilisation (useful flops / time / 2.5 PFLOP/s)
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
    p.add_argument("--copies", type=int, default=32,
                   help="distinct layer copies rotated through (defeats the 256 MB MALL)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-sweep", action="store_true", help="skip the 48-layer decode sweep")
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

    reps = max(1, -(-args.steps // L))
    warm = max(1, -(-args.warmup // L))
    steps = reps * L

    def timed(fn, n_reps):
        if args.eager:
            for _ in range(warm):
                fn()
            torch.cuda.synchronize()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(n_reps):
                fn()
            t1.record()
            torch.cuda.synchronize()
            return t0.elapsed_time(t1) / n_reps
        return time_graph(fn, n_reps, warm)[0]

    ms_step = timed(step_all, reps) / L
    tok_s = 1000.0 / ms_step
    ms_step_calls = timed(step_all_calls, max(4, reps // 2)) / L

    # ---- roofline: the expert kernels of the decode step (moe_experts_decode: the routed
    # experts and the shared one streamed once, SwiGLU, combine) -- two launches per call
    E_b = expert_bytes(base.routed)
    alg_bytes_exp = (w.k + 1) * E_b + 2 * w.d * 2

    def experts_all():
        for i in range(L):
            layers[i].experts_decode(xs[i])

    ms_exp = timed(experts_all, max(4, reps // 2)) / L
    achieved = alg_bytes_exp / (ms_exp * 1e-3) / 1e9
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
                   "entry_point": "moe_layer_decode",
                   "step_weight_stream_GBps": round(alg_bytes_step / (ms_step * 1e-3) / 1e9, 1),
                   "alg_bytes_per_step": alg_bytes_step,
                   "ms_per_step_four_calls": round(ms_step_calls, 5)},
        "roofline": {"bound": "hbm",
                     "kernel": "decode_gateup_kernel + decode_down_kernel (moe_experts_decode:"
                               " 10 routed + 1 shared expert FFN and combine)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "alg_bytes_per_launch": alg_bytes_exp,
                     "avg_launch_us": round(ms_exp * 1e3, 3)},
    }

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


def decode_sweep(moe, synth, np, torch, args):
    """48 distinct layers chained through the residual, x_{l+1} = bf16(x_l + out_l), one
    token and four tokens (one real + three drafts) per step; the whole 48-layer step is
    one graph.  Weights: 48 x 0.91 GB resident, so no cache holds them between steps."""
    w = synth.WORKLOADS["decode_sweep_48_layers"]
    lays = [synth.make_layer(w, seed=0, layer=l, device="cuda") for l in range(w.layers)]
    E_b = expert_bytes(lays[0].routed)
    r_b = lays[0].router.w.numel() * lays[0].router.w.element_size()
    out = {"workload": "decode_sweep_48_layers", "layers": w.layers, "router_bias": "zipf"}
    for T in (1, 4):
        mls = [moe.MoeLayer(L.router, L.routed, L.shared, w.k, T) for L in lays]
        xs = [synth.make_tokens(w, T=T, seed=0, device="cuda")]
        xs += [torch.empty_like(xs[0]) for _ in range(w.layers)]

        def step():
            for l in range(w.layers):
                mls[l].decode(xs[l], residual=xs[l], out=xs[l + 1])

        step()
        torch.cuda.synchronize()
        moe.moe_check_device_error()
        # distinct routed experts per layer (the bytes a step must stream)
        U = [int(np.unique(m.ids[:T].cpu().numpy()).size) for m in mls]
        reps = max(4, args.steps // (8 * w.layers))
        ms = time_graph(step, reps, 2)[0]
        bytes_step = sum(r_b + (u + 1) * E_b + 2 * T * w.d * 2 for u in U)
        out["T%d" % T] = {"tokens_per_s": round(T / (ms * 1e-3), 1),
                          "ms_per_step": round(ms, 4),
                          "us_per_layer": round(ms * 1e3 / w.layers, 3),
                          "distinct_experts_per_layer_mean": round(float(np.mean(U)), 2),
                          "alg_bytes_per_step": bytes_step,
                          "weight_stream_GBps": round(bytes_step / (ms * 1e-3) / 1e9, 1)}
        del mls, xs
    del lays
    return out


def prefill_bench(moe, synth, np, torch, name, bias):
    w = synth.WORKLOADS[name]
    lay = synth.make_layer(w, seed=0, device="cuda", bias=bias)
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
    del layer, lay
    return {"workload": name, "router_bias": bias or w.bias, "tokens": w.T,
            "tokens_per_s": round(w.T / (ms_layer * 1e-3), 1),
            "ms_layer": round(ms_layer, 4), "ms_routed_grouped_gemm": round(ms_gemm, 4),
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
