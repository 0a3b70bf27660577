"""GPU: moe_layer_decode (two launches) equals the four-call composition bit for bit, and
through it the oracle.  Covers one token, MTP-style batches, the tiny layer, a residual,
repeated calls (the workspace counters must come back to zero) and graph replay."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_sparse_moe_router_amd as moe
    return moe


_LAYERS = {}


def _layer(name, bias=None):
    key = (name, bias)
    if key not in _LAYERS:
        _LAYERS.clear()
        w = synth.WORKLOADS[name]
        _LAYERS[key] = (w, synth.make_layer(w, seed=0, device="cuda", bias=bias))
    return _LAYERS[key]


def _same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("name,T,bias", [
    ("tiny_d256_e16_top2", 1, None),
    ("tiny_d256_e16_top2", 4, None),
    ("tiny_d256_e16_top2", 32, None),
    ("decode_d2048_e512_top10_t1", 1, None),
    ("decode_sweep_48_layers", 1, "zipf"),
    ("decode_sweep_48_layers", 4, "zipf"),
    ("decode_sweep_48_layers", 6, "zipf"),
    ("decode_d2048_e512_top10_t1", 2, None),
    ("int6_tiny_d256_e16_top2", 4, None),
    ("int6_d2048_e64_top10", 1, None),
    ("int6_d2048_e64_top10", 4, None),
    ("int3_tiny_d256_e16_top2", 4, None),
    ("int3_d2048_e512_top10", 1, None),
    ("int3_d2048_e512_top10", 6, "zipf"),
    ("int2_tiny_d256_e16_top2", 4, None),
    ("int2_d2048_e512_top10", 1, None),
    ("int2_d2048_e512_top10", 6, "zipf"),
])
def test_decode_equals_composition(name, T, bias):
    moe = _gpu()
    w, lay = _layer(name, bias)
    print("case %s T=%d bias=%s" % (name, T, bias), flush=True)
    x = synth.make_tokens(w, T=T, seed=3, device="cuda")
    res = synth.make_tokens(w, T=T, seed=4, device="cuda")
    a = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, T)
    b = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, T)
    assert b.can_decode
    ref = a.forward(x, residual=res).clone()
    for rep in range(3):            # counters must be back at zero after every call
        got = b.decode(x, residual=res)
        torch.cuda.synchronize()
        moe.moe_check_device_error()
        assert torch.equal(a.ids[:T], b.ids[:T])
        assert torch.equal(a.weights[:T].view(torch.int32), b.weights[:T].view(torch.int32))
        assert _same(got, ref), "rep %d: %d values differ" % (
            rep, int((got.view(torch.int16) != ref.view(torch.int16)).sum()))
    # a call is a few microseconds; a wait that only ends at its bound takes about a second
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    b.decode(x, residual=res)
    t1.record()
    torch.cuda.synchronize()
    assert t0.elapsed_time(t1) < 20.0, "decode call took %.1f ms" % t0.elapsed_time(t1)
    # without residual, and out aliasing the residual buffer
    ref2 = a.forward(x).clone()
    assert _same(b.decode(x), ref2)
    buf = res.clone()
    ref3 = a.forward(x, residual=buf).clone()
    assert _same(b.decode(x, residual=buf, out=buf), ref3)


def test_decode_graph_replay():
    moe = _gpu()
    w, lay = _layer("decode_d2048_e512_top10_t1")
    T = 1
    xs = [synth.make_tokens(w, T=T, seed=10 + i, device="cuda") for i in range(3)]
    x = xs[0].clone()
    b = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, T)
    a = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, T)
    b.decode(x)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        b.decode(x)
    for i in range(6):
        x.copy_(xs[i % 3])
        g.replay()
        torch.cuda.synchronize()
        ref = a.forward(xs[i % 3])
        torch.cuda.synchronize()
        assert _same(b.out[:T], ref), "replay %d differs" % i
    moe.moe_check_device_error()
