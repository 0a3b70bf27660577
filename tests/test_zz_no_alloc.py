"""moe_layer_decode_noalloc (the decode layer on the library's fixed workspace, for callers
that cannot allocate) against moe_layer_decode through the C ABI: ids, weights and output
bit for bit, on two calls in a row, the second with a smaller input, and again after a
call of another shape has left its contents in the fixed workspace."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_sparse_moe_router_amd as moe
    return moe


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def _pair(moe, lay, w, T, x, res):
    """moe_layer_decode on its own workspace, and moe_layer_decode_noalloc."""
    a = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, T)
    ref = a.decode(x, residual=res).clone()
    ids = torch.full((T, w.k), -1, dtype=torch.int32, device="cuda")
    wts = torch.zeros((T, w.k), dtype=torch.float32, device="cuda")
    out = torch.zeros_like(x)
    moe.moe_layer_decode_noalloc(a.router, a.routed, a.shared, x, T, w.k, ids, wts, res, out)
    torch.cuda.synchronize()
    moe.moe_check_device_error()
    assert torch.equal(ids, a.ids[:T])
    assert torch.equal(wts.view(torch.int32), a.weights[:T].view(torch.int32))
    assert _same(out, ref), "%d values differ" % int((out.view(torch.int16) !=
                                                      ref.view(torch.int16)).sum())


@pytest.mark.parametrize("name,bias,T1,T2", [
    ("decode_sweep_48_layers", "zipf", 4, 1),      # several tokens (counter hand-off), then one
    ("decode_d2048_e512_top10_t1", None, 6, 2),
    ("tiny_d256_e16_top2", None, 32, 3),
])
def test_noalloc_equals_decode(name, bias, T1, T2):
    moe = _gpu()
    w = synth.WORKLOADS[name]
    print("case %s T=%d then T=%d" % (name, T1, T2), flush=True)
    lay = synth.make_layer(w, seed=0, device="cuda", bias=bias)
    x1 = synth.make_tokens(w, T=T1, seed=41, device="cuda")
    r1 = synth.make_tokens(w, T=T1, seed=42, device="cuda")
    _pair(moe, lay, w, T1, x1, r1)
    x2 = synth.make_tokens(w, T=T2, seed=43, device="cuda")
    _pair(moe, lay, w, T2, x2, None)         # smaller input, no residual


def test_noalloc_rejects_like_decode():
    moe = _gpu()
    w = synth.WORKLOADS["decode_d2048_e512_top10_t1"]
    lay = synth.make_layer(w, seed=0, device="cuda")
    a = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, 8)
    x = synth.make_tokens(w, T=7, seed=1, device="cuda")
    ids = torch.empty((7, w.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((7, w.k), dtype=torch.float32, device="cuda")
    out = torch.empty_like(x)
    with pytest.raises(moe.MoeError) as ei:          # 70 pairs: beyond the decode layer
        moe.moe_layer_decode_noalloc(a.router, a.routed, a.shared, x, 7, w.k, ids, wts, None,
                                     out)
    assert ei.value.status == moe._lib.MOE_ERR_UNSUPPORTED
    # T = 0 is a no-op
    moe.moe_layer_decode_noalloc(a.router, a.routed, a.shared, x[:0], 0, w.k, ids, wts, None,
                                 out)
