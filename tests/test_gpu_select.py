"""GPU: expert selection on inputs built to stress it, against the oracle.

The selection must give the k largest fp32 logits in descending order, equal logits lower
expert id first, for any input.  Random Gaussian logits almost never tie, so these cases
construct routers whose logits tie a lot: rows drawn from a handful of distinct rows
(many exact ties; more candidates than the fast form's compaction holds), integer-valued
weights and activations (exact sums with occasional ties), and an all-zero router (every
logit equal: ids 0..k-1, weights 1/k).  Each case runs the three places the selection
runs: moe_route for few tokens (one launch), moe_route for many tokens, and the gate/up
kernel of moe_layer_decode; all must agree with the oracle and with each other.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import inputs as si

pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_sparse_moe_router_amd as moe
    return moe


def _router(kind, E, d, gen):
    if kind == "few_rows":       # 6 distinct rows: each logit value shared by ~E/6 experts
        base = torch.randn((6, d), generator=gen) * 0.02
        pick = torch.randint(0, 6, (E,), generator=gen)
        return base[pick].contiguous()
    if kind == "integers":       # integer multiples of 1/64: exact sums, some ties
        return (torch.randint(-2, 3, (E, d), generator=gen).float() / 64.0).contiguous()
    if kind == "zero":
        return torch.zeros((E, d))
    raise ValueError(kind)


def _tokens(kind, T, d, gen):
    if kind == "integers":
        x = torch.randint(-1, 2, (T, d), generator=gen).float()
    else:
        x = torch.randn((T, d), generator=gen)
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("name", ["decode_d2048_e512_top10_t1", "tiny_d256_e16_top2"])
@pytest.mark.parametrize("kind", ["few_rows", "integers", "zero"])
def test_selection_with_ties(name, kind):
    moe = _gpu()
    w = synth.WORKLOADS[name]
    lay = synth.make_layer(w, seed=0, device="cuda")
    gen = torch.Generator().manual_seed(17)
    rw = _router(kind, w.E, w.d, gen).cuda()
    router = si.Router("fp32", w.E, w.d, rw, None, None)
    r_h = router.host()
    k = w.k
    T_dec = min(6, 64 // k)
    for T in (T_dec, 4, 40):
        print("case %s %s T=%d" % (name, kind, T), flush=True)
        x = _tokens(kind, T, w.d, gen).cuda()
        x_h = si.bits16(x)
        logits_ref = oracle.router_logits(r_h, x_h)
        ids_ref = oracle.select_topk(logits_ref, k)
        w_ref = oracle.topk_weights(logits_ref, ids_ref)
        layer = moe.MoeLayer(router, lay.routed, lay.shared, k, T)
        out = layer.forward(x).clone()
        torch.cuda.synchronize()
        moe.moe_check_device_error()
        logits = layer.logits[:T].cpu().numpy()
        assert np.array_equal(logits.view(np.uint32), logits_ref.view(np.uint32))
        assert np.array_equal(layer.ids[:T].cpu().numpy(), ids_ref)
        assert np.abs(layer.weights[:T].cpu().numpy().astype(np.float64) - w_ref).max() <= 1e-6
        if kind == "zero":
            assert (ids_ref == np.arange(k)[None, :]).all()
        if T * k <= 64 and layer.can_decode:
            dec = moe.MoeLayer(router, lay.routed, lay.shared, k, T)
            got = dec.decode(x)
            torch.cuda.synchronize()
            moe.moe_check_device_error()
            assert np.array_equal(dec.ids[:T].cpu().numpy(), ids_ref)
            assert torch.equal(dec.weights[:T], layer.weights[:T])
            assert torch.equal(got[:T].view(torch.int16), out[:T].view(torch.int16))
