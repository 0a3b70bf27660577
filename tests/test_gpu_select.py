"""GPU: expert selection on inputs built to stress it, against the oracle.

The selection must give the k largest fp32 logits in descending order, equal logits lower
expert id first, for any input.  Random Gaussian logits almost never tie, so these cases
construct routers whose logits tie a lot: rows drawn from a handful of distinct rows
(many exact ties; more candidates than the fast form's compaction holds), integer-valued
weights and activations (exact sums with occasional ties), and an all-zero router (every
logit equal: ids 0..k-1, weights 1/k).  Each case runs every place the selection runs:
moe_route for up to 4 tokens (one launch) and for 6 or 40 (logits, then a selection
kernel), moe_route for many tokens with logits requested
(fixed-order GEMM) and without (MFMA logits with an error bound, exact recomputation of
the experts the bound cannot rule out), and the gate/up kernel of moe_layer_decode; all
must agree with the oracle and with each other, weights bit for bit.
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


def _check_both_forms(layer, x, T, logits_ref, ids_ref, w_ref):
    """layer.forward() has run (no logits requested); run the logits-returning path too."""
    ids2 = torch.empty_like(layer.ids)
    w2 = torch.empty_like(layer.weights)
    logits = layer.route_logits(x, ids2, w2).cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(logits.view(np.uint32), logits_ref.view(np.uint32))
    assert np.array_equal(layer.ids[:T].cpu().numpy(), ids_ref)
    assert np.array_equal(ids2[:T].cpu().numpy(), ids_ref)
    assert torch.equal(w2[:T].view(torch.int32), layer.weights[:T].view(torch.int32))
    assert np.abs(layer.weights[:T].cpu().numpy().astype(np.float64) - w_ref).max() <= 1e-6


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
    for T in (T_dec, 4, 40, 300, 600):
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
        _check_both_forms(layer, x, T, logits_ref, ids_ref, w_ref)
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


@pytest.mark.parametrize("kind", ["few_rows", "integers", "zero"])
def test_selection_with_ties_int8_router(kind):
    # the same stress cases through an INT8_ROW router (per-row scale), many tokens
    moe = _gpu()
    w = synth.WORKLOADS["decode_d2048_e512_top10_t1"]
    lay = synth.make_layer(w, seed=0, device="cuda")
    gen = torch.Generator().manual_seed(23)
    q, sc = si.quantize_int8_row(_router(kind, w.E, w.d, gen))
    gb = torch.Generator().manual_seed(5)
    bias = si.zipf_bias(w.E, 1.1, gb, "cpu") if kind == "few_rows" else None
    router = si.Router("int8_row", w.E, w.d, q.cuda(), sc.cuda(),
                       None if bias is None else bias.cuda())
    r_h = router.host()
    for T in (40, 300, 600):
        print("case int8 %s T=%d" % (kind, T), flush=True)
        x = _tokens(kind, T, w.d, gen).cuda()
        logits_ref = oracle.router_logits(r_h, si.bits16(x))
        ids_ref = oracle.select_topk(logits_ref, w.k)
        w_ref = oracle.topk_weights(logits_ref, ids_ref)
        layer = moe.MoeLayer(router, lay.routed, lay.shared, w.k, T)
        layer.forward(x)
        torch.cuda.synchronize()
        moe.moe_check_device_error()
        _check_both_forms(layer, x, T, logits_ref, ids_ref, w_ref)


def _round256(n):
    return (n + 255) & ~255


@pytest.mark.parametrize("name", ["prefill_8192_zipf", "prefill_32768_mixed"])
def test_bounded_logits_within_bound(name):
    # The bounded form's MFMA logits (kept in the route workspace after the counter) must
    # lie within 2^-11 (|x_t| |w_e| + |b_e|) of the fixed-order logits; the measured error
    # is expected far inside it, so a quarter of the bound is asserted.  The row norm
    # bounds that follow the plane rows must bound the true norms from above, tightly.
    moe = _gpu()
    w = synth.WORKLOADS[name]
    T = 2048
    lay = synth.make_layer(w, seed=0, device="cuda")
    x = synth.make_tokens(w, T=T, seed=0, device="cuda")
    layer = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, T)
    layer.forward(x)
    torch.cuda.synchronize()
    moe.moe_check_device_error()
    E, d = w.E, w.d
    ws = layer.ws_route.cpu()
    off_lf = 256
    off_nw = off_lf + _round256(T * E * 4) + _round256(E * 2 * d * 2)
    lf = ws[off_lf:off_lf + T * E * 4].view(torch.float32).numpy().reshape(T, E)
    nw_gpu = ws[off_nw:off_nw + E * 4].view(torch.float32).numpy().astype(np.float64)
    r_h = lay.router.host()
    x_h = si.bits16(x)
    ref = oracle.router_logits(r_h, x_h).astype(np.float64)
    xf = (x_h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nx = np.sqrt((xf * xf).sum(axis=1))
    wr = r_h["w"].astype(np.float64)
    nw = np.sqrt((wr * wr).sum(axis=1))
    if r_h["scale"] is not None:
        s = (r_h["scale"].astype(np.uint16)).view(np.float16).astype(np.float64)
        nw = nw * np.abs(s)
    assert (nw_gpu >= nw).all() and (nw_gpu <= nw * (1 + 2.0 ** -9)).all()
    b = np.zeros(E) if r_h["bias"] is None else np.abs(r_h["bias"].astype(np.float64))
    bound = 2.0 ** -11 * (nx[:, None] * nw[None, :] + b[None, :])
    ratio = np.abs(lf.astype(np.float64) - ref) / bound
    print("%s: max |lf - logit| / bound = %.3g" % (name, ratio.max()), flush=True)
    assert ratio.max() <= 0.25


@pytest.mark.parametrize("scale", [1e-31, 1e30])
def test_bounded_selection_tiny_and_huge_rows(scale):
    # Rows scaled so that |x| |w_e| falls below the bounded form's underflow guard (every
    # expert is then recomputed in the fixed order, more than 64 candidates: the general
    # selection runs), or is huge (the bound is wide; more candidates, still exact).
    moe = _gpu()
    w = synth.WORKLOADS["decode_d2048_e512_top10_t1"]
    lay = synth.make_layer(w, seed=0, device="cuda")
    gen = torch.Generator().manual_seed(29)
    rw = (torch.randn((w.E, w.d), generator=gen) * 0.02 * scale).contiguous()
    router = si.Router("fp32", w.E, w.d, rw.cuda(), None, None)
    r_h = router.host()
    T = 40
    print("case scale %g T=%d" % (scale, T), flush=True)
    x = _tokens("normal", T, w.d, gen).cuda()
    logits_ref = oracle.router_logits(r_h, si.bits16(x))
    assert np.isfinite(logits_ref).all()
    ids_ref = oracle.select_topk(logits_ref, w.k)
    w_ref = oracle.topk_weights(logits_ref, ids_ref)
    layer = moe.MoeLayer(router, lay.routed, lay.shared, w.k, T)
    layer.forward(x)
    torch.cuda.synchronize()
    moe.moe_check_device_error()
    _check_both_forms(layer, x, T, logits_ref, ids_ref, w_ref)
