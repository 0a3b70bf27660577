"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded
inputs.

Bar (what the pages and the arithmetic fix):
  router logits, expert ids, offsets / sorted_pairs / pair_pos   bit-exact
  gate weights                                                    |dw| <= 1e-6
  per-pair and shared expert rows, layer output   |g - r| <= 2e-2 + 1e-2 |r| elementwise
                                                  and ||g - r|| / ||r|| <= 1e-2
The float bar is the layer tolerance max-abs 2e-2 / rel 1e-2 (fp32 accumulation, bf16
activations); the relative-Frobenius check keeps a dropped pair (weight ~0.05, error ~1%
of the row) from hiding under the elementwise bound.  Largest sizes are checked on
sampled tokens the oracle evaluates one by one, plus full-size bit-exact routing.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import inputs as si

pytestmark = pytest.mark.gpu

ATOL, RTOL, FROB = 2e-2, 1e-2, 1e-2


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_sparse_moe_router_amd as moe
    return moe


_CACHE = {}


def _setup(name, bias=None, seed=0):
    key = (name, bias, seed)
    if key not in _CACHE:
        w = synth.WORKLOADS[name]
        lay = synth.make_layer(w, seed=seed, device="cuda", bias=bias)
        host = (lay.router.host(), lay.routed.host(), lay.shared.host())
        _CACHE.clear()
        _CACHE[key] = (w, lay, host)
    return _CACHE[key]


def _bf16_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _close(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), "%s: %d elements out of tolerance, max err %.3g" % (
        what, int(bad.sum()), float(err.max()))
    frob = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert frob <= FROB, "%s: rel-Frobenius %.3g" % (what, frob)
    return float(err.max()), float(frob)


def _run(moe, lay, w, x):
    T = x.shape[0]
    layer = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, T)
    out = layer.forward(x)
    torch.cuda.synchronize()
    moe.moe_check_device_error()
    return layer, out


def _check_tiles(layer, w, x_h, ex_h, sh_h, ids_ref, off_ref, sp_ref, T):
    """Pair rows at the first and last row of every (expert, 256-row tile) entry of the
    grouped GEMM's work list, which includes every expert's last row, and shared-expert
    rows at the first and last token of every 256-token tile, against the oracle."""
    k, BM = w.k, 256
    pos = []
    for e in range(w.E):
        for m0 in range(int(off_ref[e]), int(off_ref[e + 1]), BM):
            pos += [m0, min(m0 + BM, int(off_ref[e + 1])) - 1]
    pos = np.unique(np.array(pos, np.int64))
    pairs = sp_ref[pos]
    tok = (pairs // k).astype(np.int32)
    exp = ids_ref.reshape(-1)[pairs].astype(np.int32)
    ref = oracle.expert_ffn_pairs(ex_h, x_h, tok, exp)
    got = _bf16_np(layer.y_pairs[torch.from_numpy(pos).long().cuda()])
    _close(got, ref, "pair rows at every tile's first and last row (%d rows)" % pos.size)
    nrm = np.linalg.norm(got - ref, axis=1) <= FROB * np.linalg.norm(ref, axis=1) + 1e-6
    assert nrm.all(), "%d pair rows above the per-pair bound" % int((~nrm).sum())
    st = np.unique(np.concatenate([np.arange(0, T, BM), np.minimum(np.arange(0, T, BM) + BM,
                                                                   T) - 1])).astype(np.int32)
    ref_sh = oracle.expert_ffn_pairs(sh_h, x_h, st, np.zeros_like(st))
    got_sh = _bf16_np(layer.y_shared[torch.from_numpy(st).long().cuda()])
    _close(got_sh, ref_sh, "shared rows at every tile's first and last token")
    print("tile coverage: %d pair rows, %d shared rows" % (pos.size, st.size), flush=True)


def _check_layer(name, T=None, sample=None, bias=None, seed=0, stream=0, tiles=False):
    moe = _gpu()
    w, lay, (r_h, ex_h, sh_h) = _setup(name, bias=bias, seed=seed)
    T = w.T if T is None else T
    x = synth.make_tokens(w, T=T, seed=seed, device="cuda", stream=stream)
    x_h = si.bits16(x)
    print("case %s T=%d seed=%d bias=%s" % (name, T, seed, bias), flush=True)
    layer, out = _run(moe, lay, w, x)
    k, E = w.k, w.E

    # routing: full size, bit-exact.  forward() selects without logits (for T > 512 the
    # bounded MFMA form); route_logits() runs the fixed-order path that returns them.
    logits_ref = oracle.router_logits(r_h, x_h)
    ids2 = torch.empty_like(layer.ids)
    w2 = torch.empty_like(layer.weights)
    logits = layer.route_logits(x, ids2, w2).cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(logits.view(np.uint32), logits_ref.view(np.uint32)), \
        "logits differ in %d places" % int((logits != logits_ref).sum())
    ids_ref = oracle.select_topk(logits_ref, k)
    ids = layer.ids[:T].cpu().numpy()
    assert np.array_equal(ids, ids_ref)
    assert np.array_equal(ids2[:T].cpu().numpy(), ids_ref)
    assert torch.equal(w2[:T].view(torch.int32), layer.weights[:T].view(torch.int32))
    w_ref = oracle.topk_weights(logits_ref, ids_ref)
    wts = layer.weights[:T].cpu().numpy().astype(np.float64)
    assert np.abs(wts - w_ref).max() <= 1e-6
    # the invariants on the GPU's own outputs: k distinct experts per token, gate weights
    # positive and summing to 1 up to fp32 rounding
    assert all(len(set(row)) == k for row in ids.tolist())
    assert (wts > 0).all() and np.abs(wts.sum(axis=1) - 1.0).max() <= 1e-5
    off_ref, sp_ref, pp_ref, bad = oracle.permute(ids_ref, E)
    assert bad == 0
    assert np.array_equal(layer.offsets.cpu().numpy(), off_ref)
    assert np.array_equal(layer.sorted_pairs[:T * k].cpu().numpy(), sp_ref)
    assert np.array_equal(layer.pair_pos[:T * k].cpu().numpy(), pp_ref)

    if tiles:
        _check_tiles(layer, w, x_h, ex_h, sh_h, ids_ref, off_ref, sp_ref, T)

    # experts and combine: every token, or a sample
    if sample is None or sample >= T:
        toks = np.arange(T, dtype=np.int32)
    else:
        rng = np.random.default_rng(1234 + T)
        toks = np.unique(np.concatenate([[0, T - 1], rng.choice(T, sample, replace=False)]))
        toks = toks.astype(np.int32)
    res = oracle.layer_tokens(r_h, ex_h, sh_h, x_h, toks, k, keep_pairs=True)
    assert np.array_equal(res["ids"], ids_ref[toks])
    y_pairs = layer.y_pairs[:T * k]
    pos = pp_ref.reshape(T, k)[toks]                       # [n][k] sorted positions
    got_pairs = _bf16_np(y_pairs[torch.from_numpy(pos.reshape(-1)).long().cuda()])
    _close(got_pairs, res["y_sel"].reshape(-1, w.d), name + " pair rows")
    for i in range(len(toks)):   # per-pair relative error
        for j in range(k):
            ref = res["y_sel"][i, j]
            g = got_pairs[i * k + j]
            assert np.linalg.norm(g - ref) <= FROB * np.linalg.norm(ref) + 1e-6
    got_sh = _bf16_np(layer.y_shared[torch.from_numpy(toks).long().cuda()])
    _close(got_sh, res["y_shared"], name + " shared rows")
    got_out = _bf16_np(out[torch.from_numpy(toks).long().cuda()])
    return _close(got_out, res["out"], name + " layer out")


def test_tiny_layer_all_tokens():
    _check_layer("tiny_d256_e16_top2")


def test_tiny_layer_ragged_token_counts():
    for T in (1, 3, 33, 100):
        _check_layer("tiny_d256_e16_top2", T=T, stream=T)


def test_decode_single_token():
    _check_layer("decode_d2048_e512_top10_t1")


@pytest.mark.parametrize("T", [4, 6, 17])
def test_decode_small_batches_zipf(T):
    # 4 = one token plus three drafts verified together; Zipf bias makes experts shared
    _check_layer("decode_d2048_e512_top10_t1", T=T, bias="zipf", stream=T)


@pytest.mark.parametrize("T,bias", [(8, None), (16, None), (32, "zipf"), (64, None),
                                    (64, "zipf"), (96, "zipf"), (102, None), (160, None),
                                    (200, "zipf")])
def test_decode_batches_sorted_gemv(T, bias):
    # 65..4096 pairs: the GEMV kernels in sorted mode (chunks of consecutive sorted positions
    # of one expert, from moe_permute's grouping); under Zipf the hot experts span several
    # chunks, and from 640 pairs the experts with many pairs take the grouped GEMM in the
    # same call.  Up to 512 tokens the router computes its logits by GEMV.
    _check_layer("decode_d2048_e512_top10_t1", T=T, bias=bias, stream=T,
                 sample=None if T <= 102 else 40, tiles=T > 102)


def _hot_rows(rows):
    # the split of the library's expert FFN: from 640 pairs an expert with at least this many
    # pairs takes the grouped GEMM (0: every expert on the GEMV)
    return 0 if rows < 640 else (8 if rows <= 1024 else 4)


def test_batch_invariance_of_the_gemv_paths():
    """A token's ids and weights are bit-identical alone and among 48, 64 or 102 tokens.  A
    routed-expert row is bit-identical too whenever its expert runs on the GEMV in the
    larger call (the ballot and sorted modes share the per-pair arithmetic): every expert
    below 640 pairs, the experts with few pairs above (the others take the grouped GEMM,
    another accumulation order; the layer tests check them against the oracle).  The
    token's output too at 48 tokens.  Zipf routing, so that some experts are hot."""
    moe = _gpu()
    w, lay, _ = _setup("decode_d2048_e512_top10_t1", bias="zipf")
    k = w.k
    xall = synth.make_tokens(w, T=102, device="cuda", stream=77)
    for T in (48, 64, 102):
        x = xall[:T].contiguous()
        big, out = _run(moe, lay, w, x)
        out = out.clone()
        pp = big.pair_pos[:T * k].cpu().numpy()
        ids_big = big.ids[:T].cpu().numpy()
        counts = np.diff(big.offsets.cpu().numpy())
        hot = _hot_rows(T * k)
        yb = big.y_pairs.clone()
        checked = 0
        for t in (0, 13, T - 1):
            one, o1 = _run(moe, lay, w, x[t:t + 1].contiguous())
            assert torch.equal(one.ids[:1], big.ids[t:t + 1])
            assert torch.equal(one.weights[:1].view(torch.int32),
                               big.weights[t:t + 1].view(torch.int32))
            pp1 = one.pair_pos[:k].cpu().numpy()
            for j in range(k):
                if hot and counts[ids_big[t, j]] >= hot:
                    continue
                assert torch.equal(yb[int(pp[t * k + j])].view(torch.int16),
                                   one.y_pairs[int(pp1[j])].view(torch.int16)), \
                    "T %d token %d slot %d" % (T, t, j)
                checked += 1
            if T * k < 640:
                assert torch.equal(o1.view(torch.int16), out[t:t + 1].view(torch.int16)), \
                    "T %d token %d" % (T, t)
        assert checked > 0, "T %d: no sampled row ran on the GEMV" % T


def test_decode_sweep_layer_batch4():
    _check_layer("decode_sweep_48_layers", T=4)


@pytest.mark.parametrize("T", [1, 4, 17, 65, 513])
def test_int6_experts_int8_router_small_batches(T):
    # int6 routed and shared experts through the GEMV kernels (ballot, then sorted mode) and
    # at 5130 pairs the grouped GEMM; the int8 router by its one-launch form, its split form
    # (T = 17, 65) and its bounded MFMA form (T = 513)
    if T > 512:
        _check_layer("int6_d2048_e64_top10", T=T, stream=T, sample=40, tiles=True)
    else:
        _check_layer("int6_d2048_e64_top10", T=T, stream=T)


@pytest.mark.parametrize("name", ["int3_d2048_e512_top10", "int2_d2048_e512_top10"])
@pytest.mark.parametrize("T,bias", [(1, None), (8, "zipf"), (64, None), (200, "zipf")])
def test_low_bit_experts(name, T, bias):
    # every expert at 3 or 2 bits: the decode-layer shape through the ballot GEMV (T = 1),
    # the sorted GEMV (T = 8, 64) and the grouped MFMA GEMM (T = 200, 2000 pairs)
    _check_layer(name, T=T, bias=bias, stream=T, sample=min(T, 24), tiles=T > 100)


def test_int6_tiny_layer_all_tokens():
    _check_layer("int6_tiny_d256_e16_top2")


@pytest.mark.parametrize("T", [1, 5])
def test_mixed_precision_layer_at_decode_sizes(T):
    # int4 routed, int6 shared, int8 router with few tokens: the four calls on the GEMV
    # kernels (the mixed formats do not take the decode layer's two launches)
    _check_layer("prefill_32768_mixed", T=T, stream=T, sample=T)


def test_prefill_8192_zipf():
    _check_layer("prefill_8192_zipf", sample=24, tiles=True)


def test_prefill_batch_ids_equal_smaller_calls():
    """A token's ids and gate weights do not depend on the batch it is routed in: the same
    16 tokens inside the 8192-token Zipf prefill (bounded MFMA router), alone (the decode
    layer, and moe_route's one-launch form), four at a time (one launch), 16 together
    (GEMV logits + selection kernel) and among 100 with logits requested (fixed-order LDS
    GEMM) all get the same ids and weights, bit for bit."""
    moe = _gpu()
    w, lay, _ = _setup("prefill_8192_zipf")
    x = synth.make_tokens(w, seed=0, device="cuda", stream=41)
    big, _ = _run(moe, lay, w, x)
    ids_big = big.ids[:w.T].clone()
    wt_big = big.weights[:w.T].clone().view(torch.int32)
    del big
    rng = np.random.default_rng(8192)
    toks = np.unique(np.concatenate([[0, 1, w.T // 2, w.T - 1],
                                     rng.choice(w.T, 12, replace=False)]))[:16]
    tt = torch.from_numpy(toks).long().cuda()

    one = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, 1)
    for t in toks:
        xt = x[int(t):int(t) + 1].contiguous()
        one.decode(xt)
        torch.cuda.synchronize()
        assert torch.equal(one.ids[:1], ids_big[int(t):int(t) + 1]), "token %d decode" % t
        assert torch.equal(one.weights[:1].view(torch.int32), wt_big[int(t):int(t) + 1])
        one.route_only(xt)
        torch.cuda.synchronize()
        assert torch.equal(one.ids[:1], ids_big[int(t):int(t) + 1]), "token %d route" % t
        assert torch.equal(one.weights[:1].view(torch.int32), wt_big[int(t):int(t) + 1])
    for T in (4, 16):
        small, _ = _run(moe, lay, w, x[tt[:T]].contiguous())
        assert torch.equal(small.ids[:T], ids_big[tt[:T]]), "T %d" % T
        assert torch.equal(small.weights[:T].view(torch.int32), wt_big[tt[:T]]), "T %d" % T
    others = torch.from_numpy(np.setdiff1d(np.arange(w.T), toks)[:100 - toks.size]).long().cuda()
    idx = torch.cat([tt, others])
    lg = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, 100, keep_logits=True)
    lg.forward(x[idx].contiguous())
    torch.cuda.synchronize()
    moe.moe_check_device_error()
    assert torch.equal(lg.ids[:100], ids_big[idx])
    assert torch.equal(lg.weights[:100].view(torch.int32), wt_big[idx])


def test_prefill_32768_mixed_zipf():
    _check_layer("prefill_32768_mixed", sample=16, tiles=True)


def test_prefill_32768_mixed_uniform():
    _check_layer("prefill_32768_mixed", sample=16, bias="none", tiles=True)


def test_batch_invariance_and_rerun_determinism():
    moe = _gpu()
    w, lay, _ = _setup("decode_d2048_e512_top10_t1", bias="zipf")
    x4 = synth.make_tokens(w, T=4, device="cuda", stream=99)
    layer4, out4 = _run(moe, lay, w, x4)
    out4 = out4.clone()
    ids4, w4 = layer4.ids[:4].clone(), layer4.weights[:4].clone()
    for t in range(4):
        layer1, out1 = _run(moe, lay, w, x4[t:t + 1].contiguous())
        assert torch.equal(layer1.ids[:1], ids4[t:t + 1])
        assert torch.equal(layer1.weights[:1], w4[t:t + 1])
        assert torch.equal(out1, out4[t:t + 1])
    layer4b, out4b = _run(moe, lay, w, x4)
    assert torch.equal(out4b, out4)


def test_stacked_residual():
    # x_next = bf16(x + bf16(out)): the GPU's fused residual must equal the same two fp32
    # steps done by torch on the host from the GPU's own plain output, and stay within the
    # layer tolerance of the oracle's x_next built from the oracle's own output.
    moe = _gpu()
    w, lay, (r_h, ex_h, sh_h) = _setup("tiny_d256_e16_top2")
    x = synth.make_tokens(w, device="cuda", stream=5)
    layer = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, w.T)
    plain = layer.forward(x).clone()
    nxt = torch.empty_like(x)
    layer.forward(x, residual=x, out=nxt)
    torch.cuda.synchronize()
    host_sum = (x.cpu().float() + plain.cpu().float()).to(torch.bfloat16)
    assert torch.equal(nxt.cpu(), host_sum)
    res = oracle.layer_tokens(r_h, ex_h, sh_h, si.bits16(x), np.arange(w.T, dtype=np.int32),
                              w.k)
    ref_next = oracle.residual(si.bits16(x), res["out"])
    ref = (ref_next.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    _close(_bf16_np(nxt), ref, "residual")


def test_zero_tokens_and_bad_ids():
    moe = _gpu()
    E, k = 16, 2
    ids = torch.tensor([[0, 3], [16, 2], [5, -1]], dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    sp = torch.full((6,), -7, dtype=torch.int32, device="cuda")
    pp = torch.full((6,), -7, dtype=torch.int32, device="cuda")
    moe.moe_permute(ids, 3, k, E, offsets, sp, pp)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_check_device_error()
    assert ei.value.status == moe._lib.MOE_ERR_DEVICE
    off_ref, sp_ref, pp_ref, bad = oracle.permute(ids.cpu().numpy(), E)
    assert bad == 2
    assert np.array_equal(offsets.cpu().numpy(), off_ref)
    assert np.array_equal(sp[:4].cpu().numpy(), sp_ref[:4])
    assert np.array_equal(pp.cpu().numpy(), pp_ref)
    moe.moe_check_device_error()          # flag was cleared by the previous check
    # T = 0: route and combine are no-ops
    w, lay, _ = _setup("tiny_d256_e16_top2")
    layer = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, 4)
    out = layer.forward(torch.empty((0, w.d), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert out.shape == (0, w.d)
