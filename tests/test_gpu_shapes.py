"""GPU: the layer at every (d_model, d_ff) pair that has GEMV and decode kernels besides the
workloads' own ((256, 128) and (2048, 512)), and at one that only the grouped GEMM serves,
against the oracle.  16 experts, top-4 plus the shared expert; T = 1 and 4 (GEMV by ballot,
and the decode layer, which must equal the four calls bit for bit), 20 (80 pairs: the GEMV in
sorted mode), 300 (1200 pairs: the grouped MFMA GEMM, the shared expert dense on it too) and
600 (the router's bounded MFMA form).  int8 routers where the router has an int8 kernel (d >= 1024), int3 / int6 experts on two of
the shapes.  Bar as everywhere: ids bit-exact, weights |dw| <= 1e-6, rows and outputs within
2e-2 + 1e-2 |r| and rel-Frobenius 1e-2."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import inputs as si

pytestmark = pytest.mark.gpu

ATOL, RTOL, FROB = 2e-2, 1e-2, 1e-2

SHAPES = [
    # (d, F, routed, shared, router)
    (1024, 512, "int4_g32", "int4_g32", "int8_row"),
    (2048, 1024, "int3_g32", "int3_g32", "fp32"),
    (2048, 2048, "int4_g32", "int4_g32", "fp32"),
    (4096, 1024, "int6_g32", "int6_g32", "int8_row"),
    (512, 256, "int4_g32", "int4_g32", "fp32"),        # no GEMV kernel: grouped GEMM only
]


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_sparse_moe_router_amd as moe
    return moe


def _workload(i, d, F, routed, shared, router):
    return synth.Workload("shape_d%d_f%d" % (d, F), 40 + i, d=d, E=16, k=4, F=F, T=1,
                          routed_fmt=routed, shared_fmt=shared, router_fmt=router)


def _close(got, ref, what):
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), "%s: %d elements out of tolerance, max err %.3g" % (
        what, int(bad.sum()), float(err.max()))
    frob = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert frob <= FROB, "%s: rel-Frobenius %.3g" % (what, frob)


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _check_layer(moe, w, lay, T, seed, can_decode):
    """forward() at T tokens against the oracle (all tokens up to 20, else a sample that
    holds the first and last), and decode() against forward() bit for bit where it runs.
    Returns (ids [T][k], weights [T][k]) of the GPU."""
    d = w.d
    hosts = (lay.router.host(), lay.routed.host(), lay.shared.host())
    x = synth.make_tokens(w, T=T, seed=seed, device="cuda", stream=T)
    m = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, T)
    out = m.forward(x).clone()
    torch.cuda.synchronize()
    moe.moe_check_device_error()
    if T <= 20:
        toks = np.arange(T, dtype=np.int32)
    else:
        rng = np.random.default_rng(d + w.F + T)
        toks = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 30, replace=False)]))
        toks = toks.astype(np.int32)
    ref = oracle.layer_tokens(*hosts, si.bits16(x), toks, w.k, keep_pairs=True)
    ids = m.ids[:T].cpu().numpy()
    wts = m.weights[:T].cpu().numpy()
    assert np.array_equal(ids[toks], ref["ids"]), "T %d ids" % T
    assert np.abs(wts[toks] - ref["w"]).max() <= 1e-6
    pos = m.pair_pos[:T * w.k].cpu().numpy().reshape(T, w.k)[toks]
    got_pairs = _f64(m.y_pairs[torch.from_numpy(pos.reshape(-1)).long().cuda()])
    _close(got_pairs, ref["y_sel"].reshape(-1, d), "T %d pair rows" % T)
    _close(_f64(m.y_shared[torch.from_numpy(toks).long().cuda()]), ref["y_shared"],
           "T %d shared rows" % T)
    _close(_f64(out[torch.from_numpy(toks).long().cuda()]), ref["out"], "T %d out" % T)
    assert m.can_decode == can_decode, "T %d" % T
    if m.can_decode:
        dec = m.decode(x).clone()
        torch.cuda.synchronize()
        moe.moe_check_device_error()
        assert torch.equal(dec.view(torch.int16), out.view(torch.int16)), \
            "T %d: decode layer differs from the four calls" % T
    del m
    return ids, wts


@pytest.mark.parametrize("i", range(len(SHAPES)))
def test_layer_shapes_against_oracle(i):
    moe = _gpu()
    d, F, routed, shared, router = SHAPES[i]
    w = _workload(i, d, F, routed, shared, router)
    lay = synth.make_layer(w, seed=0, device="cuda", bias="zipf")
    for T in (1, 4, 20, 300, 600):
        print("case d=%d F=%d %s/%s/%s T=%d" % (d, F, routed, shared, router, T), flush=True)
        # the decode layer runs for at most 64 pairs on the shapes with GEMV kernels
        _check_layer(moe, w, lay, T, 5, T * w.k <= 64 and (d, F) != (512, 256))


@pytest.mark.parametrize("E,k,bias", [(1, 1, "none"), (8, 8, "zipf"), (16, 1, "zipf"),
                                      (64, 64, "none")])
def test_degenerate_routing(E, k, bias):
    """The method's degenerate routings at d 256 / F 128: one routed expert (the router
    decides nothing: every id 0, every weight exactly 1), every expert selected (k = E: the
    ids are a permutation of all experts in descending logit order, the weights a softmax
    over all of them, summing to 1), and top-1 (a single pair per token, weight exactly 1).
    k = E = 64 at one token fills the 64 pairs of the decode layer (the four calls take the
    sorted GEMV from 25 pairs);
    T = 4, 20 and 300 take the sorted GEMV, the GEMV / grouped GEMM split and the grouped
    GEMM."""
    moe = _gpu()
    w = synth.Workload("degenerate_e%d_k%d" % (E, k), 60 + E + k, d=256, E=E, k=k, F=128, T=1)
    lay = synth.make_layer(w, seed=0, device="cuda", bias=bias)
    for T in (1, 4, 20, 300):
        print("case E=%d k=%d bias=%s T=%d" % (E, k, bias, T), flush=True)
        ids, wts = _check_layer(moe, w, lay, T, 7, T * k <= 64)
        if k == 1:
            assert np.all(wts == 1.0)
        if E == 1:
            assert np.all(ids == 0)
        if k == E:
            assert np.array_equal(np.sort(ids, axis=1), np.tile(np.arange(E), (T, 1)))
            assert np.all(np.abs(wts.astype(np.float64).sum(axis=1) - 1.0) <= k * 2.0 ** -23)


@pytest.mark.parametrize("E,k", [(1000, 10), (1024, 10), (1024, 64)])
def test_most_experts(E, k):
    """The largest expert counts the library takes (E up to 1024: 16 router keys per lane in
    every selection form), at d 256 / F 128, Zipf routing, T = 1 and 4 (one-launch router,
    the decode layer selecting in its gate/up blocks), 20 (logits then the selection
    kernel), 300 (the split router past 64 tokens) and 600 (the bounded MFMA router),
    against the oracle."""
    moe = _gpu()
    w = synth.Workload("most_experts_e%d_k%d" % (E, k), 70 + k, d=256, E=E, k=k, F=128, T=1)
    lay = synth.make_layer(w, seed=0, device="cuda", bias="zipf")
    for T in (1, 4, 20, 300, 600):
        print("case E=%d k=%d T=%d" % (E, k, T), flush=True)
        ids, wts = _check_layer(moe, w, lay, T, 9, T * k <= 64)
        assert np.all((ids >= 0) & (ids < E))
        assert all(len(set(r)) == k for r in ids.tolist())
