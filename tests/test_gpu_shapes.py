"""GPU: the layer at every (d_model, d_ff) pair that has GEMV and decode kernels besides the
workloads' own ((256, 128) and (2048, 512)), and at one that only the grouped GEMM serves,
against the oracle.  16 experts, top-4 plus the shared expert; T = 1 and 4 (GEMV by ballot,
and the decode layer, which must equal the four calls bit for bit), 20 (80 pairs: the GEMV in
sorted mode) and 300 (1200 pairs: the grouped MFMA GEMM, the shared expert dense on it too).
int8 routers where the router has an int8 kernel (d >= 1024), int3 / int6 experts on two of
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


@pytest.mark.parametrize("i", range(len(SHAPES)))
def test_layer_shapes_against_oracle(i):
    moe = _gpu()
    d, F, routed, shared, router = SHAPES[i]
    w = _workload(i, d, F, routed, shared, router)
    lay = synth.make_layer(w, seed=0, device="cuda", bias="zipf")
    hosts = (lay.router.host(), lay.routed.host(), lay.shared.host())
    for T in (1, 4, 20, 300):
        print("case d=%d F=%d %s/%s/%s T=%d" % (d, F, routed, shared, router, T), flush=True)
        x = synth.make_tokens(w, T=T, seed=5, device="cuda", stream=T)
        m = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, T)
        out = m.forward(x).clone()
        torch.cuda.synchronize()
        moe.moe_check_device_error()
        if T <= 20:
            toks = np.arange(T, dtype=np.int32)
        else:
            rng = np.random.default_rng(d + F + T)
            toks = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 30, replace=False)]))
            toks = toks.astype(np.int32)
        ref = oracle.layer_tokens(*hosts, si.bits16(x), toks, w.k, keep_pairs=True)
        ids = m.ids[:T].cpu().numpy()
        assert np.array_equal(ids[toks], ref["ids"]), "T %d ids" % T
        assert np.abs(m.weights[:T].cpu().numpy()[toks] - ref["w"]).max() <= 1e-6
        pos = m.pair_pos[:T * w.k].cpu().numpy().reshape(T, w.k)[toks]
        got_pairs = _f64(m.y_pairs[torch.from_numpy(pos.reshape(-1)).long().cuda()])
        _close(got_pairs, ref["y_sel"].reshape(-1, d), "T %d pair rows" % T)
        _close(_f64(m.y_shared[torch.from_numpy(toks).long().cuda()]), ref["y_shared"],
               "T %d shared rows" % T)
        _close(_f64(out[torch.from_numpy(toks).long().cuda()]), ref["out"], "T %d out" % T)
        # the decode layer runs for at most 64 pairs on the shapes with GEMV kernels
        assert m.can_decode == (T * w.k <= 64 and (d, F) != (512, 256)), "T %d" % T
        if m.can_decode:
            dec = m.decode(x).clone()
            torch.cuda.synchronize()
            moe.moe_check_device_error()
            assert torch.equal(dec.view(torch.int16), out.view(torch.int16)), \
                "T %d: decode layer differs from the four calls" % T
        del m
