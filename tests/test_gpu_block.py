"""GPU: the MoE block of a stacked model -- pre-layer RMS norm, the layer, gated residual --
against the CPU oracle and against its own composition.

Reading (the pages put a gated residual on the GPU without a formula, 本地部署Qwen3.8-Flash-Next
模型的两条路线, section 硬件形态决定了各自的走法): x_next = bf16(x + bf16(sigmoid(z) * out)),
out = the layer on xn = RMSNorm(x), z = <gate_w, xn> + gate_b.  48 blocks are stacked
[Strata 与 Qwen3.8-Flash-Next (telli.sh), section 稀疏架构创造了机会].
Bar: xn, z, ids bit-exact; weights |dw| <= 1e-6; x_next |g - r| <= 2e-2 + 1e-2 |r| and the
update within rel-Frobenius 1e-2 of the oracle's plus the stream's own bf16 rounding;
moe_block_decode equal to the composition bit for bit.
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


def _f64_bits(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32).astype(np.float64)


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _close_next(got, res, x, what):
    """x_next elementwise within the layer tolerance of the oracle's x_next; and the block's
    update within rel-Frobenius 1e-2 of the oracle's unrounded update g * out, on top of the
    bf16 rounding of the stream itself (half an ulp of x_next per element: every bf16
    residual stream pays it, and at |x| ~ 1 it is a few per cent of an update ~ 0.1)."""
    ref = _f64_bits(res["x_next"])
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), "%s: %d elements out of tolerance, max err %.3g" % (
        what, int(bad.sum()), float(err.max()))
    exact = x + res["update"]
    floor = np.linalg.norm(2.0 ** -9 * np.abs(exact))
    dev = np.linalg.norm(got - exact)
    assert dev <= FROB * np.linalg.norm(res["update"]) + floor, \
        "%s: ||x_next - (x + update)|| = %.4g > %.4g + %.4g" % (
            what, dev, FROB * np.linalg.norm(res["update"]), floor)
    return float(err.max())


@pytest.mark.parametrize("d", [256, 2048, 4096])
def test_rmsnorm_bit_exact(d):
    moe = _gpu()
    g = torch.Generator(device="cuda").manual_seed(d)
    T = 1024
    x = torch.randn((T, d), generator=g, device="cuda")
    # rows of very different scales, an all-zero row, a row with a single element
    scale = 2.0 ** torch.randint(-40, 40, (T, 1), generator=g, device="cuda").float()
    x = (x * scale).to(torch.bfloat16)
    x[3] = 0
    x[4] = 0
    x[4, 5] = 1.5
    gamma = (1 + 0.1 * torch.randn((d,), generator=g, device="cuda")).float()
    gw = (0.02 * torch.randn((d,), generator=g, device="cuda")).float()
    xh = si.bits16(x)
    for eps, gate in ((1e-6, True), (0.0, False)):
        nd = moe.norm_desc(gamma, eps, gw if gate else None, 0.25)
        xn = torch.empty_like(x)
        z = torch.empty((T,), dtype=torch.float32, device="cuda")
        moe.moe_rmsnorm(nd, x, T, d, xn, z)
        torch.cuda.synchronize()
        ref, _ = oracle.rmsnorm(xh, gamma.cpu().numpy(), eps)
        keep = np.ones(T, bool)
        if eps == 0.0:
            keep[3] = False              # 0/0: the all-zero row has no norm without eps
        got = si.bits16(xn)
        assert np.array_equal(got[keep], ref[keep]), "d %d eps %g: %d values differ" % (
            d, eps, int((got[keep] != ref[keep]).sum()))
        if gate:
            zr = oracle.gate_logits(gw.cpu().numpy(), 0.25, ref)
            assert np.array_equal(z.cpu().numpy().view(np.uint32), zr.view(np.uint32))


def _layer(name, bias, gate=True, seed=0, layer=0):
    w = synth.WORKLOADS[name]
    lay = synth.make_layer(w, seed=seed, layer=layer, device="cuda", bias=bias)
    nrm = synth.make_norm(w, seed=seed, layer=layer, device="cuda", gate=gate)
    return w, lay, nrm


@pytest.mark.parametrize("name,bias,T,gate", [
    ("decode_d2048_e512_top10_t1", None, 1, True),
    ("decode_d2048_e512_top10_t1", None, 4, True),
    ("decode_sweep_48_layers", "zipf", 1, True),
    ("decode_sweep_48_layers", "zipf", 4, True),
    ("decode_sweep_48_layers", "zipf", 4, False),
    ("tiny_d256_e16_top2", None, 16, True),
    ("int6_d2048_e64_top10", None, 4, True),      # int6 experts, int8 router
    ("int6_d2048_e64_top10", None, 1, False),
])
def test_block_decode_against_composition_and_oracle(name, bias, T, gate):
    moe = _gpu()
    w, lay, nrm = _layer(name, bias, gate)
    print("case %s bias=%s T=%d gate=%s" % (name, bias, T, gate), flush=True)
    x = (synth.make_tokens(w, T=T, seed=51, device="cuda").float() * 1.7).to(torch.bfloat16)
    a = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, T, norm=nrm)
    b = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, T, norm=nrm)
    assert b.can_decode
    ref = a.block_forward(x).clone()
    for rep in range(2):
        got = b.block_decode(x)
        torch.cuda.synchronize()
        moe.moe_check_device_error()
        assert torch.equal(a.ids[:T], b.ids[:T])
        assert torch.equal(a.weights[:T].view(torch.int32), b.weights[:T].view(torch.int32))
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), \
            "rep %d: %d values differ" % (rep, int((got.view(torch.int16) !=
                                                     ref.view(torch.int16)).sum()))
    # out aliasing x
    buf = x.clone()
    b.block_decode(buf, out=buf)
    torch.cuda.synchronize()
    assert torch.equal(buf.view(torch.int16), ref.view(torch.int16))
    # the oracle: xn and z bit-exact (from the composition's buffers), routing, x_next
    res = oracle.block_tokens(nrm.host(), lay.router.host(), lay.routed.host(),
                              lay.shared.host(), si.bits16(x), np.arange(T, dtype=np.int32),
                              w.k)
    assert np.array_equal(si.bits16(a.xn[:T]), res["xn"])
    if gate:
        assert np.array_equal(a.z[:T].cpu().numpy().view(np.uint32), res["z"].view(np.uint32))
    assert np.array_equal(b.ids[:T].cpu().numpy(), res["ids"])
    assert np.abs(b.weights[:T].cpu().numpy() - res["w"]).max() <= 1e-6
    _close_next(_f64(ref), res, _f64(x), name)


@pytest.mark.parametrize("name,bias,T", [
    ("tiny_d256_e16_top2", None, 300),             # split router, grouped GEMM
    ("tiny_d256_e16_top2", None, 600),             # bounded router, grouped GEMM
    ("decode_d2048_e512_top10_t1", "zipf", 96),
])
def test_block_forward_many_tokens_against_oracle(name, bias, T):
    moe = _gpu()
    w, lay, nrm = _layer(name, bias, True)
    x = synth.make_tokens(w, T=T, seed=52, device="cuda")
    a = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, T, norm=nrm)
    out = a.block_forward(x).clone()
    torch.cuda.synchronize()
    moe.moe_check_device_error()
    toks = np.unique(np.concatenate([[0, T - 1], np.arange(0, T, 7)])).astype(np.int32)
    res = oracle.block_tokens(nrm.host(), lay.router.host(), lay.routed.host(),
                              lay.shared.host(), si.bits16(x), toks, w.k)
    assert np.array_equal(si.bits16(a.xn[:T])[toks], res["xn"])
    assert np.array_equal(a.ids[:T].cpu().numpy()[toks], res["ids"])
    _close_next(_f64(out)[toks], res, _f64(x)[toks], name)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_block_chain_48_teacher_forced():
    """48 normed, gated blocks chained as the decode sweep runs them, at one and four tokens
    per step; every block checked by the oracle on the GPU's own input x_l."""
    moe = _gpu()
    w = synth.WORKLOADS["decode_sweep_48_layers"]
    lays = [synth.make_layer(w, seed=0, layer=l, device="cuda") for l in range(w.layers)]
    nrms = [synth.make_norm(w, seed=0, layer=l, device="cuda") for l in range(w.layers)]
    chains = {}
    for T in (1, 4):
        mls = [moe.MoeLayer(L.router, L.routed, L.shared, w.k, T, norm=N)
               for L, N in zip(lays, nrms)]
        xs = [synth.make_tokens(w, T=T, seed=0, device="cuda")]
        xs += [torch.empty_like(xs[0]) for _ in range(w.layers)]
        for l in range(w.layers):
            mls[l].block_decode(xs[l], out=xs[l + 1])
        torch.cuda.synchronize()
        moe.moe_check_device_error()
        ids = [m.ids[:T].cpu().numpy().copy() for m in mls]
        chains[T] = (xs, ids)
        rms = [float(t.float().pow(2).mean().sqrt()) for t in xs]
        print("chain T=%d built; rms(x) at layers 0, 16, 32, 48: %.3f %.3f %.3f %.3f"
              % (T, rms[0], rms[16], rms[32], rms[48]), flush=True)
        assert all(np.isfinite(rms)) and max(rms) < 8.0
        del mls
    worst = {1: 0.0, 4: 0.0}
    for l in range(w.layers):
        L, N = lays[l], nrms[l]
        hosts = (N.host(), L.router.host(), L.routed.host(), L.shared.host())
        for T, (xs, ids) in chains.items():
            res = oracle.block_tokens(*hosts, si.bits16(xs[l]), np.arange(T, dtype=np.int32),
                                      w.k)
            assert np.array_equal(ids[l], res["ids"]), "T %d layer %d ids" % (T, l)
            worst[T] = max(worst[T], _close_next(_f64(xs[l + 1]), res, _f64(xs[l]),
                                                 "T %d layer %d" % (T, l)))
        if l % 8 == 7:
            print("layers 0..%d checked" % l, flush=True)
    print("48 blocks at T = 1 and 4: ids bit-exact, max |x_next - oracle| %.3g / %.3g"
          % (worst[1], worst[4]), flush=True)
