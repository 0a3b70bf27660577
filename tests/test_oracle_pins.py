"""Pins of the CPU oracle against facts that do not come from the oracle itself:
hand-derived fixtures (tests/golden), IEEE definitions checked against numpy/torch,
closed forms, invariants, brute force on tiny inputs, and textbook special cases.

Page citations: 512 routed experts, 10 active plus 1 shared per token [Strata 与
Qwen3.8-Flash-Next (telli.sh), section 稀疏架构创造了机会]; 4-bit experts, 6-bit mixed
layers, 8-bit dense projection [本地部署Qwen3.8-Flash-Next模型的两条路线 (blog.cycleuser.org),
section 精度和内存占用].
"""
import itertools
import math
import os
import random

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TINY = synth.WORKLOADS["tiny_d256_e16_top2"]


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.strip()
            if ln and not ln.startswith("#"):
                yield ln


# ---------------------------------------------------------------- number formats

def test_fp16_golden():
    for ln in _lines("fp16_bf16.txt"):
        kind, a, b = ln.split()
        if kind == "fp16":
            v = oracle.half_to_double(int(a, 16))
            assert v == float(b) and math.copysign(1, v) == math.copysign(1, float(b)), ln


def test_fp16_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got), np.isinf(ref))


def test_bf16_rounding_golden():
    for ln in _lines("fp16_bf16.txt"):
        kind, a, b = ln.split()
        if kind == "bf16":
            assert oracle.double_to_bf16(float(a)) == int(b, 16), ln


def test_bf16_array_rounding_golden():
    vals, want = [], []
    for ln in _lines("fp16_bf16.txt"):
        kind, a, b = ln.split()
        if kind == "bf16":
            vals.append(float(a))
            want.append(int(b, 16))
    got = oracle.double_to_bf16_array(np.array(vals))
    assert got.tolist() == want


def test_bf16_rounding_matches_torch_on_fp32_values():
    g = torch.Generator().manual_seed(7)
    v = torch.randn(20000, generator=g) * torch.exp(torch.randn(20000, generator=g) * 8)
    v = torch.cat([v, torch.tensor([0.0, -0.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 65504.0])])
    ref = v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.double_to_bf16(float(x)) for x in v.numpy()], np.uint16)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- weight codes

def test_code_golden():
    fmts = {"int4": oracle.FMT_INT4_G32, "int6": oracle.FMT_INT6_G32,
            "int3": oracle.FMT_INT3_G32, "int2": oracle.FMT_INT2_G32,
            "int8": oracle.FMT_INT8_ROW}
    for ln in _lines("codes.txt"):
        kind, hexbytes, *codes = ln.split()
        row = np.frombuffer(bytes.fromhex(hexbytes), np.uint8)
        got = [oracle.code(fmts[kind], row, c) for c in range(len(codes))]
        assert got == [int(c) for c in codes], ln


@pytest.mark.parametrize("fmt,qmin,qmax,packer", [
    (oracle.FMT_INT4_G32, -8, 7, si.pack_int4),
    (oracle.FMT_INT6_G32, -32, 31, si.pack_int6),
    (oracle.FMT_INT3_G32, -4, 3, si.pack_int3),
    (oracle.FMT_INT2_G32, -2, 1, si.pack_int2),
])
def test_pack_unpack_bijection(fmt, qmin, qmax, packer):
    # every code value at every position of a group (positions cycle through the codes)
    n = qmax - qmin + 1
    K = 32 * n
    q = torch.tensor([qmin + ((c + c // 32) % n) for c in range(K)], dtype=torch.int32)
    row = packer(q[None, :])[0].numpy()
    got = [oracle.code(fmt, row, c) for c in range(K)]
    assert got == q.tolist()


@pytest.mark.parametrize("fmt,quant,qmax", [
    (oracle.FMT_INT4_G32, si.quantize_int4_g32, 7),
    (oracle.FMT_INT6_G32, si.quantize_int6_g32, 31),
    (oracle.FMT_INT3_G32, si.quantize_int3_g32, 3),
    (oracle.FMT_INT2_G32, si.quantize_int2_g32, 1),
])
def test_dequant_within_half_step_of_weight(fmt, quant, qmax):
    # closed-form bound of round-to-nearest quantisation: |w - s*q| <= s/2 per element,
    # and no code is clamped away from its nearest value (|w/s| <= qmax*(1 + 2^-11)).
    g = torch.Generator().manual_seed(3)
    w = torch.randn((8, 256), generator=g) * 0.02
    w[0, :32] = 0.0                                     # an all-zero group -> s = 0
    packed, s = quant(w)
    deq = oracle.dequant_rows(fmt, packed.numpy(), si.bits16(s), 256)
    sd = np.repeat(s.to(torch.float64).numpy(), 32, axis=1)
    err = np.abs(deq - w.double().numpy())
    assert np.all(err <= sd / 2 + 1e-18)
    assert np.all(deq[0, :32] == 0.0)
    # exactness: s*q is exact in fp32 (11-bit x <= 6-bit significands), so the value
    # survives a round trip through binary32 unchanged
    assert np.array_equal(deq.astype(np.float32).astype(np.float64), deq)


def test_int8_row_dequant():
    g = torch.Generator().manual_seed(4)
    w = torch.randn((4, 1024), generator=g) * 0.02
    q, s = si.quantize_int8_row(w)
    row = q[1].numpy().view(np.uint8)
    codes = [oracle.code(oracle.FMT_INT8_ROW, row, c) for c in range(1024)]
    assert codes == q[1].tolist()
    sv = oracle.half_to_double(int(si.bits16(s)[1]))
    assert np.all(np.abs(np.array(codes) * sv - w[1].double().numpy()) <= sv / 2 + 1e-18)


# ---------------------------------------------------------------- router

def _router_case(d, triples, bias=None):
    x = torch.zeros((1, d), dtype=torch.bfloat16)
    w = torch.zeros((1, d), dtype=torch.float32)
    for idx, xv, wv in triples:
        x[0, idx] = xv
        w[0, idx] = wv
    r = {"fmt": oracle.FMT_FP32, "E": 1, "d": d, "w": w.numpy(), "scale": None,
         "bias": None if bias is None else np.array([bias], np.float32)}
    return oracle.router_logits(r, si.bits16(x))[0, 0]


def test_router_order_golden():
    n = 0
    for ln in _lines("router_order.txt"):
        head, *trip = [p.strip() for p in ln.split("|")]
        name, d, expect = head.split()
        triples = [(int(a), float(b), float(c)) for a, b, c in (t.split() for t in trip)]
        for tx in triples:   # fixture values must be exact in their formats
            assert float(torch.tensor(tx[1]).to(torch.bfloat16)) == tx[1]
            assert float(np.float32(tx[2])) == tx[2]
        got = _router_case(int(d), triples)
        assert got == np.float32(float(expect)), (name, got)
        n += 1
    assert n == 4


def test_router_bias_added_after_sum():
    got = _router_case(256, [(0, 1.0, 2.0), (4, 1.0, 3.0)], bias=0.5)
    assert got == np.float32(5.5)


def test_router_exact_on_integers_matches_matmul():
    # small integers: every product and partial sum is exact, so any order gives the
    # library matmul's value
    g = torch.Generator().manual_seed(11)
    E, d, T = 16, 512, 5
    x = torch.randint(-4, 5, (T, d), generator=g).to(torch.bfloat16)
    w = torch.randint(-8, 9, (E, d), generator=g).to(torch.float32)
    b = torch.randint(-3, 4, (E,), generator=g).to(torch.float32)
    r = {"fmt": oracle.FMT_FP32, "E": E, "d": d, "w": w.numpy(), "bias": b.numpy()}
    got = oracle.router_logits(r, si.bits16(x))
    ref = (x.double() @ w.double().T + b.double()).numpy()
    assert np.array_equal(got.astype(np.float64), ref)


def test_router_int8_exact_on_integers():
    g = torch.Generator().manual_seed(12)
    E, d, T = 8, 1024, 3
    x = torch.randint(-3, 4, (T, d), generator=g).to(torch.bfloat16)
    q = torch.randint(-127, 128, (E, d), generator=g).to(torch.int8)
    s = torch.full((E,), 0.25, dtype=torch.float16)     # power of two: exact scaling
    b = torch.randint(-3, 4, (E,), generator=g).to(torch.float32)
    r = {"fmt": oracle.FMT_INT8_ROW, "E": E, "d": d, "w": q.numpy(),
         "scale": si.bits16(s), "bias": b.numpy()}
    got = oracle.router_logits(r, si.bits16(x))
    ref = ((x.double() @ q.double().T) * 0.25 + b.double()).numpy()
    assert np.array_equal(got.astype(np.float64), ref)


def test_router_int8_order_golden():
    # hand-derived int8 cases (tests/golden/router_int8_order.txt): the code dealing (16
    # per vector), the chain order, the butterfly and the two roundings of scale and bias
    # each change the expected bits
    n = 0
    for ln in _lines("router_int8_order.txt"):
        head, *trip = [p.strip() for p in ln.split("|")]
        name, d, s_hex, bias, expect = head.split()
        d = int(d)
        x = torch.zeros((1, d), dtype=torch.bfloat16)
        q = torch.zeros((1, d), dtype=torch.int8)
        for t in trip:
            idx, xv, qv = t.split()
            assert float(torch.tensor(float(xv)).to(torch.bfloat16)) == float(xv)
            assert -127 <= int(qv) <= 127
            x[0, int(idx)] = float(xv)
            q[0, int(idx)] = int(qv)
        assert float(np.float32(float(bias))) == float(bias)
        r = {"fmt": oracle.FMT_INT8_ROW, "E": 1, "d": d, "w": q.numpy(),
             "scale": np.array([int(s_hex, 16)], np.uint16),
             "bias": np.array([float(bias)], np.float32)}
        got = oracle.router_logits(r, si.bits16(x))[0, 0]
        assert got == np.float32(float(expect)), (name, got)
        n += 1
    assert n == 4


def test_router_fp32_within_rounding_bound_of_exact():
    # Higham's bound for a chain of n fp32 roundings: |fl - exact| <= gamma_n * sum|x*w|,
    # n = per-lane chain length (d/256 vectors * 4 elements) + 6 butterfly levels.
    g = torch.Generator().manual_seed(5)
    E, d, T = 64, 2048, 6
    x = torch.randn((T, d), generator=g).to(torch.bfloat16)
    rw = torch.randn((E, d), generator=g) * 0.02
    r = {"fmt": oracle.FMT_FP32, "E": E, "d": d, "w": rw.numpy(), "bias": None}
    l32 = oracle.router_logits(r, si.bits16(x)).astype(np.float64)
    l64 = oracle.router_logits_fp64(r, si.bits16(x))
    exact = x.double() @ rw.double().T
    assert np.allclose(l64, exact.numpy(), rtol=0, atol=1e-12)
    n = d // 256 * 4 + 6
    u = 2.0 ** -24
    gamma = n * u / (1 - n * u)
    mag = (x.double().abs() @ rw.double().abs().T).numpy()
    assert np.all(np.abs(l32 - exact.numpy()) <= gamma * mag)


def _exact_logits(x, w, scale=None, bias=None):
    """Real-number logits in torch fp64, independent of the oracle: bf16 x fp32 (or int8)
    products and their sums are exact to ~1e-16 relative in double."""
    l = x.double() @ torch.as_tensor(w).double().T
    if scale is not None:
        l = l * torch.as_tensor(scale).double()[None, :]
    if bias is not None:
        l = l + torch.as_tensor(bias).double()[None, :]
    return l.numpy()


@pytest.mark.parametrize("fmt", ["fp32", "int8"])
def test_router_error_bound_holds_and_is_not_vacuous(fmt):
    # The fp32 logits in the fixed order lie within the rigorous summation bound of the
    # exact value (a theorem of floating-point summation), and the bound is within a few
    # orders of magnitude of the observed error (a bound missing the unit roundoff or the
    # row scale would fail one side).
    g = torch.Generator().manual_seed(11)
    E, d, T = 64, 2048, 8
    x = torch.randn((T, d), generator=g).to(torch.bfloat16)
    bias = (torch.randn(E, generator=g) * 0.5).float().numpy()
    if fmt == "fp32":
        w = (torch.randn((E, d), generator=g) * 0.02).float().numpy()
        r = {"fmt": oracle.FMT_FP32, "E": E, "d": d, "w": w, "bias": bias}
        exact = _exact_logits(x, w, bias=bias)
    else:
        q = torch.randint(-127, 128, (E, d), generator=g).to(torch.int8).numpy()
        s16 = (torch.rand(E, generator=g) * 1e-3 + 1e-4).half()
        r = {"fmt": oracle.FMT_INT8_ROW, "E": E, "d": d, "w": q,
             "scale": s16.view(torch.int16).numpy().view(np.uint16), "bias": bias}
        exact = _exact_logits(x, q.astype(np.float64), scale=s16.double().numpy(), bias=bias)
    xb = si.bits16(x)
    l32 = oracle.router_logits(r, xb).astype(np.float64)
    bnd = oracle.router_error_bound(r, xb)
    err = np.abs(l32 - exact)
    assert np.all(err <= bnd)
    assert (err / bnd).max() > 1e-4
    assert np.allclose(oracle.router_logits_fp64(r, xb), exact, rtol=0, atol=1e-12)


def test_router_error_bound_on_one_sided_rounding():
    # x = 1 and every weight 1 + 2^-21: once a lane's running sum passes 16 each fma adds
    # less than half an ulp and rounds the same way, so the fixed-order result falls
    # short of the exact 2048 (1 + 2^-21) by a sizeable share of the worst-case bound.
    # The bound must hold here and not be inflated by more than a small factor.
    E, d, eps = 2, 2048, 2.0 ** -21
    w = np.full((E, d), np.float32(1 + eps))
    w[1] = -w[1]
    x = torch.ones((1, d)).to(torch.bfloat16)
    r = {"fmt": oracle.FMT_FP32, "E": E, "d": d, "w": w, "bias": None}
    l32 = oracle.router_logits(r, si.bits16(x)).astype(np.float64)[0]
    exact = d * (1 + eps)
    bnd = oracle.router_error_bound(r, si.bits16(x))[0]
    err = np.abs(np.abs(l32) - exact)
    assert l32[0] < exact and l32[1] == -l32[0]
    assert np.all(err <= bnd) and np.all(err / bnd > 0.05)


def _tiny_router(seed, E=16, d=256, T=5):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((T, d), generator=g).to(torch.bfloat16)
    w = (torch.randn((E, d), generator=g) * 0.05).float().numpy()
    return x, w


def test_tie_audit_identical_rows_are_flagged():
    # two identical router rows give exactly equal logits for every token; placing them
    # at ranks k and k + 1 (bias) makes every token's cut a true tie
    x, w = _tiny_router(3)
    E, k = w.shape[0], 2
    w[5] = w[9]
    bias = np.full(E, -50.0, np.float32)
    bias[[0, 5, 9]] = [50.0, 0.0, 0.0]
    r = {"fmt": oracle.FMT_FP32, "E": E, "d": w.shape[1], "w": w, "bias": bias}
    a = oracle.router_tie_audit(r, si.bits16(x), k, factor=1.0)
    assert a["count"] == x.shape[0] and np.all(a["margin"] <= 0)
    # a tie goes to the lower index in both selections, so the sets agree
    assert a["differs"] == 0


def test_tie_audit_separated_cut_is_clear():
    x, w = _tiny_router(4)
    E, k = w.shape[0], 3
    bias = np.zeros(E, np.float32)
    bias[[2, 7, 11]] = 10.0
    r = {"fmt": oracle.FMT_FP32, "E": E, "d": w.shape[1], "w": w, "bias": bias}
    a = oracle.router_tie_audit(r, si.bits16(x), k)
    assert a["count"] == 0 and a["differs"] == 0 and np.all(a["margin"] > 0)
    a0 = oracle.router_tie_audit({**r, "w": np.zeros_like(w), "bias": None}, si.bits16(x), k)
    assert a0["count"] == x.shape[0]          # all logits exactly zero: every cut is a tie


def test_tie_audit_sub_ulp_gap_changes_the_fp32_choice():
    # expert 1 = expert 0 with one weight raised by one ulp where x > 0: exactly, expert 1
    # is larger; where the fp32 chain absorbs the difference the fixed-order logits tie and
    # the lower index (0) is chosen.  The audit must see the different choice and flag it.
    x, w = _tiny_router(6, T=1)
    E, d, k = w.shape[0], w.shape[1], 1
    bias = np.full(E, -50.0, np.float32)
    bias[:2] = 0.0
    xb = si.bits16(x)
    found = False
    for c in np.nonzero(x[0].float().numpy() > 0)[0]:
        w2 = w.copy()
        w2[1] = w2[0]
        w2[1, c] = np.nextafter(w2[0, c], np.float32(np.inf))
        r = {"fmt": oracle.FMT_FP32, "E": E, "d": d, "w": w2, "bias": bias}
        l32 = oracle.router_logits(r, xb)
        if l32[0, 0] == l32[0, 1]:
            found = True
            break
    assert found
    assert _exact_logits(x, w2, bias=bias)[0, 1] > _exact_logits(x, w2, bias=bias)[0, 0]
    a = oracle.router_tie_audit(r, xb, k, factor=1.0)
    assert a["differs"] == 1 and a["count"] == 1
    assert oracle.select_topk(l32, k)[0, 0] == 0


# ---------------------------------------------------------------- pre-layer norm, gate

def _bf16_bits(v):
    return int(si.bits16(torch.tensor([v], dtype=torch.float32).to(torch.bfloat16))[0])


def test_rms_sumsq_order_golden():
    n = 0
    for ln in _lines("rmsnorm.txt"):
        if not ln.startswith("S "):
            continue
        head, *items = [p.strip() for p in ln.split("|")]
        _, name, d, expect = head.split()
        x = np.zeros(int(d), np.uint16)
        for it in items:
            idx, xv = it.split()
            assert float(torch.tensor(float(xv)).to(torch.bfloat16)) == float(xv)
            x[int(idx)] = _bf16_bits(float(xv))
        assert oracle.rms_sumsq(x) == np.float32(float(expect)), name
        n += 1
    assert n == 2


def test_rmsnorm_golden():
    n = 0
    for ln in _lines("rmsnorm.txt"):
        if not ln.startswith("N "):
            continue
        head, *items = [p.strip() for p in ln.split("|")]
        _, name, d, eps, xv, r_hex = head.split()
        d = int(d)
        x = np.full((1, d), _bf16_bits(float(xv)), np.uint16)
        gamma = np.ones(d, np.float32)
        want = {}
        for it in items:
            idx, g, xn_hex = it.split()
            assert float(np.float32(float(g))) == float(g)
            gamma[int(idx)] = float(g)
            want[int(idx)] = int(xn_hex, 16)
        xn, r = oracle.rmsnorm(x, gamma, float(eps))
        assert r.view(np.uint32)[0] == int(r_hex, 16), (name, hex(r.view(np.uint32)[0]))
        for idx, h in want.items():
            assert xn[0, idx] == h, (name, idx, hex(xn[0, idx]))
        if gamma[0] == 1:
            assert (xn[0, gamma == 1] == xn[0, 0]).all()
        n += 1
    assert n == 3


def test_rmsnorm_zero_row_and_eps():
    x = np.zeros((2, 512), np.uint16)
    x[1, 7] = _bf16_bits(1e-3)
    xn, r = oracle.rmsnorm(x, np.ones(512, np.float32), 1e-6)
    assert (xn[0] == 0).all() and np.isfinite(r).all() and (r > 0).all()
    # 1 / sqrt(eps) within two ulps of fp32 (the eps of the empty row dominates)
    assert abs(float(r[0]) - 1.0 / math.sqrt(float(np.float32(1e-6)))) <= 2 * 2.0 ** -24 * 1000
    # a lone element far below sqrt(eps): xn = x * r, r ~ 1/sqrt(1e-6 + 1e-6/512)
    assert xn[1, 7] != 0 and (np.delete(xn[1], 7) == 0).all()


def test_rmsnorm_scale_invariance_and_exact_value():
    # eps = 0: scaling a row by a power of two scales ss by its square exactly, so r and
    # x * r, hence xn, do not change; and xn is within half a bf16 ulp (plus the fp32
    # roundings before it) of the real-number value x * gamma / sqrt(mean(x^2)), which a
    # dropped factor (mean vs sum, a missing square root, gamma unused) would break
    g = torch.Generator().manual_seed(21)
    T, d = 64, 2048
    x = torch.randn((T, d), generator=g).to(torch.bfloat16)
    gamma = (1 + 0.1 * torch.randn(d, generator=g)).numpy().astype(np.float32)
    xn, _ = oracle.rmsnorm(si.bits16(x), gamma, 0.0)
    for k in (-20, -3, 5, 30):
        xs = (x.float() * 2.0 ** k).to(torch.bfloat16)
        assert torch.equal(xs.float(), x.float() * 2.0 ** k)
        assert np.array_equal(oracle.rmsnorm(si.bits16(xs), gamma, 0.0)[0], xn)
    xd = x.double().numpy()
    exact = xd * gamma / np.sqrt((xd ** 2).mean(axis=1, keepdims=True))
    got = (xn.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    # half a bf16 ulp is at most 2^-8 of the value; the fp32 steps before the rounding add
    # well under 2^-16 of it
    assert np.all(np.abs(got - exact) <= (2.0 ** -8 + 2.0 ** -16) * np.abs(exact) + 1e-30)


def test_gated_residual_closed_forms():
    g = torch.Generator().manual_seed(22)
    T, d = 3, 256
    x = torch.randn((T, d), generator=g).to(torch.bfloat16)
    out = torch.randn((T, d), generator=g, dtype=torch.float64).numpy()
    xb = si.bits16(x)
    plain = oracle.residual(xb, out)
    # z large: g = 1 exactly in double -> the plain residual
    assert np.array_equal(oracle.gated_residual(xb, out, np.full(T, 100.0, np.float32)), plain)
    assert np.array_equal(oracle.gated_residual(xb, out, None), plain)
    # z = 0: g = 1/2 exactly -> the plain residual of out / 2
    assert np.array_equal(oracle.gated_residual(xb, out, np.zeros(T, np.float32)),
                          oracle.residual(xb, out / 2))
    # z very negative: g * out rounds to 0 in bf16 -> x unchanged
    assert np.array_equal(oracle.gated_residual(xb, out, np.full(T, -200.0, np.float32)), xb)


# ---------------------------------------------------------------- selection + weights

def _brute_topk(row, k):
    order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
    return order[:k]


def test_topk_brute_force_tiny():
    rnd = random.Random(1)
    for trial in range(3000):
        E = rnd.choice([2, 3, 5, 16, 33])
        k = rnd.randint(1, E)
        pool = [0.0, -0.0, 1.0, -1.0, 0.5] if trial % 2 else None
        row = np.array([rnd.choice(pool) if pool else rnd.gauss(0, 1) for _ in range(E)],
                       np.float32)
        ids = oracle.select_topk(row[None, :], k)[0].tolist()
        assert ids == _brute_topk(row, k), (row, k)


def test_topk_all_pairs_of_sixteen():
    # every choice of 2 "winners" among 16 logits of the tiny workload's shape
    for a, b in itertools.combinations(range(16), 2):
        row = np.full(16, -1.0, np.float32)
        row[a], row[b] = 2.0, 1.0
        assert oracle.select_topk(row[None, :], 2)[0].tolist() == [a, b]
        row[a] = row[b] = 1.5                   # tie -> lower index first
        assert oracle.select_topk(row[None, :], 2)[0].tolist() == [min(a, b), max(a, b)]


def test_all_equal_logits_give_first_k_and_uniform_weights():
    logits = np.zeros((3, 512), np.float32)
    logits[1, :] = -0.0
    logits[2, :] = 7.25
    ids = oracle.select_topk(logits, 10)
    assert np.array_equal(ids, np.tile(np.arange(10, dtype=np.int32), (3, 1)))
    w = oracle.topk_weights(logits, ids)
    assert np.allclose(w, 0.1, rtol=0, atol=1e-15)


def test_weights_closed_form_two_experts():
    # logits (0, ln 3): weights 3/4 and 1/4 up to the fp32 rounding of ln 3
    l3 = np.float32(math.log(3.0))
    logits = np.array([[0.0, l3, -5.0, -6.0]], np.float32)
    ids = oracle.select_topk(logits, 2)
    assert ids[0].tolist() == [1, 0]
    w = oracle.topk_weights(logits, ids)[0]
    assert abs(w[0] - 0.75) < 1e-7 and abs(w[1] - 0.25) < 1e-7
    assert abs(w[0] - 1.0 / (1.0 + math.exp(-float(l3)))) < 1e-15


def test_weights_equal_renormalised_full_softmax():
    rng = np.random.default_rng(2)
    logits = (rng.standard_normal((50, 512)) * 0.9).astype(np.float32)
    ids = oracle.select_topk(logits, 10)
    w = oracle.topk_weights(logits, ids)
    full = np.exp(logits.astype(np.float64) - logits.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(full, ids.astype(np.int64), axis=1)
    ren = sel / sel.sum(axis=1, keepdims=True)
    assert np.allclose(w, ren, rtol=0, atol=1e-15)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(w > 0) and np.all(np.diff(w, axis=1) <= 0)
    # k distinct ids in range; every unselected logit ranks after every selected one
    for t in range(50):
        assert len(set(ids[t].tolist())) == 10
        sel_min = logits[t, ids[t]].min()
        rest = np.setdiff1d(np.arange(512), ids[t])
        assert np.all(logits[t, rest] <= sel_min)


# ---------------------------------------------------------------- grouping

def test_permute_equals_stable_sort():
    rng = np.random.default_rng(3)
    for T, k, E in [(4, 2, 16), (1, 10, 512), (37, 3, 5), (200, 10, 512), (0, 10, 512)]:
        ids = rng.integers(0, E, (T, k)).astype(np.int32)
        offsets, sp, pp, bad = oracle.permute(ids, E)
        flat = ids.reshape(-1)
        ref = sorted(range(T * k), key=lambda p: (int(flat[p]), p))
        assert bad == 0
        assert sp.tolist() == ref
        assert offsets[0] == 0 and offsets[E] == T * k
        assert np.all(np.diff(offsets) >= 0)
        assert np.array_equal(np.diff(offsets), np.bincount(flat, minlength=E))
        assert np.array_equal(sp[pp], np.arange(T * k))


def test_permute_counts_out_of_range_ids():
    ids = np.array([[0, 5], [16, -1]], np.int32)
    offsets, sp, pp, bad = oracle.permute(ids, 16)
    assert bad == 2 and offsets[16] == 2 and pp[2] == -1 and pp[3] == -1


# ---------------------------------------------------------------- expert FFN

def _unit_scale_experts(q_gate, q_up, q_down, fmt="int4_g32"):
    pack = {"int4_g32": si.pack_int4, "int6_g32": si.pack_int6, "int3_g32": si.pack_int3,
            "int2_g32": si.pack_int2}[fmt]
    one = lambda n, K: torch.full((1, n, K // 32), 1.0, dtype=torch.float16)  # noqa: E731
    F, d = q_gate.shape
    return {"fmt": si.FMT_BY_NAME[fmt], "E": 1, "d": d, "F": F,
            "w_gate": pack(q_gate[None]).numpy(), "w_up": pack(q_up[None]).numpy(),
            "w_down": pack(q_down[None]).numpy(), "s_gate": si.bits16(one(F, d)),
            "s_up": si.bits16(one(F, d)), "s_down": si.bits16(one(d, F))}


@pytest.mark.parametrize("fmt,lo,hi", [("int4_g32", -8, 7), ("int6_g32", -32, 31),
                                      ("int3_g32", -4, 3), ("int2_g32", -2, 1)])
def test_expert_ffn_is_textbook_swiglu(fmt, lo, hi):
    # unit scales make the weights the integer codes themselves; then the expert must be
    # the dense SwiGLU MLP  y = Wd (silu(Wg x) * (Wu x))  evaluated by torch in fp64.
    g = torch.Generator().manual_seed(9)
    d, F = 256, 128
    qg = torch.randint(lo, hi + 1, (F, d), generator=g, dtype=torch.int32)
    qu = torch.randint(lo, hi + 1, (F, d), generator=g, dtype=torch.int32)
    qd = torch.randint(lo, hi + 1, (d, F), generator=g, dtype=torch.int32)
    ex = _unit_scale_experts(qg, qu, qd, fmt)
    x = (torch.randn((3, d), generator=g) * 0.01).to(torch.bfloat16)
    for t in range(3):
        y = oracle.expert_ffn(ex, 0, si.bits16(x[t]))
        xd = x[t].double()
        ref = (torch.nn.functional.silu(qg.double() @ xd) * (qu.double() @ xd)) @ qd.double().T
        assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-9)


def _tiny_layer(seed=0):
    lay = synth.make_layer(TINY, seed=seed, device="cpu")
    x = synth.make_tokens(TINY, seed=seed)
    return lay.router.host(), lay.routed.host(), lay.shared.host(), si.bits16(x)


def test_zero_scales_leave_only_shared_expert():
    r, ex, sh, x = _tiny_layer()
    for key in ("s_gate", "s_up", "s_down"):
        ex[key] = np.zeros_like(ex[key])
    res = oracle.layer_tokens(r, ex, sh, x, np.arange(4), 2)
    for t in range(4):
        assert np.array_equal(res["out"][t], oracle.expert_ffn(sh, 0, x[t]))


def test_identical_experts_make_routing_irrelevant():
    r, ex, sh, x = _tiny_layer()
    for key in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down"):
        ex[key] = np.ascontiguousarray(np.repeat(ex[key][:1], 16, axis=0))
    res = oracle.layer_tokens(r, ex, sh, x, np.arange(4), 2)
    for t in range(4):
        ref = oracle.expert_ffn(sh, 0, x[t]) + oracle.expert_ffn(ex, 0, x[t])
        assert np.allclose(res["out"][t], ref, rtol=0, atol=1e-12)


def test_dense_then_mask_equals_sparse():
    # evaluate every expert for every token, weight all but the top-k by zero: same layer
    r, ex, sh, x = _tiny_layer(seed=1)
    T, E, k = 4, 16, 2
    logits = oracle.router_logits(r, x)
    full = np.exp(logits.astype(np.float64) - logits.max(axis=1, keepdims=True))
    ids = np.array([_brute_topk(logits[t], k) for t in range(T)])
    mask = np.zeros((T, E))
    for t in range(T):
        mask[t, ids[t]] = 1.0
    wdense = full * mask
    wdense /= wdense.sum(axis=1, keepdims=True)
    tok = np.repeat(np.arange(T), E)
    exp_ = np.tile(np.arange(E), T)
    y_all = oracle.expert_ffn_pairs(ex, x, tok, exp_).reshape(T, E, -1)
    dense = np.einsum("te,ted->td", wdense, y_all)
    dense += np.stack([oracle.expert_ffn(sh, 0, x[t]) for t in range(T)])
    res = oracle.layer_tokens(r, ex, sh, x, np.arange(T), k)
    assert np.array_equal(res["ids"], ids)
    assert np.allclose(res["out"], dense, rtol=0, atol=1e-12)


def test_grouped_path_equals_token_path():
    # permute -> per-pair expert outputs in sorted order -> combine via pair_pos gives
    # the same layer output as the per-token composition
    r, ex, sh, x = _tiny_layer(seed=2)
    T, E, k = 4, 16, 2
    logits = oracle.router_logits(r, x)
    ids = oracle.select_topk(logits, k)
    w = oracle.topk_weights(logits, ids)
    offsets, sp, pp, _ = oracle.permute(ids, E)
    y_sorted = oracle.expert_ffn_pairs(ex, x, sp // k, ids.reshape(-1)[sp])
    y_sh = np.stack([oracle.expert_ffn(sh, 0, x[t]) for t in range(T)])
    out = oracle.combine(y_sorted, pp, w, y_sh)
    res = oracle.layer_tokens(r, ex, sh, x, np.arange(T), k)
    assert np.allclose(out, res["out"], rtol=0, atol=1e-12)
    assert np.array_equal(ids, res["ids"])


def test_residual_rounding():
    x = np.array([0x3F80, 0x3F80, 0xC000], np.uint16)          # 1, 1, -2
    out = np.array([2.0 ** -8, 3 * 2.0 ** -8, 0.5])
    xn = oracle.residual(x, out)
    # bf16(out) = 2^-8 (exact); 1 + 2^-8 is a tie -> 1.  3*2^-8 exact; 1 + 3*2^-8 -> tie
    # between 1+2^-7 and 1+2^-6 -> even -> 1+2^-6 (0x3f82).  -2 + 0.5 = -1.5 (0xbfc0).
    assert xn.tolist() == [0x3F80, 0x3F82, 0xBFC0]
