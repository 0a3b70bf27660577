"""CPU oracle of the quantized routed-expert MoE layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU-baseline
leg may import this package.  It wraps ``moe_oracle.c`` (plain C, fp64 arithmetic,
compiled with gcc) with ctypes; this file only marshals numpy arrays.  It imports
nothing from the GPU package and the GPU package imports nothing from here.

Inputs are numpy arrays holding raw encodings:
  bf16 / fp16 values as ``uint16`` bit patterns, packed weight codes as ``uint8``,
  the fp32 router as ``float32``, the int8 router as ``int8``.
A router is a dict ``{fmt, E, d, w, scale, bias}``; an expert set is a dict
``{fmt, E, d, F, w_gate, w_up, w_down, s_gate, s_up, s_down}`` (shared expert: E = 1).
"""
import ctypes
import os
import subprocess

import numpy as np

FMT_FP32, FMT_INT8_ROW, FMT_INT4_G32, FMT_INT6_G32, FMT_INT3_G32, FMT_INT2_G32 = 0, 1, 2, 3, 4, 5

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_SO = os.path.join(_HERE, "libmoe_oracle.so")
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared"]


def build(force=True):
    """Compile moe_oracle.c into libmoe_oracle.so with gcc."""
    if not force and os.path.exists(_SO):
        return _SO
    tmp = _SO + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _SO)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_SO)
        _declare(_lib)
    return _lib


class _Router(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("d_model", ctypes.c_int32), ("pad_", ctypes.c_int32),
                ("w", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("bias", ctypes.c_void_p)]


class _Experts(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("s_gate", ctypes.c_void_p),
                ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int


def _declare(L):
    sig = {
        "oracle_half_to_double": (ctypes.c_double, [ctypes.c_uint16]),
        "oracle_double_to_bf16": (ctypes.c_uint16, [ctypes.c_double]),
        "oracle_double_to_bf16_n": (None, [_P, _I64, _P]),
        "oracle_code": (_I, [_I, _P, _I]),
        "oracle_dequant_row": (None, [_I, _P, _P, _I, _I64, _P]),
        "oracle_router_logits": (None, [_P, _P, _I64, _P]),
        "oracle_router_logits_fp64": (None, [_P, _P, _I64, _P]),
        "oracle_select_topk": (None, [_P, _I64, _I, _I, _P]),
        "oracle_topk_weights": (None, [_P, _P, _I64, _I, _I, _P]),
        "oracle_permute": (_I64, [_P, _I64, _I, _I, _P, _P, _P]),
        "oracle_expert_ffn": (None, [_P, _I, _P, _P]),
        "oracle_expert_ffn_pairs": (None, [_P, _P, _P, _P, _I64, _P]),
        "oracle_combine": (None, [_P, _P, _P, _P, _I64, _I, _I, _P]),
        "oracle_layer_tokens": (None, [_P, _P, _P, _P, _P, _I64, _I, _P, _P, _P, _P, _P]),
        "oracle_residual": (None, [_P, _P, _I64, _P]),
        "oracle_rms_sumsq": (ctypes.c_float, [_P, _I]),
        "oracle_rmsnorm": (None, [_P, _I64, _I, _P, ctypes.c_float, _P, _P]),
        "oracle_gated_residual": (None, [_P, _P, _P, _I64, _I, _P]),
        "oracle_num_threads": (_I, []),
        "oracle_set_num_threads": (None, [_I]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class _Keep:
    """Holds the contiguous arrays a ctypes struct points into."""

    def __init__(self):
        self.refs = []

    def __call__(self, a, dtype):
        if a is None:
            return None
        a = _c(a, dtype)
        self.refs.append(a)
        return a


def _router_struct(r, keep):
    fmt = int(r["fmt"])
    w = keep(r["w"], np.int8 if fmt == FMT_INT8_ROW else np.float32)
    scale = keep(r.get("scale"), np.uint16) if fmt == FMT_INT8_ROW else None
    bias = keep(r.get("bias"), np.float32)
    return _Router(fmt, int(r["E"]), int(r["d"]), 0, _ptr(w), _ptr(scale), _ptr(bias))


def _experts_struct(ex, keep):
    a = {k: keep(ex[k], np.uint8) for k in ("w_gate", "w_up", "w_down")}
    s = {k: keep(ex[k], np.uint16) for k in ("s_gate", "s_up", "s_down")}
    return _Experts(int(ex["fmt"]), int(ex["E"]), int(ex["d"]), int(ex["F"]),
                    _ptr(a["w_gate"]), _ptr(a["w_up"]), _ptr(a["w_down"]),
                    _ptr(s["s_gate"]), _ptr(s["s_up"]), _ptr(s["s_down"]))


# ---------------------------------------------------------------- scalar helpers

def half_to_double(h):
    return lib().oracle_half_to_double(int(h))


def double_to_bf16(v):
    return lib().oracle_double_to_bf16(float(v))


def double_to_bf16_array(v):
    """double_to_bf16 over an array: uint16 bit patterns of the same shape."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_double_to_bf16_n(_ptr(v), v.size, _ptr(out))
    return out


def code(fmt, row_bytes, c):
    row = _c(row_bytes, np.uint8)
    return lib().oracle_code(int(fmt), _ptr(row), int(c))


def dequant_rows(fmt, w, s, K):
    """All rows of a packed [N][K] matrix, exactly, as float64 [N][K]."""
    w = _c(w, np.uint8)
    s = _c(s, np.uint16)
    N = s.size // (K // 32)
    out = np.empty((N, K), np.float64)
    for n in range(N):
        lib().oracle_dequant_row(int(fmt), _ptr(w), _ptr(s), int(K), n,
                                 out[n].ctypes.data_as(ctypes.c_void_p))
    return out


# ---------------------------------------------------------------- the layer's steps

def router_logits(router, x_bits):
    keep = _Keep()
    r = _router_struct(router, keep)
    x = _c(x_bits, np.uint16)
    T = x.shape[0]
    out = np.empty((T, int(router["E"])), np.float32)
    lib().oracle_router_logits(ctypes.byref(r), _ptr(x), T, _ptr(out))
    return out


def router_logits_fp64(router, x_bits):
    keep = _Keep()
    r = _router_struct(router, keep)
    x = _c(x_bits, np.uint16)
    T = x.shape[0]
    out = np.empty((T, int(router["E"])), np.float64)
    lib().oracle_router_logits_fp64(ctypes.byref(r), _ptr(x), T, _ptr(out))
    return out


def select_topk(logits, k):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    lib().oracle_select_topk(_ptr(logits), T, E, int(k), _ptr(ids))
    return ids


def topk_weights(logits, ids):
    logits = _c(logits, np.float32)
    ids = _c(ids, np.int32)
    T, E = logits.shape
    k = ids.shape[1]
    w = np.empty((T, k), np.float64)
    lib().oracle_topk_weights(_ptr(logits), _ptr(ids), T, E, k, _ptr(w))
    return w


def permute(ids, E):
    ids = _c(ids, np.int32)
    T, k = ids.shape
    P = T * k
    offsets = np.empty(E + 1, np.int32)
    sorted_pairs = np.empty(P, np.int32)
    pair_pos = np.empty(P, np.int32)
    bad = lib().oracle_permute(_ptr(ids), T, k, int(E), _ptr(offsets), _ptr(sorted_pairs),
                               _ptr(pair_pos))
    return offsets, sorted_pairs, pair_pos, int(bad)


def expert_ffn(experts, e, x_row_bits):
    keep = _Keep()
    ex = _experts_struct(experts, keep)
    x = _c(x_row_bits, np.uint16)
    y = np.empty(int(experts["d"]), np.float64)
    lib().oracle_expert_ffn(ctypes.byref(ex), int(e), _ptr(x), _ptr(y))
    return y


def expert_ffn_pairs(experts, x_bits, tok, expert):
    keep = _Keep()
    ex = _experts_struct(experts, keep)
    x = _c(x_bits, np.uint16)
    tok = _c(tok, np.int32)
    expert = _c(expert, np.int32)
    y = np.empty((tok.size, int(experts["d"])), np.float64)
    lib().oracle_expert_ffn_pairs(ctypes.byref(ex), _ptr(x), _ptr(tok), _ptr(expert),
                                  tok.size, _ptr(y))
    return y


def combine(y_pairs, pair_pos, w, y_shared=None):
    y_pairs = _c(y_pairs, np.float64)
    pair_pos = _c(pair_pos, np.int32)
    w = _c(w, np.float64)
    T, k = w.shape
    d = y_pairs.shape[1]
    ys = None if y_shared is None else _c(y_shared, np.float64)
    out = np.empty((T, d), np.float64)
    lib().oracle_combine(_ptr(y_pairs), _ptr(pair_pos), _ptr(w), _ptr(ys), T, k, d, _ptr(out))
    return out


def layer_tokens(router, routed, shared, x_bits, tokens, k, keep_pairs=False):
    """Routing, experts and combine for the listed tokens (fp64 outputs)."""
    keep = _Keep()
    r = _router_struct(router, keep)
    ex = _experts_struct(routed, keep)
    sh = _experts_struct(shared, keep) if shared is not None else None
    x = _c(x_bits, np.uint16)
    tokens = _c(tokens, np.int32)
    n = tokens.size
    d = int(router["d"])
    ids = np.empty((n, k), np.int32)
    w = np.empty((n, k), np.float64)
    y_sel = np.empty((n, k, d), np.float64) if keep_pairs else None
    y_sh = np.empty((n, d), np.float64) if (keep_pairs and shared is not None) else None
    out = np.empty((n, d), np.float64)
    lib().oracle_layer_tokens(ctypes.byref(r), ctypes.byref(ex),
                              ctypes.byref(sh) if sh is not None else None, _ptr(x),
                              _ptr(tokens), n, int(k), _ptr(ids), _ptr(w), _ptr(y_sel),
                              _ptr(y_sh), _ptr(out))
    return {"ids": ids, "w": w, "y_sel": y_sel, "y_shared": y_sh, "out": out}


def rms_sumsq(x_row_bits):
    x = _c(x_row_bits, np.uint16)
    return lib().oracle_rms_sumsq(_ptr(x), x.size)


def rmsnorm(x_bits, gamma, eps):
    """(xn bf16 bits [T][d], r fp32 [T]) of the pre-layer RMS norm."""
    x = _c(x_bits, np.uint16)
    T, d = x.shape
    g = _c(gamma, np.float32)
    xn = np.empty_like(x)
    r = np.empty(T, np.float32)
    lib().oracle_rmsnorm(_ptr(x), T, d, _ptr(g), float(np.float32(eps)), _ptr(xn), _ptr(r))
    return xn, r


def gate_logits(gate_w, gate_b, xn_bits):
    """z [T] fp32: the gate row through the router's fixed fp32 order, plus its bias."""
    gw = _c(gate_w, np.float32).reshape(1, -1)
    r = {"fmt": FMT_FP32, "E": 1, "d": gw.shape[1], "w": gw,
         "bias": np.array([gate_b], np.float32)}
    return router_logits(r, xn_bits)[:, 0].copy()


def gated_residual(x_bits, out, z=None):
    x = _c(x_bits, np.uint16)
    out = _c(out, np.float64)
    T, d = x.shape
    zz = None if z is None else _c(z, np.float32)
    xn = np.empty_like(x)
    lib().oracle_gated_residual(_ptr(x), _ptr(out), _ptr(zz), T, d, _ptr(xn))
    return xn


def block_tokens(norm, router, routed, shared, x_bits, tokens, k, keep_pairs=False):
    """One MoE block on the listed tokens: xn = RMSNorm(x), the layer on xn, and the gated
    residual x_next = bf16(x + bf16(g * out)).  norm: {gamma, eps, gate_w, gate_b}
    (gate_w None: g = 1).  Returns layer_tokens' dict plus xn, z, x_next."""
    x = _c(x_bits, np.uint16)
    tokens = _c(tokens, np.int32)
    xs = x[tokens]
    xn, _ = rmsnorm(xs, norm["gamma"], norm["eps"])
    res = layer_tokens(router, routed, shared, xn, np.arange(tokens.size, dtype=np.int32), k,
                       keep_pairs=keep_pairs)
    z = None
    if norm.get("gate_w") is not None:
        z = gate_logits(norm["gate_w"], norm.get("gate_b", 0.0), xn)
    res["xn"], res["z"] = xn, z
    res["x_next"] = gated_residual(xs, res["out"], z)
    # the unrounded update g * out (fp64): x_next is bf16(x + bf16(update))
    g = np.ones(tokens.size) if z is None else 1.0 / (1.0 + np.exp(-z.astype(np.float64)))
    res["update"] = g[:, None] * res["out"]
    return res


def residual(x_bits, out):
    x = _c(x_bits, np.uint16)
    out = _c(out, np.float64)
    xn = np.empty_like(x)
    lib().oracle_residual(_ptr(x), _ptr(out), x.size, _ptr(xn))
    return xn


def num_threads():
    return lib().oracle_num_threads()


def set_num_threads(n):
    lib().oracle_set_num_threads(int(n))


# ---------------------------------------------------------------- fp32 error audit of the router

def _bf16_bits_to_f64(x_bits):
    x = _c(x_bits, np.uint16).astype(np.uint32) << 16
    return x.view(np.float32).astype(np.float64)


def router_error_bound(router, x_bits):
    """Rigorous bound [T][E] on |fp32 logit - exact logit| for any summation order whose
    every product passes through at most m roundings.

    The fixed fp32 order gives each product term one fma rounding per remaining step of its
    lane's chain (d/64 of them at most), 6 butterfly additions and the bias addition; the
    int8 form adds the rounding of the product with the row scale.  Error analysis of
    summation (Higham, Accuracy and Stability of Numerical Algorithms, Lemma 3.1 and
    section 3.1): |fl - exact| <= gamma_m * (sum_c |x_c w_c| * |s| + |b|), gamma_m =
    m u / (1 - m u), u = 2^-24, with m = d/64 + 7 (fp32) or d/64 + 8 (int8).  The sum of
    absolute terms is taken in double (products of a bf16 and an fp32 or int8 value are
    exact there; the non-negative sum is inflated by its own fp64 bound)."""
    x = _bf16_bits_to_f64(x_bits)
    d = int(router["d"])
    if int(router["fmt"]) == FMT_INT8_ROW:
        w = np.abs(_c(router["w"], np.int8).astype(np.float64).reshape(-1, d))
        s = np.array([half_to_double(h) for h in _c(router["scale"], np.uint16)])
        m = d // 64 + 8
    else:
        w = np.abs(_c(router["w"], np.float32).astype(np.float64).reshape(-1, d))
        s = np.ones(w.shape[0])
        m = d // 64 + 7
    a = (np.abs(x) @ w.T) * (1.0 + (d + 1) * 2.0 ** -52) * np.abs(s)[None, :]
    b = router.get("bias")
    if b is not None:
        a = a + np.abs(_c(b, np.float32).astype(np.float64))[None, :]
    u = 2.0 ** -24
    return (m * u / (1.0 - m * u)) * a


def router_tie_audit(router, x_bits, k, factor=2.0):
    """Tokens whose top-k set another valid fp32 summation order could change.

    The router sends each token to 10 of a layer's 512 routed experts [Strata 与
    Qwen3.8-Flash-Next (telli.sh), section 稀疏架构创造了机会]; the pages fix no summation
    order, so this audit reports where the choice rests on the fixed order alone.

    With exact logits l (the fp64 audit copy) and bounds B (router_error_bound, scaled by
    `factor`), a token is flagged when some expert inside the exact top-k and some expert
    outside it have overlapping intervals: min over selected (l - B) <= max over the
    others (l + B).  Exactly tied logits are always flagged.  The fixed-order fp32 logits
    still decide one selection; the flag says where only that fixed order makes it unique.
    Also compares the selection made on the fixed-order fp32 logits (select_topk) with the
    exact top-k set: where they differ the two intervals must overlap at factor 1.
    Returns {flags [T] bool, count, margin [T], fp32_set_differs [T] bool, differs} with
    margin = min(l - B) - max(l + B)."""
    l64 = router_logits_fp64(router, x_bits)
    bnd = factor * router_error_bound(router, x_bits)
    T, E = l64.shape
    if k >= E:
        z = np.zeros(T, bool)
        return {"flags": z, "count": 0, "margin": np.full(T, np.inf),
                "fp32_set_differs": z, "differs": 0}
    order = np.argsort(-l64, axis=1, kind="stable")
    sel = np.zeros((T, E), bool)
    np.put_along_axis(sel, order[:, :k], True, axis=1)
    lo = np.where(sel, l64 - bnd, np.inf).min(axis=1)
    hi = np.where(sel, -np.inf, l64 + bnd).max(axis=1)
    margin = lo - hi
    flags = margin <= 0.0
    sel32 = np.zeros((T, E), bool)
    np.put_along_axis(sel32, select_topk(router_logits(router, x_bits), k).astype(np.int64),
                      True, axis=1)
    differs = (sel32 != sel).any(axis=1)
    return {"flags": flags, "count": int(flags.sum()), "margin": margin,
            "fp32_set_differs": differs, "differs": int(differs.sum())}
