"""Seeded generators and format encoders for the layer's inputs.

Every tensor is drawn with its own ``torch.Generator`` whose seed mixes
(workload id, seed, layer, tensor id, ...), so any one tensor can be regenerated alone.
The stream depends on the device kind the generator runs on (CPU and GPU generators
differ); a test draws its inputs once and hands the same bytes to both sides.

Recipe (fixed by the workload descriptions; the pages give no weight statistics):
  expert weights  fp32 N(0, 0.02), then quantised per group of 32 along the input dim
  router          fp32 N(0, 0.02) [E][d]; int8 variant quantised per row
  activations     fp32 N(0, 1) rounded to bf16 (round to nearest even)
  Zipf bias       b_e = -s * ln(rank_e), rank = 1 + a seeded permutation of 0..E-1

Encodings (the layer's input formats; decoding them is the layer's job, not this file's):
  int4_g32  s = fp16(max|w_group| / 7); q = clamp(round_half_even(w / s), -8, 7);
            byte = (q[2i] + 8) | (q[2i+1] + 8) << 4
  int6_g32  s = fp16(max|w_group| / 31); q in [-32, 31]; code u = q + 32; the 32 codes of
            a group form a 24-byte little-endian bit string, code i at bits [6i, 6i+6)
  int3_g32  s = fp16(max|w_group| / 3); q in [-4, 3]; code u = q + 4; the 32 codes of a
            group form a 12-byte little-endian bit string, code i at bits [3i, 3i+3)
  int2_g32  s = fp16(max|w_group| / 1); q in [-2, 1]; code u = q + 2; 8 bytes per group,
            code i at bits [2i, 2i+2).  A max-abs scale never needs q = -2: this encoder
            uses {-1, 0, 1}; the all-codes layers below reach -2 too
  int8_row  s = fp16(max|w_row| / 127); q = clamp(round_half_even(w / s), -127, 127)
An all-zero group gets s = 0 and every code q = 0.
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

FMT_FP32, FMT_INT8_ROW, FMT_INT4_G32, FMT_INT6_G32, FMT_INT3_G32, FMT_INT2_G32 = range(6)
FMT_BY_NAME = {"fp32": FMT_FP32, "int8_row": FMT_INT8_ROW, "int4_g32": FMT_INT4_G32,
               "int6_g32": FMT_INT6_G32, "int3_g32": FMT_INT3_G32, "int2_g32": FMT_INT2_G32}

# tensor ids inside one layer's seed
_T_ROUTER, _T_BIAS, _T_GATE, _T_UP, _T_DOWN, _T_SGATE, _T_SUP, _T_SDOWN, _T_X = range(9)
_MASK = (1 << 63) - 1


def _seed(*parts):
    h = 0x243F6A8885A308D3
    for p in parts:
        h = (h * 0x100000001B3 + int(p) + 0x9E3779B97F4A7C15) & _MASK
        h ^= h >> 29
    return h & _MASK


def _gen(device, *parts):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


# ---------------------------------------------------------------- encoders

def pack_int4(q):
    """q int codes in [-8, 7], [..., K] -> uint8 [..., K/2]."""
    u = (q + 8).to(torch.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).contiguous()


def pack_int6(q):
    """q int codes in [-32, 31], [..., K] (K % 32 == 0) -> uint8 [..., K*3/4]."""
    u = (q + 32).to(torch.int32)
    lead = u.shape[:-1]
    u4 = u.reshape(*lead, -1, 4)              # 4 codes = 24 bits = 3 bytes
    v = u4[..., 0] | (u4[..., 1] << 6) | (u4[..., 2] << 12) | (u4[..., 3] << 18)
    b = torch.stack([v & 255, (v >> 8) & 255, (v >> 16) & 255], dim=-1)
    return b.reshape(*lead, -1).to(torch.uint8).contiguous()


def pack_int3(q):
    """q int codes in [-4, 3], [..., K] (K % 32 == 0) -> uint8 [..., K*3/8]."""
    u = (q + 4).to(torch.int32)
    lead = u.shape[:-1]
    u8 = u.reshape(*lead, -1, 8)              # 8 codes = 24 bits = 3 bytes
    v = torch.zeros_like(u8[..., 0])
    for j in range(8):
        v = v | (u8[..., j] << (3 * j))
    b = torch.stack([v & 255, (v >> 8) & 255, (v >> 16) & 255], dim=-1)
    return b.reshape(*lead, -1).to(torch.uint8).contiguous()


def pack_int2(q):
    """q int codes in [-2, 1], [..., K] (K % 32 == 0) -> uint8 [..., K/4]."""
    u = (q + 2).to(torch.int32)
    b = u[..., 0::4] | (u[..., 1::4] << 2) | (u[..., 2::4] << 4) | (u[..., 3::4] << 6)
    return b.to(torch.uint8).contiguous()


def _group_quant(w, qmax, qmin):
    *lead, N, K = w.shape
    g = w.reshape(*lead, N, K // 32, 32)
    s16 = (g.abs().amax(dim=-1) / float(qmax)).to(torch.float16)
    s = s16.to(torch.float32)[..., None]
    q = torch.where(s > 0, torch.round(g / torch.where(s > 0, s, torch.ones_like(s))),
                    torch.zeros_like(g))
    q = q.clamp(qmin, qmax).to(torch.int32).reshape(*lead, N, K)
    return q, s16.contiguous()


def quantize_int4_g32(w):
    """fp32 [..., N, K] -> (packed uint8 [..., N, K/2], fp16 scales [..., N, K/32])."""
    q, s = _group_quant(w, 7, -8)
    return pack_int4(q), s


def quantize_int6_g32(w):
    """fp32 [..., N, K] -> (packed uint8 [..., N, K*3/4], fp16 scales [..., N, K/32])."""
    q, s = _group_quant(w, 31, -32)
    return pack_int6(q), s


def quantize_int3_g32(w):
    """fp32 [..., N, K] -> (packed uint8 [..., N, K*3/8], fp16 scales [..., N, K/32])."""
    q, s = _group_quant(w, 3, -4)
    return pack_int3(q), s


def quantize_int2_g32(w):
    """fp32 [..., N, K] -> (packed uint8 [..., N, K/4], fp16 scales [..., N, K/32])."""
    q, s = _group_quant(w, 1, -2)
    return pack_int2(q), s


def quantize_int8_row(w):
    """fp32 [E, d] -> (int8 [E, d], fp16 scales [E])."""
    s16 = (w.abs().amax(dim=-1) / 127.0).to(torch.float16)
    s = s16.to(torch.float32)[:, None]
    q = torch.where(s > 0, torch.round(w / torch.where(s > 0, s, torch.ones_like(s))),
                    torch.zeros_like(w))
    return q.clamp(-127, 127).to(torch.int8).contiguous(), s16.contiguous()


_QUANT = {"int4_g32": quantize_int4_g32, "int6_g32": quantize_int6_g32,
          "int3_g32": quantize_int3_g32, "int2_g32": quantize_int2_g32}


def zipf_bias(E, s, gen, device):
    """Router bias making expert popularity heavy-headed: b_e = -s * ln(rank_e)."""
    rank = torch.randperm(E, generator=gen, device=device).to(torch.float64) + 1.0
    return (-s * torch.log(rank)).to(torch.float32).contiguous()


def bits16(t):
    """bf16 / fp16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- a layer's tensors

@dataclass
class ExpertSet:
    fmt: str
    E: int
    d: int
    F: int
    w_gate: torch.Tensor   # uint8 [E][F][d packed]
    w_up: torch.Tensor     # uint8 [E][F][d packed]
    w_down: torch.Tensor   # uint8 [E][d][F packed]
    s_gate: torch.Tensor   # fp16 [E][F][d/32]
    s_up: torch.Tensor     # fp16 [E][F][d/32]
    s_down: torch.Tensor   # fp16 [E][d][F/32]

    def host(self):
        return {"fmt": FMT_BY_NAME[self.fmt], "E": self.E, "d": self.d, "F": self.F,
                "w_gate": self.w_gate.cpu().numpy(), "w_up": self.w_up.cpu().numpy(),
                "w_down": self.w_down.cpu().numpy(), "s_gate": bits16(self.s_gate),
                "s_up": bits16(self.s_up), "s_down": bits16(self.s_down)}

    def nbytes(self):
        return sum(t.numel() * t.element_size() for t in
                   (self.w_gate, self.w_up, self.w_down, self.s_gate, self.s_up, self.s_down))


@dataclass
class Router:
    fmt: str
    E: int
    d: int
    w: torch.Tensor                 # fp32 [E][d] or int8 [E][d]
    scale: Optional[torch.Tensor]   # fp16 [E] (int8 only)
    bias: Optional[torch.Tensor]    # fp32 [E] or None

    def host(self):
        return {"fmt": FMT_BY_NAME[self.fmt], "E": self.E, "d": self.d,
                "w": self.w.cpu().numpy(),
                "scale": None if self.scale is None else bits16(self.scale),
                "bias": None if self.bias is None else self.bias.cpu().numpy()}


@dataclass
class Layer:
    router: Router
    routed: ExpertSet
    shared: Optional[ExpertSet]


def _experts(fmt, E, d, F, device, gens):
    gg, gu, gd = gens
    wg = torch.randn((E, F, d), generator=gg, device=device, dtype=torch.float32) * 0.02
    pg, sg = _QUANT[fmt](wg)
    del wg
    wu = torch.randn((E, F, d), generator=gu, device=device, dtype=torch.float32) * 0.02
    pu, su = _QUANT[fmt](wu)
    del wu
    wd = torch.randn((E, d, F), generator=gd, device=device, dtype=torch.float32) * 0.02
    pd, sd = _QUANT[fmt](wd)
    del wd
    return ExpertSet(fmt, E, d, F, pg, pu, pd, sg, su, sd)


def make_layer(w, seed=0, layer=0, device="cpu", bias=None, with_shared=True,
               expert_chunk=64):
    """All weights of one layer of workload ``w``.

    bias: None -> the workload's own choice ("none" | "zipf"); or "none" / "zipf".
    Routed experts are drawn in chunks of ``expert_chunk`` experts (each chunk its own
    generator) to bound the fp32 staging memory.
    """
    bias = w.bias if bias is None else bias
    dev = torch.device(device)
    g = _gen(dev, w.wid, seed, layer, _T_ROUTER)
    rw = torch.randn((w.E, w.d), generator=g, device=dev, dtype=torch.float32) * 0.02
    if w.router_fmt == "int8_row":
        rq, rs = quantize_int8_row(rw)
        router_w, router_s = rq, rs
    else:
        router_w, router_s = rw.contiguous(), None
    b = zipf_bias(w.E, 1.1, _gen(dev, w.wid, seed, layer, _T_BIAS), dev) if bias == "zipf" \
        else None
    router = Router(w.router_fmt, w.E, w.d, router_w, router_s, b)

    parts = []
    for e0 in range(0, w.E, expert_chunk):
        n = min(expert_chunk, w.E - e0)
        gens = [_gen(dev, w.wid, seed, layer, tid, e0) for tid in (_T_GATE, _T_UP, _T_DOWN)]
        parts.append(_experts(w.routed_fmt, n, w.d, w.F, dev, gens))
    routed = ExpertSet(w.routed_fmt, w.E, w.d, w.F,
                       *[torch.cat([getattr(p, a) for p in parts]).contiguous() for a in
                         ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down")])
    del parts
    shared = None
    if with_shared:
        gens = [_gen(dev, w.wid, seed, layer, tid, 1 << 20) for tid in (_T_SGATE, _T_SUP,
                                                                         _T_SDOWN)]
        shared = _experts(w.shared_fmt, 1, w.d, w.F, dev, gens)
    return Layer(router, routed, shared)


@dataclass
class Norm:
    gamma: torch.Tensor             # fp32 [d]
    gate_w: Optional[torch.Tensor]  # fp32 [d] or None
    eps: float
    gate_b: float

    def host(self):
        return {"gamma": self.gamma.cpu().numpy(), "eps": self.eps,
                "gate_w": None if self.gate_w is None else self.gate_w.cpu().numpy(),
                "gate_b": self.gate_b}


_T_NORM, _T_GATE_ROW = 20, 21


def make_norm(w, seed=0, layer=0, device="cpu", gate=True):
    """A block's pre-layer norm and residual gate: gamma = 1 + 0.1 N(0, 1), gate row
    N(0, 0.02) like a router row (so z = <gate_w, xn> has a spread of about 0.9 and the gate
    sigmoid(z) stays inside (0.2, 0.8) for most tokens), gate bias 0, eps 1e-6."""
    dev = torch.device(device)
    g = _gen(dev, w.wid, seed, layer, _T_NORM)
    gamma = (1.0 + 0.1 * torch.randn((w.d,), generator=g, device=dev)).to(torch.float32)
    gw = None
    if gate:
        g2 = _gen(dev, w.wid, seed, layer, _T_GATE_ROW)
        gw = (0.02 * torch.randn((w.d,), generator=g2, device=dev)).to(torch.float32)
    return Norm(gamma.contiguous(), None if gw is None else gw.contiguous(), 1e-6, 0.0)


_QRANGE = {"int4_g32": (-8, 7), "int6_g32": (-32, 31), "int3_g32": (-4, 3),
           "int2_g32": (-2, 1)}
_PACK = {"int4_g32": pack_int4, "int6_g32": pack_int6, "int3_g32": pack_int3,
         "int2_g32": pack_int2}


def _all_codes_matrix(fmt, E, N, K, gen, device):
    """Packed codes and fp16 scales of E matrices [N][K] in which every code of the format,
    the lowest included (int4 -8, int6 -32, int3 -4, int2 -2), sits at every position of a
    group: row n,
    element c of matrix e holds qmin + ((n + c + e) mod ncodes) for the first ncodes rows,
    uniform random codes elsewhere.  Scales are fp16 of U(0.5, 1.5) * 0.02 / sd, sd the
    standard deviation of a code drawn uniformly from the format's range (int4 4.61, int6
    18.47, int3 2.29, int2 1.12), so the weights spread like the N(0, 0.02) draws of make_layer; every 7th group
    of a matrix (in row-major group order, from a random start) has scale 0."""
    qmin, qmax = _QRANGE[fmt]
    nc = qmax - qmin + 1
    q = torch.randint(qmin, qmax + 1, (E, N, K), generator=gen, device=device,
                      dtype=torch.int32)
    n = torch.arange(min(nc, N), device=device, dtype=torch.int32)[:, None]
    c = torch.arange(K, device=device, dtype=torch.int32)[None, :]
    for e in range(E):
        q[e, :min(nc, N)] = qmin + (n + c + e) % nc
    sd = ((nc * nc - 1) / 12.0) ** 0.5
    s = (torch.rand((E, N, K // 32), generator=gen, device=device) + 0.5) * (0.02 / sd)
    s = s.to(torch.float16)
    start = int(torch.randint(0, 7, (1,), generator=gen, device=device))
    flat = s.view(-1)
    flat[start::7] = 0
    return _PACK[fmt](q), s.contiguous()


def make_layer_all_codes(w, seed=0, device="cpu", with_shared=True):
    """A layer of workload ``w``'s shapes whose expert codes cover the whole code range at
    every group position, with some all-zero-scale groups (see _all_codes_matrix); the
    router is drawn as in make_layer.  For parity tests of the decoders."""
    dev = torch.device(device)
    base = make_layer(w, seed=seed, device=device, with_shared=False)
    tid = 1 << 21

    def ex(fmt, E, salt):
        mats = []
        for t, (N, K) in enumerate(((w.F, w.d), (w.F, w.d), (w.d, w.F))):
            mats.append(_all_codes_matrix(fmt, E, N, K,
                                          _gen(dev, w.wid, seed, tid, salt, t), dev))
        (pg, sg), (pu, su), (pd, sd) = mats
        return ExpertSet(fmt, E, w.d, w.F, pg, pu, pd, sg, su, sd)

    routed = ex(w.routed_fmt, w.E, 0)
    shared = ex(w.shared_fmt, 1, 1) if with_shared else None
    return Layer(base.router, routed, shared)


def make_tokens(w, T=None, seed=0, layer=0, device="cpu", stream=0):
    """bf16 [T][d] activations, N(0, 1) rounded to bf16."""
    T = w.T if T is None else T
    g = _gen(torch.device(device), w.wid, seed, layer, _T_X, stream, T)
    x = torch.randn((T, w.d), generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16).contiguous()
