"""MI355X-native quantized routed-expert MoE layer.

The compute path is the C ABI of ``libmoe_mi355x.so`` (include/moe.h): moe_route,
moe_permute, moe_expert_ffn and moe_combine, and moe_layer_decode (the same composition
in three launches on one stream for a few tokens), all HIP kernels for gfx950.  This package is its
Python binding (``_lib``) plus ``MoeLayer``, which owns the buffers of one layer call and
enqueues the calls on the current stream.  Torch only provides device memory and streams.
"""
import torch

from . import _lib
from ._lib import (  # noqa: F401
    MOE_FMT_FP32, MOE_FMT_INT8_ROW, MOE_FMT_INT4_G32, MOE_FMT_INT6_G32, MOE_FMT_INT3_G32,
    MOE_FMT_INT2_G32, MOE_OP_ROUTE, MOE_OP_PERMUTE, MOE_OP_EXPERT_FFN, MOE_OP_LAYER_DECODE,
    MOE_OP_EXPERTS_DECODE, MOE_OP_BLOCK_DECODE, MoeError,
    moe_route, moe_permute, moe_expert_ffn, moe_combine, moe_layer_decode, moe_experts_decode,
    moe_layer_decode_noalloc,
    moe_dequant_probe, moe_rmsnorm, moe_combine_gated, moe_block_decode, moe_workspace_size,
    moe_check_device_error, moe_status_string, moe_last_error, moe_version,
    router_desc, experts_desc, norm_desc,
)

_FMT = {"fp32": MOE_FMT_FP32, "int8_row": MOE_FMT_INT8_ROW, "int4_g32": MOE_FMT_INT4_G32,
        "int6_g32": MOE_FMT_INT6_G32, "int3_g32": MOE_FMT_INT3_G32,
        "int2_g32": MOE_FMT_INT2_G32}


def _fmt(f):
    return _FMT[f] if isinstance(f, str) else int(f)


def router_desc_of(r):
    """Descriptor of an object with fmt, w, scale, bias attributes (tensors on the GPU)."""
    return router_desc(_fmt(r.fmt), r.w, r.scale, r.bias)


def experts_desc_of(ex):
    """Descriptor of an object with fmt, d, F, w_gate.. s_down attributes."""
    return experts_desc(_fmt(ex.fmt), ex.d, ex.F, ex.w_gate, ex.w_up, ex.w_down, ex.s_gate,
                        ex.s_up, ex.s_down)


class MoeLayer:
    """Buffers and calls of one MoE layer for up to ``T_max`` tokens.

    forward(x) enqueues moe_route -> moe_permute -> moe_expert_ffn(routed) ->
    moe_expert_ffn(shared, dense) -> moe_combine on the current stream and returns ``out``
    (bf16 [T][d]).  Above SHARED_SIDE_STREAM_ABOVE_TOKENS tokens the shared expert runs on a
    side stream forked from it instead (joined before the combine), beside the router and
    the routed experts; graph capture records the fork and join.  Below that a fork and join
    cost more than the overlap gives.  Intermediate results stay readable
    as attributes (ids, weights, offsets, sorted_pairs, pair_pos, y_pairs, y_shared, and
    logits when ``keep_logits``).  Without ``keep_logits``, moe_route gets no logits buffer
    and, for more than 512 tokens, selects through MFMA logits with an error bound and exact
    recomputation of the experts near the cut (the same ids and weights, bit for bit).

    decode(x) computes the same output bit for bit with moe_layer_decode (three launches, no
    side streams) when T*k <= 64 and the shapes allow it (``can_decode``); it fills ids,
    weights and out only.
    """

    # forward() runs the shared expert on a side stream above this many tokens, where the
    # overlap pays (per layer call 220 -> 202 us at 96 tokens, 276 -> 250 us at 128, 457 ->
    # 415 us at 512); at 64 and below the fork and join cost more than they hide (one token
    # 42 -> 29 us, 64 tokens 173 -> 169 us without them).
    SHARED_SIDE_STREAM_ABOVE_TOKENS = 64

    def __init__(self, router, routed, shared, k, T_max, device="cuda", keep_logits=False,
                 norm=None):
        self.router = router_desc_of(router)
        # the block's pre-layer norm and residual gate (an object with gamma, eps, gate_w,
        # gate_b), for block_forward / block_decode
        self.norm = None if norm is None else norm_desc(norm.gamma, norm.eps, norm.gate_w,
                                                        norm.gate_b)
        self.routed = experts_desc_of(routed)
        self.shared = experts_desc_of(shared) if shared is not None else None
        self.E, self.d, self.F, self.k = routed.E, routed.d, routed.F, k
        self.T_max = T_max
        self.keep_logits = keep_logits
        dev = torch.device(device)
        T, E, d, F = T_max, self.E, self.d, self.F
        P = T * k
        i32, f32, bf = torch.int32, torch.float32, torch.bfloat16
        self.logits = torch.empty((T, E), dtype=f32, device=dev)
        self.ids = torch.empty((T, k), dtype=i32, device=dev)
        self.weights = torch.empty((T, k), dtype=f32, device=dev)
        self.offsets = torch.empty((E + 1,), dtype=i32, device=dev)
        self.sorted_pairs = torch.empty((P,), dtype=i32, device=dev)
        self.pair_pos = torch.empty((P,), dtype=i32, device=dev)
        self.y_pairs = torch.empty((P, d), dtype=bf, device=dev)
        self.y_shared = torch.empty((T, d), dtype=bf, device=dev) if shared is not None \
            else None
        self.out = torch.empty((T, d), dtype=bf, device=dev)
        ws_route = moe_workspace_size(MOE_OP_ROUTE, T, k, E, d, F)
        ws_perm = moe_workspace_size(MOE_OP_PERMUTE, T, k, E, d, F)
        ws_ffn = moe_workspace_size(MOE_OP_EXPERT_FFN, T, k, E, d, F)
        ws_sh = moe_workspace_size(MOE_OP_EXPERT_FFN, T, 1, 1, d, F)
        # workspaces start zeroed: their counter areas must be zero before first use
        u8 = torch.uint8
        self.ws_route = torch.zeros((max(ws_route, 256),), dtype=u8, device=dev)
        self.ws_perm = torch.zeros((max(ws_perm, 256),), dtype=u8, device=dev)
        self.ws_ffn = torch.zeros((max(ws_ffn, 1024),), dtype=u8, device=dev)
        self.ws_shared = torch.zeros((max(ws_sh, 1024),), dtype=u8, device=dev)
        self.can_decode = (P <= 64 and (shared is None or (shared.fmt == routed.fmt and
                                                          shared.F == F)))
        ws_dec = moe_workspace_size(MOE_OP_LAYER_DECODE, T, k, E, d, F) if self.can_decode \
            else 0
        self.can_decode = self.can_decode and ws_dec > 0
        self.ws_decode = torch.zeros((max(ws_dec, 256),), dtype=u8, device=dev)
        ws_xd = moe_workspace_size(MOE_OP_EXPERTS_DECODE, T, k, E, d, F) if self.can_decode \
            else 0
        self.ws_experts_decode = torch.zeros((max(ws_xd, 256),), dtype=u8, device=dev)
        if norm is not None:
            self.xn = torch.empty((T, d), dtype=bf, device=dev)
            self.z = torch.empty((T,), dtype=f32, device=dev)
            ws_blk = moe_workspace_size(MOE_OP_BLOCK_DECODE, T, k, E, d, F) \
                if self.can_decode else 0
            self.ws_block = torch.zeros((max(ws_blk, 256),), dtype=u8, device=dev)
        self.side = torch.cuda.Stream(device=dev)     # default priority

    def forward(self, x, residual=None, out=None):
        T = x.shape[0]
        if T > self.T_max:
            raise ValueError("T = %d exceeds T_max = %d" % (T, self.T_max))
        out = self.out[:T] if out is None else out
        self._experts(x, T)
        moe_combine(self.y_pairs, self.pair_pos, self.weights,
                    self.y_shared if self.shared is not None else None, residual, T, self.k,
                    self.d, out)
        return out

    def block_forward(self, x, out=None):
        """One block of a stack: xn = RMSNorm(x) (moe_rmsnorm), the layer on xn, and the
        gated residual (moe_combine_gated with residual x; moe_combine without a gate row).
        Returns x_next."""
        T = x.shape[0]
        if T > self.T_max:
            raise ValueError("T = %d exceeds T_max = %d" % (T, self.T_max))
        out = self.out[:T] if out is None else out
        moe_rmsnorm(self.norm, x, T, self.d, self.xn, self.z)
        self._experts(self.xn[:T], T)
        ys = self.y_shared if self.shared is not None else None
        if self.norm.gate_w:
            moe_combine_gated(self.y_pairs, self.pair_pos, self.weights, ys, self.z, x, T,
                              self.k, self.d, out)
        else:
            moe_combine(self.y_pairs, self.pair_pos, self.weights, ys, x, T, self.k, self.d,
                        out)
        return out

    def block_decode(self, x, out=None):
        """block_forward's result, bit for bit, in three launches (moe_block_decode)."""
        T = x.shape[0]
        out = self.out[:T] if out is None else out
        moe_block_decode(self.norm, self.router, self.routed, self.shared, x, T, self.k,
                         self.ids, self.weights, out, self.ws_block)
        return out

    def _experts(self, x, T):
        """route, permute and both expert FFNs of x (the combine's inputs)."""
        k, E = self.k, self.E
        main = torch.cuda.current_stream()
        side = self.shared is not None and T > self.SHARED_SIDE_STREAM_ABOVE_TOKENS
        if side:
            # the shared expert does not depend on routing: beside the router
            self.side.wait_stream(main)
            moe_expert_ffn(self.shared, x, T, 1, None, None, None, self.y_shared,
                           self.ws_shared, stream=self.side)
        moe_route(self.router, x, T, k, self.ids, self.weights,
                  self.logits if self.keep_logits else None, self.ws_route)
        moe_permute(self.ids, T, k, E, self.offsets, self.sorted_pairs, self.pair_pos,
                    self.ws_perm)
        moe_expert_ffn(self.routed, x, T, k, self.ids, self.offsets, self.sorted_pairs,
                       self.y_pairs, self.ws_ffn)
        if side:
            main.wait_stream(self.side)
        elif self.shared is not None:
            moe_expert_ffn(self.shared, x, T, 1, None, None, None, self.y_shared,
                           self.ws_shared)

    def route_logits(self, x, ids, weights):
        """moe_route with the logits requested (the fixed-order path) into self.logits; ids
        and weights go to the given buffers."""
        T = x.shape[0]
        moe_route(self.router, x, T, self.k, ids, weights, self.logits, self.ws_route)
        return self.logits[:T]

    def route_only(self, x):
        """moe_route alone (no logits returned) into ids and weights."""
        T = x.shape[0]
        moe_route(self.router, x, T, self.k, self.ids, self.weights, None, self.ws_route)
        return self.ids[:T]

    def decode(self, x, residual=None, out=None):
        T = x.shape[0]
        if T > self.T_max:
            raise ValueError("T = %d exceeds T_max = %d" % (T, self.T_max))
        out = self.out[:T] if out is None else out
        moe_layer_decode(self.router, self.routed, self.shared, x, T, self.k, self.ids,
                         self.weights, residual, out, self.ws_decode)
        return out

    def experts_decode(self, x, residual=None, out=None):
        """The expert side of decode() on its own, from the current ids and weights."""
        T = x.shape[0]
        out = self.out[:T] if out is None else out
        moe_experts_decode(self.routed, self.shared, x, T, self.k, self.ids, self.weights,
                           residual, out, self.ws_experts_decode)
        return out

    __call__ = forward
