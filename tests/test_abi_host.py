"""Host-side checks of the C ABI: the library loads, exports every entry point declared in
include/moe.h, sizes workspaces, and rejects bad arguments before launching anything.
No call here reaches a kernel, so these run without a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def L():
    from quantized_sparse_moe_router_amd import _lib
    return _lib.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(moe_\w+)\s*\(", src, re.M)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    from quantized_sparse_moe_router_amd import _lib
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def test_peaks_library_exports_its_declared_symbols():
    # bench.py's measurement helpers: a library of their own, declared in moe_peaks.h
    import re
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    hdr = open(os.path.join(root, "include", "moe_peaks.h")).read()
    names = re.findall(r"^int\s+(moe_peaks_\w+)\(", hdr, re.M)
    assert set(names) == {"moe_peaks_stream_blocks", "moe_peaks_stream_read",
                          "moe_peaks_mfma_loop"}
    P = ctypes.CDLL(os.path.join(root, "quantized_sparse_moe_router_amd", "libmoe_peaks.so"))
    for n in names:
        assert hasattr(P, n), n
    assert P.moe_peaks_stream_blocks() > 0


def test_version_and_status_strings(L):
    assert b"gfx950" in L.moe_version()
    assert L.moe_status_string(0) == b"ok"
    assert L.moe_status_string(-3) == b"workspace too small"


def test_workspace_sizes(L):
    from quantized_sparse_moe_router_amd import _lib
    assert L.moe_workspace_size(_lib.MOE_OP_ROUTE, 1, 10, 512, 2048, 512) == 256 + 2048
    assert L.moe_workspace_size(_lib.MOE_OP_ROUTE, 0, 10, 512, 2048, 512) == 0
    # small permutes run in one block without workspace
    assert L.moe_workspace_size(_lib.MOE_OP_PERMUTE, 1, 10, 512, 2048, 512) == 0
    assert L.moe_workspace_size(_lib.MOE_OP_PERMUTE, 8192, 10, 512, 2048, 512) >= 80 * 512 * 4
    # the one-block grouping (up to 2048 pairs, two per thread) needs none; above, a chunk
    # table of 1024-pair chunks plus the expert totals
    assert L.moe_workspace_size(_lib.MOE_OP_PERMUTE, 204, 10, 512, 0, 0) == 0
    assert L.moe_workspace_size(_lib.MOE_OP_PERMUTE, 128, 16, 1024, 0, 0) == 0
    assert L.moe_workspace_size(_lib.MOE_OP_PERMUTE, 205, 10, 512, 0, 0) == (3 + 1) * 512 * 4
    assert L.moe_workspace_size(_lib.MOE_OP_EXPERT_FFN, 1, 10, 512, 2048, 512) >= 10 * 512 * 2
    # the decode operations report 0 where they do not run: more than 64 pairs, or a
    # (d_model, d_ff) pair without decode kernels
    for op in (_lib.MOE_OP_LAYER_DECODE, _lib.MOE_OP_EXPERTS_DECODE, _lib.MOE_OP_BLOCK_DECODE):
        assert L.moe_workspace_size(op, 6, 10, 512, 2048, 512) > 0
        assert L.moe_workspace_size(op, 7, 10, 512, 2048, 512) == 0
        assert L.moe_workspace_size(op, 1, 4, 16, 512, 256) == 0
        assert L.moe_workspace_size(op, 1, 4, 16, 1024, 512) > 0
    # 640 pairs (the GEMV's sorted mode): h rows and a chunk list of two int4 per entry, at
    # most one entry per pair
    assert L.moe_workspace_size(_lib.MOE_OP_EXPERT_FFN, 64, 10, 512, 2048, 512) >= \
        640 * 512 * 2 + 640 * 32
    # more than 512 tokens without a logits output: the bounded form also keeps bf16 plane
    # rows of the router (two per fp32 row) and one norm bound per expert
    assert L.moe_workspace_size(_lib.MOE_OP_ROUTE, 8192, 10, 512, 2048, 0) == \
        256 + 8192 * 512 * 4 + 512 * 2 * 2048 * 2 + 512 * 4
    assert L.moe_workspace_size(_lib.MOE_OP_ROUTE, 16, 10, 512, 2048, 0) == 256 + 16 * 512 * 4
    assert L.moe_workspace_size(_lib.MOE_OP_ROUTE, 64, 10, 512, 2048, 0) == 256 + 64 * 512 * 4
    assert L.moe_workspace_size(_lib.MOE_OP_ROUTE, 512, 10, 512, 2048, 0) == \
        256 + 512 * 512 * 4
    assert L.moe_workspace_size(_lib.MOE_OP_ROUTE, 513, 10, 512, 2048, 0) == \
        256 + 513 * 512 * 4 + 512 * 2 * 2048 * 2 + 512 * 4


def _router(fmt=0, E=512, d=2048, w=16, scale=None, reserved=0):
    from quantized_sparse_moe_router_amd import _lib
    return _lib.moe_router(fmt, E, d, reserved, w, scale, None)


def _experts(fmt=2, E=512, d=2048, F=512, p=16):
    from quantized_sparse_moe_router_amd import _lib
    return _lib.moe_experts(fmt, E, d, F, p, p, p, p, p, p)


def _err(L):
    return L.moe_last_error().decode()


@pytest.mark.parametrize("kw,T,k,expect", [
    (dict(fmt=3), 1, 10, "format"),
    (dict(E=0), 1, 10, "n_experts"),
    (dict(E=2000), 1, 10, "n_experts"),
    (dict(d=300), 1, 10, "d_model"),
    (dict(fmt=1, d=256), 1, 10, "d_model"),
    (dict(), -1, 10, "T"),
    (dict(), 1, 0, "k"),
    (dict(E=8), 1, 9, "k"),
    (dict(), 1, 65, "k"),
    (dict(w=None), 1, 10, "router weights"),
    (dict(w=8), 1, 10, "aligned"),
    (dict(fmt=1), 1, 10, "scales"),
    (dict(reserved=1), 1, 10, "reserved"),
])
def test_route_rejects(L, kw, T, k, expect):
    r = _router(**kw)
    st = L.moe_route(ctypes.byref(r), 16, T, k, 16, 16, None, None, 0, None)
    assert st == -1 and expect in _err(L)


def test_route_null_descriptor_and_workspace(L):
    assert L.moe_route(None, 16, 1, 10, 16, 16, None, None, 0, None) == -1
    r = _router()
    st = L.moe_route(ctypes.byref(r), 16, 1, 10, 16, 16, None, None, 0, None)
    assert st == -3 and "workspace" in _err(L)
    st = L.moe_route(ctypes.byref(r), 16, 1, 10, 16, 16, None, 16, 100, None)
    assert st == -3
    # bounded form (513 tokens, no logits): counter + logits alone are not enough
    st = L.moe_route(ctypes.byref(r), 16, 513, 10, 16, 16, None, 16, 256 + 513 * 512 * 4, None)
    assert st == -3 and "workspace" in _err(L)
    # with a logits output the workspace still holds the arrival counter
    st = L.moe_route(ctypes.byref(r), 16, 1, 10, 16, 16, 16, None, 0, None)
    assert st == -3
    st = L.moe_route(ctypes.byref(r), 8, 1, 10, 16, 16, 16, None, 0, None)
    assert st == -1 and "x" in _err(L)


def test_route_zero_tokens_is_noop(L):
    r = _router()
    assert L.moe_route(ctypes.byref(r), None, 0, 10, None, None, None, None, 0, None) == 0


def test_permute_rejects(L):
    assert L.moe_permute(16, -1, 10, 512, 16, 16, 16, None, 0, None) == -1
    assert L.moe_permute(16, 1, 0, 512, 16, 16, 16, None, 0, None) == -1
    assert L.moe_permute(16, 1, 10, 0, 16, 16, 16, None, 0, None) == -1
    assert L.moe_permute(16, 1, 10, 512, None, 16, 16, None, 0, None) == -1
    assert L.moe_permute(None, 1, 10, 512, 16, 16, 16, None, 0, None) == -1
    assert L.moe_permute(16, 8192, 10, 512, 16, 16, 16, None, 0, None) == -3
    assert L.moe_permute(16, 2 ** 30, 10, 512, 16, 16, 16, None, 0, None) == -1


def test_expert_ffn_rejects(L):
    def call(ex, x=16, T=1, k=10, ids=16, off=16, sp=16, y=16, ws=16, wsb=1 << 30):
        return L.moe_expert_ffn(ctypes.byref(ex) if ex is not None else None, x, T, k, ids,
                                off, sp, y, ws, wsb, None)
    assert call(None) == -1
    assert call(_experts(fmt=0)) == -1
    assert call(_experts(fmt=6)) == -1
    assert call(_experts(d=300)) == -1
    assert call(_experts(F=96)) == -1
    assert call(_experts(p=None)) == -1
    assert call(_experts(p=8)) == -1
    assert call(_experts(), ids=None) == -1                     # partly grouped
    assert call(_experts(), ids=None, off=None, sp=None) == -1  # dense needs E == 1
    assert call(_experts(), x=8) == -1
    assert call(_experts(), ws=None) == -3
    assert call(_experts(), wsb=10) == -3
    assert call(_experts(), T=-1) == -1
    assert call(_experts(), T=0) == 0
    # the grouped GEMM addresses x and h with 32-bit byte offsets: 2^20 tokens of d 2048
    # bf16 are 4 GiB
    assert call(_experts(), T=1 << 20, k=1, wsb=1 << 62) == -2
    assert "4 GiB" in _err(L)


def test_combine_rejects(L):
    assert L.moe_combine(16, 16, 16, None, None, 1, 10, 2047, 16, None) == -1
    assert L.moe_combine(16, 16, 16, None, None, 1, 0, 2048, 16, None) == -1
    assert L.moe_combine(None, 16, 16, None, None, 1, 10, 2048, 16, None) == -1
    assert L.moe_combine(8, 16, 16, None, None, 1, 10, 2048, 16, None) == -1
    assert L.moe_combine(16, 16, 16, 8, None, 1, 10, 2048, 16, None) == -1
    assert L.moe_combine(None, None, None, None, None, 0, 10, 2048, None, None) == 0


def test_layer_decode_rejects(L):
    from quantized_sparse_moe_router_amd import _lib
    r = _router()
    ex = _experts()

    def call(r=r, ex=ex, sh=None, T=1, k=10, x=16, ids=16, w=16, res=None, out=16, ws=16,
             wsb=1 << 30):
        return L.moe_layer_decode(ctypes.byref(r) if r is not None else None,
                                  ctypes.byref(ex) if ex is not None else None,
                                  ctypes.byref(sh) if sh is not None else None,
                                  x, T, k, ids, w, res, out, ws, wsb, None)
    assert call(r=None) == -1
    assert call(ex=None) == -1
    assert call(ex=_experts(E=256)) == -1 and "differ" in _err(L)
    assert call(sh=_experts(E=2)) == -1
    assert call(sh=_experts(E=1, F=1024)) == -2
    assert call(sh=_experts(E=1, fmt=3)) == -2
    assert call(T=7) == -2 and "four calls" in _err(L)          # 70 pairs
    assert call(ex=_experts(F=4096)) == -2                       # no GEMV shape
    assert call(k=0) == -1
    assert call(T=-1) == -1
    assert call(x=8) == -1
    assert call(res=8) == -1
    assert call(ids=None) == -1
    assert call(ws=None) == -3
    assert call(wsb=100) == -3
    assert call(T=0, x=None, out=None, ids=None, w=None, ws=None, wsb=0) == 0
    need = L.moe_workspace_size(_lib.MOE_OP_LAYER_DECODE, 1, 10, 512, 2048, 512)
    assert need > 256 + 512 * 4
    assert call(wsb=need - 1) == -3
    assert L.moe_workspace_size(_lib.MOE_OP_LAYER_DECODE, 7, 10, 512, 2048, 512) == 0


def test_norm_calls_reject(L):
    from quantized_sparse_moe_router_amd import _lib
    P = ctypes.c_void_p

    def nd(gamma=16, gate_w=16, eps=1e-6, gate_b=0.0):
        return _lib.moe_norm(gamma, gate_w, eps, gate_b)

    def rms(n=nd(), x=16, T=2, d=2048, xn=16, z=16):
        return L.moe_rmsnorm(ctypes.byref(n) if n is not None else None, P(x), T, d, P(xn),
                             P(z), None)
    assert rms(n=None) == -1
    assert rms(n=nd(gamma=None)) == -1
    assert rms(n=nd(gamma=8)) == -1                       # misaligned gamma
    assert rms(n=nd(gate_w=8)) == -1
    assert rms(n=nd(eps=-1.0)) == -1
    assert rms(n=nd(eps=float("nan"))) == -1
    assert rms(n=nd(gate_b=float("inf"))) == -1
    assert rms(d=768) == -1
    assert rms(T=-1) == -1
    assert rms(z=0) == -1                                 # a gate row needs z
    assert rms(x=8) == -1
    assert rms(T=0, x=0, xn=0, z=0) == 0
    # gated combine: z required
    assert L.moe_combine_gated(P(16), P(16), P(16), None, None, None, 2, 10, 2048, P(16),
                               None) == -1
    assert L.moe_combine_gated(P(16), P(16), P(16), None, P(16), None, 2, 10, 12, P(16),
                               None) == -1
    # the decode block: the layer's checks, the norm's, and T <= 16
    r, ex = _router(), _experts()
    n = nd()

    def blk(n=n, T=1, k=10, ws=16, wsb=1 << 30):
        return L.moe_block_decode(ctypes.byref(n) if n is not None else None,
                                  ctypes.byref(r), ctypes.byref(ex), None, P(16), T, k,
                                  P(16), P(16), P(16), P(ws), wsb, None)
    assert blk(n=None) == -1
    assert blk(n=nd(gamma=None)) == -1
    assert blk(T=7) == -2                                 # 70 pairs
    assert blk(T=17, k=1) == -2 and "T = 17" in _err(L)
    assert blk(wsb=100) == -3
    need = L.moe_workspace_size(_lib.MOE_OP_BLOCK_DECODE, 4, 10, 512, 2048, 512)
    assert need == L.moe_workspace_size(_lib.MOE_OP_LAYER_DECODE, 4, 10, 512, 2048, 512) + \
        4 * 2048 * 2 + 256
    assert blk(T=4, wsb=need - 1) == -3


def test_dequant_probe_rejects(L):
    P = ctypes.c_void_p
    dummy = P(16)
    # bad format, bad form, negative count, NULL pointers: rejected before any launch
    assert L.moe_dequant_probe(0, 0, dummy, dummy, 1, dummy, None) == -1
    assert L.moe_dequant_probe(6, 0, dummy, dummy, 1, dummy, None) == -1
    assert L.moe_dequant_probe(2, 2, dummy, dummy, 1, dummy, None) == -1
    assert L.moe_dequant_probe(2, 0, dummy, dummy, -1, dummy, None) == -1
    assert L.moe_dequant_probe(3, 1, None, dummy, 1, dummy, None) == -1
    assert L.moe_dequant_probe(2, 0, P(8), dummy, 1, dummy, None) == -1   # misaligned
    assert L.moe_dequant_probe(2, 0, None, None, 0, None, None) == 0      # no-op


def test_bench_refuses_more_than_one_gpu():
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


# ---------------------------------------------------------------- workspace sizes, fuzzed

from hypothesis import given, settings, strategies as st  # noqa: E402

_I32 = st.one_of(st.integers(-2 ** 31, 2 ** 31 - 1),
                 st.sampled_from([0, 1, 2, 4, 10, 16, 64, 65, 127, 128, 256, 512, 513, 640, 1023,
                                  1024, 1025, 2048, 4096, 8192, 32768, 2 ** 31 - 1]))


@settings(max_examples=3000, deadline=None)
@given(op=st.integers(-1, 7), T=_I32, k=_I32, E=_I32, d=_I32, F=_I32)
def test_workspace_size_never_wraps(L, op, T, k, E, d, F):
    """Over the whole int32 range of every argument: 0 for the sizes every call rejects, and
    otherwise at least the buffers the operation's calls place in the workspace (so a
    wrapped product, which would come out small, fails), never near 2^64."""
    n = L.moe_workspace_size(op, T, k, E, d, F)
    assert 0 <= n < 2 ** 63
    pairs = T * k
    if T <= 0 or k <= 0 or E <= 0 or E > 1024 or pairs > 2 ** 31 - 1:
        assert n == 0
        return
    if op == 0:                                   # route: counter + logits [T][E] fp32
        if T > 512 and d <= 0:
            assert n == 0
        else:
            assert n >= 256 + T * E * 4
            if T > 512:                            # + bf16 router planes and row norms
                assert n >= 256 + T * E * 4 + E * 2 * d * 2 + E * 4
    elif op == 2:                                 # expert FFN: h rows [pairs][d_ff] bf16
        assert n == 0 if F <= 0 else n >= pairs * F * 2
    elif op in (3, 4, 5):                         # decode operations: at most 64 pairs
        if pairs > 64 or F <= 0 or d <= 0:
            assert n == 0
        elif n:
            assert n >= pairs * F * 2
    elif op not in (1,):
        assert n == 0
