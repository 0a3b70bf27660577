"""GPU: the expert FFN's sorted mode when one expert takes many of a call's pairs.  Below
640 pairs every expert runs the GEMV in chunks of a few consecutive sorted positions, one
block per chunk, so such an expert spans many chunks; from 640 pairs an expert with at least
8 pairs (4 above 1024 pairs) takes the grouped MFMA GEMM instead and the others stay on the
GEMV.  Forced routing over T tokens: expert 7 in the first n7, expert 9 in the first n9, the
other slots spread.  T = 60 (600 pairs, all GEMV: expert 7 in every token, over 20 chunks,
expert 9 with 17 pairs), T = 80 (800 pairs: expert 7 in every token, on the GEMM, expert 9
with 7 pairs on the GEMV, over 3 chunks) and T = 64 at the split's threshold (640 pairs:
expert 7 with 8 pairs on the GEMM, expert 9 with 7 on the GEMV).  Bar: the pair rows of experts 7 and 9 and of a sample of the rest against the
oracle (|g - r| <= 2e-2 + 1e-2 |r|, rel-Frobenius 1e-2); for tokens at and around chunk
boundaries, the rows of the pairs that ran on the GEMV bit-identical to the same token
computed alone (one token, ballot mode: the per-pair arithmetic does not depend on the
mode)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import inputs as si

pytestmark = pytest.mark.gpu

ATOL, RTOL, FROB = 2e-2, 1e-2, 1e-2


def _close(got, ref, what):
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), "%s: %d elements out of tolerance, max err %.3g" % (
        what, int(bad.sum()), float(err.max()))
    frob = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert frob <= FROB, "%s: rel-Frobenius %.3g" % (what, frob)


def _forced_ids(T, k, E, n7, n9, seed):
    rng = np.random.default_rng(seed)
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        row = ([7] if t < n7 else []) + ([9] if t < n9 else [])
        rest = [e for e in rng.permutation(E) if e not in (7, 9)]
        row += rest[:k - len(row)]
        ids[t] = row
    return ids


def _expert_call(moe, lay, x, ids, k):
    """moe_permute + moe_expert_ffn (routed experts) on the given ids; returns the pair rows
    in pair order and the positions."""
    from quantized_sparse_moe_router_amd import _lib
    T = x.shape[0]
    E, d, F = lay.routed.E, lay.routed.d, lay.routed.F
    dev = x.device
    ids_d = torch.from_numpy(ids).to(dev)
    P = T * k
    offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    sp = torch.empty((P,), dtype=torch.int32, device=dev)
    pp = torch.empty((P,), dtype=torch.int32, device=dev)
    ws_p = torch.zeros((max(_lib.moe_workspace_size(_lib.MOE_OP_PERMUTE, T, k, E, d, F), 256),),
                       dtype=torch.uint8, device=dev)
    _lib.moe_permute(ids_d, T, k, E, offsets, sp, pp, ws_p)
    y = torch.empty((P, d), dtype=torch.bfloat16, device=dev)
    ws_f = torch.zeros((max(_lib.moe_workspace_size(_lib.MOE_OP_EXPERT_FFN, T, k, E, d, F),
                            1024),), dtype=torch.uint8, device=dev)
    ex = moe.experts_desc_of(lay.routed)
    _lib.moe_expert_ffn(ex, x, T, k, ids_d, offsets, sp, y, ws_f)
    torch.cuda.synchronize()
    moe.moe_check_device_error()
    pos = pp.cpu().numpy().astype(np.int64)
    return y[torch.from_numpy(pos).to(dev)], offsets.cpu().numpy()


def _hot_rows(rows):
    # the split of the library's expert FFN: experts with at least this many pairs take the
    # grouped GEMM (0: none)
    return 0 if rows < 640 else (8 if rows <= 1024 else 4)


@pytest.mark.parametrize("T,n7,n9", [(60, 60, 17), (80, 80, 7), (64, 8, 7)])
def test_expert_with_many_pairs_spans_chunks(T, n7, n9):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_sparse_moe_router_amd as moe
    w = synth.WORKLOADS["decode_d2048_e512_top10_t1"]
    lay = synth.make_layer(w, seed=0, device="cuda")
    k, E = w.k, w.E
    x = synth.make_tokens(w, T=T, seed=3, device="cuda", stream=80)
    ids = _forced_ids(T, k, E, n7, n9, seed=5)
    print("case forced routing T=%d k=%d: expert 7 x %d pairs, expert 9 x %d" % (T, k, n7, n9),
          flush=True)
    y, offsets = _expert_call(moe, lay, x, ids, k)
    # the other slots are spread at random: 7 and 9 keep exactly n7 and n9 pairs
    assert offsets[8] - offsets[7] == n7 and offsets[10] - offsets[9] == n9
    y_h = y.float().cpu().numpy().astype(np.float64).reshape(T, k, -1)
    ex_h = lay.routed.host()
    x_h = si.bits16(x)
    # every pair of experts 7 and 9, and one more slot of 24 tokens
    rng = np.random.default_rng(11)
    pairs = [(t, 0) for t in range(n7)] + [(t, 1) for t in range(n9)]
    pairs += [(int(t), 2 + int(rng.integers(0, k - 2))) for t in rng.choice(T, 24, replace=False)]
    tok = np.array([t for t, _ in pairs], np.int32)
    exp = np.array([ids[t, j] for t, j in pairs], np.int32)
    ref = oracle.expert_ffn_pairs(ex_h, x_h, tok, exp)
    got = np.stack([y_h[t, j] for t, j in pairs])
    _close(got[:n7], ref[:n7], "expert 7 (%d pairs)" % n7)
    _close(got[n7:n7 + n9], ref[n7:n7 + n9], "expert 9 (%d pairs)" % n9)
    _close(got, ref, "all sampled pairs")
    # tokens at and around chunk boundaries: the pairs whose expert ran on the GEMV are
    # bit-identical to the token alone
    hot = _hot_rows(T * k)
    counts = np.diff(offsets)
    yb = y.view(torch.int16).reshape(T, k, -1)
    checked = 0
    for t in (0, 1, 2, 3, 5, 6, 15, 16, 17, T - 1):
        y1, _ = _expert_call(moe, lay, x[t:t + 1].contiguous(), ids[t:t + 1], k)
        for j in range(k):
            if hot == 0 or counts[ids[t, j]] < hot:
                assert torch.equal(y1.view(torch.int16)[j], yb[t, j]), "token %d slot %d" % (t, j)
                checked += 1
    assert checked >= 10 * (k - 1)
