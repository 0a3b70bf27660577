"""GPU: moe_permute against the oracle's stable counting sort, on id tables built to
exercise each form -- one wave (at most 64 pairs), one block with a thread per pair (at most
1024) and the chunked form (more): ragged last chunks, expert counts that are not powers of
two, every pair on one expert, and ids outside [0, E) (dropped, flag raised,
pair_pos = -1)."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_sparse_moe_router_amd as moe
    return moe


def _ids(kind, T, k, E, rng):
    if kind == "uniform":
        return rng.integers(0, E, size=(T, k))
    if kind == "skewed":        # Zipf-like: a few experts take most pairs
        r = rng.zipf(1.3, size=(T, k)) - 1
        return np.minimum(r, E - 1)
    if kind == "one_expert":
        return np.full((T, k), E // 2)
    if kind == "bad_ids":       # 1 % of ids outside [0, E), the first and last always
        a = rng.integers(0, E, size=(T, k))
        bad = rng.random((T, k)) < 0.01
        a[bad] = np.where(rng.random(bad.sum()) < 0.5, -1, E + 3)
        a[0, 0] = -1
        a[-1, -1] = E + 3
        return a
    raise ValueError(kind)


@pytest.mark.parametrize("T,k,E", [
    (1, 10, 512), (6, 10, 512), (32, 2, 16),                       # one wave
    (7, 10, 512), (64, 10, 512), (100, 10, 1000), (128, 8, 1024),  # one block
    (33, 2, 16), (93, 11, 1000),
    (103, 10, 512), (204, 10, 512), (128, 16, 1024), (1000, 2, 16),  # one block, 2 per thread
    (205, 10, 512), (500, 10, 512), (4001, 10, 512),               # chunked
    (2100, 2, 16), (900, 7, 1000), (12289, 8, 1024)])
@pytest.mark.parametrize("kind", ["uniform", "skewed", "one_expert", "bad_ids"])
def test_permute_every_form(T, k, E, kind):
    moe = _gpu()
    rng = np.random.default_rng(T * 31 + E + len(kind))
    ids_h = _ids(kind, T, k, E, rng).astype(np.int32)
    print("case T=%d k=%d E=%d %s" % (T, k, E, kind), flush=True)
    P = T * k
    ids = torch.from_numpy(ids_h).cuda()
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    sp = torch.full((P,), -7, dtype=torch.int32, device="cuda")
    pp = torch.full((P,), -7, dtype=torch.int32, device="cuda")
    ws_n = moe.moe_workspace_size(moe.MOE_OP_PERMUTE, T, k, E, 0, 0)
    ws = torch.zeros((max(ws_n, 256),), dtype=torch.uint8, device="cuda")
    moe.moe_permute(ids, T, k, E, offsets, sp, pp, ws)
    torch.cuda.synchronize()
    off_ref, sp_ref, pp_ref, bad = oracle.permute(ids_h, E)
    if bad:
        with pytest.raises(moe.MoeError):
            moe.moe_check_device_error()
    else:
        moe.moe_check_device_error()
    n = int(off_ref[E])
    assert np.array_equal(offsets.cpu().numpy(), off_ref)
    assert np.array_equal(sp[:n].cpu().numpy(), sp_ref[:n])
    assert np.array_equal(pp.cpu().numpy(), pp_ref)
