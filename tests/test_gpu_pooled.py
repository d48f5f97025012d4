"""GPU parity of gdn_chunk_prefill_pooled: sequence n starts from
state_pool[state_indices[n]] and writes its final state back there (in
place); entries outside the pool mean a zero state and no write; rows no
sequence names stay bitwise unchanged.  Reference: the oracle with the
gathered initial states."""
import numpy as np
import pytest
import torch

import gdn_workloads as W
from _harness import BF16_TOL, F32_TOL, nerr, say

import oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _check(gdn, w, pool_rows, indices, bi, tol, pool_dtype=torch.float32, seed=3):
    gen = torch.Generator().manual_seed(seed)
    pool = (torch.randn(pool_rows, w.Hv, 128, 128, generator=gen) * 0.01).to(pool_dtype)
    idx = torch.tensor(indices, dtype=torch.int64)
    say(f"[gpu] pooled {w.name}: lengths {w.meta.get('lengths')} pool {pool_rows} rows {pool_dtype} "
        f"indices {indices} batch_invariant={bi}")
    # reference: initial states gathered from the pool (zeros for out-of-range entries)
    s0 = torch.zeros(w.N, w.Hv, 128, 128, dtype=pool_dtype)
    valid = [(n, int(i)) for n, i in enumerate(indices) if 0 <= i < pool_rows]
    for n, i in valid:
        s0[n] = pool[i]
    ref_out, ref_fin = oracle.run(w.q, w.k, w.v, w.g, w.beta, w.scale, w.cu_seqlens, s0, w.use_qk_l2norm)
    wd = w.to(DEV)
    dpool = pool.to(DEV)
    out = torch.empty(wd.T, wd.Hv, 128, dtype=wd.q.dtype, device=DEV)
    gdn.gdn_chunk_prefill_pooled(wd.q, wd.k, wd.v, wd.g, wd.beta, wd.scale, wd.cu_seqlens, dpool,
                                 idx.to(torch.int32 if len(indices) % 2 else torch.int64).to(DEV), wd.use_qk_l2norm,
                                 bi, out)
    torch.cuda.synchronize()
    e_out = nerr(out, ref_out)
    say(f"      out {e_out:.3e}")
    assert e_out <= tol
    got = dpool.cpu()
    named = {i for _, i in valid}
    for r in range(pool_rows):
        if r not in named:
            assert torch.equal(got[r], pool[r]), f"pool row {r} (not named) changed"
    worst = 0.0
    for n, i in valid:
        e = nerr(got[i], ref_fin[n])
        worst = max(worst, e)
        assert np.isfinite(e) and e <= tol, f"sequence {n} -> row {i}: {e}"
    say(f"      worst final-state error {worst:.3e}")


def test_pooled_varlen_bf16(gdn):
    w = W.build([100, 64, 0, 300, 17], 2, 4, torch.bfloat16, seed=41, gate="long", state_in=None, name="pool_varlen")
    _check(gdn, w, 9, [7, 2, 5, -1, 0], True, BF16_TOL)


def test_pooled_bf16_pool_out_of_range(gdn):
    w = W.build([130, 65, 200], 2, 4, torch.bfloat16, seed=42, gate="long", state_in=None, name="pool_bf16")
    _check(gdn, w, 4, [3, 11, 1], True, BF16_TOL, pool_dtype=torch.bfloat16)


def test_pooled_fp32(gdn):
    w = W.build([37, 91], 2, 2, torch.float32, seed=43, gate="uniform", state_in=None, name="pool_fp32")
    _check(gdn, w, 3, [2, 0], True, F32_TOL)


def test_pooled_split_path(gdn):
    # one long sequence on few heads takes the split path: the pooled row is read
    # by the fix-up and rewritten by the last segment only
    w = W.build([8200, 50], 1, 4, torch.bfloat16, seed=44, gate="long", state_in=None, name="pool_split")
    _check(gdn, w, 6, [4, 1], False, BF16_TOL)


def test_decode_pooled(gdn):
    """One decode step on a pool: rows named by the index are stepped in place,
    the others stay bitwise unchanged, out-of-range entries start from zero."""
    w = W.build([1] * 5, 2, 4, torch.bfloat16, seed=45, state_in=None, name="pool_decode")
    rows, indices = 8, [6, 0, -1, 3, 9]
    gen = torch.Generator().manual_seed(46)
    pool = torch.randn(rows, w.Hv, 128, 128, generator=gen) * 0.01
    s0 = torch.zeros(w.N, w.Hv, 128, 128)
    valid = [(n, i) for n, i in enumerate(indices) if 0 <= i < rows]
    for n, i in valid:
        s0[n] = pool[i]
    ref_out, ref_fin = oracle.run(w.q, w.k, w.v, w.g, w.beta, w.scale, w.cu_seqlens, s0, w.use_qk_l2norm)
    wd = w.to(DEV)
    dpool = pool.to(DEV)
    out = torch.empty(w.N, w.Hv, 128, dtype=w.q.dtype, device=DEV)
    gdn.gdn_decode_step_pooled(wd.q, wd.k, wd.v, wd.g, wd.beta, 0.0, dpool,
                               torch.tensor(indices, dtype=torch.int32, device=DEV), True, out)
    torch.cuda.synchronize()
    say(f"[gpu] pooled decode: out {nerr(out, ref_out):.3e}")
    assert nerr(out, ref_out) <= BF16_TOL
    got = dpool.cpu()
    for r in set(range(rows)) - {i for _, i in valid}:
        assert torch.equal(got[r], pool[r])
    for n, i in valid:
        assert nerr(got[i], ref_fin[n]) <= BF16_TOL
