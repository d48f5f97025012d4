"""GPU parity of the state checkpoints written by gdn_chunk_prefill_checkpointed:
slot n * P + i must equal the oracle's state of sequence n after its first
(i + 1) * I tokens (the oracle run on that prefix alone), slots past a
sequence's end stay untouched, and the outputs and final states equal those
of the plain scan's contract."""
import numpy as np
import pytest
import torch

import gdn_workloads as W
from _harness import BF16_TOL, F32_TOL, nerr, run_oracle, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _prefix(w, n, L):
    """One-sequence workload: the first L tokens of sequence n of w (all heads)."""
    one = W.slice_item(w, n, range(w.Hv))
    cut = lambda t: None if t is None else t[:L]
    return W.Workload(f"{w.name}[n={n},:{L}]", cut(one.q), cut(one.k), cut(one.v), cut(one.g), cut(one.beta),
                      torch.tensor([0, L], dtype=torch.int64), one.initial_state, torch.float32,
                      w.use_qk_l2norm, w.scale)


def _run(gdn, w, P, interval, bi, ck_dtype=torch.float32):
    wd = w.to(DEV)
    out = torch.empty(wd.T, wd.Hv, 128, dtype=wd.q.dtype, device=DEV)
    fin = torch.empty(wd.N, wd.Hv, 128, 128, dtype=wd.state_dtype, device=DEV)
    ck = torch.full((wd.N * P, wd.Hv, 128, 128), float("nan"), dtype=ck_dtype, device=DEV)
    gdn.gdn_chunk_prefill_checkpointed(wd.q, wd.k, wd.v, wd.g, wd.beta, wd.scale, wd.cu_seqlens, wd.initial_state,
                                       fin, wd.use_qk_l2norm, bi, ck, P, interval, out)
    torch.cuda.synchronize()
    return out, fin, ck


def _check(gdn, w, P, interval, bi, tol, ck_dtype=torch.float32):
    say(f"[gpu] checkpoints {w.name}: lengths {w.meta.get('lengths')} Hv={w.Hv} P={P} interval={interval} "
        f"batch_invariant={bi} dtype={ck_dtype}")
    out, fin, ck = _run(gdn, w, P, interval, bi, ck_dtype)
    ref_out, ref_fin = run_oracle(w)
    e_out, e_fin = nerr(out, ref_out), nerr(fin, ref_fin)
    say(f"      out {e_out:.3e} final state {e_fin:.3e}")
    assert e_out <= tol and e_fin <= tol
    ck = ck.float().cpu()
    lengths = w.meta["lengths"]
    worst = 0.0
    for n, length in enumerate(lengths):
        for i in range(P):
            slot = ck[n * P + i]
            L = (i + 1) * interval
            if L > length:
                assert torch.isnan(slot).all(), f"slot {n},{i} past the end was written"
                continue
            _, ref = run_oracle(_prefix(w, n, L))
            e = nerr(slot, ref[0])
            worst = max(worst, e)
            assert np.isfinite(e) and e <= tol, f"checkpoint n={n} i={i}: {e}"
    say(f"      worst checkpoint error {worst:.3e}")


def test_checkpoints_varlen_bf16(gdn):
    w = W.build([64, 130, 256, 300, 1, 0, 192], 2, 4, torch.bfloat16, seed=31, gate="long", name="ck_varlen")
    _check(gdn, w, 4, 64, True, BF16_TOL)


def test_checkpoints_interval_and_bf16_slots(gdn):
    w = W.build([512, 300, 129], 2, 4, torch.bfloat16, seed=32, gate="long", name="ck_interval")
    _check(gdn, w, 3, 128, True, BF16_TOL, ck_dtype=torch.bfloat16)


def test_checkpoints_fp32(gdn):
    w = W.build([37, 128, 200], 2, 2, torch.float32, seed=33, gate="uniform", name="ck_fp32")
    _check(gdn, w, 3, 64, True, F32_TOL)


def test_checkpoints_split_path(gdn):
    # one long sequence on few heads takes the split path (segments of 1024
    # tokens, state fix-up); checkpoints every 512 tokens cross segment bounds
    w = W.build([4096], 1, 4, torch.bfloat16, seed=34, gate="long", name="ck_split")
    _check(gdn, w, 8, 512, False, BF16_TOL)


def test_checkpoint_at_end_equals_final_state(gdn):
    w = W.build([256, 192], 2, 4, torch.bfloat16, seed=35, gate="long", name="ck_end")
    out, fin, ck = _run(gdn, w, 1, 192, True)
    # sequence 1 ends exactly on its first checkpoint; sequence 0 passes it
    assert torch.equal(ck[1], fin[1]), "checkpoint at the sequence end must equal the final state"
