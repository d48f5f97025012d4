"""gdn_chunk_prefill_noalloc through the C ABI: the entry point for callers
that cannot allocate (its split-path workspace is the library's fixed scratch
array).  Its output and final state must equal gdn_chunk_prefill's on the
same inputs, on consecutive calls that share the scratch, the second smaller
than the first, and on the largest split plan of the 65,536-token sequence."""
import pytest
import torch

import gdn_workloads as W
from _harness import BF16_TOL, nerr, record, run_oracle, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _both(gdn, w, bi=False):
    wd = w if w.q.is_cuda else w.to(DEV)
    res = []
    for fn in (gdn.gdn_chunk_prefill, gdn.gdn_chunk_prefill_noalloc):
        out = torch.full((wd.T, wd.Hv, 128), float("nan"), dtype=wd.q.dtype, device=DEV)
        fin = torch.full((wd.N, wd.Hv, 128, 128), float("nan"), dtype=wd.state_dtype, device=DEV)
        fn(wd.q, wd.k, wd.v, wd.g, wd.beta, wd.scale, wd.cu_seqlens, wd.initial_state, fin, wd.use_qk_l2norm, bi, out)
        torch.cuda.synchronize()
        res.append((out, fin))
    return res


def test_noalloc_matches_allocating_entry_point(gdn):
    first = W.build([14000, 5000, 0, 1500, 64], 2, 4, torch.bfloat16, seed=81, gate="long", name="noalloc_first")
    second = W.build([9000, 300], 2, 4, torch.bfloat16, seed=82, gate="long", name="noalloc_second")
    for w in (first, second):
        assert gdn.prefill_plan(w.N, w.T, w.Hv, w.q.dtype, False, False,
                                torch.cuda.get_device_properties(0).multi_processor_count)[0] == "split"
        (o1, f1), (o2, f2) = _both(gdn, w)
        say(f"[gpu] no-allocation entry point, {w.name}: T={w.T} N={w.N}")
        assert torch.equal(o1, o2) and torch.equal(f1, f2), w.name
        ro, rf = run_oracle(w)
        e1, e2 = nerr(o2, ro), nerr(f2, rf)
        say(f"      equal to gdn_chunk_prefill bitwise; vs the oracle: out {e1:.3e} state {e2:.3e}")
        record(f"noalloc {w.name} bi=0", e1, e2, BF16_TOL)
        assert e1 <= BF16_TOL and e2 <= BF16_TOL


def test_noalloc_largest_split_and_unsplit(gdn):
    """The 65,536-token sequence on 32 heads (16 segments: the largest split
    workspace on this part), then a small unsplit call."""
    w = W.make(2, device="cuda")
    (o1, f1), (o2, f2) = _both(gdn, w)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    say(f"[gpu] no-allocation entry point, {w.name}: bitwise equal to gdn_chunk_prefill")
    small = W.build([300, 64, 1, 129], 2, 4, torch.bfloat16, seed=83, name="noalloc_unsplit")
    (o1, f1), (o2, f2) = _both(gdn, small, True)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
