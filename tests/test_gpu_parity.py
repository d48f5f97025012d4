"""GPU parity: the HIP scan against the CPU oracle on seeded workloads.

Tolerances (max normalised error over each tensor): 1e-4 for fp32 inputs,
2e-2 for bf16 inputs; out and final state are checked separately.
Full-size workloads are checked whole: every element of the output and of
the final state against the fp64 oracle on the same inputs.
"""
import numpy as np
import pytest
import torch

import gdn_workloads as W
from _harness import BF16_TOL, F32_TOL, check, nerr, nerr_dev, record, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("variant", [None, "raw_l2"])
@pytest.mark.parametrize("bi", [True, False])
def test_tiny_fp32(gdn, variant, bi):
    check(gdn, W.make(0, variant=variant), F32_TOL, bi)


@pytest.mark.parametrize("variant", [None, "gates_bf16", "long_memory"])
@pytest.mark.parametrize("bi", [True, False])
def test_varlen_bf16(gdn, variant, bi):
    check(gdn, W.make(1, variant=variant), BF16_TOL, bi)


@pytest.mark.parametrize("bi", [True, False])
def test_many_short_bf16_state(gdn, bi):
    w = W.make(3)
    out, fin = check(gdn, w, BF16_TOL, bi)
    # empty sequences pass the (bf16) initial state through bitwise
    for n in (0, 127, 255):
        assert torch.equal(fin[n].cpu(), w.initial_state[n])


_ORACLE_CACHE = {}


def _whole(gdn, w, bi, tol=BF16_TOL):
    """The whole output and final state of a full-size run against the fp64
    oracle on the same inputs (the oracle's result is kept for the workload's
    other batch_invariant mode)."""
    say(f"[gpu] {w.name}: T={w.T} N={w.N} Hqk={w.Hqk} Hv={w.Hv} batch_invariant={bi} (whole tensors)")
    out, fin = run_gpu(gdn, w, bi)
    assert torch.isfinite(out).all() and (fin is None or torch.isfinite(fin).all())
    if w.name not in _ORACLE_CACHE:
        _ORACLE_CACHE.clear()
        _ORACLE_CACHE[w.name] = run_oracle(w.to("cpu"))
    ro, rf = _ORACLE_CACHE[w.name]
    e1 = nerr_dev(out, ro)
    e2 = nerr_dev(fin, rf) if fin is not None else 0.0
    say(f"      max normalised error: out {e1:.3e}  state {e2:.3e}  (tol {tol:g})")
    record(f"{w.name} T={w.T} bi={int(bool(bi))} (whole)", e1, e2 if fin is not None else None, tol)
    assert e1 <= tol and e2 <= tol


@pytest.mark.parametrize("variant", [None, "alt_gates", "long_memory"])
@pytest.mark.parametrize("bi", [False, True])
def test_long_single_whole(gdn, variant, bi):
    """One 65,536-token sequence: the split path (segment maps, state fix-up,
    per-segment scan) with batch_invariant off, one work item per head with it
    on; the sigmoid gates, the U[0.9, 1) / U(0, 1) gates, and long-memory gates
    (g ~ U[0.999, 1]) that carry the state across every chunk and segment."""
    _whole(gdn, W.make(2, device="cuda", variant=variant), bi)


@pytest.mark.parametrize("variant", [None, "alt_gates"])
@pytest.mark.parametrize("bi", [False, True])
def test_large_batch_whole(gdn, variant, bi):
    _whole(gdn, W.make(4, device="cuda", variant=variant), bi)


@pytest.mark.parametrize("bi", [False, True])
def test_many_short_alt_gates(gdn, bi):
    w = W.make(3, variant="alt_gates")
    out, fin = check(gdn, w, BF16_TOL, bi)
    for n in (0, 127, 255):   # empty sequences pass their bf16 state through
        assert torch.equal(fin[n].cpu(), w.initial_state[n])


@pytest.mark.parametrize("lengths,label", [([8192] * 34, "four-wave"), ([34816] * 8, "pipelined")])
def test_offsets_beyond_2gib(gdn, lengths, label):
    """278,528 tokens: the v and out rows of the last sequences (Hv 32, bf16,
    8 KB per token) lie beyond 2^31 bytes from the buffer start, on both scan
    kernels (1088 work items, and 256 = one per CU)."""
    w = W.build(lengths, 16, 32, torch.bfloat16, seed=71, device="cuda", name=f"beyond_2gib_{label}")
    assert (w.T - 1) * w.Hv * 128 * 2 >= 2 ** 31
    _whole(gdn, w, True)


def _extreme_gates(w, second):
    """Chunk 0 of every sequence decays by -27.5 (the lazy scale ends just above
    2^-40), chunk 1 by `second` (above -60, so the shared-Vnew path), which
    renormalises with sigma gamma_L ~ 3e-38 (-59) or ~ 1.8e-30 (-41)."""
    t = torch.arange(w.T)
    starts = w.cu_seqlens.to(torch.int64)
    seq = torch.searchsorted(starts[1:], t, right=True)
    chunk = ((t - starts[seq]) // 64).unsqueeze(1)
    return torch.where(chunk == 0, torch.full_like(w.g, float(np.exp(-27.5 / 64))),
                       torch.where(chunk == 1, torch.full_like(w.g, float(np.exp(second / 64))), w.g))


@pytest.mark.parametrize("second", [-59.0, -41.0])
@pytest.mark.parametrize("qk_scale", [2 ** 10, 2 ** 14])
@pytest.mark.parametrize("lengths", [(300, 64 * 3 + 5), (9000, 200)])
def test_qk_scale_invariance_with_l2norm(gdn, qk_scale, second, lengths):
    """With the in-kernel L2 norm the result does not depend on the scale of raw
    q and k ("flashinfer.cudnn.cudnn_chunk_gated_delta_rule", Parameters:
    use_qk_l2norm_in_kernel).  q and k times a power of two (exact in bf16),
    under gates that renormalise the lazy decay on a fast-path chunk, against
    the oracle on the unscaled inputs.  The first case runs one work item per
    head, the second (batch_invariant off) the split path too."""
    w = W.build(list(lengths), 2, 4, torch.bfloat16, seed=37, name=f"qk_scale{qk_scale}")
    w = W.Workload(**{**w.__dict__, "g": _extreme_gates(w, second)})
    big = W.Workload(**{**w.__dict__, "q": w.q * qk_scale, "k": w.k * qk_scale})
    assert torch.equal(big.q.float() / qk_scale, w.q.float())
    bi = lengths[0] < 1000
    say(f"[gpu] q/k x {qk_scale}, chunk-1 log-decay {second}, lengths {lengths}, batch_invariant={bi}")
    out, fin = run_gpu(gdn, big, bi)
    assert torch.isfinite(out).all() and torch.isfinite(fin).all()
    ro, rf = run_oracle(w)
    e1, e2 = nerr(out, ro), nerr(fin, rf)
    say(f"      vs the oracle on unscaled q/k: out {e1:.3e} state {e2:.3e}")
    record(f"q/k x{qk_scale} decay {second} T={w.T} bi={int(bi)}", e1, e2, BF16_TOL)
    assert e1 <= BF16_TOL and e2 <= BF16_TOL


@pytest.mark.parametrize("lengths", [[1], [63], [64], [65], [1, 127, 128, 129, 0, 200]])
def test_ragged_lengths(gdn, lengths):
    w = W.build(lengths, 2, 4, torch.bfloat16, seed=7, gate="long", name=f"ragged{lengths}")
    check(gdn, w, BF16_TOL, True)


def test_ragged_lengths_fp32(gdn):
    w = W.build([1, 63, 64, 65, 130], 2, 2, torch.float32, seed=8, gate="long", name="ragged_fp32")
    check(gdn, w, F32_TOL, True)


@pytest.mark.parametrize("r", [1, 4, 8])
def test_head_ratios(gdn, r):
    w = W.build([100, 37], 4, 4 * r, torch.bfloat16, seed=9, name=f"ratio{r}")
    check(gdn, w, BF16_TOL, True)


@pytest.mark.parametrize("bi", [True, False])
def test_odd_head_counts(gdn, bi):
    """3 q/k heads, 6 value heads, 3 sequences: 9 (sequence, q/k head) pairs, not
    a multiple of the 8 XCDs the workgroup mapping groups by."""
    w = W.build([100, 37, 64], 3, 6, torch.bfloat16, seed=12, name="odd_heads")
    check(gdn, w, BF16_TOL, bi)


def test_no_states(gdn):
    w = W.build([70, 5], 2, 4, torch.bfloat16, seed=10, state_in=None, state_out=None, name="nostate")
    check(gdn, w, BF16_TOL, True)


@pytest.mark.parametrize("gate", ["sigmoid", "long"])
def test_bf16_states_few_items(gdn, gate):
    """bf16 initial and final states on a launch with fewer work items than CUs
    (the pipelined scan), ragged lengths with an empty sequence; the empty one
    passes its bf16 state through bitwise."""
    w = W.build([200, 0, 64, 1, 333], 2, 4, torch.bfloat16, seed=12, gate=gate, state_in=torch.bfloat16,
                state_out=torch.bfloat16, name="bf16_states_small")
    check(gdn, w, BF16_TOL, True)
    _, fin = run_gpu(gdn, w, False)
    assert torch.equal(fin[1].cpu(), w.initial_state[1])


@pytest.mark.parametrize("many", [False, True])
def test_prenormalized_bf16_without_kernel_norm(gdn, many):
    """bf16 q/k normalised on the host, use_qk_l2norm off (row factors 1): a
    launch below one work item per CU (pipelined scan) and one above it
    (four-wave scan)."""
    if many:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        gen = torch.Generator().manual_seed(13)
        lens = torch.randint(1, 200, (cus // 4 + 5,), generator=gen).tolist()
    else:
        lens = [300, 17, 128]
    w = W.build(lens, 2, 4, torch.bfloat16, seed=14, gate="long", use_qk_l2norm=False, prenormalize=True,
                name="prenorm_bf16")
    check(gdn, w, BF16_TOL, True)


def test_all_empty_batch(gdn):
    w = W.build([0, 0, 0], 2, 4, torch.bfloat16, seed=11, name="all_empty")
    out, fin = run_gpu(gdn, w, True)
    assert out.shape[0] == 0
    assert torch.equal(fin.cpu(), w.initial_state)
