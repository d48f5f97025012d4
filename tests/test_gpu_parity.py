"""GPU parity: the HIP scan against the CPU oracle on seeded workloads.

Tolerances (max normalised error over each tensor): 1e-4 for fp32 inputs,
2e-2 for bf16 inputs; out and final state are checked separately.
Full-size workloads are checked on sampled (sequence, head) items that the
oracle computes one by one, from the same device-resident run.
"""
import numpy as np
import pytest
import torch

import gdn_workloads as W
from _harness import BF16_TOL, F32_TOL, check, nerr, run_gpu, run_oracle, say

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


def _sampled(gdn, w, items, bi):
    say(f"[gpu] {w.name}: T={w.T} N={w.N} batch_invariant={bi} (sampled {items})")
    out, fin = run_gpu(gdn, w, bi)
    cu = w.cu_seqlens.cpu().to(torch.int64)
    worst = 0.0
    for n, heads in items:
        sub = W.slice_item(w, n, heads)
        ro, rf = run_oracle(sub)
        bos, eos = int(cu[n]), int(cu[n + 1])
        e1 = nerr(out[bos:eos][:, heads], ro)
        e2 = nerr(fin[n][heads], rf[0])
        say(f"      n={n} heads={heads}: out {e1:.3e} state {e2:.3e}")
        worst = max(worst, e1, e2)
    assert worst <= BF16_TOL


@pytest.mark.parametrize("bi", [True, False])
def test_long_single_sampled(gdn, bi):
    w = W.make(2, device="cuda")
    _sampled(gdn, w, [(0, [0, 1, 17, 31])], bi)


@pytest.mark.parametrize("bi", [True, False])
def test_large_batch_sampled(gdn, bi):
    w = W.make(4, device="cuda")
    _sampled(gdn, w, [(0, [0, 1]), (17, [12, 30]), (31, [31])], bi)


@pytest.mark.parametrize("lengths,label", [([8192] * 34, "four-wave"), ([34816] * 8, "pipelined")])
def test_offsets_beyond_2gib_sampled(gdn, lengths, label):
    """278,528 tokens: the v and out rows of the last sequences (Hv 32, bf16,
    8 KB per token) lie beyond 2^31 bytes from the buffer start, on both scan
    kernels (1088 work items, and 256 = one per CU)."""
    w = W.build(lengths, 16, 32, torch.bfloat16, seed=71, device="cuda", name=f"beyond_2gib_{label}")
    assert (w.T - 1) * w.Hv * 128 * 2 >= 2 ** 31
    last = len(lengths) - 1
    _sampled(gdn, w, [(last, [0, 31]), (last - 1, [15])], True)


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
