"""GPU parity on a seeded sweep of random shapes: sequence counts and ragged
lengths (empty ones included), head counts and GVA ratios, bf16 or fp32 q/k/v,
fp32, bf16 or absent states, the three gate recipes with fp32 or bf16 gates
and absent g or beta, in-kernel norm on or off, custom scales, both
batch_invariant modes.  Small batches take the prepared plan, larger ones the
pipelined or the four-wave scan, a middle band batches of 16-64 short
sequences on many heads (the four-wave scan with more workgroups than the GPU
holds at once), the last cases few long sequences (the split path where
batch_invariant is off), so the sweep runs every plan; each case
prints the plan it took and compares out and the final state element by
element with the fp64 oracle on the same inputs."""
import numpy as np
import pytest
import torch

import gdn_workloads as W
from _harness import BF16_TOL, F32_TOL, check, say

pytestmark = pytest.mark.gpu

SHORT, MID, LONG = 20, 8, 4


def random_case(seed):
    """The workload and batch_invariant flag of case `seed` (seeded numpy draws)."""
    rng = np.random.default_rng(7000 + seed)
    if seed < SHORT:
        N = int(rng.integers(1, 12))
        lengths = [int(x) for x in rng.integers(0, 700, size=N)]
        if rng.random() < 0.3:
            lengths[int(rng.integers(0, N))] = 0          # an empty sequence
        Hqk, r = int(rng.choice([1, 2, 4, 8])), int(rng.choice([1, 2, 4]))
        bi = bool(rng.random() < 0.5)
    elif seed < SHORT + MID:                              # many short sequences, many heads
        N = int(rng.integers(16, 65))
        lengths = [int(x) for x in rng.integers(0, 300, size=N)]
        Hqk, r = int(rng.choice([4, 8, 16])), int(rng.choice([2, 4]))
        bi = bool(rng.random() < 0.5)
    else:                                                 # few long sequences
        N = int(rng.integers(1, 3))
        lengths = [int(x) for x in rng.integers(4200, 9000, size=N)]
        Hqk, r = int(rng.choice([1, 2])), int(rng.choice([1, 2]))
        bi = seed % 2 == 1
    io = torch.float32 if rng.random() < 0.2 else torch.bfloat16
    dtypes = [None, torch.float32, torch.bfloat16]
    state_in, state_out = dtypes[int(rng.integers(0, 3))], dtypes[int(rng.integers(0, 3))]
    gate = str(rng.choice(["sigmoid", "uniform", "long"]))
    gate_dtype = torch.bfloat16 if (io == torch.bfloat16 and rng.random() < 0.3) else torch.float32
    with_g, with_beta = bool(rng.random() < 0.9), bool(rng.random() < 0.9)
    l2 = bool(rng.random() < 0.8)
    scale = 0.0 if rng.random() < 0.7 else float(rng.uniform(0.02, 0.2))
    w = W.build(lengths, Hqk, Hqk * r, io, seed=8000 + seed, gate=gate, gate_dtype=gate_dtype,
                state_in=state_in, state_out=state_out, use_qk_l2norm=l2, prenormalize=not l2,
                with_g=with_g, with_beta=with_beta, scale=scale, name=f"random{seed}")
    return w, bi


def tolerance(w):
    """fp32 bar only where nothing is rounded to bf16 (q/k/v and the final state)."""
    return F32_TOL if (w.q.dtype == torch.float32 and w.state_dtype != torch.bfloat16) else BF16_TOL


@pytest.mark.parametrize("seed", range(SHORT + MID + LONG))
def test_random_shapes(gdn, seed):
    w, bi = random_case(seed)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    kind, lseg = gdn.prefill_plan(w.N, w.T, w.Hv, w.q.dtype, False, bi, cus)
    say(f"random {seed}: lengths {w.lengths()} Hqk {w.Hqk} Hv {w.Hv} {str(w.q.dtype)[6:]} plan {kind}"
        + (f" (segments of {lseg})" if lseg else ""))
    check(gdn, w, tolerance(w), bi, label=f"random{seed} {kind}")
