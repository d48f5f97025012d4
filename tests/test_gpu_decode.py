"""GPU parity of the single-token decode step (gdn_decode_step) against the
oracle: a batch of one-token sequences is exactly one recurrent step per
sequence, and K decode steps after a prefill must continue the same
recurrence over the prompt plus those K tokens ("flashinfer.gdn_prefill": the
prefill builds the state the decode loop then consumes)."""
import numpy as np
import pytest
import torch

import gdn_workloads as W
from _harness import BF16_TOL, F32_TOL, nerr, run_oracle, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _decode(gdn, w, state_in=True, state_out=True, in_place=False):
    """One decode step on device copies of the one-token workload w."""
    wd = w.to(DEV)
    out = torch.full((wd.T, wd.Hv, 128), float("nan"), dtype=wd.q.dtype, device=DEV)
    s_in = wd.initial_state if state_in else None
    if in_place:
        s_out = s_in
    elif state_out:
        s_out = torch.full((wd.N, wd.Hv, 128, 128), float("nan"), dtype=wd.state_dtype, device=DEV)
    else:
        s_out = None
    gdn.gdn_decode_step(wd.q, wd.k, wd.v, wd.g, wd.beta, wd.scale, s_in, s_out, wd.use_qk_l2norm, out)
    torch.cuda.synchronize()
    return out, s_out


def _check(gdn, w, tol, **kw):
    say(f"[gpu] decode {w.name}: N={w.N} Hqk={w.Hqk} Hv={w.Hv} dtype={w.q.dtype} "
        f"state {None if w.initial_state is None else w.initial_state.dtype} -> {w.state_dtype} {kw}")
    out, fin = _decode(gdn, w, **kw)
    ref_w = w if kw.get("state_in", True) else W.Workload(**{**w.__dict__, "initial_state": None})
    ref_out, ref_fin = run_oracle(ref_w)
    e_out = nerr(out, ref_out)
    say(f"      max normalised error: out {e_out:.3e}")
    assert np.isfinite(e_out) and e_out <= tol
    if fin is not None:
        e_fin = nerr(fin, ref_fin)
        say(f"      state {e_fin:.3e}")
        assert np.isfinite(e_fin) and e_fin <= tol


def _one_token(N, Hqk=16, Hv=32, dtype=torch.bfloat16, seed=7, **kw):
    return W.build([1] * N, Hqk, Hv, dtype, seed=seed, name=f"decode_{N}", **kw)


@pytest.mark.parametrize("N", [1, 3, 64])
def test_decode_bf16(gdn, N):
    _check(gdn, _one_token(N), BF16_TOL)


def test_decode_fp32(gdn):
    _check(gdn, _one_token(5, 2, 4, torch.float32, gate="uniform"), F32_TOL)


def test_decode_fp32_prenormalised(gdn):
    _check(gdn, _one_token(4, 2, 2, torch.float32, prenormalize=True, use_qk_l2norm=False), F32_TOL)


def test_decode_bf16_state(gdn):
    _check(gdn, _one_token(6, state_in=torch.bfloat16, state_out=torch.bfloat16), BF16_TOL)


def test_decode_mixed_state_dtypes(gdn):
    _check(gdn, _one_token(6, state_in=torch.bfloat16, state_out=torch.float32), BF16_TOL)


def test_decode_in_place(gdn):
    _check(gdn, _one_token(8), BF16_TOL, in_place=True)


def test_decode_zero_state_and_no_state_out(gdn):
    _check(gdn, _one_token(4), BF16_TOL, state_in=False)
    _check(gdn, _one_token(4), BF16_TOL, state_out=False)


def test_decode_no_gates_bf16_gates(gdn):
    _check(gdn, _one_token(4, with_g=False, with_beta=False), BF16_TOL)
    _check(gdn, _one_token(4, gate_dtype=torch.bfloat16), BF16_TOL)


@pytest.mark.parametrize("r", [1, 4])
def test_decode_head_ratios(gdn, r):
    _check(gdn, _one_token(3, 4, 4 * r), BF16_TOL)


def test_decode_empty_batch(gdn):
    w = _one_token(0)
    out, fin = _decode(gdn, w)
    assert out.numel() == 0 and fin.numel() == 0


def test_prefill_then_decode_steps(gdn):
    """Prompt of L_n tokens through the prefill, then K decode steps on the
    state it returns (in place): the decode outputs and the final state must
    match the oracle run over all L_n + K tokens."""
    prompt, K = [37, 64, 200, 1], 4
    full = W.build([L + K for L in prompt], 4, 8, torch.bfloat16, seed=21, gate="long", name="handoff")
    ref_out, ref_fin = run_oracle(full)
    cu = full.cu_seqlens.to(torch.int64).tolist()
    pre_idx = [t for n, L in enumerate(prompt) for t in range(cu[n], cu[n] + L)]
    pick = lambda t, idx: None if t is None else t[idx]
    pre = W.Workload("handoff_prompt", pick(full.q, pre_idx), pick(full.k, pre_idx), pick(full.v, pre_idx),
                     pick(full.g, pre_idx), pick(full.beta, pre_idx),
                     torch.tensor([0] + list(np.cumsum(prompt)), dtype=torch.int64), full.initial_state,
                     torch.float32, True)
    pd = pre.to(DEV)
    state = torch.empty(pd.N, pd.Hv, 128, 128, dtype=torch.float32, device=DEV)
    pout = torch.empty(pd.T, pd.Hv, 128, dtype=pd.q.dtype, device=DEV)
    gdn.gdn_chunk_prefill(pd.q, pd.k, pd.v, pd.g, pd.beta, 0.0, pd.cu_seqlens, pd.initial_state, state,
                          True, True, pout)
    e_pre = nerr(pout, ref_out[pre_idx])
    say(f"[gpu] handoff prompt out error {e_pre:.3e}")
    assert e_pre <= BF16_TOL
    for j in range(K):
        idx = [cu[n] + L + j for n, L in enumerate(prompt)]
        dev = lambda t: None if t is None else t[idx].to(DEV)
        out = torch.empty(len(idx), full.Hv, 128, dtype=full.q.dtype, device=DEV)
        gdn.gdn_decode_step(dev(full.q), dev(full.k), dev(full.v), dev(full.g), dev(full.beta), 0.0, state, state,
                            True, out)
        e = nerr(out, ref_out[idx])
        say(f"      decode step {j}: out error {e:.3e}")
        assert e <= BF16_TOL
    torch.cuda.synchronize()
    e_fin = nerr(state, ref_fin)
    say(f"      final state error {e_fin:.3e}")
    assert e_fin <= BF16_TOL


def test_decode_full_batch_in_place(gdn):
    """The benchmarked decode configuration (256 sequences, Hqk 16, Hv 32, fp32 state updated in place)."""
    _check(gdn, W.decode_batch(), BF16_TOL, in_place=True)
