"""A CPU model of how the scan kernels keep the decay of the state lazily (no
GPU): the state is held as sigma * S~, a chunk multiplies sigma by its decay
gamma_L, and S~ absorbs sigma ("renormalises") when sigma gamma_L falls below
2^-40.  The model follows the chunk (UT / WY) algebra of the scan with those
scale factors, in fp64, and records the largest magnitude reaching each
bf16 / fp32 matrix operand.  It pins two things the GPU tests cannot see:

* the factors cancel: the model equals the token recurrence (the oracle) to
  rounding, in every regime (mild gates, a chunk log-decay below -60,
  renormalising chunks, a hard reset);
* on a renormalising chunk the output products stay in range even when raw
  q and k are huge and the in-kernel L2 norm rescales them: the output tile P
  is the plain masked q.k (no 1 / sigma' factor), and the state part of the
  output is carried as (Y sigma) gamma_L against a row factor divided by
  gamma_L.  The form used before (P scaled by 1 / sigma') overflows bf16 on
  the same inputs, which the last test shows.

The model is not the oracle and not the kernel: it shares no code with
either.  It restates the chunk algebra derived from the recurrence (the
method of "flashinfer.gdn_prefill", the chunked GDN scan; argument meanings of
"flashinfer.cudnn.cudnn_chunk_gated_delta_rule", Parameters).
"""
import numpy as np
import pytest

import oracle

C = 64
D = 128
RENORM = 2.0 ** -40
FAST_DECAY = -60.0
BF16_MAX = 3.3895e38


def kernel_model(q, k, v, g, b, scale, s0, l2, old_scheme=False):
    """One sequence, one head: q, k, v [T, D], g, b [T], s0 [D, D] (V-major).
    Returns (out [T, D], final state [D, D], largest magnitudes per operand)."""
    T = q.shape[0]
    St = s0.astype(np.float64).copy()       # S~ (V-major)
    sigma = 1.0
    out = np.zeros((T, D))
    mx = {}

    def note(name, x):
        mx[name] = max(mx.get(name, 0.0), float(np.max(np.abs(x))) if np.size(x) else 0.0)

    for t0 in range(0, T, C):
        L = min(C, T - t0)
        kc, qc, vc = k[t0:t0 + L], q[t0:t0 + L], v[t0:t0 + L]
        la = np.maximum(np.log(np.maximum(g[t0:t0 + L], 1e-300)), -80.0)
        G = np.cumsum(la)
        GL = G[-1]
        gam, gL = np.exp(G), np.exp(GL)
        rk = 1.0 / np.sqrt((kc * kc).sum(1) + 1e-6) if l2 else np.ones(L)
        rq = 1.0 / np.sqrt((qc * qc).sum(1) + 1e-6) if l2 else np.ones(L)
        bb = b[t0:t0 + L]
        sig_next = sigma * gL
        renorm = not (sig_next >= RENORM)
        fast = GL > FAST_DECAY and (not old_scheme or sig_next >= 2.0 ** -100)
        X = kc @ St.T                          # K S~^T  (raw K)
        Y = qc @ St.T                          # Q S~^T  (raw Q)
        note("X", X)
        note("Y", Y)
        KK = kc @ kc.T
        QK = qc @ kc.T
        E = np.exp(np.minimum(G[:, None] - G[None, :], 0.0))
        A = np.tril(bb[:, None] * rk[:, None] * rk[None, :] * KK * E, -1)
        Tp = np.linalg.inv(np.eye(L) + A) * bb[None, :]      # (I + A)^-1 diag(b)
        FZ = sigma * (gam * rk)
        Zp = vc - FZ[:, None] * X
        Vn = Tp @ Zp
        note("Z'", Zp)
        dec = np.exp(GL - G)
        FU = rk * dec if renorm else (rk * dec) / sig_next
        ub = FU[:, None] * Vn
        note("ub", ub)
        base_y = (scale * gam) * rq
        if fast:
            P = np.tril(QK)
            if renorm and old_scheme:
                P = P / sig_next
                FY = sigma * base_y
                O = FY[:, None] * (Y + P @ ub)
            elif renorm:
                FY = base_y * np.exp(-GL)
                Yp = (Y * sigma) * gL
                note("Y'", Yp)
                O = FY[:, None] * (Yp + P @ ub)
            else:
                FY = sigma * base_y
                O = FY[:, None] * (Y + P @ ub)
        else:
            P = np.tril(scale * rq[:, None] * rk[None, :] * QK * E)
            FY = sigma * base_y
            O = FY[:, None] * Y + P @ Vn
        note("P", P)
        out[t0:t0 + L] = O
        if renorm:
            St = St * sig_next
            sigma = 1.0
        else:
            sigma = sig_next
        St = St + ub.T @ kc                   # S~ += K^T ub  (V-major)
        note("S~", St)
    return out, sigma * St, mx


def _inputs(T, seed, qk_scale=1.0, gates=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, D)) * qk_scale
    k = rng.standard_normal((T, D)) * qk_scale
    v = rng.standard_normal((T, D))
    g = np.exp(-np.log1p(np.exp(rng.standard_normal(T))) * 0.1) if gates is None else gates
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    s0 = rng.standard_normal((D, D)) * 0.01
    return q, k, v, g, b, s0


def _extreme_gates(T, second=-59.0):
    """Chunk 0 leaves sigma just above 2^-40 (log-decay -27.5); chunk 1 decays
    by `second` (above the entry-wise exp limit of -60), so it renormalises
    with sigma gamma_L ~ 3e-38 (-59) or ~ 1.8e-30 (-41); later chunks mild."""
    c = np.arange(T) // C
    return np.where(c == 0, np.exp(-27.5 / C), np.where(c == 1, np.exp(second / C), 0.97))


def _oracle(q, k, v, g, b, s0, scale, l2):
    o, f = oracle.run(q[:, None], k[:, None], v[:, None], g[:, None], b[:, None], scale, [0, q.shape[0]],
                      s0[None, None], l2)
    return o[:, 0], f[0, 0]


def _err(a, r):
    return float(np.max(np.abs(a - r)) / np.max(np.abs(r)))


@pytest.mark.parametrize("case", ["mild", "strong", "extreme", "reset", "mixed"])
def test_model_equals_recurrence(case):
    T = 300
    gates = {"mild": None, "strong": np.full(T, 0.2), "extreme": _extreme_gates(T),
             "reset": np.where(np.arange(T) % 97 == 5, 0.0, 0.95),
             "mixed": np.where((np.arange(T) // C) % 2 == 1, 0.2, 0.93)}[case]
    q, k, v, g, b, s0 = _inputs(T, 5, gates=gates)
    scale = 1.0 / np.sqrt(D)
    o, f, _ = kernel_model(q, k, v, g, b, scale, s0, True)
    ro, rf = _oracle(q, k, v, g, b, s0, scale, True)
    assert _err(o, ro) < 1e-10 and _err(f, rf) < 1e-10


@pytest.mark.parametrize("second", [-59.0, -41.0])
@pytest.mark.parametrize("qk_scale", [1.0, 2.0 ** 10, 2.0 ** 14])
def test_renorm_chunk_operands_stay_in_range(qk_scale, second):
    """Raw q, k multiplied by a power of two with the in-kernel L2 norm: the
    result equals the recurrence on the same inputs and, up to the norm's
    epsilon, on the unscaled ones; no operand comes near the bf16 limit."""
    T = 64 * 3 + 5
    q, k, v, g, b, s0 = _inputs(T, 7, gates=_extreme_gates(T, second))
    scale = 1.0 / np.sqrt(D)
    o, f, mx = kernel_model(q * qk_scale, k * qk_scale, v, g, b, scale, s0, True)
    ro, rf = _oracle(q * qk_scale, k * qk_scale, v, g, b, s0, scale, True)
    assert _err(o, ro) < 1e-10 and _err(f, rf) < 1e-10
    uo, uf = _oracle(q, k, v, g, b, s0, scale, True)
    assert _err(o, uo) < 1e-7 and _err(f, uf) < 1e-7
    for name, m in mx.items():
        assert np.isfinite(m) and m < BF16_MAX * 2.0 ** -30, (name, m)


def test_previous_scheme_overflows_on_the_same_inputs():
    """P carrying 1 / sigma' on a renormalising chunk (taken while sigma' >=
    2^-100) exceeds the bf16 range for raw q, k scaled by 2^14 under the -41
    schedule: what the test above rules out for the present form."""
    T = 64 * 3 + 5
    q, k, v, g, b, s0 = _inputs(T, 7, gates=_extreme_gates(T, -41.0))
    s = 2.0 ** 14
    _, _, mx = kernel_model(q * s, k * s, v, g, b, 1.0 / np.sqrt(D), s0, True, old_scheme=True)
    assert mx["P"] > BF16_MAX
