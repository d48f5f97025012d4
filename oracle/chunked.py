"""Naive chunked form of the gated delta rule, numpy fp64 (test infrastructure).

A second CPU form, independent of the HIP library, that applies the chunk
(UT / WY) algebra literally, with no tiling, fusion or reordering beyond what
the algebra states.  It exists to pin the algebra the GPU kernels use against
the token recurrence in ``gdn_oracle.c``; the pages name the chunked method
("flashinfer.gdn_prefill": chunk_gated_delta_rule is the chunked GDN scan)
without printing it, so the algebra below is derived from the recurrence.

Derivation (one chunk of L tokens, state S0 [V, K] on entry, a_i > 0):
  G_i = sum_{s<=i} ln a_s,  gamma_i = exp(G_i)                    (in-chunk)
  u_i := b_i (v_i - a_i S_{i-1} k_i)  so  S_i = a_i S_{i-1} + u_i k_i^T
  =>  S_i = gamma_i S0 + sum_{j<=i} exp(G_i - G_j) u_j k_j^T
  =>  u_i + sum_{j<i} A_ij u_j = b_i (v_i - gamma_i S0 k_i),
      A_ij = b_i (k_i . k_j) exp(G_i - G_j)   (j < i, strictly lower)
  =>  U_new = T (V - diag(gamma) K S0^T),     T = (I + A)^{-1} diag(b)
  O   = scale [ diag(gamma) Q S0^T + ((Q K^T) o D) U_new ],  D_ij = exp(G_i-G_j) [j<=i]
  S_L = gamma_L S0 + U_new^T diag(exp(G_L - G)) K

Segment composition: the state map is affine, S_end = S0 M + N, with
N = scan from S0 = 0, and M = the map of the scan with v = 0 started from
S0 = I (each row of S evolves on its own, so rows of the identity give M).

Inputs here are per (sequence, head) slices: q, k [L, K], v [L, V], g, beta [L].
"""
import numpy as np


def l2norm_rows(x, eps=1e-6):
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + eps)


def forward_substitution_inverse(A, beta):
    """T = (I + A)^{-1} diag(beta) for strictly lower A, row by row:
    T_i = beta_i e_i - sum_{j<i} A_ij T_j."""
    L = A.shape[0]
    T = np.zeros_like(A)
    for i in range(L):
        T[i, i] = beta[i]
        for j in range(i):
            T[i] -= A[i, j] * T[j]
    return T


def chunk_step(S0, q, k, v, g, beta, scale):
    """One chunk. Returns (O [L, V], S_L [V, K]) and the intermediates."""
    G = np.cumsum(np.log(g))
    gam = np.exp(G)
    Dm = np.exp(G[:, None] - G[None, :])
    L = q.shape[0]
    lower = np.tril(np.ones((L, L)), -1)
    A = beta[:, None] * (k @ k.T) * Dm * lower
    T = forward_substitution_inverse(A, beta)
    W = T @ (gam[:, None] * k)
    U = T @ v
    Vn = U - W @ S0.T
    P = (q @ k.T) * Dm * np.tril(np.ones((L, L)))
    O = scale * ((gam[:, None] * q) @ S0.T + P @ Vn)
    SL = gam[-1] * S0 + Vn.T @ (np.exp(G[-1] - G)[:, None] * k)
    return O, SL, dict(G=G, A=A, T=T, W=W, U=U, Vnew=Vn, P=P)


def scan(q, k, v, g=None, beta=None, S0=None, scale=0.0, C=64, l2norm=False):
    """Chunked scan of one sequence and one head, chunks aligned to its start."""
    L, K = k.shape
    V = v.shape[1]
    g = np.ones(L) if g is None else np.asarray(g, np.float64)
    beta = np.ones(L) if beta is None else np.asarray(beta, np.float64)
    scale = 1.0 / np.sqrt(K) if scale == 0.0 else scale
    if l2norm:
        q, k = l2norm_rows(q), l2norm_rows(k)
    S = np.zeros((V, K)) if S0 is None else np.array(S0, np.float64)
    O = np.zeros((L, V))
    for c0 in range(0, L, C):
        sl = slice(c0, min(L, c0 + C))
        O[sl], S, _ = chunk_step(S, q[sl], k[sl], v[sl], g[sl], beta[sl], scale)
    return O, S


def segment_maps(q, k, v, g=None, beta=None, C=64, l2norm=False):
    """(M [K, K], N [V, K]) with S_end = S0 @ M + N for this segment."""
    L, K = k.shape
    V = v.shape[1]
    _, N = scan(q, k, v, g, beta, np.zeros((V, K)), 1.0, C, l2norm)
    _, M = scan(q, k, np.zeros((L, K)), g, beta, np.eye(K), 1.0, C, l2norm)
    return M, N
