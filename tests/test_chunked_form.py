"""Pins the chunk (UT / WY) algebra, in its naive numpy form, to the token
recurrence (no GPU).  The GPU kernels use this algebra; these tests show the
algebra itself reproduces the recurrence at any chunk length and that the
segment maps compose."""
import numpy as np
import pytest
import scipy.linalg

import oracle
from oracle import chunked

D = 128


def _seq(seed, L, K=D, V=D, glo=0.85):
    r = np.random.default_rng(seed)
    return dict(q=r.standard_normal((L, K)), k=r.standard_normal((L, K)), v=r.standard_normal((L, V)),
                g=r.uniform(glo, 1.0, L), beta=r.uniform(0, 1, L), s0=r.standard_normal((V, K)) * 0.1)


def _nerr(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


@pytest.mark.parametrize("C", [1, 2, 16, 64, 128])
def test_chunked_equals_recurrence(C):
    s = _seq(1, 150)
    o_ref, f_ref = oracle.run(s["q"][:, None], s["k"][:, None], s["v"][:, None], s["g"][:, None],
                              s["beta"][:, None], 0.0, [0, 150], s["s0"][None, None], True)
    o, f = chunked.scan(s["q"], s["k"], s["v"], s["g"], s["beta"], s["s0"], 0.0, C, l2norm=True)
    assert _nerr(o, o_ref[:, 0]) < 1e-11
    assert _nerr(f, f_ref[0, 0]) < 1e-11


def test_forward_substitution_matches_library_solve():
    r = np.random.default_rng(2)
    L = 64
    k = chunked.l2norm_rows(r.standard_normal((L, D)))
    beta = r.uniform(0, 1, L)
    G = np.cumsum(np.log(r.uniform(0.9, 1.0, L)))
    A = beta[:, None] * (k @ k.T) * np.exp(G[:, None] - G[None, :]) * np.tril(np.ones((L, L)), -1)
    T = chunked.forward_substitution_inverse(A, beta)
    ref = scipy.linalg.solve_triangular(np.eye(L) + A, np.diag(beta), lower=True, unit_diagonal=True)
    assert _nerr(T, ref) < 1e-12


def test_segment_maps_compose():
    s = _seq(3, 200)
    cut = 130
    M, N = chunked.segment_maps(s["q"][cut:], s["k"][cut:], s["v"][cut:], s["g"][cut:],
                                s["beta"][cut:], C=64, l2norm=True)
    _, S_mid = chunked.scan(s["q"][:cut], s["k"][:cut], s["v"][:cut], s["g"][:cut], s["beta"][:cut],
                            s["s0"], 1.0, 64, l2norm=True)
    _, S_end = chunked.scan(s["q"], s["k"], s["v"], s["g"], s["beta"], s["s0"], 1.0, 64, l2norm=True)
    assert _nerr(S_mid @ M + N, S_end) < 1e-11


def test_chunk_size_one_intermediates_reduce_to_the_token_step():
    """At C = 1: A = 0, T = beta, W = beta*a*k, U = beta*v."""
    s = _seq(4, 1)
    _, _, it = chunked.chunk_step(s["s0"], s["q"], s["k"], s["v"], s["g"], s["beta"], 1.0)
    assert np.all(it["A"] == 0)
    assert np.isclose(it["T"][0, 0], s["beta"][0])
    assert np.allclose(it["W"][0], s["beta"][0] * s["g"][0] * s["k"][0], rtol=1e-14, atol=0)
    assert np.allclose(it["U"][0], s["beta"][0] * s["v"][0], rtol=1e-14, atol=0)
