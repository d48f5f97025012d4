"""Pins of the CPU oracle against what the mathematics fixes (no GPU).

Every pin is a function ``pin_*(run) -> (ok, detail)`` taking an oracle
``run`` callable, so the same pins check the real oracle (all must hold) and
each oracle with a planted mistake (at least one must fail).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

D = 128
HERE = os.path.dirname(os.path.abspath(__file__))


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _close(a, b, tol):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    ref = max(float(np.max(np.abs(b))) if np.size(b) else 0.0, 1e-30)
    return err / ref <= tol, f"max normalised error {err / ref:.3e} (tol {tol:g})"


# ---------------------------------------------------------------- pins ----

def pin_hand_example(run):
    """Two tokens, K = V = 2, derived by hand (tests/golden/hand_d2.json)."""
    ex = json.load(open(os.path.join(HERE, "golden", "hand_d2.json")))
    a = lambda key: np.array(ex[key], dtype=np.float64)
    q, k, v = a("q")[:, None, :], a("k")[:, None, :], a("v")[:, None, :]
    out, fin = run(q, k, v, a("g")[:, None], a("beta")[:, None], ex["scale"], [0, 2])
    ok1, d1 = _close(out[:, 0], a("out"), 1e-12)
    ok2, d2 = _close(fin[0, 0], a("final_state"), 1e-12)
    return ok1 and ok2, d1 + "; " + d2


def pin_beta_zero(run):
    """b = 0: S_T = (prod a) S0 and o_t = scale * gamma_t * S0 q_t."""
    r = _rng(1)
    T = 9
    q, k, v = r.standard_normal((T, 1, D)), r.standard_normal((T, 1, D)), r.standard_normal((T, 1, D))
    g = r.uniform(0.5, 1.0, (T, 1))
    s0 = r.standard_normal((1, 1, D, D))
    out, fin = run(q, k, v, g, np.zeros((T, 1)), 0.3, [0, T], s0)
    gam = np.cumprod(g[:, 0])
    exp_out = 0.3 * gam[:, None] * (s0[0, 0] @ q[:, 0].T).T
    ok1, d1 = _close(fin[0, 0], gam[-1] * s0[0, 0], 1e-13)
    ok2, d2 = _close(out[:, 0], exp_out, 1e-12)
    return ok1 and ok2, d1 + "; " + d2


def pin_single_token(run):
    """One token from a zero state: o = b scale (k.q) v and S = b v k^T
    (default scale 1/sqrt(128), in-kernel L2 norm on)."""
    r = _rng(2)
    q, k, v = r.standard_normal((1, 1, D)), r.standard_normal((1, 1, D)), r.standard_normal((1, 1, D))
    b = 0.37
    out, fin = run(q, k, v, np.array([[0.9]]), np.array([[b]]), 0.0, [0, 1], None, True)
    qn = q[0, 0] / np.sqrt((q[0, 0] ** 2).sum() + 1e-6)
    kn = k[0, 0] / np.sqrt((k[0, 0] ** 2).sum() + 1e-6)
    ok1, d1 = _close(out[0, 0], b * (1 / np.sqrt(D)) * (kn @ qn) * v[0, 0], 1e-12)
    ok2, d2 = _close(fin[0, 0], b * np.outer(v[0, 0], kn), 1e-12)
    return ok1 and ok2, d1 + "; " + d2


def pin_orthonormal_keys(run):
    """a = 1, b = 1, orthonormal keys: S_T k_i = v_i for every i, any S0."""
    r = _rng(3)
    T = 40
    Qm, _ = np.linalg.qr(r.standard_normal((D, T)))
    k = Qm.T[:, None, :]
    q, v = r.standard_normal((T, 1, D)), r.standard_normal((T, 1, D))
    s0 = r.standard_normal((1, 1, D, D))
    _, fin = run(q, k, v, None, None, 1.0, [0, T], s0)
    return _close((fin[0, 0] @ k[:, 0].T).T, v[:, 0], 1e-11)


def pin_alpha_zero_reset(run):
    """a_t = 0 erases the past: S_t = b_t v_t k_t^T."""
    r = _rng(4)
    T = 6
    q, k, v = r.standard_normal((T, 1, D)), _unit(r.standard_normal((T, 1, D))), r.standard_normal((T, 1, D))
    g = r.uniform(0.5, 1.0, (T, 1))
    g[-1] = 0.0
    b = r.uniform(0.1, 1.0, (T, 1))
    _, fin = run(q, k, v, g, b, 1.0, [0, T], r.standard_normal((1, 1, D, D)))
    return _close(fin[0, 0], b[-1, 0] * np.outer(v[-1, 0], k[-1, 0]), 1e-13)


def pin_literal_formula(run):
    """Brute force against S = a S (I - b k k^T) + b v k^T, o = scale S q,
    evaluated with explicit matrix products (tiny input, varlen, GVA)."""
    r = _rng(5)
    lens = [3, 0, 5]
    T, Hqk, Hv = sum(lens), 1, 2
    q, k = r.standard_normal((T, Hqk, D)), _unit(r.standard_normal((T, Hqk, D)))
    v = r.standard_normal((T, Hv, D))
    g, b = r.uniform(0.3, 1.0, (T, Hv)), r.uniform(0.0, 1.0, (T, Hv))
    s0 = r.standard_normal((3, Hv, D, D)) * 0.1
    cu = np.concatenate([[0], np.cumsum(lens)])
    out, fin = run(q, k, v, g, b, 0.25, cu, s0)
    eo, ef = np.zeros_like(out), np.zeros_like(fin)
    I = np.eye(D)
    for n in range(3):
        for h in range(Hv):
            S = s0[n, h].copy()
            for t in range(cu[n], cu[n + 1]):
                kk = k[t, h // 2]
                S = g[t, h] * S @ (I - b[t, h] * np.outer(kk, kk)) + b[t, h] * np.outer(v[t, h], kk)
                eo[t, h] = 0.25 * S @ q[t, h // 2]
            ef[n, h] = S
    ok1, d1 = _close(out, eo, 1e-12)
    ok2, d2 = _close(fin, ef, 1e-12)
    return ok1 and ok2, d1 + "; " + d2


def pin_l2norm(run):
    """In-kernel L2 norm == torch.nn.functional.normalize applied beforehand
    (up to the eps of the reading x / sqrt(sum x^2 + 1e-6))."""
    r = _rng(6)
    T = 7
    q, k, v = r.standard_normal((T, 1, D)) * 3, r.standard_normal((T, 1, D)) * 2, r.standard_normal((T, 1, D))
    g, b = r.uniform(0.8, 1.0, (T, 1)), r.uniform(0.0, 1.0, (T, 1))
    o1, f1 = run(q, k, v, g, b, 0.0, [0, T], None, True)
    qn = torch.nn.functional.normalize(torch.from_numpy(q), dim=-1).numpy()
    kn = torch.nn.functional.normalize(torch.from_numpy(k), dim=-1).numpy()
    o2, f2 = run(qn, kn, v, g, b, 0.0, [0, T], None, False)
    ok1, d1 = _close(o1, o2, 1e-6)
    ok2, d2 = _close(f1, f2, 1e-6)
    return ok1 and ok2, d1 + "; " + d2


def pin_api_defaults(run):
    """scale 0 == 1/sqrt(128); g None == ones; beta None == ones (bitwise)."""
    r = _rng(7)
    T = 5
    q, k, v = r.standard_normal((T, 1, D)), _unit(r.standard_normal((T, 1, D))), r.standard_normal((T, 1, D))
    o1, f1 = run(q, k, v, None, None, 0.0, [0, T])
    o2, f2 = run(q, k, v, np.ones((T, 1)), np.ones((T, 1)), 1 / np.sqrt(D), [0, T])
    same = np.array_equal(o1, o2) and np.array_equal(f1, f2)
    return same, "bitwise" if same else "differs"


def pin_gva(run):
    """Hqk = 2, Hv = 4 == the same with q, k repeat_interleave(2) (Hqk = 4)."""
    r = _rng(8)
    T = 6
    q, k = r.standard_normal((T, 2, D)), _unit(r.standard_normal((T, 2, D)))
    v = r.standard_normal((T, 4, D))
    g, b = r.uniform(0.8, 1.0, (T, 4)), r.uniform(0, 1, (T, 4))
    o1, f1 = run(q, k, v, g, b, 0.0, [0, T])
    o2, f2 = run(np.repeat(q, 2, 1), np.repeat(k, 2, 1), v, g, b, 0.0, [0, T])
    same = np.array_equal(o1, o2) and np.array_equal(f1, f2)
    return same, "bitwise" if same else "differs"


PINS = [pin_hand_example, pin_beta_zero, pin_single_token, pin_orthonormal_keys,
        pin_alpha_zero_reset, pin_literal_formula, pin_l2norm, pin_api_defaults, pin_gva]


def _runner(precision="f64", mutant=0):
    def run(q, k, v, g=None, beta=None, scale=0.0, cu=None, s0=None, l2=False):
        return oracle.run(q, k, v, g, beta, scale, np.asarray(cu), s0, l2, precision=precision,
                          nthreads=2, mutant=mutant)
    return run


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin_holds(pin):
    ok, detail = pin(_runner())
    assert ok, detail


MUTANTS = {1: "gate dropped", 2: "sign of delta", 3: "readout before update",
           4: "transposed readout", 5: "beta dropped", 6: "wrong head map",
           7: "default scale", 8: "q not normalised", 9: "predict before decay"}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: MUTANTS[m].replace(" ", "_"))
def test_planted_mistake_is_caught(mutant):
    run = _runner(mutant=mutant)
    failed = [p.__name__ for p in PINS if not p(run)[0]]
    assert failed, f"planted mistake '{MUTANTS[mutant]}' passed every pin"


# ------------------------------------------------------- invariants ----

def _batch(seed, lens, Hqk=2, Hv=4, K=D, V=D):
    r = _rng(seed)
    T = sum(lens)
    return dict(q=r.standard_normal((T, Hqk, K)), k=r.standard_normal((T, Hqk, K)),
                v=r.standard_normal((T, Hv, V)), g=r.uniform(0.9, 1.0, (T, Hv)),
                beta=r.uniform(0, 1, (T, Hv)), s0=r.standard_normal((len(lens), Hv, V, K)) * 0.1,
                cu=np.concatenate([[0], np.cumsum(lens)]).astype(np.int64))


def test_linearity_in_v_and_state():
    a, b = _batch(10, [20, 13]), _batch(11, [20, 13])
    run = lambda v, s0: oracle.run(a["q"], a["k"], v, a["g"], a["beta"], 0.0, a["cu"], s0, True)
    o1, f1 = run(a["v"], a["s0"])
    o2, f2 = run(b["v"], b["s0"])
    o3, f3 = run(a["v"] + 2.5 * b["v"], a["s0"] + 2.5 * b["s0"])
    assert _close(o3, o1 + 2.5 * o2, 1e-12)[0] and _close(f3, f1 + 2.5 * f2, 1e-12)[0]


def test_rows_of_state_are_independent():
    a = _batch(12, [17, 9])
    o, f = oracle.run(a["q"], a["k"], a["v"], a["g"], a["beta"], 0.0, a["cu"], a["s0"], True)
    sl = slice(40, 72)
    o2, f2 = oracle.run(a["q"], a["k"], a["v"][:, :, sl], a["g"], a["beta"], 0.0, a["cu"],
                        a["s0"][:, :, sl, :], True)
    assert np.array_equal(o[:, :, sl], o2) and np.array_equal(f[:, :, sl, :], f2)


def test_packing_is_invisible():
    lens = [11, 0, 29, 4]
    a = _batch(13, lens)
    o, f = oracle.run(a["q"], a["k"], a["v"], a["g"], a["beta"], 0.0, a["cu"], a["s0"], True)
    for n in range(len(lens)):
        s, e = a["cu"][n], a["cu"][n + 1]
        on, fn = oracle.run(a["q"][s:e], a["k"][s:e], a["v"][s:e], a["g"][s:e], a["beta"][s:e], 0.0,
                            [0, e - s], a["s0"][n:n + 1], True)
        assert np.array_equal(o[s:e], on) and np.array_equal(f[n:n + 1], fn)


def test_state_chaining_equals_whole():
    a = _batch(14, [50], Hqk=1, Hv=2)
    o, f = oracle.run(a["q"], a["k"], a["v"], a["g"], a["beta"], 0.0, a["cu"], a["s0"], True)
    cut = 23
    p = lambda x, s: x[s]
    o1, f1 = oracle.run(a["q"][:cut], a["k"][:cut], a["v"][:cut], a["g"][:cut], a["beta"][:cut], 0.0,
                        [0, cut], a["s0"], True)
    o2, f2 = oracle.run(a["q"][cut:], a["k"][cut:], a["v"][cut:], a["g"][cut:], a["beta"][cut:], 0.0,
                        [0, 50 - cut], f1, True)
    assert np.array_equal(o, np.concatenate([o1, o2])) and np.array_equal(f, f2)


def test_empty_sequence_passes_state_through():
    a = _batch(15, [0, 5, 0])
    _, f = oracle.run(a["q"], a["k"], a["v"], a["g"], a["beta"], 0.0, a["cu"], a["s0"], True)
    assert np.array_equal(f[0], a["s0"][0]) and np.array_equal(f[2], a["s0"][2])


def test_fp32_oracle_tracks_fp64():
    a = _batch(16, [300, 77])
    o64, f64 = oracle.run(a["q"], a["k"], a["v"], a["g"], a["beta"], 0.0, a["cu"], a["s0"], True)
    o32, f32 = oracle.run(a["q"], a["k"], a["v"], a["g"], a["beta"], 0.0, a["cu"], a["s0"], True,
                          precision="f32")
    assert _close(o32, o64, 2e-5)[0] and _close(f32, f64, 2e-5)[0]


def test_thread_count_does_not_change_results():
    a = _batch(17, [40, 33, 7])
    r1 = oracle.run(a["q"], a["k"], a["v"], a["g"], a["beta"], 0.0, a["cu"], a["s0"], True, nthreads=1)
    r8 = oracle.run(a["q"], a["k"], a["v"], a["g"], a["beta"], 0.0, a["cu"], a["s0"], True, nthreads=8)
    assert np.array_equal(r1[0], r8[0]) and np.array_equal(r1[1], r8[1])
