"""Pins of the fp64 oracle against things other than itself (CPU only).

* exact rational brute force of the definition on tiny inputs, including exact
  gradients obtained from the forward definition by linearity;
* hand-worked examples (tests/golden/hand_examples.json);
* closed forms for constant inputs (forward, final state and backward);
* a library routine at lam = 1: ((Q K^T).tril()) V in torch float64;
* invariants: the two forms agree, split-and-continue, decode steps == forward;
* the derivative with respect to lam against the exact derivative of the loss,
  a polynomial in lam fixed by exact values at n + 1 points, against central
  differences and against torch float64 autograd;
* planted mistakes in a copy of the quadratic form are caught by these pins.

The definition is causal linear attention with per-head decay,
O_t = sum_{j<=t} lam^(t-j) (q_t . k_j) v_j, as reorganised by Lightning
Attention-2 (Tiling paragraph, mechanism field) and as in the recurrent and
parallel forms the glossary page "Lightning Attention" lists.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import quadratic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


# ----------------------------------------------------------------- exact brute force
def exact_forward(q, k, v, lam, s0=None):
    """Direct sums of the definition in exact rationals. Returns (O, S_final)."""
    n, d = len(q), len(q[0])
    lam = Fraction(lam)
    O = []
    for t in range(n):
        row = [Fraction(0)] * d
        for j in range(t + 1):
            w = lam ** (t - j) * sum(Fraction(q[t][a]) * Fraction(k[j][a]) for a in range(d))
            for c in range(d):
                row[c] += w * Fraction(v[j][c])
        if s0 is not None:
            for c in range(d):
                row[c] += lam ** (t + 1) * sum(Fraction(q[t][a]) * Fraction(s0[a][c]) for a in range(d))
        O.append(row)
    S = [[Fraction(0)] * d for _ in range(d)]
    for j in range(n):
        w = lam ** (n - 1 - j)
        for a in range(d):
            for c in range(d):
                S[a][c] += w * Fraction(k[j][a]) * Fraction(v[j][c])
    if s0 is not None:
        for a in range(d):
            for c in range(d):
                S[a][c] += lam ** n * Fraction(s0[a][c])
    return O, S


def exact_loss(q, k, v, g, lam, s0=None, gf=None):
    """L = <dO, O> + <G, S_final> from the exact forward (G = gf, the gradient arriving at
    the final state; absent when None)."""
    O, S = exact_forward(q, k, v, lam, s0)
    L = sum(O[t][c] * Fraction(g[t][c]) for t in range(len(O)) for c in range(len(O[0])))
    if gf is not None:
        L += sum(S[a][c] * Fraction(gf[a][c]) for a in range(len(S)) for c in range(len(S)))
    return L


def exact_grads(q, k, v, g, lam, s0=None, gf=None, want_ds0=False):
    """Exact dL/dQ, dL/dK, dL/dV (and dL/dS0) of L = <dO, O> + <G, S_final>.

    L is affine in each of Q, K, V and S0 separately, so each partial derivative is an
    exact difference of two loss evaluations of the forward definition."""
    n, d = len(q), len(q[0])
    zero = [[0] * d for _ in range(n)]

    def unit(t, a, rows=n):
        m = [[0] * d for _ in range(rows)]
        m[t][a] = 1
        return m

    base_q = exact_loss(zero, k, v, g, lam, s0, gf)
    base_k = exact_loss(q, zero, v, g, lam, s0, gf)
    base_v = exact_loss(q, k, zero, g, lam, s0, gf)
    dq = [[exact_loss(unit(t, a), k, v, g, lam, s0, gf) - base_q for a in range(d)] for t in range(n)]
    dk = [[exact_loss(q, unit(t, a), v, g, lam, s0, gf) - base_k for a in range(d)] for t in range(n)]
    dv = [[exact_loss(q, k, unit(t, a), g, lam, s0, gf) - base_v for a in range(d)] for t in range(n)]
    if not want_ds0:
        return dq, dk, dv
    zs = [[0] * d for _ in range(d)]
    base_s = exact_loss(q, k, v, g, lam, zs, gf)
    ds0 = [[exact_loss(q, k, v, g, lam, unit(a, c, d), gf) - base_s for c in range(d)] for a in range(d)]
    return dq, dk, dv, ds0


def as_f64(m):
    return np.array([[float(x) for x in row] for row in m], dtype=np.float64)


LAMS = [Fraction(0), Fraction(1, 2), Fraction(3, 4), Fraction(1)]


@pytest.mark.parametrize("lam", LAMS)
@pytest.mark.parametrize("n,d,seed,with_s0", [(1, 1, 0, False), (5, 2, 1, False), (9, 3, 2, True),
                                              (16, 4, 3, False), (12, 2, 4, True)])
def test_forward_matches_exact_rationals(lam, n, d, seed, with_s0):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.integers(-3, 4, size=(n, d)).tolist() for _ in range(3))
    s0 = rng.integers(-3, 4, size=(d, d)).tolist() if with_s0 else None
    O_ex, S_ex = exact_forward(q, k, v, lam, s0)
    O_ex, S_ex = as_f64(O_ex), as_f64(S_ex)
    lamf = float(lam)
    o2, s2 = oracle.fwd_recurrent(np.array(q), np.array(k), np.array(v), lamf,
                                  None if s0 is None else np.array(s0))
    # Small integers and dyadic lam keep every intermediate exact in binary64.
    assert np.array_equal(o2, O_ex)
    assert np.array_equal(s2, S_ex)
    o1, s1 = oracle.fwd_quadratic(q, k, v, lamf, s0)
    np.testing.assert_allclose(o1, O_ex, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(s1, S_ex, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("lam", LAMS)
@pytest.mark.parametrize("n,d,seed,with_s0", [(4, 2, 10, False), (7, 3, 11, True), (10, 2, 12, False)])
def test_backward_matches_exact_gradients(lam, n, d, seed, with_s0):
    rng = np.random.default_rng(seed)
    q, k, v, g = (rng.integers(-3, 4, size=(n, d)).tolist() for _ in range(4))
    s0 = rng.integers(-3, 4, size=(d, d)).tolist() if with_s0 else None
    dq_ex, dk_ex, dv_ex = (as_f64(m) for m in exact_grads(q, k, v, g, lam, s0))
    lamf = float(lam)
    s0a = None if s0 is None else np.array(s0)
    dq, dk, dv = oracle.bwd_recurrent(np.array(q), np.array(k), np.array(v), np.array(g), lamf, s0a)
    assert np.array_equal(dq, dq_ex)
    assert np.array_equal(dk, dk_ex)
    assert np.array_equal(dv, dv_ex)
    dq1, dk1, dv1, _ = oracle.bwd_quadratic(q, k, v, g, lamf, s0)
    for a, b in ((dq1, dq_ex), (dk1, dk_ex), (dv1, dv_ex)):
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("lam", LAMS)
@pytest.mark.parametrize("n,d,seed,with_s0", [(1, 2, 30, True), (5, 2, 31, False), (8, 3, 32, True)])
def test_state_gradients_match_exact(lam, n, d, seed, with_s0):
    """With a gradient G arriving at the final state: dK, dV and the initial-state gradient
    dS0 equal the exact partial derivatives of L = <dO, O> + <G, S_final>; G is not
    symmetric, so a transposed G fails."""
    rng = np.random.default_rng(seed)
    q, k, v, g = (rng.integers(-3, 4, size=(n, d)).tolist() for _ in range(4))
    gf = rng.integers(-3, 4, size=(d, d)).tolist()
    gf[0][d - 1] = 5 if gf[d - 1][0] != 5 else 4
    s0 = rng.integers(-3, 4, size=(d, d)).tolist() if with_s0 else None
    ex = [as_f64(m) for m in exact_grads(q, k, v, g, lam, s0, gf, want_ds0=True)]
    lamf = float(lam)
    s0a = None if s0 is None else np.array(s0, float)
    got = oracle.bwd_recurrent(np.array(q, float), np.array(k, float), np.array(v, float),
                               np.array(g, float), lamf, s0a, g_final=np.array(gf, float), want_ds_init=True)
    for a, b, name in zip(got, ex, ("dQ", "dK", "dV", "dS0")):
        np.testing.assert_array_equal(a, b, err_msg=name)
    got1 = oracle.bwd_quadratic(q, k, v, g, lamf, s0, g_final=gf)
    for a, b, name in zip(got1, ex, ("dQ", "dK", "dV", "dS0")):
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13, err_msg=name)


@pytest.mark.parametrize("lam", LAMS)
def test_decode_matches_exact_rationals(lam):
    rng = np.random.default_rng(7)
    n, d = 8, 3
    q, k, v = (rng.integers(-3, 4, size=(n, d)).tolist() for _ in range(3))
    O_ex, S_ex = exact_forward(q, k, v, lam)
    S = np.zeros((d, d))
    for t in range(n):
        o, S = oracle.decode_step(S, np.array(q[t], float), np.array(k[t], float), np.array(v[t], float),
                                  float(lam))
        assert np.array_equal(o, as_f64([O_ex[t]])[0])
    assert np.array_equal(S, as_f64(S_ex))


# ----------------------------------------------------------------- hand-worked golden values
def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("ex", _golden()["examples"], ids=lambda e: e["name"])
def test_hand_worked_examples(ex):
    q, k, v, g = (np.array(ex[key], dtype=np.float64) for key in ("q", "k", "v", "dO"))
    s0 = np.array(ex["S0"], dtype=np.float64) if "S0" in ex else None
    lam = ex["lam"]
    for o, s in (oracle.fwd_recurrent(q, k, v, lam, s0), oracle.fwd_quadratic(q, k, v, lam, s0)):
        np.testing.assert_allclose(o, ex["O"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(s, ex["S_final"], rtol=0, atol=1e-14)
    for grads in (oracle.bwd_recurrent(q, k, v, g, lam, s0), oracle.bwd_quadratic(q, k, v, g, lam, s0)):
        for got, key in zip(grads, ("dQ", "dK", "dV")):
            np.testing.assert_allclose(got, ex[key], rtol=0, atol=1e-14, err_msg=key)


@pytest.mark.parametrize("ex", _golden()["decode"], ids=lambda e: e["name"])
def test_hand_worked_decode(ex):
    o, s = oracle.decode_step(np.array(ex["S"], float), np.array(ex["q"], float),
                              np.array(ex["k"], float), np.array(ex["v"], float), ex["lam"])
    np.testing.assert_array_equal(o, ex["o"])
    np.testing.assert_array_equal(s, ex["S_new"])


# ----------------------------------------------------------------- closed forms
@pytest.mark.parametrize("lam", [1.0, 0.9375, 0.5, 0.0])
def test_closed_forms_all_ones(lam):
    n, d = 1000, 16
    ones = np.ones((n, d))
    t = np.arange(n, dtype=np.float64)
    if lam == 1.0:
        geo_t = t + 1                      # sum_{m=0}^{t} lam^m
        geo_rev = n - t                    # sum_{m=0}^{n-1-t} lam^m
        geo_n = float(n)
    else:
        geo_t = (1 - lam ** (t + 1)) / (1 - lam)
        geo_rev = (1 - lam ** (n - t)) / (1 - lam)
        geo_n = (1 - lam ** n) / (1 - lam)
    o_exp = d * geo_t[:, None] * ones
    s_exp = geo_n * np.ones((d, d))
    for o, s in (oracle.fwd_recurrent(ones, ones, ones, lam), oracle.fwd_quadratic(ones, ones, ones, lam)):
        np.testing.assert_allclose(o, o_exp, rtol=1e-12)
        np.testing.assert_allclose(s, s_exp, rtol=1e-12)
    dq_exp = d * geo_t[:, None] * ones
    dkv_exp = d * geo_rev[:, None] * ones
    for grads in (oracle.bwd_recurrent(ones, ones, ones, ones, lam),
                  oracle.bwd_quadratic(ones, ones, ones, ones, lam)):
        dq, dk, dv = grads[:3]
        np.testing.assert_allclose(dq, dq_exp, rtol=1e-12)
        np.testing.assert_allclose(dk, dkv_exp, rtol=1e-12)
        np.testing.assert_allclose(dv, dkv_exp, rtol=1e-12)
    # with G = 1 1^T arriving at the final state: dK_j, dV_j gain lam^(n-1-j) d, and
    # dS0 = (sum_t lam^(t+1)) 1 1^T + lam^n G
    ones_dd = np.ones((d, d))
    tail = lam ** (n - 1 - t) if lam != 0.0 else (t == n - 1).astype(np.float64)
    head = lam * geo_n
    ds0_exp = (head + lam ** n) * ones_dd
    for grads in (oracle.bwd_recurrent(ones, ones, ones, ones, lam, g_final=ones_dd, want_ds_init=True),
                  oracle.bwd_quadratic(ones, ones, ones, ones, lam, g_final=ones_dd)):
        np.testing.assert_allclose(grads[1], (dkv_exp + d * tail[:, None]), rtol=1e-12)
        np.testing.assert_allclose(grads[2], (dkv_exp + d * tail[:, None]), rtol=1e-12)
        np.testing.assert_allclose(grads[3], ds0_exp, rtol=1e-12)


def test_no_decay_is_one_based_i_d_v():
    """lam = 1 and all-ones q, k, v: the 1-based position i gives O_i = i * d * v."""
    n, d = 300, 8
    ones = np.ones((n, d))
    o, _ = oracle.fwd_recurrent(ones, ones, ones, 1.0)
    i = np.arange(1, n + 1, dtype=np.float64)
    np.testing.assert_array_equal(o, (i * d)[:, None] * ones)


def test_d1_n2_by_hand():
    q = np.array([[1.5], [-2.0]]); k = np.array([[3.0], [0.25]]); v = np.array([[2.0], [4.0]])
    lam = 0.75
    o, s = oracle.fwd_recurrent(q, k, v, lam)
    assert o[0, 0] == 1.5 * 3.0 * 2.0
    assert o[1, 0] == -2.0 * (lam * 3.0 * 2.0 + 0.25 * 4.0)
    assert s[0, 0] == lam * 6.0 + 1.0


# ----------------------------------------------------------------- library special case
def test_no_decay_equals_library_masked_product():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    n, d = 512, 32
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = (torch.matmul(tq, tk.T.contiguous()).tril() @ tv).numpy()
    o, s = oracle.fwd_recurrent(q, k, v, 1.0)
    np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(s, (tk.T.contiguous() @ tv).numpy(), rtol=1e-10, atol=1e-10)


# ----------------------------------------------------------------- invariants
@pytest.mark.parametrize("lam", [0.0, 0.5, 0.97, 1.0])
def test_two_forms_agree_random(lam):
    rng = np.random.default_rng(int(lam * 100) + 3)
    n, d = 700, 16
    q, k, v, g = (rng.standard_normal((n, d)) / 4 for _ in range(4))
    s0 = rng.standard_normal((d, d))
    o1, s1 = oracle.fwd_quadratic(q, k, v, lam, s0)
    o2, s2 = oracle.fwd_recurrent(q, k, v, lam, s0)
    assert oracle.rel_l2(o2, o1) < 1e-12 and oracle.rel_l2(s2, s1) < 1e-12
    for a, b in zip(oracle.bwd_recurrent(q, k, v, g, lam, s0), oracle.bwd_quadratic(q, k, v, g, lam, s0)):
        assert oracle.rel_l2(a, b) < 1e-12


def test_two_forms_agree_per_decay_head():
    import synth
    H, n, d = 16, 1024, 32
    lams = synth.decay_schedule(H).astype(np.float64)
    q, k, v = (synth.normal(0, i, (H, n, d), d ** -0.5, "f64") for i in (1, 2, 3))
    o2, s2 = oracle.fwd_recurrent(q, k, v, lams)
    for h in range(H):
        o1, s1 = oracle.fwd_quadratic(q[h], k[h], v[h], lams[h])
        assert oracle.rel_l2(o2[h], o1) < 1e-12
        assert oracle.rel_l2(s2[h], s1) < 1e-12


@pytest.mark.parametrize("m", [1, 63, 64, 65, 200])
def test_split_and_continue(m):
    rng = np.random.default_rng(m)
    n, d, lam = 257, 8, 0.9
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    o, s = oracle.fwd_recurrent(q, k, v, lam)
    oa, sa = oracle.fwd_recurrent(q[:m], k[:m], v[:m], lam)
    ob, sb = oracle.fwd_recurrent(q[m:], k[m:], v[m:], lam, sa)
    np.testing.assert_allclose(np.concatenate([oa, ob]), o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sb, s, rtol=1e-12, atol=1e-12)


def test_block_states_are_prefix_states():
    rng = np.random.default_rng(9)
    n, d, lam, bk = 200, 4, 0.8, 64
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    _, _, sb = oracle.fwd_recurrent(q, k, v, lam, block=bk)
    assert sb.shape == (4, d, d)
    assert np.all(sb[0] == 0)
    for b in range(1, 4):
        _, s = oracle.fwd_recurrent(q[:b * bk], k[:b * bk], v[:b * bk], lam)
        np.testing.assert_allclose(sb[b], s, rtol=1e-13, atol=1e-13)


def test_linear_in_v_and_q():
    rng = np.random.default_rng(11)
    n, d, lam = 100, 6, 0.7
    q, k, v, v2, q2 = (rng.standard_normal((n, d)) for _ in range(5))
    o_a, _ = oracle.fwd_recurrent(q, k, v, lam)
    o_b, _ = oracle.fwd_recurrent(q, k, v2, lam)
    o_ab, _ = oracle.fwd_recurrent(q, k, 2 * v - 3 * v2, lam)
    np.testing.assert_allclose(o_ab, 2 * o_a - 3 * o_b, rtol=1e-11, atol=1e-11)
    o_c, _ = oracle.fwd_recurrent(q2, k, v, lam)
    o_ac, _ = oracle.fwd_recurrent(q + q2, k, v, lam)
    np.testing.assert_allclose(o_ac, o_a + o_c, rtol=1e-11, atol=1e-11)


def test_state_gradient_adjoint_identity():
    """L = <dO, O> + <G, S_final> is affine in S0 and in K: L(X + dX) - L(X) = <dL/dX, dX>
    with L evaluated by the forward form only."""
    rng = np.random.default_rng(14)
    n, d, lam = 70, 5, 0.9
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    s0, gf, dS, = (rng.standard_normal((d, d)) for _ in range(3))
    dX = rng.standard_normal((n, d))

    def loss(kk, ss):
        o, sf = oracle.fwd_recurrent(q, kk, v, lam, ss)
        return np.sum(g * o) + np.sum(gf * sf)
    dq, dk, dv, ds0 = oracle.bwd_recurrent(q, k, v, g, lam, s0, g_final=gf, want_ds_init=True)
    base = loss(k, s0)
    lhs_s, lhs_k = loss(k, s0 + dS) - base, loss(k + dX, s0) - base
    assert abs(lhs_s - np.sum(ds0 * dS)) < 1e-10 * (1 + abs(lhs_s))
    assert abs(lhs_k - np.sum(dk * dX)) < 1e-10 * (1 + abs(lhs_k))


def test_adjoint_identity_random():
    """<dO, J dX> == <J^T dO, dX> for the exact linear maps X -> O (each of Q, K, V)."""
    rng = np.random.default_rng(13)
    n, d, lam = 64, 5, 0.85
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    dq, dk, dv = oracle.bwd_recurrent(q, k, v, g, lam)
    dX = rng.standard_normal((n, d))
    # O is linear in Q and in V, so J dX is O evaluated with dX in that slot.
    lhs_q = np.sum(g * oracle.fwd_recurrent(dX, k, v, lam)[0])
    lhs_v = np.sum(g * oracle.fwd_recurrent(q, k, dX, lam)[0])
    lhs_k = np.sum(g * oracle.fwd_recurrent(q, dX, v, lam)[0])
    assert abs(lhs_q - np.sum(dq * dX)) < 1e-10 * (1 + abs(lhs_q))
    assert abs(lhs_v - np.sum(dv * dX)) < 1e-10 * (1 + abs(lhs_v))
    assert abs(lhs_k - np.sum(dk * dX)) < 1e-10 * (1 + abs(lhs_k))


def test_decode_equals_forward_random():
    rng = np.random.default_rng(17)
    P, n, d = 6, 40, 8
    lams = np.linspace(0.3, 1.0, P)
    q, k, v = (rng.standard_normal((P, n, d)) for _ in range(3))
    o_ref, s_ref = oracle.fwd_recurrent(q, k, v, lams)
    S = np.zeros((P, d, d))
    for t in range(n):
        o, S = oracle.decode_step(S, q[:, t], k[:, t], v[:, t], lams)
        np.testing.assert_allclose(o, o_ref[:, t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, s_ref, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------- the pins catch planted mistakes
def _brute_force_fails(fwd):
    rng = np.random.default_rng(21)
    q, k, v = (rng.integers(-3, 4, size=(9, 3)).tolist() for _ in range(3))
    O_ex, _ = exact_forward(q, k, v, Fraction(1, 2))
    o, _ = fwd(q, k, v, 0.5)
    return not np.allclose(o, as_f64(O_ex), rtol=1e-12, atol=1e-12)


def test_planted_mistakes_are_caught(monkeypatch):
    orig = quadratic.decay_matrix
    assert not _brute_force_fails(quadratic.fwd_quadratic)
    # decay exponent off by one
    monkeypatch.setattr(quadratic, "decay_matrix", lambda n, lam: orig(n, lam) * lam)
    assert _brute_force_fails(quadratic.fwd_quadratic)
    # diagonal dropped (strictly causal)
    monkeypatch.setattr(quadratic, "decay_matrix", lambda n, lam: np.tril(orig(n, lam), -1))
    assert _brute_force_fails(quadratic.fwd_quadratic)
    # anti-causal mask (transposed decay matrix)
    monkeypatch.setattr(quadratic, "decay_matrix", lambda n, lam: orig(n, lam).T)
    assert _brute_force_fails(quadratic.fwd_quadratic)
    monkeypatch.setattr(quadratic, "decay_matrix", orig)

    # q and k swapped in the score (P = K Q^T): caught by the brute force
    def swapped(q, k, v, lam):
        q, k, v = (np.asarray(x, float) for x in (q, k, v))
        D = orig(len(q), lam)
        return ((k @ q.T) * D) @ v, None
    assert _brute_force_fails(swapped)


def test_planted_state_gradient_mistakes_are_caught():
    """Plausible slips in the final-state gradient terms fail the exact pin."""
    rng = np.random.default_rng(33)
    n, d, lam = 6, 3, Fraction(1, 2)
    q, k, v, g = (rng.integers(-3, 4, size=(n, d)).tolist() for _ in range(4))
    gf = rng.integers(-3, 4, size=(d, d)).tolist()
    gf[0][2], gf[2][0] = 3, -2
    s0 = rng.integers(-3, 4, size=(d, d)).tolist()
    _, dk_ex, _, ds0_ex = (as_f64(m) for m in exact_grads(q, k, v, g, lam, s0, gf, want_ds0=True))
    qa, ka, va, ga, fa, sa = (np.array(x, float) for x in (q, k, v, g, gf, s0))
    _, dk0, _, ds00 = oracle.bwd_quadratic(qa, ka, va, ga, 0.5, sa)   # no G term
    w_ok = 0.5 ** np.arange(n - 1, -1, -1)[:, None]
    assert np.allclose(dk0 + w_ok * (va @ fa.T), dk_ex, rtol=1e-13, atol=1e-13)
    assert not np.allclose(dk0 + 0.5 * w_ok * (va @ fa.T), dk_ex)       # exponent n - j
    assert not np.allclose(dk0 + w_ok * (va @ fa), dk_ex)               # G not transposed
    assert np.allclose(ds00 + 0.5 ** n * fa, ds0_ex, rtol=1e-13, atol=1e-13)
    assert not np.allclose(ds00 + fa, ds0_ex)                           # G without lam^n
    assert not np.allclose(ds00, ds0_ex)                                # G dropped


# ----------------------------------------------------------------- feature maps
@pytest.mark.parametrize("kind", ["elu1", "relu"])
def test_feature_maps_match_library(kind):
    """phi and phi' against torch's float64 elu / relu and autograd."""
    torch = pytest.importorskip("torch")
    from oracle import feature
    x = np.linspace(-6.0, 6.0, 2001)
    x = x[np.abs(x) > 1e-9]                                  # relu' is undefined at 0
    tx = torch.from_numpy(x).requires_grad_(True)
    ty = torch.nn.functional.elu(tx) + 1.0 if kind == "elu1" else torch.relu(tx)
    ty.sum().backward()
    # torch forms elu(x) + 1 as (exp(x) - 1) + 1: equal up to a few ulps of 1
    np.testing.assert_allclose(feature.phi(x, kind), ty.detach().numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(feature.dphi(x, kind), tx.grad.numpy(), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("kind", ["elu1", "relu"])
def test_feature_map_gradients_finite_differences(kind):
    """dQ, dK of L = <dO, O> + <G, S_final> through phi, against central differences of the
    forward (inputs kept away from the kink of relu)."""
    rng = np.random.default_rng(41)
    n, d, lam, h = 9, 3, 0.8, 1e-6
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    for x in (q, k):
        x[np.abs(x) < 0.1] += 0.3
    gf = rng.standard_normal((d, d))

    def loss(qq, kk):
        o, s = oracle.fwd_recurrent(qq, kk, v, lam, phi=kind)
        return np.sum(g * o) + np.sum(gf * s)
    dq, dk, _ = oracle.bwd_recurrent(q, k, v, g, lam, g_final=gf, phi=kind)
    fd_q, fd_k = np.zeros_like(q), np.zeros_like(k)
    for t in range(n):
        for a in range(d):
            e = np.zeros_like(q); e[t, a] = h
            fd_q[t, a] = (loss(q + e, k) - loss(q - e, k)) / (2 * h)
            fd_k[t, a] = (loss(q, k + e) - loss(q, k - e)) / (2 * h)
    np.testing.assert_allclose(dq, fd_q, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(dk, fd_k, rtol=1e-6, atol=1e-7)
    for a, b in zip(oracle.bwd_recurrent(q, k, v, g, lam, g_final=gf, phi=kind),
                    oracle.bwd_quadratic(q, k, v, g, lam, g_final=gf, phi=kind)):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_feature_map_closed_forms():
    """elu1 maps q = k = 0 to all ones (the all-ones closed form); relu maps q = -1 to zero, so
    O, dQ and dK vanish."""
    n, d, lam = 200, 8, 0.9
    zero, ones = np.zeros((n, d)), np.ones((n, d))
    t = np.arange(n, dtype=np.float64)
    o, _ = oracle.fwd_recurrent(zero, zero, ones, lam, phi="elu1")
    np.testing.assert_allclose(o, d * ((1 - lam ** (t + 1)) / (1 - lam))[:, None] * ones, rtol=1e-12)
    o, _ = oracle.fwd_recurrent(-ones, ones, ones, lam, phi="relu")
    assert not np.any(o)
    dq, dk, dv = oracle.bwd_recurrent(-ones, ones, ones, ones, lam, phi="relu")
    assert not np.any(dq) and not np.any(dk) and not np.any(dv)


# ----------------------------------------------------------------- derivative with respect to lam
def exact_dlam(q, k, v, g, lam0, s0=None, gf=None):
    """Exact dL/dlam at lam0 without any derivative formula: L(lam) is a polynomial of degree
    at most n in lam, so its values at lam = 0..n (exact rationals from the forward
    definition) fix it, and the derivative of that interpolating polynomial at lam0 is exact."""
    n = len(q)
    xs = [Fraction(i) for i in range(n + 1)]
    ys = [exact_loss(q, k, v, g, x, s0, gf) for x in xs]
    x0 = Fraction(lam0)
    total = Fraction(0)
    for i, xi in enumerate(xs):
        # derivative of the Lagrange basis polynomial l_i at x0
        dli = Fraction(0)
        for m, xm in enumerate(xs):
            if m == i:
                continue
            term = Fraction(1) / (xi - xm)
            for l_, xl in enumerate(xs):
                if l_ != i and l_ != m:
                    term *= (x0 - xl) / (xi - xl)
            dli += term
        total += ys[i] * dli
    return total


@pytest.mark.parametrize("lam", LAMS)
@pytest.mark.parametrize("n,d,seed,with_s0,with_g", [(1, 2, 40, True, True), (4, 2, 41, False, False),
                                                      (6, 3, 42, True, False), (7, 2, 43, True, True)])
def test_dlam_matches_exact_polynomial_derivative(lam, n, d, seed, with_s0, with_g):
    rng = np.random.default_rng(seed)
    q, k, v, g = (rng.integers(-3, 4, size=(n, d)).tolist() for _ in range(4))
    s0 = rng.integers(-3, 4, size=(d, d)).tolist() if with_s0 else None
    gf = rng.integers(-3, 4, size=(d, d)).tolist() if with_g else None
    ex = float(exact_dlam(q, k, v, g, lam, s0, gf))
    arr = lambda m: None if m is None else np.array(m, dtype=np.float64)
    args = (arr(q), arr(k), arr(v), arr(g), float(lam), arr(s0), arr(gf))
    for got in (oracle.dlam_recurrent(*args), oracle.dlam_quadratic(*args)):
        assert got == pytest.approx(ex, rel=1e-12, abs=1e-12)


@pytest.mark.parametrize("ex", _golden()["dlam"], ids=lambda e: e["name"])
def test_hand_worked_dlam(ex):
    q, k, v, g, s0, gf = (np.array(ex[key], dtype=np.float64) for key in ("q", "k", "v", "dO", "S0", "G"))
    for got in (oracle.dlam_recurrent(q, k, v, g, ex["lam"], s0, gf),
                oracle.dlam_quadratic(q, k, v, g, ex["lam"], s0, gf)):
        assert got == pytest.approx(ex["dL_dlam"], rel=0, abs=1e-14)


@pytest.mark.parametrize("lam", [0.3, 0.9, 0.99, 0.999])
def test_dlam_central_differences(lam):
    """The derivative against central differences of the quadratic-form loss (fp64)."""
    rng = np.random.default_rng(44)
    n, d = 300, 8
    q, k, v, g = (rng.standard_normal((n, d)) / np.sqrt(d) for _ in range(4))
    s0, gf = rng.standard_normal((d, d)), rng.standard_normal((d, d))

    def loss(x):
        o, s = quadratic.fwd_quadratic(q, k, v, x, s0)
        return float(np.sum(o * g) + np.sum(s * gf))

    h = 1e-5 * (1 - lam)
    fd = (loss(lam + h) - loss(lam - h)) / (2 * h)
    got = oracle.dlam_recurrent(q, k, v, g, lam, s0, gf)
    assert got == pytest.approx(fd, rel=1e-6)


def test_dlam_torch_autograd():
    """The derivative against torch float64 autograd of the parallel-form loss, one value per
    sequence with per-head decays, with a feature map on q and k."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(45)
    B, H, n, d = 2, 3, 97, 6
    q, k, v, g = (rng.standard_normal((B, H, n, d)) for _ in range(4))
    lams = np.array([0.5, 0.9, 0.995])
    got = oracle.dlam_recurrent(q, k, v, g, np.tile(lams, B), phi="elu1")
    lam_t = torch.tensor(lams, dtype=torch.float64, requires_grad=True)
    qt, kt = (torch.nn.functional.elu(torch.from_numpy(x)) + 1 for x in (q, k))
    vt, gt = torch.from_numpy(v), torch.from_numpy(g)
    i = torch.arange(n)[:, None]
    j = torch.arange(n)[None, :]
    e = (i - j).clamp(min=0).to(torch.float64)
    per = []
    for h in range(H):
        D = torch.where(i >= j, lam_t[h] ** e, torch.zeros((), dtype=torch.float64))
        o = ((qt[:, h] @ kt[:, h].transpose(-1, -2).contiguous()) * D) @ vt[:, h]
        per.append((o * gt[:, h]).sum(dim=(-1, -2)))
    ref = []
    for b in range(B):
        for h in range(H):
            (gl,) = torch.autograd.grad(per[h][b], lam_t, retain_graph=True)
            ref.append(gl[h].item())
    np.testing.assert_allclose(got.reshape(-1), ref, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("n", [1, 2, 5, 64])
def test_dlam_closed_form_all_ones(n):
    """lam = 1, all-ones q, k, v, dO, S0, G (d = 3): every pair (t, j <= t) contributes
    (t - j) d^2, S0 contributes (t + 1) d^2 per t, and G contributes n d^2 + sum_j (n-1-j) d^2:
    dL/dlam = d^2 ((n-1) n (n+1) / 6 + n^2 + n)."""
    d = 3
    ones = np.ones((n, d))
    s1 = np.ones((d, d))
    want = d * d * ((n - 1) * n * (n + 1) / 6 + n * n + n)
    for got in (oracle.dlam_recurrent(ones, ones, ones, ones, 1.0, s1, s1),
                oracle.dlam_quadratic(ones, ones, ones, ones, 1.0, s1, s1)):
        assert got == pytest.approx(want, rel=1e-14)


def test_dlam_at_zero_decay_is_the_first_order_term():
    """At lam = 0 only terms linear in lam survive: each token with its predecessor, the
    initial state's first step, and the final state's last-but-one token."""
    rng = np.random.default_rng(46)
    n, d = 9, 4
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    s0, gf = rng.standard_normal((d, d)), rng.standard_normal((d, d))
    want = sum((q[t] @ k[t - 1]) * (g[t] @ v[t - 1]) for t in range(1, n))
    want += q[0] @ s0 @ g[0] + np.sum(gf * np.outer(k[n - 2], v[n - 2]))
    assert oracle.dlam_recurrent(q, k, v, g, 0.0, s0, gf) == pytest.approx(want, rel=1e-13)


def test_dlam_log_derivative_identity():
    """lam dL/dlam = sum_t t <dO_t, O_t> - sum_j j <v_j, dV_j> + (n-1) <G, S_n> + <S0, dS0>: the
    exponent t - j of every term split into its query and key positions (S0 at position -1,
    G at position n-1), evaluated from the pinned forward and backward."""
    rng = np.random.default_rng(47)
    n, d, lam = 200, 5, 0.97
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    s0, gf = rng.standard_normal((d, d)), rng.standard_normal((d, d))
    o, sn = oracle.fwd_recurrent(q, k, v, lam, s0)
    _, _, dv, ds0 = oracle.bwd_recurrent(q, k, v, g, lam, s0, want=("dv",), g_final=gf, want_ds_init=True)
    t = np.arange(n)[:, None]
    rhs = np.sum(t * o * g) - np.sum(t * v * dv) + (n - 1) * np.sum(gf * sn) + np.sum(s0 * ds0)
    assert lam * oracle.dlam_recurrent(q, k, v, g, lam, s0, gf) == pytest.approx(rhs, rel=1e-10)


def test_planted_dlam_mistakes_are_caught(monkeypatch):
    """Plausible slips in the derivative fail the exact pin: the derivative weights of the
    powers off by one, and the state-derivative recurrence fed the updated state."""
    rng = np.random.default_rng(48)
    n, d, lam = 5, 2, Fraction(1, 2)
    q, k, v, g = (rng.integers(-3, 4, size=(n, d)).tolist() for _ in range(4))
    s0, gf = (rng.integers(-3, 4, size=(d, d)).tolist() for _ in range(2))
    ex = float(exact_dlam(q, k, v, g, lam, s0, gf))
    qa, ka, va, ga, sa, fa = (np.array(x, float) for x in (q, k, v, g, s0, gf))
    ok = quadratic.dlam_quadratic(qa, ka, va, ga, 0.5, sa, fa)
    assert ok == pytest.approx(ex, rel=1e-13)
    orig = quadratic._dpowers
    for wrong in (lambda l, e: e * np.power(l, e.astype(float)),            # e lam^e
                  lambda l, e: (e + 1) * np.power(l, e.astype(float)),      # (e+1) lam^e
                  lambda l, e: orig(l, e + 1)):                             # exponent shifted
        monkeypatch.setattr(quadratic, "_dpowers", wrong)
        assert quadratic.dlam_quadratic(qa, ka, va, ga, 0.5, sa, fa) != pytest.approx(ex, rel=1e-6)
    monkeypatch.setattr(quadratic, "_dpowers", orig)

    def recurrent(use_updated_state=False, drop_g=False, s_for_t=False):
        S, T, tot = sa.copy(), np.zeros((d, d)), 0.0
        for t in range(n):
            S_new = 0.5 * S + np.outer(ka[t], va[t])
            T = (S_new if use_updated_state else S) + 0.5 * T
            S = S_new
            tot += qa[t] @ T @ ga[t]
        if not drop_g:
            tot += np.sum(fa * (S if s_for_t else T))
        return tot
    assert recurrent() == pytest.approx(ex, rel=1e-13)
    for kw in ({"use_updated_state": True}, {"drop_g": True}, {"s_for_t": True}):
        assert recurrent(**kw) != pytest.approx(ex, rel=1e-6), kw


@pytest.mark.parametrize("lam", [0.0, 0.5, 0.9, 1.0])
@pytest.mark.parametrize("phi", ["identity", "elu1"])
def test_dlam_magnitude_is_the_derivative_when_no_term_cancels(lam, phi):
    """The magnitude scale of dL/dlam (the sum of its terms' absolute values) equals the
    recurrent oracle's dL/dlam itself when every input is nonnegative, so that no term can
    cancel another; on signed inputs it bounds |dL/dlam| from above."""
    rng = np.random.default_rng(49)
    n, d = 40, 6
    q, k, v, g = (rng.uniform(0.0, 1.0, (n, d)) for _ in range(4))
    s0, gf = rng.uniform(0.0, 1.0, (d, d)), rng.uniform(0.0, 1.0, (d, d))
    for s_init, g_final in ((None, None), (s0, None), (None, gf), (s0, gf)):
        mag = oracle.dlam_magnitude(q, k, v, g, lam, s_init, g_final, phi=phi)
        assert mag == pytest.approx(oracle.dlam_recurrent(q, k, v, g, lam, s_init, g_final, phi=phi), rel=1e-12)
    qs, ks, vs, gs = (rng.standard_normal((n, d)) for _ in range(4))
    signed = oracle.dlam_recurrent(qs, ks, vs, gs, lam, s0 - 0.5, gf - 0.5, phi=phi)
    assert abs(signed) <= oracle.dlam_magnitude(qs, ks, vs, gs, lam, s0 - 0.5, gf - 0.5, phi=phi) * (1 + 1e-12)


# ------------------------------------------------------------------ the error measure itself
def test_rel_l2_known_values():
    """rel-L2 = ||y - ref|| / ||ref||, with ref in the denominator: values fixed by hand."""
    assert abs(oracle.rel_l2([1.0, 0.0], [1.0, 1.0]) - 1.0 / np.sqrt(2.0)) < 1e-15
    x = np.array([3.0, -4.0])
    assert oracle.rel_l2(2 * x, x) == 1.0          # ||x|| / ||x||
    assert oracle.rel_l2(x, 2 * x) == 0.5          # ||x|| / ||2x||: the reference is the second argument
    assert oracle.rel_l2(x, x) == 0.0
    assert oracle.rel_l2(np.zeros(3), np.zeros(3)) == 0.0
    assert oracle.rel_l2([1e-300, 0.0], [0.0, 0.0]) == float("inf")
    assert oracle.rel_l2([[1.0, 2.0], [2.0, 0.0]], [[1.0, 2.0], [2.0, 4.0]]) == 4.0 / 5.0   # all elements


def test_rel_l2_sees_a_planted_difference():
    rng = np.random.default_rng(7)
    ref = rng.standard_normal((3, 50, 8))
    y = ref.copy()
    y[1, 17, 5] += 0.25
    assert abs(oracle.rel_l2(y, ref) - 0.25 / np.linalg.norm(ref)) < 1e-15
    assert not oracle.rel_l2(ref * (1 + 3e-2), ref) <= 2e-2   # a 3% scale error fails the bf16 bar
    y[0, 0, 0] = np.nan
    assert not oracle.rel_l2(y, ref) <= 2e-2                  # NaN never passes a bar


def test_rel_per_pair_is_the_worst_sequence():
    from helpers import rel_per_pair, worst_row
    ref = np.ones((3, 4, 2))
    y = ref.copy()
    y[2, 1, 0] = 3.0                   # sequence 2: ||diff|| = 2 over ||ref|| = sqrt(8)
    assert abs(rel_per_pair(y, ref) - 2.0 / np.sqrt(8.0)) < 1e-15
    assert abs(oracle.rel_l2(y, ref) - 2.0 / np.sqrt(24.0)) < 1e-15
    # worst row: ||diff of row|| over the sequence's RMS row norm (sqrt(2) here)
    assert abs(worst_row(y, ref) - 2.0 / np.sqrt(2.0)) < 1e-15
    assert rel_per_pair(ref, ref) == 0.0 and worst_row(ref, ref) == 0.0


def test_dlam_magnitude_signed_hand_example():
    """n = 2, d = 1, lam = 1/2 with mixed signs.  The terms of dL/dlam, by hand:
    g1 q1 k0 v0 = 18, g0 q0 s0 = -3, 2 lam g1 q1 s0 = 9, f k0 v0 = -1.5, 2 lam f s0 = -0.75,
    so dL/dlam = 21.75 and the sum of their magnitudes 32.25 (a dropped abs() or term shows)."""
    q = np.array([[1.0], [-2.0]])
    k = np.array([[3.0], [-1.0]])
    v = np.array([[-1.0], [2.0]])
    g = np.array([[2.0], [3.0]])
    s0 = np.array([[-1.5]])
    f = np.array([[0.5]])
    assert oracle.dlam_magnitude(q, k, v, g, 0.5, s0, f) == 32.25
    assert oracle.dlam_quadratic(q, k, v, g, 0.5, s0, f) == 21.75
    assert float(oracle.dlam_recurrent(q, k, v, g, 0.5, s0, f)) == 21.75


def test_rel_l2_has_no_underflow_or_overflow():
    """Squares of 1e-300 underflow and of 1e300 overflow in fp64; the measure must not."""
    assert abs(oracle.rel_l2([2e-300, 0.0], [1e-300, 0.0]) - 1.0) < 1e-15
    assert abs(oracle.rel_l2([2e300, 0.0], [1e300, 0.0]) - 1.0) < 1e-15
    assert abs(oracle.rel_l2([1e-300, 1.0], [0.0, 1.0]) - 1e-300) < 1e-315
