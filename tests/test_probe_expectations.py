"""The exact results the bit-exact GPU probes expect (tests/probes.py) equal the fp64
oracle's on the same probe inputs, and the comparison flags a one-ulp or one-token slip.

CPU only.  The oracle is pinned elsewhere against exact rational arithmetic; this pins the
probes' closed forms to it, so a probe cannot expect a wrong value of its own making."""
import numpy as np
import pytest

import oracle
import probes

N, d = 203, 16


def small_pairs(lam_val, limit=24):
    plan = {"chunks": 3, "chunk_len": 64, "agg_parts": 2}
    return probes.probe_pairs(N, 32, plan, lam_val, limit)


@pytest.mark.parametrize("lam_val", [0.5, 1.0])
@pytest.mark.parametrize("with_state,with_gf", [(False, False), (True, True), (True, False), (False, True)])
def test_grad_expectations_equal_oracle(lam_val, with_state, with_gf):
    pairs = small_pairs(lam_val)
    q, k, v, g, s0, f = probes.build(N, pairs, with_state, with_gf, d=d)
    H = len(pairs)
    dq, dk, dv, ds0 = oracle.bwd_recurrent(q, k, v, g, np.full(H, lam_val), s_init=s0, g_final=f,
                                           want_ds_init=True)
    e = probes.expected_grads(N, pairs, lam_val, with_state, with_gf, d=d)
    for name, y, ref in zip(("dQ", "dK", "dV", "dS0"), (dq, dk, dv, ds0), e):
        np.testing.assert_array_equal(y, ref, err_msg=name)
        assert probes.mismatch(name, y, ref, pairs) is None


@pytest.mark.parametrize("lam_val,with_terms", [(0.5, False), (1.0, True), (1.0, False)])
def test_dlam_expectations_equal_oracle(lam_val, with_terms):
    pairs = small_pairs(lam_val)
    q, k, v, g, s0, _ = probes.build(N, pairs, with_terms, False, d=d)
    H = len(pairs)
    f = probes.dlam_final_gradient(H, d=d) if with_terms else None
    y = oracle.dlam_recurrent(q, k, v, g, np.full(H, lam_val), s_init=s0, g_final=f).reshape(-1)
    np.testing.assert_array_equal(y, probes.expected_dlam(N, pairs, lam_val, with_terms))


@pytest.mark.parametrize("with_state", [False, True])
def test_varlen_expectations_equal_oracle(with_state):
    L = 32
    offs = probes.varlen_offsets(L)
    lam_vals = [0.5, 1.0]
    q, k, v, s0, j0s = probes.build_varlen(offs, 2, with_state, d=d)
    e_o, e_s = probes.expected_varlen(offs, lam_vals, j0s, with_state, d=d)
    for b in range(len(offs) - 1):
        a, z = offs[b], offs[b + 1]
        for h in range(2):
            o, s = oracle.fwd_recurrent(q[a:z, h], k[a:z, h], v[a:z, h], lam_vals[h],
                                        None if s0 is None else s0[b, h])
            np.testing.assert_array_equal(o, e_o[a:z, h])
            np.testing.assert_array_equal(s, e_s[b, h])


def test_mismatch_flags_slips():
    pairs = small_pairs(0.5)
    e = probes.expected_grads(N, pairs, 0.5, True, True, d=d)[0]
    assert probes.mismatch("x", e.copy(), e) is None
    one_ulp = e.copy()
    i = np.argwhere(e != 0)[0]
    one_ulp[tuple(i)] = np.nextafter(e[tuple(i)], 2.0)
    assert probes.mismatch("x", one_ulp, e) is not None
    # a key impulse one token late (an index slip in the bookkeeping)
    late = [(i0, min(j0 + 1, i0)) if j0 < i0 else (i0, j0) for i0, j0 in pairs]
    assert probes.mismatch("x", probes.expected_grads(N, late, 0.5, True, True, d=d)[0], e) is not None
    nan = e.copy()
    nan[0, 0, 0, 0] = np.nan
    assert probes.mismatch("x", nan, e) is not None
    # below 2^-100 only the magnitude bound applies
    tiny_ref = np.array([2.0 ** -120, 0.0, 1.0])
    assert probes.mismatch("x", np.array([0.0, 0.0, 1.0]), tiny_ref) is None
    assert probes.mismatch("x", np.array([2.0 ** -99, 0.0, 1.0]), tiny_ref) is not None


def test_probe_pairs_cover_boundaries():
    plan = {"chunks": 4, "chunk_len": 384, "agg_parts": 2}
    pairs = probes.probe_pairs(1489, 64, plan, 0.5, 128)
    assert len(pairs) == 128
    assert all(0 <= j0 <= i0 and i0 - j0 <= 100 for i0, j0 in pairs)
    i_set = {i0 for i0, _ in pairs}
    assert {383, 384, 385, 767, 768}.issubset(i_set | {p[1] for p in pairs})
