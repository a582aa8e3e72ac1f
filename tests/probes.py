"""Impulse probes whose exact results are representable, for the bit-exact bookkeeping tests.

Lightning Attention-2 (phantomic12 record, Tiling paragraph) runs one block tiling in the
forward and in the backward pass and computes the plain causal sum, so wherever the exact
result is representable the kernels must return it bit for bit.

Each (batch, head) sequence holds one query / output-gradient impulse at token i0 and one
key / value impulse at token j0 <= i0:

    q_i0 = e0 (+ e_a),  dO_i0 = e_c (+ e_c2),  k_j0 = e0,  v_j0 = e_c,
    initial state S0 = e_a e_c2^T (optional),  final-state gradient F = e_a2 e_c^T (optional).

With L = <dO, O> + <F, S_N> the exact gradients are (0 in every other row)

    dQ_i0 = lam^(i0-j0) e0 + lam^(i0+1) e_a
    dK_j0 = lam^(i0-j0) (e0 + e_a) + lam^(N-1-j0) e_a2
    dV_j0 = lam^(i0-j0) (e_c + e_c2)
    dS0   = lam^(i0+1) (e0 + e_a)(e_c + e_c2)^T + lam^N F

(the e_a, e_c2 and e_a2 terms only when S0 / F are given), and dL/dlam is the derivative
of lam^(i0-j0) + lam^(i0+1) (+ <F, S_N>).  Every component holds one term, so at
lam = 1/2 it is an exact power of two and at lam = 1 exactly 1.  Terms below 2^-100 (long
distances at lam = 1/2, where float32 decay tables underflow on the way) are only required
to be at most 2^-100 in magnitude.

The expectations here are checked against the fp64 oracle on the CPU
(tests/test_probe_expectations.py); this module holds no kernel code and no oracle code.
"""
from __future__ import annotations

import numpy as np

D = 128
C_V, A_S, C2_V, A2_F = 5, 3, 9, 11     # component indices e_c, e_a, e_c2, e_a2
TINY = 2.0 ** -100


def boundaries(N, Bk, plan):
    """Block, chunk and aggregate-part boundaries of a plan ({chunks, chunk_len, agg_parts}),
    with their neighbours; 64 and 128 are the block halves some sweeps step."""
    L, parts = plan["chunk_len"], plan["agg_parts"]
    P = L // parts
    marks = {0, 1, 63, 64, 65, 127, 128, 129, Bk - 1, Bk, Bk + 1, N - 2, N - 1}
    for c in range(plan["chunks"]):
        for p in range(parts):
            b = c * L + p * P
            marks |= {b - 1, b, b + 1}
    return sorted(m for m in marks if 0 <= m < N)


def probe_pairs(N, Bk, plan, lam_val, limit):
    """Exactly `limit` (i0, j0) pairs: every boundary as i0, with j0 on the same and on
    earlier boundaries, one, two, 64 and 100 tokens back; at lam < 1 the distance stays
    <= 100, so every term is a power of two above 2^-100."""
    marks = boundaries(N, Bk, plan)
    pairs = set()
    for i0 in marks:
        cands = {i0, i0 - 1, i0 - 2, i0 - 64, i0 - 100} | {m for m in marks if m <= i0}
        for j0 in cands:
            if 0 <= j0 <= i0 and (lam_val == 1.0 or i0 - j0 <= 100):
                pairs.add((i0, j0))
    pairs = sorted(pairs)
    if len(pairs) > limit:  # a spread-out subset, first and last kept
        idx = np.unique(np.round(np.linspace(0, len(pairs) - 1, limit)).astype(int))
        pairs = [pairs[i] for i in idx]
    return [pairs[i % len(pairs)] for i in range(limit)]


def build(N, pairs, with_state, with_gf, d=D):
    """float32 q, k, v, dO [1, H, N, d] and S0, F [1, H, d, d] (None when not asked for)."""
    H = len(pairs)
    q = np.zeros((1, H, N, d), np.float32)
    k, v, g = np.zeros_like(q), np.zeros_like(q), np.zeros_like(q)
    for h, (i0, j0) in enumerate(pairs):
        q[0, h, i0, 0] = 1.0
        g[0, h, i0, C_V] = 1.0
        k[0, h, j0, 0] = 1.0
        v[0, h, j0, C_V] = 1.0
        if with_state:
            q[0, h, i0, A_S] = 1.0
            g[0, h, i0, C2_V] = 1.0
    s0 = f = None
    if with_state:
        s0 = np.zeros((1, H, d, d), np.float32)
        s0[0, :, A_S, C2_V] = 1.0
    if with_gf:
        f = np.zeros((1, H, d, d), np.float32)
        f[0, :, A2_F, C_V] = 1.0
    return q, k, v, g, s0, f


def expected_grads(N, pairs, lam_val, with_state, with_gf, d=D):
    """Exact dQ, dK, dV [1, H, N, d] and dS0 [1, H, d, d] of the probes from build()."""
    H = len(pairs)
    lam = np.float64(lam_val)
    dq, dk, dv = (np.zeros((1, H, N, d)) for _ in range(3))
    ds0 = np.zeros((1, H, d, d))
    for h, (i0, j0) in enumerate(pairs):
        w, wi = lam ** (i0 - j0), lam ** (i0 + 1)
        dq[0, h, i0, 0] = w
        dk[0, h, j0, 0] = w
        dv[0, h, j0, C_V] = w
        ds0[0, h, 0, C_V] = wi
        if with_state:
            dq[0, h, i0, A_S] = wi
            dk[0, h, j0, A_S] = w
            dv[0, h, j0, C2_V] = w
            ds0[0, h, 0, C2_V] = wi
            ds0[0, h, A_S, C_V] = wi
            ds0[0, h, A_S, C2_V] = wi
        if with_gf:
            dk[0, h, j0, A2_F] = lam ** (N - 1 - j0)
            ds0[0, h, A2_F, C_V] = lam ** N
    return dq, dk, dv, ds0


def dlam_final_gradient(H, d=D):
    """F = e0 e_c^T + e_a e_c2^T: reaches both the key impulse's and the initial state's
    contribution to S_N, so <F, S_N> = lam^(N-1-j0) + lam^N."""
    f = np.zeros((1, H, d, d), np.float32)
    f[0, :, 0, C_V] = 1.0
    f[0, :, A_S, C2_V] = 1.0
    return f


def expected_dlam(N, pairs, lam_val, with_terms):
    """Exact dL/dlam per probe.  Without S0 and F: (i0-j0) lam^(i0-j0-1) (0 for i0 = j0).
    With S0 = e_a e_c2^T and F from dlam_final_gradient(), add (i0+1) lam^i0 +
    (N-1-j0) lam^(N-2-j0) + N lam^(N-1)."""
    lam = np.float64(lam_val)
    out = []
    for i0, j0 in pairs:
        x = (i0 - j0) * lam ** (i0 - j0 - 1) if i0 > j0 else 0.0
        if with_terms:
            x += (i0 + 1) * lam ** i0 + (N - 1 - j0) * lam ** (N - 2 - j0) + N * lam ** (N - 1)
        out.append(x)
    return np.array(out)


def varlen_offsets(L):
    """Sequence boundaries on multiples of the chunk length L and next to them, with
    one-token sequences."""
    return sorted({0, L, L + 1, 2 * L - 1, 2 * L, 3 * L + 1, 3 * L + 2, 5 * L, 5 * L + 37, 7 * L - 1})


def build_varlen(offs, H, with_state, d=D):
    """Packed q, k, v [T, H, d]: sequence b has q = e0 (+ e_(1+b)) on every token and its key
    impulse k = e0, v = e_c at local position j0_b; S0_b = e_(1+b) e_c2^T.  Returns
    (q, k, v, s0 [B, H, d, d] or None, j0 list)."""
    B, T = len(offs) - 1, offs[-1]
    q = np.zeros((T, H, d), np.float32)
    k, v = np.zeros_like(q), np.zeros_like(q)
    s0 = np.zeros((B, H, d, d), np.float32) if with_state else None
    j0s = []
    for b in range(B):
        n = offs[b + 1] - offs[b]
        j0 = [0, n - 1, n // 2, max(0, n - 65), max(0, n - 2)][b % 5]
        j0s.append(j0)
        q[offs[b]:offs[b + 1], :, 0] = 1.0
        k[offs[b] + j0, :, 0] = 1.0
        v[offs[b] + j0, :, C_V] = 1.0
        if with_state:
            q[offs[b]:offs[b + 1], :, 1 + b] = 1.0
            s0[b, :, 1 + b, C2_V] = 1.0
    return q, k, v, s0, j0s


def expected_varlen(offs, lam_vals, j0s, with_state, d=D):
    """O_t = lam^(t-j0) e_c [t >= j0] + lam^(t-start+1) e_c2 and
    S_N = lam^n S0_b + lam^(n-1-j0) e0 e_c^T per sequence; nothing crosses a boundary."""
    B, T, H = len(offs) - 1, offs[-1], len(lam_vals)
    e_o = np.zeros((T, H, d))
    e_s = np.zeros((B, H, d, d))
    for b in range(B):
        n, j0 = offs[b + 1] - offs[b], j0s[b]
        tau = np.arange(n)
        rows = offs[b] + tau
        for h, lam in enumerate(np.asarray(lam_vals, dtype=np.float64)):
            e_o[rows[j0:], h, C_V] = lam ** (tau[j0:] - j0)
            e_s[b, h, 0, C_V] = lam ** (n - 1 - j0)
            if with_state:
                e_o[rows, h, C2_V] = lam ** (tau + 1)
                e_s[b, h, 1 + b, C2_V] = lam ** n
    return e_o, e_s


def mismatch(name, y, ref, pairs=None):
    """None when y is bit-exact where the exact value is 0 or at least 2^-100 and at most
    2^-100 in magnitude below that; else a message naming the first difference."""
    if not np.all(np.isfinite(y)):
        return f"{name}: non-finite values"
    exact = (ref == 0) | (np.abs(ref) >= TINY)
    bad = np.argwhere(exact & (y != ref))
    if bad.size:
        first = tuple(int(x) for x in bad[0])
        where = f" (probe i0, j0 = {pairs[first[1]]})" if pairs is not None and len(first) > 1 else ""
        return (f"{name}: {len(bad)} elements differ; first at {first}{where}: "
                f"got {y[first]!r}, exact {ref[first]!r}")
    if not np.all(np.abs(y[~exact]) <= TINY):
        return f"{name}: an underflowing term came out larger than 2^-100"
    return None
