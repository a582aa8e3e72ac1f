"""Oracle for causal linear attention with per-head decay (fp64, CPU).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package.  The GPU library never
imports or links it, and this package imports nothing from the library.

Two independent routes to the same function (Lightning Attention-2, Tiling
paragraph and mechanism field of the phantomic12 record; the glossary page
"Lightning Attention", features list, on the parallel and recurrent forms):

* F1, quadratic masked (parallel) form, ``quadratic.py``:
  O = ((Q K^T) * D) V with D[i, j] = lam^(i-j) for i >= j, else 0.
* F2, recurrent form, ``oracle.c``: S <- lam S + k_t v_t^T, o_t = q_t S.

Readings where the pages are silent: the formula and the decay lam come from
the workload definition, the feature map is the identity unless one of the
elementwise maps in ``feature.py`` is asked for, there is no normaliser,
position t attends to itself, lam is a float32 value promoted to double with
lam^0 = 1 (so lam = 0 keeps only the diagonal), an optional initial state S0
adds lam^(t+1) q_t S0, and the backward is that of L = <dO, O> + <G, S_N> for
an optional gradient G arriving at the final state, giving dQ, dK, dV, the
gradient of S0, and the derivative of the same loss with respect to lam
(``dlam_recurrent``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .quadratic import (decay_matrix, fwd_quadratic, bwd_quadratic, dlam_quadratic, dlam_magnitude)  # noqa: F401
from . import feature  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
# LA_SANITIZE=1 (tests/sanitize_host.py): the build with AddressSanitizer and UBSan
_SANITIZE = os.environ.get("LA_SANITIZE") == "1"
_SO = os.path.join(_HERE, "liboracle_san.so" if _SANITIZE else "liboracle.so")
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
_lib_handle = None


def build() -> str:
    """Compile liboracle.so with gcc (always recompiles).

    Portable x86-64 code (the library may be built on one host and run on another) and no
    contraction of a*b + c into fused multiply-adds, so every host rounds the fp64 sums the
    same way."""
    src = os.path.join(_HERE, "oracle.c")
    tmp = _SO + ".tmp"
    if _SANITIZE:  # clang, so that one sanitizer runtime serves every library in the process
        cmd = ["/opt/rocm/llvm/bin/clang", "-O1", *_SAN_FLAGS, "-ffp-contract=off", "-fPIC", "-shared",
               "-fopenmp", "-o", tmp, src]
    else:
        cmd = ["gcc", "-O3", "-ffp-contract=off", "-fPIC", "-shared", "-fopenmp", "-o", tmp, src]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        lib.oracle_fwd_recurrent.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, i64]
        lib.oracle_bwd_recurrent.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]
        lib.oracle_decode_step.argtypes = [vp, vp, vp, vp, i64, i64, vp, vp]
        lib.oracle_dlam_recurrent.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp, vp, vp]
        _lib_handle = lib
    return _lib_handle


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _lams(lam, pairs) -> np.ndarray:
    lam = np.asarray(lam, dtype=np.float64).reshape(-1)
    if lam.size == 1:
        lam = np.full(pairs, lam[0])
    assert lam.size == pairs
    return np.ascontiguousarray(lam)


def fwd_recurrent(q, k, v, lam, s_init=None, want_state=True, block=0, phi="identity"):
    """F2 forward over sequences shaped [..., n, d].

    lam: one value or one per sequence (the product of the leading dims).
    phi: the feature map applied to q and k (oracle.feature).
    Returns (O, S_final) and, if ``block`` > 0, also the states before every
    block start t = b*block, shaped [..., ceil(n/block), d, d].
    """
    q, k, v = feature.phi(q, phi), feature.phi(k, phi), _f64(v)
    *lead, n, d = q.shape
    pairs = int(np.prod(lead)) if lead else 1
    lam_arr = _lams(lam, pairs)
    s0 = None if s_init is None else _f64(s_init).reshape(pairs, d, d)
    o = np.empty_like(q)
    sf = np.empty((pairs, d, d)) if want_state else None
    nb = (n + block - 1) // block if block > 0 else 0
    sb = np.empty((pairs, nb, d, d)) if block > 0 else None
    _lib().oracle_fwd_recurrent(q.ctypes.data, k.ctypes.data, v.ctypes.data, pairs, n, d,
                                lam_arr.ctypes.data, _ptr(s0), o.ctypes.data, _ptr(sf), _ptr(sb),
                                block)
    out = [o, None if sf is None else sf.reshape(*lead, d, d)]
    if block > 0:
        out.append(sb.reshape(*lead, nb, d, d))
    return tuple(out)


def bwd_recurrent(q, k, v, dout, lam, s_init=None, want=("dq", "dk", "dv"), g_final=None,
                  want_ds_init=False, phi="identity"):
    """F2 backward of L = <dO, O> + <G, S_N> (G = ``g_final``, the gradient arriving at the
    final state; zero when None), with the feature map ``phi`` on q and k.

    Returns (dQ, dK, dV) (None for those not wanted), followed by dS0, the gradient of the
    initial state, when ``want_ds_init``.  dQ and dK are with respect to the raw q and k."""
    q_raw, k_raw = _f64(q), _f64(k)
    q, k, v, dout = feature.phi(q_raw, phi), feature.phi(k_raw, phi), _f64(v), _f64(dout)
    *lead, n, d = q.shape
    pairs = int(np.prod(lead)) if lead else 1
    lam_arr = _lams(lam, pairs)
    s0 = None if s_init is None else _f64(s_init).reshape(pairs, d, d)
    gf = None if g_final is None else _f64(g_final).reshape(pairs, d, d)
    dq = np.empty_like(q) if "dq" in want else None
    dk = np.empty_like(q) if "dk" in want else None
    dv = np.empty_like(q) if "dv" in want else None
    ds0 = np.empty((pairs, d, d)) if want_ds_init else None
    _lib().oracle_bwd_recurrent(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data, pairs,
                                n, d, lam_arr.ctypes.data, _ptr(s0), _ptr(gf), _ptr(dq), _ptr(dk),
                                _ptr(dv), _ptr(ds0))
    if phi != "identity":
        # chain rule through the elementwise feature map
        if dq is not None:
            dq *= feature.dphi(q_raw, phi)
        if dk is not None:
            dk *= feature.dphi(k_raw, phi)
    if want_ds_init:
        return dq, dk, dv, ds0.reshape(*lead, d, d)
    return dq, dk, dv


def dlam_recurrent(q, k, v, dout, lam, s_init=None, g_final=None, phi="identity"):
    """F2 derivative of L = <dO, O> + <G, S_N> with respect to the decay lam, one value per
    sequence (shape: the leading dims), by forward-mode differentiation of the recurrence
    (T = dS/dlam carried next to S; oracle.c).  The feature map ``phi`` on q and k does not
    depend on lam."""
    q, k, v, dout = feature.phi(q, phi), feature.phi(k, phi), _f64(v), _f64(dout)
    *lead, n, d = q.shape
    pairs = int(np.prod(lead)) if lead else 1
    lam_arr = _lams(lam, pairs)
    s0 = None if s_init is None else _f64(s_init).reshape(pairs, d, d)
    gf = None if g_final is None else _f64(g_final).reshape(pairs, d, d)
    out = np.empty(pairs)
    _lib().oracle_dlam_recurrent(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data, pairs,
                                 n, d, lam_arr.ctypes.data, _ptr(s0), _ptr(gf), out.ctypes.data)
    return out.reshape(lead) if lead else out[0]


def decode_step(state, q, k, v, lam, phi="identity"):
    """One recurrent step for states [..., d, d] (updated copy returned) and q, k, v [..., d],
    with the feature map ``phi`` on q and k.

    Returns (o, new_state)."""
    state = _f64(state).copy()
    q, k, v = feature.phi(q, phi), feature.phi(k, phi), _f64(v)
    *lead, d = q.shape
    pairs = int(np.prod(lead)) if lead else 1
    lam_arr = _lams(lam, pairs)
    o = np.empty_like(q)
    _lib().oracle_decode_step(state.ctypes.data, q.ctypes.data, k.ctypes.data, v.ctypes.data, pairs, d,
                              lam_arr.ctypes.data, o.ctypes.data)
    return o, state


def _norm2(x: np.ndarray) -> float:
    """Euclidean norm without underflow or overflow of the squares: scaled by the largest
    magnitude first (NaN propagates)."""
    x = np.abs(x.ravel())
    if x.size == 0:
        return 0.0
    m = float(np.max(x))
    if not np.isfinite(m) or m == 0.0:
        return m
    return m * float(np.sqrt(np.sum((x / m) ** 2)))


def rel_l2(y, ref) -> float:
    """||y - ref||_2 / ||ref||_2 in fp64 (0 when both are exactly zero; NaN anywhere gives NaN)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = _norm2(ref)
    num = _norm2(y - ref)
    if np.isnan(num) or np.isnan(den):
        return float("nan")
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den
