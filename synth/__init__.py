"""Seeded synthetic inputs shared by the GPU tests, the oracle checks and the bench.

The module holds no arithmetic of the attention method: it turns a seed, a
stream id and element indices into N(0, 1) * scale values (SplitMix64 counters
and Box-Muller, see ``synth.c``), rounds them to the storage type, and builds
the per-head decay table of the workloads.  Because every element depends only
on its flat index, one (batch, head) sequence can be regenerated on its own.

Stream ids used throughout: Q=1, K=2, V=3, dO=4, initial state=5, and for
recurrent decode step t the ids 16+3t (q), 17+3t (k), 18+3t (v).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# LA_SANITIZE=1 (tests/sanitize_host.py): the build with AddressSanitizer and UBSan
_SANITIZE = os.environ.get("LA_SANITIZE") == "1"
_SO = os.path.join(_HERE, "libsynth_san.so" if _SANITIZE else "libsynth.so")
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
_lib_handle = None

ID_Q, ID_K, ID_V, ID_DO, ID_STATE = 1, 2, 3, 4, 5


def decode_ids(step: int):
    """Stream ids (q, k, v) of recurrent decode step ``step``."""
    return 16 + 3 * step, 17 + 3 * step, 18 + 3 * step


def build() -> str:
    """Compile libsynth.so with gcc (always recompiles)."""
    src = os.path.join(_HERE, "synth.c")
    tmp = _SO + ".tmp"
    if _SANITIZE:  # clang, so that one sanitizer runtime serves every library in the process
        cmd = ["/opt/rocm/llvm/bin/clang", "-O1", *_SAN_FLAGS, "-ffp-contract=off", "-fPIC", "-shared",
               "-fopenmp", "-o", tmp, src, "-lm"]
    else:
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-fopenmp", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        u64, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int,
                                  ctypes.c_double, ctypes.c_void_p)
        lib.synth_normal.argtypes = [u64, u64, i64, i64, dbl, i32, vp]
        lib.synth_raw_u64.argtypes = [u64, u64, i64, i64, vp]
        lib.synth_splitmix64_sequence.argtypes = [u64, i64, vp]
        lib.synth_f32_to_bf16.argtypes = [vp, i64, vp]
        _lib_handle = lib
    return _lib_handle


_DT = {"f32": (0, np.float32), "bf16": (1, np.uint16), "f64": (2, np.float64)}


def normal(seed: int, sid: int, shape, scale: float, dtype: str = "f32", start: int = 0,
           out: np.ndarray | None = None) -> np.ndarray:
    """N(0,1)*scale draws for flat indices [start, start+prod(shape)) of stream (seed, sid).

    dtype "f32" gives float32, "bf16" gives uint16 bf16 bit patterns, "f64" gives the
    unrounded scaled doubles.  ``out`` (C-contiguous, matching dtype) is filled in place.
    """
    code, npdt = _DT[dtype]
    count = int(np.prod(shape)) if len(shape) else 1
    if out is None:
        out = np.empty(shape, dtype=npdt)
    assert out.dtype == npdt and out.flags["C_CONTIGUOUS"] and out.size == count
    _lib().synth_normal(seed, sid, start, count, float(scale), code, out.ctypes.data)
    return out


def raw_u64(seed: int, sid: int, start: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.uint64)
    _lib().synth_raw_u64(seed, sid, start, count, out.ctypes.data)
    return out


def splitmix64_sequence(seed: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.uint64)
    _lib().synth_splitmix64_sequence(seed, count, out.ctypes.data)
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _lib().synth_f32_to_bf16(x.ctypes.data, x.size, out.ctypes.data)
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns as float64."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def decay_schedule(num_heads: int) -> np.ndarray:
    """Per-head decay of the synthetic workloads, as float32.

    lambda_h = exp(-2^(-8 (h+1) / H)), evaluated in double and rounded to float.
    For H = 16 this is the schedule exp(-2^(-8(h+1)/16)) the workloads name; for
    other H the exponent keeps the same spread (lambda in about [0.40, 0.9961]).
    """
    return np.array([math.exp(-(2.0 ** (-8.0 * (h + 1) / num_heads))) for h in range(num_heads)],
                    dtype=np.float32)


def qkv(seed: int, B: int, H: int, N: int, D: int, dtype: str, with_do: bool = False):
    """Q, K, V (and dO) of shape [B, H, N, D], N(0,1)/sqrt(D), in the storage dtype."""
    scale = 1.0 / math.sqrt(D)
    ids = [ID_Q, ID_K, ID_V] + ([ID_DO] if with_do else [])
    return [normal(seed, i, (B, H, N, D), scale, dtype) for i in ids]


def pair_slice(seed: int, sid: int, B: int, H: int, N: int, D: int, b: int, h: int, dtype: str,
               t0: int = 0, t1: int | None = None) -> np.ndarray:
    """Tokens [t0, t1) of sequence (b, h) of a [B, H, N, D] stream, generated on its own."""
    t1 = N if t1 is None else t1
    start = ((b * H + h) * N + t0) * D
    return normal(seed, sid, (t1 - t0, D), 1.0 / math.sqrt(D), dtype, start=start)
