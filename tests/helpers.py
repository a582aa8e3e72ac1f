"""Shared helpers for the GPU parity tests (input staging and comparison only)."""
from __future__ import annotations

import math

import numpy as np

import synth

BF16_BAR = 2e-2
F32_BAR = 1e-5


def torch_dev():
    import torch
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dtype: str):
    """Host array from synth (float32 or bf16 bit patterns) -> device tensor of that dtype."""
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(torch_dev())
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch_dev())


def host_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact value of a synth array as float64."""
    if dtype == "bf16":
        return synth.bf16_bits_to_f64(a)
    return np.asarray(a, dtype=np.float64)


def got(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def lam_pairs(lam: np.ndarray, B: int) -> np.ndarray:
    """Per-sequence decay for [B, H] sequences (sequence p = b*H + h uses lam[h])."""
    return np.tile(np.asarray(lam, dtype=np.float32).astype(np.float64), B)


def bar(dtype: str) -> float:
    return BF16_BAR if dtype == "bf16" else F32_BAR


def row_bar(dtype: str) -> float:
    """Bound on worst_row: five times the tensor bar.  Rounding spreads evenly over rows, so
    the worst of a sequence's rows stays within a few times its RMS error; a slip confined to
    one row of 10% or more of a typical row's size exceeds it."""
    return 5 * bar(dtype)


def inputs(seed, B, H, N, D, dtype, with_do=False):
    arrs = synth.qkv(seed, B, H, N, D, dtype, with_do=with_do)
    return arrs, [to_dev(a, dtype) for a in arrs], [host_f64(a, dtype) for a in arrs]


def state_input(seed, B, H, D):
    """A seeded float32 initial state [B, H, D, D] (entries N(0,1)/sqrt(D))."""
    return synth.normal(seed, synth.ID_STATE, (B, H, D, D), 1.0 / math.sqrt(D), "f32")


def rel_per_pair(y: np.ndarray, ref: np.ndarray) -> float:
    """Worst rel-L2 over the leading (sequence) index of [P, ...] arrays."""
    import oracle
    worst = 0.0
    for i in range(y.shape[0]):
        e = oracle.rel_l2(y[i], ref[i])
        if not e <= worst:  # NaN sticks
            worst = e
    return worst


def device_stream(seed, sid, shape, dtype, group_elems=1 << 27):
    """A [..] tensor of stream (seed, sid) generated slice by slice straight into device memory.

    Values are N(0,1)/sqrt(shape[-1]); host memory stays bounded by ``group_elems``."""
    import torch
    D = shape[-1]
    total = int(np.prod(shape))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = torch.empty(total, dtype=tdt, device=torch_dev())
    flat = out.view(torch.int16) if dtype == "bf16" else out
    step = max(D, (group_elems // D) * D)
    for s0 in range(0, total, step):
        n = min(step, total - s0)
        host = synth.normal(seed, sid, (n,), 1.0 / math.sqrt(D), dtype, start=s0)
        if dtype == "bf16":
            flat[s0:s0 + n].copy_(torch.from_numpy(host.view(np.int16)))
        else:
            flat[s0:s0 + n].copy_(torch.from_numpy(host))
    return out.view(*shape)


def sample_pairs(B, H, count):
    """A fixed, spread-out sample of (b, h) sequence indices (first and last always included)."""
    P = B * H
    idx = sorted({0, P - 1} | {int(round(i * (P - 1) / max(1, count - 1))) for i in range(count)})
    return [(p // H, p % H) for p in idx]


def worst_row(y: np.ndarray, ref: np.ndarray) -> float:
    """Worst token row of [P, N, D] arrays: max over (p, t) of ||y[p,t] - ref[p,t]|| divided by
    the RMS row norm of ref[p] (so a wrong row shows even where whole-tensor and
    whole-sequence rel-L2 average it away)."""
    y = np.asarray(y, dtype=np.float64).reshape(-1, *y.shape[-2:])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, *ref.shape[-2:])
    worst = 0.0
    for i in range(y.shape[0]):
        rms = np.sqrt(np.mean(np.sum(ref[i] ** 2, axis=-1)))
        rows = np.sqrt(np.sum((y[i] - ref[i]) ** 2, axis=-1))
        m = float(rows.max()) if rows.size else 0.0
        worst = max(worst, m / rms if rms > 0 else (0.0 if m == 0 else math.inf))
    return worst
