"""A sequence past the 2 GiB per-tensor reach of the direct-to-LDS kernels' 32-bit buffer
offsets (N = 2^23 + 100 tokens at D = 128 in bf16): the library routes it to the
register-staged kernels (64-bit offsets), which the per-launch profile confirms.  No oracle
runs at this size; the check is a property that holds at any length: the same sequence
split in two halves, each within the direct-to-LDS kernels' reach, joined through the
state arguments (the first half's final state is the second half's initial state; the
second half's initial-state gradient is the first half's final-state gradient), gives the
same O, final state, dQ, dK, dV and dL/dlam.  Inputs: N(0, 1)/sqrt(D) from a seeded torch
generator on the device (the host generator would take minutes at 4.3 G elements)."""
import math

import numpy as np
import pytest

import oracle
from helpers import BF16_BAR, got

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import causal_linear_attention_tiled_amd as la  # noqa: E402

D = 128


def test_sequence_past_32bit_offsets_matches_its_halves():
    N = (1 << 23) + 100
    N1 = 1 << 22
    assert N * D * 2 > (1 << 31) and N1 * D * 2 < (1 << 31) and (N - N1) * D * 2 < (1 << 31)
    print(f"[large] N={N} (halves {N1} + {N - N1}) D={D} bf16", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(2023)
    q, k, v, g = (torch.randn((1, 1, N, D), generator=gen, device="cuda").div_(math.sqrt(D)).to(torch.bfloat16)
                  for _ in range(4))
    lam = np.array([0.999], np.float32)
    half = lambda t, a, b: t[:, :, a:b].contiguous()

    la.la_prof_enable(True)
    o, s = la.la_fwd(q, k, v, lam, Bk=64)
    dq, dk, dv = la.la_bwd(q, k, v, g, lam, Bk=64)
    dl = la.la_dlam(q, k, v, g, lam, Bk=64)
    torch.cuda.synchronize()
    full_kernels = set(la.la_prof_collect())
    print(f"    full-length kernels: {sorted(full_kernels)}", flush=True)
    assert {"fwd_mfma", "dq_mfma", "dkdv_mfma"} <= full_kernels
    assert not any(name.endswith("_dma") for name in full_kernels)

    q1, k1, v1, g1 = (half(t, 0, N1) for t in (q, k, v, g))
    q2, k2, v2, g2 = (half(t, N1, N) for t in (q, k, v, g))
    del q, k, v, g
    o1, s1 = la.la_fwd(q1, k1, v1, lam, Bk=64)
    o2, s2 = la.la_fwd(q2, k2, v2, lam, Bk=64, kv_in=s1)
    dq2, dk2, dv2, ds1 = la.la_bwd(q2, k2, v2, g2, lam, Bk=64, kv_in=s1, want_dkv_in=True)
    dq1, dk1, dv1 = la.la_bwd(q1, k1, v1, g1, lam, Bk=64, dkv_out=ds1)
    dl1 = la.la_dlam(q1, k1, v1, g1, lam, Bk=64, dkv_out=ds1)
    dl2 = la.la_dlam(q2, k2, v2, g2, lam, Bk=64, kv_in=s1)
    torch.cuda.synchronize()
    half_kernels = set(la.la_prof_collect())
    la.la_prof_enable(False)
    assert {"fwd_dma", "dq_dma", "dkdv_dma", "dlam_dma"} <= half_kernels

    errs = {}
    for name, a, (b1, b2) in (("O", o, (o1, o2)), ("dQ", dq, (dq1, dq2)), ("dK", dk, (dk1, dk2)), ("dV", dv, (dv1, dv2))):
        errs[name] = max(oracle.rel_l2(got(a[:, :, :N1]), got(b1)), oracle.rel_l2(got(a[:, :, N1:]), got(b2)))
    errs["kv_out"] = oracle.rel_l2(got(s), got(s2))
    d_full, d_split = float(got(dl)[0]), float(got(dl1)[0] + got(dl2)[0])
    errs["dlam"] = abs(d_full - d_split) / abs(d_split)
    print("    " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()) + f"  dL/dlam {d_full:.6e} vs {d_split:.6e}",
          flush=True)
    for name, e in errs.items():
        assert np.isfinite(e) and e <= BF16_BAR, name
