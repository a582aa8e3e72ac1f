"""Bit-exact bookkeeping probes driven through the output gradient dO: the dQ sweep (with
and without the forward's chunk states), the reverse dK/dV sweep with its chunked suffix,
the initial-state gradient, the decay derivative and the ragged-batch forward, on the
default, generic and alternative kernels, block sizes 64, 128 and 256, one chunk and
several, with aggregates over chunk parts.

The probes and their exact results are in tests/probes.py (Lightning Attention-2,
phantomic12 record, Tiling paragraph: the same tiling in forward and backward computes the
plain causal sum, so representable results must come out bit for bit).
"""
import numpy as np
import pytest

import synth
from helpers import got, to_dev
from probes import (D, build, build_varlen, dlam_final_gradient, expected_dlam,
                    expected_grads, expected_varlen, mismatch, probe_pairs, varlen_offsets)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import causal_linear_attention_tiled_amd as la  # noqa: E402

PROBES = 128  # sequences (heads) per call, one probe each


def _sync():
    torch.cuda.synchronize()


def assert_exact(name, y, ref, pairs=None):
    msg = mismatch(name, y, ref, pairs)
    assert msg is None, msg


@pytest.fixture
def env(monkeypatch):
    """Kernel selection: 'default', 'generic' (plain float32 kernels), 'v1' (register-staged
    matrix-core kernels), 'w4' (4-wave forward and reverse sweeps), 'w8' (8-wave forward),
    'dma128' (the 128-token-block forward-direction sweep for Bk = 128 and 256), 'dma2' (the
    chunk aggregates with every wave loading, two workgroups per CU)."""
    def set_(kernel="default", chunks=None, agg=None):
        vals = {"LA_KERNEL": "generic" if kernel == "generic" else None,
                "LA_FWD": "v1" if kernel == "v1" else None, "LA_REV": "v1" if kernel == "v1" else None,
                "LA_STATE": {"v1": "v1", "dma2": "dma2"}.get(kernel),
                "LA_FWD128": "1" if kernel == "dma128" else None,
                "LA_FWD_WAVES": {"w4": "4", "w8": "8"}.get(kernel),
                "LA_REV_WAVES": {"w4": "4", "w8": "8"}.get(kernel),
                "LA_CHUNKS": chunks, "LA_AGG_K": agg}
        for name, val in vals.items():
            if val is None:
                monkeypatch.delenv(name, raising=False)
            else:
                monkeypatch.setenv(name, str(val))
    return set_


def run_bwd_probe(Bk, lam_val, with_state, with_gf, use_fwd_ws, label, N=64 * 23 + 17):
    H = PROBES
    plan = la.la_plan(1, H, N, D, Bk, la.LA_BF16)
    pairs = probe_pairs(N, Bk, plan, lam_val, limit=H)
    print(f"[probe bwd] {label} Bk={Bk} lam={lam_val} kv_in={with_state} dkv_out={with_gf} "
          f"fwd_ws={use_fwd_ws} plan={plan} probes={H}", flush=True)
    q, k, v, g, s0, f = build(N, pairs, with_state, with_gf)
    qd, kd, vd, gd = (to_dev(synth.f32_to_bf16_bits(x), "bf16") for x in (q, k, v, g))
    kv_in = None if s0 is None else torch.from_numpy(s0).cuda()
    dkv_out = None if f is None else torch.from_numpy(f).cuda()
    lam = [lam_val] * H
    fws = None
    if use_fwd_ws:
        nb = la.la_fwd_workspace_bytes(1, H, N, D, Bk, la.LA_BF16)
        fws = torch.full((max(nb, 1),), 0xFF, dtype=torch.uint8, device="cuda")
        la.la_fwd(qd, kd, vd, lam, Bk=Bk, kv_in=kv_in, ws=fws)
    dq, dk, dv, ds0 = la.la_bwd(qd, kd, vd, gd, lam, Bk=Bk, kv_in=kv_in, dkv_out=dkv_out, fwd_ws=fws,
                                want_dkv_in=True)
    _sync()
    e_dq, e_dk, e_dv, e_ds0 = expected_grads(N, pairs, lam_val, with_state, with_gf)
    assert_exact("dQ", got(dq), e_dq, pairs)
    assert_exact("dK", got(dk), e_dk, pairs)
    assert_exact("dV", got(dv), e_dv, pairs)
    assert_exact("dS0", got(ds0), e_ds0, pairs)


# ------------------------------------------------------------------ la_bwd
@pytest.mark.parametrize("kern", ["default", "generic"])
@pytest.mark.parametrize("Bk,cks,agg", [(64, 1, None), (64, 4, None), (64, 3, 2), (64, 2, 4), (128, 3, None),
                                        (128, 2, 2), (256, 2, None), (256, 3, 1)])
@pytest.mark.parametrize("lam_val", [0.5, 1.0])
@pytest.mark.parametrize("use_fwd_ws", [False, True])
def test_bwd_impulse_bit_exact(env, kern, Bk, cks, agg, lam_val, use_fwd_ws):
    env(kernel=kern, chunks=cks, agg=agg)
    run_bwd_probe(Bk, lam_val, with_state=False, with_gf=False, use_fwd_ws=use_fwd_ws,
                  label=f"{kern} chunks={cks} agg={agg}")


@pytest.mark.parametrize("kern", ["default", "generic"])
@pytest.mark.parametrize("Bk,cks,agg", [(64, 3, 2), (128, 3, None), (256, 2, None)])
@pytest.mark.parametrize("lam_val", [0.5, 1.0])
@pytest.mark.parametrize("use_fwd_ws", [False, True])
def test_bwd_impulse_state_paths_bit_exact(env, kern, Bk, cks, agg, lam_val, use_fwd_ws):
    """The same probes with an initial state (its path into dQ and dS0) and a final-state
    gradient (its path into dK and dS0)."""
    env(kernel=kern, chunks=cks, agg=agg)
    run_bwd_probe(Bk, lam_val, with_state=True, with_gf=True, use_fwd_ws=use_fwd_ws,
                  label=f"{kern} chunks={cks} agg={agg}")


@pytest.mark.parametrize("kern", ["v1", "w4", "w8", "dma2"])
@pytest.mark.parametrize("lam_val", [0.5, 1.0])
def test_bwd_impulse_kernel_variants(env, kern, lam_val):
    """The register-staged kernels, the 4- and 8-wave sweeps and the chunk aggregates in the
    two-workgroup form (dma2), chunked with parts."""
    env(kernel=kern, chunks=3, agg=2)
    run_bwd_probe(64, lam_val, with_state=True, with_gf=True, use_fwd_ws=True, label=kern)


@pytest.mark.parametrize("Bk,cks,agg", [(128, 3, None), (128, 2, 2), (256, 2, None)])
@pytest.mark.parametrize("lam_val", [0.5, 1.0])
@pytest.mark.parametrize("use_fwd_ws", [False, True])
def test_bwd_impulse_block128_kernel(env, Bk, cks, agg, lam_val, use_fwd_ws):
    """The dQ sweep on the 128-token-block kernel (LA_FWD128=1), with and without the forward's
    chunk states (the forward then on that kernel too)."""
    env(kernel="dma128", chunks=cks, agg=agg)
    run_bwd_probe(Bk, lam_val, with_state=True, with_gf=True, use_fwd_ws=use_fwd_ws, label="dma128")


# 27 blocks in 3 chunks of 9 admit no 2 parts: the plan grows the chunks to 10 blocks (the
# last keeping 7), the aggregates taken over parts of 5
GROWN_N = 64 * 26 + 17
GROWN_PLAN = {"chunks": 3, "chunk_len": 640, "agg_parts": 2}


@pytest.mark.parametrize("kern", ["default", "generic"])
@pytest.mark.parametrize("lam_val", [0.5, 1.0])
@pytest.mark.parametrize("use_fwd_ws", [False, True])
def test_bwd_impulse_grown_chunks(env, kern, lam_val, use_fwd_ws):
    env(kernel=kern, chunks=3, agg=2)
    assert la.la_plan(1, PROBES, GROWN_N, D, 64, la.LA_BF16) == GROWN_PLAN
    run_bwd_probe(64, lam_val, with_state=True, with_gf=True, use_fwd_ws=use_fwd_ws,
                  label=f"{kern} grown chunks", N=GROWN_N)


# ------------------------------------------------------------------ la_dlam
def run_dlam_probe(Bk, lam_val, with_terms, label, N=64 * 23 + 17):
    """lam = 1/2 without S0 and F: dL/dlam = (i0-j0) 2^-(i0-j0-1) (0 for i0 = j0), one exact
    term.  lam = 1 with S0 = e_a e_c2^T and F = e0 e_c^T + e_a e_c2^T: the four terms
    (i0-j0) + (i0+1) + (N-1-j0) + N are integers, exact in float32."""
    H = PROBES
    plan = la.la_plan(1, H, N, D, Bk, la.LA_BF16)
    pairs = probe_pairs(N, Bk, plan, lam_val, limit=H)
    print(f"[probe dlam] {label} Bk={Bk} lam={lam_val} terms={with_terms} plan={plan} probes={H}", flush=True)
    q, k, v, g, s0, _ = build(N, pairs, with_terms, False)
    kv_in = dkv_out = None
    if with_terms:
        kv_in, dkv_out = torch.from_numpy(s0).cuda(), torch.from_numpy(dlam_final_gradient(H)).cuda()
    qd, kd, vd, gd = (to_dev(synth.f32_to_bf16_bits(x), "bf16") for x in (q, k, v, g))
    out = la.la_dlam(qd, kd, vd, gd, [lam_val] * H, Bk=Bk, kv_in=kv_in, dkv_out=dkv_out)
    _sync()
    exp = expected_dlam(N, pairs, lam_val, with_terms)
    y = got(out)
    bad = np.flatnonzero(y != exp)
    assert bad.size == 0, (f"dlam differs for {bad.size} probes; first (i0, j0) = {pairs[bad[0]]}: "
                           f"got {y[bad[0]]!r}, exact {exp[bad[0]]!r}")


@pytest.mark.parametrize("kern", ["default", "dma4", "v1", "generic"])
@pytest.mark.parametrize("Bk,cks,agg", [(64, 1, None), (64, 4, None), (64, 3, 2), (128, 3, None),
                                        (256, 2, None)])
@pytest.mark.parametrize("lam_val,with_terms", [(0.5, False), (1.0, True)])
def test_dlam_impulse_bit_exact(monkeypatch, kern, Bk, cks, agg, lam_val, with_terms):
    for name, val in (("LA_KERNEL", "generic" if kern == "generic" else None),
                      ("LA_DLAM", "v1" if kern == "v1" else None),
                      ("LA_DLAM_WAVES", "4" if kern == "dma4" else None),
                      ("LA_CHUNKS", cks), ("LA_AGG_K", agg)):
        if val is None:
            monkeypatch.delenv(name, raising=False)
        else:
            monkeypatch.setenv(name, str(val))
    run_dlam_probe(Bk, lam_val, with_terms, label=f"{kern} chunks={cks} agg={agg}")


@pytest.mark.parametrize("kern", ["default", "generic"])
@pytest.mark.parametrize("lam_val,with_terms", [(0.5, False), (1.0, True)])
def test_dlam_impulse_grown_chunks(monkeypatch, kern, lam_val, with_terms):
    for name, val in (("LA_KERNEL", "generic" if kern == "generic" else None), ("LA_DLAM", None),
                      ("LA_DLAM_WAVES", None), ("LA_CHUNKS", 3), ("LA_AGG_K", 2)):
        if val is None:
            monkeypatch.delenv(name, raising=False)
        else:
            monkeypatch.setenv(name, str(val))
    assert la.la_plan(1, PROBES, GROWN_N, D, 64, la.LA_BF16) == GROWN_PLAN
    run_dlam_probe(64, lam_val, with_terms, label=f"{kern} grown chunks", N=GROWN_N)


# ------------------------------------------------------------------ la_fwd_varlen
@pytest.mark.parametrize("L", [64, 128, 256])
@pytest.mark.parametrize("with_state", [False, True])
def test_varlen_impulse_bit_exact(monkeypatch, L, with_state):
    """Ragged forward: sequence boundaries on chunk boundaries (chunk length forced to L) and
    next to them, one-token sequences, every sequence with its own key impulse and, with an
    initial state, its own S0_b = e_(1+b) e_c2^T read by q = e0 + e_(1+b).  Head 0 decays
    by 1/2, head 1 not at all.  Nothing may cross a sequence boundary:
    O_t = lam^(t-j0) e_c [t >= j0] + lam^(t-start+1) e_c2 and
    S_N = lam^n S0_b + lam^(n-1-j0) e0 e_c^T, bit for bit."""
    monkeypatch.setenv("LA_VARLEN_L", str(L))
    offs = varlen_offsets(L)
    lam_vals = [0.5, 1.0]
    q, k, v, s0, j0s = build_varlen(offs, len(lam_vals), with_state)
    print(f"[probe varlen] L={L} kv_in={with_state} offsets={offs}", flush=True)
    qd, kd, vd = (to_dev(synth.f32_to_bf16_bits(x), "bf16") for x in (q, k, v))
    kv_in = torch.from_numpy(s0).cuda() if with_state else None
    o, s = la.la_fwd_varlen(qd, kd, vd, lam_vals, offs, Bk=64, kv_in=kv_in)
    _sync()
    e_o, e_s = expected_varlen(offs, lam_vals, j0s, with_state)
    assert_exact("O", got(o), e_o)
    assert_exact("kv_out", got(s), e_s)


@pytest.mark.parametrize("with_state", [False, True])
@pytest.mark.parametrize("Bk", [32, 64])
def test_varlen_impulse_generic_bit_exact(Bk, with_state):
    """The same ragged probes in float32 storage, which la_fwd_varlen serves on the generic
    kernels (one workgroup per sequence and head, no chunks): nothing crosses a sequence
    boundary, bit for bit."""
    offs = varlen_offsets(64)
    lam_vals = [0.5, 1.0]
    q, k, v, s0, j0s = build_varlen(offs, len(lam_vals), with_state)
    print(f"[probe varlen generic] Bk={Bk} kv_in={with_state} offsets={offs}", flush=True)
    qd, kd, vd = (to_dev(x.astype(np.float32), "f32") for x in (q, k, v))
    kv_in = torch.from_numpy(s0).cuda() if with_state else None
    o, s = la.la_fwd_varlen(qd, kd, vd, lam_vals, offs, Bk=Bk, kv_in=kv_in)
    _sync()
    e_o, e_s = expected_varlen(offs, lam_vals, j0s, with_state)
    assert_exact("O", got(o), e_o)
    assert_exact("kv_out", got(s), e_s)
