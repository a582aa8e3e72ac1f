"""The fused feature maps (elu + 1, relu on queries and keys) through every path:
the direct-to-LDS kernels (map applied to the tiles in LDS), the generic kernels,
the shapes the register-staged kernels would take (routed to the generic ones),
decode and the ragged prefill; against the oracle with the same map."""
import math

import numpy as np
import pytest

import oracle
import synth
from helpers import BF16_BAR, bar, got, host_f64, inputs, lam_pairs, state_input, to_dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import causal_linear_attention_tiled_amd as la  # noqa: E402


@pytest.fixture
def env(monkeypatch):
    def set_(kernel=None, chunks=None):
        for name, val in (("LA_KERNEL", kernel), ("LA_CHUNKS", chunks)):
            if val is None:
                monkeypatch.delenv(name, raising=False)
            else:
                monkeypatch.setenv(name, str(val))
    return set_


def run_case(B, H, N, D, Bk, dtype, phi, seed, with_state, with_gf, use_fwd_ws, label):
    print(f"[phi] {label} phi={phi} B={B} H={H} N={N} D={D} Bk={Bk} {dtype} kv_in={with_state} "
          f"dkv_out={with_gf} fwd_ws={use_fwd_ws}", flush=True)
    lam = synth.decay_schedule(H)
    _, (q, k, v, g), (qh, kh, vh, gh) = inputs(seed, B, H, N, D, dtype, with_do=True)
    s0 = state_input(seed, B, H, D) if with_state else None
    gf = state_input(seed + 1000, B, H, D) if with_gf else None
    kv_in = torch.from_numpy(s0).cuda() if with_state else None
    dkv_out = torch.from_numpy(gf).cuda() if with_gf else None
    code = la.LA_BF16 if dtype == "bf16" else la.LA_F32
    nb = la.la_fwd_workspace_bytes(B, H, N, D, Bk, code)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    o, s = la.la_fwd(q, k, v, lam, Bk=Bk, kv_in=kv_in, ws=ws, phi=phi)
    dq, dk, dv, ds0 = la.la_bwd(q, k, v, g, lam, Bk=Bk, kv_in=kv_in, dkv_out=dkv_out, want_dkv_in=True,
                                fwd_ws=ws if (use_fwd_ws and nb) else None, phi=phi)
    torch.cuda.synchronize()
    lp = lam_pairs(lam, B)
    s0h = None if s0 is None else s0.astype(np.float64)
    o_ref, s_ref = oracle.fwd_recurrent(qh, kh, vh, lp, s0h, phi=phi)
    refs = oracle.bwd_recurrent(qh, kh, vh, gh, lp, s0h, g_final=None if gf is None else gf.astype(np.float64),
                                want_ds_init=True, phi=phi)
    errs = [oracle.rel_l2(got(o), o_ref), oracle.rel_l2(got(s), s_ref)]
    errs += [oracle.rel_l2(got(x), r) for x, r in zip((dq, dk, dv, ds0), refs)]
    print("    rel-L2 O={:.2e} S={:.2e} dQ={:.2e} dK={:.2e} dV={:.2e} dS0={:.2e}".format(*errs), flush=True)
    assert max(errs) <= bar(dtype)


@pytest.mark.parametrize("phi", ["elu1", "relu"])
@pytest.mark.parametrize("kernel", ["default", "generic"])
@pytest.mark.parametrize("N,cks,with_state,with_gf,use_fwd_ws", [(64 * 13 + 5, 3, True, True, True),
                                                                (64 * 13 + 5, 3, False, False, False),
                                                                (700, 1, True, False, False)])
def test_feature_map_bf16(phi, kernel, N, cks, with_state, with_gf, use_fwd_ws, env):
    env(kernel="generic" if kernel == "generic" else None, chunks=cks)
    run_case(1, 3, N, 128, 64, "bf16", phi, seed=N + cks, with_state=with_state, with_gf=with_gf,
             use_fwd_ws=use_fwd_ws, label=kernel)


@pytest.mark.parametrize("phi", ["elu1", "relu"])
def test_feature_map_block_128_and_float32(phi, env):
    """Block size 128 (the register-staged shapes, routed to the generic kernels with a map)
    and float32 storage at the float32 bar."""
    env(chunks=2)
    run_case(1, 2, 600, 128, 128, "bf16", phi, seed=5, with_state=True, with_gf=True, use_fwd_ws=True,
             label="Bk128")
    run_case(1, 2, 300, 32, 32, "f32", phi, seed=6, with_state=True, with_gf=True, use_fwd_ws=False,
             label="f32")


@pytest.mark.parametrize("phi", ["elu1", "relu"])
def test_feature_map_decode_and_varlen(phi):
    """Decode steps continue the forward with the map; the ragged prefill with the map
    equals the oracle per sequence."""
    Bs, H, D, steps = 2, 3, 128, 12
    lam = synth.decay_schedule(H)
    state = torch.zeros((Bs, H, D, D), dtype=torch.float32, device="cuda")
    S_ref = np.zeros((Bs * H, D, D))
    worst = 0.0
    for t in range(steps):
        arrs = [synth.normal(70 + t, sid, (Bs, H, D), 1.0 / math.sqrt(D), "bf16") for sid in (1, 2, 3)]
        o = la.la_decode_step(state, *(to_dev(a, "bf16") for a in arrs), lam, phi=phi)
        torch.cuda.synchronize()
        hq, hk, hv = (host_f64(a, "bf16").reshape(Bs * H, D) for a in arrs)
        o_ref, S_ref = oracle.decode_step(S_ref, hq, hk, hv, lam_pairs(lam, Bs), phi=phi)
        worst = max(worst, oracle.rel_l2(got(o).reshape(Bs * H, D), o_ref))
    assert worst <= BF16_BAR and oracle.rel_l2(got(state).reshape(Bs * H, D, D), S_ref) <= BF16_BAR

    lens = [5, 130, 0, 700]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(offs[-1])
    bits = [synth.normal(80, sid, (T, H, D), 1.0 / math.sqrt(D), "bf16") for sid in (1, 2, 3)]
    q, k, v = (torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda() for b in bits)
    qh, kh, vh = (synth.bf16_bits_to_f64(b) for b in bits)
    o, s = la.la_fwd_varlen(q, k, v, lam, offs, phi=phi)
    torch.cuda.synchronize()
    for b in range(len(lens)):
        a_, e_ = int(offs[b]), int(offs[b + 1])
        for h in range(H):
            if e_ == a_:
                assert not np.any(got(s[b, h]))
                continue
            o_ref, s_ref = oracle.fwd_recurrent(qh[a_:e_, h], kh[a_:e_, h], vh[a_:e_, h], float(lam[h]), phi=phi)
            assert oracle.rel_l2(got(o[a_:e_, h]), o_ref) <= BF16_BAR
            assert oracle.rel_l2(got(s[b, h]), s_ref) <= BF16_BAR
