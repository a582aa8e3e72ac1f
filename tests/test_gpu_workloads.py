"""Parity at the full workload sizes, in the launch configuration the benchmark times.

Each workload runs on the GPU at its real shape through the C ABI; the fp64
oracle then recomputes a spread-out sample of whole sequences, regenerated on
their own from the counter-based input streams, and every sampled sequence must
meet the bf16 bar (relative L2 <= 2e-2) for each output.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from helpers import BF16_BAR, device_stream, got, sample_pairs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import causal_linear_attention_tiled_amd as la  # noqa: E402

D = 128


def qkv_dev(B, H, N, with_do=False, seed=0):
    ids = [synth.ID_Q, synth.ID_K, synth.ID_V] + ([synth.ID_DO] if with_do else [])
    return [device_stream(seed, i, (B, H, N, D), "bf16") for i in ids]


def pair_inputs(B, H, N, b, h, with_do=False, seed=0):
    ids = [synth.ID_Q, synth.ID_K, synth.ID_V] + ([synth.ID_DO] if with_do else [])
    return [synth.bf16_bits_to_f64(synth.pair_slice(seed, i, B, H, N, D, b, h, "bf16")) for i in ids]


def check_fwd_sampled(o, s, B, H, N, lam, samples):
    for b, h in samples:
        q, k, v = pair_inputs(B, H, N, b, h)
        o_ref, s_ref = oracle.fwd_recurrent(q, k, v, float(lam[h]))
        e_o = oracle.rel_l2(got(o[b, h]), o_ref)
        e_s = oracle.rel_l2(got(s[b, h]), s_ref)
        print(f"    (b={b}, h={h}) lam={lam[h]:.5f} rel-L2 O={e_o:.3e} kv_out={e_s:.3e}", flush=True)
        assert e_o <= BF16_BAR and e_s <= BF16_BAR


def test_fwd_b4_h16_n2048():
    """bf16 forward, B=4 H=16 N=2048 D=128 Bk=64: every sequence against the oracle."""
    B, H, N = 4, 16, 2048
    print(f"[workload] fwd B={B} H={H} N={N} Bk=64", flush=True)
    lam = synth.decay_schedule(H)
    q, k, v = qkv_dev(B, H, N)
    o, s = la.la_fwd(q, k, v, lam, Bk=64)
    torch.cuda.synchronize()
    qh, kh, vh = (synth.bf16_bits_to_f64(x) for x in synth.qkv(0, B, H, N, D, "bf16"))
    o_ref, s_ref = oracle.fwd_recurrent(qh, kh, vh, np.tile(lam.astype(np.float64), B))
    e_o, e_s = oracle.rel_l2(got(o), o_ref), oracle.rel_l2(got(s), s_ref)
    print(f"    rel-L2 O={e_o:.3e} kv_out={e_s:.3e}", flush=True)
    assert e_o <= BF16_BAR and e_s <= BF16_BAR


@pytest.mark.parametrize("N", [1024, 4096, 16384, 65536])
def test_fwd_sweep_131072_tokens(N):
    """bf16 forward sweep at 131072 tokens per head: B = 131072 / N, H=16, D=128, Bk=64."""
    B, H = 131072 // N, 16
    print(f"[workload] fwd sweep B={B} H={H} N={N} Bk=64", flush=True)
    lam = synth.decay_schedule(H)
    q, k, v = qkv_dev(B, H, N)
    o, s = la.la_fwd(q, k, v, lam, Bk=64)
    torch.cuda.synchronize()
    check_fwd_sampled(o, s, B, H, N, lam, sample_pairs(B, H, 5))


def training_step(B, H, N):
    """la_fwd then la_bwd as the benchmark runs them: the backward takes the forward's chunk
    states from the forward's workspace."""
    lam = synth.decay_schedule(H)
    q, k, v, g = qkv_dev(B, H, N, with_do=True)
    nb = la.la_fwd_workspace_bytes(B, H, N, D, 64, la.LA_BF16)
    ws_f = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda") if nb else None
    o, s = la.la_fwd(q, k, v, lam, Bk=64, ws=ws_f)
    dq, dk, dv = la.la_bwd(q, k, v, g, lam, Bk=64, fwd_ws=ws_f)
    torch.cuda.synchronize()
    return lam, (o, s), (dq, dk, dv)


def check_bwd_sampled(grads, B, H, N, lam, samples):
    for b, h in samples:
        qh, kh, vh, gh = pair_inputs(B, H, N, b, h, with_do=True)
        refs = oracle.bwd_recurrent(qh, kh, vh, gh, float(lam[h]))
        errs = [oracle.rel_l2(got(x[b, h]), r) for x, r in zip(grads, refs)]
        print(f"    (b={b}, h={h}) rel-L2 dQ={errs[0]:.3e} dK={errs[1]:.3e} dV={errs[2]:.3e}", flush=True)
        assert max(errs) <= BF16_BAR


def test_fwd_bwd_b2_h32_n8192():
    """bf16 training step, B=2 H=32 N=8192 D=128 Bk=64: O, dQ, dK, dV on sampled sequences."""
    B, H, N = 2, 32, 8192
    print(f"[workload] fwd+bwd B={B} H={H} N={N} Bk=64", flush=True)
    lam, (o, s), grads = training_step(B, H, N)
    check_fwd_sampled(o, s, B, H, N, lam, sample_pairs(B, H, 4))
    check_bwd_sampled(grads, B, H, N, lam, sample_pairs(B, H, 4))


@pytest.mark.parametrize("N", [1024, 4096, 16384, 65536])
def test_fwd_bwd_sweep_131072_tokens(N):
    """bf16 training step of the sweep at 131072 tokens per head (B = 131072 / N, H=16, D=128,
    Bk=64), launched as the benchmark launches it: dQ, dK, dV on sampled sequences."""
    B, H = 131072 // N, 16
    print(f"[workload] fwd+bwd sweep B={B} H={H} N={N} Bk=64", flush=True)
    lam, _, grads = training_step(B, H, N)
    check_bwd_sampled(grads, B, H, N, lam, sample_pairs(B, H, 3))


def test_long_prefill_then_decode():
    """bf16 prefill B=1 H=64 N=262144 D=128 Bk=128, then 256 recurrent decode steps for 256
    sequences that all start from the prefill's final state; checked against the oracle,
    against la_fwd continued from that state, and (slot 0) against one la_fwd over all
    262144 + 256 tokens."""
    B, H, N, Bs, steps = 1, 64, 262144, 256, 256
    print(f"[workload] prefill B={B} H={H} N={N} Bk=128", flush=True)
    lam = synth.decay_schedule(H)
    q, k, v = qkv_dev(B, H, N)
    o, s = la.la_fwd(q, k, v, lam, Bk=128)
    torch.cuda.synchronize()
    heads = [0, 21, 42, 63]
    s_oracle = {}
    for h in heads:
        qh, kh, vh = pair_inputs(B, H, N, 0, h)
        o_ref, s_ref = oracle.fwd_recurrent(qh, kh, vh, float(lam[h]))
        s_oracle[h] = s_ref
        e_o, e_s = oracle.rel_l2(got(o[0, h]), o_ref), oracle.rel_l2(got(s[0, h]), s_ref)
        print(f"    prefill h={h} lam={lam[h]:.5f} rel-L2 O={e_o:.3e} kv_out={e_s:.3e}", flush=True)
        assert e_o <= BF16_BAR and e_s <= BF16_BAR
    del q, k, v, o

    print(f"[workload] decode Bs={Bs} H={H} steps={steps}", flush=True)
    state = s.expand(Bs, H, D, D).contiguous()
    slots = [0, 77, 255]
    lam64 = lam.astype(np.float64)
    s_gpu0 = got(s[0])                       # the GPU's own prefill state, promoted
    S_a = {(sl, h): s_gpu0[h].copy() for sl in slots for h in heads}
    S_b = {(sl, h): s_oracle[h].copy() for sl in slots for h in heads}
    dec_q, dec_k, dec_v, dec_o = [], [], [], []
    worst_a = worst_b = 0.0
    for t in range(steps):
        arrs = [synth.normal(0, i, (Bs, H, D), 1.0 / math.sqrt(D), "bf16") for i in synth.decode_ids(t)]
        dev = [torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda() for x in arrs]
        od = la.la_decode_step(state, *dev, lam)
        torch.cuda.synchronize()
        od_h = od.float().cpu().numpy()
        f = [synth.bf16_bits_to_f64(x) for x in arrs]
        for sl in slots:
            for h in heads:
                o_a, S_a[(sl, h)] = oracle.decode_step(S_a[(sl, h)], f[0][sl, h], f[1][sl, h], f[2][sl, h], lam64[h])
                o_b, S_b[(sl, h)] = oracle.decode_step(S_b[(sl, h)], f[0][sl, h], f[1][sl, h], f[2][sl, h], lam64[h])
                worst_a = max(worst_a, oracle.rel_l2(od_h[sl, h].astype(np.float64), o_a))
                worst_b = max(worst_b, oracle.rel_l2(od_h[sl, h].astype(np.float64), o_b))
        dec_q.append(arrs[0]); dec_k.append(arrs[1]); dec_v.append(arrs[2]); dec_o.append(od_h)
    st_h = got(state)
    e_sa = max(oracle.rel_l2(st_h[sl, h], S_a[(sl, h)]) for sl in slots for h in heads)
    e_sb = max(oracle.rel_l2(st_h[sl, h], S_b[(sl, h)]) for sl in slots for h in heads)
    print(f"    decode worst rel-L2 o: from GPU prefill state {worst_a:.3e}, end to end {worst_b:.3e}; "
          f"state {e_sa:.3e} / {e_sb:.3e}", flush=True)
    assert max(worst_a, worst_b, e_sa, e_sb) <= BF16_BAR

    # the same 256 tokens through la_fwd continued from the prefill state, every slot
    stack = lambda xs: torch.from_numpy(np.ascontiguousarray(np.stack(xs, axis=2)).view(np.int16)).view(
        torch.bfloat16).cuda()
    kv_in = s.expand(Bs, H, D, D).contiguous()
    of, sf = la.la_fwd(stack(dec_q), stack(dec_k), stack(dec_v), lam, Bk=128, kv_in=kv_in)
    torch.cuda.synchronize()
    o_dec = np.stack(dec_o, axis=2)
    e_f = oracle.rel_l2(o_dec.astype(np.float64), got(of))
    e_fs = oracle.rel_l2(st_h, got(sf))
    print(f"    decode vs la_fwd(kv_in) rel-L2 o={e_f:.3e} state={e_fs:.3e}", flush=True)
    assert e_f <= BF16_BAR and e_fs <= BF16_BAR
    del of, sf, kv_in

    # slot 0 against one la_fwd over all N + 256 tokens (2050 blocks of 128): the prefill's
    # tokens followed by the slot's decode tokens
    print(f"[workload] slot 0 against la_fwd over {N + steps} tokens", flush=True)
    q, k, v = qkv_dev(B, H, N)
    tail = [stack(x)[0:1] for x in (dec_q, dec_k, dec_v)]
    q, k, v = (torch.cat([a, b], dim=2).contiguous() for a, b in zip((q, k, v), tail))
    del tail
    oa, sa = la.la_fwd(q, k, v, lam, Bk=128)
    torch.cuda.synchronize()
    e_all = oracle.rel_l2(o_dec[0:1].astype(np.float64), got(oa[:, :, N:]))
    e_alls = oracle.rel_l2(st_h[0], got(sa[0]))
    print(f"    slot 0 decode vs la_fwd over {N + steps} tokens rel-L2 o={e_all:.3e} state={e_alls:.3e}", flush=True)
    assert e_all <= BF16_BAR and e_alls <= BF16_BAR
