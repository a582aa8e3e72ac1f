"""The serving path: ragged batched prefill (la_fwd_varlen) and paged decode
slots (la_decode_step_paged), against the fp64 oracle per sequence.

Inputs are seeded, packed token-major [T][H][D] with N(0,1)/sqrt(D) entries;
each sequence is checked alone against the oracle's recurrent form, and
against la_fwd over that sequence alone.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from helpers import BF16_BAR, got, state_input

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import causal_linear_attention_tiled_amd as la  # noqa: E402

D = 128


def packed(seed, T, H):
    """Seeded packed [T, H, D] bf16 Q, K, V (device) and their float64 values (host)."""
    dev, host = [], []
    for sid in (synth.ID_Q, synth.ID_K, synth.ID_V):
        bits = synth.normal(seed, sid, (T, H, D), 1.0 / math.sqrt(D), "bf16")
        dev.append(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda())
        host.append(synth.bf16_bits_to_f64(bits))
    return dev, host


def packed_dev(seed, T, H):
    """The same device tensors, generated in slices (no host copy of the whole batch)."""
    out = []
    total = T * H * D
    for sid in (synth.ID_Q, synth.ID_K, synth.ID_V):
        t = torch.empty(total, dtype=torch.bfloat16, device="cuda")
        flat = t.view(torch.int16)
        for s0 in range(0, total, 1 << 26):
            n = min(1 << 26, total - s0)
            host = synth.normal(seed, sid, (n,), 1.0 / math.sqrt(D), "bf16", start=s0)
            flat[s0:s0 + n].copy_(torch.from_numpy(host.view(np.int16)))
        out.append(t.view(T, H, D))
    return out


def packed_rows(seed, sid, a, e, H, h):
    """Host float64 values of rows a .. e of head h, regenerated from the counter-based stream."""
    bits = synth.normal(seed, sid, ((e - a) * H * D,), 1.0 / math.sqrt(D), "bf16", start=a * H * D)
    return synth.bf16_bits_to_f64(bits).reshape(e - a, H, D)[:, h]


@pytest.fixture
def varlen_chunk(monkeypatch):
    def set_(L):
        if L is None:
            monkeypatch.delenv("LA_VARLEN_L", raising=False)
        else:
            monkeypatch.setenv("LA_VARLEN_L", str(L))
    return set_


@pytest.mark.parametrize("L", [None, 128, 64])
@pytest.mark.parametrize("with_state", [False, True])
def test_varlen_prefill_matches_oracle(L, with_state, varlen_chunk):
    """Ragged lengths (empty, one token, block edges, several chunks), every sequence and
    head against the oracle, and against la_fwd over the sequence alone."""
    varlen_chunk(L)
    lens = [1, 63, 64, 65, 300, 0, 1000, 129]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    H, T, B = 3, int(offs[-1]), len(lens)
    print(f"[varlen] lens={lens} H={H} L={L} kv_in={with_state}", flush=True)
    lam = synth.decay_schedule(H)
    (q, k, v), (qh, kh, vh) = packed(11, T, H)
    s0 = state_input(12, B, H, D) if with_state else None
    kv_in = torch.from_numpy(s0).cuda() if with_state else None
    o, s = la.la_fwd_varlen(q, k, v, lam, offs, Bk=64, kv_in=kv_in)
    torch.cuda.synchronize()
    o_h, s_h = got(o), got(s)
    for b in range(B):
        a, e = int(offs[b]), int(offs[b + 1])
        for h in range(H):
            init = None if s0 is None else s0[b, h].astype(np.float64)
            if e > a:
                o_ref, s_ref = oracle.fwd_recurrent(qh[a:e, h], kh[a:e, h], vh[a:e, h], float(lam[h]), init)
                assert oracle.rel_l2(o_h[a:e, h], o_ref) <= BF16_BAR, (b, h)
            else:
                s_ref = np.zeros((D, D)) if init is None else init
            assert oracle.rel_l2(s_h[b, h], s_ref) <= BF16_BAR, (b, h)
        if e > a:
            # the same sequence through the dense entry point
            seq = [x[a:e].permute(1, 0, 2).contiguous().unsqueeze(0) for x in (q, k, v)]
            kin = None if kv_in is None else kv_in[b:b + 1].contiguous()
            od, sd = la.la_fwd(*seq, lam, Bk=64, kv_in=kin)
            torch.cuda.synchronize()
            assert oracle.rel_l2(o_h[a:e], got(od)[0].transpose(1, 0, 2)) <= 1e-2
            assert oracle.rel_l2(s_h[b], got(sd)[0]) <= 1e-2


def test_varlen_prefill_serving_batch():
    """A serving-sized ragged batch: 64 sequences, lengths log-uniform in [128, 8192]
    (seeded), 16 heads; sampled sequences against the oracle."""
    rng = np.random.default_rng(2024)
    lens = np.exp(rng.uniform(np.log(128), np.log(8192), 64)).astype(np.int64)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    H, T = 16, int(offs[-1])
    print(f"[varlen] serving batch B=64 T={T} H={H}", flush=True)
    lam = synth.decay_schedule(H)
    q, k, v = packed_dev(21, T, H)
    o, s = la.la_fwd_varlen(q, k, v, lam, offs)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (17, 5), (40, 15), (63, 9), (int(np.argmax(lens)), 3)]:
        a, e = int(offs[b]), int(offs[b + 1])
        qh, kh, vh = (packed_rows(21, sid, a, e, H, h) for sid in (synth.ID_Q, synth.ID_K, synth.ID_V))
        o_ref, s_ref = oracle.fwd_recurrent(qh, kh, vh, float(lam[h]))
        e_o = oracle.rel_l2(got(o[a:e, h]), o_ref)
        e_s = oracle.rel_l2(got(s[b, h]), s_ref)
        print(f"    (b={b}, h={h}) n={e - a} rel-L2 O={e_o:.3e} kv_out={e_s:.3e}", flush=True)
        assert e_o <= BF16_BAR and e_s <= BF16_BAR


def test_paged_decode_matches_oracle():
    """Four sequences at pool slots 7, 2, 9, 0 of a 10-slot pool, 20 steps: outputs and the
    stepped slots against the oracle; the other slots stay bit-identical."""
    P, Bs, H, steps = 10, 4, 3, 20
    slots = np.array([7, 2, 9, 0], np.int32)
    lam = synth.decay_schedule(H)
    pool0 = state_input(31, P, H, D)
    pool = torch.from_numpy(pool0.copy()).cuda()
    slot_of = torch.from_numpy(slots).cuda()
    S_ref = {i: pool0[slots[i]].astype(np.float64) for i in range(Bs)}
    worst = 0.0
    for t in range(steps):
        arrs = [synth.normal(40 + t, sid, (Bs, H, D), 1.0 / math.sqrt(D), "bf16") for sid in (1, 2, 3)]
        dev = [torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda() for x in arrs]
        o = la.la_decode_step_paged(pool, slot_of, *dev, lam)
        torch.cuda.synchronize()
        f = [synth.bf16_bits_to_f64(x) for x in arrs]
        o_h = got(o)
        for i in range(Bs):
            o_ref, S_ref[i] = oracle.decode_step(S_ref[i], f[0][i], f[1][i], f[2][i], lam.astype(np.float64))
            worst = max(worst, oracle.rel_l2(o_h[i], o_ref))
    print(f"    paged decode worst rel-L2 o={worst:.3e}", flush=True)
    assert worst <= BF16_BAR
    pool_h = got(pool)
    for i in range(Bs):
        assert oracle.rel_l2(pool_h[slots[i]], S_ref[i]) <= BF16_BAR
    for p in set(range(P)) - set(slots.tolist()):
        np.testing.assert_array_equal(pool_h[p], pool0[p])


def test_paged_decode_bad_slot_writes_nan():
    """A slot index outside the pool leaves the pool untouched and gives a NaN output row;
    the other sequences step normally."""
    P, H = 4, 2
    lam = synth.decay_schedule(H)
    pool0 = state_input(51, P, H, D)
    pool = torch.from_numpy(pool0.copy()).cuda()
    slot_of = torch.tensor([1, 9, -1], dtype=torch.int32, device="cuda")
    q, k, v = (torch.from_numpy(synth.normal(52, sid, (3, H, D), 0.1, "bf16").view(np.int16)).view(
        torch.bfloat16).cuda() for sid in (1, 2, 3))
    o = la.la_decode_step_paged(pool, slot_of, q, k, v, lam)
    torch.cuda.synchronize()
    o_h = got(o)
    assert np.all(np.isnan(o_h[1])) and np.all(np.isnan(o_h[2]))
    assert not np.any(np.isnan(o_h[0]))
    pool_h = got(pool)
    for p in (0, 2, 3):
        np.testing.assert_array_equal(pool_h[p], pool0[p])
    assert not np.array_equal(pool_h[1], pool0[1])


def check_varlen_against_oracle(lens, H, Bk, seed, with_state):
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, B = int(offs[-1]), len(lens)
    lam = synth.decay_schedule(H)
    (q, k, v), (qh, kh, vh) = packed(seed, T, H)
    s0 = state_input(seed + 1, B, H, D) if with_state else None
    kv_in = torch.from_numpy(s0).cuda() if with_state else None
    o, s = la.la_fwd_varlen(q, k, v, lam, offs, Bk=Bk, kv_in=kv_in)
    torch.cuda.synchronize()
    o_h, s_h = got(o), got(s)
    worst = 0.0
    for b in range(B):
        a, e = int(offs[b]), int(offs[b + 1])
        for h in range(H):
            init = None if s0 is None else s0[b, h].astype(np.float64)
            if e > a:
                o_ref, s_ref = oracle.fwd_recurrent(qh[a:e, h], kh[a:e, h], vh[a:e, h], float(lam[h]), init)
                err = oracle.rel_l2(o_h[a:e, h], o_ref)
                worst = max(worst, err)
                assert err <= BF16_BAR, (b, h, err)
            else:
                s_ref = np.zeros((D, D)) if init is None else init
            assert oracle.rel_l2(s_h[b, h], s_ref) <= BF16_BAR, (b, h)
    print(f"    worst per-sequence rel-L2 of O {worst:.3e}", flush=True)


@pytest.mark.parametrize("Bk", [128, 256])
@pytest.mark.parametrize("L", [None, 512])
def test_varlen_block_sizes(Bk, L, varlen_chunk):
    """Bk 128 and 256: chunk boundaries on multiples of Bk (forced or planned), blocks stepped as
    64 tokens; ragged lengths on and next to those boundaries."""
    varlen_chunk(L)
    lens = [1, 127, 128, 129, 511, 512, 513, 1500, 0, 2100, 257]
    print(f"[varlen] Bk={Bk} L={L} lens={lens}", flush=True)
    check_varlen_against_oracle(lens, 3, Bk, 31 + Bk, with_state=True)


@pytest.mark.parametrize("with_state", [False, True])
def test_varlen_more_than_256_sequences(with_state):
    """600 sequences (three launch groups of at most 256), seeded lengths 0..300 with a few long
    ones, every sequence and head against the oracle; group boundaries fall between sequences
    255/256 and 511/512."""
    rng = np.random.default_rng(600)
    lens = rng.integers(0, 301, 600)
    lens[[3, 255, 256, 511, 599]] = [2000, 1, 1700, 999, 2500]
    print(f"[varlen] B=600 T={int(lens.sum())} kv_in={with_state}", flush=True)
    check_varlen_against_oracle(list(lens), 2, 64, 77, with_state)


# ------------------------------------------------------------------ the generic ragged path
def packed_any(seed, T, H, Dd, dtype):
    """Seeded packed [T, H, Dd] Q, K, V of dtype "bf16" or "f32" (device) and their float64
    values (host)."""
    from helpers import host_f64, to_dev
    dev, host = [], []
    for sid in (synth.ID_Q, synth.ID_K, synth.ID_V):
        a = synth.normal(seed, sid, (T, H, Dd), 1.0 / math.sqrt(Dd), dtype)
        dev.append(to_dev(a, dtype))
        host.append(host_f64(a, dtype))
    return dev, host


@pytest.mark.parametrize("dtype,Dd,Bk,phi", [("f32", 128, 64, "identity"), ("f32", 64, 32, "elu1"),
                                             ("bf16", 64, 64, "identity"), ("bf16", 32, 16, "relu"),
                                             ("bf16", 128, 32, "identity"), ("f32", 16, 256, "identity")])
@pytest.mark.parametrize("with_state", [False, True])
def test_varlen_generic_matches_oracle(dtype, Dd, Bk, phi, with_state):
    """Shapes outside the direct-to-LDS kernels (float32 storage, D != 128, Bk of 16 or 32)
    run the ragged forward on the generic kernels: every sequence and head against the
    oracle (empty and one-token sequences, block edges), and against la_fwd over the
    sequence alone."""
    from helpers import bar
    lens = [1, 63, 64, 65, 300, 0, 129, 7]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    H, T, B = 3, int(offs[-1]), len(lens)
    print(f"[varlen generic] {dtype} D={Dd} Bk={Bk} phi={phi} lens={lens} H={H} kv_in={with_state}", flush=True)
    lam = synth.decay_schedule(H)
    (q, k, v), (qh, kh, vh) = packed_any(31, T, H, Dd, dtype)
    s0 = state_input(32, B, H, Dd) if with_state else None
    kv_in = torch.from_numpy(s0).cuda() if with_state else None
    assert la.la_fwd_varlen_workspace_bytes(offs, H, Dd, Bk, la.LA_BF16 if dtype == "bf16" else la.LA_F32) == 0
    o, s = la.la_fwd_varlen(q, k, v, lam, offs, Bk=Bk, kv_in=kv_in, phi=phi)
    torch.cuda.synchronize()
    o_h, s_h = got(o), got(s)
    for b in range(B):
        a, e = int(offs[b]), int(offs[b + 1])
        for h in range(H):
            init = None if s0 is None else s0[b, h].astype(np.float64)
            if e > a:
                o_ref, s_ref = oracle.fwd_recurrent(qh[a:e, h], kh[a:e, h], vh[a:e, h], float(lam[h]), init,
                                                    phi=phi)
                assert oracle.rel_l2(o_h[a:e, h], o_ref) <= bar(dtype), (b, h)
            else:
                s_ref = np.zeros((Dd, Dd)) if init is None else init
            assert oracle.rel_l2(s_h[b, h], s_ref) <= bar(dtype), (b, h)
        if e > a:
            seq = [x[a:e].permute(1, 0, 2).contiguous().unsqueeze(0) for x in (q, k, v)]
            kin = None if kv_in is None else kv_in[b:b + 1].contiguous()
            od, sd = la.la_fwd(*seq, lam, Bk=Bk, kv_in=kin, phi=phi)
            torch.cuda.synchronize()
            assert oracle.rel_l2(o_h[a:e], got(od)[0].transpose(1, 0, 2)) <= max(bar(dtype), 1e-5)
            assert oracle.rel_l2(s_h[b], got(sd)[0]) <= max(bar(dtype), 1e-5)


def test_varlen_generic_many_sequences():
    """More than 256 sequences on the generic path (groups of 256), float32 D = 32, each with
    its own initial state; sampled sequences of both groups against the oracle."""
    rng = np.random.default_rng(77)
    lens = rng.integers(0, 40, 300)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    H, T, B, Dd = 2, int(offs[-1]), len(lens), 32
    print(f"[varlen generic] B={B} T={T} H={H} D={Dd} f32", flush=True)
    lam = synth.decay_schedule(H)
    (q, k, v), (qh, kh, vh) = packed_any(41, T, H, Dd, "f32")
    s0 = state_input(42, B, H, Dd)
    o, s = la.la_fwd_varlen(q, k, v, lam, offs, Bk=32, kv_in=torch.from_numpy(s0).cuda())
    torch.cuda.synchronize()
    o_h, s_h = got(o), got(s)
    for b in [0, 1, 100, 255, 256, 257, 299]:
        a, e = int(offs[b]), int(offs[b + 1])
        for h in range(H):
            init = s0[b, h].astype(np.float64)
            if e > a:
                o_ref, s_ref = oracle.fwd_recurrent(qh[a:e, h], kh[a:e, h], vh[a:e, h], float(lam[h]), init)
                assert oracle.rel_l2(o_h[a:e, h], o_ref) <= 1e-5, (b, h)
            else:
                s_ref = init
            assert oracle.rel_l2(s_h[b, h], s_ref) <= 1e-5, (b, h)
