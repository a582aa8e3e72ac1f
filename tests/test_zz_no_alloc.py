"""la_fwd_noalloc through the C ABI: the chunk states live in the library's static
per-device scratch instead of a caller workspace.  Two calls in a row, the second with a
smaller input (the scratch then holds the first call's larger contents beyond what the
second writes), each against la_fwd on the same inputs (bit-identical: the same kernels
and plan) and against the fp64 oracle within the bf16 bar.  A call too large for the
scratch is rejected with LA_ESCRATCH and launches nothing."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from helpers import BF16_BAR, got, inputs, lam_pairs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import causal_linear_attention_tiled_amd as la  # noqa: E402


def noalloc_via_abi(q, k, v, lam, Bk, kv_in=None, want_state=True):
    """Call the C entry point directly (ctypes), with outputs the test allocates."""
    B, H, N, D = q.shape
    out = torch.full_like(q, float("nan"))
    kv_out = torch.full((B, H, D, D), float("nan"), dtype=torch.float32, device=q.device) if want_state else None
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    lam_arr = (ctypes.c_float * H)(*[float(x) for x in lam])
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = la.lib.la_fwd_noalloc(p(q), p(k), p(v), lam_arr, B, H, N, D, Bk, la.LA_BF16, 0, p(kv_in), p(out),
                               p(kv_out), stream)
    assert rc == la.LA_OK, la.la_strerror(rc)
    return out, kv_out


@pytest.mark.parametrize("cases", [[(2, 8, 3000, 64, 7, True), (1, 4, 700, 64, 8, False)],
                                   [(1, 16, 4096, 128, 9, True), (2, 2, 1000, 128, 10, True)]])
def test_noalloc_matches_fwd_twice(cases):
    for (B, H, N, Bk, seed, with_state) in cases:
        plan = la.la_plan(B, H, N, 128, Bk, la.LA_BF16)
        need = la.la_fwd_workspace_bytes(B, H, N, 128, Bk, la.LA_BF16)
        print(f"[noalloc] B={B} H={H} N={N} Bk={Bk} plan={plan} scratch bytes used={need}", flush=True)
        assert plan["chunks"] > 1 and 0 < need <= la.la_scratch_bytes()
        lam = synth.decay_schedule(H)
        _, (q, k, v), (qh, kh, vh) = inputs(seed, B, H, N, 128, "bf16")
        s0 = None
        if with_state:
            s0 = synth.normal(seed, synth.ID_STATE, (B, H, 128, 128), 1.0 / np.sqrt(128), "f32")
        kv_in = None if s0 is None else torch.from_numpy(s0).cuda()
        o_n, s_n = noalloc_via_abi(q, k, v, lam, Bk, kv_in)
        o_f, s_f = la.la_fwd(q, k, v, lam, Bk=Bk, kv_in=kv_in)
        torch.cuda.synchronize()
        assert torch.equal(o_n, o_f) and torch.equal(s_n, s_f)
        o_ref, s_ref = oracle.fwd_recurrent(qh, kh, vh, lam_pairs(lam, B),
                                            None if s0 is None else s0.astype(np.float64))
        e_o, e_s = oracle.rel_l2(got(o_n), o_ref), oracle.rel_l2(got(s_n), s_ref)
        print(f"    rel-L2 O={e_o:.3e} kv_out={e_s:.3e}", flush=True)
        assert e_o <= BF16_BAR and e_s <= BF16_BAR


def test_noalloc_binding_and_limit(monkeypatch):
    B, H, N = 1, 4, 900
    lam = synth.decay_schedule(H)
    _, (q, k, v), _ = inputs(3, B, H, N, 128, "bf16")
    out = torch.empty_like(q)
    o, s = la.la_fwd_noalloc(q, k, v, lam, out, Bk=64)
    assert o is out and s is None
    o_f, _ = la.la_fwd(q, k, v, lam, Bk=64)
    torch.cuda.synchronize()
    assert torch.equal(o, o_f)
    # more chunk states than the scratch holds: rejected before any launch, outputs untouched
    monkeypatch.setenv("LA_CHUNKS", "32")
    Hb, Nb = 64, 32 * 4 * 64
    assert la.la_fwd_workspace_bytes(1, Hb, Nb, 128, 64, la.LA_BF16) > la.la_scratch_bytes()
    qb = torch.zeros((1, Hb, Nb, 128), dtype=torch.bfloat16, device="cuda")
    ob = torch.full_like(qb, 7.0)
    with pytest.raises(la.LaError) as e:
        la.la_fwd_noalloc(qb, qb.clone(), qb.clone(), [0.5] * Hb, ob, Bk=64)
    assert e.value.code == la.LA_ESCRATCH
    torch.cuda.synchronize()
    assert bool((ob == 7.0).all())


def test_noalloc_fused_prefix_falls_back(monkeypatch):
    """Chunk states that fit the static scratch while the fused prefix's aggregates and flags
    would not (4 chunks over 256 sequences: 48 MiB of states, 96 MiB with the aggregates):
    la_fwd_noalloc runs the three-launch prefix instead, bit-identical to la_fwd with
    LA_FUSED=0, within float rounding of la_fwd's fused form, and within the bar of the oracle
    on sampled sequences."""
    monkeypatch.setenv("LA_CHUNKS", "4")
    monkeypatch.delenv("LA_FUSED", raising=False)
    monkeypatch.delenv("LA_AGG_K", raising=False)
    B, H, N, D = 16, 16, 1024, 128
    plan = la.la_plan(B, H, N, D, 64, la.LA_BF16)
    states = B * H * (plan["chunks"] - 1) * D * D * 4
    need = la.la_fwd_workspace_bytes(B, H, N, D, 64, la.LA_BF16)
    print(f"[noalloc fallback] plan={plan} chunk states {states} B, fused workspace {need} B, "
          f"scratch {la.la_scratch_bytes()} B", flush=True)
    assert plan["chunks"] == 4 and plan["agg_parts"] == 1
    assert states <= la.la_scratch_bytes() < need
    lam = synth.decay_schedule(H)
    _, (q, k, v), (qh, kh, vh) = inputs(12, B, H, N, D, "bf16")
    o_n, s_n = noalloc_via_abi(q, k, v, lam, 64)
    monkeypatch.setenv("LA_FUSED", "0")
    o_3, s_3 = la.la_fwd(q, k, v, lam, Bk=64)
    monkeypatch.delenv("LA_FUSED")
    o_f, s_f = la.la_fwd(q, k, v, lam, Bk=64)
    torch.cuda.synchronize()
    assert torch.equal(o_n, o_3) and torch.equal(s_n, s_3)
    assert oracle.rel_l2(got(o_f), got(o_n)) <= 1e-2 and oracle.rel_l2(got(s_f), got(s_n)) <= 2e-3
    for b, h in [(0, 0), (7, 5), (15, 15)]:
        o_ref, s_ref = oracle.fwd_recurrent(qh[b, h], kh[b, h], vh[b, h], float(lam[h]))
        assert oracle.rel_l2(got(o_n[b, h]), o_ref) <= BF16_BAR, (b, h)
        assert oracle.rel_l2(got(s_n[b, h]), s_ref) <= BF16_BAR, (b, h)
