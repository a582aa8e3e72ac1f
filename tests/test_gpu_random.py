"""Seeded random configurations over the whole argument space (short sequences, and a set of
longer ones with more chunks), each against the oracle:
storage dtype, head dim, block size, sequence length (ragged), batch and heads, decays
(including 0 and 1), feature map, initial state, final-state gradient, forced chunk
counts and aggregate parts.  Forward, backward (with and without the forward's chunk
states, with the state gradients) and the decay derivative."""
import numpy as np
import pytest

import oracle
from helpers import bar, got, inputs, lam_pairs, state_input

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import causal_linear_attention_tiled_amd as la  # noqa: E402


def draw(seed):
    r = np.random.default_rng(1000 + seed)
    dtype = "bf16" if r.random() < 0.75 else "f32"
    D = int(r.choice([16, 32, 64, 128], p=[0.15, 0.15, 0.2, 0.5]))
    Bk = int(r.choice([16, 32, 64, 128], p=[0.15, 0.15, 0.45, 0.25]))
    N = int(r.integers(1, 1400))
    B, H = int(r.integers(1, 3)), int(r.integers(1, 4))
    lam = r.choice([0.0, 1.0, 0.5, 0.9, 0.99, 0.999], size=H).astype(np.float32)
    phi = str(r.choice(["identity", "identity", "elu1", "relu"]))
    cks = int(r.choice([0, 0, 2, 3, 5]))
    agg = int(r.choice([0, 2])) if cks else 0
    return dict(dtype=dtype, D=D, Bk=Bk, N=N, B=B, H=H, lam=lam, phi=phi, cks=cks, agg=agg,
                with_state=bool(r.random() < 0.5), with_gf=bool(r.random() < 0.5), fwd_ws=bool(r.random() < 0.5))


def draw_long(seed):
    """Longer sequences (1000-6000 tokens) with more chunks and aggregate parts, block sizes up
    to 256."""
    r = np.random.default_rng(5000 + seed)
    dtype = "bf16" if r.random() < 0.85 else "f32"
    D = int(r.choice([64, 128], p=[0.2, 0.8]))
    Bk = int(r.choice([64, 128, 256]))
    N = int(r.integers(1000, 6000))
    B, H = int(r.integers(1, 3)), int(r.integers(1, 3))
    lam = r.choice([0.0, 1.0, 0.9, 0.99, 0.999, 0.9999], size=H).astype(np.float32)
    phi = str(r.choice(["identity", "identity", "elu1", "relu"]))
    cks = int(r.choice([0, 2, 3, 5, 8, 13]))
    agg = int(r.choice([0, 2, 3, 4])) if cks else 0
    return dict(dtype=dtype, D=D, Bk=Bk, N=N, B=B, H=H, lam=lam, phi=phi, cks=cks, agg=agg,
                with_state=bool(r.random() < 0.5), with_gf=bool(r.random() < 0.5), fwd_ws=bool(r.random() < 0.5))


@pytest.mark.parametrize("seed", range(8))
def test_random_long_configuration(seed, monkeypatch):
    check_configuration(draw_long(seed), seed, monkeypatch)


@pytest.mark.parametrize("seed", range(24))
def test_random_configuration(seed, monkeypatch):
    check_configuration(draw(seed), seed, monkeypatch)


def check_configuration(c, seed, monkeypatch):
    monkeypatch.delenv("LA_KERNEL", raising=False)
    monkeypatch.delenv("LA_AGG_K", raising=False)
    if c["cks"]:
        monkeypatch.setenv("LA_CHUNKS", str(c["cks"]))
    else:
        monkeypatch.delenv("LA_CHUNKS", raising=False)
    code = la.LA_BF16 if c["dtype"] == "bf16" else la.LA_F32
    B, H, N, D, Bk = c["B"], c["H"], c["N"], c["D"], c["Bk"]
    plan = la.la_plan(B, H, N, D, Bk, code)
    if c["agg"] and plan["chunks"] > 1 and (plan["chunk_len"] // Bk) % c["agg"] == 0:
        monkeypatch.setenv("LA_AGG_K", str(c["agg"]))
        plan = la.la_plan(B, H, N, D, Bk, code)
    print(f"[random {seed}] {c['dtype']} B={B} H={H} N={N} D={D} Bk={Bk} lam={c['lam'].tolist()} phi={c['phi']} "
          f"kv_in={c['with_state']} dkv_out={c['with_gf']} fwd_ws={c['fwd_ws']} plan={plan}", flush=True)
    lam, dtype, phi = c["lam"], c["dtype"], c["phi"]
    _, (q, k, v, g), (qh, kh, vh, gh) = inputs(seed + 77, B, H, N, D, dtype, with_do=True)
    s0 = state_input(seed + 77, B, H, D) if c["with_state"] else None
    gf = state_input(seed + 1077, B, H, D) if c["with_gf"] else None
    kv_in = None if s0 is None else torch.from_numpy(s0).cuda()
    dkv_out = None if gf is None else torch.from_numpy(gf).cuda()
    ws = torch.empty(max(la.la_fwd_workspace_bytes(B, H, N, D, Bk, code), 1), dtype=torch.uint8, device="cuda")
    o, s = la.la_fwd(q, k, v, lam, Bk=Bk, kv_in=kv_in, ws=ws, phi=phi)
    dq, dk, dv, ds0 = la.la_bwd(q, k, v, g, lam, Bk=Bk, kv_in=kv_in, dkv_out=dkv_out, want_dkv_in=True,
                                fwd_ws=ws if c["fwd_ws"] else None, phi=phi)
    dl = la.la_dlam(q, k, v, g, lam, Bk=Bk, kv_in=kv_in, dkv_out=dkv_out, phi=phi)
    torch.cuda.synchronize()

    lp = lam_pairs(lam, B)
    s0h = None if s0 is None else s0.astype(np.float64)
    gfh = None if gf is None else gf.astype(np.float64)
    o_ref, s_ref = oracle.fwd_recurrent(qh, kh, vh, lp, s0h, phi=phi)
    refs = oracle.bwd_recurrent(qh, kh, vh, gh, lp, s0h, g_final=gfh, want_ds_init=True, phi=phi)
    per = np.asarray(oracle.dlam_recurrent(qh, kh, vh, gh, lp, s0h, gfh, phi=phi)).reshape(B, H)
    errs = {"O": oracle.rel_l2(got(o), o_ref), "kv_out": oracle.rel_l2(got(s), s_ref)}
    for name, x, r in zip(("dQ", "dK", "dV", "dS0"), (dq, dk, dv, ds0), refs):
        errs[name] = oracle.rel_l2(got(x), r)
    y = got(dl)
    errs["dlam"] = oracle.rel_l2(y, per.sum(axis=0))
    # each head against the size of its per-sequence terms (a batch sum can cancel)
    errs["dlam_head"] = float(np.max(np.abs(y - per.sum(axis=0)) / np.maximum(np.abs(per).sum(axis=0), 1e-300)))
    print("    " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
    for name, e in errs.items():
        assert np.isfinite(e) and e <= bar(dtype), name
