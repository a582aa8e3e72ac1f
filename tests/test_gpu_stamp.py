"""la_bwd with fwd_ws checks, on the device, the stamp la_fwd leaves after its chunk states
(shape, plan, decay values, input addresses).  A matching workspace is used; a workspace
from another call (other decay, other tensors) or one la_fwd never wrote makes the dQ rows
of every chunk that would start from those states NaN, instead of silently wrong; chunk 0
(which starts from kv_in) and dK, dV are unaffected."""
import numpy as np
import pytest

import oracle
import synth
from helpers import bar, got, inputs, lam_pairs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import causal_linear_attention_tiled_amd as la  # noqa: E402


@pytest.fixture
def variant(monkeypatch):
    def set_(v):
        for name in ("LA_KERNEL", "LA_FWD", "LA_REV", "LA_STATE", "LA_FWD128"):
            monkeypatch.delenv(name, raising=False)
        if v == "generic":
            monkeypatch.setenv("LA_KERNEL", "generic")
        elif v == "v1":
            for name in ("LA_FWD", "LA_REV", "LA_STATE"):
                monkeypatch.setenv(name, "v1")
        elif v == "dma128":
            monkeypatch.setenv("LA_FWD128", "1")
    return set_


@pytest.mark.parametrize("kern,Bk", [("default", 64), ("generic", 64), ("v1", 64), ("default", 128),
                                     ("dma128", 128), ("default", 256)])
def test_forward_workspace_stamp(kern, Bk, variant, monkeypatch):
    variant(kern)
    monkeypatch.setenv("LA_CHUNKS", "3")
    B, H, N, D = 1, 3, 256 * 5 + 17, 128
    lam = synth.decay_schedule(H)
    print(f"[stamp] {kern} Bk={Bk}", flush=True)
    _, (q, k, v, g), (qh, kh, vh, gh) = inputs(17, B, H, N, D, "bf16", with_do=True)
    plan = la.la_plan(B, H, N, D, Bk, la.LA_BF16)
    assert plan["chunks"] == 3
    L = plan["chunk_len"]
    nb = la.la_fwd_workspace_bytes(B, H, N, D, Bk, la.LA_BF16)
    fws = torch.full((nb,), 0x3F, dtype=torch.uint8, device="cuda")
    la.la_fwd(q, k, v, lam, Bk=Bk, ws=fws)

    # the matching call uses the states: same result as recomputing them, within the bar
    dq, dk, dv = la.la_bwd(q, k, v, g, lam, Bk=Bk, fwd_ws=fws)
    dq0, _, _ = la.la_bwd(q, k, v, g, lam, Bk=Bk)
    torch.cuda.synchronize()
    ref = oracle.bwd_recurrent(qh, kh, vh, gh, lam_pairs(lam, B))
    assert np.all(np.isfinite(got(dq)))
    assert oracle.rel_l2(got(dq), ref[0]) <= bar("bf16")
    assert oracle.rel_l2(got(dq), got(dq0)) <= bar("bf16")

    def poisoned(dq_t):
        y = got(dq_t)[0]
        return bool(np.all(np.isfinite(y[:, :L])) and np.all(np.isnan(y[:, L:])))

    # another decay
    lam2 = lam.copy()
    lam2[1] = np.float32(0.5)
    dq_b, dk_b, dv_b = la.la_bwd(q, k, v, g, lam2, Bk=Bk, fwd_ws=fws)
    torch.cuda.synchronize()
    assert poisoned(dq_b)
    assert np.all(np.isfinite(got(dk_b))) and np.all(np.isfinite(got(dv_b)))
    # other tensors (a copy of Q at another address)
    dq_c, _, _ = la.la_bwd(q.clone(), k, v, g, lam, Bk=Bk, fwd_ws=fws)
    torch.cuda.synchronize()
    assert poisoned(dq_c)
    # a workspace no forward pass wrote
    blank = torch.zeros_like(fws)
    dq_d, _, _ = la.la_bwd(q, k, v, g, lam, Bk=Bk, fwd_ws=blank)
    torch.cuda.synchronize()
    assert poisoned(dq_d)
