"""The derivative of L = <dO, O> + <F, S_N> with respect to the per-head decay (la_dlam)
against the oracle's forward-mode derivative of the recurrence, summed over the batch
per head.  Covered: the matrix-core path (bf16, D=128, Bk=64) and the generic kernels
(other shapes, float32 storage), one chunk and several (the chunked prefix over the pair
(S, T)), initial state and final-state gradient, the feature maps, ragged tails, lam = 0
and lam = 1, and the training-step sizes on sampled heads.  The bar is the relative L2
error of the [H] result, and also each head's error against the sum of the magnitudes of
its per-sequence values; each head's cancellation (the magnitude of its terms over its
value) is printed beside it."""
import numpy as np
import pytest

import oracle
import synth
from helpers import BF16_BAR, bar, device_stream, got, inputs, lam_pairs, state_input

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import causal_linear_attention_tiled_amd as la  # noqa: E402


@pytest.fixture
def env(monkeypatch):
    def set_(kernel=None, chunks=None):
        # kernel: "default" (direct-to-LDS sweep with 8 compute waves and aggregates, for bf16
        # D=128 Bk=64), "dma4" (the same sweep with 4 compute waves), "v1" (the register-staged
        # matrix-core kernels), "generic"
        for name, val in (("LA_KERNEL", "generic" if kernel == "generic" else None),
                          ("LA_DLAM", "v1" if kernel == "v1" else None),
                          ("LA_DLAM_WAVES", "4" if kernel == "dma4" else None), ("LA_CHUNKS", chunks)):
            if val is None:
                monkeypatch.delenv(name, raising=False)
            else:
                monkeypatch.setenv(name, str(val))
    return set_


def run_case(B, H, N, D, Bk, dtype, lam, seed, with_state, with_gf, phi="identity", label=""):
    print(f"[dlam] {label} B={B} H={H} N={N} D={D} Bk={Bk} {dtype} phi={phi} kv_in={with_state} "
          f"dkv_out={with_gf} lam={np.round(np.asarray(lam, dtype=np.float64), 4).tolist()}", flush=True)
    lam = np.asarray(lam, dtype=np.float32)
    _, (q, k, v, g), (qh, kh, vh, gh) = inputs(seed, B, H, N, D, dtype, with_do=True)
    s0 = state_input(seed, B, H, D) if with_state else None
    gf = state_input(seed + 1000, B, H, D) if with_gf else None
    out = la.la_dlam(q, k, v, g, lam, Bk=Bk, kv_in=None if s0 is None else torch.from_numpy(s0).cuda(),
                     dkv_out=None if gf is None else torch.from_numpy(gf).cuda(), phi=phi)
    torch.cuda.synchronize()
    per = oracle.dlam_recurrent(qh, kh, vh, gh, lam_pairs(lam, B),
                                None if s0 is None else s0.astype(np.float64),
                                None if gf is None else gf.astype(np.float64), phi=phi)
    per = np.asarray(per).reshape(B, H)
    ref = per.sum(axis=0)
    y = got(out)
    err = oracle.rel_l2(y, ref)
    # each head against the size of its per-sequence values: a batch sum can cancel (elu + 1
    # features make every q . k positive and large), so |ref| alone is no scale for it
    scale = np.abs(per).sum(axis=0)
    head = np.abs(y - ref) / np.maximum(scale, 1e-300)
    # how far each head's value cancels within its terms (diagnostic: sum of the terms'
    # magnitudes over the value; random inputs give hundreds to thousands)
    mag = np.array([[oracle.dlam_magnitude(qh[b, h], kh[b, h], vh[b, h], gh[b, h], float(lam[h]),
                                           None if s0 is None else s0[b, h].astype(np.float64),
                                           None if gf is None else gf[b, h].astype(np.float64), phi=phi)
                     for h in range(H)] for b in range(B)]).sum(axis=0)
    print(f"    rel-L2 {err:.2e}; per head |err| / sum_b |dL/dlam_bh| "
          f"{np.array2string(head, precision=2, floatmode='unique')}; cancellation "
          f"{np.array2string(mag / np.maximum(scale, 1e-300), precision=0)}", flush=True)
    assert np.all(np.isfinite(y))
    assert err <= bar(dtype)
    assert np.all(head <= bar(dtype))
    return y, ref


@pytest.mark.parametrize("kernel", ["default", "dma4", "v1", "generic"])
@pytest.mark.parametrize("N,cks,with_state,with_gf", [(64 * 13 + 5, 3, True, True), (64 * 13 + 5, None, True, True),
                                                      (64 * 13 + 5, 3, False, False), (64 * 8, 4, False, True),
                                                      (37, None, True, True), (64, None, False, True)])
def test_dlam_bf16_d128(env, kernel, N, cks, with_state, with_gf):
    env(kernel=kernel, chunks=cks)
    run_case(2, 4, N, 128, 64, "bf16", synth.decay_schedule(4), 3, with_state, with_gf, label=kernel)


@pytest.mark.parametrize("phi", ["elu1", "relu"])
@pytest.mark.parametrize("kernel", ["default", "dma4", "v1", "generic"])
def test_dlam_feature_maps(env, kernel, phi):
    env(kernel=kernel, chunks=3)
    run_case(2, 4, 64 * 11 + 9, 128, 64, "bf16", synth.decay_schedule(4), 5, True, True, phi=phi, label=kernel)


@pytest.mark.parametrize("kernel", ["default", "dma4", "v1", "generic"])
@pytest.mark.parametrize("lam", [[0.0, 0.0], [1.0, 1.0], [0.0, 1.0]])
def test_dlam_degenerate_decays(env, kernel, lam):
    """lam = 0 (only first-order terms survive: each token with its predecessor, S0's first
    step, the final state's last-but-one token) and lam = 1 (no decay: every age counts)."""
    env(kernel=kernel, chunks=3)
    run_case(1, 2, 64 * 7 + 3, 128, 64, "bf16", lam, 7, True, True, label=kernel)


@pytest.mark.parametrize("D,Bk,N,cks", [(64, 32, 300, 3), (16, 16, 70, None), (128, 128, 300, 2), (32, 64, 1, None),
                                           (16, 256, 600, 2)])
def test_dlam_float32(env, D, Bk, N, cks):
    env(chunks=cks)
    run_case(2, 3, N, D, Bk, "f32", np.array([0.3, 0.9, 0.999]), 9, True, True)


@pytest.mark.parametrize("D,Bk", [(64, 64), (128, 128), (128, 32), (128, 256)])
def test_dlam_bf16_generic_shapes(env, D, Bk):
    """bf16 shapes outside the 64-token matrix-core sweep: D = 64 and Bk = 32 run the generic
    kernels, Bk = 128 and 256 the direct-to-LDS sweep in 64-token steps."""
    env(chunks=3)
    run_case(2, 3, 5 * Bk + 7, D, Bk, "bf16", np.array([0.5, 0.97, 1.0]), 11, True, True)


@pytest.mark.parametrize("kernel", ["default", "v1", "generic"])
@pytest.mark.parametrize("cks,agg", [(2, 2), (2, 4), (3, 2)])
def test_dlam_aggregate_parts(env, kernel, cks, agg, monkeypatch):
    """The (S, T) chunk aggregates and their scan over agg parts of each chunk."""
    env(kernel=kernel, chunks=cks)
    monkeypatch.setenv("LA_AGG_K", str(agg))
    run_case(2, 3, 64 * 15 + 17, 128, 64, "bf16", synth.decay_schedule(3), 17 + agg, True, True,
             label=f"{kernel} parts={agg}")


def test_dlam_per_head_batch_sum(env):
    """Heads with equal decays but different inputs: the result is the sum over the batch of
    each head's own sequences (not mixed across heads)."""
    env(chunks=2)
    y, ref = run_case(3, 4, 300, 128, 64, "bf16", np.array([0.95, 0.95, 0.95, 0.95]), 13, False, False)
    assert len(set(np.round(ref, 6).tolist())) == 4


D = 128


def _dev(B, H, N, seed=0):
    return [device_stream(seed, i, (B, H, N, D), "bf16") for i in (synth.ID_Q, synth.ID_K, synth.ID_V, synth.ID_DO)]


def _pair(B, H, N, b, h, seed=0):
    return [synth.bf16_bits_to_f64(synth.pair_slice(seed, i, B, H, N, D, b, h, "bf16"))
            for i in (synth.ID_Q, synth.ID_K, synth.ID_V, synth.ID_DO)]


@pytest.mark.parametrize("B,H,N,heads", [(2, 32, 8192, [0, 13, 31]), (2, 16, 65536, [0, 15])])
def test_dlam_training_sizes(B, H, N, heads):
    """The training step's shapes (B=2 H=32 N=8192, and the 64K point of the 131072-token sweep):
    sampled heads, each against the oracle summed over the batch."""
    print(f"[dlam] workload B={B} H={H} N={N} Bk=64 heads={heads}", flush=True)
    lam = synth.decay_schedule(H)
    q, k, v, g = _dev(B, H, N)
    out = la.la_dlam(q, k, v, g, lam, Bk=64)
    torch.cuda.synchronize()
    y = got(out)
    assert np.all(np.isfinite(y))
    for h in heads:
        per = [oracle.dlam_recurrent(*_pair(B, H, N, b, h), float(lam[h])) for b in range(B)]
        ref = float(np.sum(per))
        err = abs(y[h] - ref) / float(np.sum(np.abs(per)))
        print(f"    h={h} lam={lam[h]:.5f} dlam={y[h]:.6e} oracle={ref:.6e} rel {err:.2e}", flush=True)
        assert err <= BF16_BAR
