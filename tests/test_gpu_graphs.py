"""The library's calls captured in a HIP graph (through torch.cuda.CUDAGraph) and
replayed: every replay, with eager work and synchronisations between replays,
must equal the eager calls bit for bit (the kernels are deterministic and
launch no memsets or copies, so a capture records kernels only)."""
import math

import numpy as np
import pytest

import synth
from helpers import state_input

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import causal_linear_attention_tiled_amd as la  # noqa: E402

D = 128


def dev_normal(seed, sid, shape):
    bits = synth.normal(seed, sid, shape, 1.0 / math.sqrt(D), "bf16")
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def test_training_step_graph_replays_match_eager():
    """la_fwd + la_bwd of a chunked shape (B=2, H=4, N=4096: several chunks per sequence,
    forward chunk states reused by the backward) captured once, replayed three times."""
    B, H, N = 2, 4, 4096
    print(f"[graph] training step B={B} H={H} N={N}", flush=True)
    lam = synth.decay_schedule(H)
    q, k, v, g = (dev_normal(3, sid, (B, H, N, D)) for sid in (1, 2, 3, 4))
    outs = [torch.empty_like(q) for _ in range(4)]
    s_out = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    ds0 = torch.empty_like(s_out)
    wf = la.la_fwd_workspace_bytes(B, H, N, D, 64, la.LA_BF16)
    wb = la.la_bwd_workspace_bytes(B, H, N, D, 64, la.LA_BF16)
    assert wf > 0, "the shape must be chunked"
    ws_f = torch.empty(wf, dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(wb, dtype=torch.uint8, device="cuda")
    gf = torch.from_numpy(state_input(4, B, H, D)).cuda()

    def step():
        la.la_fwd(q, k, v, lam, 64, out=outs[0], kv_out=s_out, ws=ws_f)
        la.la_bwd(q, k, v, g, lam, 64, dq=outs[1], dk=outs[2], dv=outs[3], ws=ws_b, fwd_ws=ws_f,
                  dkv_out=gf, dkv_in=ds0)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = [x.clone() for x in outs] + [s_out.clone(), ds0.clone()]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for x in outs + [s_out, ds0]:
            x.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for x, ref in zip(outs + [s_out, ds0], eager):
            assert torch.equal(x, ref), f"replay {rep} differs"


def test_paged_decode_graph_replays_continue_the_recurrence():
    """Four paged decode steps captured once; two replays give the states and outputs of
    eight eager steps over the same inputs."""
    P, Bs, H = 6, 3, 4
    lam = synth.decay_schedule(H)
    pool0 = torch.from_numpy(state_input(8, P, H, D)).cuda()
    slot_of = torch.tensor([4, 0, 2], dtype=torch.int32, device="cuda")
    qkv = [[dev_normal(60 + t, sid, (Bs, H, D)) for sid in (1, 2, 3)] for t in range(4)]
    outs = [torch.empty((Bs, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(4)]

    def steps(pool):
        for t in range(4):
            la.la_decode_step_paged(pool, slot_of, *qkv[t], lam, out=outs[t])

    ref_pool = pool0.clone()
    steps(ref_pool)
    torch.cuda.synchronize()
    first = [o.clone() for o in outs]
    steps(ref_pool)
    torch.cuda.synchronize()
    second = [o.clone() for o in outs]

    pool = pool0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        warm = pool0.clone()
        steps(warm)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps(pool)
    # capture records without running: the pool still holds the initial states
    torch.cuda.synchronize()
    assert torch.equal(pool, pool0)
    for expect in (first, second):
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, expect):
            assert torch.equal(o, e)
    assert torch.equal(pool, ref_pool)
