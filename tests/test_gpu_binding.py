"""Every caller-supplied tensor of every binding entry point is checked before the library is
called: device (a CPU tensor where device memory is expected), exact shape, dtype and
contiguity.  Each case raises ValueError; nothing is launched, so a bad buffer can never
reach a kernel as a bare pointer."""
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import causal_linear_attention_tiled_amd as la  # noqa: E402

B, H, N, D = 1, 2, 70, 128
LAM = [0.5, 0.9]


def dev(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype, device="cuda")


def bad_variants(t):
    """A CPU copy, a wrong shape, a wrong dtype and a non-contiguous view of t."""
    out = [("cpu", t.cpu())]
    out.append(("shape", torch.zeros(*t.shape[:-1], t.shape[-1] + 1, dtype=t.dtype, device=t.device)))
    other = torch.float64 if t.dtype != torch.float64 else torch.float32
    out.append(("dtype", torch.zeros(t.shape, dtype=other, device=t.device)))
    if t.dim() >= 2 and t.shape[-1] > 1 and t.shape[-2] > 1:
        out.append(("stride", t.transpose(-1, -2).contiguous().transpose(-1, -2)))
    return out


def seq():
    return dev(B, H, N, D)


def state():
    return dev(B, H, D, D, dtype=torch.float32)


def calls():
    """(entry point, argument name, valid arguments, call(args))."""
    fwd_args = dict(q=seq(), k=seq(), v=seq(), kv_in=state(), out=seq(), kv_out=state())
    yield "la_fwd", fwd_args, lambda a: la.la_fwd(a["q"], a["k"], a["v"], LAM, kv_in=a["kv_in"], out=a["out"],
                                                  kv_out=a["kv_out"])
    bwd_args = dict(q=seq(), k=seq(), v=seq(), g=seq(), kv_in=state(), dkv_out=state(), dq=seq(), dk=seq(),
                    dv=seq(), dkv_in=state())
    yield "la_bwd", bwd_args, lambda a: la.la_bwd(a["q"], a["k"], a["v"], a["g"], LAM, kv_in=a["kv_in"],
                                                  dkv_out=a["dkv_out"], dq=a["dq"], dk=a["dk"], dv=a["dv"],
                                                  dkv_in=a["dkv_in"])
    dlam_args = dict(q=seq(), k=seq(), v=seq(), g=seq(), kv_in=state(), dkv_out=state(),
                     out=dev(H, dtype=torch.float32))
    yield "la_dlam", dlam_args, lambda a: la.la_dlam(a["q"], a["k"], a["v"], a["g"], LAM, kv_in=a["kv_in"],
                                                     dkv_out=a["dkv_out"], out=a["out"])
    T = 70
    vl_args = dict(q=dev(T, H, D), k=dev(T, H, D), v=dev(T, H, D), kv_in=dev(2, H, D, D, dtype=torch.float32),
                   out=dev(T, H, D), kv_out=dev(2, H, D, D, dtype=torch.float32))
    yield "la_fwd_varlen", vl_args, lambda a: la.la_fwd_varlen(a["q"], a["k"], a["v"], LAM, [0, 30, T],
                                                               kv_in=a["kv_in"], out=a["out"],
                                                               kv_out=a["kv_out"])
    dc_args = dict(state=dev(3, H, D, D, dtype=torch.float32), q=dev(3, H, D), k=dev(3, H, D), v=dev(3, H, D),
                   out=dev(3, H, D))
    yield "la_decode_step", dc_args, lambda a: la.la_decode_step(a["state"], a["q"], a["k"], a["v"], LAM,
                                                                 out=a["out"])
    pg_args = dict(pool=dev(5, H, D, D, dtype=torch.float32),
                   slot_of=torch.tensor([4, 0, 2], dtype=torch.int32, device="cuda"), q=dev(3, H, D),
                   k=dev(3, H, D), v=dev(3, H, D), out=dev(3, H, D))
    yield "la_decode_step_paged", pg_args, lambda a: la.la_decode_step_paged(a["pool"], a["slot_of"], a["q"],
                                                                             a["k"], a["v"], LAM, out=a["out"])


def test_valid_calls_run():
    for name, args, call in calls():
        call(args)
    torch.cuda.synchronize()


@pytest.mark.parametrize("entry", ["la_fwd", "la_bwd", "la_dlam", "la_fwd_varlen", "la_decode_step",
                                   "la_decode_step_paged"])
def test_every_argument_checked(entry):
    (name, args, call), = [c for c in calls() if c[0] == entry]
    for arg in args:
        # the first operand fixes shape and dtype of the rest, so its own shape/dtype changes
        # can be consistent; its device and layout are still checked
        for kind, badt in bad_variants(args[arg]):
            if arg in ("q", "pool") and kind in ("shape", "dtype"):
                continue
            bad = dict(args)
            bad[arg] = badt
            print(f"[binding] {entry} {arg} {kind}", flush=True)
            with pytest.raises((ValueError, TypeError)):
                call(bad)


def test_workspaces_checked():
    q = seq()
    with pytest.raises(ValueError):
        la.la_fwd(q, q.clone(), q.clone(), LAM, ws=torch.zeros(1 << 20, dtype=torch.uint8))   # host memory
    with pytest.raises(ValueError):
        la.la_bwd(q, q.clone(), q.clone(), q.clone(), LAM, fwd_ws=torch.zeros(16, dtype=torch.uint8))
    nb = la.la_bwd_workspace_bytes(B, H, 64 * 64, D, 64, la.LA_BF16)
    big = dev(B, H, 64 * 64, D)
    if nb:
        with pytest.raises(ValueError):
            la.la_bwd(big, big.clone(), big.clone(), big.clone(), LAM,
                      ws=torch.zeros(nb - 1, dtype=torch.uint8, device="cuda"))
