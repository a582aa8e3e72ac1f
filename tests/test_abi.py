"""The C-ABI library: it loads, exports every declared symbol, and rejects bad arguments.

No test here computes anything on a GPU: every call below fails validation, which
runs before the library touches the HIP runtime.
"""
import ctypes
import os
import re

import pytest

import causal_linear_attention_tiled_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "liblinattn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert {"la_fwd", "la_bwd", "la_decode_step", "la_fwd_workspace_bytes", "la_bwd_workspace_bytes",
            "la_strerror"} <= set(names)
    handle = ctypes.CDLL(la.LIB_PATH)
    for n in names:
        assert hasattr(handle, n), f"{n} declared in liblinattn.h but not exported"
    assert set(names) == set(la.EXPORTS)


def test_version_and_strerror():
    assert la.la_version() >= 10000
    for code in range(8):
        assert isinstance(la.la_strerror(code), str) and la.la_strerror(code)
    assert "unknown" in la.la_strerror(99)


# Fake, 256-byte aligned addresses far apart; validation never dereferences them.
A = 1 << 40
Q_, K_, V_, O_, S_, W_ = (A * (i + 1) for i in range(6))
LAM = (ctypes.c_float * 4)(0.5, 0.9, 1.0, 0.0)


def fwd(**kw):
    args = dict(Q=Q_, K=K_, V=V_, lam=LAM, B=2, H=4, N=1000, D=128, Bk=64, dt=la.LA_BF16, phi=0, kv_in=None,
                O=O_, kv_out=None, ws=W_, ws_bytes=1 << 40, stream=None)
    args.update(kw)
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return la.lib.la_fwd(v(args["Q"]), v(args["K"]), v(args["V"]), args["lam"], args["B"], args["H"],
                         args["N"], args["D"], args["Bk"], args["dt"], args["phi"], v(args["kv_in"]), v(args["O"]),
                         v(args["kv_out"]), v(args["ws"]), args["ws_bytes"], v(args["stream"]))


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), la.LA_EINVAL),
    (dict(O=None), la.LA_EINVAL),
    (dict(lam=None), la.LA_EINVAL),
    (dict(B=0), la.LA_EINVAL),
    (dict(N=-5), la.LA_EINVAL),
    (dict(dt=7), la.LA_EINVAL),
    (dict(phi=3), la.LA_EINVAL),                     # unknown feature map
    (dict(phi=-1), la.LA_EINVAL),
    (dict(D=48), la.LA_EUNSUPPORTED),
    (dict(D=256), la.LA_EUNSUPPORTED),
    (dict(Bk=48), la.LA_EUNSUPPORTED),
    (dict(Bk=512), la.LA_EUNSUPPORTED),
    (dict(Bk=0), la.LA_EINVAL),
    (dict(H=300, lam=(ctypes.c_float * 300)(*([0.5] * 300))), la.LA_EUNSUPPORTED),
    (dict(Q=Q_ + 8), la.LA_EALIGN),
    (dict(kv_out=S_ + 4), la.LA_EALIGN),
    (dict(O=Q_), la.LA_EINVAL),                      # output aliases an input
    (dict(O=K_ + 1024), la.LA_EINVAL),               # output overlaps an input
    (dict(kv_in=S_, kv_out=S_), la.LA_EINVAL),       # kv_out aliases kv_in
    (dict(lam=(ctypes.c_float * 4)(0.5, float("nan"), 1.0, 0.0)), la.LA_EINVAL),
    (dict(lam=(ctypes.c_float * 4)(0.5, 1.5, 1.0, 0.0)), la.LA_EINVAL),
    (dict(lam=(ctypes.c_float * 4)(0.5, -0.1, 1.0, 0.0)), la.LA_EINVAL),
])
def test_fwd_rejects(kw, code):
    assert fwd(**kw) == code


def test_fwd_workspace_checked():
    # one long sequence is split into chunks, so it needs a workspace
    need = la.la_fwd_workspace_bytes(1, 1, 4096, 128, 64, la.LA_BF16)
    assert need > 0
    lam1 = (ctypes.c_float * 1)(0.9)
    assert fwd(B=1, H=1, N=4096, lam=lam1, ws=None, ws_bytes=0) == la.LA_EWORKSPACE
    assert fwd(B=1, H=1, N=4096, lam=lam1, ws_bytes=need - 1) == la.LA_EWORKSPACE
    assert fwd(B=1, H=1, N=4096, lam=lam1, ws=Q_) == la.LA_EINVAL  # workspace aliases Q


def test_workspace_sizes():
    # enough sequences to fill the chip: no chunks, no workspace
    assert la.la_fwd_workspace_bytes(128, 16, 1024, 128, 64, la.LA_BF16) == 0
    assert la.la_bwd_workspace_bytes(128, 16, 1024, 128, 64, la.LA_BF16) == 0
    # few long sequences: chunked; the workspace holds (chunks-1) x parts D x D float32 states
    # per sequence, the fused prefix's (chunks-1) aggregates and 4 flags per sequence, then a
    # 256-byte stamp (each region from a 256-byte boundary)
    n = la.la_fwd_workspace_bytes(2, 16, 65536, 128, 64, la.LA_BF16)
    state = 128 * 128 * 4
    assert n == 32 * 7 * state + 32 * 7 * state + 32 * 7 * 4 * 8 + 256
    # the backward holds the forward direction's slots (for its dQ sweep) and the reverse ones
    assert la.la_bwd_workspace_bytes(2, 16, 65536, 128, 64, la.LA_BF16) == 2 * 32 * 7 * state
    # invalid shapes report 0
    assert la.la_fwd_workspace_bytes(0, 16, 1024, 128, 64, la.LA_BF16) == 0
    assert la.la_fwd_workspace_bytes(1, 16, 1024, 100, 64, la.LA_BF16) == 0


def test_bwd_rejects():
    v = ctypes.c_void_p
    lam = (ctypes.c_float * 2)(0.5, 0.5)
    G_ = A * 10
    call = lambda dq, dk, dv, g=G_, gf=None, ds=None: la.lib.la_bwd(
        v(Q_), v(K_), v(V_), v(g), lam, 1, 2, 128, 64, 64, la.LA_BF16, 0, None, v(gf) if gf else None,
        v(dq) if dq else None, v(dk), v(dv), v(ds) if ds else None, None, None, 0, None)
    assert call(None, S_, W_) == la.LA_EINVAL          # dQ missing
    assert call(O_, O_, W_) == la.LA_EINVAL            # dQ and dK alias
    assert call(O_, S_, V_) == la.LA_EINVAL            # dV aliases V
    assert call(O_ + 2, S_, W_) == la.LA_EALIGN
    assert call(O_, S_, W_, g=None) == la.LA_EINVAL    # dO missing
    X_ = A * 11
    assert call(O_, S_, W_, gf=X_ + 4) == la.LA_EALIGN  # dkv_out misaligned
    assert call(O_, S_, W_, ds=X_ + 4) == la.LA_EALIGN  # dkv_in misaligned
    assert call(O_, S_, W_, ds=Q_) == la.LA_EINVAL      # dkv_in aliases Q
    assert call(O_, S_, W_, ds=O_ + 1024) == la.LA_EINVAL  # dkv_in inside dQ
    assert call(O_, S_, W_, gf=X_, ds=X_) == la.LA_EINVAL  # dkv_in aliases dkv_out


def test_bwd_forward_workspace_checked():
    """fwd_ws (the forward pass's chunk states) is an input: aligned, and disjoint from every output."""
    v = ctypes.c_void_p
    lam1 = (ctypes.c_float * 1)(0.9)
    G_, X_, Y_, WB_ = A * 10, A * 11, A * 12, A * 13
    N = 4096  # one long sequence: split into chunks
    assert la.la_fwd_workspace_bytes(1, 1, N, 128, 64, la.LA_BF16) > 0
    call = lambda fws, ws=WB_: la.lib.la_bwd(v(Q_), v(K_), v(V_), v(G_), lam1, 1, 1, N, 128, 64, la.LA_BF16, 0,
                                             None, None, v(O_), v(X_), v(Y_), None, v(fws) if fws else None,
                                             v(ws), 1 << 40, None)
    assert call(WB_ + 8) == la.LA_EALIGN
    assert call(WB_ + 4096) == la.LA_EINVAL            # inside the backward's own workspace
    assert call(X_) == la.LA_EINVAL                    # aliases dK


def test_decode_rejects():
    v = ctypes.c_void_p
    lam = (ctypes.c_float * 2)(0.5, 0.5)
    call = lambda st, o, D=128, dt=la.LA_BF16, lm=lam, phi=0: la.lib.la_decode_step(
        v(st) if st else None, v(Q_), v(K_), v(V_), lm, 4, 2, D, dt, phi, v(o) if o else None, None)
    assert call(None, O_) == la.LA_EINVAL
    assert call(S_, None) == la.LA_EINVAL
    assert call(S_, O_, D=100) == la.LA_EUNSUPPORTED
    assert call(S_, O_, dt=3) == la.LA_EINVAL
    assert call(S_ + 4, O_) == la.LA_EALIGN
    assert call(Q_, O_) == la.LA_EINVAL                # state aliases q
    assert call(S_, O_, lm=(ctypes.c_float * 2)(0.5, 2.0)) == la.LA_EINVAL
    assert call(S_, O_, phi=9) == la.LA_EINVAL


def test_no_device_reported_without_gpu():
    torch = pytest.importorskip("torch")
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: a valid call would run kernels on the fake pointers")
    lam1 = (ctypes.c_float * 1)(0.9)
    assert fwd(B=1, H=1, N=64, lam=lam1, ws=None, ws_bytes=0) == la.LA_ENODEV


def test_python_binding_checks_shapes():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 2, 8, 16)
    with pytest.raises(ValueError):
        la.la_fwd(q, q, q[..., :8].contiguous(), [0.5, 0.5])
    with pytest.raises(ValueError):
        la.la_fwd(q, q, q, [0.5])


def _offs(xs):
    return (ctypes.c_int64 * len(xs))(*xs)


def test_fwd_varlen_rejects():
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    lam = (ctypes.c_float * 2)(0.5, 0.9)

    def call(offs, B=None, H=2, D=128, Bk=64, dt=la.LA_BF16, O=O_, ws=W_, ws_bytes=1 << 40, kv_out=None):
        B = len(offs) - 1 if B is None else B
        return la.lib.la_fwd_varlen(v(Q_), v(K_), v(V_), lam, _offs(offs), B, H, D, Bk, dt, 0, None, v(O),
                                    v(kv_out), v(ws), ws_bytes, None)
    assert call([1, 5, 9]) == la.LA_EINVAL                    # offsets must start at 0
    assert call([0, 9, 5]) == la.LA_EINVAL                    # and not decrease
    assert call([0, 5, 9] + [9] * 300 + [5]) == la.LA_EINVAL  # also in a later group of 256
    # float32 storage, D != 128 and Bk of 16 or 32 take the generic kernels (no workspace):
    # valid arguments get as far as the device query, invalid ones are rejected before it
    assert call([0, 64], dt=la.LA_F32) == la.LA_ENODEV
    assert call([0, 64], D=64) == la.LA_ENODEV
    assert call([0, 64], Bk=32) == la.LA_ENODEV
    assert call([0, 64], D=100) == la.LA_EUNSUPPORTED
    assert call([0, 64], Bk=48) == la.LA_EUNSUPPORTED
    assert call([0, 64], D=64, H=257) == la.LA_EUNSUPPORTED  # 256 heads at most (checked before lambda is read)
    assert call([1, 5, 9], D=64) == la.LA_EINVAL
    assert call([0, 9, 5], dt=la.LA_F32) == la.LA_EINVAL
    assert call([0, 64], D=64, O=Q_) == la.LA_EINVAL
    assert call([0, 64], D=64, O=O_ + 8) == la.LA_EALIGN
    assert call([0, 1 << 31], D=64) == la.LA_EUNSUPPORTED     # int32 token offsets
    assert la.la_fwd_varlen_workspace_bytes([0, 100000], 2, 64, 64, la.LA_BF16) == 0
    assert la.la_fwd_varlen_workspace_bytes([0, 100000], 2, 128, 32, la.LA_F32) == 0
    assert call([0, 64], O=Q_) == la.LA_EINVAL                # output aliases Q
    assert call([0, 64], O=O_ + 8) == la.LA_EALIGN
    assert call([0, 1 << 30]) == la.LA_EUNSUPPORTED           # 32-bit buffer offsets
    big = [0, 100000]
    need = la.la_fwd_varlen_workspace_bytes(big, 2, 128, 64, la.LA_BF16)
    assert need > 0
    assert call(big, ws=None, ws_bytes=0) == la.LA_EWORKSPACE
    assert call(big, ws_bytes=need - 1) == la.LA_EWORKSPACE
    assert la.la_fwd_varlen_workspace_bytes([0, 10, 20], 2, 128, 64, la.LA_BF16) == 0  # one chunk each
    # more than 256 sequences: groups of 256, each with its own workspace slice
    many = [0] + [333 * (i + 1) for i in range(300)]      # 300 short sequences: one chunk each
    assert la.la_fwd_varlen_workspace_bytes(many, 2, 128, 64, la.LA_BF16) == 0
    many[-1] = many[-2] + 200000                              # a long last one, in the second group
    assert la.la_fwd_varlen_workspace_bytes(many, 2, 128, 64, la.LA_BF16) > 0
    for bk in (128, 256):
        nb = la.la_fwd_varlen_workspace_bytes(big, 2, 128, bk, la.LA_BF16)
        assert nb > 0 and call(big, Bk=bk, ws_bytes=nb - 1) == la.LA_EWORKSPACE


def test_decode_paged_rejects():
    v = ctypes.c_void_p
    lam = (ctypes.c_float * 2)(0.5, 0.5)
    IDX_ = A * 12
    call = lambda pool=S_, P=8, idx=IDX_, o=O_, D=128: la.lib.la_decode_step_paged(
        v(pool), P, v(idx) if idx else None, v(Q_), v(K_), v(V_), lam, 4, 2, D, la.LA_BF16, 0, v(o), None)
    assert call(P=0) == la.LA_EINVAL
    assert call(idx=None) == la.LA_EINVAL
    assert call(idx=IDX_ + 4) == la.LA_EALIGN
    assert call(D=100) == la.LA_EUNSUPPORTED
    assert call(o=S_ + 4096) == la.LA_EINVAL                  # output inside the pool
    assert call(idx=S_ + 1024) == la.LA_EINVAL               # slot table inside the pool


def test_dlam_rejects():
    """la_dlam validates like la_bwd; its workspace is never empty (one partial per
    (sequence, chunk)) and its [H] output may sit anywhere 4-byte aligned."""
    v = ctypes.c_void_p
    lam = (ctypes.c_float * 2)(0.5, 0.0)
    G_, X_ = A * 10, A * 11
    need = la.la_dlam_workspace_bytes(1, 2, 128, 64, 64, la.LA_BF16)
    assert need >= 2 * 8
    call = lambda out=O_, ws=W_, nb=1 << 40, g=G_, gf=None, kv=None, lm=lam, phi=0: la.lib.la_dlam(
        v(Q_), v(K_), v(V_), v(g) if g else None, lm, 1, 2, 128, 64, 64, la.LA_BF16, phi, v(kv) if kv else None,
        v(gf) if gf else None, v(out) if out else None, v(ws) if ws else None, nb, None)
    assert call(out=None) == la.LA_EINVAL                 # output missing
    assert call(g=None) == la.LA_EINVAL                   # dO missing
    assert call(ws=None, nb=0) == la.LA_EWORKSPACE        # workspace always needed
    assert call(nb=need - 1) == la.LA_EWORKSPACE
    assert call(out=O_ + 2) == la.LA_EALIGN               # float output misaligned
    assert call(out=Q_ + 64) == la.LA_EINVAL              # output inside Q
    assert call(out=W_ + 64) == la.LA_EINVAL              # output inside the workspace
    assert call(ws=K_) == la.LA_EINVAL                    # workspace aliases K
    assert call(gf=X_ + 4) == la.LA_EALIGN
    assert call(out=X_, gf=X_) == la.LA_EINVAL            # output aliases dkv_out
    assert call(phi=5) == la.LA_EINVAL
    assert call(lm=(ctypes.c_float * 2)(0.5, 1.25)) == la.LA_EINVAL
    assert la.la_dlam_workspace_bytes(1, 2, 128, 100, 64, la.LA_BF16) == 0


def test_plan():
    """The chunk plan: none when the sequences fill the chip (one workgroup per CU), else
    chunks of whole blocks, and the forward aggregates over parts of a chunk when the chunks
    alone would leave the aggregate pass short of workgroups."""
    assert la.la_plan(128, 16, 1024, 128, 64, la.LA_BF16) == {"chunks": 1, "chunk_len": 1024, "agg_parts": 1}
    assert la.la_plan(8, 16, 16384, 128, 64, la.LA_BF16) == {"chunks": 2, "chunk_len": 8192, "agg_parts": 2}
    assert la.la_plan(2, 16, 65536, 128, 64, la.LA_BF16) == {"chunks": 8, "chunk_len": 8192, "agg_parts": 1}
    assert la.la_plan(1, 64, 262144, 128, 128, la.LA_BF16) == {"chunks": 4, "chunk_len": 65536, "agg_parts": 4}
    # 4097 blocks: chunks of 1025 blocks admit no parts, so they grow to 1028 (4 parts of 257),
    # the last chunk keeping 1013
    assert la.la_plan(1, 64, 262208, 128, 64, la.LA_BF16) == {"chunks": 4, "chunk_len": 65792, "agg_parts": 4}
    # whatever the rounding, the chunks cover the sequence, the last one non-empty, in whole parts
    for B, H, N, Bk in [(1, 64, 100000, 64), (1, 64, 262272, 128), (2, 32, 8000, 64), (8, 16, 16320, 64),
                        (1, 16, 77777, 64), (3, 7, 54321, 128), (1, 64, 4 * 16385 * 64 - 192, 64)]:
        p = la.la_plan(B, H, N, 128, Bk, la.LA_BF16)
        assert (p["chunks"] - 1) * p["chunk_len"] < N <= p["chunks"] * p["chunk_len"], (B, H, N, p)
        assert p["chunk_len"] % (p["agg_parts"] * Bk) == 0, (B, H, N, p)
    p = la.la_plan(1, 2, 1000, 64, 32, la.LA_F32)
    assert p["chunks"] > 1 and p["chunk_len"] % 32 == 0 and (p["chunks"] - 1) * p["chunk_len"] < 1000
    # forward workspace: agg_parts float32 D x D slots per chunk boundary per sequence
    # (then the fused prefix's aggregates and flags, and a 256-byte stamp identifying the forward
    # call, checked by la_bwd when given as fwd_ws)
    assert la.la_fwd_workspace_bytes(2, 16, 65536, 128, 64, la.LA_BF16) == \
        2 * 32 * 7 * 128 * 128 * 4 + 32 * 7 * 32 + 256
    with pytest.raises(la.LaError):
        la.la_plan(1, 16, 1024, 100, 64, la.LA_BF16)
    # a 256-token block: chunk boundaries on multiples of 256 (the kernels step 128-token blocks)
    p = la.la_plan(2, 16, 65536, 128, 256, la.LA_BF16)
    assert p["chunks"] > 1 and p["chunk_len"] % 256 == 0 and (p["chunk_len"] // p["agg_parts"]) % 256 == 0
    assert la.la_plan(1, 2, 300, 16, 256, la.LA_F32) == {"chunks": 1, "chunk_len": 512, "agg_parts": 1}
    with pytest.raises(la.LaError):
        la.la_plan(1, 16, 1024, 128, 512, la.LA_BF16)


def test_grid_limit_rejected_before_any_enqueue():
    """A call whose launches would exceed 2^32 threads in one grid dimension (at most
    4194303 workgroups of up to 1024 threads) fails validation with LA_EUNSUPPORTED,
    before the library looks for a device or enqueues anything: here 2^20 x 16 sequences
    of one token each (one workgroup per sequence)."""
    v = ctypes.c_void_p
    lam16 = (ctypes.c_float * 16)(*([0.5] * 16))
    assert fwd(B=1 << 20, H=16, N=1, lam=lam16, ws=None, ws_bytes=0) == la.LA_EUNSUPPORTED
    assert fwd(B=(1 << 18) - 1, H=16, N=1, lam=lam16, ws=None, ws_bytes=0) != la.LA_EUNSUPPORTED
    G_ = A * 10
    rc = la.lib.la_bwd(v(Q_), v(K_), v(V_), v(G_), lam16, 1 << 20, 16, 1, 128, 64, la.LA_BF16, 0, None, None,
                       v(O_), v(A * 20), v(A * 30), None, None, None, 0, None)
    assert rc == la.LA_EUNSUPPORTED
    rc = la.lib.la_dlam(v(Q_), v(K_), v(V_), v(G_), lam16, 1 << 20, 16, 1, 128, 64, la.LA_BF16, 0, None, None,
                        v(O_), v(W_), 1 << 40, None)
    assert rc == la.LA_EUNSUPPORTED
    rc = la.lib.la_decode_step(v(S_), v(Q_), v(K_), v(V_), lam16, 1 << 19, 16, 16, la.LA_BF16, 0, v(O_), None)
    assert rc == la.LA_EUNSUPPORTED
    IDX_ = A * 12
    rc = la.lib.la_decode_step_paged(v(S_), 8, v(IDX_), v(Q_), v(K_), v(V_), lam16, 1 << 19, 16, 16, la.LA_BF16,
                                     0, v(O_), None)
    assert rc == la.LA_EUNSUPPORTED


def test_noalloc_scratch_limit():
    """la_fwd_noalloc rejects, before touching any device, a call whose chunk states exceed
    the static scratch (LA_ESCRATCH), and validates like la_fwd otherwise."""
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    limit = la.la_scratch_bytes()
    assert limit == 64 << 20
    lam = (ctypes.c_float * 64)(*([0.9] * 64))

    def call(B=1, H=64, N=32 * 4 * 64, Q=Q_, O=O_):
        return la.lib.la_fwd_noalloc(v(Q), v(K_), v(V_), lam, B, H, N, 128, 64, la.LA_BF16, 0, None, v(O),
                                     None, None)
    import os
    old = os.environ.get("LA_CHUNKS")
    try:
        os.environ["LA_CHUNKS"] = "32"          # 64 sequences x 31 chunk states x 64 KiB = 124 MiB
        assert la.la_fwd_workspace_bytes(1, 64, 32 * 4 * 64, 128, 64, la.LA_BF16) > limit
        assert call() == la.LA_ESCRATCH
        assert "scratch" in la.la_strerror(la.LA_ESCRATCH)
        os.environ["LA_CHUNKS"] = "8"           # 64 x 7 x 64 KiB = 28 MiB: fits (then no device here)
        assert 0 < la.la_fwd_workspace_bytes(1, 64, 32 * 4 * 64, 128, 64, la.LA_BF16) <= limit
        assert call(Q=None) == la.LA_EINVAL
        assert call(O=Q_) == la.LA_EINVAL        # output aliases an input
        assert call(O=O_ + 8) == la.LA_EALIGN
    finally:
        if old is None:
            os.environ.pop("LA_CHUNKS", None)
        else:
            os.environ["LA_CHUNKS"] = old


def test_trace_prints_the_plan():
    """LA_TRACE=1: a call prints its plan (chunks, chunk length, parts, workgroups, workspace)
    on stderr; host only (la_plan)."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r); import causal_linear_attention_tiled_amd as la; "
            "la.la_plan(2, 16, 65536, 128, 64, la.LA_BF16)") % os.path.dirname(os.path.dirname(la.__file__))
    r = subprocess.run([sys.executable, "-c", code], env=dict(os.environ, LA_TRACE="1"), capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    line = [x for x in r.stderr.splitlines() if x.startswith("[liblinattn] la_plan")]
    assert line, r.stderr
    assert "chunks=8 chunk_len=8192 agg_parts=1 sweep_wgs=256 aggregate_wgs=224" in line[0]
    assert " fused=0 " in line[0]


def test_fused_wait_bound_scales_with_the_chunk():
    """The bound on each wait of the fused prefix grows with the awaited chunk's walk (4096
    polls per 64-token block on a base of 2^17): LA_FUSED=1 fuses chunks of any length, here
    16388 blocks (a walk of tens of ms), where a fixed bound would let the waiting chunks give
    up and return NaN.  By default the fused form takes the plans whose cost model keeps one
    aggregate part, chunks of a few thousand tokens.  Host only (la_plan under LA_TRACE=1)."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(la.__file__))
    code = ("import sys; sys.path.insert(0, %r); import causal_linear_attention_tiled_amd as la; "
            "la.la_plan(1, 64, 4 * 16385 * 64 - 3 * 64, 128, 64, la.LA_BF16); "
            "la.la_plan(4, 16, 2048, 128, 64, la.LA_BF16)") % root
    env = dict(os.environ, LA_TRACE="1")
    for name in ("LA_FUSED", "LA_CHUNKS", "LA_AGG_K"):
        env.pop(name, None)
    fields = {}
    for fused in (None, "1"):
        if fused:
            env["LA_FUSED"] = fused
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr
        lines = [x for x in r.stderr.splitlines() if x.startswith("[liblinattn] la_plan")]
        assert len(lines) == 2, r.stderr
        fields[fused] = [dict(f.split("=", 1) for f in x.split() if "=" in f) for x in lines]
    (long_, short), (long_forced, _) = fields[None], fields["1"]
    # the long chunks: 4 parts (the chunk grown from 16385 to 16388 blocks), not fused by default
    assert (long_["chunks"], long_["chunk_len"], long_["agg_parts"], long_["fused"]) == ("4", str(16388 * 64), "4", "0")
    assert long_forced["fused"] == "1"
    assert int(long_forced["fused_spin"]) == (1 << 17) + 4096 * 16388
    assert (short["chunks"], short["chunk_len"], short["agg_parts"], short["fused"]) == ("4", "512", "1", "1")
    assert int(short["fused_spin"]) == (1 << 17) + 4096 * 8