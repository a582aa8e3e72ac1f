"""Python binding of liblinattn (tiled causal linear attention with per-head decay, gfx950).

Argument marshalling only: every function here checks tensor types, takes device
pointers and the current HIP stream from PyTorch, and calls the C entry point of
the same name in ``liblinattn.so`` (declared in ``include/liblinattn.h``).  All
arithmetic runs in the library's HIP kernels; there is no fallback.  If the
shared library is missing or fails to load, importing this package raises.

Layouts: Q, K, V, O, dO, dQ, dK, dV are contiguous [B, H, N, D] tensors of
dtype float32 or bfloat16 on one GPU; states are contiguous [B, H, D, D]
float32; ``lam`` is a sequence (or CPU tensor / array) of H floats in [0, 1].
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# LA_SANITIZE=1 loads the build whose host code carries AddressSanitizer and UBSan
# (tests/sanitize_host.py); its kernels are the same.
LIB_PATH = os.path.join(_HERE, "liblinattn_san.so" if os.environ.get("LA_SANITIZE") == "1" else "liblinattn.so")

LA_F32, LA_BF16 = 0, 1
LA_PHI_IDENTITY, LA_PHI_ELU1, LA_PHI_RELU = 0, 1, 2
PHI_CODES = {"identity": LA_PHI_IDENTITY, "elu1": LA_PHI_ELU1, "relu": LA_PHI_RELU}


def _phi_code(phi) -> int:
    if isinstance(phi, str):
        if phi not in PHI_CODES:
            raise ValueError(f"unknown feature map {phi!r}; one of {sorted(PHI_CODES)}")
        return PHI_CODES[phi]
    return int(phi)
LA_OK, LA_EINVAL, LA_EUNSUPPORTED, LA_EALIGN, LA_EWORKSPACE, LA_EHIP, LA_ENODEV, LA_ESCRATCH = range(8)


class LaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: status {code}: {la_strerror(code)}")


class la_prof_entry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"liblinattn.so is not built ({LIB_PATH}); run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    fp = ctypes.POINTER(ctypes.c_float)
    lib.la_fwd.argtypes = [vp, vp, vp, fp, i64, i64, i64, i64, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.la_fwd.restype = ctypes.c_int
    lib.la_fwd_noalloc.argtypes = [vp, vp, vp, fp, i64, i64, i64, i64, i32, i32, i32, vp, vp, vp, vp]
    lib.la_fwd_noalloc.restype = ctypes.c_int
    lib.la_scratch_bytes.argtypes = []
    lib.la_scratch_bytes.restype = sz
    lib.la_fwd_workspace_bytes.argtypes = [i64, i64, i64, i64, i32, i32]
    lib.la_fwd_workspace_bytes.restype = sz
    lib.la_bwd.argtypes = [vp, vp, vp, vp, fp, i64, i64, i64, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.la_bwd.restype = ctypes.c_int
    lib.la_plan.argtypes = [i64, i64, i64, i64, i32, i32, vp, vp, vp]
    lib.la_plan.restype = ctypes.c_int
    lib.la_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, i32, i32]
    lib.la_bwd_workspace_bytes.restype = sz
    lib.la_dlam.argtypes = [vp, vp, vp, vp, fp, i64, i64, i64, i64, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.la_dlam.restype = ctypes.c_int
    lib.la_dlam_workspace_bytes.argtypes = [i64, i64, i64, i64, i32, i32]
    lib.la_dlam_workspace_bytes.restype = sz
    lib.la_decode_step.argtypes = [vp, vp, vp, vp, fp, i64, i64, i64, i32, i32, vp, vp]
    lib.la_decode_step.restype = ctypes.c_int
    ip = ctypes.POINTER(ctypes.c_int64)
    lib.la_fwd_varlen.argtypes = [vp, vp, vp, fp, ip, i64, i64, i64, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.la_fwd_varlen.restype = ctypes.c_int
    lib.la_fwd_varlen_workspace_bytes.argtypes = [ip, i64, i64, i64, i32, i32]
    lib.la_fwd_varlen_workspace_bytes.restype = sz
    lib.la_decode_step_paged.argtypes = [vp, i64, vp, vp, vp, vp, fp, i64, i64, i64, i32, i32, vp, vp]
    lib.la_decode_step_paged.restype = ctypes.c_int
    lib.la_strerror.argtypes = [ctypes.c_int]
    lib.la_strerror.restype = ctypes.c_char_p
    lib.la_version.restype = ctypes.c_int
    lib.la_prof_enable.argtypes = [ctypes.c_int]
    lib.la_prof_collect.argtypes = [ctypes.POINTER(la_prof_entry), ctypes.c_int]
    return lib


lib = _load()

EXPORTS = ("la_fwd", "la_fwd_noalloc", "la_scratch_bytes", "la_fwd_workspace_bytes", "la_plan", "la_bwd", "la_bwd_workspace_bytes", "la_dlam",
           "la_dlam_workspace_bytes", "la_decode_step",
           "la_fwd_varlen", "la_fwd_varlen_workspace_bytes", "la_decode_step_paged",
           "la_strerror", "la_version", "la_prof_enable", "la_prof_collect")


def la_strerror(code: int) -> str:
    return lib.la_strerror(code).decode()


def la_version() -> int:
    return lib.la_version()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return LA_F32
    if t.dtype == torch.bfloat16:
        return LA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _lam_array(lam, H: int):
    vals = [float(x) for x in (lam.tolist() if hasattr(lam, "tolist") else lam)]
    if len(vals) != H:
        raise ValueError(f"lam has {len(vals)} values, expected H={H}")
    return (ctypes.c_float * H)(*vals)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_tensor(name, t, shape, dtype, device):
    """A caller-supplied tensor: a contiguous GPU tensor on ``device`` with exactly this shape
    and dtype.  The C ABI receives bare pointers and can check none of this itself."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got one on {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other operands on {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_lead(name, t, dims):
    """The first operand of a call: a contiguous float32 or bfloat16 GPU tensor of ``dims`` dims."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dimensions (got {t.dim()})")
    _check_tensor(name, t, None, None, None)
    _dtype_code(t)


def _check_seq(name, t, ref=None):
    if ref is None:
        _check_lead(name, t, 4)
    else:
        _check_tensor(name, t, ref.shape, ref.dtype, ref.device)


def _check_state(name, t, B, H, D, device):
    if t is not None:
        _check_tensor(name, t, (B, H, D, D), torch.float32, device)


def la_fwd_workspace_bytes(B, H, N, D, Bk, dtype_code) -> int:
    return int(lib.la_fwd_workspace_bytes(B, H, N, D, Bk, dtype_code))


def la_plan(B, H, N, D, Bk, dtype_code) -> dict:
    """The chunk plan of la_fwd / la_bwd for this shape: chunks, chunk_len, agg_parts."""
    c, n, k = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int32()
    rc = lib.la_plan(B, H, N, D, Bk, dtype_code, ctypes.byref(c), ctypes.byref(n), ctypes.byref(k))
    if rc != LA_OK:
        raise LaError(rc, "la_plan")
    return {"chunks": c.value, "chunk_len": n.value, "agg_parts": k.value}


def la_bwd_workspace_bytes(B, H, N, D, Bk, dtype_code) -> int:
    return int(lib.la_bwd_workspace_bytes(B, H, N, D, Bk, dtype_code))


def _check_bytes(name, t, nbytes, device):
    """A caller's byte buffer: contiguous, on ``device``, at least ``nbytes`` long."""
    _check_tensor(name, t, None, None, device)
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} needs {nbytes} bytes (got {t.numel() * t.element_size()})")


def _workspace(nbytes, device, ws):
    if ws is not None:
        _check_bytes("ws", ws, nbytes, device)
        return ws
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def la_fwd(q, k, v, lam, Bk: int = 64, kv_in=None, out=None, kv_out=None, want_state: bool = True,
           ws=None, phi="identity"):
    """O (and the final float32 state) of causal linear attention with per-head decay.

    Returns (O, kv_out); kv_out is None when ``want_state`` is False and none is given."""
    _check_seq("Q", q)
    _check_seq("K", k, q)
    _check_seq("V", v, q)
    B, H, N, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    _check_seq("O", out, q)
    if kv_out is None and want_state:
        kv_out = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    _check_state("kv_in", kv_in, B, H, D, q.device)
    _check_state("kv_out", kv_out, B, H, D, q.device)
    code = _dtype_code(q)
    nbytes = la_fwd_workspace_bytes(B, H, N, D, Bk, code)
    ws = _workspace(nbytes, q.device, ws)
    rc = lib.la_fwd(_ptr(q), _ptr(k), _ptr(v), _lam_array(lam, H), B, H, N, D, Bk, code, _phi_code(phi), _ptr(kv_in),
                    _ptr(out), _ptr(kv_out), _ptr(ws), nbytes if ws is not None else 0, _stream(q.device))
    if rc != LA_OK:
        raise LaError(rc, "la_fwd")
    return out, kv_out


def la_scratch_bytes() -> int:
    return int(lib.la_scratch_bytes())


def la_fwd_noalloc(q, k, v, lam, out, Bk: int = 64, kv_in=None, kv_out=None, phi="identity"):
    """la_fwd without a workspace, for callers that cannot allocate: the chunk states go to
    the library's static per-device scratch (la_scratch_bytes()).  The caller passes the
    output O (and kv_out, or None to skip the final state); nothing is allocated here.
    Calls overlapping in time on one device race (they share the scratch)."""
    _check_seq("Q", q)
    _check_seq("K", k, q)
    _check_seq("V", v, q)
    _check_seq("O", out, q)
    B, H, N, D = q.shape
    _check_state("kv_in", kv_in, B, H, D, q.device)
    _check_state("kv_out", kv_out, B, H, D, q.device)
    rc = lib.la_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _lam_array(lam, H), B, H, N, D, Bk, _dtype_code(q),
                            _phi_code(phi), _ptr(kv_in), _ptr(out), _ptr(kv_out), _stream(q.device))
    if rc != LA_OK:
        raise LaError(rc, "la_fwd_noalloc")
    return out, kv_out


def la_bwd(q, k, v, dout, lam, Bk: int = 64, kv_in=None, dq=None, dk=None, dv=None, ws=None,
           fwd_ws=None, dkv_out=None, dkv_in=None, want_dkv_in: bool = False, phi="identity"):
    """dQ, dK, dV of L = <dO, O> + <dkv_out, S_N> for la_fwd.

    ``dkv_out``: float32 [B, H, D, D] gradient arriving at the final state (None for zero).
    ``dkv_in`` / ``want_dkv_in``: receive the gradient of the initial state; returned as a
    fourth value when either is given.
    ``fwd_ws``: the tensor passed as ``ws`` to the la_fwd call over the same inputs, unchanged
    since; the dQ sweep then takes the chunk states from it instead of recomputing them."""
    for name, t in (("Q", q), ("K", k), ("V", v), ("dO", dout)):
        _check_seq(name, t, q)
    B, H, N, D = q.shape
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dQ", dq), ("dK", dk), ("dV", dv)):
        _check_seq(name, t, q)
    _check_state("kv_in", kv_in, B, H, D, q.device)
    _check_state("dkv_out", dkv_out, B, H, D, q.device)
    if dkv_in is None and want_dkv_in:
        dkv_in = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    _check_state("dkv_in", dkv_in, B, H, D, q.device)
    code = _dtype_code(q)
    nbytes = la_bwd_workspace_bytes(B, H, N, D, Bk, code)
    ws = _workspace(nbytes, q.device, ws)
    if fwd_ws is not None:
        _check_bytes("fwd_ws", fwd_ws, la_fwd_workspace_bytes(B, H, N, D, Bk, code), q.device)
    rc = lib.la_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _lam_array(lam, H), B, H, N, D, Bk, code,
                    _phi_code(phi), _ptr(kv_in), _ptr(dkv_out), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dkv_in), _ptr(fwd_ws),
                    _ptr(ws), nbytes if ws is not None else 0, _stream(q.device))
    if rc != LA_OK:
        raise LaError(rc, "la_bwd")
    if dkv_in is not None:
        return dq, dk, dv, dkv_in
    return dq, dk, dv


def la_dlam_workspace_bytes(B, H, N, D, Bk, dtype_code) -> int:
    return int(lib.la_dlam_workspace_bytes(B, H, N, D, Bk, dtype_code))


def la_dlam(q, k, v, dout, lam, Bk: int = 64, kv_in=None, dkv_out=None, out=None, ws=None, phi="identity"):
    """dL/dlam_h summed over the batch, float32 [H], for L = <dO, O> + <dkv_out, S_N> of la_fwd
    (same inputs, kv_in and feature map)."""
    for name, t in (("Q", q), ("K", k), ("V", v), ("dO", dout)):
        _check_seq(name, t, q)
    B, H, N, D = q.shape
    _check_state("kv_in", kv_in, B, H, D, q.device)
    _check_state("dkv_out", dkv_out, B, H, D, q.device)
    if out is None:
        out = torch.empty(H, dtype=torch.float32, device=q.device)
    _check_tensor("out", out, (H,), torch.float32, q.device)
    code = _dtype_code(q)
    nbytes = la_dlam_workspace_bytes(B, H, N, D, Bk, code)
    ws = _workspace(nbytes, q.device, ws)
    rc = lib.la_dlam(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _lam_array(lam, H), B, H, N, D, Bk, code,
                     _phi_code(phi), _ptr(kv_in), _ptr(dkv_out), _ptr(out), _ptr(ws),
                     nbytes if ws is not None else 0, _stream(q.device))
    if rc != LA_OK:
        raise LaError(rc, "la_dlam")
    return out


def _offsets(seq_offsets):
    arr = (ctypes.c_int64 * len(seq_offsets))(*[int(x) for x in seq_offsets])
    return arr, len(seq_offsets) - 1


def la_fwd_varlen_workspace_bytes(seq_offsets, H, D, Bk, dtype_code) -> int:
    arr, B = _offsets(seq_offsets)
    return int(lib.la_fwd_varlen_workspace_bytes(arr, B, H, D, Bk, dtype_code))


def la_fwd_varlen(q, k, v, lam, seq_offsets, Bk: int = 64, kv_in=None, out=None, kv_out=None,
                  want_state: bool = True, ws=None, phi="identity"):
    """Forward over a ragged batch packed token-major: q, k, v [T, H, D] bf16, sequence b is
    rows seq_offsets[b] .. seq_offsets[b+1].  Returns (O [T, H, D], kv_out [B, H, D, D])."""
    _check_lead("Q", q, 3)
    for name, t in (("K", k), ("V", v)):
        _check_tensor(name, t, q.shape, q.dtype, q.device)
    T, H, D = q.shape
    arr, B = _offsets(seq_offsets)
    if arr[B] != T:
        raise ValueError("seq_offsets[-1] must equal the packed token count")
    out = torch.empty_like(q) if out is None else out
    _check_tensor("out", out, q.shape, q.dtype, q.device)
    if kv_out is None and want_state:
        kv_out = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    _check_state("kv_in", kv_in, B, H, D, q.device)
    _check_state("kv_out", kv_out, B, H, D, q.device)
    code = _dtype_code(q)
    nbytes = int(lib.la_fwd_varlen_workspace_bytes(arr, B, H, D, Bk, code))
    ws = _workspace(nbytes, q.device, ws)
    rc = lib.la_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _lam_array(lam, H), arr, B, H, D, Bk, code,
                           _phi_code(phi), _ptr(kv_in),
                           _ptr(out), _ptr(kv_out), _ptr(ws), nbytes if ws is not None else 0, _stream(q.device))
    if rc != LA_OK:
        raise LaError(rc, "la_fwd_varlen")
    return out, kv_out


def la_decode_step_paged(pool, slot_of, q, k, v, lam, out=None, phi="identity"):
    """One recurrent step for Bs sequences whose float32 states live in ``pool``
    [P, H, D, D] at slots ``slot_of`` (int32 [Bs], distinct); q, k, v [Bs, H, D].  Returns o."""
    if not isinstance(pool, torch.Tensor) or pool.dim() != 4:
        raise ValueError("pool must be a float32 [P, H, D, D] tensor")
    P, H, D, _ = pool.shape
    _check_tensor("pool", pool, (P, H, D, D), torch.float32, None)
    _check_lead("q", q, 3)
    Bs = q.shape[0]
    _check_tensor("q", q, (Bs, H, D), None, pool.device)
    _check_tensor("slot_of", slot_of, (Bs,), torch.int32, pool.device)
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, q.shape, q.dtype, q.device)
    out = torch.empty_like(q) if out is None else out
    _check_tensor("out", out, q.shape, q.dtype, q.device)
    rc = lib.la_decode_step_paged(_ptr(pool), P, _ptr(slot_of), _ptr(q), _ptr(k), _ptr(v), _lam_array(lam, H),
                                  Bs, H, D, _dtype_code(q), _phi_code(phi), _ptr(out), _stream(q.device))
    if rc != LA_OK:
        raise LaError(rc, "la_decode_step_paged")
    return out


def la_decode_step(state, q, k, v, lam, out=None, phi="identity"):
    """One recurrent step S <- lam S + k v^T, o = q S; ``state`` [Bs, H, D, D] float32 is updated in place.

    q, k, v are [Bs, H, D]; returns o."""
    _check_lead("q", q, 3)
    Bs, H, D = q.shape
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, q.shape, q.dtype, q.device)
    _check_tensor("state", state, (Bs, H, D, D), torch.float32, q.device)
    out = torch.empty_like(q) if out is None else out
    _check_tensor("out", out, q.shape, q.dtype, q.device)
    rc = lib.la_decode_step(_ptr(state), _ptr(q), _ptr(k), _ptr(v), _lam_array(lam, H), Bs, H, D,
                            _dtype_code(q), _phi_code(phi), _ptr(out), _stream(q.device))
    if rc != LA_OK:
        raise LaError(rc, "la_decode_step")
    return out


def la_prof_enable(on: bool = True) -> None:
    lib.la_prof_enable(1 if on else 0)


def la_prof_collect(max_entries: int = 64) -> dict:
    """{kernel name: (launches, total milliseconds)} since the last collect."""
    arr = (la_prof_entry * max_entries)()
    n = lib.la_prof_collect(arr, max_entries)
    if n < 0:
        raise LaError(-n, "la_prof_collect")
    return {arr[i].name.decode(): (int(arr[i].launches), float(arr[i].total_ms)) for i in range(n)}
