"""gated_delta_rule_100_amd -- the gated delta rule on AMD Instinct MI355X.

Python binding of libgdr.so (the C ABI declared in include/gdr.h).  It only
marshals arguments: it takes torch device tensors (torch is used for device
memory and streams), checks their dtype/shape/placement, and passes raw
pointers and sizes to the library.  Every step of the computation runs in the
HIP kernels of libgdr; there is no CPU path.  If the library is not built, or
a tensor is not on the GPU, the call raises.

    S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t,
    alpha_t = exp(g_t), state S of shape dv x dk per (sequence, head).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "GdrError",
    "GDR_BF16",
    "GDR_FP32",
    "library_path",
    "gdr_decode_step",
    "gdr_decode_mtp",
    "gdr_chunk_prefill",
    "gdr_chunk_prefill_noalloc",
    "gdr_chunk_prefill_workspace_bytes",
    "gdr_state_fixup",
    "gdr_chunk_layout",
    "gdr_max_chunks",
    "gdr_status_string",
    "gdr_last_error",
]

GDR_BF16 = 0
GDR_FP32 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgdr.so")
_lib = None


class GdrError(RuntimeError):
    """A libgdr call returned a non-OK status."""


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise GdrError(f"{_LIB_PATH} is missing: build it with gated_delta_rule_100_amd/build.py "
                       "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.gdr_decode_step.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P]
    lib.gdr_decode_mtp.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P]
    lib.gdr_decode_step.restype = I
    lib.gdr_decode_mtp.restype = I
    lib.gdr_max_chunks.argtypes = [I, I, I]
    lib.gdr_max_chunks.restype = I
    lib.gdr_chunk_layout.argtypes = [P, I, I, P, P, I, P]
    lib.gdr_chunk_layout.restype = I
    lib.gdr_chunk_prefill_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.gdr_chunk_prefill_workspace_bytes.restype = S
    lib.gdr_chunk_prefill.argtypes = [P, P, P, P, P, P, I, P, P, P, P, P, P,
                                      I, I, I, I, I, I, I, P, S, P]
    lib.gdr_chunk_prefill.restype = I
    lib.gdr_chunk_prefill_noalloc.argtypes = [P, P, P, P, P, P, I, P, P, P, P, P, P,
                                              I, I, I, I, I, I, I, P]
    lib.gdr_chunk_prefill_noalloc.restype = I
    lib.gdr_state_fixup.argtypes = [P, P, P, P, I, P, I, I, I, I, P]
    lib.gdr_state_fixup.restype = I
    lib.gdr_status_string.argtypes = [I]
    lib.gdr_status_string.restype = ctypes.c_char_p
    lib.gdr_last_error.argtypes = []
    lib.gdr_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def gdr_status_string(status: int) -> str:
    return _load().gdr_status_string(status).decode()


def gdr_last_error() -> str:
    return _load().gdr_last_error().decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise GdrError(f"{what}: {gdr_status_string(status)}: {gdr_last_error()}")


def _dev_ptr(t, name, dtypes=None, optional=False):
    if t is None:
        if optional:
            return None
        raise GdrError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise GdrError(f"{name} must be a torch tensor on the GPU")
    if not t.is_contiguous():
        raise GdrError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise GdrError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t.data_ptr()


def _code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return GDR_BF16
    if dt == torch.float32:
        return GDR_FP32
    raise GdrError(f"unsupported dtype {dt}")


def _stream_obj(stream):
    """The launch stream as a torch stream (a raw hipStream_t handle is wrapped)."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


_IO = (torch.bfloat16, torch.float32)
_F32 = (torch.float32,)
_I32 = (torch.int32,)


def gdr_decode_step(q, k, v, g, beta, state, o, stream=None) -> None:
    """One decode token, state updated in place.  q, k [N, H, dk], v [N, H, dv]
    (bf16 or fp32, one dtype); g, beta [N, H] fp32; state [N, H, dv, dk] fp32;
    o [N, H, dv] bf16 or fp32."""
    N, H, dk = q.shape
    dv = v.shape[2]
    if k.shape != q.shape or v.shape[:2] != (N, H) or g.shape != (N, H) or beta.shape != (N, H) \
            or state.shape != (N, H, dv, dk) or o.shape != (N, H, dv):
        raise GdrError("gdr_decode_step: inconsistent shapes")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise GdrError("gdr_decode_step: q, k, v must share a dtype")
    st = _load().gdr_decode_step(
        _dev_ptr(q, "q", _IO), _dev_ptr(k, "k", _IO), _dev_ptr(v, "v", _IO),
        _dev_ptr(g, "g", _F32), _dev_ptr(beta, "beta", _F32), _dev_ptr(state, "state", _F32),
        _dev_ptr(o, "o", _IO), N, H, dk, dv, _code(q.dtype), _code(o.dtype), _stream(stream))
    _check(st, "gdr_decode_step")


def gdr_decode_mtp(q, k, v, g, beta, state_in, state_out, o, inter=None, stream=None) -> None:
    """T decode tokens per (sequence, head).  q, k [N, T, H, dk], v [N, T, H, dv]
    (bf16 or fp32, one dtype); g, beta [N, T, H] fp32; state_in [N, H, dv, dk]
    fp32; state_out like state_in, the same tensor (in place) or None (no final
    state written); o [N, T, H, dv] bf16 or fp32; inter [N, T, H, dv, dk] fp32
    or None (the state after every token)."""
    N, T, H, dk = q.shape
    dv = v.shape[3]
    if k.shape != q.shape or v.shape[:3] != (N, T, H) or g.shape != (N, T, H) \
            or beta.shape != (N, T, H) or state_in.shape != (N, H, dv, dk) \
            or o.shape != (N, T, H, dv) \
            or (state_out is not None and state_out.shape != state_in.shape) \
            or (inter is not None and inter.shape != (N, T, H, dv, dk)):
        raise GdrError("gdr_decode_mtp: inconsistent shapes")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise GdrError("gdr_decode_mtp: q, k, v must share a dtype")
    st = _load().gdr_decode_mtp(
        _dev_ptr(q, "q", _IO), _dev_ptr(k, "k", _IO), _dev_ptr(v, "v", _IO),
        _dev_ptr(g, "g", _F32), _dev_ptr(beta, "beta", _F32),
        _dev_ptr(state_in, "state_in", _F32), _dev_ptr(state_out, "state_out", _F32, optional=True),
        _dev_ptr(o, "o", _IO), _dev_ptr(inter, "inter", _F32, optional=True), N, T, H, dk, dv,
        _code(q.dtype), _code(o.dtype), _stream(stream))
    _check(st, "gdr_decode_mtp")


def gdr_max_chunks(T_total: int, N: int, chunk: int) -> int:
    return int(_load().gdr_max_chunks(T_total, N, chunk))


def gdr_chunk_prefill_workspace_bytes(T_total, N, H, dk, dv, chunk, in_dtype=GDR_BF16) -> int:
    """in_dtype: GDR_BF16 / GDR_FP32 or the torch dtype of q, k, v."""
    if isinstance(in_dtype, torch.dtype):
        in_dtype = _code(in_dtype)
    return int(_load().gdr_chunk_prefill_workspace_bytes(T_total, N, H, dk, dv, chunk, in_dtype))


def gdr_chunk_layout(cu_seqlens, chunk, chunk_offsets, chunk_indices, stream=None) -> None:
    """cu_seqlens [N+1] int32 -> chunk_offsets [N+1] int32, chunk_indices
    [max_chunks, 2] int32 (rows past the real count = (-1, -1))."""
    N = cu_seqlens.shape[0] - 1
    if chunk_offsets.shape != (N + 1,) or chunk_indices.dim() != 2 or chunk_indices.shape[1] != 2:
        raise GdrError("gdr_chunk_layout: inconsistent shapes")
    st = _load().gdr_chunk_layout(
        _dev_ptr(cu_seqlens, "cu_seqlens", _I32), N, chunk,
        _dev_ptr(chunk_offsets, "chunk_offsets", _I32),
        _dev_ptr(chunk_indices, "chunk_indices", _I32), chunk_indices.shape[0], _stream(stream))
    _check(st, "gdr_chunk_layout")


def _prefill_args(q, k, v, g, beta, cu_seqlens, state_in, state_out, o, chunk, L_out, M_out,
                  fixed_out, who):
    """Checks the shapes and dtypes of a prefill call; returns the pointer and
    size arguments shared by gdr_chunk_prefill and gdr_chunk_prefill_noalloc
    (everything up to out_dtype) and (T, N, H, dk, dv)."""
    T, H, dk = q.shape
    dv = v.shape[2]
    N = cu_seqlens.shape[0] - 1
    if k.shape != q.shape or v.shape[:2] != (T, H) or g.shape != (T, H) or beta.shape != (T, H) \
            or state_out.shape != (N, H, dv, dk) or o.shape != (T, H, dv) \
            or (state_in is not None and state_in.shape != (N, H, dv, dk)):
        raise GdrError(f"{who}: inconsistent shapes")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise GdrError(f"{who}: q, k, v must share a dtype")
    mc = gdr_max_chunks(T, N, chunk)
    for name, t, shape in (("L_out", L_out, (mc, H, dv, dk)), ("M_out", M_out, (mc, H, dk, dk)),
                           ("fixed_out", fixed_out, (mc, H, dv, dk))):
        if t is not None and tuple(t.shape) != shape:
            raise GdrError(f"{who}: {name} must have shape {shape}")
    args = [
        _dev_ptr(q, "q", _IO), _dev_ptr(k, "k", _IO), _dev_ptr(v, "v", _IO),
        _dev_ptr(g, "g", _F32), _dev_ptr(beta, "beta", _F32),
        _dev_ptr(cu_seqlens, "cu_seqlens", _I32), N,
        _dev_ptr(state_in, "state_in", _F32, optional=True),
        _dev_ptr(state_out, "state_out", _F32), _dev_ptr(o, "o", _IO),
        _dev_ptr(L_out, "L_out", _F32, optional=True), _dev_ptr(M_out, "M_out", _F32, optional=True),
        _dev_ptr(fixed_out, "fixed_out", _F32, optional=True),
        T, H, dk, dv, chunk, _code(q.dtype), _code(o.dtype)]
    return args, (T, N, H, dk, dv)


def gdr_chunk_prefill(q, k, v, g, beta, cu_seqlens, state_in, state_out, o, *, chunk=64,
                      L_out=None, M_out=None, fixed_out=None, workspace=None,
                      stream=None) -> None:
    """Chunked prefill over packed sequences.  q, k [T, H, dk], v [T, H, dv];
    g, beta [T, H] fp32; cu_seqlens [N+1] int32 (device); state_in
    [N, H, dv, dk] fp32 or None; state_out [N, H, dv, dk] fp32; o [T, H, dv];
    optional L_out / fixed_out [max_chunks, H, dv, dk], M_out [max_chunks, H,
    dk, dk] with max_chunks = gdr_max_chunks(T, N, chunk); M_out[c, h] is M_c
    with S_end = S_start @ M_c + L_c.  workspace: a uint8 device tensor of
    gdr_chunk_prefill_workspace_bytes(...) bytes, or None to allocate one here
    (on the launch stream, so that the caching allocator does not hand its
    memory to work on another stream while the kernels still use it)."""
    args, (T, N, H, dk, dv) = _prefill_args(q, k, v, g, beta, cu_seqlens, state_in, state_out, o,
                                            chunk, L_out, M_out, fixed_out, "gdr_chunk_prefill")
    if workspace is None:
        need = gdr_chunk_prefill_workspace_bytes(T, N, H, dk, dv, chunk, q.dtype)
        with torch.cuda.stream(_stream_obj(stream)):
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = _load().gdr_chunk_prefill(
        *args, _dev_ptr(workspace, "workspace", (torch.uint8,)), workspace.numel(),
        _stream(stream))
    _check(st, "gdr_chunk_prefill")


def gdr_chunk_prefill_noalloc(q, k, v, g, beta, cu_seqlens, state_in, state_out, o, *, chunk=64,
                              L_out=None, M_out=None, fixed_out=None, stream=None) -> None:
    """gdr_chunk_prefill on the library's static device scratch: no workspace
    argument and no allocation, for callers that cannot allocate (e.g. under
    HIP graph capture).  Same arguments and results as gdr_chunk_prefill; a
    call that needs more than the scratch holds raises GdrError.  Calls that
    overlap on one device share the scratch and race."""
    args, _ = _prefill_args(q, k, v, g, beta, cu_seqlens, state_in, state_out, o, chunk, L_out,
                            M_out, fixed_out, "gdr_chunk_prefill_noalloc")
    st = _load().gdr_chunk_prefill_noalloc(*args, _stream(stream))
    _check(st, "gdr_chunk_prefill_noalloc")


def gdr_state_fixup(L, M, state_in, chunk_offsets, fixed, stream=None) -> None:
    """fixed[c] = fixed[c-1] @ M_c + L_c over each sequence's chunk slots.
    L, fixed [n_chunks, H, dv, dk], M [n_chunks, H, dk, dk] fp32 (M[c, h] = M_c);
    state_in [N, H, dv, dk] fp32 or None; chunk_offsets [N+1] int32 (device)."""
    n_chunks, H, dv, dk = L.shape
    N = chunk_offsets.shape[0] - 1
    if M.shape != (n_chunks, H, dk, dk) or fixed.shape != L.shape or \
            (state_in is not None and state_in.shape != (N, H, dv, dk)):
        raise GdrError("gdr_state_fixup: inconsistent shapes")
    st = _load().gdr_state_fixup(
        _dev_ptr(L, "L", _F32), _dev_ptr(M, "M", _F32),
        _dev_ptr(state_in, "state_in", _F32, optional=True),
        _dev_ptr(chunk_offsets, "chunk_offsets", _I32), N, _dev_ptr(fixed, "fixed", _F32),
        n_chunks, H, dk, dv, _stream(stream))
    _check(st, "gdr_state_fixup")
