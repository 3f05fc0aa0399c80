"""Binding of the beam-decode attention over a shared context KV
(include/hstu_beam.h).  Argument marshalling only: the attention runs in the
HIP kernels of libhstu."""
from __future__ import annotations

import ctypes

from . import _lib

P, I32 = ctypes.c_void_p, ctypes.c_int32


class BeamDesc(ctypes.Structure):
    _fields_ = [
        ("num_requests", I32),
        ("beam_width", I32),
        ("num_q_heads", I32),
        ("num_kv_heads", I32),
        ("head_dim", I32),
        ("max_ctx", I32),
        ("step", I32),
        ("max_steps", I32),
        ("scale", ctypes.c_float),
        ("dtype", I32),
    ]


_bound = None


def _lib_beam() -> ctypes.CDLL:
    global _bound
    lib = _lib.load()
    if _bound is lib:
        return lib
    lib.hstu_beam_workspace_size.argtypes = [ctypes.POINTER(BeamDesc), ctypes.POINTER(ctypes.c_size_t)]
    lib.hstu_beam_workspace_size.restype = I32
    lib.hstu_beam_decode_attn.argtypes = [ctypes.POINTER(BeamDesc)] + [P] * 9 + [ctypes.c_size_t, P]
    lib.hstu_beam_decode_attn.restype = I32
    _bound = lib
    return lib


def make_desc(q, ctx_k, beam_k, step: int, scale: float) -> BeamDesc:
    """Descriptor from the tensors' shapes: q [R, W, Hq, d], ctx_k [R, Hkv,
    max_ctx, d], beam_k [R, max_steps, W, Hkv, d]."""
    import torch
    R, W, Hq, d = (int(v) for v in q.shape)
    return BeamDesc(num_requests=R, beam_width=W, num_q_heads=Hq, num_kv_heads=int(ctx_k.shape[1]), head_dim=d,
                    max_ctx=int(ctx_k.shape[2]), step=int(step), max_steps=int(beam_k.shape[1]), scale=float(scale),
                    dtype=_lib.HSTU_BF16 if q.dtype == torch.bfloat16 else _lib.HSTU_F32)


def workspace_size(desc: BeamDesc) -> int:
    n = ctypes.c_size_t(0)
    rc = _lib_beam().hstu_beam_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if rc != 0:
        raise _lib.HSTUError(rc, "hstu_beam_workspace_size")
    return int(n.value)


def decode_attn(q, ctx_k, ctx_vt, ctx_len, beam_k, beam_v, path, out, step: int, scale: float,
                workspace=None, stream=None):
    """Enqueue one decode step's attention (include/hstu_beam.h).  Returns the
    workspace (its first int32 is the device status word)."""
    import torch
    desc = make_desc(q, ctx_k, beam_k, step, scale)
    need = workspace_size(desc)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    dt = q.dtype
    rc = _lib_beam().hstu_beam_decode_attn(
        ctypes.byref(desc), _lib._ptr(q, "q", dt), _lib._ptr(ctx_k, "ctx_k", dt), _lib._ptr(ctx_vt, "ctx_vt", dt),
        _lib._ptr(ctx_len, "ctx_len", torch.int32), _lib._ptr(beam_k, "beam_k", dt), _lib._ptr(beam_v, "beam_v", dt),
        _lib._ptr(path, "path", torch.int32, allow_none=step == 0), _lib._ptr(out, "out", dt),
        _lib._ptr(workspace, "workspace"), ctypes.c_size_t(workspace.numel()), _lib._stream(stream))
    if rc != 0:
        raise _lib.HSTUError(rc, "hstu_beam_decode_attn")
    return workspace
