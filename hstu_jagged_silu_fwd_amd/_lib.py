"""ctypes binding of libhstu (argument marshalling only).

Every step of the layer runs in the HIP kernels of libhstu.so; this module
only turns torch tensors into device pointers and the current HIP stream.
There is no fallback: if the library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libhstu.so")
HEADER_PATH = os.path.join(os.path.dirname(PKG), "include", "hstu.h")

HSTU_F32 = 0
HSTU_BF16 = 1
FLAG_BATCH_INVARIANT = 1        # hstu_layer_desc.flags bit (HSTU_FLAG_BATCH_INVARIANT)
INVARIANT_CHUNK_KEYS = 256      # HSTU_INVARIANT_CHUNK_KEYS
NUM_STAGES = 5
STAGES = ("prep", "proj", "attn", "norm", "out")

_lib = None


class HSTUError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = int(code)
        super().__init__(f"{what}: {status_string(code)} ({code})" if what else f"{status_string(code)} ({code})")


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("num_users", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_user", ctypes.c_int32),
        ("num_pool_pages", ctypes.c_int64),
        ("total_new", ctypes.c_int32),
        ("pos_buckets", ctypes.c_int32),
        ("pos_mbits", ctypes.c_int32),
        ("ts_buckets", ctypes.c_int32),
        ("ts_mbits", ctypes.c_int32),
        ("attn_scale", ctypes.c_float),
        ("norm_eps", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("flags", ctypes.c_int32),
    ]


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libhstu.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with `python -m hstu_jagged_silu_fwd_amd.build`")
    # torch ships its own HIP runtime under the same soname (libamdhip64.so.7).
    # Importing torch first makes the loader bind libhstu to that runtime, so
    # torch's device pointers and streams are valid in our calls and only one
    # HIP runtime lives in the process.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    dp = ctypes.POINTER(LayerDesc)
    lib.hstu_layer_workspace_size.argtypes = [dp, ctypes.POINTER(SZ)]
    lib.hstu_layer_workspace_size.restype = I32
    layer_args = [dp, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.hstu_layer_fwd.argtypes = layer_args
    lib.hstu_layer_fwd.restype = I32
    lib.hstu_layer_fwd_timed.argtypes = layer_args + [P]
    lib.hstu_layer_fwd_timed.restype = I32
    lib.hstu_layer_fwd_cand.argtypes = [dp, P, P, P, P] + layer_args[4:] + [P]
    lib.hstu_layer_fwd_cand.restype = I32
    lib.hstu_layer_fwd_noalloc.argtypes = [dp] + [P] * 15
    lib.hstu_layer_fwd_noalloc.restype = I32
    lib.hstu_stack_workspace_size.argtypes = [dp, I32, ctypes.POINTER(SZ)]
    lib.hstu_stack_workspace_size.restype = I32
    lib.hstu_stack_fwd.argtypes = [dp, I32] + [P] * 15 + [SZ, P]
    lib.hstu_stack_fwd.restype = I32
    lib.hstu_preprocess.argtypes = [ctypes.POINTER(PrepDesc)] + [P] * 17
    lib.hstu_preprocess.restype = I32
    lib.kv_pages_append.argtypes = [dp, P, P, P, P, P, P, P, P, P]
    lib.kv_pages_append.restype = I32
    lib.hstu_read_device_status.argtypes = [P, ctypes.POINTER(I32), P]
    lib.hstu_read_device_status.restype = I32
    lib.hstu_status_string.argtypes = [I32]
    lib.hstu_status_string.restype = ctypes.c_char_p
    _ = I64
    _lib = lib
    return lib


def hip_runtime() -> ctypes.CDLL:
    """The HIP runtime the library is bound to (for events in benchmarks)."""
    load()
    return ctypes.CDLL("libamdhip64.so.7")


def loaded_hip_runtimes() -> Sequence[str]:
    """Paths of every libamdhip64 mapped into this process."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                paths.add(line.split()[-1])
    return sorted(paths)


class PrepDesc(ctypes.Structure):
    _fields_ = [
        ("num_users", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("total_new", ctypes.c_int32),
        ("item_rows", ctypes.c_int64),
        ("action_rows", ctypes.c_int64),
        ("ctx_rows", ctypes.c_int64),
        ("max_positions", ctypes.c_int32),
    ]


def header_functions(path: str = HEADER_PATH) -> Sequence[str]:
    """Names of the functions the C header declares."""
    src = open(path).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:hstu_status|const char\*)\s+([A-Za-z_][A-Za-z0-9_]*)\s*\(", src, flags=re.M)


def status_string(code: int) -> str:
    try:
        return load().hstu_status_string(int(code)).decode()
    except ImportError:
        return "status"


def make_desc(*, num_users: int, num_heads: int, head_dim: int, page_size: int,
              max_pages_per_user: int, num_pool_pages: int, total_new: int,
              pos_buckets: int, pos_mbits: int, attn_scale: float, norm_eps: float,
              dtype: str, ts_buckets: int = 0, ts_mbits: int = 0,
              batch_invariant: bool = False) -> LayerDesc:
    """batch_invariant sets FLAG_BATCH_INVARIANT: every row's result is then
    bit-identical whatever the batch and however the user's sequence was split
    into calls (cached history or recompute)."""
    return LayerDesc(num_users=num_users, num_heads=num_heads, head_dim=head_dim,
                     hidden=num_heads * head_dim, page_size=page_size,
                     max_pages_per_user=max_pages_per_user, num_pool_pages=num_pool_pages,
                     total_new=total_new, pos_buckets=pos_buckets, pos_mbits=pos_mbits,
                     ts_buckets=ts_buckets, ts_mbits=ts_mbits, attn_scale=attn_scale,
                     norm_eps=norm_eps, dtype=HSTU_BF16 if dtype == "bf16" else HSTU_F32,
                     flags=FLAG_BATCH_INVARIANT if batch_invariant else 0)


def _ptr(t, what: str, dtype=None, allow_none: bool = False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{what} is required")
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def stream_scope(stream):
    """Context for a call on `stream` (a torch stream or a raw hipStream_t):
    the binding's staging copies and output allocations then go on that
    stream too, so they are ordered with the library's kernels there and the
    caching allocator does not hand their memory to another stream early.
    None: the current stream, nothing changes."""
    import contextlib
    import torch
    if stream is None:
        return contextlib.nullcontext()
    if isinstance(stream, int):
        stream = torch.cuda.ExternalStream(stream)
    return torch.cuda.stream(stream)


def _tdtype(desc: LayerDesc):
    import torch
    return torch.bfloat16 if desc.dtype == HSTU_BF16 else torch.float32


def workspace_size(desc: LayerDesc) -> int:
    n = ctypes.c_size_t(0)
    rc = load().hstu_layer_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if rc != 0:
        raise HSTUError(rc, "hstu_layer_workspace_size")
    return int(n.value)


def layer_fwd(desc: LayerDesc, x, new_offsets, hist_len, page_table, k_pool, v_pool,
              w1t, w2t, pos_bias, y, workspace, ts_bias=None, timestamps=None,
              ts_offsets=None, stream=None, stage_events=None, num_candidates=None) -> None:
    """Enqueue one layer (see include/hstu.h).  `workspace` is a uint8 device
    tensor of at least workspace_size(desc) bytes; `stage_events` optionally
    a sequence of 2*NUM_STAGES raw hipEvent_t handles; `num_candidates` an
    int32 device tensor [B] of trailing candidate rows per user
    (hstu_layer_fwd_cand)."""
    import torch
    lib = load()
    dt = _tdtype(desc)
    args = [
        ctypes.byref(desc),
        _ptr(x, "x", dt, allow_none=desc.total_new == 0),
        _ptr(new_offsets, "new_offsets", torch.int32),
        _ptr(hist_len, "hist_len", torch.int32),
        _ptr(page_table, "page_table", torch.int32),
        _ptr(k_pool, "k_pool", dt),
        _ptr(v_pool, "v_pool", dt),
        _ptr(w1t, "w1t", dt),
        _ptr(w2t, "w2t", dt),
        _ptr(pos_bias, "pos_bias", torch.float32),
        _ptr(ts_bias, "ts_bias", torch.float32, allow_none=True),
        _ptr(timestamps, "timestamps", torch.int64, allow_none=True),
        _ptr(ts_offsets, "ts_offsets", torch.int32, allow_none=True),
        _ptr(y, "y", dt, allow_none=desc.total_new == 0),
        _ptr(workspace, "workspace"),
        ctypes.c_size_t(workspace.numel() * workspace.element_size()),
        _stream(stream),
    ]
    arr = None
    if stage_events is not None:
        arr = (ctypes.c_void_p * (2 * NUM_STAGES))(*[ctypes.c_void_p(e) for e in stage_events])
    if num_candidates is not None:
        nc = _ptr(num_candidates, "num_candidates", torch.int32)
        rc = lib.hstu_layer_fwd_cand(*args[:4], nc, *args[4:], arr)
    elif arr is not None:
        rc = lib.hstu_layer_fwd_timed(*args, arr)
    else:
        rc = lib.hstu_layer_fwd(*args)
    if rc != 0:
        raise HSTUError(rc, "hstu_layer_fwd")


# bytes of the library's static scratch array (HSTU_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


def layer_fwd_noalloc(desc: LayerDesc, x, new_offsets, hist_len, page_table, k_pool, v_pool,
                      w1t, w2t, pos_bias, y, device_status, ts_bias=None, timestamps=None,
                      ts_offsets=None, stream=None) -> None:
    """Enqueue hstu_layer_fwd_noalloc (include/hstu.h): hstu_layer_fwd with the
    library's static scratch array as its workspace; `device_status` (int32
    device tensor) receives the call's device code."""
    import torch
    dt = _tdtype(desc)
    none_rows = desc.total_new == 0
    rc = load().hstu_layer_fwd_noalloc(
        ctypes.byref(desc), _ptr(x, "x", dt, allow_none=none_rows),
        _ptr(new_offsets, "new_offsets", torch.int32), _ptr(hist_len, "hist_len", torch.int32),
        _ptr(page_table, "page_table", torch.int32), _ptr(k_pool, "k_pool", dt), _ptr(v_pool, "v_pool", dt),
        _ptr(w1t, "w1t", dt), _ptr(w2t, "w2t", dt), _ptr(pos_bias, "pos_bias", torch.float32),
        _ptr(ts_bias, "ts_bias", torch.float32, allow_none=True),
        _ptr(timestamps, "timestamps", torch.int64, allow_none=True),
        _ptr(ts_offsets, "ts_offsets", torch.int32, allow_none=True),
        _ptr(y, "y", dt, allow_none=none_rows), _ptr(device_status, "device_status", torch.int32),
        _stream(stream))
    if rc != 0:
        raise HSTUError(rc, "hstu_layer_fwd_noalloc")


def stack_workspace_size(desc: LayerDesc, num_layers: int) -> int:
    n = ctypes.c_size_t(0)
    rc = load().hstu_stack_workspace_size(ctypes.byref(desc), int(num_layers), ctypes.byref(n))
    if rc != 0:
        raise HSTUError(rc, "hstu_stack_workspace_size")
    return int(n.value)


def stack_fwd(desc: LayerDesc, x, new_offsets, hist_len, page_tables, k_pools, v_pools, w1t, w2t, pos_bias,
              ys, workspace, ts_bias=None, timestamps=None, ts_offsets=None, num_candidates=None,
              stream=None) -> None:
    """Enqueue hstu_stack_fwd (include/hstu.h): per-layer arguments are
    sequences of device tensors, one per layer; ys[l] receives layer l."""
    import torch
    dt = _tdtype(desc)
    nl = len(w1t)
    arr = lambda vals: (ctypes.c_void_p * nl)(*[ctypes.c_void_p(v) for v in vals])
    none_rows = desc.total_new == 0
    rc = load().hstu_stack_fwd(
        ctypes.byref(desc), nl, _ptr(x, "x", dt, allow_none=none_rows), _ptr(new_offsets, "new_offsets", torch.int32),
        _ptr(hist_len, "hist_len", torch.int32), _ptr(num_candidates, "num_candidates", torch.int32, allow_none=True),
        arr([_ptr(t, "page_table", torch.int32) for t in page_tables]),
        arr([_ptr(t, "k_pool", dt) for t in k_pools]), arr([_ptr(t, "v_pool", dt) for t in v_pools]),
        arr([_ptr(t, "w1t", dt) for t in w1t]), arr([_ptr(t, "w2t", dt) for t in w2t]),
        arr([_ptr(t, "pos_bias", torch.float32) for t in pos_bias]),
        None if ts_bias is None else arr([_ptr(t, "ts_bias", torch.float32) for t in ts_bias]),
        _ptr(timestamps, "timestamps", torch.int64, allow_none=True),
        _ptr(ts_offsets, "ts_offsets", torch.int32, allow_none=True),
        arr([_ptr(t, "y", dt, allow_none=none_rows) or 0 for t in ys]), _ptr(workspace, "workspace"),
        ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream(stream))
    if rc != 0:
        raise HSTUError(rc, "hstu_stack_fwd")


def preprocess(*, hist_len, ctx_offsets, ctx_ids, hist_offsets, item_ids, action_ids, cand_offsets,
               cand_ids, item_emb, action_emb, ctx_emb, pos_emb, x, new_offsets, num_candidates,
               device_status, stream=None) -> None:
    """Enqueue hstu_preprocess (include/hstu.h): token ids -> x [T, D] plus the
    layer's new_offsets and num_candidates.  Tables and x share one dtype;
    action_ids / action_emb None = no action tokens."""
    import torch
    dt = x.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise ValueError("x must be float32 or bfloat16")
    T, D = int(x.shape[0]), int(x.shape[1])
    desc = PrepDesc(num_users=int(hist_len.shape[0]), hidden=D,
                    dtype=HSTU_BF16 if dt == torch.bfloat16 else HSTU_F32, total_new=T,
                    item_rows=int(item_emb.shape[0]),
                    action_rows=0 if action_emb is None else int(action_emb.shape[0]),
                    ctx_rows=int(ctx_emb.shape[0]), max_positions=int(pos_emb.shape[0]))
    i64 = torch.int64
    rc = load().hstu_preprocess(
        ctypes.byref(desc), _ptr(hist_len, "hist_len", torch.int32) or None,
        _ptr(ctx_offsets, "ctx_offsets", torch.int32), _ptr(ctx_ids, "ctx_ids", i64),
        _ptr(hist_offsets, "hist_offsets", torch.int32), _ptr(item_ids, "item_ids", i64),
        _ptr(action_ids, "action_ids", i64, allow_none=True),
        _ptr(cand_offsets, "cand_offsets", torch.int32), _ptr(cand_ids, "cand_ids", i64),
        _ptr(item_emb, "item_emb", dt), _ptr(action_emb, "action_emb", dt, allow_none=True),
        _ptr(ctx_emb, "ctx_emb", dt), _ptr(pos_emb, "pos_emb", dt), _ptr(x, "x", dt),
        _ptr(new_offsets, "new_offsets", torch.int32), _ptr(num_candidates, "num_candidates", torch.int32) or None,
        _ptr(device_status, "device_status", torch.int32), _stream(stream))
    if rc != 0:
        raise HSTUError(rc, "hstu_preprocess")


def kv_pages_append(desc: LayerDesc, k_new, v_new, new_offsets, hist_len, page_table,
                    k_pool, v_pool, device_status, stream=None) -> None:
    import torch
    dt = _tdtype(desc)
    rc = load().kv_pages_append(
        ctypes.byref(desc),
        _ptr(k_new, "k_new", dt, allow_none=desc.total_new == 0),
        _ptr(v_new, "v_new", dt, allow_none=desc.total_new == 0),
        _ptr(new_offsets, "new_offsets", torch.int32),
        _ptr(hist_len, "hist_len", torch.int32),
        _ptr(page_table, "page_table", torch.int32),
        _ptr(k_pool, "k_pool", dt),
        _ptr(v_pool, "v_pool", dt),
        _ptr(device_status, "device_status", torch.int32),
        _stream(stream))
    if rc != 0:
        raise HSTUError(rc, "kv_pages_append")


def read_device_status(status, stream=None) -> int:
    """Synchronise `stream` and return the device status word at `status`
    (a workspace tensor, an int32 status tensor or a raw pointer)."""
    code = ctypes.c_int32(0)
    rc = load().hstu_read_device_status(_ptr(status, "status"), ctypes.byref(code), _stream(stream))
    if rc not in (0, -5):
        raise HSTUError(rc, "hstu_read_device_status")
    return int(code.value)
