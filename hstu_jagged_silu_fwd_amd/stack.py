"""A stack of HSTU layers sharing one paged KV pool (device buffers owned by
torch; every layer step runs in libhstu).

Each layer has its own weights, bias tables and page table into the shared
pool; layer l's output rows are layer l+1's input rows.
"""
from __future__ import annotations

import collections
from typing import List, Optional

import torch

from . import _lib


class HSTUStack:
    def __init__(self, *, num_users: int, num_heads: int, head_dim: int, page_size: int,
                 num_pool_pages: int, max_pages_per_user: int, pos_buckets: int,
                 pos_mbits: int, attn_scale: float, norm_eps: float = 1e-6,
                 dtype: str = "bf16", ts_buckets: int = 0, ts_mbits: int = 0,
                 num_layers: int = 1, device: str = "cuda", pool_fill: Optional[float] = None,
                 batch_invariant: bool = False):
        """batch_invariant: every call runs with FLAG_BATCH_INVARIANT (rows
        bit-identical whatever the batch and however a user's sequence is
        split into calls)."""
        self.B, self.H, self.d = num_users, num_heads, head_dim
        self.D = num_heads * head_dim
        self.ps, self.P, self.maxP = page_size, num_pool_pages, max_pages_per_user
        self.dtype = dtype
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.device = torch.device(device)
        self.common = dict(num_users=num_users, num_heads=num_heads, head_dim=head_dim,
                           page_size=page_size, max_pages_per_user=max_pages_per_user,
                           num_pool_pages=num_pool_pages, pos_buckets=pos_buckets,
                           pos_mbits=pos_mbits, attn_scale=attn_scale, norm_eps=norm_eps,
                           dtype=dtype, ts_buckets=ts_buckets, ts_mbits=ts_mbits,
                           batch_invariant=batch_invariant)
        shape_k = (num_pool_pages, num_heads, page_size, head_dim)
        shape_v = (num_pool_pages, num_heads, head_dim, page_size)
        if pool_fill is None:
            self.k_pool = torch.empty(shape_k, dtype=self.tdtype, device=self.device)
            self.v_pool = torch.empty(shape_v, dtype=self.tdtype, device=self.device)
        else:
            self.k_pool = torch.full(shape_k, pool_fill, dtype=self.tdtype, device=self.device)
            self.v_pool = torch.full(shape_v, pool_fill, dtype=self.tdtype, device=self.device)
        self.layers: List[dict] = [dict() for _ in range(num_layers)]
        self.status = torch.zeros(1, dtype=torch.int32, device=self.device)
        self._ws = None
        self._sws = None          # workspace of the stack calls
        self._last_ws = None      # workspace of the last call (its status word)
        self._last_stream = None  # stream of the last call
        # workspace address -> stream of its last call (the most recent
        # kWsStreams workspaces; callers that make a new workspace per call
        # do not grow it without bound)
        self._ws_stream: "collections.OrderedDict[int, object]" = collections.OrderedDict()

    kWsStreams = 64

    def _note_stream(self, stream) -> None:
        key = self._last_ws.data_ptr()
        self._ws_stream.pop(key, None)
        self._ws_stream[key] = stream
        while len(self._ws_stream) > self.kWsStreams:
            self._ws_stream.popitem(last=False)

    def desc(self, total_new: int, num_users: Optional[int] = None) -> _lib.LayerDesc:
        kw = dict(self.common)
        if num_users is not None:
            kw["num_users"] = num_users
        return _lib.make_desc(total_new=total_new, **kw)

    def _dev(self, a, dtype):
        t = torch.as_tensor(a)
        return t.to(device=self.device, dtype=dtype).contiguous()

    def set_layer(self, l: int, *, w1t, w2t, pos_bias, page_table, ts_bias=None) -> None:
        """Layer l's parameters; w1t [4D, D] and w2t [D, D] are the projection
        weights in out-features x in-features layout (W1 and W2 transposed)."""
        self.layers[l] = dict(
            w1t=self._dev(w1t, self.tdtype), w2t=self._dev(w2t, self.tdtype),
            pos_bias=self._dev(pos_bias, torch.float32),
            ts_bias=None if ts_bias is None else self._dev(ts_bias, torch.float32),
            page_table=self._dev(page_table, torch.int32))

    def workspace(self, total_new: int) -> torch.Tensor:
        need = _lib.workspace_size(self.desc(total_new))
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws

    def append(self, l: int, k_new, v_new, new_offsets, hist_len, stream=None) -> None:
        """kv_pages_append of rows into layer l's pages (status in self.status),
        on `stream` (default: the current stream; inputs are staged there)."""
        with _lib.stream_scope(stream):
            self._append(l, k_new, v_new, new_offsets, hist_len)

    def _append(self, l, k_new, v_new, new_offsets, hist_len) -> None:
        k_new = self._dev(k_new, self.tdtype)
        v_new = self._dev(v_new, self.tdtype)
        off = self._dev(new_offsets, torch.int32)
        T = int(k_new.shape[0])
        _lib.kv_pages_append(self.desc(T), k_new, v_new, off, self._dev(hist_len, torch.int32),
                             self.layers[l]["page_table"], self.k_pool, self.v_pool, self.status)

    def layer(self, l: int, x: torch.Tensor, new_offsets: torch.Tensor, hist_len: torch.Tensor,
              y: torch.Tensor, workspace: Optional[torch.Tensor] = None, timestamps=None,
              ts_offsets=None, stream=None, stage_events=None, page_table=None,
              num_candidates=None) -> None:
        """Layer l over a batch; page_table [B, max_pages] overrides the layer's
        own table (the batch size is then taken from new_offsets);
        num_candidates [B] int32 marks each user's trailing candidate rows."""
        with _lib.stream_scope(stream):
            self._layer(l, x, new_offsets, hist_len, y, workspace, timestamps, ts_offsets, stage_events,
                        page_table, num_candidates)
        self._last_stream = stream
        self._note_stream(stream)

    def _layer(self, l, x, new_offsets, hist_len, y, workspace, timestamps, ts_offsets, stage_events,
               page_table, num_candidates) -> None:
        T = int(x.shape[0])
        L = self.layers[l]
        nu = None if page_table is None else int(new_offsets.shape[0]) - 1
        desc = self.desc(T, nu)
        ws = self.workspace(T) if workspace is None else workspace
        if nu is not None and workspace is None:
            need = _lib.workspace_size(desc)
            if ws.numel() < need:
                self._ws = ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        self._last_ws = ws
        _lib.layer_fwd(desc, x, new_offsets, hist_len, L["page_table"] if page_table is None else page_table, self.k_pool,
                       self.v_pool, L["w1t"], L["w2t"], L["pos_bias"], y, ws,
                       ts_bias=L["ts_bias"], timestamps=timestamps, ts_offsets=ts_offsets,
                       stage_events=stage_events, num_candidates=num_candidates)

    def forward(self, x, new_offsets, hist_len, timestamps=None, ts_offsets=None,
                stream=None, return_all: bool = False, page_tables=None, num_candidates=None,
                workspace: Optional[torch.Tensor] = None):
        """Run every layer in one hstu_stack_fwd call (the batch metadata is
        prepared once for all layers); returns the last layer's output (or
        all outputs).  page_tables: optional per-layer [B, max_pages] tables
        (e.g. a KV cache plan's, from KVCache.build_tables) instead of the
        layers' own.  stream: where the call runs (default: the current
        stream); inputs are staged and outputs allocated there too.
        workspace: a uint8 device tensor of at least stack_workspace_size
        bytes for this call (default: one the stack keeps).  Calls that
        overlap in time (batches in flight on different streams) each need
        a workspace of their own, and their users' pages must not overlap."""
        with _lib.stream_scope(stream):
            out = self._forward(x, new_offsets, hist_len, timestamps, ts_offsets, return_all, page_tables,
                                num_candidates, workspace)
        self._last_stream = stream
        self._note_stream(stream)
        return out

    def _forward(self, x, new_offsets, hist_len, timestamps, ts_offsets, return_all, page_tables,
                 num_candidates, workspace=None):
        x = self._dev(x, self.tdtype)
        off = self._dev(new_offsets, torch.int32)
        hl = self._dev(hist_len, torch.int32)
        ts = None if timestamps is None else self._dev(timestamps, torch.int64)
        tso = None if ts_offsets is None else self._dev(ts_offsets, torch.int32)
        nc = None if num_candidates is None else self._dev(num_candidates, torch.int32)
        T = int(x.shape[0])
        nl = len(self.layers)
        nu = None if page_tables is None else int(off.shape[0]) - 1
        desc = self.desc(T, nu)
        need = _lib.stack_workspace_size(desc, nl)
        if workspace is not None:
            if workspace.dtype != torch.uint8 or workspace.device.type != "cuda" or workspace.numel() < need:
                raise ValueError(f"workspace: a uint8 device tensor of at least {need} bytes is needed")
            ws = workspace
        else:
            if self._sws is None or self._sws.numel() < need:
                self._sws = torch.empty(need, dtype=torch.uint8, device=self.device)
            ws = self._sws
        outs = [torch.empty_like(x) for _ in range(nl)]
        L = self.layers
        pts = [L[l]["page_table"] for l in range(nl)] if page_tables is None else \
            [self._dev(page_tables[l], torch.int32) for l in range(nl)]
        has_ts = L[0]["ts_bias"] is not None
        _lib.stack_fwd(desc, x, off, hl, pts, [self.k_pool] * nl, [self.v_pool] * nl, [l["w1t"] for l in L],
                       [l["w2t"] for l in L], [l["pos_bias"] for l in L], outs, ws,
                       ts_bias=[l["ts_bias"] for l in L] if has_ts else None, timestamps=ts, ts_offsets=tso,
                       num_candidates=nc)
        self._last_ws = ws
        return outs if return_all else outs[-1]

    def read_status(self, workspace: Optional[torch.Tensor] = None) -> int:
        """Device status of the last call on the given workspace, else of the
        last forward (stack call) or layer call, whichever ran last
        (synchronises the stream that call ran on)."""
        ws = self._last_ws if workspace is None else workspace
        return _lib.read_device_status(ws, stream=self._ws_stream.get(ws.data_ptr(), self._last_stream))
