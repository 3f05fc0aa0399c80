"""Host-side checks of libhstu that need no GPU: the library loads, exports
every function the header declares, sizes workspaces, and rejects bad
descriptors before touching the device."""
import ctypes
import os

import pytest

import hstu_jagged_silu_fwd_amd as hs
from hstu_jagged_silu_fwd_amd import _lib


def desc(**over):
    kw = dict(num_users=8, num_heads=4, head_dim=128, page_size=32, max_pages_per_user=136,
              num_pool_pages=1 << 16, total_new=1000, pos_buckets=128, pos_mbits=3,
              attn_scale=1 / 4096, norm_eps=1e-6, dtype="bf16")
    kw.update(over)
    return hs.make_desc(**kw)


def test_exports_every_header_function():
    lib = hs.load()
    names = list(hs.header_functions())
    assert set(names) == {"hstu_layer_workspace_size", "hstu_layer_fwd", "hstu_layer_fwd_timed",
                          "hstu_layer_fwd_cand", "hstu_layer_fwd_noalloc", "hstu_stack_workspace_size",
                          "hstu_stack_fwd",
                          "hstu_preprocess", "kv_pages_append", "hstu_read_device_status",
                          "hstu_status_string"}
    for n in names:
        assert hasattr(lib, n), n


def test_exports_every_kvcache_header_function():
    """include/hstu_kvcache.h: every declared function is exported."""
    import os
    import re
    path = os.path.join(os.path.dirname(_lib.HEADER_PATH), "hstu_kvcache.h")
    src = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
    names = re.findall(r"^\s*(?:hstu_kv_status|hstu_kvcache\*|void|int64_t)\s+([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       src, flags=re.M)
    assert set(names) == {"hstu_kvcache_create", "hstu_kvcache_destroy", "hstu_kvcache_directory_elems",
                          "hstu_kvcache_plan", "hstu_kvcache_lookup", "hstu_kvcache_evict",
                          "hstu_kvcache_stats", "hstu_kvcache_trim", "hstu_kvcache_pin", "hstu_kv_tables_build",
                          "hstu_kv_copy_pages"}
    lib = hs.load()
    for n in names:
        assert hasattr(lib, n), n


def test_desc_struct_layout():
    # int32 x6, int64, int32 x5, float x2, int32 x2 -> 72 bytes with the int64 aligned at 24.
    assert ctypes.sizeof(_lib.LayerDesc) == 72
    assert _lib.LayerDesc.num_pool_pages.offset == 24
    assert _lib.LayerDesc.flags.offset == 64


def test_desc_struct_matches_the_header(tmp_path):
    """The ctypes mirror against the C compiler's own layout of the header's
    struct: size and every field's offset."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = [f[0] for f in _lib.LayerDesc._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"hstu.h\"\nint main(void) {\n"
                   '  printf("%zu\\n", sizeof(hstu_layer_desc));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(hstu_layer_desc, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.dirname(_lib.HEADER_PATH), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    assert got[0] == ctypes.sizeof(_lib.LayerDesc)
    assert got[1:] == [getattr(_lib.LayerDesc, f).offset for f in fields]
    assert _lib.FLAG_BATCH_INVARIANT == 1 and _lib.INVARIANT_CHUNK_KEYS == 256
    hdr = open(_lib.HEADER_PATH).read()
    assert "#define HSTU_FLAG_BATCH_INVARIANT 1" in hdr and "#define HSTU_INVARIANT_CHUNK_KEYS 256" in hdr


@pytest.mark.parametrize("flags", [2, 3, -1])
def test_unknown_flag_bits_are_rejected(flags):
    d = desc()
    d.flags = flags
    with pytest.raises(hs.HSTUError) as ei:
        hs.workspace_size(d)
    assert ei.value.code == -1


def test_batch_invariant_workspace_holds_its_fixed_chunks():
    """The invariant split has ceil(max_len / 256) pieces per (q-block, head):
    its workspace is at least that many 256-row fp32 partial blocks."""
    plain = hs.workspace_size(desc())
    inv = hs.workspace_size(desc(batch_invariant=True))
    assert inv >= plain
    nqb_cap = (1000 + 255) // 256 + 8
    per_entry = (136 * 32 + 255) // 256
    assert inv >= 4 * nqb_cap * per_entry * 256 * 128 * 4
    assert hs.workspace_size(desc(dtype="f32", batch_invariant=True)) >= 4 * nqb_cap * per_entry * 256 * 128 * 4


def test_workspace_size_grows_with_rows():
    a = hs.workspace_size(desc(total_new=100))
    b = hs.workspace_size(desc(total_new=10000))
    assert 0 < a < b
    assert a % 256 == 0


@pytest.mark.parametrize("over,code", [
    (dict(head_dim=96), -2),
    (dict(page_size=24), -2),
    (dict(page_size=8), -2),
    (dict(num_heads=0), -1),
    (dict(pos_buckets=0), -1),
    (dict(pos_buckets=4096), -1),
    (dict(norm_eps=0.0), -1),
    (dict(dtype="f32", head_dim=32, num_heads=1), -2),   # hidden 32 not a multiple of 64
    (dict(total_new=-1), -1),
])
def test_bad_descriptors_rejected(over, code):
    with pytest.raises(hs.HSTUError) as ei:
        hs.workspace_size(desc(**over))
    assert ei.value.code == code


def test_null_pointers_rejected_before_any_device_work():
    lib = hs.load()
    d = desc()
    rc = lib.hstu_layer_fwd(ctypes.byref(d), *([None] * 14), ctypes.c_size_t(0), None)
    assert rc == -1
    rc = lib.kv_pages_append(ctypes.byref(d), *([None] * 8), None)
    assert rc == -1
    code = ctypes.c_int32(0)
    assert lib.hstu_read_device_status(None, ctypes.byref(code), None) == -1


def test_status_strings():
    assert hs.status_string(0) == "ok"
    assert "workspace" in hs.status_string(-3)
    assert "page" in hs.status_string(4)


def test_single_hip_runtime_in_process():
    hs.load()
    rts = _lib.loaded_hip_runtimes()
    assert len(rts) == 1, rts


def test_candidate_and_preprocess_host_checks():
    """Host-checkable errors of the candidate layer call and of the
    preprocessing return before anything is enqueued (no GPU needed)."""
    import ctypes
    lib = hs.load()
    d = desc()
    # num_candidates is required (desc, x, offsets, hist, num_candidates, then
    # the 11 pointers page_table .. workspace, bytes, stream, events)
    assert lib.hstu_layer_fwd_cand(ctypes.byref(d), None, None, None, None, *([None] * 11), 0, None, None) == -1
    P = _lib.PrepDesc
    args = [None] * 17
    assert lib.hstu_preprocess(None, *args) == -1
    good = dict(num_users=2, hidden=512, dtype=1, total_new=10, item_rows=100, action_rows=4,
                ctx_rows=8, max_positions=8320)
    for over, code in [(dict(hidden=96), -2), (dict(hidden=4096), -2), (dict(dtype=7), -2),
                       (dict(num_users=5000), -2), (dict(item_rows=0), -1), (dict(ctx_rows=0), -1),
                       (dict(action_rows=-1), -1), (dict(max_positions=0), -1), (dict(total_new=-1), -1),
                       ({}, -1)]:          # {}: valid sizes, null pointers
        kw = dict(good)
        kw.update(over)
        assert lib.hstu_preprocess(ctypes.byref(P(**kw)), *args) == code, over


def test_beam_header_exports_and_host_checks():
    """include/hstu_beam.h: every declared function is exported, and bad
    descriptors are rejected on the host (no GPU needed)."""
    import os
    import re
    from hstu_jagged_silu_fwd_amd import beam as hb
    path = os.path.join(os.path.dirname(_lib.HEADER_PATH), "hstu_beam.h")
    src = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
    names = re.findall(r"^\s*hstu_status\s+([A-Za-z_][A-Za-z0-9_]*)\s*\(", src, flags=re.M)
    assert set(names) == {"hstu_beam_workspace_size", "hstu_beam_decode_attn"}
    lib = hb._lib_beam()
    for n in names:
        assert hasattr(lib, n)
    good = dict(num_requests=4, beam_width=256, num_q_heads=16, num_kv_heads=8, head_dim=128, max_ctx=1024,
                step=2, max_steps=3, scale=128 ** -0.5, dtype=1)
    n = ctypes.c_size_t(0)
    assert lib.hstu_beam_workspace_size(ctypes.byref(hb.BeamDesc(**good)), ctypes.byref(n)) == 0 and n.value > 0
    for over, code in [(dict(head_dim=32), -2), (dict(dtype=5), -2), (dict(max_ctx=1000), -1),
                       (dict(num_q_heads=12, num_kv_heads=8), -1), (dict(step=3), -1), (dict(beam_width=0), -1),
                       (dict(scale=0.0), -1), (dict(num_requests=-1), -1)]:
        kw = dict(good)
        kw.update(over)
        assert lib.hstu_beam_workspace_size(ctypes.byref(hb.BeamDesc(**kw)), ctypes.byref(n)) == code, over
    # valid sizes, null pointers
    assert lib.hstu_beam_decode_attn(ctypes.byref(hb.BeamDesc(**good)), *([None] * 9), 0, None) == -1


def test_stack_host_checks():
    """hstu_stack_fwd / hstu_stack_workspace_size reject bad layer counts and
    missing per-layer arrays before touching the GPU."""
    import ctypes
    lib = hs.load()
    d = desc()
    n = ctypes.c_size_t(0)
    assert lib.hstu_stack_workspace_size(ctypes.byref(d), 3, ctypes.byref(n)) == 0
    one = ctypes.c_size_t(0)
    assert lib.hstu_stack_workspace_size(ctypes.byref(d), 1, ctypes.byref(one)) == 0 and n.value >= one.value
    for nl in (0, 33):
        assert lib.hstu_stack_workspace_size(ctypes.byref(d), nl, ctypes.byref(n)) == -1
    # desc, layers, x, offsets, hist, candidates, 9 per-layer arrays and tensors, y, ws, bytes, stream
    assert lib.hstu_stack_fwd(ctypes.byref(d), 3, *([None] * 15), 0, None) == -1


def test_noalloc_host_checks():
    """hstu_layer_fwd_noalloc: a missing status int or any null pointer is
    rejected, and a call whose workspace would exceed the static scratch
    array returns HSTU_ERR_SCRATCH, all before any device work."""
    lib = hs.load()
    d = desc()
    assert hs.workspace_size(d) <= _lib.NOALLOC_SCRATCH_BYTES
    # desc, 13 pointers (x .. y), device_status, stream
    assert lib.hstu_layer_fwd_noalloc(ctypes.byref(d), *([None] * 14), None) == -1
    big = desc(total_new=200000, num_users=4000, max_pages_per_user=1100)
    assert hs.workspace_size(big) > _lib.NOALLOC_SCRATCH_BYTES
    status = ctypes.c_int32(0)
    rc = lib.hstu_layer_fwd_noalloc(ctypes.byref(big), *([None] * 13), ctypes.byref(status), None)
    assert rc == -6
    assert "scratch" in hs.status_string(-6)


def test_stack_workspace_stream_map_is_bounded():
    """HSTUStack remembers the stream of each workspace's last call (for
    read_status) only for its most recent workspaces, so callers that make a
    new workspace per call do not grow it; a workspace used again moves to
    the most recent end."""
    import torch
    from hstu_jagged_silu_fwd_amd.stack import HSTUStack
    st = HSTUStack(num_users=1, num_heads=1, head_dim=32, page_size=16, num_pool_pages=1,
                   max_pages_per_user=1, pos_buckets=32, pos_mbits=3, attn_scale=1.0, device="cpu")
    keep = [torch.empty(256, dtype=torch.uint8) for _ in range(3 * st.kWsStreams)]
    first = keep[0]
    for i, w in enumerate(keep):
        st._last_ws = w
        st._note_stream(i)
        st._last_ws = first                  # the first workspace stays in use
        st._note_stream("first")
    assert len(st._ws_stream) == st.kWsStreams
    assert st._ws_stream[first.data_ptr()] == "first"
    assert st._ws_stream[keep[-1].data_ptr()] == len(keep) - 1
    assert keep[1].data_ptr() not in st._ws_stream
