"""MI355X-native HSTU layer forward over jagged sequences with a paged KV cache.

The compute lives in libhstu.so (hand-written gfx950 HIP kernels behind the C
ABI in include/hstu.h); this package is its thin Python binding plus a small
layer/stack driver that owns device buffers.
"""
from ._lib import (  # noqa: F401
    HSTU_BF16, HSTU_F32, NUM_STAGES, STAGES, HSTUError, LayerDesc, header_functions,
    kv_pages_append, layer_fwd, load, make_desc, read_device_status, status_string,
    workspace_size,
)
