// C ABI of libhstu: descriptor validation, workspace layout and the launch
// sequence of one layer (prep -> X W1 + SiLU/split/append -> paged SiLU
// attention -> norm * U -> G W2).
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

#include "common.h"

using namespace hstu;

// ---------------------------------------------------------------------------
// Workspace of hstu_layer_fwd_noalloc: a file-scope device array.  Each GPU
// holds its own copy at its own address; host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol) but
// the address hipGetSymbolAddress returns on that device, looked up once per
// device with the device current and kept in scratch_base_of.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[HSTU_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kAttnWgPerCu = 1;     // resident attention workgroups per CU

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct Layout {
  size_t row_loc, qb_first, qb_nch, qb_row0, qb_rows, items, q, u, part, tables, total;
  int nqb_cap, item_cap;
};

// Attention workgroups launched (and the split target): one per CU.
int attn_grid() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return cus * kAttnWgPerCu;
}

Layout make_layout(const hstu_layer_desc& d, int target, int nl = 1) {
  Layout L{};
  const size_t T = static_cast<size_t>(d.total_new);
  const size_t B = static_cast<size_t>(d.num_users);
  const size_t es = d.dtype == HSTU_BF16 ? 2 : 4;
  L.nqb_cap = static_cast<int>((T + kQB - 1) / kQB + B);
  // items <= total/chunk + H * entries, and total/chunk <= target unless the
  // chunk hits its cap, where it is <= H * entries * ceil(max_len / cap).
  // When H * entries can reach the target, the work list rounds its target
  // up to a multiple of it (at most one target more).
  const int64_t max_len = static_cast<int64_t>(d.max_pages_per_user) * d.page_size;
  const int64_t per_entry = 1 + (max_len + kMaxChunkKeys - 1) / kMaxChunkKeys;
  const int64_t heads_entries = static_cast<int64_t>(d.num_heads) * L.nqb_cap;
  int64_t cap = heads_entries * per_entry + target + (heads_entries >= target ? target : 0);
  // batch-invariant calls cut an entry of k keys into ceil(k / chunk) pieces
  if (d.flags & HSTU_FLAG_BATCH_INVARIANT)
    cap = std::max<int64_t>(cap, d.num_heads * L.nqb_cap *
                                     ((max_len + HSTU_INVARIANT_CHUNK_KEYS - 1) / HSTU_INVARIANT_CHUNK_KEYS));
  // (an absurd bound only makes the workspace absurd; prep rejects a call
  // whose items exceed the cap)
  L.item_cap = static_cast<int>(std::min<int64_t>(cap, int64_t{1} << 30));
  size_t off = 256;  // WsHeader
  L.row_loc = off;  off = align256(off + 8 * T * static_cast<size_t>(nl));
  L.qb_first = off; off = align256(off + 4 * static_cast<size_t>(L.nqb_cap));
  L.qb_nch = off;   off = align256(off + 4 * static_cast<size_t>(L.nqb_cap));
  L.qb_row0 = off;  off = align256(off + 4 * static_cast<size_t>(L.nqb_cap));
  L.qb_rows = off;  off = align256(off + 4 * static_cast<size_t>(L.nqb_cap));
  L.items = off;    off = align256(off + sizeof(AttnItem) * static_cast<size_t>(L.item_cap));
  L.q = off;        off = align256(off + es * T * d.hidden);
  L.u = off;        off = align256(off + es * T * d.hidden);
  L.part = off;     off = align256(off + 4 * static_cast<size_t>(L.item_cap) * kQB * d.head_dim);
  L.tables = off;   off = align256(off + 4 * static_cast<size_t>(kTabFloats) * nl);
  L.total = off;
  return L;
}

WsPtrs ws_ptrs(void* base, const Layout& L) {
  char* b = static_cast<char*>(base);
  WsPtrs w;
  w.hdr = reinterpret_cast<WsHeader*>(b);
  w.row_loc = reinterpret_cast<int2*>(b + L.row_loc);
  w.qb_first = reinterpret_cast<int32_t*>(b + L.qb_first);
  w.qb_nch = reinterpret_cast<int32_t*>(b + L.qb_nch);
  w.qb_row0 = reinterpret_cast<int32_t*>(b + L.qb_row0);
  w.qb_rows = reinterpret_cast<int32_t*>(b + L.qb_rows);
  w.items = reinterpret_cast<AttnItem*>(b + L.items);
  w.q = b + L.q;
  w.u = b + L.u;
  w.part = reinterpret_cast<float*>(b + L.part);
  w.tables = reinterpret_cast<float*>(b + L.tables);
  return w;
}

bool pow2_in(int x, int lo, int hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }

// Shape checks shared by every entry point.
hstu_status check_common(const hstu_layer_desc* d) {
  if (d == nullptr) return HSTU_ERR_INVALID_ARG;
  if (d->num_users > kMaxUsers) return HSTU_ERR_UNSUPPORTED;
  if (d->total_new > kMaxRows) return HSTU_ERR_UNSUPPORTED;
  if (d->num_users < 0 || d->num_heads < 1 || d->total_new < 0 || d->max_pages_per_user < 1 ||
      d->num_pool_pages < 1)
    return HSTU_ERR_INVALID_ARG;
  if (d->dtype != HSTU_F32 && d->dtype != HSTU_BF16) return HSTU_ERR_UNSUPPORTED;
  if ((d->flags & ~HSTU_FLAG_BATCH_INVARIANT) != 0) return HSTU_ERR_INVALID_ARG;
  if (d->head_dim != 32 && d->head_dim != 64 && d->head_dim != 128) return HSTU_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(d->num_heads) * d->head_dim != d->hidden) return HSTU_ERR_INVALID_ARG;
  if (d->hidden % 64 != 0 || d->hidden > 2048) return HSTU_ERR_UNSUPPORTED;
  if (!pow2_in(d->page_size, 16, 128)) return HSTU_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(d->max_pages_per_user) * d->page_size >= (int64_t{1} << 30))
    return HSTU_ERR_UNSUPPORTED;
  if (d->num_pool_pages > (int64_t{1} << 31) - 1) return HSTU_ERR_UNSUPPORTED;
  return HSTU_OK;
}

hstu_status check_layer(const hstu_layer_desc* d) {
  hstu_status s = check_common(d);
  if (s != HSTU_OK) return s;
  if (d->pos_buckets < 1 || d->pos_buckets > kMaxBuckets || d->pos_mbits < 0 || d->pos_mbits > 16)
    return HSTU_ERR_INVALID_ARG;
  if (d->ts_buckets < 0 || d->ts_buckets > kMaxBuckets) return HSTU_ERR_INVALID_ARG;
  if (d->ts_buckets > 0 && (d->ts_mbits < 0 || d->ts_mbits > 30)) return HSTU_ERR_INVALID_ARG;
  if (!std::isfinite(d->attn_scale) || !(d->norm_eps > 0.0f) || !std::isfinite(d->norm_eps))
    return HSTU_ERR_INVALID_ARG;
  return HSTU_OK;
}

hstu_status layer_impl(const hstu_layer_desc* desc, const void* x, const int32_t* new_offsets,
                       const int32_t* hist_len, const int32_t* ncand, const int32_t* page_table, void* k_pool, void* v_pool,
                       const void* w1t, const void* w2t, const float* pos_bias, const float* ts_bias,
                       const int64_t* timestamps, const int32_t* ts_offsets, void* y, void* workspace,
                       size_t workspace_bytes, void* hip_stream, void* const* ev) {
  hstu_status s = check_layer(desc);
  if (s != HSTU_OK) return s;
  const hstu_layer_desc& d = *desc;
  const bool any_rows = d.total_new > 0;
  if (new_offsets == nullptr || hist_len == nullptr || page_table == nullptr || k_pool == nullptr ||
      v_pool == nullptr || w1t == nullptr || w2t == nullptr || pos_bias == nullptr || workspace == nullptr)
    return HSTU_ERR_INVALID_ARG;
  if (any_rows && (x == nullptr || y == nullptr)) return HSTU_ERR_INVALID_ARG;
  if (any_rows && x == y) return HSTU_ERR_INVALID_ARG;
  if (d.ts_buckets > 0 && (ts_bias == nullptr || timestamps == nullptr || ts_offsets == nullptr))
    return HSTU_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return HSTU_ERR_INVALID_ARG;
  const int grid = attn_grid();
  const Layout L = make_layout(d, grid);
  if (workspace_bytes < L.total) return HSTU_ERR_WORKSPACE;
  const WsPtrs ws = ws_ptrs(workspace, L);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const int32_t* ts_off = d.ts_buckets > 0 ? ts_offsets : nullptr;
  const int64_t* ts = d.ts_buckets > 0 ? timestamps : nullptr;
  const float* tsb = d.ts_buckets > 0 ? ts_bias : nullptr;

  // stage k's kernel is bracketed by events ev[2k] (start) and ev[2k+1] (stop)
  auto kev = [&](int stage) -> KernelEvents {
    KernelEvents k;
    if (ev != nullptr) {
      k.start = static_cast<hipEvent_t>(ev[2 * stage]);
      k.stop = static_cast<hipEvent_t>(ev[2 * stage + 1]);
    }
    return k;
  };
  hipError_t e;
  e = launch_prep(d, new_offsets, hist_len, ncand, &page_table, 1, ts_off, &pos_bias, &tsb, ws, L.nqb_cap,
                  L.item_cap, grid, st, kev(HSTU_STAGE_PREP));
  if (e != hipSuccess) return HSTU_ERR_HIP;
  if (!any_rows) return HSTU_OK;
  e = launch_gemm_qkv(d, x, w1t, k_pool, v_pool, ws, st, kev(HSTU_STAGE_PROJ));
  if (e != hipSuccess) return HSTU_ERR_HIP;
  e = launch_attn(d, page_table, k_pool, v_pool, 0, ts, ts_off, ncand, ws, grid < L.item_cap ? grid : L.item_cap,
                  st, kev(HSTU_STAGE_ATTN));
  if (e != hipSuccess) return HSTU_ERR_HIP;
  e = launch_norm_gate(d, ws, L.nqb_cap, st, kev(HSTU_STAGE_NORM));
  if (e != hipSuccess) return HSTU_ERR_HIP;
  e = launch_gemm_out(d, ws.q, w2t, y, &ws.hdr->status, st, kev(HSTU_STAGE_OUT));
  if (e != hipSuccess) return HSTU_ERR_HIP;
  return HSTU_OK;
}

// A stack of nl layers over one batch: the metadata is prepared and checked
// once (every layer's page table included), then each layer runs its four
// compute kernels; layer l reads layer l-1's output.
hstu_status stack_impl(const hstu_layer_desc* desc, int32_t nl, const void* x, const int32_t* new_offsets,
                       const int32_t* hist_len, const int32_t* ncand, const int32_t* const* pts,
                       void* const* kps, void* const* vps, const void* const* w1s, const void* const* w2s,
                       const float* const* pbs, const float* const* tsbs, const int64_t* timestamps,
                       const int32_t* ts_offsets, void* const* ys, void* workspace, size_t workspace_bytes,
                       void* hip_stream) {
  hstu_status s = check_layer(desc);
  if (s != HSTU_OK) return s;
  if (nl < 1 || nl > kMaxStackLayers) return HSTU_ERR_INVALID_ARG;
  const hstu_layer_desc& d = *desc;
  const bool any_rows = d.total_new > 0;
  const bool has_ts = d.ts_buckets > 0;
  if (new_offsets == nullptr || hist_len == nullptr || pts == nullptr || kps == nullptr || vps == nullptr ||
      w1s == nullptr || w2s == nullptr || pbs == nullptr || ys == nullptr || workspace == nullptr)
    return HSTU_ERR_INVALID_ARG;
  if (has_ts && (tsbs == nullptr || timestamps == nullptr || ts_offsets == nullptr)) return HSTU_ERR_INVALID_ARG;
  for (int l = 0; l < nl; ++l) {
    if (pts[l] == nullptr || kps[l] == nullptr || vps[l] == nullptr || w1s[l] == nullptr || w2s[l] == nullptr ||
        pbs[l] == nullptr || (has_ts && tsbs[l] == nullptr))
      return HSTU_ERR_INVALID_ARG;
    if (any_rows && (ys[l] == nullptr || ys[l] == (l == 0 ? x : ys[l - 1]))) return HSTU_ERR_INVALID_ARG;
  }
  if (any_rows && x == nullptr) return HSTU_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return HSTU_ERR_INVALID_ARG;
  const int grid = attn_grid();
  const Layout L = make_layout(d, grid, nl);
  if (workspace_bytes < L.total) return HSTU_ERR_WORKSPACE;
  const WsPtrs ws = ws_ptrs(workspace, L);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const int32_t* ts_off = has_ts ? ts_offsets : nullptr;
  const int64_t* ts = has_ts ? timestamps : nullptr;
  hipError_t e = launch_prep(d, new_offsets, hist_len, ncand, pts, nl, ts_off, pbs, has_ts ? tsbs : nullptr, ws,
                             L.nqb_cap, L.item_cap, grid, st);
  if (e != hipSuccess) return HSTU_ERR_HIP;
  if (!any_rows) return HSTU_OK;
  for (int l = 0; l < nl; ++l) {
    WsPtrs wl = ws;
    wl.row_loc = ws.row_loc + static_cast<size_t>(l) * d.total_new;   // this layer's pool slots
    e = launch_gemm_qkv(d, l == 0 ? x : ys[l - 1], w1s[l], kps[l], vps[l], wl, st);
    if (e != hipSuccess) return HSTU_ERR_HIP;
    e = launch_attn(d, pts[l], kps[l], vps[l], l, ts, ts_off, ncand, ws, grid < L.item_cap ? grid : L.item_cap, st);
    if (e != hipSuccess) return HSTU_ERR_HIP;
    e = launch_norm_gate(d, ws, L.nqb_cap, st);
    if (e != hipSuccess) return HSTU_ERR_HIP;
    e = launch_gemm_out(d, ws.q, w2s[l], ys[l], &ws.hdr->status, st);
    if (e != hipSuccess) return HSTU_ERR_HIP;
  }
  return HSTU_OK;
}

// The address of `scratch` on the current device (see the top of this file).
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_base_of[kMaxDevices];

hstu_status scratch_base(void** base) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HSTU_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_base_of[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return HSTU_ERR_HIP;
    scratch_base_of[dev] = p;
  }
  *base = scratch_base_of[dev];
  return HSTU_OK;
}

// Copies the call's status word (workspace header) to the caller's int.
__global__ void copy_status_kernel(const WsHeader* hdr, int32_t* out) {
  if (threadIdx.x == 0) *out = hdr->status;
}

}  // namespace

extern "C" {

hstu_status hstu_stack_workspace_size(const hstu_layer_desc* desc, int32_t num_layers, size_t* bytes) {
  hstu_status s = check_layer(desc);
  if (s != HSTU_OK) return s;
  if (bytes == nullptr || num_layers < 1 || num_layers > kMaxStackLayers) return HSTU_ERR_INVALID_ARG;
  *bytes = make_layout(*desc, attn_grid(), num_layers).total;
  return HSTU_OK;
}

hstu_status hstu_stack_fwd(const hstu_layer_desc* desc, int32_t num_layers, const void* x,
                           const int32_t* new_offsets, const int32_t* hist_len, const int32_t* num_candidates,
                           const int32_t* const* page_tables, void* const* k_pools, void* const* v_pools,
                           const void* const* w1t, const void* const* w2t, const float* const* pos_bias,
                           const float* const* ts_bias, const int64_t* timestamps, const int32_t* ts_offsets,
                           void* const* y, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return stack_impl(desc, num_layers, x, new_offsets, hist_len, num_candidates, page_tables, k_pools, v_pools, w1t,
                    w2t, pos_bias, ts_bias, timestamps, ts_offsets, y, workspace, workspace_bytes, hip_stream);
}

hstu_status hstu_layer_workspace_size(const hstu_layer_desc* desc, size_t* bytes) {
  hstu_status s = check_layer(desc);
  if (s != HSTU_OK) return s;
  if (bytes == nullptr) return HSTU_ERR_INVALID_ARG;
  *bytes = make_layout(*desc, attn_grid()).total;
  return HSTU_OK;
}

hstu_status hstu_layer_fwd(const hstu_layer_desc* desc, const void* x, const int32_t* new_offsets,
                           const int32_t* hist_len, const int32_t* page_table, void* k_pool, void* v_pool,
                           const void* w1t, const void* w2t, const float* pos_bias, const float* ts_bias,
                           const int64_t* timestamps, const int32_t* ts_offsets, void* y, void* workspace,
                           size_t workspace_bytes, void* hip_stream) {
  return layer_impl(desc, x, new_offsets, hist_len, nullptr, page_table, k_pool, v_pool, w1t, w2t, pos_bias,
                    ts_bias, timestamps, ts_offsets, y, workspace, workspace_bytes, hip_stream, nullptr);
}

hstu_status hstu_layer_fwd_noalloc(const hstu_layer_desc* desc, const void* x, const int32_t* new_offsets,
                                   const int32_t* hist_len, const int32_t* page_table, void* k_pool,
                                   void* v_pool, const void* w1t, const void* w2t, const float* pos_bias,
                                   const float* ts_bias, const int64_t* timestamps, const int32_t* ts_offsets,
                                   void* y, int32_t* device_status, void* hip_stream) {
  hstu_status s = check_layer(desc);
  if (s != HSTU_OK) return s;
  if (device_status == nullptr) return HSTU_ERR_INVALID_ARG;
  if (make_layout(*desc, attn_grid()).total > HSTU_NOALLOC_SCRATCH_BYTES) return HSTU_ERR_SCRATCH;
  void* base = nullptr;
  s = scratch_base(&base);
  if (s != HSTU_OK) return s;
  s = layer_impl(desc, x, new_offsets, hist_len, nullptr, page_table, k_pool, v_pool, w1t, w2t, pos_bias,
                 ts_bias, timestamps, ts_offsets, y, base, HSTU_NOALLOC_SCRATCH_BYTES, hip_stream, nullptr);
  if (s != HSTU_OK) return s;
  copy_status_kernel<<<1, 64, 0, static_cast<hipStream_t>(hip_stream)>>>(static_cast<const WsHeader*>(base),
                                                                        device_status);
  return hipGetLastError() == hipSuccess ? HSTU_OK : HSTU_ERR_HIP;
}

hstu_status hstu_layer_fwd_timed(const hstu_layer_desc* desc, const void* x, const int32_t* new_offsets,
                                 const int32_t* hist_len, const int32_t* page_table, void* k_pool,
                                 void* v_pool, const void* w1t, const void* w2t, const float* pos_bias,
                                 const float* ts_bias, const int64_t* timestamps, const int32_t* ts_offsets,
                                 void* y, void* workspace, size_t workspace_bytes, void* hip_stream,
                                 void* const* stage_events) {
  return layer_impl(desc, x, new_offsets, hist_len, nullptr, page_table, k_pool, v_pool, w1t, w2t, pos_bias,
                    ts_bias, timestamps, ts_offsets, y, workspace, workspace_bytes, hip_stream, stage_events);
}

hstu_status hstu_layer_fwd_cand(const hstu_layer_desc* desc, const void* x, const int32_t* new_offsets,
                                const int32_t* hist_len, const int32_t* num_candidates,
                                const int32_t* page_table, void* k_pool, void* v_pool, const void* w1t,
                                const void* w2t, const float* pos_bias, const float* ts_bias,
                                const int64_t* timestamps, const int32_t* ts_offsets, void* y,
                                void* workspace, size_t workspace_bytes, void* hip_stream,
                                void* const* stage_events) {
  if (num_candidates == nullptr) return HSTU_ERR_INVALID_ARG;
  return layer_impl(desc, x, new_offsets, hist_len, num_candidates, page_table, k_pool, v_pool, w1t, w2t,
                    pos_bias, ts_bias, timestamps, ts_offsets, y, workspace, workspace_bytes, hip_stream,
                    stage_events);
}

hstu_status kv_pages_append(const hstu_layer_desc* desc, const void* k_new, const void* v_new,
                            const int32_t* new_offsets, const int32_t* hist_len, const int32_t* page_table,
                            void* k_pool, void* v_pool, int32_t* device_status, void* hip_stream) {
  hstu_status s = check_common(desc);
  if (s != HSTU_OK) return s;
  if (new_offsets == nullptr || hist_len == nullptr || page_table == nullptr || k_pool == nullptr ||
      v_pool == nullptr || device_status == nullptr)
    return HSTU_ERR_INVALID_ARG;
  if (desc->total_new > 0 && (k_new == nullptr || v_new == nullptr)) return HSTU_ERR_INVALID_ARG;
  hipError_t e = launch_append(*desc, k_new, v_new, new_offsets, hist_len, page_table, k_pool, v_pool,
                               device_status, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? HSTU_OK : HSTU_ERR_HIP;
}

hstu_status hstu_read_device_status(const void* device_status, int32_t* code, void* hip_stream) {
  if (device_status == nullptr || code == nullptr) return HSTU_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (hipStreamSynchronize(st) != hipSuccess) return HSTU_ERR_HIP;
  if (hipMemcpy(code, device_status, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess) return HSTU_ERR_HIP;
  return *code == 0 ? HSTU_OK : HSTU_ERR_DEVICE;
}

const char* hstu_status_string(int32_t status) {
  switch (status) {
    case HSTU_OK: return "ok";
    case HSTU_ERR_INVALID_ARG: return "invalid argument";
    case HSTU_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case HSTU_ERR_WORKSPACE: return "workspace too small";
    case HSTU_ERR_HIP: return "HIP runtime error";
    case HSTU_ERR_DEVICE: return "device status reports an error";
    case HSTU_ERR_SCRATCH: return "call needs more workspace than the library's static scratch array";
    case HSTU_DEV_BAD_OFFSETS: return "device: new_offsets not a prefix sum ending at total_new";
    case HSTU_DEV_BAD_HIST: return "device: negative hist_len";
    case HSTU_DEV_CAPACITY: return "device: sequence longer than its page-table row";
    case HSTU_DEV_BAD_PAGE: return "device: page id outside the pool";
    case HSTU_DEV_BAD_TS: return "device: ts_offsets do not match sequence lengths";
    case HSTU_DEV_BAD_CANDIDATES: return "device: a candidate count outside [0, new rows]";
    case HSTU_DEV_BAD_TOKEN: return "device: a token id outside its embedding table";
    case HSTU_DEV_BAD_POSITION: return "device: a position outside the position table";
    case HSTU_DEV_BAD_CTX_LEN: return "device: a context length outside [0, max_ctx]";
    case HSTU_DEV_BAD_PATH: return "device: a beam path slot outside [0, beam width)";
    default: return "unknown status";
  }
}

}  // extern "C"
