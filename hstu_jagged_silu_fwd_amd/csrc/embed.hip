// Input preprocessing: the layer's input rows built from categorical tokens
// (NVIDIA blog "Deploying an HSTU generative recommender with NVIDIA
// Dynamo-Triton", section "Why use HSTU for generative recommendation":
// embedding lookup, item/action interleave when action tokens exist, context
// appended, positional encoding).  Row t of user u, at position
// hist_len[u] + t, is table[id] + pos_emb[position]; a user's rows are its
// context tokens, its history entries (item row, then action row), then its
// candidate items.
//
// Two kernels.  The scan (one workgroup) checks the jagged offsets and the
// positions and writes the layer's new_offsets and candidate counts.  The
// row builder is a pure gather: every thread moves one 16-byte chunk of one
// row (two loads, an fp32 add, one store); a row of D = 512 bf16 is exactly
// one wave, so a wave's loads are two contiguous 1 KiB runs and its store
// one.  It is bound by HBM bandwidth: 3 * D * sizeof(dtype) bytes per row.
#include "common.h"

namespace hstu {
namespace {

constexpr int kScanThreads = 1024;
constexpr int kRowThreads = 256;

struct ScanArgs {
  const int32_t* hist;
  const int32_t* ctx_off;
  const int32_t* hist_off;
  const int32_t* cand_off;
  int32_t* new_off;
  int32_t* ncand;
  int32_t* status;
  int B, T, max_pos, pair_rows;    // pair_rows: rows per history entry (2 with actions, else 1)
};

// Checks and prefix sums in chunks of kScanThreads users (an LDS scan per
// chunk, carried across chunks).  First failure in the order of the codes'
// listing: offsets, history, position.
__global__ __launch_bounds__(kScanThreads) void token_scan_kernel(ScanArgs a) {
  __shared__ int32_t s_val[kScanThreads];
  __shared__ int s_bad_off, s_bad_hist, s_bad_pos;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_bad_off = (a.ctx_off[0] != 0) | (a.hist_off[0] != 0) | (a.cand_off[0] != 0);
    s_bad_hist = 0;
    s_bad_pos = 0;
  }
  __syncthreads();
  int64_t carry = 0;
  for (int u0 = 0; u0 < a.B; u0 += kScanThreads) {
    const int u = u0 + tid;
    int rows = 0;
    if (u < a.B) {
      const int nc = a.ctx_off[u + 1] - a.ctx_off[u];
      const int nh = a.hist_off[u + 1] - a.hist_off[u];
      const int nm = a.cand_off[u + 1] - a.cand_off[u];
      const int c = a.hist[u];
      if (nc < 0 || nh < 0 || nm < 0) atomicOr(&s_bad_off, 1);
      if (c < 0) atomicOr(&s_bad_hist, 1);
      const int64_t r64 = static_cast<int64_t>(max(nc, 0)) + static_cast<int64_t>(a.pair_rows) * max(nh, 0) +
                          max(nm, 0);
      if (r64 > a.T) atomicOr(&s_bad_off, 1);
      rows = static_cast<int>(min<int64_t>(r64, a.T));
      if (static_cast<int64_t>(c) + r64 > a.max_pos) atomicOr(&s_bad_pos, 1);
      a.ncand[u] = max(nm, 0);
    }
    // inclusive scan of the chunk's row counts (Hillis-Steele in LDS)
    s_val[tid] = rows;
    __syncthreads();
    for (int d = 1; d < kScanThreads; d <<= 1) {
      const int v = tid >= d ? s_val[tid - d] : 0;
      __syncthreads();
      s_val[tid] += v;
      __syncthreads();
    }
    if (u < a.B) a.new_off[u] = static_cast<int32_t>(min<int64_t>(carry + s_val[tid] - rows, a.T));
    carry += s_val[kScanThreads - 1];
    __syncthreads();
  }
  if (tid == 0) {
    if (carry != a.T) s_bad_off = 1;
    a.new_off[a.B] = static_cast<int32_t>(min<int64_t>(carry, a.T));
    int code = HSTU_DEV_OK;
    if (s_bad_off) code = HSTU_DEV_BAD_OFFSETS;
    else if (s_bad_hist) code = HSTU_DEV_BAD_HIST;
    else if (s_bad_pos) code = HSTU_DEV_BAD_POSITION;
    *a.status = code;
  }
}

struct RowArgs {
  const int32_t* hist;
  const int32_t* ctx_off;
  const int64_t* ctx_ids;
  const int32_t* hist_off;
  const int64_t* item_ids;
  const int64_t* action_ids;      // null: no action tokens
  const int32_t* cand_off;
  const int64_t* cand_ids;
  const char* item_emb;
  const char* action_emb;
  const char* ctx_emb;
  const char* pos_emb;
  const int32_t* new_off;
  char* x;
  int32_t* status;
  int64_t item_rows, action_rows, ctx_rows;
  int B, row_bytes, chunks;         // chunks: 16-byte pieces per row
  int64_t n_chunks;                 // T * chunks
};

template <typename T>
__device__ __forceinline__ uint4 add_chunks(uint4 a, uint4 b) {
  constexpr int N = 16 / sizeof(T);
  const T* pa = reinterpret_cast<const T*>(&a);
  const T* pb = reinterpret_cast<const T*>(&b);
  uint4 r;
  T* pr = reinterpret_cast<T*>(&r);
#pragma unroll
  for (int i = 0; i < N; ++i) pr[i] = from_f32<T>(to_f32(pa[i]) + to_f32(pb[i]));
  return r;
}

template <typename T>
__global__ __launch_bounds__(kRowThreads) void token_rows_kernel(RowArgs a) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kRowThreads + threadIdx.x;
  if (idx >= a.n_chunks) return;
  if (*a.status != 0) return;                 // the scan rejected the call
  const int row = static_cast<int>(idx / a.chunks);
  const int ch = static_cast<int>(idx - static_cast<int64_t>(row) * a.chunks);
  // user of the row: the last u with new_off[u] <= row (users without rows
  // share their offset with the next one, so the search takes the last)
  int lo = 0, hi = a.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.new_off[mid] <= row) lo = mid; else hi = mid - 1;
  }
  const int u = lo;
  const int t = row - a.new_off[u];
  const int nc = a.ctx_off[u + 1] - a.ctx_off[u];
  const int nh = a.hist_off[u + 1] - a.hist_off[u];
  const bool acts = a.action_ids != nullptr;
  const int hr = acts ? 2 * nh : nh;
  int64_t id;
  const char* tab;
  int64_t nrows;
  if (t < nc) {
    id = a.ctx_ids[a.ctx_off[u] + t];
    tab = a.ctx_emb;
    nrows = a.ctx_rows;
  } else if (t < nc + hr) {
    const int k = t - nc;
    const int e = acts ? (k >> 1) : k;
    const bool is_action = acts && (k & 1);
    id = is_action ? a.action_ids[a.hist_off[u] + e] : a.item_ids[a.hist_off[u] + e];
    tab = is_action ? a.action_emb : a.item_emb;
    nrows = is_action ? a.action_rows : a.item_rows;
  } else {
    id = a.cand_ids[a.cand_off[u] + (t - nc - hr)];
    tab = a.item_emb;
    nrows = a.item_rows;
  }
  if (id < 0 || id >= nrows) {
    atomicCAS(a.status, 0, static_cast<int32_t>(HSTU_DEV_BAD_TOKEN));
    return;
  }
  const int64_t pos = static_cast<int64_t>(a.hist[u]) + t;   // < max_positions (checked by the scan)
  const uint4 ev = *reinterpret_cast<const uint4*>(tab + id * a.row_bytes + 16 * ch);
  const uint4 pv = *reinterpret_cast<const uint4*>(a.pos_emb + pos * a.row_bytes + 16 * ch);
  *reinterpret_cast<uint4*>(a.x + static_cast<int64_t>(row) * a.row_bytes + 16 * ch) = add_chunks<T>(ev, pv);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace
}  // namespace hstu

using namespace hstu;

extern "C" hstu_status hstu_preprocess(const hstu_prep_desc* d, const int32_t* hist_len,
                                       const int32_t* ctx_offsets, const int64_t* ctx_ids,
                                       const int32_t* hist_offsets, const int64_t* item_ids,
                                       const int64_t* action_ids, const int32_t* cand_offsets,
                                       const int64_t* cand_ids, const void* item_emb,
                                       const void* action_emb, const void* ctx_emb, const void* pos_emb,
                                       void* x, int32_t* new_offsets, int32_t* num_candidates,
                                       int32_t* device_status, void* hip_stream) {
  if (d == nullptr) return HSTU_ERR_INVALID_ARG;
  if (d->num_users > kMaxUsers || d->total_new > kMaxRows) return HSTU_ERR_UNSUPPORTED;
  if (d->dtype != HSTU_F32 && d->dtype != HSTU_BF16) return HSTU_ERR_UNSUPPORTED;
  if (d->hidden % 64 != 0 || d->hidden > 2048) return HSTU_ERR_UNSUPPORTED;
  if (d->num_users < 0 || d->total_new < 0 || d->hidden < 64 || d->item_rows < 1 || d->ctx_rows < 1 ||
      d->action_rows < 0 || d->max_positions < 1)
    return HSTU_ERR_INVALID_ARG;
  const bool acts = d->action_rows > 0;
  const bool users = d->num_users > 0;             // [B] arrays may be NULL for an empty batch
  if ((users && (hist_len == nullptr || num_candidates == nullptr)) || ctx_offsets == nullptr ||
      hist_offsets == nullptr || cand_offsets == nullptr || new_offsets == nullptr || device_status == nullptr ||
      item_emb == nullptr || ctx_emb == nullptr || pos_emb == nullptr || (acts && action_emb == nullptr))
    return HSTU_ERR_INVALID_ARG;
  if (d->total_new > 0 && (x == nullptr || ctx_ids == nullptr || item_ids == nullptr || cand_ids == nullptr ||
                           (acts && action_ids == nullptr)))
    return HSTU_ERR_INVALID_ARG;
  if (!aligned16(item_emb) || !aligned16(ctx_emb) || !aligned16(pos_emb) || (acts && !aligned16(action_emb)) ||
      (x != nullptr && !aligned16(x)))
    return HSTU_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const int es = d->dtype == HSTU_BF16 ? 2 : 4;

  ScanArgs sa;
  sa.hist = hist_len;
  sa.ctx_off = ctx_offsets;
  sa.hist_off = hist_offsets;
  sa.cand_off = cand_offsets;
  sa.new_off = new_offsets;
  sa.ncand = num_candidates;
  sa.status = device_status;
  sa.B = d->num_users;
  sa.T = d->total_new;
  sa.max_pos = d->max_positions;
  sa.pair_rows = acts ? 2 : 1;
  if (launch_kernel(token_scan_kernel, dim3(1), dim3(kScanThreads), st, KernelEvents{}, sa) != hipSuccess)
    return HSTU_ERR_HIP;
  if (d->total_new == 0) return HSTU_OK;

  RowArgs ra;
  ra.hist = hist_len;
  ra.ctx_off = ctx_offsets;
  ra.ctx_ids = ctx_ids;
  ra.hist_off = hist_offsets;
  ra.item_ids = item_ids;
  ra.action_ids = acts ? action_ids : nullptr;
  ra.cand_off = cand_offsets;
  ra.cand_ids = cand_ids;
  ra.item_emb = static_cast<const char*>(item_emb);
  ra.action_emb = static_cast<const char*>(action_emb);
  ra.ctx_emb = static_cast<const char*>(ctx_emb);
  ra.pos_emb = static_cast<const char*>(pos_emb);
  ra.new_off = new_offsets;
  ra.x = static_cast<char*>(x);
  ra.status = device_status;
  ra.item_rows = d->item_rows;
  ra.action_rows = d->action_rows;
  ra.ctx_rows = d->ctx_rows;
  ra.B = d->num_users;
  ra.row_bytes = d->hidden * es;
  ra.chunks = ra.row_bytes / 16;
  ra.n_chunks = static_cast<int64_t>(d->total_new) * ra.chunks;
  const dim3 grid(static_cast<unsigned>((ra.n_chunks + kRowThreads - 1) / kRowThreads));
  hipError_t e = d->dtype == HSTU_BF16
                     ? launch_kernel(token_rows_kernel<bf16>, grid, dim3(kRowThreads), st, KernelEvents{}, ra)
                     : launch_kernel(token_rows_kernel<float>, grid, dim3(kRowThreads), st, KernelEvents{}, ra);
  return e == hipSuccess ? HSTU_OK : HSTU_ERR_HIP;
}
