// kv_pages_append: the paged KV table's append (NVIDIA blog "Deploying an
// HSTU generative recommender with NVIDIA Dynamo-Triton", section "Why
// serving large sequential recommenders is hard").  Row t of user u goes to
// position hist[u] + t, i.e. page page_table[u][p / ps], slot p % ps.
//
// A single-workgroup validation kernel runs first (offsets, history
// lengths, capacity, then every page id the append touches, checked over a
// flat (user, page) index so that the loads go out back to back), and the
// scatter writes nothing unless it reported success.  The scatter takes a
// tile of 64 consecutive rows and one head per workgroup: K rows are copied
// as contiguous d-element runs with 16-byte accesses; the V tile is staged
// in LDS and written transposed, each wave storing one head-dim index for
// 64 rows at once, i.e. runs of consecutive slots of a page.
#include "common.h"

namespace hstu {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kTileRows = 64;

struct AppendMeta {
  const int32_t* new_off;
  const int32_t* hist;
  const int32_t* pt;
  int32_t* status;
  int B, T, H, hd, ps, maxP;
  int64_t P;
};

__global__ __launch_bounds__(kAppendThreads) void append_validate_kernel(AppendMeta m) {
  __shared__ int s_err;
  __shared__ int s_wsum[kAppendThreads / 64];
  __shared__ int32_t s_pgp[kMaxUsers + 1];     // first flat page index of each user's append
  const int tid = threadIdx.x;
  if (tid == 0) s_err = 0;
  __syncthreads();
  if (tid == 0 && m.B == 0 && m.T != 0) atomicCAS(&s_err, 0, HSTU_DEV_BAD_OFFSETS);
  for (int u = tid; u < m.B; u += kAppendThreads) {
    const int o0 = m.new_off[u], o1 = m.new_off[u + 1];
    if ((u == 0 && o0 != 0) || o1 < o0 || (u == m.B - 1 && o1 != m.T)) atomicCAS(&s_err, 0, HSTU_DEV_BAD_OFFSETS);
    const int c = m.hist[u];
    if (c < 0)
      atomicCAS(&s_err, 0, HSTU_DEV_BAD_HIST);
    else if (static_cast<int64_t>(c) + (o1 - o0) > static_cast<int64_t>(m.maxP) * m.ps)
      atomicCAS(&s_err, 0, HSTU_DEV_CAPACITY);
  }
  __syncthreads();
  if (s_err == 0) {
    // pages each user's append touches, then their exclusive prefix sum
    const int seg = (m.B + kAppendThreads - 1) / kAppendThreads;
    const int lo = min(m.B, tid * seg), hi = min(m.B, lo + seg);
    int run = 0;
    for (int u = lo; u < hi; ++u) {
      const int n = m.new_off[u + 1] - m.new_off[u], c = m.hist[u];
      const int np = n == 0 ? 0 : (c + n - 1) / m.ps - c / m.ps + 1;
      s_pgp[u] = np;
      run += np;
    }
    int incl = run;                           // inclusive scan of the per-thread sums
    const int lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) s_wsum[w] = incl;
    __syncthreads();
    int before = 0, total = 0;
    for (int i = 0; i < kAppendThreads / 64; ++i) {
      if (i < w) before += s_wsum[i];
      total += s_wsum[i];
    }
    int acc = before + incl - run;
    for (int u = lo; u < hi; ++u) {
      const int np = s_pgp[u];
      s_pgp[u] = acc;
      acc += np;
    }
    __syncthreads();
    constexpr int kU = 4;
    bool bad = false;
    for (int i0 = tid; i0 < total; i0 += kU * kAppendThreads) {
      int32_t pg[kU];
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        const int i = i0 + k * kAppendThreads;
        pg[k] = 0;
        if (i < total) {
          int a = 0, b = m.B - 1;                  // user owning flat page i
          while (a < b) {
            const int mid = (a + b + 1) >> 1;
            if (s_pgp[mid] <= i) a = mid; else b = mid - 1;
          }
          pg[k] = m.pt[static_cast<size_t>(a) * m.maxP + m.hist[a] / m.ps + (i - s_pgp[a])];
        }
      }
#pragma unroll
      for (int k = 0; k < kU; ++k) bad |= pg[k] < 0 || pg[k] >= m.P;
    }
    if (bad) atomicCAS(&s_err, 0, HSTU_DEV_BAD_PAGE);
  }
  __syncthreads();
  if (tid == 0) *m.status = s_err;
}

// One workgroup per (64-row tile, head).  HD: head dim.
template <typename T, int HD>
__global__ __launch_bounds__(kAppendThreads) void append_scatter_kernel(AppendMeta m, const T* __restrict__ k_new,
                                                                        const T* __restrict__ v_new,
                                                                        T* __restrict__ k_pool, T* __restrict__ v_pool) {
  constexpr int ES = static_cast<int>(sizeof(T));
  constexpr int CE = 16 / ES;                    // elements per 16-byte chunk
  constexpr int CPR = HD / CE;                   // chunks per head row
  constexpr int PITCH = HD + 2;                  // LDS row pitch (elements): column reads spread over banks
  __shared__ T s_v[kTileRows * PITCH];
  __shared__ int64_t s_kbase[kTileRows];         // element offset of the row's K run (head 0)
  __shared__ int64_t s_vbase[kTileRows];         // element offset of the row's V slot (head 0, e = 0)
  if (*m.status != 0) return;
  const int tid = threadIdx.x;
  const int r0 = blockIdx.x * kTileRows, h = blockIdx.y;
  const int rows = min(kTileRows, m.T - r0);
  const int D = m.H * HD;
  if (tid < rows) {
    const int r = r0 + tid;
    const int u = row_to_user(m.new_off, m.B, r);
    const int p = m.hist[u] + r - m.new_off[u];
    const int64_t page = m.pt[static_cast<size_t>(u) * m.maxP + p / m.ps];
    const int slot = p % m.ps;
    s_kbase[tid] = ((page * m.H) * m.ps + slot) * HD;
    s_vbase[tid] = (page * m.H) * HD * m.ps + slot;
  }
  __syncthreads();
  const int64_t head_k = static_cast<int64_t>(h) * m.ps * HD;   // head block inside a page
  // K rows straight through, V rows into the LDS tile (16-byte chunks)
  for (int c = tid; c < rows * CPR; c += kAppendThreads) {
    const int row = c / CPR, ch = c % CPR;
    const size_t src = static_cast<size_t>(r0 + row) * D + h * HD + ch * CE;
    const u32x4 kv = *reinterpret_cast<const u32x4*>(k_new + src);
    const u32x4 vv = *reinterpret_cast<const u32x4*>(v_new + src);
    *reinterpret_cast<u32x4*>(k_pool + s_kbase[row] + head_k + ch * CE) = kv;
    const T* ve = reinterpret_cast<const T*>(&vv);
#pragma unroll
    for (int e = 0; e < CE; ++e) s_v[row * PITCH + ch * CE + e] = ve[e];
  }
  __syncthreads();
  // V^T: lane = row, each wave walks head-dim indices, so a store
  // instruction covers 64 consecutive slots (or page-split runs of them)
  const int lane = tid & 63, w = tid >> 6;
  if (lane < rows) {
    T* vb = v_pool + s_vbase[lane] + static_cast<int64_t>(h) * HD * m.ps;
    for (int e = w; e < HD; e += kAppendThreads / 64)
      vb[static_cast<int64_t>(e) * m.ps] = s_v[lane * PITCH + e];
  }
}

template <typename T>
hipError_t scatter_t(const hstu_layer_desc& d, const AppendMeta& m, const void* k_new, const void* v_new,
                     void* k_pool, void* v_pool, hipStream_t stream) {
  const dim3 grid((d.total_new + kTileRows - 1) / kTileRows, d.num_heads);
  const T* kn = static_cast<const T*>(k_new);
  const T* vn = static_cast<const T*>(v_new);
  T* kp = static_cast<T*>(k_pool);
  T* vp = static_cast<T*>(v_pool);
  switch (d.head_dim) {
    case 32: append_scatter_kernel<T, 32><<<grid, kAppendThreads, 0, stream>>>(m, kn, vn, kp, vp); break;
    case 64: append_scatter_kernel<T, 64><<<grid, kAppendThreads, 0, stream>>>(m, kn, vn, kp, vp); break;
    default: append_scatter_kernel<T, 128><<<grid, kAppendThreads, 0, stream>>>(m, kn, vn, kp, vp); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const hstu_layer_desc& d, const void* k_new, const void* v_new,
                         const int32_t* new_off, const int32_t* hist, const int32_t* pt,
                         void* k_pool, void* v_pool, int32_t* status, hipStream_t stream) {
  AppendMeta m;
  m.new_off = new_off;
  m.hist = hist;
  m.pt = pt;
  m.status = status;
  m.B = d.num_users;
  m.T = d.total_new;
  m.H = d.num_heads;
  m.hd = d.head_dim;
  m.ps = d.page_size;
  m.maxP = d.max_pages_per_user;
  m.P = d.num_pool_pages;
  append_validate_kernel<<<1, kAppendThreads, 0, stream>>>(m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || d.total_new == 0) return e;
  if (d.dtype == HSTU_BF16) return scatter_t<bf16>(d, m, k_new, v_new, k_pool, v_pool, stream);
  return scatter_t<float>(d, m, k_new, v_new, k_pool, v_pool, stream);
}

}  // namespace hstu
