// kv_pages_append: the paged KV table's append (NVIDIA blog "Deploying an
// HSTU generative recommender with NVIDIA Dynamo-Triton", section "Why
// serving large sequential recommenders is hard").  Row t of user u goes to
// position hist[u] + t, i.e. page page_table[u][p / ps], slot p % ps; K rows
// are copied as contiguous d-element runs, V columns into the transposed
// per-page layout.  A single-workgroup validation kernel runs first and the
// scatter writes nothing unless it reported success.
#include "common.h"

namespace hstu {
namespace {

struct AppendMeta {
  const int32_t* new_off;
  const int32_t* hist;
  const int32_t* pt;
  int32_t* status;
  int B, T, H, hd, ps, maxP;
  int64_t P;
};

__global__ __launch_bounds__(256) void append_validate_kernel(AppendMeta m) {
  __shared__ int s_err;
  const int tid = threadIdx.x;
  if (tid == 0) s_err = 0;
  __syncthreads();
  if (tid == 0 && m.B == 0 && m.T != 0) atomicCAS(&s_err, 0, HSTU_DEV_BAD_OFFSETS);
  for (int u = tid; u < m.B; u += 256) {
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
    for (int u = 0; u < m.B; ++u) {
      const int n = m.new_off[u + 1] - m.new_off[u];
      if (n == 0) continue;
      const int c = m.hist[u];
      const int first = c / m.ps, last = (c + n - 1) / m.ps;
      const int32_t* row = m.pt + static_cast<size_t>(u) * m.maxP;
      for (int j = first + tid; j <= last; j += 256) {
        const int32_t pg = row[j];
        if (pg < 0 || pg >= m.P) atomicCAS(&s_err, 0, HSTU_DEV_BAD_PAGE);
      }
    }
  }
  __syncthreads();
  if (tid == 0) *m.status = s_err;
}

// One thread per (row, head, 8-element group of the head dim).
template <typename T>
__global__ __launch_bounds__(256) void append_scatter_kernel(AppendMeta m, const T* __restrict__ k_new,
                                                             const T* __restrict__ v_new,
                                                             T* __restrict__ k_pool, T* __restrict__ v_pool) {
  if (*m.status != 0) return;
  const int groups = m.hd / 8;
  const int64_t total = static_cast<int64_t>(m.T) * m.H * groups;
  const int D = m.H * m.hd;
  for (int64_t idx = blockIdx.x * 256ll + threadIdx.x; idx < total; idx += static_cast<int64_t>(gridDim.x) * 256) {
    const int r = static_cast<int>(idx / (m.H * groups));
    const int rem = static_cast<int>(idx % (m.H * groups));
    const int h = rem / groups, e0 = (rem % groups) * 8;
    const int u = row_to_user(m.new_off, m.B, r);
    const int p = m.hist[u] + r - m.new_off[u];
    const size_t page = static_cast<size_t>(m.pt[static_cast<size_t>(u) * m.maxP + p / m.ps]);
    const int slot = p % m.ps;
    const size_t src = static_cast<size_t>(r) * D + h * m.hd + e0;
    T* kd = k_pool + ((page * m.H + h) * m.ps + slot) * m.hd + e0;
    T* vd = v_pool + ((page * m.H + h) * m.hd + e0) * m.ps + slot;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kd[e] = k_new[src + e];
      vd[static_cast<size_t>(e) * m.ps] = v_new[src + e];
    }
  }
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
  append_validate_kernel<<<1, 256, 0, stream>>>(m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || d.total_new == 0) return e;
  const int64_t total = static_cast<int64_t>(d.total_new) * d.num_heads * (d.head_dim / 8);
  int grid = static_cast<int>((total + 255) / 256);
  if (grid > 65536) grid = 65536;
  if (d.dtype == HSTU_BF16)
    append_scatter_kernel<bf16><<<grid, 256, 0, stream>>>(m, static_cast<const bf16*>(k_new), static_cast<const bf16*>(v_new),
                                                          static_cast<bf16*>(k_pool), static_cast<bf16*>(v_pool));
  else
    append_scatter_kernel<float><<<grid, 256, 0, stream>>>(m, static_cast<const float*>(k_new), static_cast<const float*>(v_new),
                                                           static_cast<float*>(k_pool), static_cast<float*>(v_pool));
  return hipGetLastError();
}

}  // namespace hstu
