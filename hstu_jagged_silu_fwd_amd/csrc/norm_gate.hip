// Row norm and gating: O = attn_scale * (sum of the row's chunk partials, in
// chunk order; the partials hold -log2(e) * sum SiLU(s) v, undone here), then
// G = LayerNorm_row(O) * U, the elementwise gating that precedes the output
// projection (aitrends.kr article 100093, "HSTU
// sequential modelling").  One wavefront per row; mean and variance come from
// wavefront reductions over the row's D entries (population variance, no
// affine).  G overwrites the Q buffer, which is dead after the attention.
#include "common.h"

namespace hstu {
namespace {

constexpr int kMaxGroups = 8;    // D <= 64 lanes * 4 * 8 = 2048

template <typename T>
struct NormArgs {
  const int32_t* new_off;
  const int32_t* row_user;
  const int32_t* qb_base;
  const int32_t* qb_first;
  const int32_t* qb_nch;
  const float* part;
  const T* u;
  T* g;
  const int32_t* status;
  int T_rows, D, hd;
  float scale, eps;
};

template <typename T>
__device__ __forceinline__ void load4(const T* p, float* x);
template <>
__device__ __forceinline__ void load4<float>(const float* p, float* x) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
template <>
__device__ __forceinline__ void load4<bf16>(const bf16* p, float* x) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  x[0] = static_cast<float>(v[0]); x[1] = static_cast<float>(v[1]);
  x[2] = static_cast<float>(v[2]); x[3] = static_cast<float>(v[3]);
}
template <typename T>
__device__ __forceinline__ void store4(T* p, const float* x);
template <>
__device__ __forceinline__ void store4<float>(float* p, const float* x) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, const float* x) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 v;
  v[0] = static_cast<bf16>(x[0]); v[1] = static_cast<bf16>(x[1]);
  v[2] = static_cast<bf16>(x[2]); v[3] = static_cast<bf16>(x[3]);
  *reinterpret_cast<bf16x4*>(p) = v;
}

template <typename T>
__global__ __launch_bounds__(256) void norm_gate_kernel(NormArgs<T> a) {
  if (*a.status != 0) return;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= a.T_rows) return;
  const int u = a.row_user[r];
  const int t = r - a.new_off[u];
  const int qbe = a.qb_base[u] + t / kQB;
  const int tl = t % kQB;
  const int first = a.qb_first[qbe];
  const int nch = a.qb_nch[qbe];
  const int D = a.D;

  float x[kMaxGroups][4];
  float s1 = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxGroups; ++k) {
    const int col = (k * 64 + lane) * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) x[k][j] = 0.f;
    if (col < D) {
      const int h = col / a.hd, e = col % a.hd;
      const float* src = a.part + (static_cast<size_t>(first + h * nch) * kQB + tl) * a.hd + e;
      const size_t stride = static_cast<size_t>(kQB) * a.hd;
      int kc = 0;
      for (; kc + 4 <= nch; kc += 4) {   // four independent loads in flight, summed in chunk order
        const float4 v0 = *reinterpret_cast<const float4*>(src + (kc + 0) * stride);
        const float4 v1 = *reinterpret_cast<const float4*>(src + (kc + 1) * stride);
        const float4 v2 = *reinterpret_cast<const float4*>(src + (kc + 2) * stride);
        const float4 v3 = *reinterpret_cast<const float4*>(src + (kc + 3) * stride);
        x[k][0] += v0.x; x[k][1] += v0.y; x[k][2] += v0.z; x[k][3] += v0.w;
        x[k][0] += v1.x; x[k][1] += v1.y; x[k][2] += v1.z; x[k][3] += v1.w;
        x[k][0] += v2.x; x[k][1] += v2.y; x[k][2] += v2.z; x[k][3] += v2.w;
        x[k][0] += v3.x; x[k][1] += v3.y; x[k][2] += v3.z; x[k][3] += v3.w;
      }
      for (; kc < nch; ++kc) {
        const float4 v = *reinterpret_cast<const float4*>(src + kc * stride);
        x[k][0] += v.x; x[k][1] += v.y; x[k][2] += v.z; x[k][3] += v.w;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[k][j] *= a.scale;
        s1 += x[k][j];
      }
    }
  }
  const float mean = wave_sum(s1) / static_cast<float>(D);
  float s2 = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxGroups; ++k) {
    const int col = (k * 64 + lane) * 4;
    if (col < D) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float dv = x[k][j] - mean;
        s2 += dv * dv;
      }
    }
  }
  const float var = wave_sum(s2) / static_cast<float>(D);
  const float rs = rsqrtf(var + a.eps);
#pragma unroll
  for (int k = 0; k < kMaxGroups; ++k) {
    const int col = (k * 64 + lane) * 4;
    if (col < D) {
      float uu[4], gg[4];
      load4<T>(a.u + static_cast<size_t>(r) * D + col, uu);
#pragma unroll
      for (int j = 0; j < 4; ++j) gg[j] = (x[k][j] - mean) * rs * uu[j];
      store4<T>(a.g + static_cast<size_t>(r) * D + col, gg);
    }
  }
}

template <typename T>
hipError_t norm_t(const hstu_layer_desc& d, const int32_t* new_off, const WsPtrs& ws, hipStream_t stream,
                  const KernelEvents& ev) {
  NormArgs<T> a;
  a.new_off = new_off;
  a.row_user = ws.row_user;
  a.qb_base = ws.qb_base;
  a.qb_first = ws.qb_first;
  a.qb_nch = ws.qb_nch;
  a.part = ws.part;
  a.u = static_cast<const T*>(ws.u);
  a.g = static_cast<T*>(ws.q);
  a.status = &ws.hdr->status;
  a.T_rows = d.total_new;
  a.D = d.hidden;
  a.hd = d.head_dim;
  a.scale = d.attn_scale * kNegLn2;   // the attention accumulates -log2(e) * SiLU
  a.eps = d.norm_eps;
  const int grid = (d.total_new + 3) / 4;
  return launch_kernel(norm_gate_kernel<T>, dim3(grid), dim3(256), stream, ev, a);
}

}  // namespace

hipError_t launch_norm_gate(const hstu_layer_desc& d, const int32_t* new_off, const WsPtrs& ws,
                            hipStream_t stream, const KernelEvents& ev) {
  if (d.dtype == HSTU_BF16) return norm_t<bf16>(d, new_off, ws, stream, ev);
  return norm_t<float>(d, new_off, ws, stream, ev);
}

}  // namespace hstu
