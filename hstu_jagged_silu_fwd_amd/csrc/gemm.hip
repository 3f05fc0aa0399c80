// MFMA GEMMs of the layer:
//   * X W1 with the fused epilogue SiLU -> split U | V | Q | K -> U, Q into the
//     workspace and K, V appended straight into their pool pages;
//   * G W2 -> Y.
// C[M, N] = A[M, K] * B[K, N], all row-major.  64x64 output tile per
// 256-thread workgroup (2x2 waves, 32x32 per wave = 2x2 MFMA 16x16 blocks),
// 32-deep K slices staged through LDS; B is transposed on its way into LDS so
// that both operands are read as contiguous 8-element fragments.
#include "common.h"

namespace hstu {
namespace {

constexpr int BM = 64, BN = 64, BK = 32;

template <typename T> struct Vec8 { T v[8]; };

template <typename T>
__device__ __forceinline__ Vec8<T> ld8(const T* p) {
  Vec8<T> r;
  constexpr int n16 = sizeof(Vec8<T>) / 16;
#pragma unroll
  for (int i = 0; i < n16; ++i) reinterpret_cast<uint4*>(&r)[i] = reinterpret_cast<const uint4*>(p)[i];
  return r;
}
template <typename T>
__device__ __forceinline__ void st8(T* p, const Vec8<T>& x) {
  constexpr int n16 = sizeof(Vec8<T>) / 16;
#pragma unroll
  for (int i = 0; i < n16; ++i) reinterpret_cast<uint4*>(p)[i] = reinterpret_cast<const uint4*>(&x)[i];
}

template <typename T>
struct QkvEpi {
  T* q;
  T* u;
  T* k_pool;
  T* v_pool;
  const int32_t* row_user;
  const int32_t* new_off;
  const int32_t* hist;
  const int32_t* pt;
  int D, H, hd, ps, maxP;
};

template <typename T, bool kQkv>
__global__ __launch_bounds__(256) void gemm_kernel(const T* __restrict__ A, const T* __restrict__ Bm,
                                                   int M, int N, int K, T* __restrict__ Y,
                                                   QkvEpi<T> ep, const int32_t* status) {
  if (*status != 0) return;
  constexpr int PAD = 16 / sizeof(T);
  __shared__ __attribute__((aligned(16))) T As[BM][BK + PAD];
  __shared__ __attribute__((aligned(16))) T Bs[BN][BK + PAD];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int wm = w >> 1, wn = w & 1;
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int a_row = tid >> 2, a_k = (tid & 3) * 8;
  const int b_k = tid >> 3, b_n = (tid & 7) * 8;
  for (int k0 = 0; k0 < K; k0 += BK) {
    {
      Vec8<T> va;
      const int gr = m0 + a_row;
      if (gr < M) {
        va = ld8(A + static_cast<size_t>(gr) * K + k0 + a_k);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) va.v[e] = from_f32<T>(0.0f);
      }
      st8(&As[a_row][a_k], va);
      const Vec8<T> vb = ld8(Bm + static_cast<size_t>(k0 + b_k) * N + n0 + b_n);
#pragma unroll
      for (int e = 0; e < 8; ++e) Bs[b_n + e][b_k] = vb.v[e];
    }
    __syncthreads();
    Frag<T> af[2], bfr[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) load_frag(af[i], &As[wm * 32 + i * 16 + l16][g * 8]);
#pragma unroll
    for (int j = 0; j < 2; ++j) load_frag(bfr[j], &Bs[wn * 32 + j * 16 + l16][g * 8]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mma16(af[i], bfr[j], acc[i][j]);
    __syncthreads();
  }

  if constexpr (!kQkv) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm * 32 + i * 16 + g * 4 + r;
          const int col = n0 + wn * 32 + j * 16 + l16;
          if (row < M) Y[static_cast<size_t>(row) * N + col] = from_f32<T>(acc[i][j][r]);
        }
  } else {
    const int D = ep.D;
    const int blk = n0 / D;      // 0: U, 1: V, 2: Q, 3: K (tile never straddles blocks)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * 32 + i * 16 + g * 4 + r;
        if (row >= M) continue;
        size_t kbase = 0, vbase = 0;
        if (blk == 1 || blk == 3) {
          const int user = ep.row_user[row];
          const int p = ep.hist[user] + row - ep.new_off[user];
          const int page = ep.pt[static_cast<size_t>(user) * ep.maxP + p / ep.ps];
          const int slot = p % ep.ps;
          kbase = static_cast<size_t>(page) * ep.H * ep.ps * ep.hd + static_cast<size_t>(slot) * ep.hd;
          vbase = static_cast<size_t>(page) * ep.H * ep.hd * ep.ps + slot;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = n0 + wn * 32 + j * 16 + l16;
          const int cc = col - blk * D;
          const T z = from_f32<T>(silu(acc[i][j][r]));
          if (blk == 0) {
            ep.u[static_cast<size_t>(row) * D + cc] = z;
          } else if (blk == 2) {
            // queries are stored pre-scaled by -log2(e) for the exp2-domain SiLU
            ep.q[static_cast<size_t>(row) * D + cc] = from_f32<T>(-1.4426950408889634f * silu(acc[i][j][r]));
          } else {
            const int h = cc / ep.hd, e = cc % ep.hd;
            if (blk == 3)
              ep.k_pool[kbase + static_cast<size_t>(h) * ep.ps * ep.hd + e] = z;
            else
              ep.v_pool[vbase + (static_cast<size_t>(h) * ep.hd + e) * ep.ps] = z;
          }
        }
      }
  }
}

template <typename T>
hipError_t gemm_qkv_t(const hstu_layer_desc& d, const void* x, const void* w1, const int32_t* new_off,
                      const int32_t* hist, const int32_t* pt, void* k_pool, void* v_pool,
                      const WsPtrs& ws, hipStream_t stream) {
  QkvEpi<T> ep;
  ep.q = static_cast<T*>(ws.q);
  ep.u = static_cast<T*>(ws.u);
  ep.k_pool = static_cast<T*>(k_pool);
  ep.v_pool = static_cast<T*>(v_pool);
  ep.row_user = ws.row_user;
  ep.new_off = new_off;
  ep.hist = hist;
  ep.pt = pt;
  ep.D = d.hidden;
  ep.H = d.num_heads;
  ep.hd = d.head_dim;
  ep.ps = d.page_size;
  ep.maxP = d.max_pages_per_user;
  const int M = d.total_new, N = 4 * d.hidden, K = d.hidden;
  dim3 grid((M + BM - 1) / BM, N / BN);
  gemm_kernel<T, true><<<grid, 256, 0, stream>>>(static_cast<const T*>(x), static_cast<const T*>(w1),
                                                 M, N, K, nullptr, ep, &ws.hdr->status);
  return hipGetLastError();
}

template <typename T>
hipError_t gemm_out_t(const hstu_layer_desc& d, const void* g, const void* w2, void* y,
                      const int32_t* status, hipStream_t stream) {
  QkvEpi<T> ep{};
  const int M = d.total_new, N = d.hidden, K = d.hidden;
  dim3 grid((M + BM - 1) / BM, N / BN);
  gemm_kernel<T, false><<<grid, 256, 0, stream>>>(static_cast<const T*>(g), static_cast<const T*>(w2),
                                                  M, N, K, static_cast<T*>(y), ep, status);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_qkv(const hstu_layer_desc& d, const void* x, const void* w1,
                           const int32_t* new_off, const int32_t* hist, const int32_t* pt,
                           void* k_pool, void* v_pool, const WsPtrs& ws, hipStream_t stream) {
  if (d.dtype == HSTU_BF16) return gemm_qkv_t<bf16>(d, x, w1, new_off, hist, pt, k_pool, v_pool, ws, stream);
  return gemm_qkv_t<float>(d, x, w1, new_off, hist, pt, k_pool, v_pool, ws, stream);
}

hipError_t launch_gemm_out(const hstu_layer_desc& d, const void* g, const void* w2, void* y,
                           const int32_t* status, hipStream_t stream) {
  if (d.dtype == HSTU_BF16) return gemm_out_t<bf16>(d, g, w2, y, status, stream);
  return gemm_out_t<float>(d, g, w2, y, status, stream);
}

}  // namespace hstu
