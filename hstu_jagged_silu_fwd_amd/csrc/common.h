// Internal definitions shared by the gfx950 kernels of libhstu.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hstu.h"

namespace hstu {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kQB = 256;         // query rows per attention work item (q-block)
constexpr int kMaxUsers = 4096;  // users per call (metadata is cached in LDS)
constexpr float kNegLn2 = -0.6931471805599453f;
constexpr int kMaxBuckets = 1024;
constexpr int kMaxChunkKeys = 8192;   // attention split never exceeds this many keys
constexpr int kMaxRows = 1 << 18;     // new rows per call
constexpr int kMaxQBlocks = kMaxRows / kQB + kMaxUsers;
constexpr int kMaxStackLayers = 32;   // layers of one hstu_stack_fwd call

// ---------------------------------------------------------------------------
// Per-layer bias tables, built once per call by prep and copied into each
// attention workgroup's LDS with direct-to-LDS loads.  All values are in the
// attention's exponent domain (scaled by -log2(e)):
//   [0, kLut)            bias of distance kLut - 1 - x (descending distance)
//   [kLut, kTabPb)       kMasked (negative distances: the causal mask)
//   [kTabPb, kTabTb)     position-bucket bias, kMaxBuckets entries
//   [kTabTb, ...)        timestamp-bucket bias, kMaxBuckets entries
// padded to whole KiB (kTabFloats).
// ---------------------------------------------------------------------------
constexpr int kLut = 4096;
constexpr int kLutPad = 64;
constexpr int kTabPb = kLut + kLutPad;
constexpr int kTabTb = kTabPb + kMaxBuckets;
constexpr int kTabFloats = (kTabTb + kMaxBuckets + 255) / 256 * 256;
constexpr float kNegLog2e = -1.4426950408889634f;
// Exponent-domain score of a masked (query, key) pair: S' = kMasked makes
// 2^S' = inf, so SiLU = -ln2 * S' / (1 + 2^S') = S' * rcp(inf) = exactly 0
// (kMasked plus any finite q.k stays finite).
constexpr float kMasked = 1e30f;

// ---------------------------------------------------------------------------
// MFMA fragments.  A fragment holds 8 elements per lane.  For a 16x16 tile
// product D = A*B with a 32-deep contraction, lane l supplies A[l&15][k] and
// B[k][l&15] for the 8 contraction indices k = 8*(l>>4) + e, e = 0..7; the
// result lands as D[4*(l>>4) + i][l&15], i = 0..3.
// bf16: one v_mfma_f32_16x16x32_bf16.  fp32: eight v_mfma_f32_16x16x4_f32,
// instruction e contracting over {8*g + e : g = 0..3} -- the same index set,
// so both element types share every load and layout.
// ---------------------------------------------------------------------------
template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { float v[8]; };

__device__ __forceinline__ f32x4 mma16(const Frag<bf16>& a, const Frag<bf16>& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const Frag<float>& a, const Frag<float>& b, f32x4 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ void load_frag(Frag<bf16>& f, const bf16* p) {
  f.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void load_frag(Frag<float>& f, const float* p) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
__device__ __forceinline__ void zero_frag(Frag<bf16>& f) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = static_cast<bf16>(0.0f);
}
__device__ __forceinline__ void zero_frag(Frag<float>& f) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = 0.0f;
}
__device__ __forceinline__ void set_elem(Frag<bf16>& f, int e, float x) { f.v[e] = static_cast<bf16>(x); }
__device__ __forceinline__ void set_elem(Frag<float>& f, int e, float x) { f.v[e] = x; }
// All 8 elements at once (bf16: four packed conversions).
__device__ __forceinline__ void set_frag(Frag<bf16>& f, const float* x) {
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  f32x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = x[e];
  f.v = __builtin_convertvector(v, bf16x8);
}
__device__ __forceinline__ void set_frag(Frag<float>& f, const float* x) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = x[e];
}

// Fragment read from an LDS row whose 16-byte chunks are XOR-permuted by
// `sw`: the 8 elements starting at logical chunk `chunk` (bf16: one chunk,
// fp32: two).
__device__ __forceinline__ void read_frag(Frag<bf16>& f, const unsigned char* rowp, int chunk, int sw) {
  f.v = *reinterpret_cast<const bf16x8*>(rowp + ((chunk ^ sw) << 4));
}
__device__ __forceinline__ void read_frag(Frag<float>& f, const unsigned char* rowp, int chunk, int sw) {
  const float4 lo = *reinterpret_cast<const float4*>(rowp + ((chunk ^ sw) << 4));
  const float4 hi = *reinterpret_cast<const float4*>(rowp + (((chunk + 1) ^ sw) << 4));
  f.v[0] = lo.x; f.v[1] = lo.y; f.v[2] = lo.z; f.v[3] = lo.w;
  f.v[4] = hi.x; f.v[5] = hi.y; f.v[6] = hi.z; f.v[7] = hi.w;
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

// SiLU(z) = z * sigmoid(z) = z / (1 + e^-z), with the hardware exp and
// reciprocal.  Large negative z gives e^-z = inf and a result of -0.
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Log-linear relative-distance bucket (m mantissa bits, nb buckets).
__device__ __forceinline__ int bucket32(int delta, int m, int nb) {
  const uint32_t d = delta < 0 ? 0u : static_cast<uint32_t>(delta);
  int b;
  if (d < (1u << m)) {
    b = static_cast<int>(d);
  } else {
    const int e = 31 - __clz(d);
    b = ((e - m + 1) << m) + static_cast<int>(d >> (e - m)) - (1 << m);
  }
  return b < nb - 1 ? b : nb - 1;
}
__device__ __forceinline__ int bucket64(int64_t delta, int m, int nb) {
  if (delta < 0) delta = 0;
  const uint64_t d = static_cast<uint64_t>(delta);
  int64_t b;
  if (d < (1ull << m)) {
    b = static_cast<int64_t>(d);
  } else {
    const int e = 63 - __clzll(d);
    b = (static_cast<int64_t>(e - m + 1) << m) + static_cast<int64_t>(d >> (e - m)) - (1ll << m);
  }
  return b < nb - 1 ? static_cast<int>(b) : nb - 1;
}

// bucket64 with the common case, 0 <= delta < 2^32, in 32-bit arithmetic:
// with e = floor(log2 d) and t = d >> (e - m) (the top m + 1 bits, leading
// one included), the rule's (e - m + 1) * 2^m + t - 2^m is (e - m) * 2^m + t.
// Other deltas (negative, or 2^32 and beyond) take bucket64 itself.
__device__ __forceinline__ int bucket64_fast(int64_t delta, int m, int nb) {
  const uint32_t hi = static_cast<uint32_t>(static_cast<uint64_t>(delta) >> 32);
  if (__builtin_expect(hi != 0u, 0)) return bucket64(delta, m, nb);
  const uint32_t d = static_cast<uint32_t>(delta);
  int b;
  if (d < (1u << m)) {
    b = static_cast<int>(d);
  } else {
    const int sh = 31 - __clz(d) - m;
    b = (sh << m) + static_cast<int>(d >> sh);
  }
  return b < nb - 1 ? b : nb - 1;
}

// ---------------------------------------------------------------------------
// Direct global -> LDS loads.  __builtin_amdgcn_global_load_lds(src, dst, 16,
// 0, 0) copies 16 bytes per lane: lane l's bytes land at dst + 16 * l (dst is
// wave-uniform), so one wave instruction fills 1 KiB of LDS.  They count as
// vector-memory operations; wait_vm<N>() waits until at most N of this
// wave's vector-memory operations are outstanding (gfx9 s_waitcnt encoding:
// vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima).
// bar() is a workgroup barrier without the memory fence of __syncthreads
// (which would wait for every outstanding load); the empty asm statements
// keep the compiler from moving memory accesses across it.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

// The same copies issued from inline assembly (16 or 4 bytes per lane, to
// lds_base + size * lane).  The compiler does not see these as LDS writes, so
// it adds no waits of its own before later LDS reads; the caller orders them
// with wait_vm and bar.  M0, which holds the LDS base, is restored after
// the issue (the instruction reads it when issued).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}
__device__ __forceinline__ void dma_lds16(const void* src, const void* lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(src), "s"(lds_addr(lds_base)) : "memory");
}
__device__ __forceinline__ void dma_lds4(const void* src, const void* lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(src), "s"(lds_addr(lds_base)) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// wait_vm with a wave-uniform run-time count n: waits for the largest of
// 0, 2, 4, 6, 8, 12, 16, 24 and 32 that does not exceed n (waiting for a few
// more loads than needed is always safe).  A short tree of uniform branches:
// a full switch over every count costs more than the waits it saves.
__device__ __forceinline__ void wait_vm_n(int n) {
  if (n >= 12) {
    if (n >= 24) {
      if (n >= 32) wait_vm<32>(); else wait_vm<24>();
    } else {
      if (n >= 16) wait_vm<16>(); else wait_vm<12>();
    }
  } else if (n >= 6) {
    if (n >= 8) wait_vm<8>(); else wait_vm<6>();
  } else if (n >= 4) {
    wait_vm<4>();
  } else if (n >= 2) {
    wait_vm<2>();
  } else {
    wait_vm<0>();
  }
}

__device__ __forceinline__ void bar() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

// Index of the user owning jagged row r (largest u with offsets[u] <= r);
// offsets must be a validated non-decreasing prefix sum.
__device__ __forceinline__ int row_to_user(const int32_t* offsets, int B, int r) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// Workspace of one hstu_layer_fwd call (offsets computed on the host).
// ---------------------------------------------------------------------------
struct WsHeader {            // first 256 bytes of the workspace
  int32_t status;            // hstu_device_code of this call (metadata validation)
  int32_t wl_status;         // work-list build (nonzero only with metadata that
                             // `status` rejects, or a workspace too small)
  int32_t n_items;           // attention work items
  int32_t n_qb;              // q-block entries
  int32_t item_budget;       // attention cost units per work item (chunk sizing)
  int32_t counter;           // dynamic work-fetch counter
};

// One attention work item: a = {user, first row of the q-block, head, first
// key}, b = {end key, first jagged row of the user, new rows, history}.
struct AttnItem {
  int4 a;
  int4 b;
};

struct WsPtrs {
  WsHeader* hdr;
  int2* row_loc;             // [layers][T] (pool page, slot) of each new row's K/V
  int32_t* qb_first;         // [nqb_cap] first work item of a q-block entry (head 0)
  int32_t* qb_nch;           // [nqb_cap] key chunks of a q-block entry
  int32_t* qb_row0;          // [nqb_cap] first jagged row of a q-block entry
  int32_t* qb_rows;          // [nqb_cap] rows of a q-block entry
  AttnItem* items;           // [item_cap]
  void* q;                   // [T, D] dtype; reused for G after attention
  void* u;                   // [T, D] dtype
  float* part;               // [item_cap, kQB, d] fp32 partial attention outputs
  float* tables;             // [layers][kTabFloats] bias tables (see kTabFloats)
};

// Optional events that the runtime stamps at the start and the end of one
// kernel's execution (hipExtLaunchKernel), so that their difference is that
// kernel's duration alone.
struct KernelEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Launch `kernel` on `stream`; with events, through hipExtLaunchKernel so
// that they bracket exactly this kernel.
template <typename... KArgs, typename... Args>
inline hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                                const KernelEvents& ev, Args... args) {
  if (ev.start == nullptr && ev.stop == nullptr) {
    kernel<<<grid, block, 0, stream>>>(args...);
    return hipGetLastError();
  }
  hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, ev.start, ev.stop, 0, args...);
  return hipGetLastError();
}

// Host launchers (one per kernel family), all enqueue on `stream`.
hipError_t launch_prep(const hstu_layer_desc& d, const int32_t* new_off, const int32_t* hist,
                       const int32_t* ncand, const int32_t* const* pts, int nl, const int32_t* ts_off,
                       const float* const* pbs, const float* const* tbs, const WsPtrs& ws,
                       int nqb_cap, int item_cap, int target_items, hipStream_t stream,
                       const KernelEvents& ev = {});
hipError_t launch_gemm_qkv(const hstu_layer_desc& d, const void* x, const void* w1t, void* k_pool,
                           void* v_pool, const WsPtrs& ws, hipStream_t stream, const KernelEvents& ev = {});
hipError_t launch_attn(const hstu_layer_desc& d, const int32_t* pt, const void* k_pool, const void* v_pool,
                       int layer, const int64_t* ts, const int32_t* ts_off, const int32_t* ncand,
                       const WsPtrs& ws, int grid, hipStream_t stream, const KernelEvents& ev = {});
hipError_t launch_gemm_out(const hstu_layer_desc& d, const void* g, const void* w2t, void* y,
                           int32_t* status, hipStream_t stream, const KernelEvents& ev = {});
hipError_t launch_norm_gate(const hstu_layer_desc& d, const WsPtrs& ws, int nqb_cap, hipStream_t stream,
                            const KernelEvents& ev = {});
hipError_t launch_append(const hstu_layer_desc& d, const void* k_new, const void* v_new,
                         const int32_t* new_off, const int32_t* hist, const int32_t* pt,
                         void* k_pool, void* v_pool, int32_t* status, hipStream_t stream);

}  // namespace hstu
