// Row norm and gating: O = attn_scale * (sum of the row's chunk partials, in
// chunk order; the partials hold -log2(e) * sum SiLU(s) v, undone here), then
// G = LayerNorm_row(O) * U, the elementwise gating that precedes the output
// projection (aitrends.kr article 100093, "HSTU sequential modelling").
// Population variance over the row's D entries, no affine.  G overwrites the
// Q buffer, which is dead after the attention.
//
// A workgroup takes 256 / TPR consecutive rows of one q-block entry (grid:
// entry x row block), TPR threads per row (a whole wave for D = 256 or 512
// and fewer than 4096 rows, whose extra workgroups measured faster than 32
// there and slower on large batches; else 32 when D allows, 16 otherwise);
// the row statistics are TPR-lane reductions.  The entry's table entries come in one round trip and the
// partial sums and U in a second; the loads carry no data-dependent branches
// (columns beyond D load a valid column and are zeroed by a select) so each
// batch stays in flight together.
#include "common.h"

namespace hstu {
namespace {

constexpr int kThreads = 256;

template <typename T>
struct NormArgs {
  WsHeader* hdr;
  const int32_t* qb_first;          // [entries] first work item (head 0)
  const int32_t* qb_nch;            // [entries] key chunks
  const int32_t* qb_row0;           // [entries] first jagged row
  const int32_t* qb_rows;           // [entries] rows
  const float* part;                // [items][kQB][hd]
  const T* u;                       // [T][D]
  T* g;                             // [T][D]
  int D, hd;
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

// TPR: threads per row; MAXNG: (4 * TPR)-column groups per row at most.
template <typename T, int TPR, int MAXNG>
__global__ __launch_bounds__(kThreads) void norm_gate_kernel(NormArgs<T> a) {
  constexpr int kRows = kThreads / TPR;           // rows per workgroup
  constexpr int kBlocks = kQB / kRows;            // row blocks per q-block entry
  constexpr int GW = 4 * TPR;                     // columns per group
  const int tid = threadIdx.x;
  const int D = a.D;
  const int e = blockIdx.x / kBlocks, rb = blockIdx.x % kBlocks;   // q-block entry, row block in it
  const int4 hv = *reinterpret_cast<const int4*>(a.hdr);   // status, wl_status, items, entries
  // the attention kernel of this layer is done with its work-fetch counter:
  // reset it for the next layer of a stack (whose prep does not run again)
  if (blockIdx.x == 0 && tid == 0) a.hdr->counter = 0;
  const int first = a.qb_first[e], nch = a.qb_nch[e], row0 = a.qb_row0[e], rows = a.qb_rows[e];
  // all five loads are issued before the exit test (no short-circuit chain
  // of dependent loads)
  asm volatile("" ::"s"(first), "s"(nch), "s"(row0));
  if (((hv.x | hv.y) != 0) | (e >= hv.w) | (rb * kRows >= rows)) return;   // uniform

  // thread (row lr, lane sub) owns columns gi*GW + 4*sub .. +3 of its row
  const int lr = tid / TPR, sub = tid % TPR;
  const int rib = rb * kRows + lr;                // row inside the q-block
  const bool valid = rib < rows;
  const int r = row0 + min(rib, rows - 1);
  const int NG = D / GW;
  float x[MAXNG][4], uu[MAXNG][4];
  const float* psrc[MAXNG];
#pragma unroll
  for (int gi = 0; gi < MAXNG; ++gi) {
    const int col = min(gi, NG - 1) * GW + 4 * sub;          // a valid column for every gi
    const int h = col / a.hd, el = col - h * a.hd;
    psrc[gi] = a.part + (static_cast<size_t>(first + h * nch) * kQB + rib) * a.hd + el;
    load4<T>(a.u + static_cast<size_t>(r) * D + col, uu[gi]);
#pragma unroll
    for (int j = 0; j < 4; ++j) x[gi][j] = 0.f;
  }
  // chunks CU at a time: all their loads are issued before the first add
  // (a chunk index past nch re-reads the last chunk and adds zero), and each
  // element is still summed in chunk order
  constexpr int CU = MAXNG >= 32 ? 1 : 32 / MAXNG;
  const size_t stride = static_cast<size_t>(kQB) * a.hd;      // one chunk further
  for (int kc0 = 0; kc0 < nch; kc0 += CU) {
    f32x4 v[CU][MAXNG];
#pragma unroll
    for (int c = 0; c < CU; ++c)
#pragma unroll
      for (int gi = 0; gi < MAXNG; ++gi)
        v[c][gi] = *reinterpret_cast<const f32x4*>(psrc[gi] + min(kc0 + c, nch - 1) * stride);
    // keep the scheduler from interleaving the adds with the loads (it would
    // otherwise wait for each load before issuing the next)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < CU; ++c) {
      const float m = kc0 + c < nch ? 1.f : 0.f;
#pragma unroll
      for (int gi = 0; gi < MAXNG; ++gi) {
#pragma unroll
        for (int j = 0; j < 4; ++j) x[gi][j] += m * v[c][gi][j];
      }
    }
  }
  float s1 = 0.f;
#pragma unroll
  for (int gi = 0; gi < MAXNG; ++gi)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[gi][j] = gi < NG ? x[gi][j] * a.scale : 0.f;
      s1 += x[gi][j];
    }
#pragma unroll
  for (int o = TPR / 2; o >= 1; o >>= 1) s1 += __shfl_xor(s1, o, kWave);
  const float mean = s1 / static_cast<float>(D);
  float s2 = 0.f;
#pragma unroll
  for (int gi = 0; gi < MAXNG; ++gi)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float dv = gi < NG ? x[gi][j] - mean : 0.f;
      s2 += dv * dv;
    }
#pragma unroll
  for (int o = TPR / 2; o >= 1; o >>= 1) s2 += __shfl_xor(s2, o, kWave);
  const float rs = rsqrtf(s2 / static_cast<float>(D) + a.eps);
  if (valid) {
#pragma unroll
    for (int gi = 0; gi < MAXNG; ++gi) {
      if (gi < NG) {
        float gg[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) gg[j] = (x[gi][j] - mean) * rs * uu[gi][j];
        store4<T>(a.g + static_cast<size_t>(r) * D + gi * GW + 4 * sub, gg);
      }
    }
  }
}

template <typename T, int TPR, int MAXNG>
hipError_t norm_t(const hstu_layer_desc& d, const WsPtrs& ws, int nqb_cap, hipStream_t stream,
                  const KernelEvents& ev) {
  NormArgs<T> a;
  a.hdr = ws.hdr;
  a.qb_first = ws.qb_first;
  a.qb_nch = ws.qb_nch;
  a.qb_row0 = ws.qb_row0;
  a.qb_rows = ws.qb_rows;
  a.part = ws.part;
  a.u = static_cast<const T*>(ws.u);
  a.g = static_cast<T*>(ws.q);
  a.D = d.hidden;
  a.hd = d.head_dim;
  a.scale = d.attn_scale * kNegLn2;   // the attention accumulates -log2(e) * SiLU
  a.eps = d.norm_eps;
  constexpr int kRows = kThreads / TPR;
  return launch_kernel(norm_gate_kernel<T, TPR, MAXNG>, dim3(static_cast<unsigned>(nqb_cap) * (kQB / kRows)),
                       dim3(kThreads), stream, ev, a);
}

template <typename T>
hipError_t norm_dt(const hstu_layer_desc& d, const WsPtrs& ws, int nqb_cap, hipStream_t stream,
                   const KernelEvents& ev) {
  // a wave per row (4 rows per workgroup) for small batches, whose 32-thread
  // grid would leave compute units idle; large batches keep 32 per row
  // (batch-invariant calls too: the instance then depends on D alone)
  if (d.hidden % 256 == 0 && d.hidden <= 512 && d.total_new < 4096 && !(d.flags & HSTU_FLAG_BATCH_INVARIANT))
    return norm_t<T, 64, 2>(d, ws, nqb_cap, stream, ev);
  if (d.hidden % 128 == 0) {                     // 32 threads per row, 8 rows per workgroup
    const int ng = d.hidden / 128;
    if (ng <= 4) return norm_t<T, 32, 4>(d, ws, nqb_cap, stream, ev);
    if (ng <= 8) return norm_t<T, 32, 8>(d, ws, nqb_cap, stream, ev);
    return norm_t<T, 32, 16>(d, ws, nqb_cap, stream, ev);
  }
  const int ng = d.hidden / 64;                  // 16 threads per row, 16 rows per workgroup
  if (ng <= 4) return norm_t<T, 16, 4>(d, ws, nqb_cap, stream, ev);
  if (ng <= 8) return norm_t<T, 16, 8>(d, ws, nqb_cap, stream, ev);
  if (ng <= 16) return norm_t<T, 16, 16>(d, ws, nqb_cap, stream, ev);
  return norm_t<T, 16, 32>(d, ws, nqb_cap, stream, ev);
}

}  // namespace

hipError_t launch_norm_gate(const hstu_layer_desc& d, const WsPtrs& ws, int nqb_cap, hipStream_t stream,
                            const KernelEvents& ev) {
  if (d.dtype == HSTU_BF16) return norm_dt<bf16>(d, ws, nqb_cap, stream, ev);
  return norm_dt<float>(d, ws, nqb_cap, stream, ev);
}

}  // namespace hstu
