// MFMA GEMMs of the layer:
//   * X W1 with the fused epilogue SiLU -> split U | V | Q | K -> U, Q into the
//     workspace and K, V appended straight into their pool pages;
//   * G W2 -> Y.
// C[M, N] = A[M, K] * W^T with W given as [N][K] (out-features x in-features,
// the usual linear-layer weight layout), so both operands are K-contiguous rows.
//
// A BM x BN output tile per 256-thread workgroup (2 x 2 waves).  Operand rows
// are 128-byte k-tile slices (64 bf16 or 32 fp32) copied global -> LDS by the
// direct-to-LDS loads, eight rows (1 KiB) per wave instruction, with no
// register staging.  The LDS is a ring of S k-tile stages: up to S-1 stages
// are in flight while one is multiplied, which hides the load latency that
// dominates these short-K products.  Within a row the 16-byte chunks are
// XOR-permuted by (row & 7) so the MFMA fragment reads are bank-conflict free.
//
// Tiles are handed out XCD-aware: workgroup i runs on XCD i % 8, each XCD owns
// a contiguous range of tiles, and within it groups of kGroupM row blocks walk
// the column blocks together so both operand panels stay in that XCD's L2.
//
// The epilogue goes through LDS: row-major outputs (U, Q, Y) and K rows leave
// as 16-byte stores, the transposed V columns as runs of consecutive slots.
#include "common.h"

namespace hstu {
namespace {

constexpr int kRowBytes = 128;   // one k-tile row
constexpr int kGroupM = 8;

template <typename T>
struct QkvEpi {
  T* q;
  T* u;
  T* k_pool;
  T* v_pool;
  const int2* row_loc;       // (pool page, slot) of each row
  int D, H, hd, ps;
};

__device__ __forceinline__ void tile_of(int id, int Mt, int Nt, int& mt, int& nt) {
  const int nT = Mt * Nt;
  const int x = id & 7, local = id >> 3;
  const int base = nT >> 3, rem = nT & 7;
  const int t = x * base + min(x, rem) + local;
  const int per_group = kGroupM * Nt;
  const int grp = t / per_group, first = grp * kGroupM;
  const int gsz = min(Mt - first, kGroupM);
  const int r = t - grp * per_group;
  mt = first + r % gsz;
  nt = r / gsz;
}

template <typename T, int BM, int BN, int S, int WGM, int WGN, bool kQkv>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_kernel(const T* __restrict__ A, const T* __restrict__ W,
                                                   int M, int N, int K, T* __restrict__ Y,
                                                   QkvEpi<T> ep, int32_t* status) {
  constexpr int ES = static_cast<int>(sizeof(T));
  constexpr int BK = kRowBytes / ES;
  constexpr int CE = 16 / ES;                  // elements per 16-byte chunk
  constexpr int NT = 64 * WGM * WGN;           // threads (waves laid out WGM x WGN)
  constexpr int IPW = (BM + BN) / (8 * WGM * WGN);   // direct loads per wave per stage
  static_assert(IPW * 8 * WGM * WGN == BM + BN, "whole 8-row blocks per wave");
  constexpr int STAGE = (BM + BN) * kRowBytes;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int KSTEP_CHUNKS = ES == 2 ? 4 : 8;   // chunks consumed per MFMA k-step
  constexpr int OST = BN + 16 / ES;            // epilogue staging row stride (elements)
  static_assert(BM * OST * ES <= S * STAGE, "epilogue staging fits the ring");
  static_assert(IPW * (S - 2) < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[S * STAGE];

  // The call's two status words (metadata, work list), loaded now and tested
  // only before the epilogue writes anything: the operand loads are in
  // bounds either way, and the test no longer costs a round trip ahead of
  // them.  The projection folds a work-list failure into the first word,
  // the one the host reads.
  const int2 sv = *reinterpret_cast<const int2*>(status);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int wm = w / WGN, wn = w % WGN;
  const int Mt = (M + BM - 1) / BM, Nt = N / BN;
  int mt, nt;
  tile_of(blockIdx.x, Mt, Nt, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  int blk = 0;
  if constexpr (kQkv) blk = n0 / ep.D;        // 0: U, 1: V, 2: Q, 3: K (a tile never straddles blocks)
  // pool locations of a K or V tile's rows, fetched now and parked in LDS
  // after the main loop
  __shared__ int2 s_loc[kQkv ? BM : 1];
  int2 my_loc = make_int2(0, 0);
  if constexpr (kQkv)
    if ((blk & 1) && tid < BM && m0 + tid < M) my_loc = ep.row_loc[m0 + tid];

  // Lane l of a direct load fills LDS chunk (l & 7) of row (l >> 3) of its
  // 8-row block; that slot holds source chunk (l & 7) ^ (l >> 3).
  const int lchunk = (lane & 7) ^ (lane >> 3);
  const T* src[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int r = 8 * (w * IPW + j) + (lane >> 3);
    if (r < BM)
      src[j] = A + static_cast<size_t>(min(m0 + r, M - 1)) * K + lchunk * CE;   // tail rows unused
    else
      src[j] = W + static_cast<size_t>(n0 + r - BM) * K + lchunk * CE;
  }
  auto issue = [&](int kt, int buf) __attribute__((always_inline)) {
    unsigned char* base = smem + buf * STAGE + w * IPW * 1024;
#pragma unroll
    for (int j = 0; j < IPW; ++j)
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(src[j] + kt * BK), (lds_void_t*)(base + j * 1024), 16, 0, 0);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int sw = l16 & 7;
  auto compute = [&](int buf) __attribute__((always_inline)) {
    const unsigned char* As = smem + buf * STAGE + (wm * WM + l16) * kRowBytes;
    const unsigned char* Bs = smem + buf * STAGE + (BM + wn * WN + l16) * kRowBytes;
#pragma unroll
    for (int ks = 0; ks < 8 / KSTEP_CHUNKS; ++ks) {
      const int chunk = ks * KSTEP_CHUNKS + (ES == 2 ? g : 2 * g);
      Frag<T> af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) read_frag(af[i], As + i * 16 * kRowBytes, chunk, sw);
#pragma unroll
      for (int j = 0; j < FN; ++j) read_frag(bfr[j], Bs + j * 16 * kRowBytes, chunk, sw);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mma16(af[i], bfr[j], acc[i][j]);
    }
  };

  const int KT = K / BK;
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < KT) issue(s, s);
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + S - 2 < KT) wait_vm<IPW * (S - 2)>();
    else wait_vm<0>();
    bar();                                    // stage kt visible; stage kt-1 no longer read
    if (kt + S - 1 < KT) issue(kt + S - 1, (kt + S - 1) % S);
    compute(kt % S);
  }
  if (kQkv && blockIdx.x == 0 && threadIdx.x == 0 && sv.x == 0 && sv.y != 0) status[0] = sv.y;
  if ((sv.x | sv.y) != 0) return;            // uniform: nothing is written on error
  __syncthreads();

  // ---- epilogue: stage the tile (after the epilogue transform) in LDS ----
  if constexpr (kQkv)
    if ((blk & 1) && tid < BM) s_loc[tid] = my_loc;
  T* Os = reinterpret_cast<T*>(smem);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * WM + i * 16 + g * 4 + r;
        const int col = wn * WN + j * 16 + l16;
        float z = acc[i][j][r];
        if constexpr (kQkv) {
          z = silu(z);
          // queries are stored pre-scaled by -log2(e) for the exp2-domain SiLU
          if (blk == 2) z *= -1.4426950408889634f;
        }
        Os[row * OST + col] = from_f32<T>(z);
      }
  __syncthreads();

  if (!kQkv || blk != 1) {
    // row-major rows of BN elements as 16-byte chunks
    constexpr int CPR = BN / CE;
    for (int c = tid; c < BM * CPR; c += NT) {
      const int row = c / CPR, ch = c % CPR;
      const int gr = m0 + row;
      if (gr >= M) continue;
      const u32x4 v = *reinterpret_cast<const u32x4*>(Os + row * OST + ch * CE);
      const int col = n0 + ch * CE;
      T* dst;
      if constexpr (!kQkv) {
        dst = Y + static_cast<size_t>(gr) * N + col;
      } else {
        const int cc = col - blk * ep.D;
        if (blk == 0) {
          dst = ep.u + static_cast<size_t>(gr) * ep.D + cc;
        } else if (blk == 2) {
          dst = ep.q + static_cast<size_t>(gr) * ep.D + cc;
        } else {                                 // K: pool slot row of head cc / hd
          const int2 loc = s_loc[row];
          const int h = cc / ep.hd, e = cc % ep.hd;
          dst = ep.k_pool + ((static_cast<size_t>(loc.x) * ep.H + h) * ep.ps + loc.y) * ep.hd + e;
        }
      }
      *reinterpret_cast<u32x4*>(dst) = v;
    }
  } else if constexpr (kQkv) {
    // V^T: a lane takes a pair of consecutive rows of one column, so lanes
    // walk consecutive slots of a page; a pair that shares a page and starts
    // at an even slot leaves as one store of two elements.
    constexpr int RP = BM / 2;
    static_assert(NT % RP == 0, "whole columns per pass");
    const int pr = tid % RP;
    const int r0 = 2 * pr, gr0 = m0 + r0;
    if (gr0 < M) {
      const bool has1 = gr0 + 1 < M;
      const int2 l0 = s_loc[r0], l1 = s_loc[r0 + 1];
      const bool pair = has1 && l1.x == l0.x && l1.y == l0.y + 1 && (l0.y & 1) == 0;
      const size_t pb0 = static_cast<size_t>(l0.x) * ep.H, pb1 = static_cast<size_t>(l1.x) * ep.H;
      const int cc0 = n0 - ep.D;
      for (int col = tid / RP; col < BN; col += NT / RP) {
        const int cc = cc0 + col;
        const int h = cc / ep.hd, e = cc % ep.hd;
        const T v0 = Os[r0 * OST + col], v1 = Os[(r0 + 1) * OST + col];
        T* d0 = ep.v_pool + ((pb0 + h) * ep.hd + e) * ep.ps + l0.y;
        if (pair) {
          typedef T T2 __attribute__((ext_vector_type(2)));
          T2 vv;
          vv.x = v0;
          vv.y = v1;
          *reinterpret_cast<T2*>(d0) = vv;
        } else {
          *d0 = v0;
          if (has1) ep.v_pool[((pb1 + h) * ep.hd + e) * ep.ps + l1.y] = v1;
        }
      }
    }
  }
}

template <typename T, int BM, int BN, int S, int WGM, int WGN>
hipError_t gemm_qkv_t(const hstu_layer_desc& d, const void* x, const void* w1t, void* k_pool, void* v_pool,
                      const WsPtrs& ws, hipStream_t stream, const KernelEvents& ev) {
  QkvEpi<T> ep;
  ep.q = static_cast<T*>(ws.q);
  ep.u = static_cast<T*>(ws.u);
  ep.k_pool = static_cast<T*>(k_pool);
  ep.v_pool = static_cast<T*>(v_pool);
  ep.row_loc = ws.row_loc;
  ep.D = d.hidden;
  ep.H = d.num_heads;
  ep.hd = d.head_dim;
  ep.ps = d.page_size;
  const int M = d.total_new, N = 4 * d.hidden, K = d.hidden;
  const int tiles = (M + BM - 1) / BM * (N / BN);
  return launch_kernel(gemm_kernel<T, BM, BN, S, WGM, WGN, true>, dim3(tiles), dim3(64 * WGM * WGN), stream, ev,
                       static_cast<const T*>(x), static_cast<const T*>(w1t), M, N, K, static_cast<T*>(nullptr),
                       ep, &ws.hdr->status);
}

template <typename T, int BM, int BN, int S, int WGM, int WGN>
hipError_t gemm_out_t(const hstu_layer_desc& d, const void* g, const void* w2t, void* y,
                      int32_t* status, hipStream_t stream, const KernelEvents& ev) {
  QkvEpi<T> ep{};
  const int M = d.total_new, N = d.hidden, K = d.hidden;
  const int tiles = (M + BM - 1) / BM * (N / BN);
  return launch_kernel(gemm_kernel<T, BM, BN, S, WGM, WGN, false>, dim3(tiles), dim3(64 * WGM * WGN), stream,
                       ev, static_cast<const T*>(g), static_cast<const T*>(w2t), M, N, K, static_cast<T*>(y), ep,
                       status);
}

// Tile shape and ring depth by problem size (large problems: two stages, as
// several workgroups per CU beat deeper rings there, a CU's load throughput
// growing with the waves it has in flight; small ones: three stages, since
// each workgroup's few k-tiles are then latency-bound):
//   >= 1024 tiles of 128 x 128 -> 128 x 128, 8 waves, 2 stages (fewest re-reads);
//   >= 256 such tiles          -> 64 x 128, 4 waves, 2 stages;
//   otherwise                  -> 64 x 64, 4 waves, 3 stages (most workgroups);
//                                 for G W2 32 x 64 when 64 x 64 gives fewer
//                                 tiles than CUs.
// Wide tiles need N % 128 == 0 (and, for X W1, every U|V|Q|K block whole).
enum class Tile { k64x64, k64x128, k128x128 };
Tile pick_tile(int M, int N, int D) {
  if (D % 128 != 0 || N % 128 != 0) return Tile::k64x64;
  const int64_t t128 = static_cast<int64_t>((M + 127) / 128) * (N / 128);
  if (t128 >= 1024) return Tile::k128x128;
  if (t128 >= 256) return Tile::k64x128;
  return Tile::k64x64;
}

template <typename T>
hipError_t qkv_dispatch(const hstu_layer_desc& d, const void* x, const void* w1t, void* k_pool, void* v_pool,
                        const WsPtrs& ws, hipStream_t st, const KernelEvents& ev) {
  if constexpr (sizeof(T) == 4) {
    return gemm_qkv_t<T, 64, 64, 2, 2, 2>(d, x, w1t, k_pool, v_pool, ws, st, ev);   // fp32: one tile shape
  } else {
    switch (pick_tile(d.total_new, 4 * d.hidden, d.hidden)) {
      case Tile::k128x128: return gemm_qkv_t<T, 128, 128, 2, 2, 4>(d, x, w1t, k_pool, v_pool, ws, st, ev);
      case Tile::k64x128: return gemm_qkv_t<T, 64, 128, 2, 2, 2>(d, x, w1t, k_pool, v_pool, ws, st, ev);
      default: return gemm_qkv_t<T, 64, 64, 3, 2, 2>(d, x, w1t, k_pool, v_pool, ws, st, ev);
    }
  }
}

template <typename T>
hipError_t out_dispatch(const hstu_layer_desc& d, const void* g, const void* w2t, void* y,
                        int32_t* status, hipStream_t st, const KernelEvents& ev) {
  if constexpr (sizeof(T) == 4) {
    return gemm_out_t<T, 64, 64, 2, 2, 2>(d, g, w2t, y, status, st, ev);   // fp32: one tile shape
  } else {
    switch (pick_tile(d.total_new, d.hidden, d.hidden)) {
      case Tile::k128x128: return gemm_out_t<T, 128, 128, 2, 2, 4>(d, g, w2t, y, status, st, ev);
      case Tile::k64x128: return gemm_out_t<T, 64, 128, 2, 2, 2>(d, g, w2t, y, status, st, ev);
      default:
        // fewer 64 x 64 tiles than CUs: halve the tile height for more workgroups
        if (static_cast<int64_t>((d.total_new + 63) / 64) * (d.hidden / 64) < 256)
          return gemm_out_t<T, 32, 64, 3, 2, 2>(d, g, w2t, y, status, st, ev);
        return gemm_out_t<T, 64, 64, 3, 2, 2>(d, g, w2t, y, status, st, ev);
    }
  }
}

}  // namespace

hipError_t launch_gemm_qkv(const hstu_layer_desc& d, const void* x, const void* w1t, void* k_pool,
                           void* v_pool, const WsPtrs& ws, hipStream_t stream, const KernelEvents& ev) {
  return d.dtype == HSTU_BF16 ? qkv_dispatch<bf16>(d, x, w1t, k_pool, v_pool, ws, stream, ev)
                              : qkv_dispatch<float>(d, x, w1t, k_pool, v_pool, ws, stream, ev);
}

hipError_t launch_gemm_out(const hstu_layer_desc& d, const void* g, const void* w2t, void* y,
                           int32_t* status, hipStream_t stream, const KernelEvents& ev) {
  return d.dtype == HSTU_BF16 ? out_dispatch<bf16>(d, g, w2t, y, status, stream, ev)
                              : out_dispatch<float>(d, g, w2t, y, status, stream, ev);
}

}  // namespace hstu
