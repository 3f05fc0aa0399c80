// Paged jagged SiLU attention (HSTU pointwise attention over a paged KV
// cache; NVIDIA blog "Deploying an HSTU generative recommender with NVIDIA
// Dynamo-Triton", section "Why serving large sequential recommenders is hard":
// the attention kernel reads K/V straight from the paged cache; aitrends.kr
// article 100093, "HSTU sequential modelling": SiLU weighting instead of
// softmax plus a relative attention bias).
//
// One work item = (user, q-block of up to kQB = 64 new rows, head, key chunk).
// The q-block's rows form up to 4 groups of 16 queries, taken two at a time
// by "query sets".  The 4 waves of a workgroup cover QS query sets x KS key
// splits (QS = 2, KS = 2, or QS = 1, KS = 4 when the q-block has at most two
// groups): wave w owns query set w / KS and walks the chunk's 32-key steps
// w % KS, w % KS + KS, ...  A wave streams its own K and V^T fragments from
// the pool pages into registers one step ahead of use, so the key loop has no
// barriers, and each fragment feeds both of the wave's query groups.  Per
// step and group:
//   S^T[32 keys x 16 queries] = K * Q^T     (2 MFMA blocks; accumulators are
//                                           seeded with the bias)
//   A = SiLU(S) on the fp32 scores; masked only on diagonal tiles
//   O^T[d x 16]             += V^T * A
// The S^T accumulator of lane l holds 8 consecutive keys of one query, which
// is exactly the B-operand fragment of the second product, so scores never
// leave registers (K rows fed to S^T block b are permuted, row m -> key
// 8*(m/4) + 4*b + m%4, to make that true).  After the key loop the KS waves
// of a query set add their partial O through LDS (a two-round tree) and the
// first of them writes the item's output rows.  Queries are staged in LDS
// once per item and read back per step.
//
// Exponent domain: the projection stores Q' = -log2(e) * Q, and the bias
// tables here are scaled the same way, so S' = -log2(e) * s and
//   SiLU(s) = s / (1 + e^-s) = -ln(2) * S' / (1 + 2^S'),
// i.e. exp2, add, reciprocal, multiply per score.  The constant -ln(2) is
// applied with the 1/N scale by the norm kernel.
//
// Bias: a per-workgroup LDS table holds the scaled bias of every distance
// below kLut; a step whose distances all lie at or beyond kLut and span no
// more than one bucket width (2^(11-m) there) touches at most two buckets and
// takes a compare/select between two values; any other step takes the
// generic per-element bucket path.
// Partial outputs (fp32) go to the workspace; the chunks of a row are added
// by the norm kernel (no softmax, so partial sums over key ranges simply
// add).  Work items are fetched dynamically by a persistent grid (two
// workgroups per CU), one item ahead.
#include <type_traits>

#include "common.h"

namespace hstu {
namespace {

constexpr int kLut = 2048;
constexpr int kMaxChunkPages = kMaxChunkKeys / 16 + 1;
constexpr int kGroupsPerWave = 4;   // 16-query groups held by one wave
constexpr float kNegLog2e = -1.4426950408889634f;

template <typename T>
struct AttnArgs {
  const int32_t* pt;
  const T* k_pool;
  const T* v_pool;
  const T* q;
  const float* pos_bias;
  const float* ts_bias;
  const int64_t* ts;
  const int32_t* ts_off;
  WsHeader* hdr;
  const AttnItem* items;
  float* part;
  int H, D, ps_shift, maxP, nb, mbits, ntsb, tsmbits;
};

// First distance of bucket b (b >= 2^m) under the log-linear rule.
__device__ __forceinline__ int bucket_start(int b, int m) {
  const int s = 1 << m;
  if (b < s) return b;
  const int q = b >> m, r = b & (s - 1);
  return (s + r) << (q - 1);
}

template <typename T, int NC, int NO>
struct StepBuf {
  Frag<T> kf[2][NC];
  Frag<T> vf[NO];
};

template <typename T, int HD, int GPW>
__global__ __launch_bounds__(256, GPW == 2 ? 2 : 1) void attn_kernel(AttnArgs<T> a) {
  constexpr int NC = HD / 32;        // 32-wide slices of the head dim (contraction of S^T)
  constexpr int NO = HD / 16;        // 16-row blocks of O^T
  constexpr int RCH = HD / 4;        // float4 chunks per output row
  constexpr int ES = static_cast<int>(sizeof(T));
  constexpr int QCH = HD * ES / 16;  // 16-byte chunks per query row
  constexpr int FCH = 8 * ES / 16;   // chunks per 8-element fragment
  constexpr int SET_ROWS = 16 * GPW; // query rows of a query set (GPW groups)
  // The item's query tile (during the key loop) and the reduction buffers
  // (after it) share one LDS region: two slots of one query set's partial O.
  constexpr int RED_FLOATS = 2 * SET_ROWS * HD;
  constexpr int Q_FLOATS = kQB * HD * ES / 4;
  __shared__ __attribute__((aligned(16))) float s_big[RED_FLOATS > Q_FLOATS ? RED_FLOATS : Q_FLOATS];
  float* const s_red = s_big;
  T* const s_q = reinterpret_cast<T*>(s_big);
  __shared__ float s_lut[kLut];
  __shared__ float s_pb[kMaxBuckets];
  __shared__ float s_tb[kMaxBuckets];
  __shared__ int s_pages[kMaxChunkPages];
  __shared__ int s_next;
  if (a.hdr->status != 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  for (int i = tid; i < a.nb; i += 256) s_pb[i] = kNegLog2e * a.pos_bias[i];
  for (int i = tid; i < a.ntsb; i += 256) s_tb[i] = kNegLog2e * a.ts_bias[i];
  if (tid == 0) s_next = atomicAdd(&a.hdr->counter, 1);
  __syncthreads();
  for (int i = tid; i < kLut; i += 256) s_lut[i] = s_pb[bucket32(i, a.mbits, a.nb)];
  const int n_items = a.hdr->n_items;
  const int ps = 1 << a.ps_shift;
  const bool has_ts = a.ntsb > 0;
  const size_t page_elems = static_cast<size_t>(a.H) * ps * HD;

  for (;;) {
    __syncthreads();                       // previous item fully consumed; s_next published
    const int it = s_next;
    if (it >= n_items) break;
    const AttnItem item = a.items[it];
    // Per-lane values are re-derived from an opaque copy of the lane id in
    // every item so the compiler does not keep dozens of lane-dependent
    // addresses alive across the whole kernel.
    int tid_i = tid;
    asm volatile("" : "+v"(tid_i));
    const int lane_i = tid_i & 63;
    const int g = lane_i >> 4, l16 = lane_i & 15;
    const int koff0 = 8 * (l16 >> 2) + (l16 & 3);   // K row of S^T block b is koff0 + 4*b
    const int voff = 8 * g;                          // this lane's first key in a step
    const int u = item.a.x, q0 = item.a.y, h = item.a.z, k_lo = item.a.w;
    const int k_hi = item.b.x, off_u = item.b.y, n = item.b.z, c = item.b.w;
    const int len = c + n;
    const int nq = min(kQB, n - q0);
    const int ngroups = (nq + 15) >> 4;
    // page ids of the chunk, staged once per item; fetch the next item index
    const int32_t* ptu = a.pt + static_cast<size_t>(u) * a.maxP;
    const int pg0 = k_lo >> a.ps_shift;
    const int kst_end = min(k_hi, len);               // keys with a staged page
    const int npg = ((kst_end - 1) >> a.ps_shift) - pg0 + 1;
    for (int i = tid_i; i < npg; i += 256) s_pages[i] = ptu[pg0 + i];
    // query tile [kQB rows][HD], 16-byte chunks XOR-swizzled by row
    for (int q = tid_i; q < kQB * QCH; q += 256) {
      const int row = q / QCH, ch = q % QCH;
      const int t = min(q0 + row, n - 1);
      const u32x4 v = *reinterpret_cast<const u32x4*>(a.q + static_cast<size_t>(off_u + t) * a.D + h * HD + ch * (16 / ES));
      const int sw = ((row & 15) * FCH) & (QCH - 1);
      *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(s_q) + row * HD * ES + ((ch ^ sw) * 16)) = v;
    }
    __syncthreads();                       // all threads have read s_next; pages and queries staged
    if (tid == 0) s_next = atomicAdd(&a.hdr->counter, 1);

    // keys up to the q-block's last query position, in 32-key steps
    const int kend = min(k_hi, c + q0 + nq);
    const int nsteps = (kend - k_lo + 31) >> 5;

    // query sets x key splits of this item (see the top of the file)
    const int QS = ngroups > GPW ? 2 : 1;
    const int KS = 4 / QS;
    const int qs = w / KS, ks = w % KS;
    const int gb = GPW * qs;                           // first group of this wave's query set
    const int wg = min(GPW, ngroups - gb);             // its groups: 1..GPW

    f32x4 o[GPW][NO];
#pragma unroll
    for (int i = 0; i < GPW; ++i)
#pragma unroll
      for (int ob = 0; ob < NO; ++ob) o[i][ob] = f32x4{0.f, 0.f, 0.f, 0.f};
    // B-operand fragment of query group i, head-dim slice cc, from the LDS tile
    // (row & 15) == l16 for every group, so the swizzle is per lane only.
    const int q_sw = (l16 * FCH) & (QCH - 1);
    auto qfrag = [&](int qlane, int i, int cc, Frag<T>& f) __attribute__((always_inline)) {
      const int ch = (cc * 32 + g * 8) * ES / 16;
      load_frag(f, reinterpret_cast<const T*>(reinterpret_cast<const char*>(s_q) + qlane +
                                              (16 * i) * HD * ES + ((ch ^ q_sw) * 16)));
    };
    const size_t head_off = static_cast<size_t>(h) * ps * HD;
    const int64_t* tsu = has_ts ? a.ts + a.ts_off[u] : nullptr;

    // Per-lane element offsets inside a (page, head) block; together with a
    // wave-uniform page base they address every fragment of a step.
    // (A 32-key step lies in one page when page_size >= 32; with 16-token
    // pages its second half lives in the next page of the table.)
    const uint32_t k_lane0 = static_cast<uint32_t>(((koff0) & (ps - 1)) * HD + g * 8);
    const uint32_t k_lane1 = static_cast<uint32_t>(((koff0 + 4) & (ps - 1)) * HD + g * 8);
    const uint32_t v_lane = static_cast<uint32_t>(l16 * ps + (voff & (ps - 1)));
    const bool k_hi_half = koff0 >= 16;               // only matters for 16-token pages
    const bool v_hi_half = voff >= 16;

    // Loads the fragments of step s (steps past the end are clamped, so every
    // path issues the same load sequence).
    auto load_step = [&](int s, StepBuf<T, NC, NO>& sb) __attribute__((always_inline)) {
      const int kb = k_lo + 32 * min(s, nsteps - 1);
      const int pa = __builtin_amdgcn_readfirstlane(s_pages[(kb >> a.ps_shift) - pg0]);
      const int pb = (kb + 16 < kst_end) ? __builtin_amdgcn_readfirstlane(s_pages[((kb + 16) >> a.ps_shift) - pg0]) : pa;
      const size_t in_page = static_cast<size_t>(kb & (ps - 1));   // 0 for 16-token pages
      const T* ka = a.k_pool + static_cast<size_t>(pa) * page_elems + head_off + in_page * HD;
      const T* kz = a.k_pool + static_cast<size_t>(pb) * page_elems + head_off + in_page * HD;
      const T* va = a.v_pool + static_cast<size_t>(pa) * page_elems + head_off + in_page;
      const T* vz = a.v_pool + static_cast<size_t>(pb) * page_elems + head_off + in_page;
      const T* k0 = (ps >= 32 || !k_hi_half) ? ka : kz;
      const T* vb = (ps >= 32 || !v_hi_half) ? va : vz;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        load_frag(sb.kf[0][cc], k0 + k_lane0 + cc * 32);
        load_frag(sb.kf[1][cc], k0 + k_lane1 + cc * 32);
      }
#pragma unroll
      for (int ob = 0; ob < NO; ++ob) load_frag(sb.vf[ob], vb + v_lane + static_cast<uint32_t>(ob * 16 * ps));
    };

    // One 32-key step for the wave's local groups [I0, I0 + NG), as
    // straight-line code per bias case so that the S^T products, the SiLU of
    // one group and the O^T products of another can overlap.
    auto block = [&](auto i0c, auto ngc, int kb, StepBuf<T, NC, NO>& sb) __attribute__((always_inline)) {
      constexpr int I0 = decltype(i0c)::value;
      constexpr int NG = decltype(ngc)::value;
      // distance of element (local group I0 + i, block b, row r) is dl0 + 16*i - 4*b - r
      const int pset = c + q0 + 16 * (gb + I0);       // first query position of the block
      const int dl0 = pset + l16 - (kb + voff);
      const int dmin = pset - (kb + 31);
      const int dmax = pset + 16 * NG - 1 - kb;
      f32x4 st[NG][2];
      if (dmax < kLut) {
        if (dmin >= 0) {
#pragma unroll
          for (int i = 0; i < NG; ++i)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
              for (int r = 0; r < 4; ++r) st[i][b][r] = s_lut[dl0 + 16 * i - 4 * b - r];
        } else {
#pragma unroll
          for (int i = 0; i < NG; ++i)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
              for (int r = 0; r < 4; ++r) st[i][b][r] = s_lut[max(dl0 + 16 * i - 4 * b - r, 0)];
        }
      } else if (dmin >= kLut && (kLut >> a.mbits) >= dmax - dmin + 1) {
        // every distance here falls into one or two adjacent buckets
        const int blo = bucket32(dmin, a.mbits, a.nb), bhi = bucket32(dmax, a.mbits, a.nb);
        const float vlo = s_pb[blo], vhi = s_pb[bhi];
        const int bnd = blo == bhi ? 0x7fffffff : bucket_start(bhi, a.mbits);
#pragma unroll
        for (int i = 0; i < NG; ++i)
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) st[i][b][r] = (dl0 + 16 * i - 4 * b - r) >= bnd ? vhi : vlo;
      } else {
#pragma unroll
        for (int i = 0; i < NG; ++i)
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) st[i][b][r] = s_pb[bucket32(dl0 + 16 * i - 4 * b - r, a.mbits, a.nb)];
      }
      if (has_ts) {
#pragma unroll
        for (int i = 0; i < NG; ++i) {
          const int64_t tp = tsu[min(pset + 16 * i + l16, len - 1)];
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = min(kb + voff + 4 * b + r, len - 1);
              st[i][b][r] += s_tb[bucket64(tp - tsu[key], a.tsmbits, a.ntsb)];
            }
        }
      }
      // The query tile is read from LDS at every step (an opaque offset keeps
      // the compiler from hoisting all query fragments into registers).
      int qlane = l16 * HD * ES;
      asm volatile("" : "+v"(qlane));
#pragma unroll
      for (int i = 0; i < NG; ++i)
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
          Frag<T> qf;
          qfrag(qlane, gb + I0 + i, cc, qf);
#pragma unroll
          for (int b = 0; b < 2; ++b) st[i][b] = mma16(sb.kf[b][cc], qf, st[i][b]);
        }
      Frag<T> af[NG];
      if (dmin >= 0) {
#pragma unroll
        for (int i = 0; i < NG; ++i)
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float sv = st[i][b][r];
              set_elem(af[i], 4 * b + r, sv * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(sv)));
            }
      } else {                                       // causal mask on the diagonal
#pragma unroll
        for (int i = 0; i < NG; ++i)
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float sv = st[i][b][r];
              const float av = sv * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(sv));
              set_elem(af[i], 4 * b + r, (dl0 + 16 * i - 4 * b - r) >= 0 ? av : 0.0f);
            }
      }
#pragma unroll
      for (int i = 0; i < NG; ++i)
#pragma unroll
        for (int ob = 0; ob < NO; ++ob) o[I0 + i][ob] = mma16(sb.vf[ob], af[i], o[I0 + i][ob]);
    };

    // One 32-key step for the wave's NG groups, two groups at a time.
    auto compute = [&](auto ngc, int kb, StepBuf<T, NC, NO>& sb) __attribute__((always_inline)) {
      constexpr int NG = decltype(ngc)::value;
      if (kb + 32 > len) {                           // zero V of keys past the sequence
        const int nvalid = len - (kb + voff);
#pragma unroll
        for (int ob = 0; ob < NO; ++ob)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e >= nvalid) set_elem(sb.vf[ob], e, 0.0f);
      }
      block(std::integral_constant<int, 0>{}, std::integral_constant<int, (NG < 2 ? NG : 2)>{}, kb, sb);
      if constexpr (NG > 2)
        block(std::integral_constant<int, 2>{}, std::integral_constant<int, NG - 2>{}, kb, sb);
    };

    // The wave walks steps ks, ks + KS, ...; two register buffers alternate
    // so the next step's fragments are in flight while one is computed.
    const int my_steps = nsteps > ks ? (nsteps - ks + KS - 1) / KS : 0;
    auto walk = [&](auto ngc) __attribute__((always_inline)) {
      StepBuf<T, NC, NO> b0, b1;
      load_step(ks, b0);
      for (int j = 0; j < my_steps; j += 2) {
        load_step(ks + KS * (j + 1), b1);
        compute(ngc, k_lo + 32 * (ks + KS * j), b0);
        if (j + 1 >= my_steps) break;
        load_step(ks + KS * (j + 2), b0);
        compute(ngc, k_lo + 32 * (ks + KS * (j + 1)), b1);
      }
    };
    if (my_steps > 0) {
      if constexpr (GPW == 4) {
        switch (wg) {
          case 4: walk(std::integral_constant<int, 4>{}); break;
          case 3: walk(std::integral_constant<int, 3>{}); break;
          case 2: walk(std::integral_constant<int, 2>{}); break;
          default: walk(std::integral_constant<int, 1>{}); break;
        }
      } else {
        if (wg == 2) walk(std::integral_constant<int, 2>{});
        else walk(std::integral_constant<int, 1>{});
      }
    }

    // Add up the KS partial O of each query set through LDS (slot layout:
    // [32 rows][d], 16-byte chunks XOR-swizzled by row; every lane reads back
    // exactly the elements it holds), then the set's first wave writes out.
    __syncthreads();                       // every wave is done with the query tile
    int lane_r = lane;
    asm volatile("" : "+v"(lane_r));
    const int gr = lane_r >> 4, lr = lane_r & 15;
    auto slot_ptr = [&](int sl, int i, int ob) __attribute__((always_inline)) -> float* {
      const int row = 16 * i + lr;
      const int ch = (ob * 4 + gr) ^ (row & (RCH - 1));
      return s_red + sl * SET_ROWS * HD + row * HD + ch * 4;
    };
    auto park = [&](int sl) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < GPW; ++i)
#pragma unroll
        for (int ob = 0; ob < NO; ++ob) *reinterpret_cast<f32x4*>(slot_ptr(sl, i, ob)) = o[i][ob];
    };
    auto gather = [&](int sl) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < GPW; ++i)
#pragma unroll
        for (int ob = 0; ob < NO; ++ob) o[i][ob] += *reinterpret_cast<const f32x4*>(slot_ptr(sl, i, ob));
    };
    // round 1: odd splits hand their sums to the even split below them
    if (ks & 1) park(KS == 2 ? qs : (ks >> 1));
    __syncthreads();
    if (!(ks & 1)) gather(KS == 2 ? qs : (ks >> 1));
    if (KS == 4) {                          // round 2: split 2 hands over to split 0
      __syncthreads();
      if (ks == 2) park(0);
      __syncthreads();
      if (ks == 0) gather(0);
    }
    if (ks == 0) {
#pragma unroll
      for (int i = 0; i < GPW; ++i) {
        const int row = 16 * (gb + i) + lr;             // row inside the q-block
        if (i < wg && q0 + row < n) {
          float* dst = a.part + (static_cast<size_t>(it) * kQB + row) * HD + 4 * gr;
#pragma unroll
          for (int ob = 0; ob < NO; ++ob) *reinterpret_cast<f32x4*>(dst + ob * 16) = o[i][ob];
        }
      }
    }
  }
}

template <typename T, int HD>
hipError_t attn_t(const hstu_layer_desc& d, const int32_t* pt, const void* k_pool, const void* v_pool,
                  const float* pos_bias, const float* ts_bias, const int64_t* ts, const int32_t* ts_off,
                  const WsPtrs& ws, int grid, hipStream_t stream) {
  AttnArgs<T> a;
  a.pt = pt;
  a.k_pool = static_cast<const T*>(k_pool);
  a.v_pool = static_cast<const T*>(v_pool);
  a.q = static_cast<const T*>(ws.q);
  a.pos_bias = pos_bias;
  a.ts_bias = ts_bias;
  a.ts = ts;
  a.ts_off = ts_off;
  a.hdr = ws.hdr;
  a.items = ws.items;
  a.part = ws.part;
  a.H = d.num_heads;
  a.D = d.hidden;
  a.ps_shift = __builtin_ctz(static_cast<unsigned>(d.page_size));
  a.maxP = d.max_pages_per_user;
  a.nb = d.pos_buckets;
  a.mbits = d.pos_mbits;
  a.ntsb = d.ts_buckets;
  a.tsmbits = d.ts_mbits;
  attn_kernel<T, HD, kGroupsPerWave><<<grid, 256, 0, stream>>>(a);
  return hipGetLastError();
}

template <typename T>
hipError_t attn_dt(const hstu_layer_desc& d, const int32_t* pt, const void* k_pool, const void* v_pool,
                   const float* pos_bias, const float* ts_bias, const int64_t* ts, const int32_t* ts_off,
                   const WsPtrs& ws, int grid, hipStream_t stream) {
  switch (d.head_dim) {
    case 32: return attn_t<T, 32>(d, pt, k_pool, v_pool, pos_bias, ts_bias, ts, ts_off, ws, grid, stream);
    case 64: return attn_t<T, 64>(d, pt, k_pool, v_pool, pos_bias, ts_bias, ts, ts_off, ws, grid, stream);
    default: return attn_t<T, 128>(d, pt, k_pool, v_pool, pos_bias, ts_bias, ts, ts_off, ws, grid, stream);
  }
}

}  // namespace

hipError_t launch_attn(const hstu_layer_desc& d, const int32_t* pt, const void* k_pool, const void* v_pool,
                       const float* pos_bias, const float* ts_bias, const int64_t* ts,
                       const int32_t* ts_off, const WsPtrs& ws, int grid, hipStream_t stream) {
  if (d.dtype == HSTU_BF16)
    return attn_dt<bf16>(d, pt, k_pool, v_pool, pos_bias, ts_bias, ts, ts_off, ws, grid, stream);
  return attn_dt<float>(d, pt, k_pool, v_pool, pos_bias, ts_bias, ts, ts_off, ws, grid, stream);
}

}  // namespace hstu
