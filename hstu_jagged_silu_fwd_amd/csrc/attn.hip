// Paged jagged SiLU attention (HSTU pointwise attention over a paged KV
// cache; NVIDIA blog "Deploying an HSTU generative recommender with NVIDIA
// Dynamo-Triton", section "Why serving large sequential recommenders is hard":
// the attention kernel reads K/V straight from the paged cache; aitrends.kr
// article 100093, "HSTU sequential modelling": SiLU weighting instead of
// softmax plus a relative attention bias).
//
// One work item = (user, q-block of up to kQB = 256 new rows, head, key
// chunk): a q-block covers all new rows of most users, so each history key is
// read once per head and chunk.  A workgroup of eight waves takes one item at
// a time.  The q-block's 16-row query groups are taken in adjacent pairs, one
// pair per wave; when the block has few groups the waves also split the key
// steps: they form P phases (P = 4, 2 or 1, as many as the waves allow) and
// the waves of phase p multiply the steps s = p (mod P), so every wave has
// products to do even for a single 16-row group.  The chunk's keys are walked
// in 32-key steps.  A step's K rows [32][d] and V^T rows [d][32] are copied
// from their pool pages into a ring of NST LDS stages with direct-to-LDS
// loads that the waves share out; one barrier per round of P steps hands the
// round's stages from the loads to the products, and the loads of the round D
// rounds ahead (D = NST/P - 1) go into the stages the previous round freed.
// At the end of an item the phases' partial sums meet in LDS.
// Per step and wave:
//   S^T[32 keys x 16 queries] = K * Q^T     (2 MFMA blocks over d; the
//                                           accumulators start at the bias)
//   A = SiLU(S) on the fp32 scores; masked only on diagonal steps and on
//                                           steps that reach the candidates
//   O^T[d x 16]             += V^T * A
// K rows feeding S^T block b are read in the permuted order row m -> key
// 8*(m/4) + 4*b + m%4, so the S^T accumulator of a lane holds 8 consecutive
// keys of one query, which is exactly its B-operand fragment for the second
// product: scores never leave registers.  Each K and V^T fragment read from
// LDS feeds both of a wave's groups.  The query fragments stay in registers
// for the whole item.  In LDS the 16-byte chunks of every row are
// XOR-permuted so that the fragment reads of 16 lanes (16 rows, one chunk
// each) fall into distinct banks.
//
// Exponent domain: the projection stores Q' = -log2(e) * Q, and the bias
// tables here are scaled the same way, so S' = -log2(e) * s and
//   SiLU(s) = s / (1 + e^-s) = -ln(2) * S' / (1 + 2^S'),
// i.e. exp2, add, reciprocal, multiply per score.  The constant -ln(2) is
// applied with the 1/N scale by the norm kernel.
//
// Bias: a per-workgroup LDS table holds the scaled bias of every distance
// below kLut, in descending order of distance: the 8 scores a lane holds per
// group and step have 8 consecutive distances, so they read 8 consecutive
// entries at immediate offsets from one address.  A step whose distances all
// lie at or beyond kLut and span no more than one bucket width (2^(12-m)
// there) touches at most two buckets and takes a compare/select between two
// values; any other step takes the generic per-element bucket path.  Timestamps, when present, travel with
// their keys through the ring; each lane keeps its query's in a register.
//
// Candidates: when the call gives per-user candidate counts m_u, a query at
// or past the first candidate position cs = c + n - m_u sees only the keys
// before cs and itself (a key at or past cs is kept only on the diagonal).
// Rows before cs see nothing past cs anyway, so one mask covers every row.
//
// Partial outputs (fp32) go to the workspace; the chunks of a row are added
// by the norm kernel (no softmax, so partial sums over key ranges simply
// add).  The grid is persistent, one workgroup per CU: workgroup i takes
// item i first and, when there are more items than workgroups, fetches
// further items dynamically, one ahead.
#include <type_traits>

#include "common.h"

namespace hstu {
namespace {

constexpr int kLut = 4096;
constexpr int kLutPad = 64;        // entries past the table (negative distances: masked scores)
constexpr int kStepKeys = 32;
constexpr int kMaxChunkPages = kMaxChunkKeys / 16 + 1;
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
  const int32_t* ncand;      // per-user candidate counts, or null
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

constexpr int kWaves = 8;          // waves per workgroup
constexpr int kGpw = 2;            // 16-query groups per wave (an adjacent pair)
static_assert(kQB == 16 * kWaves * kGpw, "a q-block is two groups per wave");

// Sizes of one ring stage (one 32-key step of K and V^T) for element type T
// and head dim HD, and of the ring.
template <typename T, int HD>
struct StepGeo {
  static constexpr int ES = static_cast<int>(sizeof(T));
  static constexpr int CE = 16 / ES;                   // elements per 16-byte chunk
  static constexpr int KCH = HD / CE;                  // chunks per K row
  static constexpr int VCH = kStepKeys / CE;           // chunks per V^T row
  static constexpr int KBYTES = kStepKeys * HD * ES;   // the K rows of a step
  static constexpr int STAGE = 2 * KBYTES;             // K rows, then V^T rows
  static constexpr int NBLK = STAGE / 1024;            // 1 KiB loads per stage
  static constexpr int IPW = (NBLK + kWaves - 1) / kWaves;   // loads per wave and stage (at most)
  // ring: 8 stages, or as many as fit in 128 KiB (a power of two)
  static constexpr int NST_FIT = 131072 / STAGE;
  static constexpr int NST = NST_FIT >= 8 ? 8 : (NST_FIT >= 4 ? 4 : 2);
  static constexpr int PMAX = NST / 2;                 // phases: the ring holds two rounds of PMAX steps
  // chunk permutation of K row `key`: (m >> KSH) with m = (key & 3) | (((key >> 3) & 3) << 2),
  // m being the lane (mod 16) that reads the row; V^T row e: (e >> VSH) & (VCH - 1)
  static constexpr int KSH = KCH >= 16 ? 0 : (KCH == 8 ? 1 : 2);
  static constexpr int VSH = VCH == 4 ? 2 : 1;
  static_assert(KCH >= 4 && (VCH == 4 || VCH == 8), "supported geometry");
  static_assert(NBLK * 1024 == STAGE, "whole loads per stage");
  static_assert((kStepKeys * KCH) % 64 == 0, "a load never straddles K and V^T");
  static_assert((IPW + 1) * (NST - 2) <= 23, "wait count range");
  // the phase reduction reuses the ring: at most (PMAX-1) * (kWaves/PMAX)
  // waves hand over two 16 x HD fp32 tiles each
  static_assert(NST * STAGE >= (PMAX - 1) * (kWaves / PMAX) * kGpw * 16 * HD * 4, "reduction fits the ring");
};

template <typename T, int HD, bool CAND>
__global__ __launch_bounds__(64 * kWaves) void attn_kernel(AttnArgs<T> a) {
  using G = StepGeo<T, HD>;
  constexpr int CE = G::CE, KCH = G::KCH, VCH = G::VCH, NST = G::NST, IPW = G::IPW;
  constexpr int NT = 64 * kWaves;
  constexpr int NC = HD / 32;        // 32-wide slices of the head dim (contraction of S^T)
  constexpr int NO = HD / 16;        // 16-row blocks of O^T
  static_assert(kMaxChunkPages <= 2 * NT, "two page ids per thread");
  __shared__ __attribute__((aligned(1024))) unsigned char s_ring[NST * G::STAGE];
  __shared__ __attribute__((aligned(256))) int64_t s_ts[NST][kStepKeys];
  __shared__ float s_rlut[kLut + kLutPad];   // s_rlut[x]: bias of distance kLut - 1 - x
  __shared__ float s_pb[kMaxBuckets];
  __shared__ float s_tb[kMaxBuckets];
  __shared__ int s_pages[kMaxChunkPages];
  __shared__ int s_next;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  // Status words and item count, the first item (static: workgroup i takes item i;
  // the grid never exceeds the item capacity) and the bias tables (up to two
  // entries of each per thread) are all loaded at once.  The tables reach LDS
  // (and the distance table is built) inside the first item's set-up, after
  // its page-id and query loads have gone out, so those round trips overlap.
  static_assert(kMaxBuckets <= 2 * NT, "two bias entries per thread");
  const int4 hv = *reinterpret_cast<const int4*>(a.hdr);
  AttnItem item = a.items[blockIdx.x];
  float pbv[2], tbv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = tid + j * NT;
    pbv[j] = i < a.nb ? a.pos_bias[i] : 0.f;
    tbv[j] = i < a.ntsb ? a.ts_bias[i] : 0.f;
  }
  if ((hv.x | hv.y) != 0) return;          // status words: prep rejected the call
  const int n_items = hv.z;
  const bool dynamic = n_items > static_cast<int>(gridDim.x);
  bool tables_ready = false;
  const int ps = 1 << a.ps_shift;
  const bool has_ts = a.ntsb > 0;
  const int g = lane >> 4, l16 = lane & 15;
  // K row read by this lane for S^T block b is krow0 + 4*b; both rows share
  // one chunk permutation.  V^T rows 16*ob + l16 share one too.
  const int krow0 = 8 * (l16 >> 2) + (l16 & 3);
  const int ksw = l16 >> G::KSH;
  const int vsw = (l16 >> G::VSH) & (VCH - 1);
  // loads this wave issues per step (its K/V^T blocks, plus the key
  // timestamps for wave 0)
  const int my_blk = min(max(G::NBLK - w * IPW, 0), IPW);
  const int my_cnt = my_blk + ((has_ts && w == 0) ? 1 : 0);
  // Source of this lane's 16 bytes in load j, relative to the step's page
  // base: element offset lo[j] inside the (page, head) block, and whether it
  // lies in the step's second page (16-token pages only: a 32-key step then
  // spans two pages).
  uint32_t lo[IPW];
  bool hi[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int q = (w * IPW + j) * 64 + lane;             // 16-byte chunk of the stage
    if (q < kStepKeys * KCH) {                           // K row `row`, chunk position p
      const int row = q / KCH, p = q % KCH;
      const int m = (row & 3) | (((row >> 3) & 3) << 2);
      const int cch = p ^ (m >> G::KSH);
      hi[j] = row >= ps;
      lo[j] = static_cast<uint32_t>((row & (ps - 1)) * HD + cch * CE);
    } else {                                             // V^T row e, chunk position p
      const int qv = q - kStepKeys * KCH;
      const int e = qv / VCH, p = qv % VCH;
      const int key = (p ^ ((e >> G::VSH) & (VCH - 1))) * CE;
      hi[j] = key >= ps;
      lo[j] = static_cast<uint32_t>(e * ps + (key & (ps - 1)));
    }
  }

  int it = blockIdx.x;
  for (;;) {
    if (it >= n_items) break;
    const int u = __builtin_amdgcn_readfirstlane(item.a.x);
    const int q0 = __builtin_amdgcn_readfirstlane(item.a.y);
    const int h = __builtin_amdgcn_readfirstlane(item.a.z);
    const int k_lo = __builtin_amdgcn_readfirstlane(item.a.w);
    const int k_hi = __builtin_amdgcn_readfirstlane(item.b.x);
    const int off_u = __builtin_amdgcn_readfirstlane(item.b.y);
    const int n = __builtin_amdgcn_readfirstlane(item.b.z);
    const int c = __builtin_amdgcn_readfirstlane(item.b.w);
    const int len = c + n;
    // first candidate position (the instance without candidates has none)
    const int cs = CAND ? len - a.ncand[u] : 0x7fffffff;
    const int nq = min(kQB, n - q0);
    const int ngroups = (nq + 15) >> 4;
    // Phases: the waves form P phases of WP = kWaves/P waves (columns);
    // the waves of phase p multiply the steps s = p (mod P).  Few groups ->
    // several phases, so that every wave has products to do.  A column owns
    // one or two query groups (two share every K/V fragment read).  Waves w
    // and w+4 share a SIMD: they are columns j and j+WP/2 of one phase.  So
    // that no SIMD holds two pairs while another holds a single group,
    // columns below WP/2 take groups in pairs from 0, and the others take
    // the remaining groups, in pairs only as far as needed.
    const int NW = (ngroups + 1) >> 1;
    const int P = (G::PMAX >= 4 && 4 * NW <= kWaves) ? 4 : ((G::PMAX >= 2 && 2 * NW <= kWaves) ? 2 : 1);
    const int D = NST / P - 1;                         // rounds of loads in flight ahead
    const int half = kWaves / (2 * P);
    const int ph = w & (P - 1), col = w / P;
    int gi0, ng_w;                                     // this wave's first group and group count
    if (col < half) {
      gi0 = 2 * col;
      ng_w = min(max(ngroups - gi0, 0), 2);
    } else {
      const int j = col - half, rest = max(ngroups - 2 * half, 0), npairs = max(rest - half, 0);
      gi0 = j < npairs ? 2 * half + 2 * j : 2 * half + npairs + j;
      ng_w = j < npairs ? 2 : (gi0 < ngroups ? 1 : 0);
    }
    const int32_t* ptu = a.pt + static_cast<size_t>(u) * a.maxP;
    const int pg0 = k_lo >> a.ps_shift;
    const int kst_end = min(k_hi, len);                // keys whose pages are staged
    const int npg = ((kst_end - 1) >> a.ps_shift) - pg0 + 1;
    // the next item's index is fetched now, alongside the page ids and the
    // query fragments; all three have landed at the wait below.  (With no
    // more items than workgroups nothing is fetched: the shared counter's
    // atomics would only queue up behind each other.)
    int nxt = 0;
    if (dynamic && tid == 0) nxt = atomicAdd(&a.hdr->counter, 1);
    const int pid0 = tid < npg ? ptu[pg0 + tid] : 0;
    const int pid1 = tid + NT < npg ? ptu[pg0 + tid + NT] : 0;
    Frag<T> qf[kGpw][NC];
    int64_t tq[kGpw];
    const int64_t* tsu = has_ts ? a.ts + a.ts_off[u] : nullptr;
#pragma unroll
    for (int i = 0; i < kGpw; ++i) {
      const int qrow = min(q0 + 16 * (gi0 + i) + l16, n - 1);
      const T* qp = a.q + static_cast<size_t>(off_u + qrow) * a.D + h * HD + 8 * g;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) load_frag(qf[i][cc], qp + cc * 32);
      tq[i] = has_ts ? tsu[c + qrow] : 0;
    }
    const int kend = min(k_hi, c + q0 + nq);           // keys up to the block's last query
    const int nsteps = (kend - k_lo + kStepKeys - 1) / kStepKeys;
    const int nrounds = (nsteps + P - 1) / P;
    // Let these loads land before the ring starts: the compiler cannot count
    // outstanding loads across the key loop, so it would otherwise wait for
    // every in-flight stage at the first use of a query fragment.
    if (!tables_ready) {                   // first item: bias tables into LDS meanwhile
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int i = tid + j * NT;
        if (i < a.nb) s_pb[i] = kNegLog2e * pbv[j];
        if (i < a.ntsb) s_tb[i] = kNegLog2e * tbv[j];
      }
      __syncthreads();
      for (int i = tid; i < kLut + kLutPad; i += NT)
        s_rlut[i] = i < kLut ? s_pb[bucket32(kLut - 1 - i, a.mbits, a.nb)] : 0.f;
      tables_ready = true;
    }
    wait_vm<0>();
    if (tid < npg) s_pages[tid] = pid0;
    if (tid + NT < npg) s_pages[tid + NT] = pid1;
    if (tid == 0) s_next = dynamic ? static_cast<int>(gridDim.x) + nxt : n_items;
    __syncthreads();                       // pages staged; s_next published
    // the next item's descriptor, in flight during this item's key loop
    const int it_next = s_next;
    AttnItem item_next = item;
    if (it_next < n_items) item_next = a.items[it_next];

    // ---- loads of step s into stage s % NST ----
    const size_t kv_head = static_cast<size_t>(h) * ps * HD;      // head block inside a page
    const size_t page_elems = static_cast<size_t>(a.H) * ps * HD;
    // Keys past the staged range (last step only) read rows of the step's
    // own pages: in bounds; their scores are masked and their V^T columns
    // zeroed in LDS before the products.
    auto issue = [&](int s) __attribute__((always_inline)) {
      const int kb = k_lo + kStepKeys * s;
      unsigned char* stg = s_ring + (s % NST) * G::STAGE;
      const int pa = __builtin_amdgcn_readfirstlane(s_pages[(kb >> a.ps_shift) - pg0]);
      const int pb = (ps < kStepKeys && kb + ps < kst_end)
                         ? __builtin_amdgcn_readfirstlane(s_pages[((kb + ps) >> a.ps_shift) - pg0]) : pa;
      const size_t in_page = static_cast<size_t>(kb & (ps - 1));   // 0 for 16-token pages
      const size_t ha = static_cast<size_t>(pa) * page_elems + kv_head;
      const size_t hb = static_cast<size_t>(pb) * page_elems + kv_head;
#pragma unroll
      for (int j = 0; j < IPW; ++j) {
        const int blk = w * IPW + j;                   // 1 KiB block of the stage
        if (blk >= G::NBLK) break;                     // uniform
        const T* src;
        if (blk * 64 < kStepKeys * KCH)                // K rows
          src = a.k_pool + (hi[j] ? hb : ha) + in_page * HD + lo[j];
        else                                           // V^T rows
          src = a.v_pool + (hi[j] ? hb : ha) + in_page + lo[j];
        dma_lds16(src, stg + blk * 1024);
      }
      if (has_ts && w == 0) {                          // the step's key timestamps
        const int key = min(kb + (lane >> 1), len - 1);
        const int32_t* tsrc = reinterpret_cast<const int32_t*>(tsu + key) + (lane & 1);
        dma_lds4(tsrc, &s_ts[s % NST][0]);
      }
    };

    f32x4 o[kGpw][NO];
#pragma unroll
    for (int i = 0; i < kGpw; ++i)
#pragma unroll
      for (int ob = 0; ob < NO; ++ob) o[i][ob] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- products of step s for this wave's first NG query groups ----
    auto compute = [&](auto ngc, int s) __attribute__((always_inline)) {
      constexpr int NG = decltype(ngc)::value;
      const int kb = k_lo + kStepKeys * s;
      const unsigned char* stg = s_ring + (s % NST) * G::STAGE;
      f32x4 st[NG][2];
      int dl0[NG], dmn[NG];
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        // distance of element (block b, row r) is dl0 - 4*b - r
        const int pq = c + q0 + 16 * (gi0 + i);        // first query position of the group
        dl0[i] = pq + l16 - (kb + 8 * g);
        const int dmin = pq - (kb + kStepKeys - 1);
        const int dmax = pq + 15 - kb;
        dmn[i] = dmin;
        if (dmax < kLut) {
          // element (b, r) has distance dl0 - (4b + r), entry x0 + 4b + r; a
          // lane whose distances are all negative reads padding
          const float* lp = s_rlut + min(kLut - 1 - dl0[i], kLut + kLutPad - 8);
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) st[i][b][r] = lp[4 * b + r];
        } else if (dmin >= kLut && (kLut >> a.mbits) >= dmax - dmin + 1) {
          // every distance here falls into one or two adjacent buckets
          const int blo = bucket32(dmin, a.mbits, a.nb), bhi = bucket32(dmax, a.mbits, a.nb);
          const float vlo = s_pb[blo], vhi = s_pb[bhi];
          if (blo == bhi) {                          // uniform: the whole step in one bucket
#pragma unroll
            for (int b = 0; b < 2; ++b) st[i][b] = f32x4{vlo, vlo, vlo, vlo};
          } else {
            const int bnd = bucket_start(bhi, a.mbits);
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
              for (int r = 0; r < 4; ++r) st[i][b][r] = (dl0[i] - 4 * b - r) >= bnd ? vhi : vlo;
          }
        } else {
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) st[i][b][r] = s_pb[bucket32(dl0[i] - 4 * b - r, a.mbits, a.nb)];
        }
        if (has_ts) {
          const int64_t* tk = &s_ts[s % NST][8 * g];
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) st[i][b][r] += s_tb[bucket64(tq[i] - tk[4 * b + r], a.tsmbits, a.ntsb)];
        }
      }
      // S^T = K * Q^T over the head dim; each K fragment feeds every group.
      // All of the step's K fragment reads go out before the first product,
      // so their LDS latency is paid once.
      const unsigned char* k0p = stg + krow0 * (KCH * 16);
      const unsigned char* k1p = k0p + 4 * (KCH * 16);
      Frag<T> kf[NC][2];
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const int chunk = (cc * 32 + 8 * g) / CE;
        read_frag(kf[cc][0], k0p, chunk, ksw);
        read_frag(kf[cc][1], k1p, chunk, ksw);
      }
#pragma unroll
      for (int cc = 0; cc < NC; ++cc)
#pragma unroll
        for (int i = 0; i < NG; ++i) {
          st[i][0] = mma16(kf[cc][0], qf[i][cc], st[i][0]);
          st[i][1] = mma16(kf[cc][1], qf[i][cc], st[i][1]);
        }
      // V^T fragments are read now so that their LDS latency overlaps the
      // SiLU below.
      Frag<T> vf[NO];
      {
        const unsigned char* vp = stg + G::KBYTES + l16 * (VCH * 16);
        const int vchunk = (8 * g) / CE;
#pragma unroll
        for (int ob = 0; ob < NO; ++ob) read_frag(vf[ob], vp + ob * 16 * (VCH * 16), vchunk, vsw);
      }
      // SiLU in independent batches (every exp2, then every reciprocal) so
      // that no transcendental waits on the one before it
      float av[NG][8];
#pragma unroll
      for (int i = 0; i < NG; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) av[i][e] = __builtin_amdgcn_exp2f(st[i][e >> 2][e & 3]);
#pragma unroll
      for (int i = 0; i < NG; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) av[i][e] = __builtin_amdgcn_rcpf(1.0f + av[i][e]);
      Frag<T> af[NG];
#pragma unroll
      for (int i = 0; i < NG; ++i) {
#pragma unroll
        for (int e = 0; e < 8; ++e) av[i][e] *= st[i][e >> 2][e & 3];
        if (CAND && kb + kStepKeys > cs) {           // keys at or past the candidates
          const int ce = cs - (kb + 8 * g);          // element e's key is past cs when e >= ce
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int de = dl0[i] - e;
            av[i][e] = (de >= 0 && (e < ce || de == 0)) ? av[i][e] : 0.0f;
          }
        } else if (dmn[i] < 0) {                     // causal mask on the diagonal
#pragma unroll
          for (int e = 0; e < 8; ++e) av[i][e] = dl0[i] - e >= 0 ? av[i][e] : 0.0f;
        }
        set_frag(af[i], av[i]);
      }
      // O^T += V^T * A
#pragma unroll
      for (int ob = 0; ob < NO; ++ob)
#pragma unroll
        for (int i = 0; i < NG; ++i) o[i][ob] = mma16(vf[ob], af[i], o[i][ob]);
    };

    // ---- the key loop: one barrier per round of P steps.  Round r's steps
    // sit in stages rP .. rP+P-1 (mod NST); the loads of round r+D are
    // issued once round r-1's stages are free, so D rounds are in flight
    // while one is multiplied.  (The wave's group count is fixed for the
    // item, so each count gets a loop of its own.) ----
    for (int s = 0; s < min(D * P, nsteps); ++s) issue(s);
    // Only the last step can reach past the staged keys.  Those keys lie
    // beyond every query of the item, so their scores are masked; their V^T
    // columns are zeroed in LDS (by the lanes that loaded them, once their
    // loads have landed) so that stale pool memory cannot turn a masked
    // product into NaN, and the products need no tail case of their own.
    const int tail_round = k_lo + kStepKeys * nsteps > kst_end ? (nsteps - 1) / P : -1;
    auto zero_tail = [&]() __attribute__((always_inline)) {
      const int kb = k_lo + kStepKeys * (nsteps - 1);
      const int nvalid = kst_end - kb;                 // staged keys of the step
      unsigned char* stg = s_ring + ((nsteps - 1) % NST) * G::STAGE;
#pragma unroll
      for (int j = 0; j < IPW; ++j) {
        const int blk = w * IPW + j;
        if (blk >= G::NBLK) break;                     // uniform
        if (blk * 64 < kStepKeys * KCH) continue;      // K rows: masked by the scores
        const int qv = blk * 64 + lane - kStepKeys * KCH;
        const int e = qv / VCH, p = qv % VCH;
        const int key0 = (p ^ ((e >> G::VSH) & (VCH - 1))) * CE;   // first key of this lane's chunk
        T* dst = reinterpret_cast<T*>(stg + blk * 1024 + lane * 16);
#pragma unroll
        for (int t = 0; t < CE; ++t)
          if (key0 + t >= nvalid) dst[t] = from_f32<T>(0.0f);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);             // lgkmcnt(0): the zeros are in LDS
    };
    auto key_loop = [&](auto ngc) __attribute__((always_inline)) {
      for (int r = 0; r < nrounds; ++r) {
        // round r's loads have landed once only those issued after them remain
        const int later = min((r + D) * P, nsteps) - (r + 1) * P;
        if (later > 0) wait_vm_n(later * my_cnt);
        else wait_vm<0>();
        if (r == tail_round) zero_tail();
        bar();                             // round r visible; round r-1 no longer read
        const bool early = w >= 4;
        if (early)
          for (int s2 = (r + D) * P; s2 < min((r + D + 1) * P, nsteps); ++s2) issue(s2);
        if constexpr (decltype(ngc)::value > 0) {
          const int s = r * P + ph;
          if (s < nsteps) compute(ngc, s);
        }
        if (!early)
          for (int s2 = (r + D) * P; s2 < min((r + D + 1) * P, nsteps); ++s2) issue(s2);
      }
    };
    if (ng_w == 2) key_loop(std::integral_constant<int, 2>{});
    else if (ng_w == 1) key_loop(std::integral_constant<int, 1>{});
    else key_loop(std::integral_constant<int, 0>{});

    // ---- phases 1..P-1 hand their partial sums to phase 0 through the
    // (now idle) ring; phase 0 adds them and writes the item's rows ----
    if (P > 1) {
      __syncthreads();                     // every wave is done with the ring
      f32x4* red = reinterpret_cast<f32x4*>(s_ring);
      if (ph > 0 && ph < P) {
        f32x4* dst = red + ((ph - 1) * (kWaves / P) + col) * (kGpw * NO * 64);
#pragma unroll
        for (int i = 0; i < kGpw; ++i)
#pragma unroll
          for (int ob = 0; ob < NO; ++ob) dst[(i * NO + ob) * 64 + lane] = o[i][ob];
      }
      __syncthreads();
      if (ph == 0) {
        for (int p = 1; p < P; ++p) {
          const f32x4* srcp = red + ((p - 1) * (kWaves / P) + col) * (kGpw * NO * 64);
#pragma unroll
          for (int i = 0; i < kGpw; ++i)
#pragma unroll
            for (int ob = 0; ob < NO; ++ob) o[i][ob] += srcp[(i * NO + ob) * 64 + lane];
        }
      }
    }
    if (ph == 0) {
#pragma unroll
      for (int i = 0; i < kGpw; ++i) {
        const int row = 16 * (gi0 + i) + l16;          // row inside the q-block
        if (i < ng_w && q0 + row < n) {
          float* dst = a.part + (static_cast<size_t>(it) * kQB + row) * HD + 4 * g;
#pragma unroll
          for (int ob = 0; ob < NO; ++ob) *reinterpret_cast<f32x4*>(dst + ob * 16) = o[i][ob];
        }
      }
    }
    __syncthreads();                       // the ring and s_pages are free for the next item
    it = it_next;
    item = item_next;
  }
}
template <typename T, int HD>
hipError_t attn_t(const hstu_layer_desc& d, const int32_t* pt, const void* k_pool, const void* v_pool,
                  const float* pos_bias, const float* ts_bias, const int64_t* ts, const int32_t* ts_off,
                  const int32_t* ncand, const WsPtrs& ws, int grid, hipStream_t stream,
                  const KernelEvents& ev) {
  AttnArgs<T> a;
  a.pt = pt;
  a.k_pool = static_cast<const T*>(k_pool);
  a.v_pool = static_cast<const T*>(v_pool);
  a.q = static_cast<const T*>(ws.q);
  a.pos_bias = pos_bias;
  a.ts_bias = ts_bias;
  a.ts = ts;
  a.ts_off = ts_off;
  a.ncand = ncand;
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
  if (ncand != nullptr) return launch_kernel(attn_kernel<T, HD, true>, dim3(grid), dim3(64 * kWaves), stream, ev, a);
  return launch_kernel(attn_kernel<T, HD, false>, dim3(grid), dim3(64 * kWaves), stream, ev, a);
}

template <typename T>
hipError_t attn_dt(const hstu_layer_desc& d, const int32_t* pt, const void* k_pool, const void* v_pool,
                   const float* pos_bias, const float* ts_bias, const int64_t* ts, const int32_t* ts_off,
                   const int32_t* nc, const WsPtrs& ws, int grid, hipStream_t stream, const KernelEvents& ev) {
  switch (d.head_dim) {
    case 32: return attn_t<T, 32>(d, pt, k_pool, v_pool, pos_bias, ts_bias, ts, ts_off, nc, ws, grid, stream, ev);
    case 64: return attn_t<T, 64>(d, pt, k_pool, v_pool, pos_bias, ts_bias, ts, ts_off, nc, ws, grid, stream, ev);
    default: return attn_t<T, 128>(d, pt, k_pool, v_pool, pos_bias, ts_bias, ts, ts_off, nc, ws, grid, stream, ev);
  }
}

}  // namespace

hipError_t launch_attn(const hstu_layer_desc& d, const int32_t* pt, const void* k_pool, const void* v_pool,
                       const float* pos_bias, const float* ts_bias, const int64_t* ts,
                       const int32_t* ts_off, const int32_t* ncand, const WsPtrs& ws, int grid,
                       hipStream_t stream, const KernelEvents& ev) {
  if (d.dtype == HSTU_BF16)
    return attn_dt<bf16>(d, pt, k_pool, v_pool, pos_bias, ts_bias, ts, ts_off, ncand, ws, grid, stream, ev);
  return attn_dt<float>(d, pt, k_pool, v_pool, pos_bias, ts_bias, ts, ts_off, ncand, ws, grid, stream, ev);
}

}  // namespace hstu
