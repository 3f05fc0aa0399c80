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
// pair per wave; when the block has at most eight groups the waves also split
// the key steps: they form P = 2 phases and the waves of phase p multiply the
// steps s = p (mod 2).  The chunk's keys are walked in 32-key steps.  A step's
// K rows [32][d] and V^T rows [d][32] are copied from their pool pages into a
// ring of NST LDS stages with direct-to-LDS loads that the waves share out;
// one barrier per round (two steps per wave with one phase, one step per
// wave with two) hands the round's stages from the loads to the products, and
// the loads of a round two rounds behind the ring's end go into stages freed
// two rounds earlier.  The two waves of a SIMD run their steps half a step
// apart (see the key loop).  At the end of an item the phases' partial sums
// meet in LDS.
// Per step and wave:
//   S^T[32 keys x 16 queries] = K * Q^T     (2 MFMA blocks over d; the
//                                           accumulators start at the bias,
//                                           or at a masked value, below)
//   A = SiLU(S) on the fp32 scores          (no branches)
//   O^T[d x 16]             += V^T * A
// A wave with two groups runs one group's products on the matrix cores while
// the other group's SiLU runs on the vector ALUs.
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
// Bias: the layer's tables (built once per call by prep, see kTabFloats) are
// copied into LDS by direct-to-LDS loads at the workgroup's start.  The
// distance table holds the scaled bias of every distance below kLut, in
// descending order of distance: the 8 scores a lane holds per group and step
// have 8 consecutive distances, so they read 8 consecutive entries at
// immediate offsets from one address.  A step whose distances all lie at or
// beyond kLut and span no more than one bucket width (2^(12-m) there)
// touches at most two buckets and takes a compare/select between two values;
// any other step takes the generic per-element bucket path.  Timestamps
// (an instance of the kernel of their own), when present, travel with their
// keys through the ring; each lane keeps its query's in a register.
//
// Masks: a masked (query, key) pair starts its accumulator at kMasked, whose
// SiLU is exactly 0 (see kMasked).  Negative distances (the causal mask) read
// masked entries from the bias table's padding, so only steps that reach the
// candidates set masks of their own.  Candidates: when the call gives
// per-user candidate counts m_u, a query at or past the first candidate
// position cs = c + n - m_u sees only the keys before cs and itself (a key at
// or past cs is kept only on the diagonal).  Rows before cs see nothing past
// cs anyway, so one mask covers every row.
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

constexpr int kStepKeys = 32;
constexpr int kMaxChunkPages = kMaxChunkKeys / 16 + 1;

template <typename T>
struct AttnArgs {
  const int32_t* pt;
  const T* k_pool;
  const T* v_pool;
  const T* q;
  const float* tab;          // this layer's bias tables (layout at kTabFloats)
  const int64_t* ts;
  const int32_t* ts_off;
  const int32_t* ncand;      // per-user candidate counts, or null
  WsHeader* hdr;
  const AttnItem* items;
  float* part;
  int H, D, ps_shift, maxP, nb, mbits, ntsb, tsmbits;
  int pmax;                  // 1: one phase per item (batch-invariant calls), else 2
};

// First distance of bucket b (b >= 2^m) under the log-linear rule.
__device__ __forceinline__ int bucket_start(int b, int m) {
  const int s = 1 << m;
  if (b < s) return b;
  const int q = b >> m, r = b & (s - 1);
  return (s + r) << (q - 1);
}

// Wave layouts of a workgroup (a q-block is 256 rows either way):
//   8 waves of an adjacent pair of 16-query groups each: two waves per SIMD,
//     each K/V^T fragment read feeds two groups;
//   16 waves of one group each (bf16 only, <= 128 registers): four waves per
//     SIMD hide each other's LDS, matrix and transcendental latencies, at
//     twice the fragment reads per group.
// The host picks per call (launch_attn below).

// Sizes of one ring stage (one 32-key step of K and V^T) for element type T
// and head dim HD, and of the ring; WAVES is the layout.
template <typename T, int HD, int WAVES>
struct StepGeo {
  static constexpr int kWaves = WAVES;
  static constexpr int kGpw = kQB / (16 * WAVES);
  static_assert(kQB == 16 * kWaves * kGpw && (kGpw == 1 || kGpw == 2), "a q-block is 256 rows");
  static constexpr int ES = static_cast<int>(sizeof(T));
  static constexpr int CE = 16 / ES;                   // elements per 16-byte chunk
  static constexpr int KCH = HD / CE;                  // chunks per K row
  static constexpr int VCH = kStepKeys / CE;           // chunks per V^T row
  static constexpr int KBYTES = kStepKeys * HD * ES;   // the K rows of a step
  static constexpr int STAGE = 2 * KBYTES;             // K rows, then V^T rows
  static constexpr int NBLK = STAGE / 1024;            // 1 KiB loads per stage
  // waves that issue a stage's loads (the first kIssuers; the others only
  // compute) and the loads each issues per stage (at most)
  static constexpr int kIssuers = WAVES;
  static constexpr int IPW = (NBLK + kIssuers - 1) / kIssuers;
  // ring: 8 stages, or as many as fit in 128 KiB (a power of two)
  static constexpr int NST_FIT = 131072 / STAGE;
  static constexpr int NST = NST_FIT >= 8 ? 8 : (NST_FIT >= 4 ? 4 : 2);
  // phases: the ring holds at least three rounds of PMAX steps (see the
  // key loop)
  static constexpr int PMAX = NST >= 6 ? 2 : 1;
  // chunk permutation of K row `key`: (m >> KSH) with m = (key & 3) | (((key >> 3) & 3) << 2),
  // m being the lane (mod 16) that reads the row; V^T row e: (e >> VSH) & (VCH - 1)
  static constexpr int KSH = KCH >= 16 ? 0 : (KCH == 8 ? 1 : 2);
  static constexpr int VSH = VCH == 4 ? 2 : 1;
  static_assert(KCH >= 4 && (VCH == 4 || VCH == 8), "supported geometry");
  static_assert(NBLK * 1024 == STAGE, "whole loads per stage");
  static_assert((kStepKeys * KCH) % 64 == 0, "a load never straddles K and V^T");
  static_assert((IPW + 1) * (NST - 2) <= 63, "wait count range");
  // the phase reduction reuses the ring: at most (PMAX-1) * (kWaves/PMAX)
  // waves hand over two 16 x HD fp32 tiles each
  static_assert(NST * STAGE >= (PMAX - 1) * (kWaves / PMAX) * kGpw * 16 * HD * 4, "reduction fits the ring");
};

template <typename T, int HD, bool CAND, bool TS, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void attn_kernel(AttnArgs<T> a) {
  using G = StepGeo<T, HD, WAVES>;
  constexpr int CE = G::CE, KCH = G::KCH, VCH = G::VCH, NST = G::NST, IPW = G::IPW;
  constexpr int kWaves = G::kWaves, kGpw = G::kGpw;
  // the two waves of a SIMD run half a step apart in the 8-wave layout (see
  // the key loop); with four waves per SIMD every wave runs the plain order
  constexpr bool kRot = kWaves == 8;
  constexpr int NT = 64 * kWaves;
  constexpr int NC = HD / 32;        // 32-wide slices of the head dim (contraction of S^T)
  constexpr int NO = HD / 16;        // 16-row blocks of O^T
  constexpr int kPidPerThread = (kMaxChunkPages + NT - 1) / NT;   // page ids a thread stages
  __shared__ __attribute__((aligned(1024))) unsigned char s_ring[NST * G::STAGE];
  __shared__ __attribute__((aligned(256))) int64_t s_ts[NST][kStepKeys];
  // bias tables (layout at kTabFloats): s_rlut[x] is the bias of distance
  // kLut - 1 - x, s_pb / s_tb the position / timestamp buckets
  __shared__ __attribute__((aligned(1024))) float s_tab[kTabFloats];
  const float* s_rlut = s_tab;
  const float* s_pb = s_tab + kTabPb;
  const float* s_tb = s_tab + kTabTb;
  __shared__ int s_pages[kMaxChunkPages];
  __shared__ int s_next;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  // Status words and item count, the first item (static: workgroup i takes
  // item i; the grid never exceeds the item capacity) and the layer's bias
  // tables (direct-to-LDS, 1 KiB per wave instruction) all go out at once;
  // the tables have landed by the first item's wait for its page ids.
  const int4 hv = *reinterpret_cast<const int4*>(a.hdr);
  AttnItem item = a.items[blockIdx.x];
  static_assert(kTabFloats % 256 == 0, "whole KiB of tables");
  for (int j = w; j < kTabFloats / 256; j += kWaves)
    dma_lds16(a.tab + j * 256 + lane * 4, s_tab + j * 256);
  if ((hv.x | hv.y) != 0) {                // status words: prep rejected the call
    wait_vm<0>();                          // (the table loads land before the workgroup ends)
    return;
  }
  const int n_items = hv.z;
  const bool dynamic = n_items > static_cast<int>(gridDim.x);
  const int ps = 1 << a.ps_shift;
  constexpr bool has_ts = TS;             // the timestamp term (an instance of its own)
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
    const int NW = (ngroups + kGpw - 1) / kGpw;        // wave columns with groups
    // (Batch-invariant calls keep one phase: a row's steps are then added in
    // key order whatever its q-block holds.)
    const int P = (G::PMAX >= 2 && a.pmax >= 2 && 2 * NW <= kWaves) ? 2 : 1;
    // A round is RS = P * M steps, M of them per wave (two when every wave
    // multiplies every step, which halves the barriers), and the ring holds
    // R of them (at least three).
    const int M = P == 1 && NST >= 8 ? 2 : 1;
    const int RS = P * M;
    const int R = NST / RS;
    [[maybe_unused]] const int half = kWaves / (2 * P);
    const int ph = w & (P - 1), col = w / P;
    int gi0, ng_w;                                     // this wave's first group and group count
    if constexpr (kGpw == 1) {
      // one group per column; column j's waves sit on SIMD j mod 4 (with two
      // phases, the phases of a column on neighbouring SIMDs)
      gi0 = col;
      ng_w = col < ngroups ? 1 : 0;
    } else if (col < half) {
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
    // (clamped indices: no per-lane branch, see the bias tables)
    int pid[kPidPerThread];
#pragma unroll
    for (int k = 0; k < kPidPerThread; ++k) pid[k] = ptu[pg0 + min(tid + k * NT, npg - 1)];
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
    const int nrounds = (nsteps + RS - 1) / RS;
    // Let these loads land before the ring starts: the compiler cannot count
    // outstanding loads across the key loop, so it would otherwise wait for
    // every in-flight stage at the first use of a query fragment.
    wait_vm<0>();
#pragma unroll
    for (int k = 0; k < kPidPerThread; ++k)
      if (tid + k * NT < npg) s_pages[tid + k * NT] = pid[k];
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
    // own pages: in bounds; their K rows and V^T columns are zeroed in LDS
    // before the products and their scores masked.
    auto issue = [&](int s) __attribute__((always_inline)) {
      if (my_cnt == 0) return;                         // uniform: a wave that only computes
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

    // ---- the pieces of a step's products (this wave's groups) ----
    // Accumulator start of group i at step s: the bias of every (query, key)
    // pair, or kMasked for masked pairs.
    auto bias_init = [&](int i, int s, f32x4 (&sv)[2]) __attribute__((always_inline)) {
      const int kb = k_lo + kStepKeys * s;
      // distance of element (block b, row r) is dl0 - 4*b - r
      const int pq = c + q0 + 16 * (gi0 + i);          // first query position of the group
      const int dl0 = pq + l16 - (kb + 8 * g);
      const int dmin = pq - (kb + kStepKeys - 1);
      const int dmax = pq + 15 - kb;
      if (dmax < kLut) {
        // element (b, r) has distance dl0 - (4b + r), entry x0 + 4b + r; a
        // lane whose distances are all negative reads padding (masked)
        const float* lp = s_rlut + min(kLut - 1 - dl0, kLut + kLutPad - 8);
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) sv[b][r] = lp[4 * b + r];
      } else if (dmin >= kLut && (kLut >> a.mbits) >= dmax - dmin + 1) {
        // every distance here falls into one or two adjacent buckets
        const int blo = bucket32(dmin, a.mbits, a.nb), bhi = bucket32(dmax, a.mbits, a.nb);
        const float vlo = s_pb[blo], vhi = s_pb[bhi];
        if (blo == bhi) {                            // uniform: the whole step in one bucket
#pragma unroll
          for (int b = 0; b < 2; ++b) sv[b] = f32x4{vlo, vlo, vlo, vlo};
        } else {
          const int bnd = bucket_start(bhi, a.mbits);
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) sv[b][r] = (dl0 - 4 * b - r) >= bnd ? vhi : vlo;
        }
      } else {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) sv[b][r] = s_pb[bucket32(dl0 - 4 * b - r, a.mbits, a.nb)];
      }
      if (has_ts) {
        const int64_t* tk = &s_ts[s % NST][8 * g];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) sv[b][r] += s_tb[bucket64_fast(tq[i] - tk[4 * b + r], a.tsmbits, a.ntsb)];
      }
      // The causal mask is in the bias already (negative distances read the
      // table's masked padding).  Keys at or past the candidates: element e
      // (key kb + 8g + e) stays only if it is before cs or on the diagonal.
      if (CAND && kb + kStepKeys > cs) {
        const int ce = cs - (kb + 8 * g);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int de = dl0 - e;
          if (!(de >= 0 && (e < ce || de == 0))) sv[e >> 2][e & 3] = kMasked;
        }
      }
    };
    // K fragments of step s (rows read in the permuted order, see the top)
    auto read_k = [&](int s, Frag<T> (&kf)[NC][2]) __attribute__((always_inline)) {
      const unsigned char* k0p = s_ring + (s % NST) * G::STAGE + krow0 * (KCH * 16);
      const unsigned char* k1p = k0p + 4 * (KCH * 16);
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const int chunk = (cc * 32 + 8 * g) / CE;
        read_frag(kf[cc][0], k0p, chunk, ksw);
        read_frag(kf[cc][1], k1p, chunk, ksw);
      }
    };
    auto read_v = [&](int s, Frag<T> (&vf)[NO]) __attribute__((always_inline)) {
      const unsigned char* vp = s_ring + (s % NST) * G::STAGE + G::KBYTES + l16 * (VCH * 16);
      const int vchunk = (8 * g) / CE;
#pragma unroll
      for (int ob = 0; ob < NO; ++ob) read_frag(vf[ob], vp + ob * 16 * (VCH * 16), vchunk, vsw);
    };
    // S^T of group i += K * Q^T over the head dim
    auto s_mma = [&](int i, const Frag<T> (&kf)[NC][2], f32x4 (&sv)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        sv[0] = mma16(kf[cc][0], qf[i][cc], sv[0]);
        sv[1] = mma16(kf[cc][1], qf[i][cc], sv[1]);
      }
    };
    // A = SiLU(S) in the exponent domain, no branches: every exp2, then
    // every reciprocal, so no transcendental waits on the one before it
    auto silu_frag = [&](const f32x4 (&sv)[2], Frag<T>& af) __attribute__((always_inline)) {
      float av[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) av[e] = __builtin_amdgcn_exp2f(sv[e >> 2][e & 3]);
#pragma unroll
      for (int e = 0; e < 8; ++e) av[e] = __builtin_amdgcn_rcpf(1.0f + av[e]);
#pragma unroll
      for (int e = 0; e < 8; ++e) av[e] *= sv[e >> 2][e & 3];
      set_frag(af, av);
    };
    // O^T of group i += V^T * A
    auto o_mma = [&](int i, const Frag<T> (&vf)[NO], const Frag<T>& af) __attribute__((always_inline)) {
#pragma unroll
      for (int ob = 0; ob < NO; ++ob) o[i][ob] = mma16(vf[ob], af, o[i][ob]);
    };

    // Only the last step can reach past the staged keys.  Those keys lie
    // beyond every query of the item, so their scores are masked; their K
    // rows and V^T columns are zeroed in LDS (by the lanes that loaded them,
    // once their loads have landed) so that stale pool memory cannot turn a
    // masked score or product into NaN, and the products need no tail case
    // of their own.
    const int tail_round = k_lo + kStepKeys * nsteps > kst_end ? (nsteps - 1) / RS : -1;
    auto zero_tail = [&]() __attribute__((always_inline)) {
      const int kb = k_lo + kStepKeys * (nsteps - 1);
      const int nvalid = kst_end - kb;                 // staged keys of the step
      unsigned char* stg = s_ring + ((nsteps - 1) % NST) * G::STAGE;
#pragma unroll
      for (int j = 0; j < IPW; ++j) {
        const int blk = w * IPW + j;
        if (blk >= G::NBLK) break;                     // uniform
        if (blk * 64 < kStepKeys * KCH) {              // K rows: the lane's chunk of key q / KCH
          if ((blk * 64 + lane) / KCH >= nvalid)
            *reinterpret_cast<u32x4*>(stg + blk * 1024 + lane * 16) = u32x4{0u, 0u, 0u, 0u};
          continue;
        }
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
    // loads of the steps of round rr (each wave its share of every stage)
    auto issue_round = [&](int rr) __attribute__((always_inline)) {
      for (int s2 = rr * RS; s2 < min((rr + 1) * RS, nsteps); ++s2) issue(s2);
    };

    // ---- products of step s for this wave's first NG query groups ----
    auto compute = [&](auto ngc, int s) __attribute__((always_inline)) {
      constexpr int NG = decltype(ngc)::value;
      f32x4 st[NG][2];
#pragma unroll
      for (int i = 0; i < NG; ++i) bias_init(i, s, st[i]);
      Frag<T> kf[NC][2];
      read_k(s, kf);
      Frag<T> vf[NO];
      Frag<T> af[NG];
      if constexpr (NG == 2 && sizeof(T) == 2) {
        // Two groups: one group's products run on the matrix cores while the
        // other group's SiLU runs on the vector ALUs (the scheduler is told
        // to alternate one product with a few vector instructions).
        s_mma(0, kf, st[0]);
        read_v(s, vf);
        s_mma(1, kf, st[1]);
        silu_frag(st[0], af[0]);
#pragma unroll
        for (int k = 0; k < 2 * NC; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        }
        o_mma(0, vf, af[0]);
        silu_frag(st[1], af[1]);
#pragma unroll
        for (int k = 0; k < NO; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
          __builtin_amdgcn_sched_group_barrier(0x002, 5, 1);
        }
        o_mma(1, vf, af[1]);
      } else {
#pragma unroll
        for (int i = 0; i < NG; ++i) s_mma(i, kf, st[i]);
        // V^T fragments are read now so that their LDS latency overlaps the
        // SiLU below.
        read_v(s, vf);
#pragma unroll
        for (int i = 0; i < NG; ++i) silu_frag(st[i], af[i]);
#pragma unroll
        for (int i = 0; i < NG; ++i) o_mma(i, vf, af[i]);
      }
    };

    // ---- the key loop: one barrier per round of RS steps; at barrier k the
    // steps of round k (stages kRS .. kRS+RS-1 mod NST) are visible.  The two
    // waves of a SIMD take turns on its matrix core and vector ALUs: waves
    // 0-3 multiply a step in the plain order (bias, S^T, SiLU, O^T), waves
    // 4-7 half a step later (SiLU and O^T of their step after barrier k+1,
    // then the bias and S^T of their next step), so while one wave's
    // products run the other's SiLU does.  A rotated wave still reads round
    // k-1 after barrier k, so the loads issued at barrier k (round k+R-2)
    // go into round k-2's stages: R-2 rounds are in flight ahead. ----
    auto key_loop = [&](auto ngc) __attribute__((always_inline)) {
      // Without rotated waves every wave is done with round r-1 at barrier r,
      // so the loads of round r+R-1 can go into its stages: R-1 rounds ahead.
      const int D = kRot ? R - 2 : R - 1;
      for (int rr = 0; rr < min(D, nrounds); ++rr) issue_round(rr);
      for (int r = 0; r < nrounds; ++r) {
        // round r's loads have landed once only those issued after them remain
        const int later = min((r + D) * RS, nsteps) - (r + 1) * RS;
        if (later > 0) wait_vm_n(later * my_cnt);
        else wait_vm<0>();
        if (r == tail_round) zero_tail();
        bar();                             // round r visible; round r-2 no longer read
        if constexpr (decltype(ngc)::value > 0) {
          for (int j = 0; j < M; ++j) {
            const int s = r * RS + j * P + ph;
            if (s < nsteps) compute(ngc, s);
          }
        }
        issue_round(r + D);
      }
    };
    auto key_loop_rot = [&](auto ngc) __attribute__((always_inline)) {
      constexpr int NG = decltype(ngc)::value;
      const int DP = R - 1;                // one round further: this wave's issue follows a later barrier
      for (int rr = 0; rr < min(DP, nrounds); ++rr) issue_round(rr);
      f32x4 st[NG > 0 ? NG : 1][2];
      {                                    // barrier 0: round 0 visible; S^T of the first step
        const int later = min(DP * RS, nsteps) - RS;
        if (later > 0) wait_vm_n(later * my_cnt);
        else wait_vm<0>();
        if (tail_round == 0) zero_tail();
        bar();
        if constexpr (NG > 0) {
          const int s = min(ph, nsteps - 1);
#pragma unroll
          for (int i = 0; i < NG; ++i) bias_init(i, s, st[i]);
          Frag<T> kf[NC][2];
          read_k(s, kf);
#pragma unroll
          for (int i = 0; i < NG; ++i) s_mma(i, kf, st[i]);
        }
      }
      for (int r = 0; r < nrounds; ++r) {
        if (r + 1 < nrounds) {
          // barrier r+1: round r+1's loads have landed once only those issued after them remain
          const int later = min((r + DP) * RS, nsteps) - (r + 2) * RS;
          if (later > 0) wait_vm_n(later * my_cnt);
          else wait_vm<0>();
          if (r + 1 == tail_round) zero_tail();
          bar();
        }
        issue_round(r + DP);
        if constexpr (NG > 0) {
          for (int j = 0; j < M; ++j) {
          const int s = r * RS + j * P + ph;
          if (s < nsteps) {
            // this step's SiLU and O^T, then the next step's bias and S^T
            // (formed on this step's stage when there is none, so that the
            // products have no branches of their own)
            const int s1 = s + P < nsteps ? s + P : s;
            Frag<T> vf[NO];
            read_v(s, vf);
            Frag<T> kf[NC][2];
            read_k(s1, kf);
            Frag<T> af[NG];
#pragma unroll
            for (int i = 0; i < NG; ++i) silu_frag(st[i], af[i]);
#pragma unroll
            for (int i = 0; i < NG; ++i) o_mma(i, vf, af[i]);
#pragma unroll
            for (int i = 0; i < NG; ++i) bias_init(i, s1, st[i]);
#pragma unroll
            for (int i = 0; i < NG; ++i) s_mma(i, kf, st[i]);
          }
          }
        }
      }
    };
    if (!kRot || w < 4) {
      if constexpr (kGpw == 2) {
        if (ng_w == 2) key_loop(std::integral_constant<int, 2>{});
        else if (ng_w == 1) key_loop(std::integral_constant<int, 1>{});
        else key_loop(std::integral_constant<int, 0>{});
      } else {
        if (ng_w == 1) key_loop(std::integral_constant<int, 1>{});
        else key_loop(std::integral_constant<int, 0>{});
      }
    } else if constexpr (kRot) {
      if (ng_w == 2) key_loop_rot(std::integral_constant<int, 2>{});
      else if (ng_w == 1) key_loop_rot(std::integral_constant<int, 1>{});
      else key_loop_rot(std::integral_constant<int, 0>{});
    }

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
  wait_vm<0>();                            // a workgroup without items: its table loads land first
}
template <typename T, int HD>
hipError_t attn_t(const hstu_layer_desc& d, const int32_t* pt, const void* k_pool, const void* v_pool,
                  int layer, const int64_t* ts, const int32_t* ts_off,
                  const int32_t* ncand, const WsPtrs& ws, int grid, hipStream_t stream,
                  const KernelEvents& ev) {
  AttnArgs<T> a;
  a.pt = pt;
  a.k_pool = static_cast<const T*>(k_pool);
  a.v_pool = static_cast<const T*>(v_pool);
  a.q = static_cast<const T*>(ws.q);
  a.tab = ws.tables + static_cast<size_t>(layer) * kTabFloats;
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
  a.pmax = (d.flags & HSTU_FLAG_BATCH_INVARIANT) ? 1 : 2;
  const dim3 gr(grid);
  auto go = [&](auto wc) {
    constexpr int W = decltype(wc)::value;
    const dim3 bl(64 * W);
    if (d.ts_buckets > 0)
      return ncand != nullptr ? launch_kernel(attn_kernel<T, HD, true, true, W>, gr, bl, stream, ev, a)
                              : launch_kernel(attn_kernel<T, HD, false, true, W>, gr, bl, stream, ev, a);
    return ncand != nullptr ? launch_kernel(attn_kernel<T, HD, true, false, W>, gr, bl, stream, ev, a)
                            : launch_kernel(attn_kernel<T, HD, false, false, W>, gr, bl, stream, ev, a);
  };
  // 16 waves of one group where each q-block has few groups to share a
  // fragment read (short bursts of new rows: at most 96 per user on
  // average) or the timestamp term adds vector work per score; 8 waves of
  // pairs otherwise.  (fp32 fragments are twice as wide: 8 waves only.)
  if constexpr (sizeof(T) == 2) {
    const int64_t rows = d.total_new, users = d.num_users > 0 ? d.num_users : 1;
    if (d.ts_buckets > 0 || rows <= 96 * users) return go(std::integral_constant<int, 16>{});
  }
  return go(std::integral_constant<int, 8>{});
}

template <typename T>
hipError_t attn_dt(const hstu_layer_desc& d, const int32_t* pt, const void* k_pool, const void* v_pool,
                   int layer, const int64_t* ts, const int32_t* ts_off,
                   const int32_t* nc, const WsPtrs& ws, int grid, hipStream_t stream, const KernelEvents& ev) {
  switch (d.head_dim) {
    case 32: return attn_t<T, 32>(d, pt, k_pool, v_pool, layer, ts, ts_off, nc, ws, grid, stream, ev);
    case 64: return attn_t<T, 64>(d, pt, k_pool, v_pool, layer, ts, ts_off, nc, ws, grid, stream, ev);
    default: return attn_t<T, 128>(d, pt, k_pool, v_pool, layer, ts, ts_off, nc, ws, grid, stream, ev);
  }
}

}  // namespace

hipError_t launch_attn(const hstu_layer_desc& d, const int32_t* pt, const void* k_pool, const void* v_pool,
                       int layer, const int64_t* ts, const int32_t* ts_off, const int32_t* ncand,
                       const WsPtrs& ws, int grid, hipStream_t stream, const KernelEvents& ev) {
  if (d.dtype == HSTU_BF16)
    return attn_dt<bf16>(d, pt, k_pool, v_pool, layer, ts, ts_off, ncand, ws, grid, stream, ev);
  return attn_dt<float>(d, pt, k_pool, v_pool, layer, ts, ts_off, ncand, ws, grid, stream, ev);
}

}  // namespace hstu
