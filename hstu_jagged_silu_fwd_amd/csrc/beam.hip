// Beam-decode attention over a shared request-level context KV (Semantic-ID
// generative recommendation: one ContextKV per request shared by every
// beam, a short per-beam BeamKV and beam paths; Korean summary of the
// recsys-examples article, GR inference path; news.bpdata.com Hungarian
// article, section "SID-GR inference").  The operation is stated in
// include/hstu_beam.h.
//
// The context part is a dense contraction: every beam and every query head
// of a KV-head group reads the same context keys, so for one (request, KV
// head) the W * G query rows form a matrix and the context keys another.
// Kernel 1 takes one (request, KV head, 256-row query tile, context chunk)
// per workgroup of eight waves; each wave owns two 16-row query groups.  The
// chunk's keys are walked in 64-key steps, double-buffered through LDS (the
// next step's loads are in registers while the current step is multiplied),
// each step multiplied as two 32-key halves:
//   S^T [32 keys x 16 queries] = K * Q^T      (MFMA, 2 blocks over d, per half)
//   online softmax in base 2 over the step's 64 keys (a lane holds 8
//   consecutive keys of one query per half; the row maximum is reduced over
//   the four lanes that share the query, once per step; O and the sum are
//   rescaled only when a row's maximum grows by more than a set margin)
//   O^T [d x 16] = alpha * O^T + V^T * P       (MFMA)
// K rows feeding S^T block b are read in the order row m -> key 8*(m/4) +
// 4*b + m%4, so a lane's score accumulators are exactly the keys of its
// B-operand fragment for the value product (the scores stay in registers).
// K rows keep their 16-byte chunks XOR-permuted by row (kmix) and V^T rows are
// padded by 16 bytes, so the 16 lanes of a fragment read hit distinct banks.  The chunk's unnormalised O, its running maximum
// and its sum go to the workspace (fp32).
//
// Kernel 2 gives one wave to each output row (request, beam, query head): it
// merges the chunks' partial results with the beam's own keys -- its path
// tokens of earlier steps and its token of this step, at most a few, which
// differ from beam to beam -- by the usual log-sum-exp rescaling, and writes
// the normalised row.
#include "common.h"
#include "hstu_beam.h"

namespace hstu {
namespace {

constexpr int kBWaves = 8;
constexpr int kBThreads = 64 * kBWaves;
constexpr int kTileRows = 32 * kBWaves;      // two 16-row groups per wave
constexpr int kBStep = 64;                   // keys per step (two 32-key halves)
constexpr int kCtxAlign = 32;                // max_ctx granularity: every 16-byte V^T load stays in the row
constexpr int kCombineRows = 4;              // output rows (waves) per combine workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;                 // reference-maximum slack, log2 units (weights stay below 256)

struct BeamArgs {
  const void* q;
  const void* ctx_k;
  const void* ctx_vt;
  const int32_t* ctx_len;
  const void* beam_k;
  const void* beam_v;
  const int32_t* path;
  void* out;
  int32_t* status;
  float* part;       // [items][kTileRows][d]
  float* mstat;      // [items][kTileRows]
  float* lstat;      // [items][kTileRows]
  int R, W, Hq, Hkv, G, Cmax, t, S, NR, nqt, nch, csz;
  float scale2;      // softmax scale * log2(e)
};

template <typename T, int HD>
struct BGeo {
  static constexpr int ES = static_cast<int>(sizeof(T));
  static constexpr int CE = 16 / ES;                  // elements per 16-byte chunk
  static constexpr int KCH = HD * ES / 16;            // chunks per K row
  static constexpr int KROW = HD * ES;                // K row (bytes), chunks XOR-permuted (kswz)
  static constexpr int KSH = KCH >= 16 ? 0 : 1;       // 1: 8-chunk rows
  static constexpr int VROW = kBStep * ES + 16;       // padded V^T row (bytes)
  static constexpr int KBYTES = kBStep * KROW;
  static constexpr int STAGE = KBYTES + HD * VROW;
  static constexpr int VCH = kBStep * ES / 16;        // chunks per V^T row
  static constexpr int NCHK = kBStep * KCH;
  static constexpr int NCH = NCHK + HD * VCH;
  static constexpr int CPT = NCH / kBThreads;         // chunks per thread and step
  static_assert(CPT >= 1 && CPT * kBThreads == NCH, "whole chunks per thread");
  static_assert(NCHK % kWave == 0, "a wave's chunk of a step is all K or all V^T");
};

// Chunk permutation of K rows in LDS: chunk p of row `row` is stored at
// p ^ kswz(kmix(row)).  The 16 lanes of a fragment read take rows
// 8*(l/4) + l%4 (+4, +32), whose kmix is exactly l.  Rows of 16 or more
// chunks XOR with l itself; 8-chunk rows (two to a 256-byte line) with
// (l & 7) ^ (l >> 3), which keeps the 16 lanes' reads on distinct banks both
// when 8 lanes share a 128-byte pass and when 16 share a 256-byte one.
__device__ __forceinline__ int kmix(int row) { return (row & 3) | (((row >> 3) & 3) << 2); }
template <int KSH>
__device__ __forceinline__ int kswz(int m) { return KSH == 0 ? m : ((m & 7) ^ (m >> 3)); }

// Zeroes the elements at index >= nv of a 16-byte chunk.
template <typename T>
__device__ __forceinline__ uint4 keep_first(uint4 v, int nv) {
  if constexpr (sizeof(T) == 2) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = 2 * i < nv ? (w[i] & 0xffffu) : 0u;
      const uint32_t hi = 2 * i + 1 < nv ? (w[i] & 0xffff0000u) : 0u;
      w[i] = lo | hi;
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    return make_uint4(nv > 0 ? v.x : 0u, nv > 1 ? v.y : 0u, nv > 2 ? v.z : 0u, nv > 3 ? v.w : 0u);
  }
}

__device__ void validate(const BeamArgs& a) {
  __shared__ int s_bad_len, s_bad_path;
  if (threadIdx.x == 0) {
    s_bad_len = 0;
    s_bad_path = 0;
  }
  __syncthreads();
  for (int r = threadIdx.x; r < a.R; r += kBThreads)
    if (a.ctx_len[r] < 0 || a.ctx_len[r] > a.Cmax) atomicOr(&s_bad_len, 1);
  const int64_t np = static_cast<int64_t>(a.R) * a.W * a.t;
  for (int64_t i = threadIdx.x; i < np; i += kBThreads)
    if (a.path[i] < 0 || a.path[i] >= a.W) atomicOr(&s_bad_path, 1);
  __syncthreads();
  if (threadIdx.x == 0)
    *a.status = s_bad_len ? HSTU_DEV_BAD_CTX_LEN : (s_bad_path ? HSTU_DEV_BAD_PATH : HSTU_DEV_OK);
}

template <typename T, int HD>
__global__ __launch_bounds__(kBThreads) void beam_ctx_kernel(BeamArgs a) {
  using G = BGeo<T, HD>;
  constexpr int NC = HD / 32;          // 32-wide slices of d (contraction of S^T)
  constexpr int NO = HD / 16;          // 16-row blocks of O^T
  __shared__ __attribute__((aligned(16))) unsigned char s_stage[2 * G::STAGE];
  if (blockIdx.x == 0) validate(a);

  const int item = blockIdx.x;
  const int ch = item % a.nch;
  const int qt = (item / a.nch) % a.nqt;
  const int g = (item / (a.nch * a.nqt)) % a.Hkv;
  const int r = item / (a.nch * a.nqt * a.Hkv);
  const int len = min(max(a.ctx_len[r], 0), a.Cmax);  // clamped: a bad length is reported by block 0
  const int k_lo = ch * a.csz;
  if (k_lo >= len) return;                             // an empty chunk: the combine skips it
  const int k_hi = min(len, k_lo + a.csz);
  const int nsteps = (k_hi - k_lo + kBStep - 1) / kBStep;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gq = lane >> 4, l16 = lane & 15;
  const size_t rg = static_cast<size_t>(r) * a.Hkv + g;
  const unsigned char* kbase = static_cast<const unsigned char*>(a.ctx_k) + rg * a.Cmax * HD * G::ES;
  const unsigned char* vbase = static_cast<const unsigned char*>(a.ctx_vt) + rg * HD * a.Cmax * G::ES;

  // this wave's query fragments (rows past the tile's last row repeat it;
  // their results are not written)
  Frag<T> qf[2][NC];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rr = min(qt * kTileRows + 32 * w + 16 * i + l16, a.NR - 1);   // row in the (request, KV head) block
    const int bw = rr / a.G, hq = g * a.G + rr % a.G;
    const T* qp = static_cast<const T*>(a.q) + ((static_cast<size_t>(r) * a.W + bw) * a.Hq + hq) * HD + 8 * gq;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) load_frag(qf[i][cc], qp + cc * 32);
  }

  // ---- a step's K rows and V^T rows, global -> registers -> LDS ----
  uint4 regs[G::CPT];
  auto load_step = [&](int s) __attribute__((always_inline)) {
    const int kb = k_lo + kBStep * s;
#pragma unroll
    for (int j = 0; j < G::CPT; ++j) {
      const int qi = tid + j * kBThreads;
      if (qi < G::NCHK) {
        const int row = qi / G::KCH, c = qi % G::KCH;
        const int key = kb + row;
        regs[j] = key < k_hi ? *reinterpret_cast<const uint4*>(kbase + static_cast<size_t>(key) * HD * G::ES + c * 16)
                             : make_uint4(0, 0, 0, 0);
      } else {
        const int qv = qi - G::NCHK;
        const int e = qv / G::VCH, c = qv % G::VCH;
        const int key0 = kb + c * G::CE;
        const int nv = k_hi - key0;                    // valid keys of the chunk (in bounds: key0 < max_ctx)
        uint4 v = make_uint4(0, 0, 0, 0);
        if (nv > 0) v = *reinterpret_cast<const uint4*>(vbase + (static_cast<size_t>(e) * a.Cmax + key0) * G::ES);
        regs[j] = nv >= G::CE ? v : keep_first<T>(v, nv);
      }
    }
  };
  auto store_step = [&](int buf) __attribute__((always_inline)) {
    unsigned char* st = s_stage + buf * G::STAGE;
#pragma unroll
    for (int j = 0; j < G::CPT; ++j) {
      const int qi = tid + j * kBThreads;
      if (qi < G::NCHK) {
        const int row = qi / G::KCH, c = qi % G::KCH;
        *reinterpret_cast<uint4*>(st + row * G::KROW + ((c ^ kswz<G::KSH>(kmix(row))) << 4)) = regs[j];
      } else {
        const int qv = qi - G::NCHK;
        const int e = qv / G::VCH, c = qv % G::VCH;
        *reinterpret_cast<uint4*>(st + G::KBYTES + e * G::VROW + c * 16) = regs[j];
      }
    }
  };

  f32x4 o[2][NO];
  float m[2], l[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int ob = 0; ob < NO; ++ob) o[i][ob] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int krow0 = 8 * (l16 >> 2) + (l16 & 3);
  const int ksw = kswz<G::KSH>(l16);                   // every K row this lane reads has kmix l16

  load_step(0);
  store_step(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    if (s + 1 < nsteps) load_step(s + 1);            // in flight during the products
    const unsigned char* st = s_stage + (s & 1) * G::STAGE;
    const int kb = k_lo + kBStep * s;
    // S^T = K * Q^T for both 32-key halves of the step
    f32x4 sc[2][2][2];                                 // [group][half][block]
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      Frag<T> kf[NC][2];
      const unsigned char* kp = st + (32 * hf + krow0) * G::KROW;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const int chunk = (cc * 32 + 8 * gq) / G::CE;
        read_frag(kf[cc][0], kp, chunk, ksw);
        read_frag(kf[cc][1], kp + 4 * G::KROW, chunk, ksw);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        sc[i][hf][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        sc[i][hf][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
          sc[i][hf][0] = mma16(kf[cc][0], qf[i][cc], sc[i][hf][0]);
          sc[i][hf][1] = mma16(kf[cc][1], qf[i][cc], sc[i][hf][1]);
        }
      }
    }
    // online softmax over the step's 64 keys (half hf, element e: key
    // kb + 32*hf + 8*gq + e), in base 2 with the scale folded into the
    // exponent's multiply-add.  Each row keeps a reference maximum m that
    // moves only when the step's maximum exceeds it by more than kLazy (so
    // every weight stays below 2^kLazy): most steps then leave O and l
    // unscaled, and the wave rescales only when one of its rows moved.  Only
    // a chunk's last step can hold keys past its end, so only that step masks.
    const bool full = kb + kBStep <= k_hi;             // uniform
    const int nvalid = k_hi - (kb + 8 * gq);
    Frag<T> pf[2][2];
    float alpha[2];
    bool grow = false;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float p[2][8];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int e = 0; e < 8; ++e) p[hf][e] = sc[i][hf][e >> 2][e & 3];
      if (!full) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (32 * hf + e >= nvalid) p[hf][e] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, p[hf][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float mc = mx * a.scale2;                  // finite: every step has a valid key
      const bool gi = mc > m[i] + kLazy;               // always on the first step (m = -inf)
      const float mref = gi ? mc : m[i];
      alpha[i] = __builtin_amdgcn_exp2f(m[i] - mref);  // exactly 1 where the reference stays
      grow |= gi;
      float ps = 0.f;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[hf][e] = __builtin_amdgcn_exp2f(fmaf(p[hf][e], a.scale2, -mref));
          ps += p[hf][e];
        }
      l[i] = fmaf(l[i], alpha[i], ps);
      m[i] = mref;
      set_frag(pf[i][0], p[0]);
      set_frag(pf[i][1], p[1]);
    }
    if (__any(grow)) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int ob = 0; ob < NO; ++ob) o[i][ob] *= alpha[i];
    }
    // O^T += V^T * P, half by half
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      Frag<T> vf[NO];
      const unsigned char* vp = st + G::KBYTES + l16 * G::VROW;
      const int vchunk = (32 * hf + 8 * gq) / G::CE;
#pragma unroll
      for (int ob = 0; ob < NO; ++ob) read_frag(vf[ob], vp + ob * 16 * G::VROW, vchunk, 0);
#pragma unroll
      for (int ob = 0; ob < NO; ++ob)
#pragma unroll
        for (int i = 0; i < 2; ++i) o[i][ob] = mma16(vf[ob], pf[i][hf], o[i][ob]);
    }
    if (s + 1 < nsteps) store_step((s + 1) & 1);     // the buffer step s-1 used: free since the last barrier
    __syncthreads();
  }

  // partial results of the chunk
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    float lt = l[i] + __shfl_xor(l[i], 16, kWave);
    lt += __shfl_xor(lt, 32, kWave);
    const int row = 32 * w + 16 * i + l16;
    if (qt * kTileRows + row < a.NR) {
      const size_t base = static_cast<size_t>(item) * kTileRows + row;
      float* dst = a.part + base * HD + 4 * gq;
#pragma unroll
      for (int ob = 0; ob < NO; ++ob) *reinterpret_cast<f32x4*>(dst + 16 * ob) = o[i][ob];
      if (gq == 0) {
        a.mstat[base] = m[i];
        a.lstat[base] = lt;
      }
    }
  }
}

template <typename T, int HD>
__global__ __launch_bounds__(64 * kCombineRows) void beam_combine_kernel(BeamArgs a) {
  constexpr int EPL = HD / 64;                         // elements of the row per lane
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kCombineRows + (threadIdx.x >> 6);
  if (row >= static_cast<int64_t>(a.R) * a.W * a.Hq) return;
  if (*a.status != 0) return;
  const int h = static_cast<int>(row % a.Hq);
  const int w = static_cast<int>((row / a.Hq) % a.W);
  const int r = static_cast<int>(row / (static_cast<int64_t>(a.Hq) * a.W));
  const int g = h / a.G, rr = w * a.G + h % a.G;
  const int qt = rr / kTileRows, trow = rr % kTileRows;
  const T* q = static_cast<const T*>(a.q) + row * HD + lane * EPL;
  float qv[EPL], acc[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    qv[j] = to_f32(q[j]);
    acc[j] = 0.f;
  }
  float M = -INFINITY, L = 0.f;
  const int len = a.ctx_len[r];
  for (int ch = 0; ch < a.nch && ch * a.csz < len; ++ch) {
    const size_t item = ((static_cast<size_t>(r) * a.Hkv + g) * a.nqt + qt) * a.nch + ch;
    const size_t base = item * kTileRows + trow;
    const float mc = a.mstat[base], lc = a.lstat[base];
    const float mn = fmaxf(M, mc);
    const float a0 = __builtin_amdgcn_exp2f(M - mn), a1 = __builtin_amdgcn_exp2f(mc - mn);
    const float* pp = a.part + base * HD + lane * EPL;
#pragma unroll
    for (int j = 0; j < EPL; ++j) acc[j] = acc[j] * a0 + pp[j] * a1;
    L = L * a0 + lc * a1;
    M = mn;
  }
  // the beam's own keys: its path tokens, then its token of this step
  for (int s = 0; s <= a.t; ++s) {
    const int slot = s < a.t ? a.path[(static_cast<size_t>(r) * a.W + w) * a.t + s] : w;
    const size_t kv = (((static_cast<size_t>(r) * a.S + s) * a.W + slot) * a.Hkv + g) * HD + lane * EPL;
    const T* kp = static_cast<const T*>(a.beam_k) + kv;
    const T* vp = static_cast<const T*>(a.beam_v) + kv;
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) dot += qv[j] * to_f32(kp[j]);
    const float sc = wave_sum(dot) * a.scale2;
    const float mn = fmaxf(M, sc);
    const float a0 = __builtin_amdgcn_exp2f(M - mn), a1 = __builtin_amdgcn_exp2f(sc - mn);
#pragma unroll
    for (int j = 0; j < EPL; ++j) acc[j] = acc[j] * a0 + to_f32(vp[j]) * a1;
    L = L * a0 + a1;
    M = mn;
  }
  T* o = static_cast<T*>(a.out) + row * HD + lane * EPL;
  const float inv = 1.0f / L;
#pragma unroll
  for (int j = 0; j < EPL; ++j) o[j] = from_f32<T>(acc[j] * inv);
}

struct BeamLayout {
  int G, NR, nqt, nch, csz;
  size_t items, part, mstat, lstat, total;
};

size_t align256b(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return cus;
}

// The context is cut into nch chunks of csz keys (a multiple of the step)
// so that the items number about one per compute unit.
BeamLayout beam_layout(const hstu_beam_desc& d) {
  BeamLayout L{};
  L.G = d.num_q_heads / d.num_kv_heads;
  L.NR = d.beam_width * L.G;
  L.nqt = (L.NR + kTileRows - 1) / kTileRows;
  const int64_t tiles = static_cast<int64_t>(d.num_requests) * d.num_kv_heads * L.nqt;
  const int max_chunks = (d.max_ctx + kBStep - 1) / kBStep;
  int64_t want = tiles > 0 ? (device_cus() + tiles - 1) / tiles : 1;
  want = want < 1 ? 1 : (want > max_chunks ? max_chunks : want);
  L.csz = static_cast<int>((d.max_ctx + want - 1) / want + kBStep - 1) / kBStep * kBStep;
  L.nch = (d.max_ctx + L.csz - 1) / L.csz;
  L.items = static_cast<size_t>(tiles) * L.nch;
  const size_t rows = L.items * kTileRows;
  size_t off = 256;
  L.part = off;  off = align256b(off + rows * d.head_dim * 4);
  L.mstat = off; off = align256b(off + rows * 4);
  L.lstat = off; off = align256b(off + rows * 4);
  L.total = off;
  return L;
}

hstu_status check_beam(const hstu_beam_desc* d) {
  if (d == nullptr) return HSTU_ERR_INVALID_ARG;
  if (d->dtype != HSTU_F32 && d->dtype != HSTU_BF16) return HSTU_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return HSTU_ERR_UNSUPPORTED;
  if (d->num_requests < 0 || d->beam_width < 1 || d->beam_width > 1024 || d->num_kv_heads < 1 ||
      d->num_q_heads < d->num_kv_heads || d->num_q_heads % d->num_kv_heads != 0 || d->num_q_heads > 256 ||
      d->max_ctx < kCtxAlign || d->max_ctx % kCtxAlign != 0 || d->max_ctx > (1 << 20) || d->step < 0 ||
      d->max_steps <= d->step || !(d->scale > 0.0f))
    return HSTU_ERR_INVALID_ARG;
  return HSTU_OK;
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <typename T, int HD>
hipError_t launch_beam(const BeamArgs& a, size_t items, hipStream_t st) {
  hipError_t e = launch_kernel(beam_ctx_kernel<T, HD>, dim3(static_cast<unsigned>(items)), dim3(kBThreads), st,
                               KernelEvents{}, a);
  if (e != hipSuccess) return e;
  const int64_t rows = static_cast<int64_t>(a.R) * a.W * a.Hq;
  return launch_kernel(beam_combine_kernel<T, HD>, dim3(static_cast<unsigned>((rows + kCombineRows - 1) / kCombineRows)),
                       dim3(64 * kCombineRows), st, KernelEvents{}, a);
}

}  // namespace
}  // namespace hstu

using namespace hstu;

extern "C" hstu_status hstu_beam_workspace_size(const hstu_beam_desc* desc, size_t* bytes) {
  const hstu_status s = check_beam(desc);
  if (s != HSTU_OK) return s;
  if (bytes == nullptr) return HSTU_ERR_INVALID_ARG;
  *bytes = beam_layout(*desc).total;
  return HSTU_OK;
}

extern "C" hstu_status hstu_beam_decode_attn(const hstu_beam_desc* desc, const void* q, const void* ctx_k,
                                             const void* ctx_vt, const int32_t* ctx_len, const void* beam_k,
                                             const void* beam_v, const int32_t* path, void* out, void* workspace,
                                             size_t workspace_bytes, void* hip_stream) {
  const hstu_status s = check_beam(desc);
  if (s != HSTU_OK) return s;
  const hstu_beam_desc& d = *desc;
  if (d.num_requests == 0) return HSTU_OK;
  if (q == nullptr || ctx_k == nullptr || ctx_vt == nullptr || ctx_len == nullptr || beam_k == nullptr ||
      beam_v == nullptr || out == nullptr || workspace == nullptr || (d.step > 0 && path == nullptr))
    return HSTU_ERR_INVALID_ARG;
  if (!al16(q) || !al16(ctx_k) || !al16(ctx_vt) || !al16(beam_k) || !al16(beam_v) || !al16(out) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return HSTU_ERR_INVALID_ARG;
  const BeamLayout L = beam_layout(d);
  if (workspace_bytes < L.total) return HSTU_ERR_WORKSPACE;
  if (L.items > 0x7fffffffu) return HSTU_ERR_UNSUPPORTED;
  char* ws = static_cast<char*>(workspace);
  BeamArgs a;
  a.q = q;
  a.ctx_k = ctx_k;
  a.ctx_vt = ctx_vt;
  a.ctx_len = ctx_len;
  a.beam_k = beam_k;
  a.beam_v = beam_v;
  a.path = path;
  a.out = out;
  a.status = reinterpret_cast<int32_t*>(ws);
  a.part = reinterpret_cast<float*>(ws + L.part);
  a.mstat = reinterpret_cast<float*>(ws + L.mstat);
  a.lstat = reinterpret_cast<float*>(ws + L.lstat);
  a.R = d.num_requests;
  a.W = d.beam_width;
  a.Hq = d.num_q_heads;
  a.Hkv = d.num_kv_heads;
  a.G = L.G;
  a.Cmax = d.max_ctx;
  a.t = d.step;
  a.S = d.max_steps;
  a.NR = L.NR;
  a.nqt = L.nqt;
  a.nch = L.nch;
  a.csz = L.csz;
  a.scale2 = d.scale * kLog2e;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  hipError_t e;
  if (d.dtype == HSTU_BF16)
    e = d.head_dim == 128 ? launch_beam<bf16, 128>(a, L.items, st) : launch_beam<bf16, 64>(a, L.items, st);
  else
    e = d.head_dim == 128 ? launch_beam<float, 128>(a, L.items, st) : launch_beam<float, 64>(a, L.items, st);
  return e == hipSuccess ? HSTU_OK : HSTU_ERR_HIP;
}
