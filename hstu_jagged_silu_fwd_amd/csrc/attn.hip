// Paged jagged SiLU attention (HSTU pointwise attention over a paged KV
// cache; NVIDIA blog "Deploying an HSTU generative recommender with NVIDIA
// Dynamo-Triton", section "Why serving large sequential recommenders is hard":
// the attention kernel reads K/V straight from the paged cache; aitrends.kr
// article 100093, "HSTU sequential modelling": SiLU weighting instead of
// softmax plus a relative attention bias).
//
// One work item = (user, q-block of kQB new rows, head, key chunk).  Each of
// the 4 waves of a workgroup owns 16 query rows and walks the chunk's keys 32
// at a time:
//   S^T[32 keys x 16 queries] = K * Q^T    (2 MFMA blocks, K rows from pages)
//   A = SiLU(S + bias[bucket(p - j)]) masked to j <= p   (fp32, per element)
//   O^T[d x 16]              += V^T * A    (V^T rows read key-contiguous from
//                                           the transposed V pages)
// The S^T accumulator of lane l holds 8 consecutive keys of one query, which
// is exactly the B-operand fragment of the second product, so scores never
// leave registers.  The K rows fed to S^T block b are permuted
// (row m -> key 8*(m/4) + 4*b + m%4) to make that true.
// Partial outputs (fp32, unscaled) go to the workspace; chunks of one row are
// added by the norm kernel.  Work items are fetched dynamically.
#include "common.h"

namespace hstu {
namespace {

template <typename T>
struct AttnArgs {
  const int32_t* new_off;
  const int32_t* hist;
  const int32_t* pt;
  const T* k_pool;
  const T* v_pool;
  const T* q;
  const float* pos_bias;
  const float* ts_bias;
  const int64_t* ts;
  const int32_t* ts_off;
  WsHeader* hdr;
  const int4* items;
  float* part;
  int H, D, ps_shift, maxP, nb, mbits, ntsb, tsmbits;
};

template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs<T> a) {
  constexpr int NC = HD / 32;   // 32-wide slices of the head dim (contraction of S^T)
  constexpr int NO = HD / 16;   // 16-row blocks of O^T
  __shared__ float s_pb[kMaxBuckets];
  __shared__ float s_tb[kMaxBuckets];
  __shared__ int s_item;
  if (a.hdr->status != 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  for (int i = tid; i < a.nb; i += 256) s_pb[i] = a.pos_bias[i];
  for (int i = tid; i < a.ntsb; i += 256) s_tb[i] = a.ts_bias[i];
  const int n_items = a.hdr->n_items;
  const int ck = a.hdr->chunk_keys;
  const int ps = 1 << a.ps_shift;
  const bool has_ts = a.ntsb > 0;

  for (;;) {
    __syncthreads();
    if (tid == 0) s_item = atomicAdd(&a.hdr->counter, 1);
    __syncthreads();
    const int it = s_item;
    if (it >= n_items) break;
    const int4 item = a.items[it];
    const int u = item.x, qb = item.y, h = item.z, kc = item.w;
    const int off_u = a.new_off[u];
    const int n = a.new_off[u + 1] - off_u;
    const int c = a.hist[u];
    const int len = c + n;
    const int t0w = qb * kQB + w * 16;              // first query row of this wave
    if (t0w >= n) continue;                         // no valid rows for this wave
    const int k_lo = kc * ck;
    const int k_hi = min(k_lo + ck, c + min(n, (qb + 1) * kQB));
    const int kend = min(k_hi, c + min(n, t0w + 16));   // keys past the wave's last query are masked
    const int t = t0w + l16;
    const int p = c + t;                            // query position (>= len for padded rows)
    const int tq = min(t, n - 1);

    Frag<T> qf[NC];
    {
      const T* qp = a.q + static_cast<size_t>(off_u + tq) * a.D + h * HD + g * 8;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) load_frag(qf[cc], qp + cc * 32);
    }
    f32x4 o[NO];
#pragma unroll
    for (int ob = 0; ob < NO; ++ob) o[ob] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int32_t* ptu = a.pt + static_cast<size_t>(u) * a.maxP;
    const size_t head_k = static_cast<size_t>(h) * ps * HD;
    const size_t page_k = static_cast<size_t>(a.H) * ps * HD;
    const int64_t* tsu = has_ts ? a.ts + a.ts_off[u] : nullptr;
    const int64_t ts_p = has_ts ? tsu[min(p, len - 1)] : 0;

    for (int kb = k_lo; kb < kend; kb += 32) {
      f32x4 st[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int key = kb + 8 * (l16 >> 2) + 4 * b + (l16 & 3);
        const int kcl = key < len ? key : len - 1;
        const int page = ptu[kcl >> a.ps_shift];
        const T* kp = a.k_pool + static_cast<size_t>(page) * page_k + head_k +
                      static_cast<size_t>(kcl & (ps - 1)) * HD + g * 8;
        st[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
          Frag<T> kf;
          load_frag(kf, kp + cc * 32);
          st[b] = mma16(kf, qf[cc], st[b]);
        }
      }
      Frag<T> af;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb + 8 * g + 4 * b + i;
          const int delta = p - key;
          float s = st[b][i] + s_pb[bucket32(delta, a.mbits, a.nb)];
          if (has_ts) {
            const int kcl = key < len ? key : len - 1;
            s += s_tb[bucket64(ts_p - tsu[kcl], a.tsmbits, a.ntsb)];
          }
          set_elem(af, 4 * b + i, delta >= 0 ? silu(s) : 0.0f);
        }
      const int kg = kb + 8 * g;                     // first of this lane's 8 keys
      const bool vok = kg < len;
      const int kgc = vok ? kg : 0;
      const int vpage = ptu[kgc >> a.ps_shift];
      const T* vp = a.v_pool + static_cast<size_t>(vpage) * page_k + head_k + (kgc & (ps - 1));
      const int nvalid = len - kg;                   // < 8 on the sequence's last keys
#pragma unroll
      for (int ob = 0; ob < NO; ++ob) {
        Frag<T> vf;
        if (vok) {
          load_frag(vf, vp + static_cast<size_t>(ob * 16 + l16) * ps);
          if (nvalid < 8) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (e >= nvalid) set_elem(vf, e, 0.0f);
          }
        } else {
          zero_frag(vf);
        }
        o[ob] = mma16(vf, af, o[ob]);
      }
    }
    if (t < n) {
      float* dst = a.part + (static_cast<size_t>(it) * kQB + w * 16 + l16) * HD + 4 * g;
#pragma unroll
      for (int ob = 0; ob < NO; ++ob) *reinterpret_cast<f32x4*>(dst + ob * 16) = o[ob];
    }
  }
}

template <typename T, int HD>
hipError_t attn_t(const hstu_layer_desc& d, const int32_t* new_off, const int32_t* hist,
                  const int32_t* pt, const void* k_pool, const void* v_pool, const float* pos_bias,
                  const float* ts_bias, const int64_t* ts, const int32_t* ts_off, const WsPtrs& ws,
                  int grid, hipStream_t stream) {
  AttnArgs<T> a;
  a.new_off = new_off;
  a.hist = hist;
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
  attn_kernel<T, HD><<<grid, 256, 0, stream>>>(a);
  return hipGetLastError();
}

template <typename T>
hipError_t attn_dt(const hstu_layer_desc& d, const int32_t* new_off, const int32_t* hist,
                   const int32_t* pt, const void* k_pool, const void* v_pool, const float* pos_bias,
                   const float* ts_bias, const int64_t* ts, const int32_t* ts_off, const WsPtrs& ws,
                   int grid, hipStream_t stream) {
  switch (d.head_dim) {
    case 32: return attn_t<T, 32>(d, new_off, hist, pt, k_pool, v_pool, pos_bias, ts_bias, ts, ts_off, ws, grid, stream);
    case 64: return attn_t<T, 64>(d, new_off, hist, pt, k_pool, v_pool, pos_bias, ts_bias, ts, ts_off, ws, grid, stream);
    default: return attn_t<T, 128>(d, new_off, hist, pt, k_pool, v_pool, pos_bias, ts_bias, ts, ts_off, ws, grid, stream);
  }
}

}  // namespace

hipError_t launch_attn(const hstu_layer_desc& d, const int32_t* new_off, const int32_t* hist,
                       const int32_t* pt, const void* k_pool, const void* v_pool,
                       const float* pos_bias, const float* ts_bias, const int64_t* ts,
                       const int32_t* ts_off, const WsPtrs& ws, int grid, hipStream_t stream) {
  if (d.dtype == HSTU_BF16)
    return attn_dt<bf16>(d, new_off, hist, pt, k_pool, v_pool, pos_bias, ts_bias, ts, ts_off, ws, grid, stream);
  return attn_dt<float>(d, new_off, hist, pt, k_pool, v_pool, pos_bias, ts_bias, ts, ts_off, ws, grid, stream);
}

}  // namespace hstu
