// Index prep for one layer call: validates the jagged/paged metadata, maps
// rows to users and pool slots, and builds the attention work list.
// Workgroup 0 does the validation and the work list, keeping all per-user
// and per-q-block metadata in LDS while it is built; workgroups 1.. each map
// a slice of kRowsPerWg new rows to (user, page, slot).
//
// Work decomposition: the new rows of user u are cut into q-blocks of kQB
// rows; q-block qb sees keys [0, hist + min(n, (qb+1)*kQB)) (causal).  The key
// range of every (q-block, head) is split into near-equal chunks, one work
// item per (user, q-block, head, chunk).
// Because the attention has no softmax, the partial outputs of the chunks of
// a row simply add; the norm kernel sums them in chunk order.
// The chunk length bound ck is the smallest multiple of 32 keys (at least 128,
// at most kMaxChunkKeys) that keeps the item count within the number of
// resident attention workgroups; each entry's keys are then cut into
// ceil(keys / ck) chunks of near-equal length (multiples of 32).
#include "common.h"

namespace hstu {
namespace {

constexpr int kPrepThreads = 256;
constexpr int kPrepWaves = kPrepThreads / kWave;
constexpr int kStepKeys = 32;   // attention key step
constexpr int kMinChunk = 128;  // one step for each of the four waves
constexpr int kRowsPerThread = 4;
constexpr int kRowsPerWg = kPrepThreads * kRowsPerThread;

struct PrepArgs {
  const int32_t* new_off;
  const int32_t* hist;
  const int32_t* pt;
  const int32_t* ts_off;
  WsPtrs ws;
  int B, T, H, ps, maxP;
  int64_t P;
  int nqb_cap, item_cap, target_items;
};

struct PrepShared {
  int err;
  int64_t wsum[kPrepWaves];
  int32_t off[kMaxUsers + 1];
  int32_t hist[kMaxUsers];
  int32_t qbb[kMaxUsers + 1];      // first q-block entry of each user
  int32_t qbn[kMaxQBlocks];        // chunks per q-block entry
  int32_t qbf[kMaxQBlocks];        // first work item of each q-block entry
  int32_t qbu[kMaxQBlocks];        // user of each q-block entry
  int32_t pgp[kMaxUsers + 1];      // first flat page index of each user
  int32_t cnt[16];                 // which candidate chunk lengths fit
};

// Candidate chunk lengths tried at once by the chunk-length search.
constexpr int kCand = 16;
constexpr int kCandPerWave = kCand / kPrepWaves;

__device__ void set_err(PrepShared& s, int code) { atomicCAS(&s.err, 0, code); }

__device__ __forceinline__ int64_t wave_incl_scan(int64_t x, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int64_t y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  return x;
}

// In-place exclusive scan of v[0..n) (LDS) by the whole block; returns the total.
__device__ int64_t block_scan(int32_t* v, int n, PrepShared& s) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int seg = (n + kPrepThreads - 1) / kPrepThreads;
  const int lo = min(n, tid * seg), hi = min(n, lo + seg);
  int64_t sum = 0;
  for (int i = lo; i < hi; ++i) sum += v[i];
  const int64_t incl = wave_incl_scan(sum, lane);
  if (lane == kWave - 1) s.wsum[w] = incl;
  __syncthreads();
  int64_t before = 0, total = 0;
  for (int i = 0; i < kPrepWaves; ++i) {
    if (i < w) before += s.wsum[i];
    total += s.wsum[i];
  }
  int64_t run = before + incl - sum;
  for (int i = lo; i < hi; ++i) {
    const int32_t x = v[i];
    v[i] = static_cast<int32_t>(run);
    run += x;
  }
  __syncthreads();
  return total;
}

__device__ int64_t block_sum(int64_t x, PrepShared& s) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, kWave);
  if (lane == 0) s.wsum[w] = x;
  __syncthreads();
  int64_t t = 0;
  for (int i = 0; i < kPrepWaves; ++i) t += s.wsum[i];
  __syncthreads();
  return t;
}

// Entry e -> (user, q-block) by binary search over the user's first entries.
__device__ __forceinline__ int entry_user(const int32_t* qbb, int B, int e) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qbb[mid] <= e) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Rows -> user, and the pool (page, slot) their K/V go to.  Positions whose
// page-table entry would fall outside the table (only possible with metadata
// that workgroup 0 rejects) get page -1.
__device__ void map_rows(const PrepArgs& a, const PrepShared& s, int slice) {
  const int r0 = slice * kRowsPerWg + threadIdx.x;
  int user[kRowsPerThread], pos[kRowsPerThread], pg[kRowsPerThread];
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    const int r = r0 + i * kPrepThreads;
    user[i] = r < a.T ? row_to_user(s.off, a.B, r) : 0;
    pos[i] = r < a.T ? s.hist[user[i]] + (r - s.off[user[i]]) : -1;
  }
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    const bool ok = pos[i] >= 0 && pos[i] / a.ps < a.maxP;
    pg[i] = ok ? a.pt[static_cast<size_t>(user[i]) * a.maxP + pos[i] / a.ps] : -1;
  }
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    const int r = r0 + i * kPrepThreads;
    if (r < a.T) {
      a.ws.row_user[r] = user[i];
      a.ws.row_loc[r] = make_int2(pg[i], pos[i] >= 0 ? pos[i] % a.ps : 0);
    }
  }
}

__global__ __launch_bounds__(kPrepThreads) void prep_kernel(PrepArgs a) {
  __shared__ PrepShared s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  WsHeader* hdr = a.ws.hdr;
  const int B = a.B;
  if (tid == 0) s.err = 0;
  for (int u = tid; u <= B; u += kPrepThreads) s.off[u] = a.new_off[u];
  for (int u = tid; u < B; u += kPrepThreads) s.hist[u] = a.hist[u];
  __syncthreads();
  if (blockIdx.x > 0) {
    if (B > 0) map_rows(a, s, blockIdx.x - 1);   // B == 0 with rows is rejected below
    return;
  }

  // 1. metadata checks
  if (tid == 0 && B == 0 && a.T != 0) set_err(s, HSTU_DEV_BAD_OFFSETS);
  for (int u = tid; u < B; u += kPrepThreads) {
    const int o0 = s.off[u], o1 = s.off[u + 1];
    if ((u == 0 && o0 != 0) || o1 < o0 || (u == B - 1 && o1 != a.T)) set_err(s, HSTU_DEV_BAD_OFFSETS);
    const int c = s.hist[u];
    if (c < 0) {
      set_err(s, HSTU_DEV_BAD_HIST);
    } else if (static_cast<int64_t>(c) + (o1 - o0) > static_cast<int64_t>(a.maxP) * a.ps) {
      set_err(s, HSTU_DEV_CAPACITY);
    }
    if (a.ts_off != nullptr) {
      if ((u == 0 && a.ts_off[0] != 0) ||
          static_cast<int64_t>(a.ts_off[u + 1]) - a.ts_off[u] != static_cast<int64_t>(c) + (o1 - o0))
        set_err(s, HSTU_DEV_BAD_TS);
    }
  }
  __syncthreads();
  if (s.err == 0) {
    // page ids of every position in use, over a flat (user, page) index so
    // that each thread issues its loads back to back
    for (int u = tid; u < B; u += kPrepThreads)
      s.pgp[u] = (s.hist[u] + (s.off[u + 1] - s.off[u]) + a.ps - 1) / a.ps;
    __syncthreads();
    const int64_t total_pages = block_scan(s.pgp, B, s);
    if (tid == 0) s.pgp[B] = static_cast<int32_t>(total_pages);
    __syncthreads();
    constexpr int kU = 4;
    bool bad = false;
    for (int64_t i0 = tid; i0 < total_pages; i0 += kU * kPrepThreads) {
      int32_t pg[kU];
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        const int i = static_cast<int>(i0) + k * kPrepThreads;
        pg[k] = 0;
        if (i < total_pages) {
          int lo = 0, hi = B - 1;              // user owning flat page i
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s.pgp[mid] <= i) lo = mid; else hi = mid - 1;
          }
          pg[k] = a.pt[static_cast<size_t>(lo) * a.maxP + (i - s.pgp[lo])];
        }
      }
#pragma unroll
      for (int k = 0; k < kU; ++k) bad |= pg[k] < 0 || pg[k] >= a.P;
    }
    if (bad) set_err(s, HSTU_DEV_BAD_PAGE);
  }
  __syncthreads();
  if (s.err != 0) {
    if (tid == 0) {
      hdr->status = s.err;
      hdr->n_items = 0;
      hdr->chunk_keys = 0;
      hdr->counter = 0;
    }
    return;
  }

  // 2. q-block entries per user
  for (int u = tid; u < B; u += kPrepThreads) s.qbb[u] = (s.off[u + 1] - s.off[u] + kQB - 1) / kQB;
  __syncthreads();
  const int nqb = static_cast<int>(block_scan(s.qbb, B, s));
  if (tid == 0) s.qbb[B] = nqb;
  __syncthreads();

  // 3. chunk length: the smallest multiple of kStepKeys, at least kMinChunk,
  //    for which the items H * sum_e ceil(keys_e / L) fit the target (one
  //    item per resident attention workgroup), capped at kMaxChunkKeys.
  //    The entry key counts are parked in qbn meanwhile.
  for (int e = tid; e < nqb; e += kPrepThreads) {
    const int u = entry_user(s.qbb, B, e);
    const int qb = e - s.qbb[u];
    const int n = s.off[u + 1] - s.off[u];
    s.qbn[e] = s.hist[u] + min(n, (qb + 1) * kQB);
    s.qbu[e] = u;
  }
  __syncthreads();
  // H * sum_e ceil(k_e / L) lies in [H*K/L, H*K/L + H*nqb] for K = sum_e k_e,
  // so the answer sits between L_lo = H*K/T and L_hi = H*K/(T - H*nqb); up to
  // 16 candidates spread over that window are tried at once (four per wave).
  int64_t part = 0;
  for (int e = tid; e < nqb; e += kPrepThreads) part += s.qbn[e];
  const int64_t hk = block_sum(part, s) * a.H;
  const int64_t target = a.target_items;
  const int64_t slack = static_cast<int64_t>(a.H) * nqb;
  auto round_step = [](int64_t x) { return (x + kStepKeys - 1) / kStepKeys; };   // keys -> steps
  int ck;
  if (target <= slack) {
    ck = kMaxChunkKeys;                      // every entry already has an item per head
  } else {
    const int64_t cap = kMaxChunkKeys / kStepKeys;
    const int64_t lo_s = min(cap, max<int64_t>(kMinChunk / kStepKeys, round_step((hk + target - 1) / target)));
    const int64_t hi_s = min(cap, max(lo_s, round_step((hk + (target - slack) - 1) / (target - slack))));
    const int stride = static_cast<int>((hi_s - lo_s + kCand) / kCand);   // >= 1
    auto count_items = [&](int steps) {        // wave-cooperative; the same in every lane
      const int len = steps * kStepKeys;
      int cnt = 0;
      for (int e = lane; e < nqb; e += kWave) cnt += (s.qbn[e] + len - 1) / len;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o, kWave);
      return static_cast<int64_t>(cnt) * a.H;
    };
    for (int k = w * kCandPerWave; k < (w + 1) * kCandPerWave; ++k) {
      const int cand = static_cast<int>(min<int64_t>(lo_s + static_cast<int64_t>(k) * stride, hi_s));
      const bool fits = cand == hi_s || count_items(cand) <= target;
      if (lane == 0) s.cnt[k] = fits ? 1 : 0;
    }
    __syncthreads();
    int j = kCand - 1;
    for (int k = kCand - 1; k >= 0; --k)
      if (s.cnt[k]) j = k;
    ck = static_cast<int>(min<int64_t>(lo_s + static_cast<int64_t>(j) * stride, hi_s)) * kStepKeys;
  }

  // 4. chunks per entry, then first item of each entry
  for (int e = tid; e < nqb; e += kPrepThreads) {
    const int nch = (s.qbn[e] + ck - 1) / ck;
    s.qbn[e] = nch;
    s.qbf[e] = nch * a.H;
  }
  __syncthreads();
  const int64_t n_items = block_scan(s.qbf, nqb, s);
  if (n_items > a.item_cap) {
    if (tid == 0) {
      hdr->status = HSTU_DEV_CAPACITY;
      hdr->n_items = 0;
      hdr->chunk_keys = 0;
      hdr->counter = 0;
    }
    return;
  }

  // 5. the work list (one thread per item) and the per-entry tables used by
  //    the norm kernel
  for (int e = tid; e < nqb; e += kPrepThreads) {
    a.ws.qb_first[e] = s.qbf[e];
    a.ws.qb_nch[e] = s.qbn[e];
  }
  for (int i = tid; i < n_items; i += kPrepThreads) {
    int lo = 0, hi = nqb - 1;                // last entry whose first item <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s.qbf[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int e = lo, u = s.qbu[e], qb = e - s.qbb[u], nch = s.qbn[e];
    const int r = i - s.qbf[e], h = r / nch, kc = r - h * nch;
    const int n = s.off[u + 1] - s.off[u];
    const int c = s.hist[u];
    const int keys = c + min(n, (qb + 1) * kQB);
    // the entry's keys are cut into nch near-equal chunks (multiples of a
    // step); csz <= ck, so (nch - 1) * csz < keys and no chunk is empty
    const int csz = ((keys + nch - 1) / nch + kStepKeys - 1) / kStepKeys * kStepKeys;
    const int k_lo = kc * csz;
    AttnItem it;
    it.a = make_int4(u, qb * kQB, h, k_lo);
    it.b = make_int4(min(keys, k_lo + csz), s.off[u], n, c);
    a.ws.items[i] = it;
  }
  for (int u = tid; u <= B; u += kPrepThreads) a.ws.qb_base[u] = s.qbb[u];

  if (tid == 0) {
    hdr->status = 0;
    hdr->n_items = static_cast<int32_t>(n_items);
    hdr->chunk_keys = static_cast<int32_t>(ck);
    hdr->counter = 0;
  }
}

}  // namespace

hipError_t launch_prep(const hstu_layer_desc& d, const int32_t* new_off, const int32_t* hist,
                       const int32_t* pt, const int32_t* ts_off, const WsPtrs& ws,
                       int nqb_cap, int item_cap, int target_items, hipStream_t stream,
                       const KernelEvents& ev) {
  PrepArgs a;
  a.new_off = new_off;
  a.hist = hist;
  a.pt = pt;
  a.ts_off = ts_off;
  a.ws = ws;
  a.B = d.num_users;
  a.T = d.total_new;
  a.H = d.num_heads;
  a.ps = d.page_size;
  a.maxP = d.max_pages_per_user;
  a.P = d.num_pool_pages;
  a.nqb_cap = nqb_cap;
  a.item_cap = item_cap;
  a.target_items = target_items;
  return launch_kernel(prep_kernel, dim3(1 + (d.total_new + kRowsPerWg - 1) / kRowsPerWg), dim3(kPrepThreads),
                       stream, ev, a);
}

}  // namespace hstu
