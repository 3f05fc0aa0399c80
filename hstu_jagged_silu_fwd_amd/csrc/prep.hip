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

constexpr int kPrepThreads = 1024;
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
  int ck;                          // chunk length bound of the call
  int64_t wsum[kPrepWaves];
  int32_t off[kMaxUsers + 1];
  int32_t hist[kMaxUsers];
  int32_t qbb[kMaxUsers + 1];      // first q-block entry of each user
  int32_t qbn[kMaxQBlocks];        // chunks per q-block entry
  int32_t qbf[kMaxQBlocks];        // first work item of each q-block entry
};

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
    // page ids of every position in use: one wavefront per user
    for (int u = w; u < B; u += kPrepWaves) {
      const int len = s.hist[u] + (s.off[u + 1] - s.off[u]);
      const int npg = (len + a.ps - 1) / a.ps;
      const int32_t* row = a.pt + static_cast<size_t>(u) * a.maxP;
      for (int j = lane; j < npg; j += kWave) {
        const int32_t pg = row[j];
        if (pg < 0 || pg >= a.P) set_err(s, HSTU_DEV_BAD_PAGE);
      }
    }
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
  }
  __syncthreads();
  // one wave searches (no barriers); the others wait at the next barrier
  if (w == 0) {
    int lo = kMinChunk / kStepKeys, hi = kMaxChunkKeys / kStepKeys;
    while (lo < hi) {                        // uniform across the wave
      const int mid = (lo + hi) >> 1;
      const int len = mid * kStepKeys;
      int64_t cnt = 0;
      for (int e = lane; e < nqb; e += kWave) cnt += (s.qbn[e] + len - 1) / len;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o, kWave);
      if (cnt * a.H <= a.target_items) hi = mid; else lo = mid + 1;
    }
    if (lane == 0) s.ck = lo * kStepKeys;
  }
  __syncthreads();
  const int ck = s.ck;

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

  // 5. the work list and the per-entry tables used by the norm kernel
  for (int e = tid; e < nqb; e += kPrepThreads) {
    const int u = entry_user(s.qbb, B, e);
    const int qb = e - s.qbb[u];
    const int f = s.qbf[e], nch = s.qbn[e];
    a.ws.qb_first[e] = f;
    a.ws.qb_nch[e] = nch;
    const int n = s.off[u + 1] - s.off[u];
    const int c = s.hist[u];
    const int keys = c + min(n, (qb + 1) * kQB);
    // the entry's keys are cut into nch near-equal chunks (multiples of a
    // step); csz <= ck, so (nch - 1) * csz < keys and no chunk is empty
    const int csz = ((keys + nch - 1) / nch + kStepKeys - 1) / kStepKeys * kStepKeys;
    for (int h = 0; h < a.H; ++h)
      for (int kc = 0; kc < nch; ++kc) {
        const int k_lo = kc * csz;
        AttnItem it;
        it.a = make_int4(u, qb * kQB, h, k_lo);
        it.b = make_int4(min(keys, k_lo + csz), s.off[u], n, c);
        a.ws.items[f + h * nch + kc] = it;
      }
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
                       int nqb_cap, int item_cap, int target_items, hipStream_t stream) {
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
  prep_kernel<<<1 + (d.total_new + kRowsPerWg - 1) / kRowsPerWg, kPrepThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace hstu
