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
// Chunks are sized by cost, not by keys: a 32-key step of an entry with G
// query groups costs w(G) units (step_weight below).  With a budget of
// `budget` units per item an entry's chunks are at most
// clamp(budget / w, kMinSteps, kCapSteps) steps long, and the budget is the
// smallest one found that keeps the item count within the number of resident
// attention workgroups.  Each entry's keys are then cut into near-equal
// chunks (multiples of 32 keys).
#include "common.h"

namespace hstu {
namespace {

constexpr int kPrepThreads = 256;
constexpr int kPrepWaves = kPrepThreads / kWave;
constexpr int kStepKeys = 32;   // attention key step
constexpr int kMinSteps = 4;    // shortest chunk: a step for each of up to four phases
constexpr int kCapSteps = kMaxChunkKeys / kStepKeys;
// Cost of one 32-key step by the entry's query groups G, in units of about a
// tenth of a microsecond: the attention workgroup splits the steps of a
// q-block with G <= 4 over four phases, with G <= 8 over two, and multiplies
// every step with all its waves otherwise, so the time per step is a step
// function of G (measured on MI355X: about 0.85, 1.3 and 2.1 us).
__device__ __forceinline__ int step_weight(int groups) { return groups <= 4 ? 4 : (groups <= 8 ? 6 : 10); }
constexpr int kMinWeight = 4;
constexpr int kMaxWeight = 10;
constexpr int kWShift = 25;     // entry word: steps (bits 0..24) | weight << 25
constexpr int kStepMask = (1 << kWShift) - 1;
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
  int32_t qbn[kMaxQBlocks];        // chunks per q-block entry (steps | weight while searching)
  int32_t qbf[kMaxQBlocks];        // first work item of each q-block entry
  int32_t qbu[kMaxQBlocks];        // user of each q-block entry
  int32_t pgp[kMaxUsers + 1];      // first flat page index of each user
  int32_t cnt[16];                 // which candidate budgets fit
};

// Candidate budgets tried at once by the budget search.
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
      a.ws.row_loc[r] = make_int2(pg[i], pos[i] >= 0 ? pos[i] % a.ps : 0);
    }
  }
}

__device__ void work_list(const PrepArgs& a, PrepShared& s);

// Workgroup 0 validates the metadata (status), workgroup 1 builds the work
// list (wl_status), workgroups 2.. map the rows.
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
  if (blockIdx.x >= 2) {
    if (B > 0) map_rows(a, s, blockIdx.x - 2);   // B == 0 with rows is rejected below
    return;
  }
  if (blockIdx.x == 1) {
    work_list(a, s);
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
  if (tid == 0) hdr->status = s.err;
}

// Workgroup 1: the attention work list and the per-entry tables, built at
// the same time as workgroup 0 validates the metadata.  Its own checks only
// keep its writes in bounds (offsets and history lengths that workgroup 0
// rejects make it stop); its result goes to the header's wl_status.
__device__ void work_list(const PrepArgs& a, PrepShared& s) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  WsHeader* hdr = a.ws.hdr;
  const int B = a.B;
  if (tid == 0) s.err = 0;
  __syncthreads();
  if (tid == 0 && B == 0 && a.T != 0) set_err(s, HSTU_DEV_BAD_OFFSETS);
  for (int u = tid; u < B; u += kPrepThreads) {
    const int o0 = s.off[u], o1 = s.off[u + 1];
    if ((u == 0 && o0 != 0) || o1 < o0 || (u == B - 1 && o1 != a.T)) set_err(s, HSTU_DEV_BAD_OFFSETS);
    if (s.hist[u] < 0) set_err(s, HSTU_DEV_BAD_HIST);
  }
  __syncthreads();
  if (s.err != 0) {
    if (tid == 0) {
      hdr->wl_status = s.err;
      hdr->n_items = 0;
      hdr->n_qb = 0;
      hdr->item_budget = 0;
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

  // 3. item budget (see the top of this file).  The entries' step counts and
  //    weights are parked in qbn meanwhile.  With S = H * sum_e steps_e * w_e
  //    an entry gets at least steps_e * w_e / budget chunks and, while no
  //    chunk sits at its cap, fewer than steps_e * w_e / (budget - w_max) + 1,
  //    so the smallest fitting budget lies in [S / target, S / (target -
  //    H * nqb) + w_max]; kCand candidates spread over that window are tried
  //    at once (four per wave) and the smallest that fits is taken (the top
  //    one when none does, which can only happen through the cap).
  int64_t part = 0;
  for (int e = tid; e < nqb; e += kPrepThreads) {
    const int u = entry_user(s.qbb, B, e);
    const int qb = e - s.qbb[u];
    const int n = s.off[u + 1] - s.off[u];
    const int keys = s.hist[u] + min(n, (qb + 1) * kQB);
    const int steps = (keys + kStepKeys - 1) / kStepKeys;
    const int wt = step_weight((min(kQB, n - qb * kQB) + 15) / 16);
    s.qbn[e] = steps | (wt << kWShift);
    s.qbu[e] = u;
    part += static_cast<int64_t>(steps) * wt;
  }
  const int64_t hs = block_sum(part, s) * a.H;       // ends with a barrier
  const int64_t target = a.target_items;
  const int64_t slack = static_cast<int64_t>(a.H) * nqb;
  auto chunk_steps = [](int budget, int weight) { return min(kCapSteps, max(kMinSteps, budget / weight)); };
  constexpr int kBudgetLo = kMinWeight * kMinSteps, kBudgetHi = kMaxWeight * kCapSteps;
  int budget = kBudgetHi;
  if (target > slack) {
    const int64_t b_lo = min<int64_t>(kBudgetHi, max<int64_t>(kBudgetLo, (hs + target - 1) / target));
    const int64_t b_hi = min<int64_t>(kBudgetHi, max(b_lo, (hs + (target - slack) - 1) / (target - slack) + kMaxWeight));
    auto cand = [&](int k) {
      return static_cast<int>(k == kCand - 1 ? b_hi : b_lo + (b_hi - b_lo) * k / (kCand - 1));
    };
    // whether each of this wave's kCandPerWave budgets fits the target; the
    // wave counts them in one pass and reduces them together, so that the
    // shuffle latencies overlap.  Per-lane counts saturate at 2^24 (far
    // above any target), which keeps the lane sums inside int32.
    int bud[kCandPerWave], cnt[kCandPerWave];
#pragma unroll
    for (int k = 0; k < kCandPerWave; ++k) {
      bud[k] = cand(w * kCandPerWave + k);
      cnt[k] = 0;
    }
    for (int e = lane; e < nqb; e += kWave) {
      const int v = s.qbn[e];
      const int steps = v & kStepMask, wt = v >> kWShift;
#pragma unroll
      for (int k = 0; k < kCandPerWave; ++k) {
        const int L = chunk_steps(bud[k], wt);
        cnt[k] = min(cnt[k] + (steps + L - 1) / L, 1 << 24);
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
      for (int k = 0; k < kCandPerWave; ++k) cnt[k] += __shfl_xor(cnt[k], o, kWave);
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < kCandPerWave; ++k) {
        const int kk = w * kCandPerWave + k;
        s.cnt[kk] = (kk == kCand - 1 || static_cast<int64_t>(cnt[k]) * a.H <= target) ? 1 : 0;
      }
    }
    __syncthreads();
    int j = kCand - 1;
    for (int k = kCand - 1; k >= 0; --k)
      if (s.cnt[k]) j = k;
    budget = cand(j);
  }

  // 4. chunks per entry, then first item of each entry
  __syncthreads();                           // every wave is done counting
  for (int e = tid; e < nqb; e += kPrepThreads) {
    const int v = s.qbn[e];
    const int L = chunk_steps(budget, v >> kWShift);
    const int nch = ((v & kStepMask) + L - 1) / L;
    s.qbn[e] = nch;
    s.qbf[e] = nch * a.H;
  }
  __syncthreads();
  const int64_t n_items = block_scan(s.qbf, nqb, s);
  if (n_items > a.item_cap) {
    if (tid == 0) {
      hdr->wl_status = HSTU_DEV_CAPACITY;
      hdr->n_items = 0;
      hdr->n_qb = 0;
      hdr->item_budget = 0;
      hdr->counter = 0;
    }
    return;
  }

  // 5. the work list (one thread per item) and the per-entry tables used by
  //    the norm / output kernel
  for (int e = tid; e < nqb; e += kPrepThreads) {
    const int u = s.qbu[e], qb = e - s.qbb[u];
    a.ws.qb_first[e] = s.qbf[e];
    a.ws.qb_nch[e] = s.qbn[e];
    a.ws.qb_row0[e] = s.off[u] + qb * kQB;
    a.ws.qb_rows[e] = min(kQB, s.off[u + 1] - s.off[u] - qb * kQB);
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
    // step); csz is at most the entry's chunk bound, so (nch - 1) * csz <
    // keys and no chunk is empty
    const int csz = ((keys + nch - 1) / nch + kStepKeys - 1) / kStepKeys * kStepKeys;
    const int k_lo = kc * csz;
    AttnItem it;
    it.a = make_int4(u, qb * kQB, h, k_lo);
    it.b = make_int4(min(keys, k_lo + csz), s.off[u], n, c);
    a.ws.items[i] = it;
  }

  if (tid == 0) {
    hdr->wl_status = 0;
    hdr->n_items = static_cast<int32_t>(n_items);
    hdr->n_qb = nqb;
    hdr->item_budget = budget;
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
  return launch_kernel(prep_kernel, dim3(2 + (d.total_new + kRowsPerWg - 1) / kRowsPerWg), dim3(kPrepThreads),
                       stream, ev, a);
}

}  // namespace hstu
