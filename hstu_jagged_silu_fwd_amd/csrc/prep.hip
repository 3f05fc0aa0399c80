// Index prep for one layer call: validates the jagged/paged metadata, maps
// rows to users and pool slots, and builds the attention work list.
// Workgroup 0 validates, workgroup 1 builds the work list at the same time
// (each keeps the per-user and per-q-block metadata in LDS; their scans run
// inside one wave, so the only workgroup barriers are between phases), one
// workgroup per layer builds that layer's bias tables for the attention, and
// the others each map a slice of kRowsPerWg new rows to (user, page, slot).
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
// attention workgroups (when the entries alone reach that number: within
// the workgroups plus the entries, rounded up to a whole multiple of the
// workgroups).  Each entry's keys are then cut into near-equal chunks
// (multiples of 32 keys).  When the items outnumber the workgroups the list
// is ordered by chunk cost, highest first: the first items go to the
// workgroups in list order and the rest to whichever finishes first.
// Batch-invariant calls (HSTU_FLAG_BATCH_INVARIANT) skip the search: every
// entry's keys are cut at the multiples of HSTU_INVARIANT_CHUNK_KEYS, so a
// row's pieces depend only on its own position, never on the batch.
#include "common.h"

namespace hstu {
namespace {

constexpr int kPrepThreads = 256;
constexpr int kPrepWaves = kPrepThreads / kWave;
constexpr int kStepKeys = 32;   // attention key step
constexpr int kMinSteps = 4;    // shortest chunk: a step for each of up to four phases
constexpr int kCapSteps = kMaxChunkKeys / kStepKeys;
// Cost of one 32-key step by the entry's query groups G, in units
// proportional to the attention's measured time per step (per-workgroup
// s_memtime stamps of an instrumented build on MI355X, about 2 GHz: some
// 1.46k ticks up to two groups, 1.67k up to eight -- the workgroup splits
// those steps over two phases -- 2.45k up to twelve and 2.9k beyond, where
// every wave multiplies every step; the 16-wave layout's ratios are alike).
__device__ __forceinline__ int step_weight(int groups) {
  return groups <= 2 ? 9 : (groups <= 4 ? 10 : (groups <= 8 ? 11 : (groups <= 12 ? 15 : 18)));
}
constexpr int kMinWeight = 9;
constexpr int kMaxWeight = 18;
constexpr int kWShift = 25;     // entry word: steps (bits 0..24) | weight << 25
constexpr int kStepMask = (1 << kWShift) - 1;
constexpr int kRowsPerThread = 4;
constexpr int kRowsPerWg = kPrepThreads * kRowsPerThread;

struct PrepArgs {
  const int32_t* new_off;
  const int32_t* hist;
  const int32_t* ncand;
  const int32_t* pt[kMaxStackLayers];   // page table of each layer (nl of them)
  const int32_t* ts_off;
  const float* pb[kMaxStackLayers];     // position-bucket bias of each layer
  const float* tb[kMaxStackLayers];     // timestamp-bucket bias of each layer (null: none)
  WsPtrs ws;
  int B, T, H, ps, maxP, nl;
  int nb, mbits, ntsb;
  int64_t P;
  int nqb_cap, item_cap, target_items;
  int inv_steps;                        // fixed chunk length in steps (batch-invariant calls), else 0
};

struct PrepShared {
  int32_t off[kMaxUsers + 1];
  int32_t hist[kMaxUsers];
  int32_t qbb[kMaxUsers + 1];      // first q-block entry of each user
  int32_t qbn[kMaxQBlocks];        // chunks per q-block entry (steps | weight while searching)
  int32_t qbf[kMaxQBlocks];        // first work item of each q-block entry
  int32_t qbu[kMaxQBlocks];        // user of each q-block entry
  int32_t ord[kMaxQBlocks];        // entries in work-list order (heavy entries first)
  int32_t pgp[kMaxUsers + 1];      // first flat page index of each user
  int32_t cnt[kPrepWaves][16];     // per-wave item counts of the candidate budgets
  float tpb[kMaxBuckets];          // a layer's scaled bucket tables (table workgroups)
  float ttb[kMaxBuckets];
  int32_t bad[kPrepWaves];
  int32_t err, nqb, budget, n_items, b_lo, b_hi;
};

// Candidate budgets tried at once by the budget search: thread t counts for
// candidate t % kCand over the entries e = t / kCand (mod kPrepThreads / kCand).
constexpr int kCand = 16;
constexpr int kCandSlices = kPrepThreads / kCand;

// Wave-level exclusive scan; *total receives the wave's sum.  The scans over
// users and entries run in one wave, 64 values per pass with a carry, so
// that no workgroup barrier sits between their steps.
template <typename I>
__device__ __forceinline__ I wave_excl_scan(I x, int lane, I* total) {
  I incl = x;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const I y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  *total = __shfl(incl, kWave - 1, kWave);
  return incl - x;
}

template <typename I>
__device__ __forceinline__ I wave_sum(I x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

// ceil(x / y) for 0 <= x < 2^40, y > 0 through double precision: the
// quotient's fractional part is at least 1/y >= 2^-40 relative to the
// quotient's integer part whenever it is nonzero, far above the 2^-52
// rounding of the division, so the ceiling is exact.
__device__ __forceinline__ int64_t ceil_div(int64_t x, int64_t y) {
  return static_cast<int64_t>(ceil(static_cast<double>(x) / static_cast<double>(y)));
}

// Item target of the work list: the workgroups, or, when the q-block entries
// times heads (slack) reach them, target + slack rounded up to a multiple of
// target.  At most target + slack + target - 1.
__device__ __forceinline__ int64_t item_target(int64_t target, int64_t slack) {
  return target > slack ? target : ceil_div(target + slack, target) * target;
}

// Entry e -> user by binary search over the users' first entries.
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
  for (int l = 0; l < a.nl; ++l) {                   // every layer's pages (one per call but a stack's)
    const int32_t* pt = a.pt[l];
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
      const bool ok = pos[i] >= 0 && pos[i] / a.ps < a.maxP;
      pg[i] = ok ? pt[static_cast<size_t>(user[i]) * a.maxP + pos[i] / a.ps] : -1;
    }
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
      const int r = r0 + i * kPrepThreads;
      if (r < a.T) {
        a.ws.row_loc[static_cast<size_t>(l) * a.T + r] = make_int2(pg[i], pos[i] >= 0 ? pos[i] % a.ps : 0);
      }
    }
  }
}

// Offset and history checks shared by workgroups 0 and 1 (wave 0 only).
// Returns the first failing code in the order offsets, history lengths.
__device__ int check_offsets(const PrepArgs& a, const PrepShared& s, int lane) {
  const int B = a.B;
  bool bad_off = B == 0 && a.T != 0, bad_hist = false;
  for (int u0 = 0; u0 < B; u0 += kWave) {
    const int u = u0 + lane;
    if (u < B) {
      const int o0 = s.off[u], o1 = s.off[u + 1];
      bad_off |= (u == 0 && o0 != 0) || o1 < o0 || (u == B - 1 && o1 != a.T);
      bad_hist |= s.hist[u] < 0;
    }
  }
  if (__any(bad_off)) return HSTU_DEV_BAD_OFFSETS;
  if (__any(bad_hist)) return HSTU_DEV_BAD_HIST;
  return 0;
}

__device__ void validate(const PrepArgs& a, PrepShared& s);
__device__ void work_list(const PrepArgs& a, PrepShared& s);

// Layer l's bias tables (layout at kTabFloats), in the attention's exponent
// domain: the bucket tables scaled by -log2(e), the distance table read from
// them through the bucket rule, masked entries past it.
__device__ void build_tables(const PrepArgs& a, PrepShared& s, int l) {
  const int tid = threadIdx.x;
  const float* pb = a.pb[l];
  const float* tb = a.tb[l];
  for (int i = tid; i < kMaxBuckets; i += kPrepThreads) {
    s.tpb[i] = i < a.nb ? kNegLog2e * pb[i] : 0.f;
    s.ttb[i] = (tb != nullptr && i < a.ntsb) ? kNegLog2e * tb[i] : 0.f;
  }
  __syncthreads();
  float* out = a.ws.tables + static_cast<size_t>(l) * kTabFloats;
  for (int i = tid; i < kTabFloats; i += kPrepThreads) {
    float v = 0.f;
    if (i < kLut) v = s.tpb[bucket32(kLut - 1 - i, a.mbits, a.nb)];
    else if (i < kTabPb) v = kMasked;
    else if (i < kTabTb) v = s.tpb[i - kTabPb];
    else if (i < kTabTb + kMaxBuckets) v = s.ttb[i - kTabTb];
    out[i] = v;
  }
}

// Workgroup 0 validates the metadata (status), workgroup 1 builds the work
// list (wl_status), workgroups 2 .. 2+nl-1 build each layer's bias tables,
// the rest map the rows.
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(PrepArgs a) {
  __shared__ PrepShared s;
  const int tid = threadIdx.x;
  const int B = a.B;
  if (blockIdx.x >= 2 && blockIdx.x < 2 + a.nl) {
    build_tables(a, s, blockIdx.x - 2);
    return;
  }
  for (int u = tid; u <= B; u += kPrepThreads) s.off[u] = a.new_off[u];
  for (int u = tid; u < B; u += kPrepThreads) s.hist[u] = a.hist[u];
  __syncthreads();
  if (blockIdx.x >= 2) {
    if (B > 0) map_rows(a, s, blockIdx.x - 2 - a.nl);   // B == 0 with rows is rejected by workgroup 0
    return;
  }
  if (blockIdx.x == 1) work_list(a, s);
  else validate(a, s);
}

// Workgroup 0: every check of the call's metadata, including every page id
// in use, into the header's status word (first failure in the order of the
// status codes' listing in the header, page ids last).
__device__ void validate(const PrepArgs& a, PrepShared& s) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int B = a.B;
  if (w == 0) {
    int err = check_offsets(a, s, lane);
    bool cap = false, bad_ts = false, bad_cand = false;
    int carry = 0;
    for (int u0 = 0; u0 < B; u0 += kWave) {
      const int u = u0 + lane;
      int np = 0;
      if (u < B) {
        const int n = s.off[u + 1] - s.off[u];
        const int64_t len = static_cast<int64_t>(s.hist[u]) + n;
        cap |= len > static_cast<int64_t>(a.maxP) * a.ps;
        if (a.ncand != nullptr) bad_cand |= a.ncand[u] < 0 || a.ncand[u] > n;
        if (a.ts_off != nullptr)
          bad_ts |= (u == 0 && a.ts_off[0] != 0) ||
                    static_cast<int64_t>(a.ts_off[u + 1]) - a.ts_off[u] != len;
        // pages in use (bounded by the table row once the checks pass)
        np = static_cast<int>(min<int64_t>((len + a.ps - 1) / a.ps, a.maxP));
        np = max(np, 0);
      }
      int tot;
      const int ex = wave_excl_scan(np, lane, &tot);
      if (u < B) s.pgp[u] = carry + ex;
      carry += tot;
    }
    if (err == 0 && __any(cap)) err = HSTU_DEV_CAPACITY;
    if (err == 0 && __any(bad_ts)) err = HSTU_DEV_BAD_TS;
    if (err == 0 && __any(bad_cand)) err = HSTU_DEV_BAD_CANDIDATES;
    if (lane == 0) {
      s.pgp[B] = carry;
      s.err = err;
    }
  }
  __syncthreads();
  const int err = s.err;
  bool bad = false;
  if (err == 0) {
    // page ids of every position in use, over a flat (user, page) index:
    // thread t takes the contiguous range [t*m, (t+1)*m) in rounds of kU,
    // finds the user of its first index by a binary search and walks the
    // users from there, so the kU loads of a round go out back to back
    const int total_pages = s.pgp[B];
    constexpr int kU = 16;                           // loads in flight per thread
    const int m = (total_pages + kPrepThreads - 1) / kPrepThreads;
    const int i_beg = min(total_pages, tid * m), i_end = min(total_pages, i_beg + m);
    int u = i_beg < i_end ? entry_user(s.pgp, B, i_beg) : 0;
    int u_end = s.pgp[u + 1];                        // first flat index past user u
    const int u_first = u, u_end_first = u_end;
    for (int l = 0; l < a.nl; ++l) {                 // every layer's table
      const int32_t* pt = a.pt[l];
      u = u_first;
      u_end = u_end_first;
      for (int i0 = i_beg; i0 < i_end; i0 += kU) {
        int32_t pg[kU];
#pragma unroll
        for (int k = 0; k < kU; ++k) {
          const int i = i0 + k;
          pg[k] = 0;
          if (i < i_end) {
            while (i >= u_end) u_end = s.pgp[++u + 1];   // skips users without pages
            pg[k] = pt[static_cast<size_t>(u) * a.maxP + (i - s.pgp[u])];
          }
        }
#pragma unroll
        for (int k = 0; k < kU; ++k) bad |= pg[k] < 0 || pg[k] >= a.P;
      }
    }
  }
  const bool wave_bad = __any(bad);
  if (lane == 0) s.bad[w] = wave_bad ? 1 : 0;
  __syncthreads();
  if (tid == 0) {
    int code = err;
    if (code == 0)
      for (int i = 0; i < kPrepWaves; ++i)
        if (s.bad[i]) code = HSTU_DEV_BAD_PAGE;
    a.ws.hdr->status = code;
  }
}

// Workgroup 1: the attention work list and the per-entry tables, built at
// the same time as workgroup 0 validates the metadata.  Its own checks only
// keep its writes in bounds (offsets and history lengths that workgroup 0
// rejects make it stop); its result goes to the header's wl_status.  The
// scans run in wave 0; the candidate counts and the item records use every
// wave.
__device__ void work_list(const PrepArgs& a, PrepShared& s) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  WsHeader* hdr = a.ws.hdr;
  const int B = a.B, H = a.H;
  constexpr int kBudgetLo = kMinWeight * kMinSteps, kBudgetHi = kMaxWeight * kCapSteps;
  auto chunk_steps = [](int budget, int weight) { return min(kCapSteps, max(kMinSteps, budget / weight)); };
  const int64_t target = a.target_items;
  int64_t b_lo = kBudgetHi, b_hi = kBudgetHi;

  // 1.-2. checks, q-block entries per user, each entry's steps and weight
  //       (parked in qbn) and the total cost hs = H * sum_e steps_e * w_e
  if (w == 0) {
    const int err = check_offsets(a, s, lane);
    int nqb = 0;
    int64_t part = 0;
    if (err == 0) {
      for (int u0 = 0; u0 < B; u0 += kWave) {
        const int u = u0 + lane;
        const int n = u < B ? s.off[u + 1] - s.off[u] : 0;
        const int nq = (n + kQB - 1) / kQB;
        int tot;
        const int ex = nqb + wave_excl_scan(nq, lane, &tot);
        if (u < B) s.qbb[u] = ex;
        nqb += tot;
        const int c = u < B ? s.hist[u] : 0;
        for (int qb = 0; qb < nq; ++qb) {
          const int64_t keys = static_cast<int64_t>(c) + min(n, (qb + 1) * kQB);
          const int steps = static_cast<int>(min<int64_t>((keys + kStepKeys - 1) / kStepKeys, kStepMask));
          const int wt = step_weight((min(kQB, n - qb * kQB) + 15) / 16);
          s.qbn[ex + qb] = steps | (wt << kWShift);
          s.qbu[ex + qb] = u;
          part += static_cast<int64_t>(steps) * wt;
        }
      }
    }
    const int64_t hs = wave_sum(part) * H;
    if (lane == 0) {
      s.qbb[B] = nqb;
      s.nqb = nqb;
      s.err = err;
    }
    // 3. the window of the item budget (see the top of this file): with
    //    S = hs an entry gets at least steps_e * w_e / budget chunks and,
    //    while no chunk sits at its cap, fewer than steps_e * w_e /
    //    (budget - w_max) + 1, so the smallest fitting budget lies in
    //    [S / target, S / (target - H * nqb) + w_max]
    //    When the entries alone already number more than the workgroups
    //    (H * nqb >= target), the item target becomes target + H * nqb
    //    rounded up to a whole multiple of target: the heavy entries are
    //    still cut, and the attention's dynamic fetch spreads the items
    //    (without this, one workgroup would carry a whole long causal q-block
    //    while the others idle).  The rounding gives every workgroup about
    //    the same number of items: with, say, 2.1 items per workgroup a
    //    tenth of them run a third item while the rest idle (full-recompute
    //    attention 113 -> 98 us at 16,622 rows).  Either way the chosen
    //    budget keeps the item count at most that target, which is within
    //    the workspace's item capacity.
    const int64_t slack = static_cast<int64_t>(H) * nqb;
    const int64_t tgt = item_target(target, slack);
    if (err == 0) {
      b_lo = min<int64_t>(kBudgetHi, max<int64_t>(kBudgetLo, ceil_div(hs, tgt)));
      b_hi = min<int64_t>(kBudgetHi, max(b_lo, ceil_div(hs, tgt - slack) + kMaxWeight));
    }
    if (lane == 0) {
      s.b_lo = static_cast<int32_t>(b_lo);
      s.b_hi = static_cast<int32_t>(b_hi);
    }
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
  const int nqb = s.nqb;
  b_lo = s.b_lo;
  b_hi = s.b_hi;

  //    kCand budgets spread over the window are counted at once, and the
  //    smallest that fits the target is taken (the top one when none does,
  //    which can only happen through the cap)
  const int k = tid % kCand, sl = tid / kCand;
  const int bud = static_cast<int>(k == kCand - 1 ? b_hi : b_lo + (b_hi - b_lo) * k / (kCand - 1));
  {
    int cnt = 0;
    for (int e = sl; e < nqb; e += kCandSlices) {
      const int v = s.qbn[e];
      const int steps = v & kStepMask, wt = v >> kWShift;
      const int L = chunk_steps(bud, wt);
      cnt = min(cnt + (steps + L - 1) / L, 1 << 24);   // far above any target; sums stay in int32
    }
    cnt += __shfl_xor(cnt, 16, kWave);
    cnt += __shfl_xor(cnt, 32, kWave);
    if (lane < kCand) s.cnt[w][lane] = cnt;
  }
  __syncthreads();

  // 4. chunks per entry and first item of each entry (wave 0)
  if (w == 0) {
    int j = kCand - 1;
    if (lane < kCand) {
      int64_t c = 0;
      for (int i = 0; i < kPrepWaves; ++i) c += s.cnt[i][lane];
      if (c * H <= item_target(target, static_cast<int64_t>(H) * nqb))
        j = lane;
    }
    const uint64_t fits = __ballot(j == lane && lane < kCand);
    const int jj = fits ? __builtin_ctzll(fits) : kCand - 1;
    const int budget = __shfl(bud, jj, kWave);       // lanes 0..15 hold the candidates in order
    // Chunks per entry, and the order of the work list.  When the items
    // outnumber the target (the workgroups; the rest are fetched by
    // whichever workgroup finishes first) the entries go by the cost of one
    // of their chunks, highest first, in 64 classes of budget / 64 (a
    // counting sort; the order inside a class is whichever the LDS atomics
    // give), so the cheapest chunks fill the end of the launch
    // (longest-first scheduling); otherwise in entry order.  An entry's
    // items stay together, heads then chunks, as the norm kernel reads
    // them; which workgroup runs an item does not change its result.
    // qbf ends up holding the first item of the k-th entry of the list.
    static_assert(kPrepWaves * kCand == kWave, "one class counter per lane in cnt");
    int* cls_n = &s.cnt[0][0];                       // 64 class counters (the search is done with cnt)
    cls_n[lane] = 0;
    int64_t all_items = 0;
    for (int e0 = 0; e0 < nqb; e0 += kWave) {
      const int e = e0 + lane;
      int64_t ni = 0;
      if (e < nqb) {
        const int v = s.qbn[e];
        const int steps = v & kStepMask, wt = v >> kWShift;
        const int L = a.inv_steps > 0 ? a.inv_steps : chunk_steps(budget, wt);
        const int nch = (steps + L - 1) / L;
        const int64_t cost = static_cast<int64_t>((steps + nch - 1) / nch) * wt;
        const int cls = kWave - 1 - static_cast<int>(min<int64_t>(kWave - 1, cost * kWave / (budget + 1)));
        s.qbn[e] = nch;
        s.qbf[e] = cls;                              // parked until the order is known
        atomicAdd(&cls_n[cls], 1);
        ni = static_cast<int64_t>(nch) * H;
      }
      all_items += wave_sum(ni);
    }
    if (all_items > target) {
      int tot;
      const int start = wave_excl_scan(cls_n[lane], lane, &tot);   // class 0 (the costliest) first
      cls_n[lane] = start;
      for (int e0 = 0; e0 < nqb; e0 += kWave) {
        const int e = e0 + lane;
        if (e < nqb) s.ord[atomicAdd(&cls_n[s.qbf[e]], 1)] = e;
      }
    } else {
      for (int e = lane; e < nqb; e += kWave) s.ord[e] = e;
    }
    int64_t n_items = 0;
    for (int k0 = 0; k0 < nqb; k0 += kWave) {
      const int k = k0 + lane;
      const int e = k < nqb ? s.ord[k] : 0;
      const int64_t ni = k < nqb ? static_cast<int64_t>(s.qbn[e]) * H : 0;
      int64_t tot;
      const int64_t ex = n_items + wave_excl_scan(ni, lane, &tot);
      if (k < nqb) {
        const int32_t first = static_cast<int32_t>(min<int64_t>(ex, a.item_cap));
        s.qbf[k] = first;
        a.ws.qb_first[e] = first;
      }
      n_items += tot;
    }
    if (lane == 0) {
      s.budget = budget;
      s.n_items = static_cast<int32_t>(min<int64_t>(n_items, static_cast<int64_t>(a.item_cap) + 1));
    }
  }
  __syncthreads();
  const int n_items = s.n_items;
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
  //    the norm kernel
  for (int e = tid; e < nqb; e += kPrepThreads) {    // (qb_first is written with the order above)
    const int u = s.qbu[e], qb = e - s.qbb[u];
    a.ws.qb_nch[e] = s.qbn[e];
    a.ws.qb_row0[e] = s.off[u] + qb * kQB;
    a.ws.qb_rows[e] = min(kQB, s.off[u + 1] - s.off[u] - qb * kQB);
  }
  // thread t writes the contiguous items [t*m, (t+1)*m): one binary search
  // (over the list order, in which the entries' first items increase) for
  // the entry of its first item, then a walk over the entries
  const int m = (n_items + kPrepThreads - 1) / kPrepThreads;
  const int i_beg = min(n_items, tid * m), i_end = min(n_items, i_beg + m);
  int pos = i_beg < i_end ? entry_user(s.qbf, nqb, i_beg) : 0;   // last list position whose first item <= i
  for (int i = i_beg; i < i_end; ++i) {
    while (pos + 1 < nqb && s.qbf[pos + 1] <= i) ++pos;
    const int e = s.ord[pos];
    const int u = s.qbu[e], qb = e - s.qbb[u], nch = s.qbn[e];
    const int r = i - s.qbf[pos], h = r / nch, kc = r - h * nch;
    const int n = s.off[u + 1] - s.off[u];
    const int c = s.hist[u];
    const int keys = c + min(n, (qb + 1) * kQB);
    // the entry's keys are cut into nch near-equal chunks (multiples of a
    // step); csz is at most the entry's chunk bound, so (nch - 1) * csz <
    // keys and no chunk is empty
    const int csz = a.inv_steps > 0 ? a.inv_steps * kStepKeys
                                    : ((keys + nch - 1) / nch + kStepKeys - 1) / kStepKeys * kStepKeys;
    const int k_lo = kc * csz;
    AttnItem it;
    it.a = make_int4(u, qb * kQB, h, k_lo);
    it.b = make_int4(min(keys, k_lo + csz), s.off[u], n, c);
    a.ws.items[i] = it;
  }

  if (tid == 0) {
    hdr->wl_status = 0;
    hdr->n_items = n_items;
    hdr->n_qb = nqb;
    hdr->item_budget = s.budget;
    hdr->counter = 0;
  }
}

}  // namespace

hipError_t launch_prep(const hstu_layer_desc& d, const int32_t* new_off, const int32_t* hist,
                       const int32_t* ncand, const int32_t* const* pts, int nl, const int32_t* ts_off,
                       const float* const* pbs, const float* const* tbs, const WsPtrs& ws,
                       int nqb_cap, int item_cap, int target_items, hipStream_t stream,
                       const KernelEvents& ev) {
  PrepArgs a;
  a.new_off = new_off;
  a.hist = hist;
  a.ncand = ncand;
  for (int l = 0; l < kMaxStackLayers; ++l) {
    a.pt[l] = l < nl ? pts[l] : nullptr;
    a.pb[l] = l < nl ? pbs[l] : nullptr;
    a.tb[l] = (l < nl && tbs != nullptr) ? tbs[l] : nullptr;
  }
  a.nb = d.pos_buckets;
  a.mbits = d.pos_mbits;
  a.ntsb = d.ts_buckets;
  a.nl = nl;
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
  static_assert(HSTU_INVARIANT_CHUNK_KEYS % kStepKeys == 0 && HSTU_INVARIANT_CHUNK_KEYS <= kMaxChunkKeys,
                "invariant chunks are whole steps");
  a.inv_steps = (d.flags & HSTU_FLAG_BATCH_INVARIANT) ? HSTU_INVARIANT_CHUNK_KEYS / kStepKeys : 0;
  return launch_kernel(prep_kernel, dim3(2 + nl + (d.total_new + kRowsPerWg - 1) / kRowsPerWg),
                       dim3(kPrepThreads), stream, ev, a);
}

}  // namespace hstu
