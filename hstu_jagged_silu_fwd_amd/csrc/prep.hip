// Index prep for one layer call: validates the jagged/paged metadata, maps
// rows to users, and builds the attention work list.
//
// Work decomposition: the new rows of user u are cut into q-blocks of kQB
// rows; q-block qb sees keys [0, hist + min(n, (qb+1)*kQB)) (causal).  The key
// range of every (q-block, head) is split into chunks of `chunk_keys` keys
// (fixed absolute boundaries), one work item per (user, q-block, head, chunk).
// Because the attention has no softmax, the partial outputs of the chunks of
// a row simply add; the norm kernel sums them in chunk order.
// chunk_keys = max(kMinChunk, round_up(total_keys / target_items, 64)) keeps
// the item count near target_items + H * (#q-blocks).
#include "common.h"

namespace hstu {
namespace {

constexpr int kPrepThreads = 1024;
constexpr int kMinChunk = 256;

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

__device__ void set_err(int* s_err, int code) { atomicCAS(s_err, 0, code); }

// In-place exclusive scan of v[0..n) by the whole block; returns the total.
__device__ int64_t block_scan_inplace(int32_t* v, int n, int64_t* s_tmp) {
  const int tid = threadIdx.x;
  const int seg = (n + kPrepThreads - 1) / kPrepThreads;
  const int lo = min(n, tid * seg), hi = min(n, lo + seg);
  int64_t sum = 0;
  for (int i = lo; i < hi; ++i) sum += v[i];
  s_tmp[tid] = sum;
  __syncthreads();
  for (int off = 1; off < kPrepThreads; off <<= 1) {
    const int64_t add = tid >= off ? s_tmp[tid - off] : 0;
    __syncthreads();
    s_tmp[tid] += add;
    __syncthreads();
  }
  int64_t run = s_tmp[tid] - sum;
  const int64_t total = s_tmp[kPrepThreads - 1];
  for (int i = lo; i < hi; ++i) {
    const int32_t x = v[i];
    v[i] = static_cast<int32_t>(run);
    run += x;
  }
  __syncthreads();
  return total;
}

__device__ int64_t block_sum(int64_t x, int64_t* s_tmp) {
  const int tid = threadIdx.x;
  s_tmp[tid] = x;
  __syncthreads();
  for (int off = kPrepThreads / 2; off > 0; off >>= 1) {
    if (tid < off) s_tmp[tid] += s_tmp[tid + off];
    __syncthreads();
  }
  const int64_t r = s_tmp[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kPrepThreads) void prep_kernel(PrepArgs a) {
  __shared__ int s_err;
  __shared__ int64_t s_tmp[kPrepThreads];
  const int tid = threadIdx.x;
  WsHeader* hdr = a.ws.hdr;
  if (tid == 0) s_err = 0;
  __syncthreads();

  // 1. metadata checks
  if (tid == 0 && a.B == 0 && a.T != 0) set_err(&s_err, HSTU_DEV_BAD_OFFSETS);
  for (int u = tid; u < a.B; u += kPrepThreads) {
    const int o0 = a.new_off[u], o1 = a.new_off[u + 1];
    if ((u == 0 && o0 != 0) || o1 < o0 || (u == a.B - 1 && o1 != a.T)) set_err(&s_err, HSTU_DEV_BAD_OFFSETS);
    const int c = a.hist[u];
    if (c < 0) {
      set_err(&s_err, HSTU_DEV_BAD_HIST);
    } else if (static_cast<int64_t>(c) + (o1 - o0) > static_cast<int64_t>(a.maxP) * a.ps) {
      set_err(&s_err, HSTU_DEV_CAPACITY);
    }
    if (a.ts_off != nullptr) {
      if ((u == 0 && a.ts_off[0] != 0) ||
          static_cast<int64_t>(a.ts_off[u + 1]) - a.ts_off[u] != static_cast<int64_t>(c) + (o1 - o0))
        set_err(&s_err, HSTU_DEV_BAD_TS);
    }
  }
  __syncthreads();
  if (s_err == 0) {
    for (int u = 0; u < a.B; ++u) {
      const int len = a.hist[u] + (a.new_off[u + 1] - a.new_off[u]);
      const int npg = (len + a.ps - 1) / a.ps;
      const int32_t* row = a.pt + static_cast<size_t>(u) * a.maxP;
      for (int j = tid; j < npg; j += kPrepThreads) {
        const int32_t pg = row[j];
        if (pg < 0 || pg >= a.P) set_err(&s_err, HSTU_DEV_BAD_PAGE);
      }
    }
  }
  __syncthreads();
  if (s_err != 0) {
    if (tid == 0) {
      hdr->status = s_err;
      hdr->n_items = 0;
      hdr->chunk_keys = 0;
      hdr->counter = 0;
    }
    return;
  }

  // 2. q-block entries per user
  for (int u = tid; u < a.B; u += kPrepThreads)
    a.ws.qb_base[u] = (a.new_off[u + 1] - a.new_off[u] + kQB - 1) / kQB;
  __syncthreads();
  const int64_t nqb = block_scan_inplace(a.ws.qb_base, a.B, s_tmp);
  if (tid == 0) a.ws.qb_base[a.B] = static_cast<int32_t>(nqb);

  // 3. chunk size from the total key work
  int64_t local = 0;
  for (int u = 0; u < a.B; ++u) {
    const int n = a.new_off[u + 1] - a.new_off[u];
    const int c = a.hist[u];
    const int nq = (n + kQB - 1) / kQB;
    for (int qb = tid; qb < nq; qb += kPrepThreads) local += c + min(n, (qb + 1) * kQB);
  }
  const int64_t total = block_sum(local, s_tmp) * a.H;
  int64_t ck = (total + a.target_items - 1) / a.target_items;
  ck = (ck + 63) / 64 * 64;
  if (ck < kMinChunk) ck = kMinChunk;
  if (ck > (1 << 30)) ck = 1 << 30;

  // 4. chunks per entry, then first item of each entry
  for (int u = 0; u < a.B; ++u) {
    const int n = a.new_off[u + 1] - a.new_off[u];
    const int c = a.hist[u];
    const int nq = (n + kQB - 1) / kQB;
    const int base = a.ws.qb_base[u];
    for (int qb = tid; qb < nq; qb += kPrepThreads) {
      const int64_t keys = c + min(n, (qb + 1) * kQB);
      const int nch = static_cast<int>((keys + ck - 1) / ck);
      a.ws.qb_nch[base + qb] = nch;
      a.ws.qb_first[base + qb] = nch * a.H;
    }
  }
  __syncthreads();
  const int64_t n_items = block_scan_inplace(a.ws.qb_first, static_cast<int>(nqb), s_tmp);
  if (n_items > a.item_cap) {
    if (tid == 0) {
      hdr->status = HSTU_DEV_CAPACITY;
      hdr->n_items = 0;
      hdr->chunk_keys = 0;
      hdr->counter = 0;
    }
    return;
  }

  // 5. the work list
  for (int u = 0; u < a.B; ++u) {
    const int n = a.new_off[u + 1] - a.new_off[u];
    const int nq = (n + kQB - 1) / kQB;
    const int base = a.ws.qb_base[u];
    for (int qb = tid; qb < nq; qb += kPrepThreads) {
      const int f = a.ws.qb_first[base + qb];
      const int nch = a.ws.qb_nch[base + qb];
      for (int h = 0; h < a.H; ++h)
        for (int kc = 0; kc < nch; ++kc) a.ws.items[f + h * nch + kc] = make_int4(u, qb, h, kc);
    }
  }

  // 6. row -> user
  for (int r = tid; r < a.T; r += kPrepThreads) a.ws.row_user[r] = row_to_user(a.new_off, a.B, r);

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
  prep_kernel<<<1, kPrepThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace hstu
