// Paged KV cache manager: lookup, page allocation and least-recently-used
// eviction of users over the paged pool (NVIDIA blog "Deploying an HSTU
// generative recommender with NVIDIA Dynamo-Triton", section "Why serving
// large sequential recommenders is hard": a paged KV data table with lookup,
// allocation, append and eviction, old users evicted LRU-like when GPU cache
// space runs short), and the device builder of a batch's page tables.
//
// Host side: users live in slots; a doubly linked list over the slots keeps
// the recency order (head = most recent), a hash map finds a user's slot,
// and free pages and free slots are stacks.  A plan first checks that the
// batch fits (free resources plus everything held by users outside the
// batch), so that it either succeeds or changes nothing.
#include <algorithm>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include <hip/hip_runtime.h>

#include "hstu_kvcache.h"

struct hstu_kvcache {
  int32_t L = 0, ps = 0, maxP = 0, max_users = 0;
  int64_t P = 0;
  std::vector<int64_t> slot_user;    // user id of each slot (-1: free)
  std::vector<int32_t> slot_len;     // cached tokens
  std::vector<int32_t> slot_npages;  // pages held per layer
  std::vector<int32_t> pages;        // [max_users][L][maxP] page ids (host mirror of the directory)
  std::vector<int32_t> prev, next;   // recency list over cached slots
  int32_t mru = -1, lru = -1;
  std::unordered_map<int64_t, int32_t> index;
  std::vector<int32_t> free_slots;   // stacks: back() is taken first
  std::vector<int32_t> free_pages;
  int64_t held = 0;                  // pages held by cached users (all layers)

  int32_t* row(int32_t slot, int32_t layer) {
    return pages.data() + (static_cast<size_t>(slot) * L + layer) * maxP;
  }
  void unlink(int32_t s) {
    if (prev[s] >= 0) next[prev[s]] = next[s]; else if (mru == s) mru = next[s];
    if (next[s] >= 0) prev[next[s]] = prev[s]; else if (lru == s) lru = prev[s];
    prev[s] = next[s] = -1;
  }
  void push_mru(int32_t s) {
    prev[s] = -1;
    next[s] = mru;
    if (mru >= 0) prev[mru] = s;
    mru = s;
    if (lru < 0) lru = s;
  }
  void evict_slot(int32_t s) {
    for (int32_t l = 0; l < L; ++l) {
      const int32_t* r = row(s, l);
      for (int32_t i = 0; i < slot_npages[s]; ++i) free_pages.push_back(r[i]);
    }
    held -= static_cast<int64_t>(L) * slot_npages[s];
    index.erase(slot_user[s]);
    unlink(s);
    slot_user[s] = -1;
    slot_len[s] = 0;
    slot_npages[s] = 0;
    free_slots.push_back(s);
  }
};

namespace {

int32_t pages_for(int64_t tokens, int32_t ps) { return static_cast<int32_t>((tokens + ps - 1) / ps); }

__global__ void dir_scatter_kernel(int32_t* dir, int32_t L, int32_t max_users, int32_t maxP,
                                   const hstu_kv_update* up, int32_t n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const hstu_kv_update u = up[i];
  if (u.slot < 0 || u.slot >= max_users || u.layer < 0 || u.layer >= L || u.page_index < 0 ||
      u.page_index >= maxP)
    return;                                         // not from a plan of these sizes: ignored
  dir[(static_cast<size_t>(u.slot) * L + u.layer) * maxP + u.page_index] = u.page_id;
}

// One workgroup per (layer, batch row); threads walk the row in 16-byte runs
// where the row length allows.
__global__ void dir_gather_kernel(const int32_t* dir, int32_t L, int32_t max_users, int32_t maxP,
                                  const int32_t* slots, int32_t B, int32_t* tables) {
  const int l = blockIdx.x / B, b = blockIdx.x % B;
  const int32_t slot = slots[b];
  int32_t* dst = tables + (static_cast<size_t>(l) * B + b) * maxP;
  if (slot < 0 || slot >= max_users) {              // not from a plan: an empty row
    for (int j = threadIdx.x; j < maxP; j += blockDim.x) dst[j] = -1;
    return;
  }
  const int32_t* src = dir + (static_cast<size_t>(slot) * L + l) * maxP;
  if ((maxP & 3) == 0) {
    const int4* s4 = reinterpret_cast<const int4*>(src);
    int4* d4 = reinterpret_cast<int4*>(dst);
    for (int j = threadIdx.x; j < maxP / 4; j += blockDim.x) d4[j] = s4[j];
  } else {
    for (int j = threadIdx.x; j < maxP; j += blockDim.x) dst[j] = src[j];
  }
}

}  // namespace

extern "C" {

hstu_kvcache* hstu_kvcache_create(int32_t num_layers, int64_t num_pages, int32_t page_size,
                                  int32_t max_pages_per_user, int32_t max_users) {
  if (num_layers < 1 || num_pages < 1 || num_pages >= (int64_t{1} << 31) || page_size < 1 ||
      (page_size & (page_size - 1)) != 0 || max_pages_per_user < 1 || max_users < 1)
    return nullptr;
  const int64_t dir = static_cast<int64_t>(max_users) * num_layers * max_pages_per_user;
  if (dir >= (int64_t{1} << 40)) return nullptr;
  hstu_kvcache* c = new (std::nothrow) hstu_kvcache;
  if (c == nullptr) return nullptr;
  try {
    c->L = num_layers;
    c->P = num_pages;
    c->ps = page_size;
    c->maxP = max_pages_per_user;
    c->max_users = max_users;
    c->slot_user.assign(max_users, -1);
    c->slot_len.assign(max_users, 0);
    c->slot_npages.assign(max_users, 0);
    c->pages.assign(static_cast<size_t>(dir), -1);
    c->prev.assign(max_users, -1);
    c->next.assign(max_users, -1);
    c->free_slots.reserve(max_users);
    for (int32_t s = max_users - 1; s >= 0; --s) c->free_slots.push_back(s);
    c->free_pages.reserve(static_cast<size_t>(num_pages));
    for (int64_t p = num_pages - 1; p >= 0; --p) c->free_pages.push_back(static_cast<int32_t>(p));
    c->index.reserve(static_cast<size_t>(max_users) * 2);
  } catch (...) {
    delete c;
    return nullptr;
  }
  return c;
}

void hstu_kvcache_destroy(hstu_kvcache* cache) { delete cache; }

int64_t hstu_kvcache_directory_elems(const hstu_kvcache* c) {
  return c == nullptr ? 0 : static_cast<int64_t>(c->max_users) * c->L * c->maxP;
}

hstu_kv_status hstu_kvcache_plan(hstu_kvcache* c, int32_t B, const int64_t* user_ids,
                                 const int32_t* n_new, int32_t* hist_len, int32_t* slots,
                                 hstu_kv_update* updates, int32_t update_cap, int32_t* n_updates,
                                 int64_t* evicted, int32_t evicted_cap, int32_t* n_evicted) {
  if (c == nullptr || B < 0 || n_updates == nullptr || n_evicted == nullptr || update_cap < 0 ||
      evicted_cap < 0 || (evicted_cap > 0 && evicted == nullptr))
    return HSTU_KV_INVALID_ARG;
  if (B > 0 && (user_ids == nullptr || n_new == nullptr || hist_len == nullptr || slots == nullptr))
    return HSTU_KV_INVALID_ARG;
  if (update_cap > 0 && updates == nullptr) return HSTU_KV_INVALID_ARG;
  *n_updates = 0;
  *n_evicted = 0;

  // 1.-2. lookup and what the batch needs (nothing changes before it fits)
  std::vector<int32_t> bslot(B), hist(B), need(B);
  std::unordered_set<int64_t> seen;
  seen.reserve(static_cast<size_t>(B) * 2);
  int64_t need_pages = 0, batch_held = 0;
  int32_t misses = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (n_new[b] < 0 || !seen.insert(user_ids[b]).second) return HSTU_KV_INVALID_ARG;
    const auto it = c->index.find(user_ids[b]);
    const int32_t s = it == c->index.end() ? -1 : it->second;
    bslot[b] = s;
    hist[b] = s >= 0 ? c->slot_len[s] : 0;
    const int64_t tokens = static_cast<int64_t>(hist[b]) + n_new[b];
    if (tokens > static_cast<int64_t>(c->maxP) * c->ps) return HSTU_KV_TOO_LONG;
    const int32_t held = s >= 0 ? c->slot_npages[s] : 0;
    need[b] = pages_for(tokens, c->ps) - held;
    need_pages += static_cast<int64_t>(c->L) * need[b];
    if (s >= 0) batch_held += static_cast<int64_t>(c->L) * held;
    else ++misses;
  }
  if (need_pages > update_cap) return HSTU_KV_CAPACITY;
  const int64_t hits = B - misses;
  const int64_t free_after = static_cast<int64_t>(c->free_pages.size()) + (c->held - batch_held);
  const int64_t slots_after = static_cast<int64_t>(c->free_slots.size()) +
                              (static_cast<int64_t>(c->index.size()) - hits);
  if (free_after < need_pages || slots_after < misses) return HSTU_KV_FULL;

  // 3. evict least recently used users outside the batch until the batch fits
  std::vector<char> in_batch(c->max_users, 0);
  for (int32_t b = 0; b < B; ++b)
    if (bslot[b] >= 0) in_batch[bslot[b]] = 1;
  int32_t ne = 0;
  int32_t cur = c->lru;
  while (static_cast<int64_t>(c->free_pages.size()) < need_pages ||
         static_cast<int64_t>(c->free_slots.size()) < misses) {
    while (cur >= 0 && in_batch[cur]) cur = c->prev[cur];
    if (cur < 0) return HSTU_KV_FULL;              // unreachable after the check above
    const int32_t victim = cur;
    cur = c->prev[cur];
    if (ne < evicted_cap) evicted[ne] = c->slot_user[victim];
    ++ne;
    c->evict_slot(victim);
  }
  *n_evicted = std::min(ne, evicted_cap);

  // 4. slots and pages, in batch order
  int32_t nu = 0;
  for (int32_t b = 0; b < B; ++b) {
    int32_t s = bslot[b];
    if (s < 0) {
      s = c->free_slots.back();
      c->free_slots.pop_back();
      c->slot_user[s] = user_ids[b];
      c->slot_len[s] = 0;
      c->slot_npages[s] = 0;
      c->index.emplace(user_ids[b], s);
    }
    const int32_t held = c->slot_npages[s];
    for (int32_t l = 0; l < c->L; ++l) {
      int32_t* r = c->row(s, l);
      for (int32_t i = held; i < held + need[b]; ++i) {
        const int32_t p = c->free_pages.back();
        c->free_pages.pop_back();
        r[i] = p;
        updates[nu++] = hstu_kv_update{s, l, i, p};
      }
    }
    c->slot_npages[s] = held + need[b];
    c->held += static_cast<int64_t>(c->L) * need[b];
    c->slot_len[s] = hist[b] + n_new[b];
    hist_len[b] = hist[b];
    slots[b] = s;
    bslot[b] = s;
  }
  *n_updates = nu;

  // 5. recency: the batch in order, the last user most recent
  for (int32_t b = 0; b < B; ++b) {
    const int32_t s = bslot[b];
    if (c->prev[s] >= 0 || c->next[s] >= 0 || c->mru == s) c->unlink(s);
    c->push_mru(s);
  }
  return HSTU_KV_OK;
}

hstu_kv_status hstu_kvcache_lookup(const hstu_kvcache* c, int32_t B, const int64_t* user_ids,
                                   int32_t* cached_len) {
  if (c == nullptr || B < 0 || (B > 0 && (user_ids == nullptr || cached_len == nullptr)))
    return HSTU_KV_INVALID_ARG;
  for (int32_t b = 0; b < B; ++b) {
    const auto it = c->index.find(user_ids[b]);
    cached_len[b] = it == c->index.end() ? -1 : c->slot_len[it->second];
  }
  return HSTU_KV_OK;
}

hstu_kv_status hstu_kvcache_evict(hstu_kvcache* c, int64_t user_id, int32_t* found) {
  if (c == nullptr || found == nullptr) return HSTU_KV_INVALID_ARG;
  const auto it = c->index.find(user_id);
  *found = it == c->index.end() ? 0 : 1;
  if (*found) c->evict_slot(it->second);
  return HSTU_KV_OK;
}

hstu_kv_status hstu_kvcache_stats(const hstu_kvcache* c, int64_t* free_pages, int32_t* cached_users) {
  if (c == nullptr || free_pages == nullptr || cached_users == nullptr) return HSTU_KV_INVALID_ARG;
  *free_pages = static_cast<int64_t>(c->free_pages.size());
  *cached_users = static_cast<int32_t>(c->index.size());
  return HSTU_KV_OK;
}

hstu_kv_status hstu_kv_tables_build(int32_t* directory, int32_t num_layers, int32_t max_users,
                                    int32_t max_pages, const hstu_kv_update* updates,
                                    int32_t n_updates, const int32_t* slots, int32_t B,
                                    int32_t* tables, void* hip_stream) {
  if (directory == nullptr || num_layers < 1 || max_users < 1 || max_pages < 1 || n_updates < 0 ||
      B < 0 || (n_updates > 0 && updates == nullptr) || (B > 0 && (slots == nullptr || tables == nullptr)))
    return HSTU_KV_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (n_updates > 0) {
    dir_scatter_kernel<<<(n_updates + 255) / 256, 256, 0, st>>>(directory, num_layers, max_users, max_pages,
                                                                updates, n_updates);
    if (hipGetLastError() != hipSuccess) return HSTU_KV_HIP;
  }
  if (B > 0) {
    dir_gather_kernel<<<num_layers * B, 256, 0, st>>>(directory, num_layers, max_users, max_pages, slots, B,
                                                      tables);
    if (hipGetLastError() != hipSuccess) return HSTU_KV_HIP;
  }
  return HSTU_KV_OK;
}

}  // extern "C"
