// Paged KV cache manager: lookup, page allocation and least-recently-used
// eviction of users over the paged pool, with an optional host tier that
// evicted users are offloaded to and onboarded back from (NVIDIA blog
// "Deploying an HSTU generative recommender with NVIDIA Dynamo-Triton",
// section "Why serving large sequential recommenders is hard": a paged KV
// data table with lookup, allocation, append and eviction, old users evicted
// LRU-like when GPU cache space runs short, host storage as a further tier
// with onboard and offload operations), and the device side: the page-table
// builder of a batch and the page copies between the pool and the host tier.
//
// Host side: GPU-cached users live in slots; a doubly linked list over the
// slots keeps their recency order (head = most recent), a hash map finds a
// user's slot, and free pages and free slots are stacks.  Host-cached users
// are hash-map entries with their own recency list and host free-page stack.
// A plan first checks that the batch fits (free resources plus everything
// held by GPU-cached users outside the batch), so that it either succeeds or
// changes nothing.
#include <algorithm>
#include <list>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include <hip/hip_runtime.h>

#include "hstu_kvcache.h"

namespace {

struct HostUser {
  int32_t len = 0, npages = 0;          // tokens; pages per layer
  std::vector<int32_t> pages;           // [L][npages] host page ids
  std::list<int64_t>::iterator pos;     // place in the host recency list
};

}  // namespace

struct hstu_kvcache {
  int32_t L = 0, ps = 0, maxP = 0, max_users = 0;
  int64_t P = 0, PH = 0;
  std::vector<int64_t> slot_user;    // user id of each slot (-1: free)
  std::vector<int32_t> slot_len;     // cached tokens
  std::vector<int32_t> slot_npages;  // pages held per layer
  // page ids, [max_users][maxP][L]: the host mirror of the directory, with
  // a user's layers side by side so that a plan touches few memory pages
  std::vector<int32_t> pages;
  std::vector<int32_t> prev, next;   // recency list over GPU-cached slots
  int32_t mru = -1, lru = -1;
  std::unordered_map<int64_t, int32_t> index;
  std::vector<int32_t> free_slots;   // stacks: back() is taken first
  std::vector<int32_t> free_pages;
  int64_t held = 0;                  // GPU pages held by cached users (all layers)
  std::vector<int32_t> pins;         // pin count of each slot (pinned users are never evicted)
  std::unordered_set<int32_t> pinned;   // slots with pins > 0
  // host tier
  std::unordered_map<int64_t, HostUser> host;
  std::list<int64_t> host_order;     // front = most recent
  std::vector<int32_t> host_free;

  int32_t& page(int32_t slot, int32_t layer, int32_t i) {
    return pages[(static_cast<size_t>(slot) * maxP + i) * L + layer];
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
  // frees a GPU-cached user's pages and slot (its data is gone or offloaded)
  void release_slot(int32_t s) {
    for (int32_t l = 0; l < L; ++l)                // layer by layer, in page-index order
      for (int32_t i = 0; i < slot_npages[s]; ++i) free_pages.push_back(page(s, l, i));
    held -= static_cast<int64_t>(L) * slot_npages[s];
    index.erase(slot_user[s]);
    unlink(s);
    slot_user[s] = -1;
    slot_len[s] = 0;
    slot_npages[s] = 0;
    pins[s] = 0;                                   // (callers never release a pinned slot)
    pinned.erase(s);
    free_slots.push_back(s);
  }
  void drop_host(int64_t uid) {
    auto it = host.find(uid);
    for (int32_t p : it->second.pages) host_free.push_back(p);
    host_order.erase(it->second.pos);
    host.erase(it);
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

// One workgroup per copy: the K page, then the V page, in 16-byte pieces,
// kCopyUnroll loads in flight per thread (host memory is far: the loads of
// a round go out before any store).
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

__device__ void copy_bytes(char* dst, const char* src, int64_t bytes) {
  const int64_t n16 = bytes / 16;
  const int4* s = reinterpret_cast<const int4*>(src);
  int4* d = reinterpret_cast<int4*>(dst);
  for (int64_t i0 = threadIdx.x; i0 < n16; i0 += kCopyThreads * kCopyUnroll) {
    int4 v[kCopyUnroll];
#pragma unroll
    for (int j = 0; j < kCopyUnroll; ++j) {
      const int64_t i = i0 + j * kCopyThreads;
      if (i < n16) v[j] = s[i];
    }
#pragma unroll
    for (int j = 0; j < kCopyUnroll; ++j) {
      const int64_t i = i0 + j * kCopyThreads;
      if (i < n16) d[i] = v[j];
    }
  }
}

__global__ void page_copy_kernel(char* k_pool, char* v_pool, char* host_k, char* host_v, int64_t pbk,
                                 int64_t pbv, int64_t P, int64_t PH, const hstu_kv_copy* ops) {
  const hstu_kv_copy op = ops[blockIdx.x];
  if (op.gpu_page < 0 || op.gpu_page >= P || op.host_page < 0 || op.host_page >= PH) return;
  char* gk = k_pool + op.gpu_page * pbk;
  char* gv = v_pool + op.gpu_page * pbv;
  char* hk = host_k + op.host_page * pbk;
  char* hv = host_v + op.host_page * pbv;
  if (op.onboard) {
    copy_bytes(gk, hk, pbk);
    copy_bytes(gv, hv, pbv);
  } else {
    copy_bytes(hk, gk, pbk);
    copy_bytes(hv, gv, pbv);
  }
}

}  // namespace

extern "C" {

hstu_kvcache* hstu_kvcache_create(int32_t num_layers, int64_t num_pages, int32_t page_size,
                                  int32_t max_pages_per_user, int32_t max_users, int64_t host_pages) {
  if (num_layers < 1 || num_pages < 1 || num_pages >= (int64_t{1} << 31) || page_size < 1 ||
      (page_size & (page_size - 1)) != 0 || max_pages_per_user < 1 || max_users < 1 || host_pages < 0 ||
      host_pages >= (int64_t{1} << 31))
    return nullptr;
  const int64_t dir = static_cast<int64_t>(max_users) * num_layers * max_pages_per_user;
  if (dir >= (int64_t{1} << 40)) return nullptr;
  hstu_kvcache* c = new (std::nothrow) hstu_kvcache;
  if (c == nullptr) return nullptr;
  try {
    c->L = num_layers;
    c->P = num_pages;
    c->PH = host_pages;
    c->ps = page_size;
    c->maxP = max_pages_per_user;
    c->max_users = max_users;
    c->slot_user.assign(max_users, -1);
    c->slot_len.assign(max_users, 0);
    c->slot_npages.assign(max_users, 0);
    c->pages.assign(static_cast<size_t>(dir), -1);
    c->prev.assign(max_users, -1);
    c->next.assign(max_users, -1);
    c->pins.assign(max_users, 0);
    c->free_slots.reserve(max_users);
    for (int32_t s = max_users - 1; s >= 0; --s) c->free_slots.push_back(s);
    c->free_pages.reserve(static_cast<size_t>(num_pages));
    for (int64_t p = num_pages - 1; p >= 0; --p) c->free_pages.push_back(static_cast<int32_t>(p));
    c->host_free.reserve(static_cast<size_t>(host_pages));
    for (int64_t p = host_pages - 1; p >= 0; --p) c->host_free.push_back(static_cast<int32_t>(p));
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
                                 int64_t* evicted, int32_t evicted_cap, int32_t* n_evicted,
                                 hstu_kv_copy* copies, int32_t copy_cap, int32_t* n_copies) {
  if (c == nullptr || B < 0 || n_updates == nullptr || n_evicted == nullptr || n_copies == nullptr ||
      update_cap < 0 || evicted_cap < 0 || copy_cap < 0 || (evicted_cap > 0 && evicted == nullptr) ||
      (copy_cap > 0 && copies == nullptr))
    return HSTU_KV_INVALID_ARG;
  if (B > 0 && (user_ids == nullptr || n_new == nullptr || hist_len == nullptr || slots == nullptr))
    return HSTU_KV_INVALID_ARG;
  if (update_cap > 0 && updates == nullptr) return HSTU_KV_INVALID_ARG;
  *n_updates = 0;
  *n_evicted = 0;
  *n_copies = 0;

  // 1.-2. lookup and what the batch needs (nothing changes before it fits)
  std::vector<int32_t> bslot(B), hist(B), need(B);
  std::vector<char> from_host(B, 0);
  std::unordered_set<int64_t> seen;
  seen.reserve(static_cast<size_t>(B) * 2);
  int64_t need_pages = 0, batch_held = 0, onboard = 0;
  int32_t slot_need = 0, gpu_hits = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (n_new[b] < 0 || !seen.insert(user_ids[b]).second) return HSTU_KV_INVALID_ARG;
    const auto it = c->index.find(user_ids[b]);
    const int32_t s = it == c->index.end() ? -1 : it->second;
    if (s >= 0 && c->pins[s] > 0) return HSTU_KV_PINNED;   // its earlier batch is still in flight
    bslot[b] = s;
    hist[b] = 0;
    if (s >= 0) {
      hist[b] = c->slot_len[s];
      ++gpu_hits;
    } else {
      const auto h = c->host.find(user_ids[b]);
      if (h != c->host.end()) {
        hist[b] = h->second.len;
        from_host[b] = 1;
        onboard += static_cast<int64_t>(c->L) * h->second.npages;
      }
      ++slot_need;
    }
    const int64_t tokens = static_cast<int64_t>(hist[b]) + n_new[b];
    if (tokens > static_cast<int64_t>(c->maxP) * c->ps) return HSTU_KV_TOO_LONG;
    const int32_t held = s >= 0 ? c->slot_npages[s] : 0;
    need[b] = pages_for(tokens, c->ps) - held;
    need_pages += static_cast<int64_t>(c->L) * need[b];
    if (s >= 0) batch_held += static_cast<int64_t>(c->L) * held;
  }
  if (need_pages > update_cap) return HSTU_KV_CAPACITY;
  if (c->PH > 0 && onboard + (c->held - batch_held) > copy_cap) return HSTU_KV_CAPACITY;
  std::vector<char> in_batch(c->max_users, 0);
  for (int32_t b = 0; b < B; ++b)
    if (bslot[b] >= 0) in_batch[bslot[b]] = 1;
  // pinned users outside the batch keep their pages and slots
  int64_t pinned_pages = 0, pinned_users = 0;
  for (const int32_t s : c->pinned)
    if (!in_batch[s]) {
      pinned_pages += static_cast<int64_t>(c->L) * c->slot_npages[s];
      ++pinned_users;
    }
  const int64_t free_after =
      static_cast<int64_t>(c->free_pages.size()) + (c->held - batch_held - pinned_pages);
  const int64_t slots_after = static_cast<int64_t>(c->free_slots.size()) +
                              (static_cast<int64_t>(c->index.size()) - gpu_hits - pinned_users);
  if (free_after < need_pages || slots_after < slot_need) return HSTU_KV_FULL;

  // 3. evict least recently used GPU-cached users outside the batch (and not
  //    pinned) until the batch fits, offloading them to the host tier where
  //    they fit
  int32_t ne = 0, nc = 0;
  int32_t cur = c->lru;
  std::unordered_set<int64_t> offloaded;   // entered the host tier in this plan: their
                                           // copies are pending, so they are not dropped
  while (static_cast<int64_t>(c->free_pages.size()) < need_pages ||
         static_cast<int64_t>(c->free_slots.size()) < slot_need) {
    while (cur >= 0 && (in_batch[cur] || c->pins[cur] > 0)) cur = c->prev[cur];
    if (cur < 0) return HSTU_KV_FULL;              // unreachable after the check above
    const int32_t victim = cur;
    cur = c->prev[cur];
    const int64_t uid = c->slot_user[victim];
    if (ne < evicted_cap) evicted[ne] = uid;
    ++ne;
    const int64_t vp = static_cast<int64_t>(c->L) * c->slot_npages[victim];
    if (c->PH > 0 && vp <= c->PH) {
      // make room in the host tier: drop its least recently used users that
      // are neither in the batch nor offloaded by this plan
      auto h = c->host_order.end();
      while (static_cast<int64_t>(c->host_free.size()) < vp && h != c->host_order.begin()) {
        --h;
        const int64_t hu = *h;
        if (seen.count(hu) || offloaded.count(hu)) continue;
        ++h;                                        // keep the iterator valid across the erase
        c->drop_host(hu);
      }
      if (static_cast<int64_t>(c->host_free.size()) >= vp) {
        HostUser e;
        e.len = c->slot_len[victim];
        e.npages = c->slot_npages[victim];
        e.pages.reserve(static_cast<size_t>(vp));
        for (int32_t l = 0; l < c->L; ++l) {
          for (int32_t i = 0; i < e.npages; ++i) {
            const int32_t hp = c->host_free.back();
            c->host_free.pop_back();
            e.pages.push_back(hp);
            copies[nc++] = hstu_kv_copy{0, c->page(victim, l, i), hp, 0};
          }
        }
        c->host_order.push_front(uid);
        e.pos = c->host_order.begin();
        c->host.emplace(uid, std::move(e));
        offloaded.insert(uid);
      }
    }
    c->release_slot(victim);
  }
  *n_evicted = std::min(ne, evicted_cap);

  // 4. slots and pages, in batch order; host hits come back by onboard copies
  //    (pages come off the top of the free stack, the top first; the stack
  //    is cut back once at the end)
  int32_t nu = 0;
  std::vector<int64_t> to_free;
  const int32_t* fp = c->free_pages.data();
  size_t top = c->free_pages.size();
  for (int32_t b = 0; b < B; ++b) {
    int32_t s = bslot[b];
    const HostUser* hu = nullptr;
    if (s < 0) {
      s = c->free_slots.back();
      c->free_slots.pop_back();
      c->slot_user[s] = user_ids[b];
      c->slot_len[s] = 0;
      c->slot_npages[s] = 0;
      c->index.emplace(user_ids[b], s);
      if (from_host[b]) hu = &c->host.find(user_ids[b])->second;
    }
    const int32_t held = c->slot_npages[s];
    const int32_t nb = need[b];
    for (int32_t l = 0; l < c->L; ++l) {
      hstu_kv_update* u = updates + nu;
      for (int32_t k = 0; k < nb; ++k) {
        const int32_t pg = fp[--top];
        c->page(s, l, held + k) = pg;
        u[k] = hstu_kv_update{s, l, held + k, pg};
      }
      nu += nb;
      if (hu != nullptr)
        for (int32_t i = held; i < std::min(held + nb, hu->npages); ++i)
          copies[nc++] = hstu_kv_copy{1, c->page(s, l, i), hu->pages[static_cast<size_t>(l) * hu->npages + i], 0};
    }
    if (hu != nullptr) to_free.push_back(user_ids[b]);
    c->slot_npages[s] = held + need[b];
    c->held += static_cast<int64_t>(c->L) * need[b];
    c->slot_len[s] = hist[b] + n_new[b];
    hist_len[b] = hist[b];
    slots[b] = s;
    bslot[b] = s;
  }
  c->free_pages.resize(top);
  for (int64_t uid : to_free) c->drop_host(uid);
  *n_updates = nu;
  *n_copies = nc;

  // 5. recency: the batch in order, the last user most recent
  for (int32_t b = 0; b < B; ++b) {
    const int32_t s = bslot[b];
    if (c->prev[s] >= 0 || c->next[s] >= 0 || c->mru == s) c->unlink(s);
    c->push_mru(s);
  }
  return HSTU_KV_OK;
}

hstu_kv_status hstu_kvcache_lookup(const hstu_kvcache* c, int32_t B, const int64_t* user_ids,
                                   int32_t* cached_len, int32_t* tier) {
  if (c == nullptr || B < 0 || (B > 0 && (user_ids == nullptr || cached_len == nullptr)))
    return HSTU_KV_INVALID_ARG;
  for (int32_t b = 0; b < B; ++b) {
    const auto it = c->index.find(user_ids[b]);
    int32_t len = -1, t = 0;
    if (it != c->index.end()) {
      len = c->slot_len[it->second];
      t = 1;
    } else {
      const auto h = c->host.find(user_ids[b]);
      if (h != c->host.end()) {
        len = h->second.len;
        t = 2;
      }
    }
    cached_len[b] = len;
    if (tier != nullptr) tier[b] = t;
  }
  return HSTU_KV_OK;
}

hstu_kv_status hstu_kvcache_evict(hstu_kvcache* c, int64_t user_id, int32_t* found) {
  if (c == nullptr || found == nullptr) return HSTU_KV_INVALID_ARG;
  *found = 0;
  const auto it = c->index.find(user_id);
  if (it != c->index.end()) {
    if (c->pins[it->second] > 0) return HSTU_KV_PINNED;
    c->release_slot(it->second);
    *found = 1;
  } else if (c->host.count(user_id)) {
    c->drop_host(user_id);
    *found = 1;
  }
  return HSTU_KV_OK;
}

hstu_kv_status hstu_kvcache_pin(hstu_kvcache* c, int32_t B, const int64_t* user_ids, int32_t pin) {
  if (c == nullptr || B < 0 || (B > 0 && user_ids == nullptr)) return HSTU_KV_INVALID_ARG;
  // every check first, so that a rejected call changes nothing
  std::unordered_set<int64_t> seen;
  for (int32_t b = 0; b < B; ++b) {
    const auto it = c->index.find(user_ids[b]);
    if (it == c->index.end() || !seen.insert(user_ids[b]).second) return HSTU_KV_INVALID_ARG;
    if (pin == 0 && c->pins[it->second] == 0) return HSTU_KV_INVALID_ARG;
  }
  for (int32_t b = 0; b < B; ++b) {
    const int32_t s = c->index.find(user_ids[b])->second;
    if (pin != 0) {
      if (c->pins[s]++ == 0) c->pinned.insert(s);
    } else if (--c->pins[s] == 0) {
      c->pinned.erase(s);
    }
  }
  return HSTU_KV_OK;
}

hstu_kv_status hstu_kvcache_trim(hstu_kvcache* c, int32_t B, const int64_t* user_ids,
                                 const int32_t* n_drop) {
  if (c == nullptr || B < 0 || (B > 0 && (user_ids == nullptr || n_drop == nullptr)))
    return HSTU_KV_INVALID_ARG;
  // every check first, so that a rejected call changes nothing
  std::unordered_set<int64_t> seen;
  for (int32_t b = 0; b < B; ++b) {
    const auto it = c->index.find(user_ids[b]);
    if (it == c->index.end() || !seen.insert(user_ids[b]).second) return HSTU_KV_INVALID_ARG;
    if (n_drop[b] < 0 || n_drop[b] > c->slot_len[it->second]) return HSTU_KV_INVALID_ARG;
  }
  for (int32_t b = 0; b < B; ++b)
    if (c->pins[c->index.find(user_ids[b])->second] > 0) return HSTU_KV_PINNED;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t s = c->index.find(user_ids[b])->second;
    c->slot_len[s] -= n_drop[b];
    const int32_t keep = pages_for(c->slot_len[s], c->ps);
    for (int32_t l = 0; l < c->L; ++l)
      for (int32_t i = keep; i < c->slot_npages[s]; ++i) c->free_pages.push_back(c->page(s, l, i));
    c->held -= static_cast<int64_t>(c->L) * (c->slot_npages[s] - keep);
    c->slot_npages[s] = keep;
  }
  return HSTU_KV_OK;
}

hstu_kv_status hstu_kvcache_stats(const hstu_kvcache* c, int64_t* free_pages, int32_t* cached_users,
                                  int64_t* free_host_pages, int32_t* host_users) {
  if (c == nullptr || free_pages == nullptr || cached_users == nullptr) return HSTU_KV_INVALID_ARG;
  *free_pages = static_cast<int64_t>(c->free_pages.size());
  *cached_users = static_cast<int32_t>(c->index.size());
  if (free_host_pages != nullptr) *free_host_pages = static_cast<int64_t>(c->host_free.size());
  if (host_users != nullptr) *host_users = static_cast<int32_t>(c->host.size());
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

hstu_kv_status hstu_kv_copy_pages(void* k_pool, void* v_pool, void* host_k, void* host_v,
                                  int64_t page_bytes_k, int64_t page_bytes_v, int64_t num_pages,
                                  int64_t host_pages, const hstu_kv_copy* copies, int32_t n_offload,
                                  int32_t n, void* hip_stream) {
  if (n < 0 || n_offload < 0 || n_offload > n) return HSTU_KV_INVALID_ARG;
  if (n == 0) return HSTU_KV_OK;
  if (k_pool == nullptr || v_pool == nullptr || host_k == nullptr || host_v == nullptr || copies == nullptr ||
      page_bytes_k <= 0 || page_bytes_v <= 0 || (page_bytes_k % 16) != 0 || (page_bytes_v % 16) != 0 ||
      num_pages < 1 || host_pages < 1)
    return HSTU_KV_INVALID_ARG;
  // the device's view of the pinned host tier
  void* dk = nullptr;
  void* dv = nullptr;
  if (hipHostGetDevicePointer(&dk, host_k, 0) != hipSuccess || dk == nullptr ||
      hipHostGetDevicePointer(&dv, host_v, 0) != hipSuccess || dv == nullptr)
    return HSTU_KV_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  char* kp = static_cast<char*>(k_pool);
  char* vp = static_cast<char*>(v_pool);
  if (n_offload > 0) {   // every offload reads its GPU page before any onboard writes one
    page_copy_kernel<<<n_offload, kCopyThreads, 0, st>>>(kp, vp, static_cast<char*>(dk), static_cast<char*>(dv),
                                                         page_bytes_k, page_bytes_v, num_pages, host_pages,
                                                         copies);
    if (hipGetLastError() != hipSuccess) return HSTU_KV_HIP;
  }
  if (n > n_offload) {
    page_copy_kernel<<<n - n_offload, kCopyThreads, 0, st>>>(kp, vp, static_cast<char*>(dk),
                                                             static_cast<char*>(dv), page_bytes_k, page_bytes_v,
                                                             num_pages, host_pages, copies + n_offload);
    if (hipGetLastError() != hipSuccess) return HSTU_KV_HIP;
  }
  return HSTU_KV_OK;
}

}  // extern "C"
