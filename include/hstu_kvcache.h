/*
 * hstu_kvcache.h -- C ABI of the paged KV cache manager of libhstu: lookup,
 * allocation and least-recently-used eviction of users' pages in the paged
 * GPU KV pool that the layer (include/hstu.h) reads and appends to, plus a
 * device builder of the per-layer page tables of a batch.
 *
 * Source: NVIDIA technical blog "Deploying an HSTU generative recommender
 * with NVIDIA Dynamo-Triton", section "Why serving large sequential
 * recommenders is hard": the GPU cache is a paged KV data table supporting
 * lookup, allocation, append and eviction, and when GPU cache space runs
 * short, old users are evicted under an LRU-like policy.  The exact policy
 * below (whole users evicted, least recently planned first, never a user of
 * the batch being planned, all-or-nothing plans, last-in-first-out page
 * reuse) is this library's reading of that passage.
 *
 * Model.  The cache serves L layers that share one pool of P pages of
 * page_size token slots (every layer of a user holds the same number of
 * pages, in pages distinct from every other (user, layer)).  A user is a
 * 64-bit id; a cached user occupies one of max_users slots and has c cached
 * tokens, held in ceil(c / page_size) pages per layer.
 *
 * Host tier (host_pages > 0).  The blog (same section) adds host storage as
 * a further tier of cached KV data, with onboard and offload operations.
 * Here a host page holds one (layer, pool page) worth of K and V in the
 * pool's own page layout, in caller-owned pinned host arrays; a user is
 * cached either on the GPU or on the host, never both.
 *
 * hstu_kvcache_plan(batch of B distinct users, n_new[b] new tokens each):
 *   1. lookup: a user cached on the GPU or on the host is a hit with
 *      hist_len = c, any other user a miss with hist_len = 0 (its whole
 *      sequence is then sent as new rows);
 *   2. every user needs ceil((hist_len + n_new) / page_size) GPU pages per
 *      layer (a host hit all of them, as it comes back); a miss or a host hit
 *      also needs a slot.  If the free pages and slots, plus those of every
 *      GPU-cached user outside the batch that is not pinned, cannot cover
 *      the batch, the plan fails with HSTU_KV_FULL and changes nothing;
 *   3. while pages or slots are short, the least recently used GPU-cached
 *      user outside the batch that is not pinned is evicted.  With a host tier it is offloaded
 *      when its pages fit there: host-cached users outside the batch are
 *      dropped least recently used first until they do (a user with more
 *      pages than the whole tier is dropped instead), it takes host pages off
 *      the host free stack (layer 0 first, page index order) and one offload
 *      copy {GPU page -> host page} per page is reported.  Either way its GPU
 *      pages (layer by layer, page index by page index) go onto the
 *      free-page stack and its slot onto the free-slot stack;
 *   4. users are served in batch order: a miss or host hit pops a slot; the
 *      missing pages of layer 0, then layer 1, ... are popped off the
 *      free-page stack (initially pages 0, 1, 2, ... come off first); each
 *      assignment is reported as an update record {slot, layer, page index,
 *      page id}.  A host hit's first ceil(c / page_size) pages of each layer
 *      are onboard copies {host page -> GPU page} of its host pages, which
 *      then go back onto the host free stack (after all of step 3, so no
 *      offload of this plan reuses them);
 *   5. the batch's users become the most recently used, in batch order (the
 *      last one most recent), and each user's cached length becomes
 *      hist_len + n_new (the layer forward appends those tokens).
 * A user whose tokens would exceed max_pages_per_user * page_size makes the
 * plan fail with HSTU_KV_TOO_LONG, and a pinned user (hstu_kvcache_pin) with
 * HSTU_KV_PINNED, changing nothing.  The host tier keeps
 * its own recency order: a user enters it as its most recent entry.
 *
 * A plan's copies list every offload before every onboard; they must run
 * (hstu_kv_copy_pages) before the page tables are used by a layer call, on
 * the same stream: an offloaded GPU page may be handed out again by the same
 * plan.
 *
 * The page directory is a device int32 array [max_users][L][max_pages] that
 * the caller allocates (hstu_kvcache_directory_elems) and keeps: row (slot,
 * layer) lists the slot's page ids in position order.  hstu_kv_tables_build
 * applies a plan's update records to it and gathers the batch's page tables
 * [L][B][max_pages] for hstu_layer_fwd (entries past a user's pages are
 * whatever the directory holds; the layer only reads positions in use).
 *
 * Conventions: the manager is host-only (no HIP calls); its handle is owned
 * by the caller and is not thread-safe.  Pointers passed to the manager are
 * HOST pointers; pointers passed to hstu_kv_tables_build and
 * hstu_kv_copy_pages are DEVICE pointers (except the pinned host tier
 * arrays) and their work is enqueued on hip_stream.  Errors return a
 * nonzero status and leave the cache unchanged.
 */
#ifndef HSTU_KVCACHE_H_
#define HSTU_KVCACHE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HSTU_KV_OK = 0,
  HSTU_KV_INVALID_ARG = -1,   /* null pointer, bad size, duplicate user in a batch */
  HSTU_KV_FULL = -10,         /* the batch needs more pages or slots than can be freed */
  HSTU_KV_TOO_LONG = -11,     /* a user's tokens exceed max_pages_per_user * page_size */
  HSTU_KV_CAPACITY = -12,     /* an output array is too small */
  HSTU_KV_HIP = -13,          /* a HIP launch failed (hstu_kv_tables_build) */
  HSTU_KV_PINNED = -14        /* plan, evict or trim of a pinned user (hstu_kvcache_pin) */
} hstu_kv_status;

typedef struct hstu_kvcache hstu_kvcache;

/* One page assignment made by a plan. */
typedef struct {
  int32_t slot, layer, page_index, page_id;
} hstu_kv_update;

/* One page copy between the GPU pool and the host tier. */
typedef struct {
  int32_t onboard;           /* 0: offload GPU -> host, 1: onboard host -> GPU */
  int32_t gpu_page, host_page, reserved;
} hstu_kv_copy;

/* A cache over num_pages pages of page_size tokens for num_layers layers,
 * up to max_users GPU-cached users of at most max_pages_per_user pages per
 * layer, and a host tier of host_pages pages (0 = none).  Returns NULL on
 * invalid sizes (any < 1, host_pages < 0, page_size not a power of two,
 * num_pages or host_pages >= 2^31) or allocation failure. */
hstu_kvcache* hstu_kvcache_create(int32_t num_layers, int64_t num_pages, int32_t page_size,
                                  int32_t max_pages_per_user, int32_t max_users, int64_t host_pages);
void hstu_kvcache_destroy(hstu_kvcache* cache);

/* Elements of the device page directory: max_users * num_layers * max_pages. */
int64_t hstu_kvcache_directory_elems(const hstu_kvcache* cache);

/* Plans one batch (steps 1-5 above).
 *   user_ids[B], n_new[B] (n_new >= 0)                       in
 *   hist_len[B]  cached tokens reused per user (0 = miss)    out
 *   slots[B]     directory slot per user                     out
 *   updates[update_cap], *n_updates  page assignments        out
 *   evicted[evicted_cap], *n_evicted user ids evicted from the GPU (offloaded
 *                                    or dropped)                     out (may be
 *                                    NULL when evicted_cap == 0; evictions are
 *                                    then still made, only not reported)
 *   copies[copy_cap], *n_copies      offloads, then onboards         out
 * update_cap must be at least num_layers * sum_b ceil((hist_len + n_new) /
 * page_size) (num_layers * B * max_pages_per_user always suffices), and
 * copy_cap at least the pages of the batch's host hits plus the GPU pages
 * held by users outside the batch (2 * num_pages always suffices; 0 without
 * a host tier), else HSTU_KV_CAPACITY and no change; evicted ids past
 * evicted_cap are dropped from the report. */
hstu_kv_status hstu_kvcache_plan(hstu_kvcache* cache, int32_t B, const int64_t* user_ids,
                                 const int32_t* n_new, int32_t* hist_len, int32_t* slots,
                                 hstu_kv_update* updates, int32_t update_cap, int32_t* n_updates,
                                 int64_t* evicted, int32_t evicted_cap, int32_t* n_evicted,
                                 hstu_kv_copy* copies, int32_t copy_cap, int32_t* n_copies);

/* Cached tokens of each user (-1 when not cached) and its tier (0: not
 * cached, 1: GPU, 2: host; tier may be NULL); changes nothing, not even the
 * recency order. */
hstu_kv_status hstu_kvcache_lookup(const hstu_kvcache* cache, int32_t B, const int64_t* user_ids,
                                   int32_t* cached_len, int32_t* tier);

/* Drops one user from whichever tier holds it (its pages and slot are
 * freed, pushed as in step 3, nothing is offloaded).  *found = 1 when the
 * user was cached, else 0.  A pinned user is not dropped: HSTU_KV_PINNED. */
hstu_kv_status hstu_kvcache_evict(hstu_kvcache* cache, int64_t user_id, int32_t* found);

/* Shortens the cached length of each of B distinct GPU-cached users by
 * n_drop[b] tokens (0 <= n_drop[b] <= its cached length), e.g. the candidate
 * rows a layer call scored and appended but that are not history (the
 * candidates of a ranking request, NVIDIA blog above, sections "Why use
 * HSTU for generative recommendation" and "Benchmark setup"; which tokens
 * stay cached is this library's reading).  Pages past ceil(new length /
 * page_size) of every layer go onto the free-page stack layer by layer,
 * page index by page index; slots and recency are unchanged.  The device
 * directory keeps its stale entries past the new length: a later plan that
 * grows the user rewrites them.  Any invalid entry (unknown or host-cached
 * user, duplicate, count out of range) fails the whole call with
 * HSTU_KV_INVALID_ARG and no change; a pinned user fails it with
 * HSTU_KV_PINNED and no change.  Host pointers. */
hstu_kv_status hstu_kvcache_trim(hstu_kvcache* cache, int32_t B, const int64_t* user_ids,
                                 const int32_t* n_drop);

/* Pins (pin != 0) or unpins (pin == 0) B distinct GPU-cached users, for
 * callers that keep several planned batches in flight, i.e. layer calls of
 * earlier plans still running on other streams while the next batch is
 * planned.  No plan evicts a pinned user or hands out its pages: a pinned
 * user counts as neither free nor evictable in step 2.  A batch that holds
 * a pinned user fails with HSTU_KV_PINNED and no change (its earlier batch
 * has not appended its K/V yet), and hstu_kvcache_evict and
 * hstu_kvcache_trim refuse a pinned user the same way.  Pin a batch's users
 * after its plan and unpin them once its layer calls have finished.  Pins count: a user pinned twice stays
 * pinned until it is unpinned twice.  Any invalid entry (a user not cached
 * on the GPU, a duplicate, an unpin of an unpinned user) fails the whole
 * call with HSTU_KV_INVALID_ARG and no change.  Host pointers. */
hstu_kv_status hstu_kvcache_pin(hstu_kvcache* cache, int32_t B, const int64_t* user_ids, int32_t pin);

/* Free GPU pages and GPU-cached users, free host pages and host-cached
 * users (the host pointers may be NULL). */
hstu_kv_status hstu_kvcache_stats(const hstu_kvcache* cache, int64_t* free_pages,
                                  int32_t* cached_users, int64_t* free_host_pages,
                                  int32_t* host_users);

/* Applies update records to the device page directory and gathers the page
 * tables of a planned batch:
 *   directory  [max_users][num_layers][max_pages] int32 (device, in/out)
 *   updates    [n_updates] hstu_kv_update (device)
 *   slots      [B] int32 (device)
 *   tables     [num_layers][B][max_pages] int32 (device, out)
 * Two kernels on hip_stream (the scatter, then the gather).  Update records
 * and slots must come from plans of a cache with these sizes. */
hstu_kv_status hstu_kv_tables_build(int32_t* directory, int32_t num_layers, int32_t max_users,
                                    int32_t max_pages, const hstu_kv_update* updates,
                                    int32_t n_updates, const int32_t* slots, int32_t B,
                                    int32_t* tables, void* hip_stream);

/* Runs a plan's page copies between the GPU pools and the host tier:
 *   k_pool, v_pool         device pools of the layer (include/hstu.h layout)
 *   host_k, host_v         pinned host arrays with the same per-page layout,
 *                          host_pages pages each (allocated with hipHostMalloc
 *                          or any pinned allocator that maps them for the
 *                          device)
 *   page_bytes_k/_v        bytes of one page of each pool (H*page_size*d*elem)
 *   copies [n] (device)    a plan's list, offloads first
 * The offloads run as one kernel, then the onboards as another, on
 * hip_stream; each workgroup copies one page of K and V with 16-byte
 * accesses, reading or writing host memory directly over the bus. */
hstu_kv_status hstu_kv_copy_pages(void* k_pool, void* v_pool, void* host_k, void* host_v,
                                  int64_t page_bytes_k, int64_t page_bytes_v, int64_t num_pages,
                                  int64_t host_pages, const hstu_kv_copy* copies, int32_t n_offload,
                                  int32_t n, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* HSTU_KVCACHE_H_ */
