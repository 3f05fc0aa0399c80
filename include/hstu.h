/*
 * hstu.h -- C ABI of libhstu: the HSTU layer forward over jagged per-user
 * sequences whose cached history K/V lives in a paged GPU KV pool, for AMD
 * Instinct MI355X (gfx950).
 *
 * What the layer computes (per layer, per user u with c cached tokens and n
 * new rows; head h of H, head dim d, hidden D = H*d):
 *   Z = SiLU(X W1); U, V, Q, K = the four D-wide column blocks of Z, in that
 *       order; head h owns columns [h*d, (h+1)*d) of each block.
 *   New row t sits at absolute position p = c + t.  For each key j <= p:
 *       s = <Q[t,h], K[j,h]> + pos_bias[b(p-j)] (+ ts_bias[b_ts(ts[p]-ts[j])])
 *       O[t,h] = attn_scale * sum_j SiLU(s) * V[j,h]          (no softmax)
 *   G = LayerNorm_row(O) (mean/population variance over the D entries of a
 *       row, eps = norm_eps, no affine) * U;   Y = G W2.
 *   Keys/values j < c come from the pool; the new rows' K and V are appended
 *   into the pool by the same call and read back from it.
 * Sources: NVIDIA technical blog "Deploying an HSTU generative recommender
 * with NVIDIA Dynamo-Triton", section "Why serving large sequential
 * recommenders is hard" (jagged inputs, reuse of cached history K/V, a paged
 * GPU KV data table with append, an HSTU attention kernel reading the paged
 * cache); aitrends.kr article 100093, section "HSTU sequential modelling"
 * (SiLU weighting instead of softmax, relative attention bias, elementwise
 * gating before the output projection).  The exact block split, 1/N scale,
 * LayerNorm and bucket rule are this library's readings of that prose.
 *
 * Bucket rule b(delta) (mantissa bits m, s = 2^m, nb buckets):
 *   delta < 0 -> 0;  delta < s -> delta;
 *   else e = floor(log2 delta), b = s*(e-m+1) + (delta >> (e-m)) - s;
 *   b = min(b, nb-1).
 *
 * KV pool layout (both pools hold `dtype` elements, P = num_pool_pages,
 * ps = page_size):
 *   user u's position p lives in page page_table[u*max_pages_per_user + p/ps],
 *   slot p % ps;
 *   k_pool[P][H][ps][d]  -- element (page, h, slot, e)
 *   v_pool[P][H][d][ps]  -- element (page, h, e, slot)   (V stored transposed
 *                           per page so the attention kernel reads key-
 *                           contiguous V runs)
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers unless stated, row-major,
 *     allocated and owned by the caller.  The library never allocates, frees
 *     or caches device memory and keeps no mutable global state, with one
 *     exception: the static scratch array of hstu_layer_fwd_noalloc (below).
 *   - Work is enqueued on `hip_stream` (a hipStream_t; NULL = default stream)
 *     and runs asynchronously; calls return before the GPU finishes.
 *   - Host-checkable problems (null pointer, inconsistent sizes, unsupported
 *     shape/dtype, workspace too small) return a negative hstu_status and
 *     enqueue nothing.
 *   - Data-dependent problems (offsets not a non-decreasing prefix sum ending
 *     at total_new, negative history length, a sequence longer than its page
 *     table row, a page id outside [0, num_pool_pages)) are detected on the
 *     device: the call's device status word receives a nonzero
 *     hstu_device_code and every later kernel of that call writes nothing
 *     (y, pools and workspace outputs keep their previous contents).
 *   - Calls on the same stream are ordered; concurrent calls need distinct
 *     workspaces and must not append to the same pool slots.
 */
#ifndef HSTU_H_
#define HSTU_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HSTU_OK = 0,
  HSTU_ERR_INVALID_ARG = -1,   /* null pointer, bad size or inconsistent descriptor */
  HSTU_ERR_UNSUPPORTED = -2,   /* head_dim / page_size / dtype not supported */
  HSTU_ERR_WORKSPACE = -3,     /* workspace_bytes smaller than required */
  HSTU_ERR_HIP = -4,           /* a HIP runtime call or kernel launch failed */
  HSTU_ERR_DEVICE = -5,        /* device status word holds a nonzero code */
  HSTU_ERR_SCRATCH = -6        /* hstu_layer_fwd_noalloc: the call needs more than
                                  HSTU_NOALLOC_SCRATCH_BYTES of workspace */
} hstu_status;

typedef enum {
  HSTU_F32 = 0,   /* fp32 storage and fp32 arithmetic */
  HSTU_BF16 = 1   /* bf16 storage, fp32 accumulation and score math */
} hstu_dtype;

/* Codes written to the device status word. */
typedef enum {
  HSTU_DEV_OK = 0,
  HSTU_DEV_BAD_OFFSETS = 1,    /* new_offsets[0] != 0, decreasing, or [B] != total_new */
  HSTU_DEV_BAD_HIST = 2,       /* hist_len[u] < 0 */
  HSTU_DEV_CAPACITY = 3,       /* hist_len[u] + n_u > max_pages_per_user * page_size */
  HSTU_DEV_BAD_PAGE = 4,       /* a needed page id outside [0, num_pool_pages) */
  HSTU_DEV_BAD_TS = 5,         /* ts_offsets[u+1]-ts_offsets[u] != hist_len[u]+n_u */
  HSTU_DEV_BAD_CANDIDATES = 6, /* num_candidates[u] outside [0, n_u] */
  HSTU_DEV_BAD_TOKEN = 7,      /* hstu_preprocess: a token id outside its table */
  HSTU_DEV_BAD_POSITION = 8,   /* hstu_preprocess: hist_len[u] + rows of u > max_positions */
  HSTU_DEV_BAD_CTX_LEN = 9,    /* hstu_beam_decode_attn: ctx_len[r] outside [0, max_ctx] */
  HSTU_DEV_BAD_PATH = 10       /* hstu_beam_decode_attn: a path slot outside [0, W) */
} hstu_device_code;

typedef struct {
  int32_t num_users;           /* B >= 0 */
  int32_t num_heads;           /* H >= 1 */
  int32_t head_dim;            /* d: 32, 64 or 128 */
  int32_t hidden;              /* D = H*d, a multiple of 64 */
  int32_t page_size;           /* ps: 16, 32, 64 or 128 tokens */
  int32_t max_pages_per_user;  /* row stride of page_table */
  int64_t num_pool_pages;      /* P: pages in each pool */
  int32_t total_new;           /* T = new_offsets[B], rows of x and y */
  int32_t pos_buckets;         /* nb in [1, 1024] */
  int32_t pos_mbits;           /* m in [0, 16] */
  int32_t ts_buckets;          /* 0 = no timestamp term, else in [1, 1024] */
  int32_t ts_mbits;            /* m for the timestamp-delta rule */
  float attn_scale;            /* 1/N */
  float norm_eps;              /* LayerNorm epsilon (> 0) */
  int32_t dtype;               /* hstu_dtype */
  int32_t flags;               /* 0 or HSTU_FLAG_BATCH_INVARIANT */
} hstu_layer_desc;

/* desc->flags bit: batch-invariant results.  Every output row (and every K/V
 * row the call appends) is then bit-identical whatever else is in the batch
 * and however the user's sequence was split into calls: a user's rows come
 * out the same from a call with other users as from a call of its own, and
 * the same from a call that reads their history from the cache as from one
 * that recomputes the whole sequence (the cache-reuse property the NVIDIA
 * blog's "Benefits" section rests on; without the flag both hold to the
 * dtype's rounding).  The attention then cuts every user's keys at fixed
 * positions (multiples of HSTU_INVARIANT_CHUNK_KEYS) and adds a row's pieces
 * in one fixed order, and the row norm reduces a row in one fixed way; the
 * price is work balance (fewer, fixed-size pieces) and, for long causal
 * recomputes, more partial-sum traffic.  The workspace is sized for the
 * flag (hstu_layer_workspace_size takes it into account). */
#define HSTU_FLAG_BATCH_INVARIANT 1
#define HSTU_INVARIANT_CHUNK_KEYS 256

/* Bytes of device workspace hstu_layer_fwd needs for `desc` (depends only on
 * B, H, d, D, total_new, dtype, max_pages_per_user * page_size and flags).
 * Host-only; enqueues nothing. */
hstu_status hstu_layer_workspace_size(const hstu_layer_desc* desc, size_t* bytes);

/* One HSTU layer over a jagged batch of new rows (see the top of this file).
 *   x            [T, D] dtype     new rows of all users back to back
 *   new_offsets  [B+1]  int32     prefix sums of new-row counts; user u owns
 *                                 rows new_offsets[u] .. new_offsets[u+1]-1
 *   hist_len     [B]    int32     tokens of user u already in the pool (this
 *                                 layer); not advanced by the library
 *   page_table   [B, max_pages_per_user] int32, -1 = unused entry; entries
 *                                 for positions [0, hist_len+n) must be valid
 *   k_pool, v_pool                pools (layout above); the new rows' K and V
 *                                 are written at positions hist_len[u] + t
 *   w1t          [4D, D] dtype    W1 transposed (out-features x in-features,
 *                                 the usual linear-layer weight layout): row j
 *                                 holds the weights of output column j, rows
 *                                 in U | V | Q | K block order
 *   w2t          [D, D]  dtype    W2 transposed, same convention
 *   pos_bias     [pos_buckets] float32
 *   ts_bias      [ts_buckets]  float32, or NULL when ts_buckets == 0
 *   timestamps   int64, jagged over every position (history then new) of each
 *                user; user u's run starts at ts_offsets[u]; NULL when
 *                ts_buckets == 0
 *   ts_offsets   [B+1] int32 or NULL
 *   y            [T, D] dtype     output; must not alias x
 *   workspace    device scratch of hstu_layer_workspace_size bytes (256-byte
 *                aligned); its first int32 is the call's device status word
 * total_new == 0 is a valid no-op. */
hstu_status hstu_layer_fwd(const hstu_layer_desc* desc, const void* x,
                           const int32_t* new_offsets, const int32_t* hist_len,
                           const int32_t* page_table, void* k_pool, void* v_pool,
                           const void* w1t, const void* w2t, const float* pos_bias,
                           const float* ts_bias, const int64_t* timestamps,
                           const int32_t* ts_offsets, void* y, void* workspace,
                           size_t workspace_bytes, void* hip_stream);

/* Same as hstu_layer_fwd, and additionally has the runtime stamp
 * caller-created hipEvent_t handles at the start and the end of each stage's
 * kernel (hipExtLaunchKernel), so that hipEventElapsedTime of a pair is that
 * kernel's execution time alone, without launch gaps.  stage_events holds
 * 2*HSTU_NUM_STAGES events (start, stop per stage, in the order of
 * hstu_stage); a NULL array or NULL entries record nothing.  Ownership of the
 * events stays with the caller. */
typedef enum {
  HSTU_STAGE_PREP = 0,         /* index prep / validation / work list */
  HSTU_STAGE_PROJ = 1,         /* X W1 + SiLU + split + K/V append */
  HSTU_STAGE_ATTN = 2,         /* paged SiLU attention */
  HSTU_STAGE_NORM = 3,         /* row norm * U */
  HSTU_STAGE_OUT = 4,          /* G W2 */
  HSTU_NUM_STAGES = 5
} hstu_stage;
hstu_status hstu_layer_fwd_timed(const hstu_layer_desc* desc, const void* x,
                                 const int32_t* new_offsets, const int32_t* hist_len,
                                 const int32_t* page_table, void* k_pool, void* v_pool,
                                 const void* w1t, const void* w2t, const float* pos_bias,
                                 const float* ts_bias, const int64_t* timestamps,
                                 const int32_t* ts_offsets, void* y, void* workspace,
                                 size_t workspace_bytes, void* hip_stream,
                                 void* const* stage_events);

/* hstu_layer_fwd with candidate rows, and optional stage events as in
 * hstu_layer_fwd_timed (stage_events may be NULL).  num_candidates [B] int32
 * (device, required): the last num_candidates[u] new rows of user u are
 * candidate items to be scored (NVIDIA blog above, sections "Why use HSTU
 * for generative recommendation", where candidates are tokens of the
 * sequence, and "Benchmark setup", up to 100 candidates per request).  With
 * cs = hist_len[u] + n_u - num_candidates[u], a row at position p >= cs
 * attends to the keys j < cs and to j = p only: each candidate is scored as
 * if it alone followed the history and the other new rows (the pages give
 * no mask for candidates; this is the library's reading).  Rows before cs
 * are unchanged.  Candidates' K and V are appended like every new row; a
 * cache that should not keep them as history drops them afterwards
 * (hstu_kvcache_trim).  A count outside [0, n_u] is HSTU_DEV_BAD_CANDIDATES
 * on the status word.  The workspace size is that of hstu_layer_fwd. */
hstu_status hstu_layer_fwd_cand(const hstu_layer_desc* desc, const void* x,
                                const int32_t* new_offsets, const int32_t* hist_len,
                                const int32_t* num_candidates, const int32_t* page_table,
                                void* k_pool, void* v_pool, const void* w1t, const void* w2t,
                                const float* pos_bias, const float* ts_bias,
                                const int64_t* timestamps, const int32_t* ts_offsets, void* y,
                                void* workspace, size_t workspace_bytes, void* hip_stream,
                                void* const* stage_events);

/* hstu_layer_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * no workspace argument and no allocation of any kind.  The workspace is
 * instead a file-scope device array of HSTU_NOALLOC_SCRATCH_BYTES bytes
 * inside the library; each GPU the library runs on holds its own copy from
 * the moment the library is loaded until the process ends.  Arguments,
 * results and errors are those of hstu_layer_fwd, plus:
 *   device_status  one device int32 (caller-owned) that receives the call's
 *                  hstu_device_code once its kernels have run (0 = success);
 *                  the status word inside the scratch array is not exposed
 *   returns HSTU_ERR_SCRATCH (enqueuing nothing) when
 *   hstu_layer_workspace_size(desc) exceeds HSTU_NOALLOC_SCRATCH_BYTES: at
 *   D = 512, H = 4, d = 128 in bf16 that holds batches of 8 users with up to
 *   about 4,000 new rows and 4,352-token sequences, or about 1,500 new rows
 *   and 16,448-token sequences.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (every value the kernels read is written earlier in the same call,
 * so nothing carries over): calls that overlap in time on one GPU -- on two
 * streams, or from two host threads without ordering -- race on it and give
 * undefined results.  Calls ordered on one stream are safe. */
#define HSTU_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
hstu_status hstu_layer_fwd_noalloc(const hstu_layer_desc* desc, const void* x,
                                   const int32_t* new_offsets, const int32_t* hist_len,
                                   const int32_t* page_table, void* k_pool, void* v_pool,
                                   const void* w1t, const void* w2t, const float* pos_bias,
                                   const float* ts_bias, const int64_t* timestamps,
                                   const int32_t* ts_offsets, void* y, int32_t* device_status,
                                   void* hip_stream);

/* Input preprocessing: the layer's input rows built from categorical tokens
 * (NVIDIA blog above, section "Why use HSTU for generative recommendation":
 * embedding lookup, interleave of item and action embeddings when action
 * tokens are present, context appended, positional encoding; section
 * "Benchmark setup": 6 context features, history of item/action pairs, up to
 * 100 candidates).  Readings: every token is one row; user u's new rows are
 * its context tokens, then its history entries (each pair as the item's row
 * then the action's row; without action tokens, one item row per entry),
 * then its candidate items; row t sits at position hist_len[u] + t and
 *     x = table[id] + pos_emb[position]
 * added in fp32 and rounded once to dtype (tables: ctx_emb for context,
 * item_emb for items and candidates, action_emb for actions). */
typedef struct {
  int32_t num_users;           /* B >= 0 (at most 4096) */
  int32_t hidden;              /* D, a multiple of 64, at most 2048 */
  int32_t dtype;               /* hstu_dtype of every table and of x */
  int32_t total_new;           /* T: rows of x; must equal the rows the tokens make */
  int64_t item_rows;           /* rows of item_emb (>= 1) */
  int64_t action_rows;         /* rows of action_emb; 0 = no action tokens */
  int64_t ctx_rows;            /* rows of ctx_emb (>= 1) */
  int32_t max_positions;       /* rows of pos_emb (>= 1) */
} hstu_prep_desc;

/* Builds x [T, D] and the layer's row metadata from a jagged token batch.
 *   hist_len      [B]   int32  cached tokens per user (first position)
 *   ctx_offsets   [B+1] int32, ctx_ids [ctx_offsets[B]] int64    context ids
 *   hist_offsets  [B+1] int32, item_ids / action_ids [hist_offsets[B]] int64
 *                               history entries (action_ids NULL when
 *                               action_rows == 0)
 *   cand_offsets  [B+1] int32, cand_ids [cand_offsets[B]] int64  candidates
 *   item_emb [item_rows, D], action_emb [action_rows, D] (or NULL),
 *   ctx_emb [ctx_rows, D], pos_emb [max_positions, D]          dtype
 *   x              [T, D] dtype   out
 *   new_offsets    [B+1] int32    out: prefix sums of each user's rows
 *   num_candidates [B]   int32    out: candidate rows per user (for
 *                                 hstu_layer_fwd_cand)
 *   device_status  one device int32: receives 0 or a hstu_device_code
 * Device pointers, caller-owned.  Two kernels on hip_stream: a one-workgroup
 * scan that checks the offsets (each [0] == 0, non-decreasing: else
 * HSTU_DEV_BAD_OFFSETS, as is a row total != T), the histories
 * (HSTU_DEV_BAD_HIST) and the positions (HSTU_DEV_BAD_POSITION) and writes
 * new_offsets and num_candidates; then the row builder, which writes nothing
 * after a nonzero status.  A token id outside its table sets
 * HSTU_DEV_BAD_TOKEN while the rows are being built: x is then unspecified.
 * T == 0 with B == 0 is a valid call (new_offsets[0] = 0, status 0); the
 * [B] arrays may then be NULL. */
hstu_status hstu_preprocess(const hstu_prep_desc* desc, const int32_t* hist_len,
                            const int32_t* ctx_offsets, const int64_t* ctx_ids,
                            const int32_t* hist_offsets, const int64_t* item_ids,
                            const int64_t* action_ids, const int32_t* cand_offsets,
                            const int64_t* cand_ids, const void* item_emb,
                            const void* action_emb, const void* ctx_emb, const void* pos_emb,
                            void* x, int32_t* new_offsets, int32_t* num_candidates,
                            int32_t* device_status, void* hip_stream);

/* A stack of num_layers layers over one batch, layer l's output feeding
 * layer l+1 (the HSTU blocks applied in sequence, NVIDIA blog above, section
 * "Why use HSTU for generative recommendation"), in one call whose batch
 * metadata -- validation, the attention work list, every layer's pool slots
 * -- is prepared once for all layers instead of once per layer.  Results
 * are those of num_layers hstu_layer_fwd_cand (num_candidates != NULL) or
 * hstu_layer_fwd calls with the same arguments, bit for bit.
 *   num_layers in [1, 32]
 *   page_tables, k_pools, v_pools, w1t, w2t, pos_bias, ts_bias, y: HOST
 *     arrays of num_layers DEVICE pointers, one per layer, each as in
 *     hstu_layer_fwd (ts_bias may be NULL when ts_buckets == 0); y[l]
 *     receives layer l's output [T, D] and must not alias its input (x for
 *     layer 0, y[l-1] after), so two buffers used in turn suffice
 *   num_candidates: as in hstu_layer_fwd_cand, or NULL
 *   workspace: hstu_stack_workspace_size(desc, num_layers) bytes
 * Every page table is validated before any layer runs: a data problem in
 * any of them stops the whole stack (nothing is written). */
hstu_status hstu_stack_workspace_size(const hstu_layer_desc* desc, int32_t num_layers, size_t* bytes);
hstu_status hstu_stack_fwd(const hstu_layer_desc* desc, int32_t num_layers, const void* x,
                           const int32_t* new_offsets, const int32_t* hist_len,
                           const int32_t* num_candidates, const int32_t* const* page_tables,
                           void* const* k_pools, void* const* v_pools, const void* const* w1t,
                           const void* const* w2t, const float* const* pos_bias,
                           const float* const* ts_bias, const int64_t* timestamps,
                           const int32_t* ts_offsets, void* const* y, void* workspace,
                           size_t workspace_bytes, void* hip_stream);

/* Append new rows' K and V into the pools (the paged KV table's append, NVIDIA
 * blog above, same section).  k_new, v_new [T, D] dtype, rows laid out as x in
 * hstu_layer_fwd; row t of user u goes to position hist_len[u] + t.  Only
 * those slots are written; the copy is bit-exact.  Uses desc fields num_users,
 * num_heads, head_dim, hidden, page_size, max_pages_per_user, num_pool_pages,
 * total_new and dtype.  device_status: one device int32 that receives this
 * call's hstu_device_code (0 on success); on a nonzero code nothing is
 * written to the pools. */
hstu_status kv_pages_append(const hstu_layer_desc* desc, const void* k_new,
                            const void* v_new, const int32_t* new_offsets,
                            const int32_t* hist_len, const int32_t* page_table,
                            void* k_pool, void* v_pool, int32_t* device_status,
                            void* hip_stream);

/* Waits for `hip_stream`, then copies the device status word at
 * `device_status` (a workspace base or kv_pages_append's status int) to
 * *code.  Returns HSTU_ERR_DEVICE when *code != 0. */
hstu_status hstu_read_device_status(const void* device_status, int32_t* code,
                                    void* hip_stream);

/* Static description of a hstu_status or hstu_device_code value. */
const char* hstu_status_string(int32_t status);

#ifdef __cplusplus
}
#endif
#endif /* HSTU_H_ */
