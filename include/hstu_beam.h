/*
 * hstu_beam.h -- C ABI of libhstu's beam-decode attention for Semantic-ID
 * generative recommendation over a shared request-level context KV.
 *
 * Sources: the Korean summary of the recsys-examples article (its section on
 * the GR inference path) and the Hungarian article on news.bpdata.com,
 * section "SID-GR inference": a request carries a long user context (often
 * thousands of tokens) and decodes only 2-3 Semantic-ID tokens with wide
 * beams (128 or 256); serving keeps one ContextKV per request shared by all
 * of its beams instead of copying it per beam, a short per-beam BeamKV of the
 * decoded tokens and BeamPath bookkeeping of each beam's ancestry, and runs a
 * decode attention directly on that layout.  The pages give no formula; the
 * operation below is this library's reading for a standard decoder with
 * grouped query heads.
 *
 * At decode step t (0-based), for request r, beam w, query head h (KV head
 * g = h / (Hq / Hkv)):
 *   keys   = ctx_k[r][0 .. ctx_len[r]-1][g],
 *            then beam_k[r][s][path[r][w][s]][g] for s = 0 .. t-1,
 *            then beam_k[r][t][w][g]           (the beam's own token)
 *   values = the same rows of ctx_v / beam_v
 *   out[r][w][h] = softmax(scale * keys . q[r][w][h]) . values
 * The caller writes step t's K and V of every beam into beam_k/beam_v slot
 * (t, w) before the call, and keeps path: after each step's beam selection,
 * new beam w's path is its parent's path followed by the parent's slot.
 *
 * Layouts (row-major, dtype elements unless stated):
 *   q       [R][W][Hq][d]
 *   ctx_k   [R][Hkv][max_ctx][d]
 *   ctx_vt  [R][Hkv][d][max_ctx]    (context V transposed: key-contiguous
 *                                    rows, the MFMA operand order)
 *   ctx_len [R] int32               in [0, max_ctx]
 *   beam_k, beam_v [R][max_steps][W][Hkv][d]
 *   path    [R][W][step] int32      beam slots in [0, W); NULL when step == 0
 *   out     [R][W][Hq][d]
 * Device pointers, caller-owned, 16-byte aligned.  The workspace
 * (hstu_beam_workspace_size bytes, 256-byte aligned) holds the call's device
 * status word (its first int32) and fp32 partial results; the library
 * allocates nothing.  Work is enqueued on hip_stream: a split-context kernel
 * (per request, KV head, 256-row query tile and context chunk: MFMA scores,
 * online softmax, MFMA value product) and a combine kernel (one wave per
 * output row: merges the chunks and the beam's own path keys).
 * Host-checkable errors return a negative hstu_status and enqueue nothing; a
 * ctx_len outside [0, max_ctx] or a path entry outside [0, W) sets the status
 * word (HSTU_DEV_BAD_CTX_LEN, HSTU_DEV_BAD_PATH) and out is left unwritten.
 * num_requests == 0 enqueues nothing (the status word is not written).
 */
#ifndef HSTU_BEAM_H_
#define HSTU_BEAM_H_

#include "hstu.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t num_requests;   /* R >= 0 */
  int32_t beam_width;     /* W in [1, 1024] */
  int32_t num_q_heads;    /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;   /* Hkv >= 1 */
  int32_t head_dim;       /* d: 64 or 128 */
  int32_t max_ctx;        /* context row stride: a multiple of 32, >= 32 */
  int32_t step;           /* t >= 0 */
  int32_t max_steps;      /* BeamKV steps held, > step */
  float scale;            /* softmax scale, e.g. 1/sqrt(d) */
  int32_t dtype;          /* hstu_dtype (bf16: fp32 accumulation and softmax) */
} hstu_beam_desc;

/* Workspace bytes for desc (host-only). */
hstu_status hstu_beam_workspace_size(const hstu_beam_desc* desc, size_t* bytes);

/* One decode step's attention for every beam of every request (see top). */
hstu_status hstu_beam_decode_attn(const hstu_beam_desc* desc, const void* q, const void* ctx_k,
                                  const void* ctx_vt, const int32_t* ctx_len, const void* beam_k,
                                  const void* beam_v, const int32_t* path, void* out,
                                  void* workspace, size_t workspace_bytes, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* HSTU_BEAM_H_ */
