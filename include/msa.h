/*
 * msa.h — C ABI of the MSA (Memory Sparse Attention) inference hot path for
 * AMD MI355X (gfx950).
 *
 * The method (the MSA pages, arXiv 2603.23516):
 *   Stage 1, offline encoding: every document's K, V and router keys K^R are
 *     mean-pooled over fixed 64-token chunks, K under document-wise RoPE
 *     (positions restart at 0 in each document).
 *   Stage 2, online routing: the router query Q^R is scored against every
 *     pooled router key by cosine similarity (mean over heads, max over query
 *     tokens), chunk scores are max-reduced to document scores and the top-16
 *     documents are selected.
 *   Stage 3, sparse generation: the query attends over the selected documents'
 *     pooled K/V concatenated with its local KV, under global RoPE whose
 *     positions start at k.
 *   Memory Interleave repeats route → select → attend as new tokens arrive.
 * Sources: portal.techblg.uk IRMaD reading, section M "Materials & Methods"
 * (architecture, routing/sparse-attention, positional-encoding, three-stage
 * inference, Memory Parallel and Memory Interleave bullets); paper.rainbus.top
 * "method steps"; chooseai.io sections 2.1-2.4; zhichai.net "关键技术细节".
 *
 * Conventions for every call:
 *   - Return value: MSA_OK (0) or a negative msa_status. On an error nothing
 *     has been enqueued and no output has been written; msa_last_error()
 *     returns a thread-local message.
 *   - Success means the work is enqueued on `stream` (a hipStream_t passed as
 *     void*; NULL is the legacy default stream). Results are valid after the
 *     stream is synchronised.
 *   - Pointers are device pointers unless the name ends in `_h` (host memory).
 *     Where a call says so, K̄/V̄ may instead live in pinned host memory
 *     (hipHostMalloc, or torch pin_memory=True); pageable host memory is
 *     rejected.
 *   - The caller owns every buffer, including workspaces (sized by the
 *     *_workspace calls). The library keeps no allocation and no state across
 *     calls except the thread-local error string — and, for the one call
 *     that takes no workspace (msa_route_topk_noalloc), a fixed device
 *     scratch array per GPU and its looked-up address.
 *   - Inputs are never modified, except where a call says so.
 *   - bf16 tensors are raw bit patterns (msa_bf16), row-major and contiguous:
 *     token-major raw states [T, H, 128], pooled states [C, H, 128]. Each
 *     starts at a 16-byte aligned address (kernels move them in 16-byte
 *     vectors; hipMalloc, hipHostMalloc and torch allocations are aligned);
 *     a misaligned one is MSA_ERR_INVALID_ARG naming the argument.
 *   - Offsets are int64 CSR: document i owns tokens [dto[i], dto[i+1]) and
 *     chunks [dco[i], dco[i+1]). Kernels clamp every index they derive from
 *     device arrays, so malformed offsets give wrong values, never an
 *     out-of-bounds access.
 *   - Calls are re-entrant; two calls may run concurrently on different
 *     streams if they share no output or workspace buffer.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t msa_bf16; /* bf16 storage (upper half of an IEEE binary32) */

typedef enum msa_status {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = -1, /* null pointer, bad enum, unsupported memory kind */
  MSA_ERR_SHAPE = -2,       /* sizes inconsistent or out of range */
  MSA_ERR_WORKSPACE = -3,   /* workspace missing or too small */
  MSA_ERR_HIP = -4,         /* a HIP runtime call or launch failed */
  MSA_ERR_UNSUPPORTED = -5, /* valid but not implemented (e.g. head_dim != 128) */
  MSA_ERR_IO = -6           /* a store file could not be read or written, or is malformed */
} msa_status;

enum { MSA_TOKEN_REDUCE_MAX = 0, MSA_TOKEN_REDUCE_MEAN = 1 };
enum { MSA_DOC_ROPE_TOKEN = 0, MSA_DOC_ROPE_CHUNK = 1 };

/* Model dimensions. Defaults (msa_default_dims) follow the pages'
 * architecture bullet (section M): 8 KV and router heads of dimension 128,
 * chunk P = 64, top-k = 16; 32 query heads (GQA group 4); RoPE base 1e6.
 * token_reduce: how chunk scores reduce over the query's tokens — MAX (the
 *   explicit routing formula of section M) or MEAN (the method-steps wording
 *   of paper.rainbus.top).
 * doc_rope_mode: TOKEN rotates raw K at its document-local token position
 *   before pooling; CHUNK rotates the pooled chunk at its chunk index.
 * Supported: head_dim == 128, n_kv_heads == n_router_heads == 8,
 *   n_q_heads a multiple of n_kv_heads (<= 64), chunk in [1, 4096],
 *   top_k in [1, 64]. */
typedef struct msa_dims {
  int32_t n_kv_heads;
  int32_t n_router_heads;
  int32_t n_q_heads;
  int32_t head_dim;
  int32_t chunk;
  int32_t top_k;
  float rope_theta;
  int32_t token_reduce;
  int32_t doc_rope_mode;
} msa_dims;

/* Fills *d with the defaults above. */
void msa_default_dims(msa_dims* d);

/* Thread-local message of the last failed call on this thread ("" if none). */
const char* msa_last_error(void);

/* ABI version of this header (bumped on any signature change). */
int32_t msa_abi_version(void);
#define MSA_ABI_VERSION 6

/* ------------------------------------------------------------------------ */
/* Chunk plan (host, pure). Each document is cut into ceil(n_i / chunk)
 * chunks of `chunk` tokens, the last one possibly partial; a chunk never
 * spans two documents (chooseai.io section 2.1; techblg lay summary ③).
 *   doc_token_offsets_h [n_docs+1] (host): non-decreasing from 0, every
 *     document at least one token (MSA_ERR_SHAPE otherwise).
 *   doc_chunk_offsets_h [n_docs+1] (host, written).
 * Returns MSA_OK and writes nothing on error. */
int32_t msa_plan_chunks(const int64_t* doc_token_offsets_h, int32_t n_docs, int32_t chunk,
                        int64_t* doc_chunk_offsets_h);

/* ------------------------------------------------------------------------ */
/* Stage 1: pooling with document-wise RoPE (techblg section M, routing and
 * positional-encoding bullets: K̄ = φ(K), V̄ = φ(V), K̄^R = φ(K^R), φ the chunk
 * mean; positions restart at 0 per document).
 *   K, V   [n_tokens, n_kv_heads, 128] bf16; KR [n_tokens, n_router_heads, 128].
 *   doc_token_offsets, doc_chunk_offsets: device int64 [n_docs+1]; the chunk
 *     offsets must be the plan of the token offsets (msa_plan_chunks).
 *   Kbar, Vbar [n_chunks, n_kv_heads, 128], KRbar [n_chunks, n_router_heads,
 *     128] bf16 (written). Each output is the mean over the chunk's actual
 *     tokens, accumulated in fp64 and rounded to bf16 nearest-even.
 *   Any of Kbar/Vbar/KRbar may be NULL to skip that output.
 *   ws / ws_bytes: workspace of at least msa_encode_pool_workspace() bytes. */
size_t msa_encode_pool_workspace(const msa_dims* d, int32_t n_docs, int64_t n_chunks);
int32_t msa_encode_pool(const msa_dims* d, const msa_bf16* K, const msa_bf16* V,
                        const msa_bf16* KR, const int64_t* doc_token_offsets,
                        const int64_t* doc_chunk_offsets, int32_t n_docs, int64_t n_tokens,
                        int64_t n_chunks, msa_bf16* Kbar, msa_bf16* Vbar, msa_bf16* KRbar,
                        void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Stage 2: routing and top-k (techblg section M, routing bullet:
 * S_ij = max_t mean_h cos(Q^R_{t,h}, K̄^R_{ij,h}), s_i = max_j S_ij,
 * I = Top-k({s_i})).
 *   QR [B, M, n_router_heads, 128] bf16: B independent queries of M tokens.
 *   KRbar [n_chunks, n_router_heads, 128] bf16, resident in device memory.
 *   doc_chunk_offsets: device int64 [n_docs+1].
 *   doc_scores [B, n_docs] fp32: written with s_i; when accumulate != 0 it is
 *     read first and max-merged (s_i = max(previous, new)) — the incremental
 *     form of re-routing every token of a growing query under the MAX token
 *     reduction (MEAN with accumulate is MSA_ERR_UNSUPPORTED).
 *   topk_ids [B, top_k] int32, topk_scores [B, top_k] fp32: the n_sel =
 *     min(top_k, n_docs) best documents by (score descending, id ascending),
 *     in rank order; entries past n_sel are -1 / -inf.
 *   n_sel [B] int32 (written).
 *   Norms are clamped at 1e-6 before dividing; a NaN score ranks last.
 *   Precision: with a single query row in all (decode) the cosines are
 *     fp32-exact (q̂ kept as a bf16 hi + lo pair); with more rows q̂ is
 *     rounded to bf16, and when M is a multiple of 128 k̂ = k/‖k‖ is rounded
 *     to bf16 as well
 *     (the head sum is then one contraction); a chunk score moves by ~1e-4 at
 *     most. The path depends on B·M == 1 and on M only, so a query of more
 *     than one token gets the same scores alone or in any batch (with 1024 or
 *     more rows of whole 256-token tiles the contraction stages normalised
 *     keys written once per call, and runs the same products in the same
 *     order: the scores are bit-identical).
 *   ws / ws_bytes: at least msa_route_topk_workspace() bytes. */
size_t msa_route_topk_workspace(const msa_dims* d, int32_t B, int32_t M, int64_t n_chunks,
                                int32_t n_docs);
int32_t msa_route_topk(const msa_dims* d, const msa_bf16* QR, int32_t B, int32_t M,
                       const msa_bf16* KRbar, const int64_t* doc_chunk_offsets, int32_t n_docs,
                       int64_t n_chunks, float* doc_scores, int32_t accumulate, int32_t* topk_ids,
                       float* topk_scores, int32_t* n_sel, void* ws, size_t ws_bytes,
                       void* stream);

/* msa_route_topk without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Arguments, outputs and errors are those of
 * msa_route_topk; the call allocates nothing.
 *   Scratch: a fixed array of MSA_NOALLOC_SCRATCH_BYTES (16 MiB) in the
 *     library's device memory, one per GPU, held until the process ends. That
 *     covers msa_route_topk_workspace() up to 16 MiB — e.g. one single-token
 *     query over 1,562,500 chunks (a 100M-token layer), or 64 single-token
 *     queries over 60,000 chunks. A larger call returns MSA_ERR_WORKSPACE
 *     before anything is enqueued.
 *   Every call on one GPU uses the same scratch: calls that overlap on one GPU
 *     (concurrent streams, or host threads) race and give wrong results;
 *     order them on one stream or with events. The scratch keeps the last
 *     call's contents, and nothing in it needs clearing between calls.
 *   The stream must belong to the current device (MSA_ERR_INVALID_ARG
 *     otherwise). The first call on a device looks up that device's scratch
 *     address; that lookup and the library's error string are the only state
 *     the library keeps across calls. */
#define MSA_NOALLOC_SCRATCH_BYTES (16u << 20)
int32_t msa_route_topk_noalloc(const msa_dims* d, const msa_bf16* QR, int32_t B, int32_t M,
                               const msa_bf16* KRbar, const int64_t* doc_chunk_offsets,
                               int32_t n_docs, int64_t n_chunks, float* doc_scores,
                               int32_t accumulate, int32_t* topk_ids, float* topk_scores,
                               int32_t* n_sel, void* stream);

/* The two halves of msa_route_topk, for callers that want the chunk scores
 * themselves (for instance to supervise routing) or to time the scan alone.
 * msa_route_scores: chunk_scores [B, n_chunks] fp32 (written) holds
 *   S_c = max_t (or mean_t) mean_h cos(Q^R_{t,h}, K̄^R_{c,h}) for each query.
 *   Workspace: msa_route_scores_workspace() bytes: partial maxima when a
 *   query's tokens span several row tiles, and the normalised query rows when
 *   M is a multiple of 128 (when M is a multiple of 256 and B·M >= 1024 also
 *   the normalised keys, n_chunks × 2 KiB); 0 otherwise, and then ws may be
 *   NULL.
 * msa_select_topk: reduces chunk_scores [B, n_chunks] to document scores
 *   (max over each document's chunks; max-merged into doc_scores when
 *   accumulate != 0) and selects the top_k documents exactly as
 *   msa_route_topk does. Workspace: msa_select_topk_workspace() bytes. */
size_t msa_route_scores_workspace(const msa_dims* d, int32_t B, int32_t M, int64_t n_chunks);
int32_t msa_route_scores(const msa_dims* d, const msa_bf16* QR, int32_t B, int32_t M,
                         const msa_bf16* KRbar, int64_t n_chunks, float* chunk_scores, void* ws,
                         size_t ws_bytes, void* stream);
size_t msa_select_topk_workspace(const msa_dims* d, int32_t B, int32_t n_docs);
int32_t msa_select_topk(const msa_dims* d, const float* chunk_scores, int32_t B,
                        const int64_t* doc_chunk_offsets, int32_t n_docs, int64_t n_chunks,
                        float* doc_scores, int32_t accumulate, int32_t* topk_ids,
                        float* topk_scores, int32_t* n_sel, void* ws, size_t ws_bytes,
                        void* stream);

/* ------------------------------------------------------------------------ */
/* Stage 3: context assembly, global RoPE and sparse attention (techblg
 * section M, routing bullet: K_ctx = [{K̄_i}_{i∈I}; K_q], V_ctx likewise,
 * Output = Attention(Q_q, K_ctx, V_ctx); positional bullet: the active
 * context uses global RoPE with positions offset from k).
 *   Q [M, n_q_heads, 128] bf16: the M query tokens, which are the last M of
 *     the M_loc local tokens (M <= M_loc).
 *   K_loc, V_loc [M_loc, n_kv_heads, 128] bf16: local (active-context) KV.
 *     K_loc is rotated here at position pos0 + v unless k_loc_rotated != 0.
 *   Kbar, Vbar [n_chunks, n_kv_heads, 128] bf16: pooled memory; device
 *     memory, or pinned host memory when kv_on_host != 0 (read in place over
 *     PCIe by the kernel; pageable memory is MSA_ERR_INVALID_ARG).
 *   doc_chunk_offsets: device int64 [n_docs+1].
 *   sel_ids [top_k] int32 and n_sel [1] int32 (device; as written by
 *     msa_route_topk for one query). Ids outside [0, n_docs) are skipped.
 *   max_sel_chunks: an upper bound on the selected documents' total chunk
 *     count (e.g. top_k × the longest document's chunks); selections beyond
 *     it are truncated to it.
 *   pos0: global position of local token 0; -1 means n_sel (the reading "k").
 *   Query token u (local index M_loc-M+u) sees every selected memory chunk and
 *   local tokens 0..M_loc-M+u; q head h reads KV head h / (n_q_heads /
 *   n_kv_heads); logits are scaled by 1/sqrt(128); softmax in fp32.
 *   out [M, n_q_heads, 128] bf16 (written); out_f32 (may be NULL) receives the
 *   same values in fp32.
 *   ws / ws_bytes: at least msa_sparse_attend_workspace() bytes. */
size_t msa_sparse_attend_workspace(const msa_dims* d, int32_t M, int32_t M_loc,
                                   int64_t max_sel_chunks);
int32_t msa_sparse_attend(const msa_dims* d, const msa_bf16* Q, int32_t M, const msa_bf16* K_loc,
                          const msa_bf16* V_loc, int32_t M_loc, int32_t k_loc_rotated,
                          const msa_bf16* Kbar, const msa_bf16* Vbar, int32_t kv_on_host,
                          int64_t n_chunks, const int64_t* doc_chunk_offsets, int32_t n_docs,
                          const int32_t* sel_ids, const int32_t* n_sel, int64_t max_sel_chunks,
                          int64_t pos0, msa_bf16* out, float* out_f32, void* ws, size_t ws_bytes,
                          void* stream);

/* msa_sparse_attend for B queries of one shape in one set of launches (the
 * same stage, techblg section M routing bullet: each query attends over its
 * own selection and its own local context), e.g. concurrent decode queries
 * routed together by one msa_route_topk call. Each query computes exactly
 * what msa_sparse_attend computes for it alone (bit for bit).
 *   Q [B, M, n_q_heads, 128], K_loc and V_loc [B, M_loc, n_kv_heads, 128]
 *     bf16, packed (query b at b * M and b * M_loc rows); k_loc_rotated as
 *     in msa_sparse_attend, for every query.
 *   Kbar, Vbar, kv_on_host, n_chunks, doc_chunk_offsets, n_docs: the shared
 *     pooled store, as in msa_sparse_attend.
 *   sel_ids [B, top_k] int32 and n_sel [B] int32 (device): each query's
 *     selection, e.g. the topk_ids and n_sel of msa_route_topk.
 *   pos0: as in msa_sparse_attend, the same for every query (-1 means each
 *     query's own n_sel).
 *   out [B, M, n_q_heads, 128] bf16 (written); out_f32 optional, same shape.
 *   ws / ws_bytes: at least msa_sparse_attend_batch_workspace() bytes.
 *   B >= 1; B times the call's key splits must stay within 65,535
 *   (MSA_ERR_SHAPE otherwise; at most 255 queries always fit). Errors as in
 *   msa_sparse_attend. */
size_t msa_sparse_attend_batch_workspace(const msa_dims* d, int32_t B, int32_t M, int32_t M_loc,
                                         int64_t max_sel_chunks);
int32_t msa_sparse_attend_batch(const msa_dims* d, const msa_bf16* Q, int32_t B, int32_t M,
                                const msa_bf16* K_loc, const msa_bf16* V_loc, int32_t M_loc,
                                int32_t k_loc_rotated, const msa_bf16* Kbar, const msa_bf16* Vbar,
                                int32_t kv_on_host, int64_t n_chunks,
                                const int64_t* doc_chunk_offsets, int32_t n_docs,
                                const int32_t* sel_ids, const int32_t* n_sel,
                                int64_t max_sel_chunks, int64_t pos0, msa_bf16* out,
                                float* out_f32, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Memory Interleave (techblg section M, Memory Interleave bullet; chooseai.io
 * section 2.4): one round appends M_new tokens to the active context, routes
 * them (max-merged into the running document scores), re-selects the top-k
 * documents and attends the new tokens over [selected memory; every local
 * token]. The state's buffers belong to the caller.
 *   doc_scores [n_docs] fp32: running scores; set every entry to -inf (or call
 *     msa_interleave_reset) before the first round.
 *   K_loc, V_loc [cap_loc, n_kv_heads, 128] bf16: the raw (unrotated) local
 *     keys/values; the round appends K_new/V_new at row n_loc.
 *   n_loc: tokens already in K_loc/V_loc (host value, advanced by M_new on
 *     success). cap_loc: capacity in tokens (MSA_ERR_SHAPE if exceeded).
 *   topk_ids [top_k] int32, topk_scores [top_k] fp32, n_sel [1] int32: this
 *     round's selection (written).
 *   pos0: as in msa_sparse_attend (-1 means n_sel). */
typedef struct msa_interleave_state {
  float* doc_scores;
  msa_bf16* K_loc;
  msa_bf16* V_loc;
  int32_t cap_loc;
  int32_t n_loc;
  int32_t* topk_ids;
  float* topk_scores;
  int32_t* n_sel;
  int64_t pos0;
} msa_interleave_state;

int32_t msa_interleave_reset(msa_interleave_state* st, int32_t n_docs, void* stream);
size_t msa_interleave_step_workspace(const msa_dims* d, int32_t M_new, int32_t cap_loc,
                                     int64_t n_chunks, int32_t n_docs, int64_t max_sel_chunks);
int32_t msa_interleave_step(const msa_dims* d, msa_interleave_state* st, const msa_bf16* Q_new,
                            const msa_bf16* K_new, const msa_bf16* V_new, const msa_bf16* QR_new,
                            int32_t M_new, const msa_bf16* KRbar, const msa_bf16* Kbar,
                            const msa_bf16* Vbar, int32_t kv_on_host, int64_t n_chunks,
                            const int64_t* doc_chunk_offsets, int32_t n_docs,
                            int64_t max_sel_chunks, msa_bf16* out, void* ws, size_t ws_bytes,
                            void* stream);

/* Memory Interleave for B queries that advance together (same sections as
 * above): one round routes the B queries' new tokens in one batched scan
 * (each query max-merges into its own running document scores), re-selects
 * each query's top-k and attends each query's new tokens over its own
 * selection and local context. One scan launch covers every query's rows; the
 * results equal B msa_interleave_step calls on the same inputs bit for bit
 * when M_new > 1 (a single query of one row takes the fp32-exact VALU scan
 * instead, which may differ in the last bits). Buffers belong to the
 * caller (1 <= B <= 65535, MSA_ERR_SHAPE otherwise):
 *   doc_scores [B, n_docs] fp32 (msa_interleave_batch_reset sets -inf);
 *   K_loc, V_loc [B, cap_loc, n_kv_heads, 128] bf16, query b's rows at
 *     b * cap_loc; every query holds n_loc tokens (host value, advanced by
 *     M_new on success; MSA_ERR_SHAPE if n_loc + M_new > cap_loc);
 *   topk_ids [B, top_k] int32, topk_scores [B, top_k] fp32, n_sel [B] int32:
 *     this round's selections (written);
 *   pos0: as in msa_sparse_attend, the same for every query (-1 means each
 *     query's own n_sel).
 * Step inputs: Q_new [B, M_new, n_q_heads, 128], K_new and V_new [B, M_new,
 * n_kv_heads, 128], QR_new [B, M_new, n_router_heads, 128] bf16 (device); out
 * [B, M_new, n_q_heads, 128] bf16 (written). ws / ws_bytes: at least
 * msa_interleave_batch_step_workspace() bytes. On error nothing in the state
 * has changed unless the message says the error came from a launch. */
typedef struct msa_interleave_batch {
  float* doc_scores;
  msa_bf16* K_loc;
  msa_bf16* V_loc;
  int32_t B;
  int32_t cap_loc;
  int32_t n_loc;
  int32_t* topk_ids;
  float* topk_scores;
  int32_t* n_sel;
  int64_t pos0;
} msa_interleave_batch;

int32_t msa_interleave_batch_reset(msa_interleave_batch* st, int32_t n_docs, void* stream);
size_t msa_interleave_batch_step_workspace(const msa_dims* d, int32_t B, int32_t M_new,
                                           int32_t cap_loc, int64_t n_chunks, int32_t n_docs,
                                           int64_t max_sel_chunks);
int32_t msa_interleave_batch_step(const msa_dims* d, msa_interleave_batch* st,
                                  const msa_bf16* Q_new, const msa_bf16* K_new,
                                  const msa_bf16* V_new, const msa_bf16* QR_new, int32_t M_new,
                                  const msa_bf16* KRbar, const msa_bf16* Kbar,
                                  const msa_bf16* Vbar, int32_t kv_on_host, int64_t n_chunks,
                                  const int64_t* doc_chunk_offsets, int32_t n_docs,
                                  int64_t max_sel_chunks, msa_bf16* out, void* ws,
                                  size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Router supervision: the auxiliary contrastive loss of the pages and its
 * gradient (techblg section M, training bullet: L_aux = −(1/|P|) Σ_i log[
 * exp(s_i⁺/τ) / (exp(s_i⁺/τ) + Σ_j exp(s_ij⁻/τ)) ], applied to every routed
 * layer; τ fixed, its value not given). Readings: s are the query's routing
 * document scores (max over a document's chunks of the max over query tokens
 * of the head-mean cosine); the negatives of every positive are all other
 * documents of the store; τ is a parameter; through the two maxima the
 * gradient reaches one (chunk, token) pair per document — the first chunk
 * attaining the document score (by the routing scan's chunk scores) and, in
 * it, the first token attaining the chunk score (recomputed in fp32, which
 * also gives the s used in the loss).
 *   QR [B, M, n_router_heads, 128] bf16; KRbar [n_chunks, n_router_heads, 128]
 *     bf16; doc_chunk_offsets [n_docs+1] (device).
 *   pos_ids [B, max_pos] int32, n_pos [B] int32 (device): query b's positives
 *     are pos_ids[b][0 .. n_pos[b]); ids outside [0, n_docs) are ignored and
 *     repeats count once; a query with no valid positive gets loss 0 and no
 *     gradient.
 *   tau > 0 (MSA_ERR_INVALID_ARG otherwise). token_reduce must be MAX
 *     (MEAN is MSA_ERR_UNSUPPORTED).
 *   loss [B] fp32 (written). dQR [B, M, n_router_heads, 128] fp32 and dKRbar
 *     [n_chunks, n_router_heads, 128] fp32 (written densely: rows without
 *     gradient are 0; dKRbar sums over the B queries). doc_scores [B, n_docs]
 *     fp32 (written; may be NULL). best_chunk, best_token [B, n_docs] int32
 *     (written; may be NULL): the (chunk, token) pair each document's
 *     gradient went to. Only chunks inside a document are written in dKRbar.
 *   Results are deterministic (fixed reduction orders, no atomics). */
size_t msa_route_aux_loss_workspace(const msa_dims* d, int32_t B, int32_t M, int64_t n_chunks,
                                    int32_t n_docs);
int32_t msa_route_aux_loss(const msa_dims* d, const msa_bf16* QR, int32_t B, int32_t M,
                           const msa_bf16* KRbar, const int64_t* doc_chunk_offsets,
                           int32_t n_docs, int64_t n_chunks, const int32_t* pos_ids,
                           const int32_t* n_pos, int32_t max_pos, float tau, float* loss,
                           float* dQR, float* dKRbar, float* doc_scores, int32_t* best_chunk,
                           int32_t* best_token, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Streaming memory update: a pooled store that grows by whole documents
 * without re-encoding what it holds, and its save/load. The pages name the
 * offline encoding cost of a knowledge base that keeps changing as a
 * limitation and incremental encoding as a future direction
 * (paper.rainbus.top, limitations and future-directions sections); pooling
 * is per document (techblg section M, routing bullet), so appending the
 * pooled rows of new documents gives exactly the store of the whole corpus.
 *
 * The caller owns every buffer, sized for capacity:
 *   Kbar, Vbar [cap_chunks, n_kv_heads, 128] bf16: device memory, or pinned
 *     host memory (the K̄/V̄ host tier); either may be NULL (not kept).
 *   KRbar [cap_chunks, n_router_heads, 128] bf16, device; may be NULL.
 *   doc_chunk_offsets [cap_docs+1] int64, device; doc_chunk_offsets_h, its
 *     host mirror [cap_docs+1] (pinned memory keeps the uploads asynchronous).
 * n_docs / n_chunks are host fields maintained by the calls below; rows
 * [0, n_chunks) and offsets [0, n_docs] are valid once the stream that last
 * wrote them has been synchronised. The store is used by the routing and
 * attention calls like any pooled memory (KRbar, Kbar, Vbar, n_chunks,
 * doc_chunk_offsets, n_docs). */
typedef struct msa_store {
  msa_bf16* Kbar;
  msa_bf16* Vbar;
  msa_bf16* KRbar;
  int64_t* doc_chunk_offsets;
  int64_t* doc_chunk_offsets_h;
  int64_t cap_chunks;
  int32_t cap_docs;
  int32_t n_docs;
  int64_t n_chunks;
} msa_store;

/* Empties the store: n_docs = n_chunks = 0 and offset 0 (host and device)
 * set to 0. */
int32_t msa_store_reset(msa_store* st, void* stream);

/* Appends n_new documents. K, V, KR [n_new_tokens, H, 128] bf16 (device) are
 * their raw states (an input may be NULL when the store does not keep that
 * tensor); doc_token_offsets [n_new+1] (device) and doc_token_offsets_h (host)
 * are their token offsets from 0. The new documents get ids n_docs ..
 * n_docs+n_new-1 and chunks n_chunks .. ; their rows are pooled exactly as
 * msa_encode_pool does. MSA_ERR_SHAPE (store unchanged) if the documents or
 * chunks exceed the capacity; pinned host Kbar/Vbar are written over PCIe. */
int32_t msa_store_append(const msa_dims* d, msa_store* st, const msa_bf16* K, const msa_bf16* V,
                         const msa_bf16* KR, const int64_t* doc_token_offsets,
                         const int64_t* doc_token_offsets_h, int32_t n_new,
                         int64_t n_new_tokens, void* stream);

/* Store file (little-endian): a 64-byte header — magic "MSASTOR1", u32
 * version (1), u32 header bytes (64), i32 n_docs, i32 chunk, i64 n_chunks,
 * i32 heads, i32 head_dim, u32 tensor mask (1 = K̄^R, 2 = K̄, 4 = V̄),
 * i32 doc_rope_mode, f32 rope_theta, 12 reserved bytes — then the offsets
 * int64 [n_docs+1], then the present tensors in the order K̄^R, K̄, V̄, each
 * [n_chunks, heads, head_dim] bf16.
 *
 * msa_store_save writes the store's non-NULL tensors; msa_store_load reads a
 * file into a store whose non-NULL tensors must all be in the file and whose
 * capacity must hold it (MSA_ERR_SHAPE), with matching chunk size, heads and
 * head_dim, and, when K̄ is loaded, matching RoPE settings (MSA_ERR_SHAPE).
 * Both are synchronous (they return when the data is on disk / in the store)
 * and move the data through the caller's staging buffer (host memory, pinned
 * for speed, at least 1 MiB). msa_store_file_info reads only the header (no
 * GPU involved). Any read/write failure or malformed file is MSA_ERR_IO.
 * Exception to the no-partial-output rule: a load that fails after the
 * header and offsets were accepted (a truncated tensor section) leaves the
 * store empty (n_docs = n_chunks = 0). */
int32_t msa_store_save(const msa_dims* d, const msa_store* st, const char* path,
                       void* staging_h, size_t staging_bytes);
int32_t msa_store_load(const msa_dims* d, msa_store* st, const char* path, void* staging_h,
                       size_t staging_bytes);
int32_t msa_store_file_info(const char* path, int32_t* n_docs, int64_t* n_chunks,
                            uint32_t* tensor_mask);

#ifdef __cplusplus
}
#endif
#endif /* MSA_H */
