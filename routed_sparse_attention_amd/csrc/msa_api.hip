// C entry points of the MSA library: argument validation, workspace layout,
// kernel selection and error reporting. Every check runs before anything is
// enqueued, so a failed call leaves outputs untouched.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "msa_internal.h"

namespace msa {

static thread_local char g_err[1024] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = '\0'; }

int hip_fail(hipError_t e, const char* what) {
  return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int misaligned16(const char* call, const char* name) {
  return fail(MSA_ERR_INVALID_ARG, "%s: %s must start at a 16-byte aligned address", call, name);
}

int check_dims(const msa_dims* d) {
  if (d == nullptr) return fail(MSA_ERR_INVALID_ARG, "dims is NULL");
  if (d->head_dim != kDim)
    return fail(MSA_ERR_UNSUPPORTED, "head_dim %d unsupported (only 128)", d->head_dim);
  if (d->n_kv_heads != kHeads || d->n_router_heads != kHeads)
    return fail(MSA_ERR_UNSUPPORTED, "n_kv_heads=%d n_router_heads=%d unsupported (only 8)",
                d->n_kv_heads, d->n_router_heads);
  if (d->n_q_heads < kHeads || d->n_q_heads > 64 || d->n_q_heads % kHeads != 0)
    return fail(MSA_ERR_SHAPE, "n_q_heads=%d must be a multiple of 8 in [8, 64]", d->n_q_heads);
  if (d->chunk < 1 || d->chunk > 4096)
    return fail(MSA_ERR_SHAPE, "chunk=%d out of [1, 4096]", d->chunk);
  if (d->top_k < 1 || d->top_k > 64) return fail(MSA_ERR_SHAPE, "top_k=%d out of [1, 64]", d->top_k);
  if (!(d->rope_theta > 1.0f) || !std::isfinite(d->rope_theta))
    return fail(MSA_ERR_INVALID_ARG, "rope_theta must be finite and > 1");
  if (d->token_reduce != MSA_TOKEN_REDUCE_MAX && d->token_reduce != MSA_TOKEN_REDUCE_MEAN)
    return fail(MSA_ERR_INVALID_ARG, "token_reduce=%d unknown", d->token_reduce);
  if (d->doc_rope_mode != MSA_DOC_ROPE_TOKEN && d->doc_rope_mode != MSA_DOC_ROPE_CHUNK)
    return fail(MSA_ERR_INVALID_ARG, "doc_rope_mode=%d unknown", d->doc_rope_mode);
  return MSA_OK;
}

// Resolves a K̄/V̄ pointer: device memory as is, pinned host memory to its
// device-visible address; pageable host memory is rejected.
int resolve_kv(const void* p, int on_host, const void** out, const char* name) {
  hipPointerAttribute_t attr;
  std::memset(&attr, 0, sizeof(attr));
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(MSA_ERR_INVALID_ARG, "%s: not a HIP allocation (%s)", name, hipGetErrorString(e));
  }
  if (on_host) {
    if (attr.type != hipMemoryTypeHost || attr.devicePointer == nullptr)
      return fail(MSA_ERR_INVALID_ARG, "%s: kv_on_host needs pinned host memory", name);
    // devicePointer is the mapping of the allocation's base; keep the offset.
    const char* host_base = static_cast<const char*>(attr.hostPointer);
    const char* dev_base = static_cast<const char*>(attr.devicePointer);
    if (host_base != nullptr)
      *out = dev_base + (static_cast<const char*>(p) - host_base);
    else
      *out = p;
  } else {
    if (attr.type != hipMemoryTypeDevice)
      return fail(MSA_ERR_INVALID_ARG, "%s: expected device memory (pass kv_on_host=1 for "
                  "pinned host memory)", name);
    *out = p;
  }
  return MSA_OK;
}

// resolve_kv with the memory kind taken from the pointer itself.
int resolve_any(const void* p, const void** out, const char* name) {
  hipPointerAttribute_t attr;
  std::memset(&attr, 0, sizeof(attr));
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(MSA_ERR_INVALID_ARG, "%s: not a HIP allocation (%s)", name, hipGetErrorString(e));
  }
  return resolve_kv(p, attr.type == hipMemoryTypeHost ? 1 : 0, out, name);
}

namespace {

// Scan plan: kernel choice and the workspace it needs. Queries whose token
// count M is a multiple of 128 take the tiled contraction (msa_route_gemm.hip;
// the choice depends on M alone, so a query gives the same scores alone or in
// a batch); otherwise a single row in all (decode) takes the fp32-exact VALU
// scan and more rows the batched MFMA scan. A query whose rows span several row tiles needs the
// partials buffer; the tiled scan also needs the normalised query rows.
enum ScanKind { kScanValu, kScanMfma, kScanGemm };
struct ScanPlan {
  ScanKind kind;
  RouteGeom g;
  size_t parts_bytes;
  size_t qhat_bytes;
};

ScanPlan scan_plan(int32_t B, int32_t M, int64_t C) {
  ScanPlan p;
  p.qhat_bytes = 0;
  if (scan_gemm_fits(M)) {
    p.kind = kScanGemm;
    p.g = route_geom(B, M, M);                 // B, M; parts set below
    p.g.parts = scan_gemm_parts(M);
    p.qhat_bytes = scan_gemm_ws_bytes(B, M, C);
  } else {
    p.kind = (int64_t)B * M > kValuTileRows ? kScanMfma : kScanValu;
    p.g = route_geom(B, M, p.kind == kScanMfma ? kMfmaTileRows : kValuTileRows);
  }
  p.parts_bytes = p.g.parts > 1 ? align_up((size_t)p.g.parts * B * C * sizeof(float), 256) : 0;
  return p;
}

int route_scores_impl(const msa_dims* d, const msa_bf16* QR, int32_t B, int32_t M,
                      const msa_bf16* KRbar, int64_t n_chunks, float* S, void* ws, size_t ws_bytes,
                      hipStream_t s) {
  const ScanPlan p = scan_plan(B, M, n_chunks);
  if (p.kind != kScanGemm && p.g.n_tiles > 65535)
    return fail(MSA_ERR_SHAPE, "route: %d row tiles exceed the grid limit (65535)", p.g.n_tiles);
  const size_t need = p.parts_bytes + p.qhat_bytes;
  if (ws_bytes < need || (need && ws == nullptr))
    return fail(MSA_ERR_WORKSPACE, "route scores workspace: need %zu bytes, got %zu", need,
                ws_bytes);
  float* dst = p.g.parts > 1 ? static_cast<float*>(ws) : S;
  int rc;
  if (p.kind == kScanGemm) {
    uint16_t* qhat = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + p.parts_bytes);
    rc = launch_scan_gemm(QR, B, M, KRbar, n_chunks, d->token_reduce, dst, qhat, s);
  } else if (p.kind == kScanMfma) {
    rc = launch_scan_mfma(QR, p.g, KRbar, n_chunks, d->token_reduce, dst, s);
  } else {
    rc = launch_scan_valu(QR, p.g, KRbar, n_chunks, d->token_reduce, dst, s);
  }
  if (rc) return rc;
  if (p.g.parts > 1) return launch_parts_combine(dst, p.g, n_chunks, d->token_reduce, S, s);
  return MSA_OK;
}

}  // namespace

size_t route_topk_ws(int32_t B, int32_t M, int64_t C, int32_t N, int32_t K) {
  const ScanPlan p = scan_plan(B, M, C);
  const size_t sbytes = align_up((size_t)B * C * sizeof(float), 256);
  return sbytes + p.parts_bytes + p.qhat_bytes + doc_topk_workspace(B, N, K);
}

int route_topk_impl(const msa_dims* d, const msa_bf16* QR, int32_t B, int32_t M,
                    const msa_bf16* KRbar, const int64_t* dco, int32_t n_docs, int64_t n_chunks,
                    float* doc_scores, int32_t accumulate, int32_t* topk_ids, float* topk_scores,
                    int32_t* n_sel, void* ws, size_t ws_bytes, hipStream_t s) {
  const size_t need = route_topk_ws(B, M, n_chunks, n_docs, d->top_k);
  if (ws == nullptr || ws_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "route workspace: need %zu bytes, got %zu", need, ws_bytes);
  const ScanPlan p = scan_plan(B, M, n_chunks);
  char* base = static_cast<char*>(ws);
  const size_t sbytes = align_up((size_t)B * n_chunks * sizeof(float), 256);
  float* S = reinterpret_cast<float*>(base);
  uint64_t* cand = reinterpret_cast<uint64_t*>(base + sbytes + p.parts_bytes + p.qhat_bytes);
  int rc = route_scores_impl(d, QR, B, M, KRbar, n_chunks, S, base + sbytes,
                             p.parts_bytes + p.qhat_bytes, s);
  if (rc) return rc;
  return launch_doc_topk(S, B, n_chunks, dco, n_docs, doc_scores, accumulate, d->top_k, cand,
                         topk_ids, topk_scores, n_sel, s);
}

int check_route_args(const msa_dims* d, const msa_bf16* QR, int32_t B, int32_t M,
                     const msa_bf16* KRbar, const int64_t* dco, int32_t n_docs, int64_t n_chunks,
                     const float* doc_scores, int32_t accumulate, const int32_t* topk_ids,
                     const float* topk_scores, const int32_t* n_sel) {
  if (!QR || !KRbar || !dco || !doc_scores || !topk_ids || !topk_scores || !n_sel)
    return fail(MSA_ERR_INVALID_ARG, "route: NULL pointer argument");
  if (B < 1 || M < 1 || B > 65535)
    return fail(MSA_ERR_SHAPE, "route: B=%d M=%d must be >= 1 (B <= 65535)", B, M);
  if ((int64_t)B * M > (1 << 24)) return fail(MSA_ERR_SHAPE, "route: B*M too large");
  if (n_docs < 1) return fail(MSA_ERR_SHAPE, "route: n_docs=%d must be >= 1", n_docs);
  if (n_chunks < n_docs || n_chunks >= ((int64_t)1 << 31))
    return fail(MSA_ERR_SHAPE, "route: n_chunks=%lld must be in [n_docs, 2^31)",
                (long long)n_chunks);
  if (accumulate && d->token_reduce == MSA_TOKEN_REDUCE_MEAN)
    return fail(MSA_ERR_UNSUPPORTED, "route: accumulate needs the MAX token reduction");
  MSA_A16("route", QR);
  MSA_A16("route", KRbar);
  return MSA_OK;
}

namespace {

int check_attend_args(const msa_dims* d, const msa_bf16* Q, int32_t M, const msa_bf16* K_loc,
                      const msa_bf16* V_loc, int32_t M_loc, const msa_bf16* Kbar,
                      const msa_bf16* Vbar, int64_t n_chunks, const int64_t* dco, int32_t n_docs,
                      const int32_t* sel_ids, const int32_t* n_sel, int64_t max_sel_chunks,
                      const msa_bf16* out) {
  (void)d;
  if (!Q || !K_loc || !V_loc || !Kbar || !Vbar || !dco || !sel_ids || !n_sel || !out)
    return fail(MSA_ERR_INVALID_ARG, "attend: NULL pointer argument");
  if (M < 1 || M_loc < M)
    return fail(MSA_ERR_SHAPE, "attend: need 1 <= M (%d) <= M_loc (%d)", M, M_loc);
  if ((int64_t)M_loc > (1 << 20)) return fail(MSA_ERR_SHAPE, "attend: M_loc too large");
  if (n_docs < 1) return fail(MSA_ERR_SHAPE, "attend: n_docs=%d must be >= 1", n_docs);
  if (n_chunks < n_docs || n_chunks >= ((int64_t)1 << 31))
    return fail(MSA_ERR_SHAPE, "attend: n_chunks=%lld must be in [n_docs, 2^31)",
                (long long)n_chunks);
  if (max_sel_chunks < 0 || max_sel_chunks > ((int64_t)1 << 24))
    return fail(MSA_ERR_SHAPE, "attend: max_sel_chunks=%lld out of [0, 2^24]",
                (long long)max_sel_chunks);
  MSA_A16("attend", Q);
  MSA_A16("attend", K_loc);
  MSA_A16("attend", V_loc);
  MSA_A16("attend", Kbar);
  MSA_A16("attend", Vbar);
  MSA_A16("attend", out);
  return MSA_OK;
}

// Memory Interleave appends each query's new K and V rows to its local
// context: nb queries' rows [0, n_vec) (16-byte vectors) of src + b·src_stride
// go to dst + b·dst_stride, K and V in one launch (blockIdx.y: 0 = K, 1 = V,
// blockIdx.z: query). One launch for a whole batched round instead of a copy
// call per query and tensor (each a kernel of its own, ~4 µs apiece).
__global__ __launch_bounds__(256) void append_rows_kernel(const uint4* __restrict__ K_src,
                                                          const uint4* __restrict__ V_src,
                                                          uint4* __restrict__ K_dst,
                                                          uint4* __restrict__ V_dst, int64_t n_vec,
                                                          int64_t src_stride, int64_t dst_stride) {
  const int64_t b = blockIdx.z;
  const uint4* src = (blockIdx.y ? V_src : K_src) + b * src_stride;
  uint4* dst = (blockIdx.y ? V_dst : K_dst) + b * dst_stride;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_vec;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

// Rows [0, M_new) of query b's K_new / V_new (query stride M_new rows) to rows
// [n_loc, n_loc + M_new) of its local buffers (query stride cap_loc rows).
int launch_append_rows(const msa_bf16* K_new, const msa_bf16* V_new, msa_bf16* K_loc,
                       msa_bf16* V_loc, int32_t B, int32_t M_new, int32_t n_loc,
                       int32_t cap_loc, hipStream_t s) {
  constexpr int64_t kRowVec = kRowElems * 2 / 16;        // 16-byte vectors per KV row
  const int64_t n_vec = (int64_t)M_new * kRowVec;
  if (B > 65535) return fail(MSA_ERR_SHAPE, "interleave: B=%d exceeds 65535 queries", B);
  if (B < 1 || n_vec < 1) return MSA_OK;
  const int64_t blocks = std::min<int64_t>((n_vec + 255) / 256, 1024);
  const int64_t at = (int64_t)n_loc * kRowVec;
  hipLaunchKernelGGL(append_rows_kernel, dim3((unsigned)blocks, 2, (unsigned)B), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(K_new), reinterpret_cast<const uint4*>(V_new),
                     reinterpret_cast<uint4*>(K_loc) + at, reinterpret_cast<uint4*>(V_loc) + at,
                     n_vec, n_vec, (int64_t)cap_loc * kRowVec);
  MSA_LAUNCH_CHECK("append_rows_kernel launch");
  return MSA_OK;
}

}  // namespace
}  // namespace msa

using namespace msa;

extern "C" {

void msa_default_dims(msa_dims* d) {
  if (!d) return;
  d->n_kv_heads = 8;
  d->n_router_heads = 8;
  d->n_q_heads = 32;
  d->head_dim = 128;
  d->chunk = 64;
  d->top_k = 16;
  d->rope_theta = 1.0e6f;
  d->token_reduce = MSA_TOKEN_REDUCE_MAX;
  d->doc_rope_mode = MSA_DOC_ROPE_TOKEN;
}

const char* msa_last_error(void) { return g_err; }

int32_t msa_abi_version(void) { return MSA_ABI_VERSION; }

int32_t msa_plan_chunks(const int64_t* dto_h, int32_t n_docs, int32_t chunk, int64_t* dco_h) {
  clear_error();
  if (!dto_h || !dco_h) return fail(MSA_ERR_INVALID_ARG, "plan_chunks: NULL pointer argument");
  if (n_docs < 0) return fail(MSA_ERR_SHAPE, "plan_chunks: n_docs=%d < 0", n_docs);
  if (chunk < 1) return fail(MSA_ERR_SHAPE, "plan_chunks: chunk=%d < 1", chunk);
  if (dto_h[0] < 0) return fail(MSA_ERR_SHAPE, "plan_chunks: negative first offset");
  for (int32_t i = 0; i < n_docs; ++i)
    if (dto_h[i + 1] - dto_h[i] < 1)
      return fail(MSA_ERR_SHAPE, "plan_chunks: document %d has %lld tokens (needs >= 1)", i,
                  (long long)(dto_h[i + 1] - dto_h[i]));
  int64_t acc = 0;
  dco_h[0] = 0;
  for (int32_t i = 0; i < n_docs; ++i) {
    const int64_t n = dto_h[i + 1] - dto_h[i];
    acc += (n + chunk - 1) / chunk;
    dco_h[i + 1] = acc;
  }
  return MSA_OK;
}

size_t msa_encode_pool_workspace(const msa_dims* d, int32_t n_docs, int64_t n_chunks) {
  (void)d; (void)n_docs; (void)n_chunks;
  return 0;
}

int32_t msa_encode_pool(const msa_dims* d, const msa_bf16* K, const msa_bf16* V,
                        const msa_bf16* KR, const int64_t* dto, const int64_t* dco, int32_t n_docs,
                        int64_t n_tokens, int64_t n_chunks, msa_bf16* Kbar, msa_bf16* Vbar,
                        msa_bf16* KRbar, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  (void)ws; (void)ws_bytes;
  int rc = check_dims(d);
  if (rc) return rc;
  if (!dto || !dco) return fail(MSA_ERR_INVALID_ARG, "encode_pool: NULL offsets");
  if ((Kbar && !K) || (Vbar && !V) || (KRbar && !KR))
    return fail(MSA_ERR_INVALID_ARG, "encode_pool: an output is requested without its input");
  if (n_docs < 1) return fail(MSA_ERR_SHAPE, "encode_pool: n_docs=%d must be >= 1", n_docs);
  if (n_tokens < n_docs) return fail(MSA_ERR_SHAPE, "encode_pool: n_tokens < n_docs");
  if (n_chunks < n_docs || n_chunks > n_tokens)
    return fail(MSA_ERR_SHAPE, "encode_pool: n_chunks=%lld must be in [n_docs, n_tokens]",
                (long long)n_chunks);
  if (n_chunks / 8 >= ((int64_t)1 << 31)) return fail(MSA_ERR_SHAPE, "encode_pool: too many chunks");
  MSA_A16("encode_pool", K);
  MSA_A16("encode_pool", V);
  MSA_A16("encode_pool", KR);
  MSA_A16("encode_pool", Kbar);
  MSA_A16("encode_pool", Vbar);
  MSA_A16("encode_pool", KRbar);
  PoolArgs a;
  a.K = K; a.V = V; a.KR = KR; a.dto = dto; a.dco = dco;
  a.n_docs = n_docs; a.n_tokens = n_tokens; a.n_chunks = n_chunks; a.chunk = d->chunk;
  a.chunk_base = 0;
  a.theta = (double)d->rope_theta; a.rope_mode = d->doc_rope_mode;
  a.Kbar = Kbar; a.Vbar = Vbar; a.KRbar = KRbar;
  return launch_pool(a, static_cast<hipStream_t>(stream));
}

size_t msa_route_scores_workspace(const msa_dims* d, int32_t B, int32_t M, int64_t n_chunks) {
  if (!d || B < 1 || M < 1 || n_chunks < 1) return 0;
  const ScanPlan p = scan_plan(B, M, n_chunks);
  return p.parts_bytes + p.qhat_bytes;
}

int32_t msa_route_scores(const msa_dims* d, const msa_bf16* QR, int32_t B, int32_t M,
                         const msa_bf16* KRbar, int64_t n_chunks, float* chunk_scores, void* ws,
                         size_t ws_bytes, void* stream) {
  clear_error();
  int rc = check_dims(d);
  if (rc) return rc;
  if (!QR || !KRbar || !chunk_scores) return fail(MSA_ERR_INVALID_ARG, "route_scores: NULL pointer");
  if (B < 1 || M < 1) return fail(MSA_ERR_SHAPE, "route_scores: B=%d M=%d must be >= 1", B, M);
  if ((int64_t)B * M > (1 << 24)) return fail(MSA_ERR_SHAPE, "route_scores: B*M too large");
  if (n_chunks < 1 || n_chunks >= ((int64_t)1 << 31))
    return fail(MSA_ERR_SHAPE, "route_scores: n_chunks=%lld out of [1, 2^31)", (long long)n_chunks);
  MSA_A16("route_scores", QR);
  MSA_A16("route_scores", KRbar);
  return route_scores_impl(d, QR, B, M, KRbar, n_chunks, chunk_scores, ws, ws_bytes,
                           static_cast<hipStream_t>(stream));
}

size_t msa_select_topk_workspace(const msa_dims* d, int32_t B, int32_t n_docs) {
  if (!d || B < 1 || n_docs < 1 || d->top_k < 1) return 0;
  return doc_topk_workspace(B, n_docs, d->top_k);
}

int32_t msa_select_topk(const msa_dims* d, const float* chunk_scores, int32_t B, const int64_t* dco,
                        int32_t n_docs, int64_t n_chunks, float* doc_scores, int32_t accumulate,
                        int32_t* topk_ids, float* topk_scores, int32_t* n_sel, void* ws,
                        size_t ws_bytes, void* stream) {
  clear_error();
  int rc = check_dims(d);
  if (rc) return rc;
  if (!chunk_scores || !dco || !doc_scores || !topk_ids || !topk_scores || !n_sel)
    return fail(MSA_ERR_INVALID_ARG, "select_topk: NULL pointer argument");
  if (B < 1 || B > 65535) return fail(MSA_ERR_SHAPE, "select_topk: B=%d out of [1, 65535]", B);
  if (n_docs < 1) return fail(MSA_ERR_SHAPE, "select_topk: n_docs=%d must be >= 1", n_docs);
  if (n_chunks < n_docs || n_chunks >= ((int64_t)1 << 31))
    return fail(MSA_ERR_SHAPE, "select_topk: n_chunks=%lld must be in [n_docs, 2^31)",
                (long long)n_chunks);
  const size_t need = doc_topk_workspace(B, n_docs, d->top_k);
  if (need && (ws == nullptr || ws_bytes < need))
    return fail(MSA_ERR_WORKSPACE, "select_topk workspace: need %zu bytes, got %zu", need, ws_bytes);
  return launch_doc_topk(chunk_scores, B, n_chunks, dco, n_docs, doc_scores, accumulate, d->top_k,
                         static_cast<uint64_t*>(ws), topk_ids, topk_scores, n_sel,
                         static_cast<hipStream_t>(stream));
}

size_t msa_route_topk_workspace(const msa_dims* d, int32_t B, int32_t M, int64_t n_chunks,
                                int32_t n_docs) {
  if (!d || B < 1 || M < 1 || n_chunks < 1 || n_docs < 1) return 0;
  return route_topk_ws(B, M, n_chunks, n_docs, d->top_k);
}

int32_t msa_route_topk(const msa_dims* d, const msa_bf16* QR, int32_t B, int32_t M,
                       const msa_bf16* KRbar, const int64_t* dco, int32_t n_docs, int64_t n_chunks,
                       float* doc_scores, int32_t accumulate, int32_t* topk_ids,
                       float* topk_scores, int32_t* n_sel, void* ws, size_t ws_bytes,
                       void* stream) {
  clear_error();
  int rc = check_dims(d);
  if (rc) return rc;
  rc = check_route_args(d, QR, B, M, KRbar, dco, n_docs, n_chunks, doc_scores, accumulate,
                        topk_ids, topk_scores, n_sel);
  if (rc) return rc;
  return route_topk_impl(d, QR, B, M, KRbar, dco, n_docs, n_chunks, doc_scores, accumulate,
                         topk_ids, topk_scores, n_sel, ws, ws_bytes,
                         static_cast<hipStream_t>(stream));
}

size_t msa_sparse_attend_workspace(const msa_dims* d, int32_t M, int32_t M_loc,
                                   int64_t max_sel_chunks) {
  if (!d || M < 1 || M_loc < M || max_sel_chunks < 0) return 0;
  return attend_workspace(M, M_loc, d->n_q_heads, max_sel_chunks);
}

int32_t msa_sparse_attend(const msa_dims* d, const msa_bf16* Q, int32_t M, const msa_bf16* K_loc,
                          const msa_bf16* V_loc, int32_t M_loc, int32_t k_loc_rotated,
                          const msa_bf16* Kbar, const msa_bf16* Vbar, int32_t kv_on_host,
                          int64_t n_chunks, const int64_t* dco, int32_t n_docs,
                          const int32_t* sel_ids, const int32_t* n_sel, int64_t max_sel_chunks,
                          int64_t pos0, msa_bf16* out, float* out_f32, void* ws, size_t ws_bytes,
                          void* stream) {
  clear_error();
  int rc = check_dims(d);
  if (rc) return rc;
  rc = check_attend_args(d, Q, M, K_loc, V_loc, M_loc, Kbar, Vbar, n_chunks, dco, n_docs, sel_ids,
                         n_sel, max_sel_chunks, out);
  if (rc) return rc;
  const size_t need = attend_workspace(M, M_loc, d->n_q_heads, max_sel_chunks);
  if (ws == nullptr || ws_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "attend workspace: need %zu bytes, got %zu", need, ws_bytes);
  const void* kb = nullptr;
  const void* vb = nullptr;
  rc = resolve_kv(Kbar, kv_on_host, &kb, "Kbar");
  if (rc) return rc;
  rc = resolve_kv(Vbar, kv_on_host, &vb, "Vbar");
  if (rc) return rc;
  AttendArgs a;
  a.Q = Q; a.M = M; a.n_q_heads = d->n_q_heads;
  a.K_loc = K_loc; a.V_loc = V_loc; a.M_loc = M_loc; a.k_loc_rotated = k_loc_rotated;
  a.Kbar = static_cast<const uint16_t*>(kb); a.Vbar = static_cast<const uint16_t*>(vb);
  a.n_chunks = n_chunks; a.dco = dco; a.n_docs = n_docs;
  a.sel_ids = sel_ids; a.n_sel = n_sel; a.top_k = d->top_k;
  a.max_sel_chunks = max_sel_chunks; a.pos0 = pos0; a.theta = (double)d->rope_theta;
  a.kv_on_host = kv_on_host ? 1 : 0;
  a.out = out; a.out_f32 = out_f32;
  return launch_attend(a, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

size_t msa_sparse_attend_batch_workspace(const msa_dims* d, int32_t B, int32_t M, int32_t M_loc,
                                         int64_t max_sel_chunks) {
  if (!d || B < 1 || M < 1 || M_loc < M || max_sel_chunks < 0) return 0;
  return attend_workspace(M, M_loc, d->n_q_heads, max_sel_chunks, B);
}

int32_t msa_sparse_attend_batch(const msa_dims* d, const msa_bf16* Q, int32_t B, int32_t M,
                                const msa_bf16* K_loc, const msa_bf16* V_loc, int32_t M_loc,
                                int32_t k_loc_rotated, const msa_bf16* Kbar, const msa_bf16* Vbar,
                                int32_t kv_on_host, int64_t n_chunks, const int64_t* dco,
                                int32_t n_docs, const int32_t* sel_ids, const int32_t* n_sel,
                                int64_t max_sel_chunks, int64_t pos0, msa_bf16* out,
                                float* out_f32, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  int rc = check_dims(d);
  if (rc) return rc;
  if (B < 1) return fail(MSA_ERR_SHAPE, "attend_batch: B=%d must be >= 1", B);
  rc = check_attend_args(d, Q, M, K_loc, V_loc, M_loc, Kbar, Vbar, n_chunks, dco, n_docs, sel_ids,
                         n_sel, max_sel_chunks, out);
  if (rc) return rc;
  const size_t need = attend_workspace(M, M_loc, d->n_q_heads, max_sel_chunks, B);
  if (ws == nullptr || ws_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "attend_batch workspace: need %zu bytes, got %zu", need,
                ws_bytes);
  const void* kb = nullptr;
  const void* vb = nullptr;
  rc = resolve_kv(Kbar, kv_on_host, &kb, "Kbar");
  if (rc) return rc;
  rc = resolve_kv(Vbar, kv_on_host, &vb, "Vbar");
  if (rc) return rc;
  AttendArgs a;
  a.Q = Q; a.M = M; a.n_q_heads = d->n_q_heads;
  a.K_loc = K_loc; a.V_loc = V_loc; a.M_loc = M_loc; a.k_loc_rotated = k_loc_rotated;
  a.Kbar = static_cast<const uint16_t*>(kb); a.Vbar = static_cast<const uint16_t*>(vb);
  a.n_chunks = n_chunks; a.dco = dco; a.n_docs = n_docs;
  a.sel_ids = sel_ids; a.n_sel = n_sel; a.top_k = d->top_k;
  a.max_sel_chunks = max_sel_chunks; a.pos0 = pos0; a.theta = (double)d->rope_theta;
  a.kv_on_host = kv_on_host ? 1 : 0;
  a.out = out; a.out_f32 = out_f32;
  AttendBatch ab;
  ab.nb = B;
  ab.q_stride = (int64_t)M * d->n_q_heads * kDim;
  ab.kv_stride = (int64_t)M_loc * kRowElems;
  return launch_attend(a, ws, ws_bytes, static_cast<hipStream_t>(stream), B > 1 ? &ab : nullptr);
}

int32_t msa_interleave_reset(msa_interleave_state* st, int32_t n_docs, void* stream) {
  clear_error();
  if (!st || !st->doc_scores) return fail(MSA_ERR_INVALID_ARG, "interleave_reset: NULL state");
  if (n_docs < 1) return fail(MSA_ERR_SHAPE, "interleave_reset: n_docs=%d must be >= 1", n_docs);
  int rc = launch_fill_f32(st->doc_scores, n_docs, -INFINITY, static_cast<hipStream_t>(stream));
  if (rc) return rc;
  st->n_loc = 0;
  return MSA_OK;
}

size_t msa_interleave_step_workspace(const msa_dims* d, int32_t M_new, int32_t cap_loc,
                                     int64_t n_chunks, int32_t n_docs, int64_t max_sel_chunks) {
  if (!d || M_new < 1 || cap_loc < M_new || n_chunks < 1 || n_docs < 1 || max_sel_chunks < 0)
    return 0;
  const size_t r = route_topk_ws(1, M_new, n_chunks, n_docs, d->top_k);
  const size_t a = attend_workspace(M_new, cap_loc, d->n_q_heads, max_sel_chunks);
  return r > a ? r : a;
}

int32_t msa_interleave_step(const msa_dims* d, msa_interleave_state* st, const msa_bf16* Q_new,
                            const msa_bf16* K_new, const msa_bf16* V_new, const msa_bf16* QR_new,
                            int32_t M_new, const msa_bf16* KRbar, const msa_bf16* Kbar,
                            const msa_bf16* Vbar, int32_t kv_on_host, int64_t n_chunks,
                            const int64_t* dco, int32_t n_docs, int64_t max_sel_chunks,
                            msa_bf16* out, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  int rc = check_dims(d);
  if (rc) return rc;
  if (!st || !st->doc_scores || !st->K_loc || !st->V_loc || !st->topk_ids || !st->topk_scores ||
      !st->n_sel)
    return fail(MSA_ERR_INVALID_ARG, "interleave: NULL state buffer");
  if (!Q_new || !K_new || !V_new || !QR_new)
    return fail(MSA_ERR_INVALID_ARG, "interleave: NULL input");
  if (M_new < 1 || st->n_loc < 0 || (int64_t)st->n_loc + M_new > st->cap_loc)
    return fail(MSA_ERR_SHAPE, "interleave: n_loc (%d) + M_new (%d) exceeds cap_loc (%d)",
                st->n_loc, M_new, st->cap_loc);
  rc = check_route_args(d, QR_new, 1, M_new, KRbar, dco, n_docs, n_chunks, st->doc_scores, 1,
                        st->topk_ids, st->topk_scores, st->n_sel);
  if (rc) return rc;
  MSA_A16("interleave", K_new);
  MSA_A16("interleave", V_new);
  const int32_t M_loc = st->n_loc + M_new;
  rc = check_attend_args(d, Q_new, M_new, st->K_loc, st->V_loc, M_loc, Kbar, Vbar, n_chunks, dco,
                         n_docs, st->topk_ids, st->n_sel, max_sel_chunks, out);
  if (rc) return rc;
  const size_t need_r = route_topk_ws(1, M_new, n_chunks, n_docs, d->top_k);
  const size_t need_a = attend_workspace(M_new, M_loc, d->n_q_heads, max_sel_chunks);
  if (ws == nullptr || ws_bytes < need_r || ws_bytes < need_a)
    return fail(MSA_ERR_WORKSPACE, "interleave workspace too small");
  const void* kb = nullptr;
  const void* vb = nullptr;
  rc = resolve_kv(Kbar, kv_on_host, &kb, "Kbar");
  if (rc) return rc;
  rc = resolve_kv(Vbar, kv_on_host, &vb, "Vbar");
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);

  rc = route_topk_impl(d, QR_new, 1, M_new, KRbar, dco, n_docs, n_chunks, st->doc_scores, 1,
                       st->topk_ids, st->topk_scores, st->n_sel, ws, ws_bytes, s);
  if (rc) return rc;
  rc = launch_append_rows(K_new, V_new, st->K_loc, st->V_loc, 1, M_new, st->n_loc, st->cap_loc, s);
  if (rc) return rc;
  AttendArgs a;
  a.Q = Q_new; a.M = M_new; a.n_q_heads = d->n_q_heads;
  a.K_loc = st->K_loc; a.V_loc = st->V_loc; a.M_loc = M_loc; a.k_loc_rotated = 0;
  a.Kbar = static_cast<const uint16_t*>(kb); a.Vbar = static_cast<const uint16_t*>(vb);
  a.n_chunks = n_chunks; a.dco = dco; a.n_docs = n_docs;
  a.sel_ids = st->topk_ids; a.n_sel = st->n_sel; a.top_k = d->top_k;
  a.max_sel_chunks = max_sel_chunks; a.pos0 = st->pos0; a.theta = (double)d->rope_theta;
  a.kv_on_host = kv_on_host ? 1 : 0;
  a.out = out; a.out_f32 = nullptr;
  rc = launch_attend(a, ws, ws_bytes, s);
  if (rc) return rc;
  st->n_loc = M_loc;
  return MSA_OK;
}

int32_t msa_interleave_batch_reset(msa_interleave_batch* st, int32_t n_docs, void* stream) {
  clear_error();
  if (!st || !st->doc_scores) return fail(MSA_ERR_INVALID_ARG, "interleave_batch_reset: NULL state");
  if (n_docs < 1) return fail(MSA_ERR_SHAPE, "interleave_batch_reset: n_docs=%d must be >= 1", n_docs);
  if (st->B < 1) return fail(MSA_ERR_SHAPE, "interleave_batch_reset: B=%d must be >= 1", st->B);
  int rc = launch_fill_f32(st->doc_scores, (int64_t)st->B * n_docs, -INFINITY,
                           static_cast<hipStream_t>(stream));
  if (rc) return rc;
  st->n_loc = 0;
  return MSA_OK;
}

}  // extern "C"

namespace {
// Queries of a batched interleave round attended per set of launches: up to
// kAttendGroup (their partials share the workspace).
constexpr int32_t kAttendGroup = 8;
int32_t attend_group(int32_t B) { return B < kAttendGroup ? B : kAttendGroup; }
}  // namespace

extern "C" {

size_t msa_interleave_batch_step_workspace(const msa_dims* d, int32_t B, int32_t M_new,
                                           int32_t cap_loc, int64_t n_chunks, int32_t n_docs,
                                           int64_t max_sel_chunks) {
  if (!d || B < 1 || M_new < 1 || cap_loc < M_new || n_chunks < 1 || n_docs < 1 ||
      max_sel_chunks < 0)
    return 0;
  const size_t r = route_topk_ws(B, M_new, n_chunks, n_docs, d->top_k);
  const size_t a = attend_workspace(M_new, cap_loc, d->n_q_heads, max_sel_chunks,
                                    attend_group(B));
  return r > a ? r : a;
}

int32_t msa_interleave_batch_step(const msa_dims* d, msa_interleave_batch* st,
                                  const msa_bf16* Q_new, const msa_bf16* K_new,
                                  const msa_bf16* V_new, const msa_bf16* QR_new, int32_t M_new,
                                  const msa_bf16* KRbar, const msa_bf16* Kbar,
                                  const msa_bf16* Vbar, int32_t kv_on_host, int64_t n_chunks,
                                  const int64_t* dco, int32_t n_docs, int64_t max_sel_chunks,
                                  msa_bf16* out, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  int rc = check_dims(d);
  if (rc) return rc;
  if (!st || !st->doc_scores || !st->K_loc || !st->V_loc || !st->topk_ids || !st->topk_scores ||
      !st->n_sel)
    return fail(MSA_ERR_INVALID_ARG, "interleave_batch: NULL state buffer");
  if (!Q_new || !K_new || !V_new || !QR_new)
    return fail(MSA_ERR_INVALID_ARG, "interleave_batch: NULL input");
  const int32_t B = st->B;
  if (B < 1 || B > 65535)
    return fail(MSA_ERR_SHAPE, "interleave_batch: B=%d must be in [1, 65535]", B);
  if (M_new < 1 || st->n_loc < 0 || (int64_t)st->n_loc + M_new > st->cap_loc)
    return fail(MSA_ERR_SHAPE, "interleave_batch: n_loc (%d) + M_new (%d) exceeds cap_loc (%d)",
                st->n_loc, M_new, st->cap_loc);
  MSA_A16("interleave_batch", K_new);
  MSA_A16("interleave_batch", V_new);
  rc = check_route_args(d, QR_new, B, M_new, KRbar, dco, n_docs, n_chunks, st->doc_scores, 1,
                        st->topk_ids, st->topk_scores, st->n_sel);
  if (rc) return rc;
  const int32_t M_loc = st->n_loc + M_new;
  rc = check_attend_args(d, Q_new, M_new, st->K_loc, st->V_loc, M_loc, Kbar, Vbar, n_chunks, dco,
                         n_docs, st->topk_ids, st->n_sel, max_sel_chunks, out);
  if (rc) return rc;
  const int32_t grp = attend_group(B);
  const size_t need_r = route_topk_ws(B, M_new, n_chunks, n_docs, d->top_k);
  const size_t need_a = attend_workspace(M_new, M_loc, d->n_q_heads, max_sel_chunks, grp);
  if (ws == nullptr || ws_bytes < need_r || ws_bytes < need_a)
    return fail(MSA_ERR_WORKSPACE, "interleave_batch workspace too small");
  const void* kb = nullptr;
  const void* vb = nullptr;
  rc = resolve_kv(Kbar, kv_on_host, &kb, "Kbar");
  if (rc) return rc;
  rc = resolve_kv(Vbar, kv_on_host, &vb, "Vbar");
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);

  // one scan for all B queries (accumulating into each query's scores), then
  // each query's attention; the attention calls reuse the workspace in
  // stream order
  rc = route_topk_impl(d, QR_new, B, M_new, KRbar, dco, n_docs, n_chunks, st->doc_scores, 1,
                       st->topk_ids, st->topk_scores, st->n_sel, ws, ws_bytes, s);
  if (rc) return rc;
  const size_t row = (size_t)kRowElems;                       // elements per KV token row
  const size_t q_row = (size_t)d->n_q_heads * kDim;           // elements per query token row
  rc = launch_append_rows(K_new, V_new, st->K_loc, st->V_loc, B, M_new, st->n_loc, st->cap_loc, s);
  if (rc) return rc;
  // queries go through the attention launches in groups of grp (one group
  // per set of launches when the multi-token kernel serves the shape)
  for (int32_t b = 0; b < B; b += grp) {
    const int32_t nb = B - b < grp ? B - b : grp;
    msa_bf16* kl = st->K_loc + (size_t)b * st->cap_loc * row;
    msa_bf16* vl = st->V_loc + (size_t)b * st->cap_loc * row;
    AttendArgs a;
    a.Q = Q_new + (size_t)b * M_new * q_row; a.M = M_new; a.n_q_heads = d->n_q_heads;
    a.K_loc = kl; a.V_loc = vl; a.M_loc = M_loc; a.k_loc_rotated = 0;
    a.Kbar = static_cast<const uint16_t*>(kb); a.Vbar = static_cast<const uint16_t*>(vb);
    a.n_chunks = n_chunks; a.dco = dco; a.n_docs = n_docs;
    a.sel_ids = st->topk_ids + (size_t)b * d->top_k; a.n_sel = st->n_sel + b;
    a.top_k = d->top_k;
    a.max_sel_chunks = max_sel_chunks; a.pos0 = st->pos0; a.theta = (double)d->rope_theta;
    a.kv_on_host = kv_on_host ? 1 : 0;
    a.out = out + (size_t)b * M_new * q_row; a.out_f32 = nullptr;
    AttendBatch ab;
    ab.nb = nb;
    ab.q_stride = (int64_t)M_new * q_row;
    ab.kv_stride = (int64_t)st->cap_loc * row;
    rc = launch_attend(a, ws, ws_bytes, s, nb > 1 ? &ab : nullptr);
    if (rc) return rc;
  }
  st->n_loc = M_loc;
  return MSA_OK;
}

}  // extern "C"
