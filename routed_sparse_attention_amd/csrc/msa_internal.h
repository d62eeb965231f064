// Internal declarations shared by the MSA HIP sources: error reporting,
// bf16 conversions, wave-level helpers and the kernel launchers that the C
// entry points in msa_api.hip call. Nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "msa.h"

namespace msa {

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
int hip_fail(hipError_t e, const char* what);
// Argument checks shared by the entry points (msa_api.hip).
int check_dims(const msa_dims* d);
// K̄/V̄ pointer → device-visible address: device memory as is, pinned host
// memory (on_host = 1) to its mapping; anything else is MSA_ERR_INVALID_ARG.
int resolve_kv(const void* p, int on_host, const void** out, const char* name);
// Same, with the memory kind read from the pointer.
int resolve_any(const void* p, const void** out, const char* name);

// Every bf16 tensor is read and written with 16-byte vector accesses, so
// its base address must be a multiple of 16 (NULL passes; row strides are
// multiples of 16 bytes by construction). Returns MSA_ERR_INVALID_ARG
// naming the argument otherwise.
int misaligned16(const char* call, const char* name);
inline int check_a16(const char* call, const char* name, const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15) ? misaligned16(call, name) : 0;
}
#define MSA_A16(call, p)                                          \
  do {                                                            \
    int rc_ = ::msa::check_a16((call), #p, (p));                  \
    if (rc_) return rc_;                                          \
  } while (0)

#define MSA_HIP(expr)                                   \
  do {                                                  \
    hipError_t e_ = (expr);                             \
    if (e_ != hipSuccess) return ::msa::hip_fail(e_, #expr); \
  } while (0)

#define MSA_LAUNCH_CHECK(what)                          \
  do {                                                  \
    hipError_t e_ = hipGetLastError();                  \
    if (e_ != hipSuccess) return ::msa::hip_fail(e_, what); \
  } while (0)

static inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Fixed head geometry of this library: 8 KV/router heads of dimension 128, so a
// token row of one tensor is 1024 bf16 = 2 KiB = 128 × 16-byte vectors.
constexpr int kHeads = 8;
constexpr int kDim = 128;
constexpr int kRowElems = kHeads * kDim;      // 1024
constexpr int kRowVec = kRowElems / 8;        // 128 uint4 per row
constexpr float kNormEps = 1e-6f;

// ---------------------------------------------------------------------------
// bf16 helpers (device)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bf16, round to nearest even; NaN stays a quiet NaN. (Host and
// device: the host build is what the rounding tests call.)
__host__ __device__ __forceinline__ uint16_t f2bf(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  const uint32_t rne = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  // NaN stays NaN (quiet bit set); selects, not branches, so callers unroll
  return (uint16_t)(((u & 0x7fffffffu) > 0x7f800000u) ? ((u >> 16) | 0x40u) : rne);
}

// double -> bf16 with a single rounding (nearest even): first narrow to float
// rounding toward zero and make the result odd if it was inexact ("round to
// odd"), then round that float to bf16. Float keeps 24 bits, more than bf16's
// 8 + 2, so the two steps round exactly once. The toward-zero narrowing is the
// hardware's nearest-even conversion stepped back by one unit when it rounded
// away from zero (a library toward-zero conversion costs several times more).
__host__ __device__ __forceinline__ uint16_t d2bf(double x) {
  const float f = (float)x;
  const double d = (double)f;
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if (d != x) {
    if (fabs(d) > fabs(x)) u -= 1u;
    u |= 1u;
  }
  const uint16_t b = f2bf(__builtin_bit_cast(float, u));
  return (x != x) ? (uint16_t)0x7fc0u : b;
}

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

// Two floats -> packed bf16 pair with the hardware conversion (one
// v_cvt_pk_bf16_f32, round to nearest even: the same bits as f2bf for every
// non-NaN input; a NaN stays a NaN). For hot loops.
typedef __bf16 msa_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float msa_f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const msa_f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, msa_bf16x2_t));
}

// Streaming 16-byte load that is not expected to be reused (non-temporal).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Cross-lane sums with DPP (full VALU rate, no LDS traffic).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, false));
}
// Sum over the 16 lanes of each row; every lane of the row gets the sum.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f<0x141>(x);  // row_half_mirror
  x += dpp_f<0x140>(x);  // row_mirror
  return x;
}
// Given row sums in every lane, lane 63 gets the sum over the four rows.
__device__ __forceinline__ float rows_to_lane63(float x) {
  x += dpp_f<0x142, 0xA>(x);  // row_bcast15 into rows 1 and 3
  x += dpp_f<0x143, 0xC>(x);  // row_bcast31 into rows 2 and 3
  return x;
}

// Router-query slice held by lane l in the coalesced scan layout: the 16-byte
// vectors l and 64+l of a 1024-element row, i.e. dims [8(l%16), +8) of heads
// l/16 and 4 + l/16. Returns q̂ = x / max(‖x‖, eps) (fp64 norm per head) as
// bf16 hi + lo vectors: [0] head l/16, [1] head 4 + l/16.
__device__ inline void qhat_hilo_pair(const uint16_t* row, int lane, uint4* hi, uint4* lo) {
  const uint4* src = reinterpret_cast<const uint4*>(row);
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const uint4 a = src[64 * p + lane];
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
    double x[8];
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16lo(w[i]);
      x[2 * i + 1] = bf16hi(w[i]);
      ss += x[2 * i] * x[2 * i] + x[2 * i + 1] * x[2 * i + 1];
    }
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    ss += __shfl_xor(ss, 4);
    ss += __shfl_xor(ss, 8);
    const double nrm = sqrt(ss);
    const double inv = 1.0 / (nrm > (double)kNormEps ? nrm : (double)kNormEps);
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double q0 = x[2 * i] * inv, q1 = x[2 * i + 1] * inv;
      const uint16_t h0 = d2bf(q0), h1 = d2bf(q1);
      h[i] = pack2(h0, h1);
      l[i] = pack2(d2bf(q0 - (double)bf16f(h0)), d2bf(q1 - (double)bf16f(h1)));
    }
    hi[p] = make_uint4(h[0], h[1], h[2], h[3]);
    lo[p] = make_uint4(l[0], l[1], l[2], l[3]);
  }
}

// Order-preserving map of a float onto uint32 (larger float -> larger key).
// NaN maps to 0 (ranks below every number); -0 is treated as +0.
__device__ __forceinline__ uint32_t ord_key(float f) {
  if (f != f) return 0u;
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord_val(uint32_t k) {
  if (k == 0u) return __uint_as_float(0x7fc00000u);
  return (k & 0x80000000u) ? __uint_as_float(k & 0x7fffffffu) : __uint_as_float(~k);
}

// NaN-propagating max (matches numpy's max / maximum).
__device__ __forceinline__ float nan_max(float a, float b) {
  if (a != a) return a;
  if (b != b) return b;
  return b > a ? b : a;
}

// ---------------------------------------------------------------------------
// launchers (each returns MSA_OK or a negative status)
// ---------------------------------------------------------------------------
struct PoolArgs {
  const uint16_t* K; const uint16_t* V; const uint16_t* KR;
  const int64_t* dto; const int64_t* dco;
  int32_t n_docs; int64_t n_tokens; int64_t n_chunks; int32_t chunk;
  // chunk index of the first document's first chunk: the offsets in dco are
  // absolute store rows, the outputs are written at those rows
  int64_t chunk_base;
  double theta; int32_t rope_mode;
  uint16_t* Kbar; uint16_t* Vbar; uint16_t* KRbar;
  // filled by launch_pool (fp64, host): one-step rotations per frequency m
  double cw[64], sw[64];     // cos ω_m, sin ω_m
};
int launch_pool(const PoolArgs& a, hipStream_t s);

// Routing scan geometry. Query rows are processed in tiles of `tile_rows`:
// whole queries per tile when M <= tile_rows, else `parts` tiles per query.
struct RouteGeom {
  int32_t B, M;           // queries, tokens per query
  int32_t tile_rows;      // rows per tile (kernel dependent)
  int32_t q_per_tile;     // whole queries per tile (M <= tile_rows) else 1
  int32_t parts;          // tiles per query (M > tile_rows) else 1
  int32_t n_tiles;        // row tiles in the grid
};
RouteGeom route_geom(int32_t B, int32_t M, int32_t tile_rows);

// Rows of tile `ty`: queries [b0, b0+nq), tokens [m0, m0+nr) of each.
struct TileRows {
  int32_t b0, nq;
  int32_t part;
  int32_t m0, nr;
};
__host__ __device__ inline TileRows tile_rows_of(const RouteGeom& g, int ty) {
  TileRows t;
  if (g.parts == 1) {
    t.b0 = ty * g.q_per_tile;
    t.nq = g.B - t.b0 < g.q_per_tile ? g.B - t.b0 : g.q_per_tile;
    t.part = 0;
    t.m0 = 0;
    t.nr = g.M;
  } else {
    t.b0 = ty / g.parts;
    t.nq = 1;
    t.part = ty % g.parts;
    t.m0 = t.part * g.tile_rows;
    t.nr = g.M - t.m0 < g.tile_rows ? g.M - t.m0 : g.tile_rows;
  }
  return t;
}

// Scan output: with parts == 1 the kernels write final chunk scores S[B][C]
// (MEAN already divided by M); with parts > 1 they write per-part partials
// P[parts][B][C] (max, or sums under MEAN) that launch_parts_combine folds.
// The fp32-exact VALU scan serves one query row (decode); from two rows on the
// batched MFMA scan streams the store faster (the VALU form's per-row lane
// reductions make it ALU-bound: 8 rows over 1.56M chunks took 1.5 ms, the MFMA
// scan 0.63 ms).
constexpr int kValuTileRows = 1;
constexpr int kMfmaTileRows = 16;   // one segment per MFMA lane group
int launch_scan_valu(const uint16_t* QR, const RouteGeom& g, const uint16_t* KRbar,
                     int64_t n_chunks, int32_t token_reduce, float* out, hipStream_t s);
int launch_scan_mfma(const uint16_t* QR, const RouteGeom& g, const uint16_t* KRbar,
                     int64_t n_chunks, int32_t token_reduce, float* out, hipStream_t s);
int launch_parts_combine(const float* P, const RouteGeom& g, int64_t n_chunks,
                         int32_t token_reduce, float* S, hipStream_t s);
// Tiled contraction scan (msa_route_gemm.hip) for M a multiple of 128: writes
// final scores (parts == 1) or P[parts][B][C]; ws is scan_gemm_ws_bytes of
// workspace (the normalised query rows, and with many row tiles the
// normalised keys).
bool scan_gemm_fits(int32_t M);
int32_t scan_gemm_parts(int32_t M);
size_t scan_gemm_ws_bytes(int32_t B, int32_t M, int64_t n_chunks);
int launch_scan_gemm(const uint16_t* QR, int32_t B, int32_t M, const uint16_t* KRbar,
                     int64_t n_chunks, int32_t token_reduce, float* out, void* ws,
                     hipStream_t s);

// Doc reduce + top-k.
size_t doc_topk_workspace(int32_t B, int32_t n_docs, int32_t top_k);
int launch_doc_topk(const float* S, int32_t B, int64_t n_chunks, const int64_t* dco,
                    int32_t n_docs, float* doc_scores, int32_t accumulate, int32_t top_k,
                    uint64_t* cand, int32_t* topk_ids, float* topk_scores, int32_t* n_sel,
                    hipStream_t s);
int launch_fill_f32(float* p, int64_t n, float v, hipStream_t s);

// Routing as one call (msa_route_topk): workspace bytes, argument checks and
// the launches (scan, then document max and top-k); defined in msa_api.hip.
size_t route_topk_ws(int32_t B, int32_t M, int64_t C, int32_t N, int32_t K);
int check_route_args(const msa_dims* d, const msa_bf16* QR, int32_t B, int32_t M,
                     const msa_bf16* KRbar, const int64_t* dco, int32_t n_docs, int64_t n_chunks,
                     const float* doc_scores, int32_t accumulate, const int32_t* topk_ids,
                     const float* topk_scores, const int32_t* n_sel);
int route_topk_impl(const msa_dims* d, const msa_bf16* QR, int32_t B, int32_t M,
                    const msa_bf16* KRbar, const int64_t* dco, int32_t n_docs, int64_t n_chunks,
                    float* doc_scores, int32_t accumulate, int32_t* topk_ids, float* topk_scores,
                    int32_t* n_sel, void* ws, size_t ws_bytes, hipStream_t s);

// Sparse attention.
struct AttendArgs {
  const uint16_t* Q; int32_t M; int32_t n_q_heads;
  const uint16_t* K_loc; const uint16_t* V_loc; int32_t M_loc; int32_t k_loc_rotated;
  const uint16_t* Kbar; const uint16_t* Vbar; int64_t n_chunks;
  const int64_t* dco; int32_t n_docs;
  const int32_t* sel_ids; const int32_t* n_sel; int32_t top_k;
  int64_t max_sel_chunks; int64_t pos0; double theta;
  int32_t kv_on_host;             // K̄/V̄ are pinned host memory (read over PCIe)
  uint16_t* out; float* out_f32;
};
// Several queries of one shape in one set of launches: query b's Q and
// output at b·q_stride elements from a.Q / a.out (packed: q_stride is
// M · n_q_heads · 128), its
// local K/V at b·kv_stride from a.K_loc / a.V_loc, its selection at
// a.sel_ids + b·top_k and a.n_sel + b. Each query computes exactly what it
// would alone.
struct AttendBatch {
  int32_t nb;
  int64_t q_stride, kv_stride;
};
size_t attend_workspace(int32_t M, int32_t M_loc, int32_t n_q_heads, int64_t max_sel_chunks,
                        int32_t nb = 1);
int launch_attend(const AttendArgs& a, void* ws, size_t ws_bytes, hipStream_t s,
                  const AttendBatch* batch = nullptr);

}  // namespace msa
