// msa_route_score: cosine routing of router queries against the pooled
// router-key store (MSA stage 2, first half).
//
// Method (portal.techblg.uk IRMaD reading, section M, routing bullet):
//   S_tc = mean_h cos(Q^R_{t,h}, K̄^R_{c,h}),  S_c = max_t S_tc (or mean_t).
// Reading: each norm is clamped at 1e-6 before dividing.
//
// Design. The store is read once per row tile and never written; the
// [tokens × chunks] score matrix is never materialised — tokens are reduced
// inside a tile, so only S[parts][B][C] (4 bytes per chunk per query part)
// leaves the kernel. Under the MEAN reduction a tile stores the sum of its
// rows; the document stage divides by M.
//   qprep: q̂ = Q^R / max(‖Q^R‖, eps) per head, split into bf16 hi + lo parts
//     (q̂ ≈ hi + lo to ~2^-17), so bf16 dot products against the bf16 keys
//     keep fp32-level accuracy.
//   scan_valu (decode and small batches, <= 8 rows per tile): HBM-bound
//     stream. Lane l of a wave owns head l/8, dims [16(l%8), 16(l%8)+16) of
//     one chunk; it keeps its slice of every tile row's q̂ in registers for
//     the whole launch. Per chunk: two 16-byte loads, v_dot2 bf16 products for
//     q̂·k (hi and lo) and k·k, an 8-lane reduction per head, a per-head
//     1/max(‖k‖, eps) scale and an 8-group reduction over heads.
//   scan_mfma (batched rows): see msa_route_mfma.hip.
#include "msa_internal.h"

namespace msa {

RouteGeom route_geom(int32_t B, int32_t M, int32_t tile_rows) {
  RouteGeom g;
  g.B = B;
  g.M = M;
  g.tile_rows = tile_rows;
  if (M <= tile_rows) {
    g.q_per_tile = tile_rows / M;
    g.parts = 1;
    g.n_tiles = (B + g.q_per_tile - 1) / g.q_per_tile;
  } else {
    g.q_per_tile = 1;
    g.parts = (M + tile_rows - 1) / tile_rows;
    g.n_tiles = B * g.parts;
  }
  return g;
}

namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// One wave per router-query row: lane l owns head l/8, dims 16(l%8)..+16.
__global__ __launch_bounds__(256) void qprep_kernel(const uint16_t* __restrict__ QR, int32_t rows,
                                                    uint16_t* __restrict__ q_hi,
                                                    uint16_t* __restrict__ q_lo) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const uint16_t* src = QR + r * kRowElems + lane * 16;
  float x[16];
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    x[e] = bf16f(src[e]);
    ss += (double)x[e] * (double)x[e];
  }
  // sum over the 8 lanes of this head
  ss += __shfl_xor(ss, 1);
  ss += __shfl_xor(ss, 2);
  ss += __shfl_xor(ss, 4);
  const double nrm = sqrt(ss);
  const double inv = 1.0 / (nrm > (double)kNormEps ? nrm : (double)kNormEps);
  uint16_t* dh = q_hi + r * kRowElems + lane * 16;
  uint16_t* dl = q_lo + r * kRowElems + lane * 16;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const double q = (double)x[e] * inv;
    const uint16_t hb = d2bf(q);
    dh[e] = hb;
    dl[e] = d2bf(q - (double)bf16f(hb));
  }
}

// Rows of tile `ty`: for M <= tile_rows, whole queries [b0, b0+nq) with M rows
// each; otherwise rows [m0, m0+nr) of query b. Row index r -> (query, token).
struct TileRows {
  int32_t b0, nq;      // first query and query count in this tile
  int32_t part;        // part index (0 when whole queries)
  int32_t m0, nr;      // token range of each query covered by this tile
};

__device__ __forceinline__ TileRows tile_rows_of(const RouteGeom& g, int ty) {
  TileRows t;
  if (g.parts == 1) {
    t.b0 = ty * g.q_per_tile;
    t.nq = min(g.q_per_tile, g.B - t.b0);
    t.part = 0;
    t.m0 = 0;
    t.nr = g.M;
  } else {
    t.b0 = ty / g.parts;
    t.nq = 1;
    t.part = ty % g.parts;
    t.m0 = t.part * g.tile_rows;
    t.nr = min(g.tile_rows, g.M - t.m0);
  }
  return t;
}

constexpr int kScanWaves = 4;
constexpr int kScanUnroll = 4;

template <int R>
__global__ __launch_bounds__(256) void scan_valu_kernel(const uint4* __restrict__ q_hi,
                                                        const uint4* __restrict__ q_lo,
                                                        RouteGeom g, const uint4* __restrict__ KR,
                                                        int64_t n_chunks, int32_t token_reduce,
                                                        float* __restrict__ S) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const TileRows tr = tile_rows_of(g, blockIdx.y);
  const int n_rows = tr.nq * tr.nr;  // <= R
  // this lane's slice of every row's q̂ (two 16-byte vectors, hi and lo)
  uint4 qh[R][2], ql[R][2];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    if (k < n_rows) {
      const int qb = tr.b0 + k / tr.nr;
      const int m = tr.m0 + k % tr.nr;
      const int64_t row = (int64_t)qb * g.M + m;
      qh[k][0] = q_hi[row * kRowVec + 2 * lane];
      qh[k][1] = q_hi[row * kRowVec + 2 * lane + 1];
      ql[k][0] = q_lo[row * kRowVec + 2 * lane];
      ql[k][1] = q_lo[row * kRowVec + 2 * lane + 1];
    } else {
      qh[k][0] = qh[k][1] = ql[k][0] = ql[k][1] = make_uint4(0, 0, 0, 0);
    }
  }
  const int64_t wave_id = (int64_t)blockIdx.x * kScanWaves + wave;
  const int64_t n_waves = (int64_t)gridDim.x * kScanWaves;

  for (int64_t c0 = wave_id * kScanUnroll; c0 < n_chunks; c0 += n_waves * kScanUnroll) {
    uint4 k0[kScanUnroll], k1[kScanUnroll];
#pragma unroll
    for (int u = 0; u < kScanUnroll; ++u) {
      const int64_t c = c0 + u;
      if (c < n_chunks) {
        k0[u] = load_stream(KR + c * kRowVec + 2 * lane);
        k1[u] = load_stream(KR + c * kRowVec + 2 * lane + 1);
      } else {
        k0[u] = k1[u] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < kScanUnroll; ++u) {
      const int64_t c = c0 + u;
      const uint32_t kw[8] = {k0[u].x, k0[u].y, k0[u].z, k0[u].w,
                              k1[u].x, k1[u].y, k1[u].z, k1[u].w};
      float nrm = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) nrm = dot2(kw[i], kw[i], nrm);
      nrm += __shfl_xor(nrm, 1);
      nrm += __shfl_xor(nrm, 2);
      nrm += __shfl_xor(nrm, 4);
      const float kn = sqrtf(nrm);
      const float inv_k = 1.0f / (kn > kNormEps ? kn : kNormEps);
      float red[R > 0 ? R : 1];
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const uint32_t hw[8] = {qh[k][0].x, qh[k][0].y, qh[k][0].z, qh[k][0].w,
                                qh[k][1].x, qh[k][1].y, qh[k][1].z, qh[k][1].w};
        const uint32_t lw[8] = {ql[k][0].x, ql[k][0].y, ql[k][0].z, ql[k][0].w,
                                ql[k][1].x, ql[k][1].y, ql[k][1].z, ql[k][1].w};
        float d = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) d = dot2(lw[i], kw[i], d);
#pragma unroll
        for (int i = 0; i < 8; ++i) d = dot2(hw[i], kw[i], d);
        d += __shfl_xor(d, 1);
        d += __shfl_xor(d, 2);
        d += __shfl_xor(d, 4);
        float sh = d * inv_k;  // cosine of this head (q̂ is unit)
        sh += __shfl_xor(sh, 8);
        sh += __shfl_xor(sh, 16);
        sh += __shfl_xor(sh, 32);
        red[k] = sh * 0.125f;  // mean over the 8 heads
      }
      // reduce each query's rows (max, or sum for MEAN) and store
      float v = 0.0f;
#pragma unroll
      for (int k = 0; k < R; ++k) {
        if (k < n_rows) {
          const int m = k % tr.nr;
          const float x = red[k];
          v = (m == 0) ? x : (token_reduce == MSA_TOKEN_REDUCE_MAX ? nan_max(v, x) : v + x);
          if (m == tr.nr - 1 && lane == 0 && c < n_chunks)
            S[((int64_t)tr.part * g.B + tr.b0 + k / tr.nr) * n_chunks + c] = v;
        }
      }
    }
  }
}

}  // namespace

int launch_qprep(const uint16_t* QR, int32_t rows, uint16_t* q_hi, uint16_t* q_lo, hipStream_t s) {
  if (rows == 0) return MSA_OK;
  hipLaunchKernelGGL(qprep_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, QR, rows, q_hi, q_lo);
  MSA_LAUNCH_CHECK("qprep_kernel launch");
  return MSA_OK;
}

int launch_scan_valu(const uint16_t* q_hi, const uint16_t* q_lo, const RouteGeom& g,
                     const uint16_t* KRbar, int64_t n_chunks, int32_t token_reduce, float* S,
                     hipStream_t s) {
  if (n_chunks == 0 || g.n_tiles == 0) return MSA_OK;
  // enough waves to keep every CU streaming: 256 CUs × 8 workgroups
  int64_t per_wg = (int64_t)kScanWaves * kScanUnroll;
  int64_t wg = (n_chunks + per_wg - 1) / per_wg;
  if (wg > 2048) wg = 2048;
  dim3 grid((unsigned)wg, (unsigned)g.n_tiles);
  const uint4* qh = reinterpret_cast<const uint4*>(q_hi);
  const uint4* ql = reinterpret_cast<const uint4*>(q_lo);
  const uint4* kr = reinterpret_cast<const uint4*>(KRbar);
  const int rows = g.parts == 1 ? g.q_per_tile * g.M : g.tile_rows;
  if (rows <= 1) {
    hipLaunchKernelGGL(scan_valu_kernel<1>, grid, dim3(256), 0, s, qh, ql, g, kr, n_chunks,
                       token_reduce, S);
  } else if (rows <= 2) {
    hipLaunchKernelGGL(scan_valu_kernel<2>, grid, dim3(256), 0, s, qh, ql, g, kr, n_chunks,
                       token_reduce, S);
  } else if (rows <= 4) {
    hipLaunchKernelGGL(scan_valu_kernel<4>, grid, dim3(256), 0, s, qh, ql, g, kr, n_chunks,
                       token_reduce, S);
  } else {
    hipLaunchKernelGGL(scan_valu_kernel<8>, grid, dim3(256), 0, s, qh, ql, g, kr, n_chunks,
                       token_reduce, S);
  }
  MSA_LAUNCH_CHECK("scan_valu_kernel launch");
  return MSA_OK;
}

}  // namespace msa
