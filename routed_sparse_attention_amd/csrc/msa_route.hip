// msa_route_score: cosine routing of router queries against the pooled
// router-key store (MSA stage 2, first half).
//
// Method (portal.techblg.uk IRMaD reading, section M, routing bullet):
//   S_tc = mean_h cos(Q^R_{t,h}, K̄^R_{c,h}),  S_c = max_t S_tc (or mean_t).
// Reading: each norm is clamped at 1e-6 before dividing.
//
// Design. The store is read once per row tile and never written; the
// [tokens × chunks] score matrix is never materialised — tokens are reduced
// inside a tile, so only 4 bytes per chunk per query leave the kernel. When a
// query's tokens span several tiles (M > tile rows) each tile writes a
// partial (max, or sum under MEAN) and parts_combine_kernel folds them.
//   Router queries are normalised inside the scan kernels: q̂ = Q^R /
//     max(‖Q^R‖, eps) per head in fp64, split into bf16 hi + lo parts
//     (q̂ ≈ hi + lo to ~2^-17), so bf16 products against the bf16 keys keep
//     fp32-level accuracy.
//   scan_valu (one query row: decode; the kernel is written for up to R
//     rows, but past one row its per-row lane reductions make it ALU-bound
//     and the plan sends such calls to the MFMA scan): HBM-bound
//     stream, one chunk row (2 KiB) per wave per step. Lane l loads the 16-byte
//     vectors l and 64+l of the row — each load instruction covers one
//     contiguous KiB — i.e. dims [8(l%16), +8) of heads l/16 and 4 + l/16, and
//     keeps the matching slice of every tile row's q̂ in registers for the
//     whole launch. Per chunk: v_dot2 bf16 products for q̂·k (hi and lo) and
//     k·k, DPP sums over each 16-lane row (one head pair per row),
//     1/max(‖k‖, eps) by v_rsq, and a DPP row broadcast that leaves the head
//     sum in lane 63.
//   scan_mfma (batched rows): msa_route_mfma.hip.
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

constexpr int kScanWaves = 4;
// chunks per wave per group: deep for the few-row (decode) tiles, where the
// registers are free, shallower as the q̂ slices of more rows take them
constexpr int scan_unroll(int rows) { return rows <= 2 ? 8 : rows <= 4 ? 4 : 2; }

template <int R>
__global__ __launch_bounds__(256) void scan_valu_kernel(const uint16_t* __restrict__ QR,
                                                        RouteGeom g, const uint4* __restrict__ KR,
                                                        int64_t n_chunks, int32_t token_reduce,
                                                        float* __restrict__ out) {
  constexpr int kScanUnroll = scan_unroll(R);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const TileRows tr = tile_rows_of(g, blockIdx.y);
  const int n_rows = tr.nq * tr.nr;  // <= R
  uint4 qh[R][2], ql[R][2];   // q̂ slices, filled once the first loads are in flight
  const bool mean = token_reduce == MSA_TOKEN_REDUCE_MEAN;
  const float fin = (mean && g.parts == 1) ? 1.0f / (float)g.M : 1.0f;
  const float eps2 = kNormEps * kNormEps;
  const int64_t wave_id = (int64_t)blockIdx.x * kScanWaves + wave;
  const int64_t n_waves = (int64_t)gridDim.x * kScanWaves;

  const int64_t stride = n_waves * kScanUnroll;
  // Loads are branch-free (indices clamped into the store; results past the
  // end are never stored), so the compiler can wait for exactly the group it
  // is about to score while the next group, in the other buffer, is in flight.
  auto load = [&](int64_t cb, uint4* a, uint4* b) {
#pragma unroll
    for (int u = 0; u < kScanUnroll; ++u) {
      const int64_t c = min(cb + u, n_chunks - 1);
      a[u] = load_stream(KR + c * kRowVec + lane);
      b[u] = load_stream(KR + c * kRowVec + 64 + lane);
    }
  };
  auto score = [&](int64_t c0, const uint4* A, const uint4* B) {
#pragma unroll
    for (int u = 0; u < kScanUnroll; ++u) {
      const int64_t c = c0 + u;
      const uint32_t ka[4] = {A[u].x, A[u].y, A[u].z, A[u].w};
      const uint32_t kb[4] = {B[u].x, B[u].y, B[u].z, B[u].w};
      float na = 0.0f, nb = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        na = dot2(ka[i], ka[i], na);
        nb = dot2(kb[i], kb[i], nb);
      }
      const float ia = __builtin_amdgcn_rsqf(fmaxf(row_sum16(na), eps2));
      const float ib = __builtin_amdgcn_rsqf(fmaxf(row_sum16(nb), eps2));
      float red[R];
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const uint32_t ha[4] = {qh[k][0].x, qh[k][0].y, qh[k][0].z, qh[k][0].w};
        const uint32_t hb[4] = {qh[k][1].x, qh[k][1].y, qh[k][1].z, qh[k][1].w};
        const uint32_t la[4] = {ql[k][0].x, ql[k][0].y, ql[k][0].z, ql[k][0].w};
        const uint32_t lb[4] = {ql[k][1].x, ql[k][1].y, ql[k][1].z, ql[k][1].w};
        float da = 0.0f, db = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          da = dot2(la[i], ka[i], da);
          db = dot2(lb[i], kb[i], db);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          da = dot2(ha[i], ka[i], da);
          db = dot2(hb[i], kb[i], db);
        }
        // cosines of heads lane/16 and 4 + lane/16 (q̂ is unit), summed over rows
        const float sh = row_sum16(da) * ia + row_sum16(db) * ib;
        red[k] = rows_to_lane63(sh) * 0.125f;  // mean over the 8 heads (lane 63)
      }
      // reduce each query's rows (max, or sum for MEAN); lane 63 stores
      float v = 0.0f;
#pragma unroll
      for (int k = 0; k < R; ++k) {
        if (k < n_rows) {
          const int m = k % tr.nr;
          const float x = red[k];
          v = (m == 0) ? x : (mean ? v + x : nan_max(v, x));
          if (m == tr.nr - 1 && lane == 63 && c < n_chunks)
            out[((int64_t)tr.part * g.B + tr.b0 + k / tr.nr) * n_chunks + c] = v * fin;
        }
      }
    }
  };
  uint4 xa[kScanUnroll], xb[kScanUnroll], ya[kScanUnroll], yb[kScanUnroll];
  int64_t c0 = wave_id * kScanUnroll;
  if (c0 >= n_chunks) return;
  // the first group's loads go out before q̂ is prepared, so that work hides
  // under their latency
  load(c0, xa, xb);
  load(c0 + stride, ya, yb);
  // this lane's slice of every tile row's q̂: [k][0] head lane/16, [k][1] head 4 + lane/16
#pragma unroll
  for (int k = 0; k < R; ++k) {
    if (k < n_rows) {
      const int64_t row = (int64_t)(tr.b0 + k / tr.nr) * g.M + tr.m0 + k % tr.nr;
      qhat_hilo_pair(QR + row * kRowElems, lane, qh[k], ql[k]);
    } else {
      qh[k][0] = qh[k][1] = ql[k][0] = ql[k][1] = make_uint4(0, 0, 0, 0);
    }
  }
  // x holds group c0, y group c0 + stride; a buffer is refilled as soon as
  // it has been scored
  while (true) {
    score(c0, xa, xb);
    c0 += stride;
    if (c0 >= n_chunks) break;
    load(c0 + stride, xa, xb);
    score(c0, ya, yb);
    c0 += stride;
    if (c0 >= n_chunks) break;
    load(c0 + stride, ya, yb);
  }
}

// S[b][c] = fold over parts of P[part][b][c] (max, or sum / M under MEAN).
__global__ __launch_bounds__(256) void parts_combine_kernel(const float* __restrict__ P,
                                                            RouteGeom g, int64_t C,
                                                            int32_t token_reduce,
                                                            float* __restrict__ S) {
  const int64_t n = (int64_t)g.B * C;
  const bool mean = token_reduce == MSA_TOKEN_REDUCE_MEAN;
  const float inv_m = 1.0f / (float)g.M;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    float v = P[i];
    for (int p = 1; p < g.parts; ++p) {
      const float x = P[(int64_t)p * n + i];
      v = mean ? v + x : nan_max(v, x);
    }
    S[i] = mean ? v * inv_m : v;
  }
}

}  // namespace

int launch_scan_valu(const uint16_t* QR, const RouteGeom& g, const uint16_t* KRbar,
                     int64_t n_chunks, int32_t token_reduce, float* out, hipStream_t s) {
  if (n_chunks == 0 || g.n_tiles == 0) return MSA_OK;
  const uint4* kr = reinterpret_cast<const uint4*>(KRbar);
  // rows actually present in a tile (a lone decode query must not pay for 8)
  const int rows = g.parts == 1 ? (g.q_per_tile < g.B ? g.q_per_tile : g.B) * g.M : g.tile_rows;
  // At most 8192 workgroups (32 per CU, run in turn); each wave strides over
  // the store. Fewer leave the HBM queues short near the end of the scan, more
  // repeat the per-wave q̂ preparation too often (measured on the 1.56M-chunk
  // decode scan: 2048 → 500 µs, 8192 → 470 µs, 16384 → 520 µs).
  const int64_t per_wg = (int64_t)kScanWaves * scan_unroll(rows);
  int64_t wg = (n_chunks + per_wg - 1) / per_wg;
  if (wg > 8192) wg = 8192;
  const dim3 grid((unsigned)wg, (unsigned)g.n_tiles);
  if (rows != 1) return fail(MSA_ERR_UNSUPPORTED, "VALU scan: %d rows (one expected)", rows);
  hipLaunchKernelGGL(scan_valu_kernel<1>, grid, dim3(256), 0, s, QR, g, kr, n_chunks, token_reduce, out);
  MSA_LAUNCH_CHECK("scan_valu_kernel launch");
  return MSA_OK;
}

int launch_parts_combine(const float* P, const RouteGeom& g, int64_t n_chunks,
                         int32_t token_reduce, float* S, hipStream_t s) {
  const int64_t n = (int64_t)g.B * n_chunks;
  if (n == 0) return MSA_OK;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(parts_combine_kernel, dim3((unsigned)blocks), dim3(256), 0, s, P, g, n_chunks,
                     token_reduce, S);
  MSA_LAUNCH_CHECK("parts_combine_kernel launch");
  return MSA_OK;
}

}  // namespace msa
