// msa_route_score, batched form: cosine routing of many query rows on MFMA.
//
// Method (portal.techblg.uk IRMaD reading, section M, routing bullet):
//   S_tc = mean_h cos(Q^R_{t,h}, K̄^R_{c,h}),  S_c = max_t S_tc (or mean_t).
//
// With many router rows (batched queries, or a long query) the scan becomes a
// dense contraction, [rows × 128] · [128 × chunks] per head, so it runs on
// v_mfma_f32_32x32x16_bf16. The per-head key norm cannot be folded into the
// contraction (it scales columns per head), so every head keeps its own
// accumulator and the head sum happens afterwards.
//
// Design: one workgroup of 8 waves per 64-row tile; wave w owns router head w.
//   - q̂ = Q^R / max(‖Q^R‖, eps) (fp64 norm), rounded once to bf16 and kept as
//     MFMA A fragments for the whole launch (2 row blocks × 8 k-steps). The
//     rounding moves a cosine by ~1e-4 (relative error 2^-9 per element,
//     averaged over 128 dims and 8 heads) — inside the 1e-3 score tolerance;
//     the decode path (scan_valu) keeps a hi + lo split instead;
//   - per 32-chunk tile each lane loads its 8 B fragments (16 contiguous bytes
//     of one chunk's head row per k-step) straight from HBM, one tile ahead of
//     use, so the next tile streams in while this one is multiplied; the same
//     registers give ‖k‖² (v_dot2) and 1/max(‖k‖, eps) by v_rsq;
//   - 2 × 8 MFMAs give q̂·k for 64 rows × 32 chunks; the accumulator columns
//     are scaled by the lane's 1/‖k‖ (lane = chunk column) and parked in LDS;
//   - heads are summed and each query's rows reduced (max, or sum for MEAN)
//     from LDS. The LDS buffer alternates between two halves, so one barrier
//     per tile separates writers from readers.
// Workgroups stride over chunk tiles, so every tile of the store is read once
// per row tile.
#include "msa_internal.h"

namespace msa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;          // one per router head
constexpr int kThreads = kWaves * 64;
constexpr int kTileRows = kMfmaTileRows;   // 64
constexpr int kChunkTile = 32;
constexpr int kRedPitch = 33;
constexpr int kRedHalf = kWaves * kTileRows * kRedPitch;

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__global__ __launch_bounds__(512) void scan_mfma_kernel(const uint16_t* __restrict__ QR,
                                                        RouteGeom g,
                                                        const uint16_t* __restrict__ KR,
                                                        int64_t n_chunks, int32_t token_reduce,
                                                        float* __restrict__ out) {
  extern __shared__ float red[];   // 2 × [8 heads][64 rows][33]

  const int tid = threadIdx.x;
  const int h = tid >> 6;          // router head of this wave
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const TileRows tr = tile_rows_of(g, blockIdx.y);
  const int n_rows = tr.nq * tr.nr;  // <= 64
  const bool mean = token_reduce == MSA_TOKEN_REDUCE_MEAN;
  const float fin = (mean && g.parts == 1) ? 1.0f / (float)g.M : 1.0f;
  const float eps2 = kNormEps * kNormEps;

  // ---- q̂ A fragments: [row block][k-step]
  uint4 qa[2][8];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int k = rb * 32 + col;
    uint4 raw[8];
    if (k < n_rows) {
      const int64_t row = (int64_t)(tr.b0 + k / tr.nr) * g.M + tr.m0 + k % tr.nr;
      const uint4* src = reinterpret_cast<const uint4*>(QR + (row * kHeads + h) * kDim);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) raw[ks] = src[ks * 2 + half];
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) raw[ks] = make_uint4(0, 0, 0, 0);
    }
    double ss = 0.0;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint32_t w[4] = {raw[ks].x, raw[ks].y, raw[ks].z, raw[ks].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double a = bf16lo(w[i]), b = bf16hi(w[i]);
        ss += a * a + b * b;
      }
    }
    ss += __shfl_xor(ss, 32);  // the other 64 dims of this row's head
    const double nrm = sqrt(ss);
    const double inv = 1.0 / (nrm > (double)kNormEps ? nrm : (double)kNormEps);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint32_t w[4] = {raw[ks].x, raw[ks].y, raw[ks].z, raw[ks].w};
      uint32_t hw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        hw[i] = pack2(d2bf((double)bf16lo(w[i]) * inv), d2bf((double)bf16hi(w[i]) * inv));
      qa[rb][ks] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    }
  }

  const int64_t n_ct = (n_chunks + kChunkTile - 1) / kChunkTile;
  auto load_b = [&](int64_t ct, uint4* kb) {
    const int64_t c = ct * kChunkTile + col;
    if (ct < n_ct && c < n_chunks) {
      const uint4* src = reinterpret_cast<const uint4*>(KR + (c * kHeads + h) * kDim);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) kb[ks] = load_stream(src + ks * 2 + half);
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ks++) kb[ks] = make_uint4(0, 0, 0, 0);
    }
  };

  uint4 kb[8], kn[8];
  int64_t ct = blockIdx.x;
  load_b(ct, kb);
  for (int it = 0; ct < n_ct; ct += gridDim.x, ++it) {
    load_b(ct + gridDim.x, kn);   // next tile streams in during this one
    float* buf = red + (it & 1) * kRedHalf;

    // ---- 1/max(‖k‖, eps) for this lane's chunk column and head
    float nk = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      nk = dot2(kb[ks].x, kb[ks].x, nk);
      nk = dot2(kb[ks].y, kb[ks].y, nk);
      nk = dot2(kb[ks].z, kb[ks].z, nk);
      nk = dot2(kb[ks].w, kb[ks].w, nk);
    }
    nk += __shfl_xor(nk, 32);
    const float inv_k = __builtin_amdgcn_rsqf(fmaxf(nk, eps2));

    // ---- q̂·k for 64 rows × 32 chunks of this head, scaled per column
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      f32x16_t acc;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qa[rb][ks]), as_bf16x8(kb[ks]),
                                                      acc, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = rb * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        buf[(h * kTileRows + row) * kRedPitch + col] = acc[v] * inv_k;
      }
    }
    __syncthreads();

    // ---- head mean, token reduction per query, store
    const int64_t c0 = ct * kChunkTile;
    for (int o = tid; o < tr.nq * kChunkTile; o += kThreads) {
      const int q = o / kChunkTile, cc = o % kChunkTile;
      float v = 0.0f;
      for (int m = 0; m < tr.nr; ++m) {
        const int row = q * tr.nr + m;
        float sum = 0.0f;
#pragma unroll
        for (int hh = 0; hh < kWaves; ++hh) sum += buf[(hh * kTileRows + row) * kRedPitch + cc];
        const float x = sum * 0.125f;
        v = (m == 0) ? x : (mean ? v + x : nan_max(v, x));
      }
      if (c0 + cc < n_chunks)
        out[((int64_t)tr.part * g.B + tr.b0 + q) * n_chunks + c0 + cc] = v * fin;
    }

#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kb[ks] = kn[ks];
  }
}

}  // namespace

int launch_scan_mfma(const uint16_t* QR, const RouteGeom& g, const uint16_t* KRbar,
                     int64_t n_chunks, int32_t token_reduce, float* out, hipStream_t s) {
  if (n_chunks == 0 || g.n_tiles == 0) return MSA_OK;
  if (g.tile_rows != kTileRows) return fail(MSA_ERR_UNSUPPORTED, "MFMA scan needs 64-row tiles");
  const int64_t n_ct = (n_chunks + kChunkTile - 1) / kChunkTile;
  // one resident workgroup per CU per row tile; they stride over chunk tiles
  int64_t wg = 256 / g.n_tiles;
  if (wg < 32) wg = 32;
  if (wg > n_ct) wg = n_ct;
  const size_t lds = 2 * (size_t)kRedHalf * sizeof(float);
  // more than 64 KiB of dynamic LDS has to be allowed once per process
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(scan_mfma_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)lds);
  if (attr != hipSuccess) return hip_fail(attr, "hipFuncSetAttribute(scan_mfma_kernel)");
  hipLaunchKernelGGL(scan_mfma_kernel, dim3((unsigned)wg, (unsigned)g.n_tiles), dim3(kThreads), lds,
                     s, QR, g, KRbar, n_chunks, token_reduce, out);
  MSA_LAUNCH_CHECK("scan_mfma_kernel launch");
  return MSA_OK;
}

}  // namespace msa
