// msa_route_score for long queries: cosine routing of many rows per query on
// MFMA, each key tile read from memory once per 128 query rows.
//
// Method (portal.techblg.uk IRMaD reading, section M, routing bullet):
//   S_tc = mean_h cos(Q^R_{t,h}, K̄^R_{c,h}),  S_c = max_t S_tc (or mean_t);
// with M query tokens the score is a [M × 128] · [128 × chunks] contraction
// per head, tiled over the chunks (section M, Memory Parallel bullet: the
// score matrix is computed in tiles and never held whole).
//
// Design (queries of 64 tokens or more):
//   - a workgroup of eight waves owns 128 query rows: each wave keeps 16 rows
//     of q̂ = Q^R / max(‖Q^R‖, eps) (fp32 norm, bf16 values) in registers as
//     the A operands of v_mfma_f32_16x16x32_bf16 for all 8 heads (128 VGPRs),
//     so the only LDS traffic per tile is the keys themselves (32 rows per
//     wave would double the rows each key read serves, but their 256 VGPRs of
//     q̂ leave too few registers for the rest);
//   - the workgroup walks its range of the store in tiles of 32 chunks (all
//     8 heads, 64 KiB). The next tile's loads (whole 256-byte head rows) are
//     in flight while the current tile is multiplied. The threads that write
//     a tile into LDS normalise it on the way: k̂ = k / max(‖k‖, eps) per
//     (chunk, head) from the values they hold (a DPP sum over the 16 lanes
//     that share the chunk), rounded to bf16. With both sides unit vectors
//     the head mean of cosines is one contraction over all 1024 dims, so each
//     16-chunk block accumulates all 8 heads in one MFMA chain. (Rounding k̂
//     as well as q̂ to bf16 moves a score by ~1e-4, inside the 1e-3 bar.);
//   - S = q̂ · K̂^T puts one chunk in each lane and the rows in the
//     accumulator registers, so the token reduction is a register reduction
//     plus two exchanges between the four lane groups; waves holding rows of
//     the same query meet in LDS;
//   - a query is padded to whole 16-row blocks (padding rows are masked out of
//     the reduction). Up to eight blocks form one workgroup row group; longer
//     queries span several row groups, which write per-part maxima (or sums)
//     that parts_combine_kernel folds.
#include "msa_internal.h"

namespace msa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlockRows = 16;                 // rows per wave
constexpr int kTileChunks = 32;                // chunks per tile
constexpr int kPitch = kRowElems + 8;          // bf16 per chunk row in LDS
constexpr int kTileElems = kTileChunks * kPitch;
constexpr int kLoads = kTileChunks * kRowVec / kThreads;   // 16-byte loads per thread per tile
constexpr size_t kLdsBytes = 2 * (size_t)kTileElems * 2 +           // key tiles
                             2 * (size_t)kWaves * kTileChunks * 4;   // per-wave row reductions
static_assert(kLoads == kHeads, "one 16-byte vector of every head per thread");

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// max that returns NaN when either side is NaN (as numpy's max does), with
// selects only
__device__ __forceinline__ float max_nan(float a, float b) {
  const float m = fmaxf(a, b);
  return (a != a) ? a : ((b != b) ? b : m);
}

struct RowsGeom {
  int32_t B, M;
  int32_t rbq;      // 16-row blocks per query
  int32_t qpw;      // whole queries per workgroup (parts == 1)
  int32_t parts;    // row groups per query (> 1 for queries over 128 rows)
  int32_t n_rg;     // row groups in the grid
  int64_t tiles_per_wg;
};

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void scan_rows_kernel(const uint16_t* __restrict__ QR, RowsGeom g, const uint16_t* __restrict__ KR,
                      int64_t n_chunks, int32_t token_reduce, float* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint16_t* kt = reinterpret_cast<uint16_t*>(smem);                          // [2][32][kPitch]
  float* red = reinterpret_cast<float*>(smem + 2 * (size_t)kTileElems * 2);     // [2][8][32]

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c16 = lane & 15;      // MFMA column (chunk) / A row
  const int grp = lane >> 4;      // lane group: k slice of the operands, rows 4grp.. of D
  const bool mean = token_reduce == MSA_TOKEN_REDUCE_MEAN;

  // ---- rows of this wave: query b, 16-row block j of it
  const int y = blockIdx.y;
  int b, j, q_local;
  if (g.parts == 1) {
    q_local = wave / g.rbq;
    b = y * g.qpw + q_local;
    j = wave % g.rbq;
  } else {
    q_local = 0;
    b = y / g.parts;
    j = (y % g.parts) * kWaves + wave;
  }
  const bool wave_on = (g.parts == 1 ? q_local < g.qpw : true) && b < g.B && j < g.rbq;
  const int m_row = j * kBlockRows + c16;          // this lane's A row (token of query b)
  const bool row_ok = wave_on && m_row < g.M;

  // ---- tile range of this workgroup
  const int64_t n_ct = (n_chunks + kTileChunks - 1) / kTileChunks;
  const int64_t t_begin = (int64_t)blockIdx.x * g.tiles_per_wg;
  const int64_t t_end = min(t_begin + g.tiles_per_wg, n_ct);

  // tile loads: thread t reads the 16-byte vector t % 16 of every head of
  // chunk t / 16 (each load instruction covers four whole 256-byte head rows)
  const int lc = tid >> 4;
  const int lv = tid & 15;
  u32x4 kx[kLoads];
  auto load_tile = [&](int64_t tile) {
    int64_t c = tile * kTileChunks + lc;
    c = c < n_chunks ? c : n_chunks - 1;
    const u32x4* src = reinterpret_cast<const u32x4*>(KR + c * kRowElems);
#pragma unroll
    for (int h = 0; h < kLoads; ++h) kx[h] = src[h * 16 + lv];
  };
  auto store_tile = [&](int buf) {
    // k̂ = k / max(‖k‖, eps) per head: the squares of this thread's 8 values,
    // summed over the 16 lanes of the chunk (one DPP row), then scaled
    uint16_t* dst = kt + buf * kTileElems + lc * kPitch;
#pragma unroll
    for (int h = 0; h < kLoads; ++h) {
      float x[8];
      float ss = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        x[2 * w] = bf16lo(kx[h][w]);
        x[2 * w + 1] = bf16hi(kx[h][w]);
        ss = fmaf(x[2 * w], x[2 * w], ss);
        ss = fmaf(x[2 * w + 1], x[2 * w + 1], ss);
      }
      ss = row_sum16(ss);
      const float inv = __builtin_amdgcn_rsqf(fmaxf(ss, kNormEps * kNormEps));
      u32x4 o;
#pragma unroll
      for (int w = 0; w < 4; ++w) o[w] = pack2(f2bf(x[2 * w] * inv), f2bf(x[2 * w + 1] * inv));
      *reinterpret_cast<u32x4*>(dst + (h * 16 + lv) * 8) = o;
    }
  };

  if (t_begin < t_end) load_tile(t_begin);

  // ---- q̂ of this lane's row as A fragments: head h, k-step ks covers dims
  //      32ks + 8·grp .. +7 of the head
  u32x4 qa[kHeads][4];
  {
    const int64_t row = row_ok ? (int64_t)b * g.M + m_row : 0;
    const u32x4* src = reinterpret_cast<const u32x4*>(QR + row * kRowElems);
#pragma unroll
    for (int h = 0; h < kHeads; ++h)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qa[h][ks] = src[h * 16 + ks * 4 + grp];
    // one head at a time (the barriers keep the compiler from expanding all
    // 128 dims of every head to fp32 at once)
#pragma unroll
    for (int h = 0; h < kHeads; ++h) {
      float ss = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float a = bf16lo(qa[h][ks][w]), c2 = bf16hi(qa[h][ks][w]);
          ss = fmaf(a, a, ss);
          ss = fmaf(c2, c2, ss);
        }
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      const float inv = row_ok ? __builtin_amdgcn_rsqf(fmaxf(ss, kNormEps * kNormEps)) : 0.0f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int w = 0; w < 4; ++w)
          qa[h][ks][w] = pack2(f2bf(bf16lo(qa[h][ks][w]) * inv), f2bf(bf16hi(qa[h][ks][w]) * inv));
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  if (t_begin < t_end) store_tile(0);
  __syncthreads();

  const float fin = (mean && g.parts == 1) ? 0.125f / (float)g.M : 0.125f;
  for (int64_t t = t_begin; t < t_end; ++t) {
    const int buf = (int)((t - t_begin) & 1);
    if (t + 1 < t_end) load_tile(t + 1);

    // ---- S = q̂ K̂^T for the tile's two 16-chunk blocks: all 8 heads × 4
    //      k-steps in one accumulator chain per block; the two chains share
    //      each A fragment
    f32x4_t tot[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
    {
      const uint16_t* kb0 = kt + buf * kTileElems + c16 * kPitch + grp * 8;
      const uint16_t* kb1 = kb0 + 16 * kPitch;
#pragma unroll
      for (int h = 0; h < kHeads; ++h) {
        u32x4 f0[4], f1[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          f0[ks] = *reinterpret_cast<const u32x4*>(kb0 + h * kDim + ks * 32);
          f1[ks] = *reinterpret_cast<const u32x4*>(kb1 + h * kDim + ks * 32);
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          tot[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[h][ks]), as_bf16x8(f0[ks]),
                                                           tot[0], 0, 0, 0);
          tot[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[h][ks]), as_bf16x8(f1[ks]),
                                                           tot[1], 0, 0, 0);
        }
      }
    }

    // ---- reduce this wave's rows: register v holds row 4·grp + v
    float* rb = red + buf * kWaves * kTileChunks;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      // padding rows add nothing: -inf under MAX, and q̂ = 0 (so 0) under MEAN
      float r = mean ? 0.0f : -INFINITY;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const bool valid = j * kBlockRows + 4 * grp + v < g.M;
        const float x = valid ? tot[cb][v] : (mean ? 0.0f : -INFINITY);
        r = mean ? r + x : max_nan(r, x);
      }
#pragma unroll
      for (int x = 16; x <= 32; x <<= 1) {
        const float o = __shfl_xor(r, x);
        r = mean ? r + o : max_nan(r, o);
      }
      if (grp == 0) rb[wave * kTileChunks + cb * 16 + c16] = r;
    }

    if (t + 1 < t_end) store_tile(buf ^ 1);
    __syncthreads();

    // ---- the waves of each query meet here; one thread per (query, chunk)
    const int n_q = g.parts == 1 ? g.qpw : 1;
    if (tid < n_q * kTileChunks) {
      const int qi = tid / kTileChunks;
      const int c = tid % kTileChunks;
      const int bq = g.parts == 1 ? y * g.qpw + qi : b;
      const int64_t chunk = t * kTileChunks + c;
      if (bq < g.B && chunk < n_chunks) {
        int w0, w1;
        if (g.parts == 1) {
          w0 = qi * g.rbq;
          w1 = w0 + g.rbq;
        } else {
          w0 = 0;
          w1 = min(kWaves, g.rbq - (y % g.parts) * kWaves);
        }
        float v = rb[w0 * kTileChunks + c];
        for (int w = w0 + 1; w < w1; ++w) {
          const float x = rb[w * kTileChunks + c];
          v = mean ? v + x : max_nan(v, x);
        }
        const int part = g.parts == 1 ? 0 : y % g.parts;
        out[((int64_t)part * g.B + bq) * n_chunks + chunk] = v * fin;
      }
    }
  }
}

}  // namespace

int32_t scan_rows_parts(int32_t M) {
  const int32_t rbq = (M + kBlockRows - 1) / kBlockRows;
  return rbq <= kWaves ? 1 : (rbq + kWaves - 1) / kWaves;
}

int launch_scan_rows(const uint16_t* QR, int32_t B, int32_t M, const uint16_t* KRbar,
                     int64_t n_chunks, int32_t token_reduce, float* out, hipStream_t s) {
  if (n_chunks == 0) return MSA_OK;
  RowsGeom g;
  g.B = B;
  g.M = M;
  g.rbq = (M + kBlockRows - 1) / kBlockRows;
  if (g.rbq <= kWaves) {
    g.qpw = kWaves / g.rbq;
    g.parts = 1;
    g.n_rg = (B + g.qpw - 1) / g.qpw;
  } else {
    g.qpw = 1;
    g.parts = (g.rbq + kWaves - 1) / kWaves;
    g.n_rg = B * g.parts;
  }
  if (g.n_rg > 65535) return fail(MSA_ERR_SHAPE, "route: %d row groups exceed the grid", g.n_rg);
  // one resident workgroup per CU (135 KiB of LDS); the store is split so
  // that all row groups together cover about 256 CUs
  const int64_t n_ct = (n_chunks + kTileChunks - 1) / kTileChunks;
  int64_t n_x = 256 / g.n_rg;
  if (n_x < 1) n_x = 1;
  if (n_x > n_ct) n_x = n_ct;
  g.tiles_per_wg = (n_ct + n_x - 1) / n_x;
  n_x = (n_ct + g.tiles_per_wg - 1) / g.tiles_per_wg;
  MSA_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(scan_rows_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes));
  hipLaunchKernelGGL(scan_rows_kernel, dim3((unsigned)n_x, (unsigned)g.n_rg), dim3(kThreads),
                     kLdsBytes, s, QR, g, KRbar, n_chunks, token_reduce, out);
  MSA_LAUNCH_CHECK("scan_rows_kernel launch");
  return MSA_OK;
}

}  // namespace msa
