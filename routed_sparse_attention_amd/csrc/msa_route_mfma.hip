// msa_route_score, batched form: cosine routing of many query rows on MFMA.
//
// Method (portal.techblg.uk IRMaD reading, section M, routing bullet):
//   S_tc = mean_h cos(Q^R_{t,h}, K̄^R_{c,h}),  S_c = max_t S_tc (or mean_t).
//
// With many router rows (batched queries, or a long query) the scan becomes a
// dense contraction, [rows × 128] · [128 × chunks] per head, so it runs on
// v_mfma_f32_16x16x32_bf16. The per-head key norm scales columns per head, so
// it cannot be folded into one contraction over all heads; each head's product
// is scaled by its 1/‖k‖ and added to a running head sum in registers.
//
// Design: a workgroup of 8 waves holds 64 query rows; each wave owns whole
// 32-chunk tiles (all 8 heads) and strides over the store on its own, with no
// barrier once the rows are staged:
//   - q̂ = Q^R / max(‖Q^R‖, eps) (fp64 norm; the scaled value is formed in
//     fp32 and rounded to bf16, which moves a cosine by ~1e-4, inside the 1e-3
//     score tolerance; the decode scan keeps a hi + lo split instead) is
//     prepared while the wave's first key loads are in flight and laid out in
//     LDS as MFMA A fragments [head][row block][k-step][lane] (128 KiB), so
//     every fragment read is one contiguous ds_read_b128 per lane; each
//     fragment read serves the tile's two 16-chunk column blocks;
//   - keys: the B operand puts four lanes on each chunk column, so every load
//     instruction reads 64 contiguous bytes of each of 16 chunk rows (the
//     L1→L2 request size of a fully coalesced load). Two heads' loads are in
//     flight while one head is multiplied. Plain (cached) loads: when several
//     row tiles scan the same store at once, L2 serves the repeats. The same
//     registers give ‖k‖² (v_dot2) and 1/max(‖k‖, eps) by v_rsq;
//   - per head, 4 row blocks × 2 column blocks × 4 k-steps of MFMA give q̂·k
//     for 64 rows × 32 chunks, scaled by 1/‖k‖ and summed over heads in fp32;
//   - row placement: the 64 A rows are four 16-row segments (row tiles of the
//     scan geometry), one per lane group of the accumulator layout, so a
//     segment's rows all land in its lane group's registers. Single-token
//     queries are stored straight from registers after a 4×4 lane-quad
//     transpose, as 16-byte stores that fill whole 128-byte lines; otherwise
//     each wave parks its scores in its own LDS slice and reduces each query's
//     rows (max, or sum under MEAN) with an ordinary loop.
#include "msa_internal.h"

namespace msa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kCB = 2;                         // 16-chunk column blocks per tile
constexpr int kChunkTile = 16 * kCB;           // 32 chunks per wave step
constexpr int kSegRows = kMfmaTileRows;        // 16 rows per lane group
constexpr int kRows = 4 * kSegRows;            // 64 rows per workgroup
constexpr int kKSteps = kDim / 32;             // 4 k-steps of 32 per head
constexpr int kFrags = kHeads * 4 * kKSteps;   // [head][row block][k-step]
constexpr int kRing = 2;                       // head buffers in flight
// q̂ fragments (128 KiB) + each wave's 64 × 16 fp32 score block (4 KiB): 160 KiB
constexpr size_t kLdsBytes =
    (size_t)kFrags * 64 * sizeof(uint4) + (size_t)kWaves * kRows * 16 * sizeof(float);

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// A row r of the 64-row tile ↔ (lane group, position u in that group). The
// 16x16 accumulator gives lane (col, group) rows 16·rb + 4·group + i in
// register i of row block rb, so u = 4·rb + i walks a group's own rows.
__device__ __forceinline__ int arow_group(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int arow_pos(int r) { return (r >> 4) * 4 + (r & 3); }

__global__ __launch_bounds__(kThreads) void scan_mfma_kernel(const uint16_t* __restrict__ QR,
                                                             RouteGeom g,
                                                             const uint4* __restrict__ KR,
                                                             int64_t n_chunks, int32_t token_reduce,
                                                             float* __restrict__ out) {
  extern __shared__ uint4 qs[];   // [kFrags][64 lanes], then the waves' score tiles

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int nr_u = g.M < kSegRows ? g.M : kSegRows;   // rows per segment

  const int64_t n_ct = (n_chunks + kChunkTile - 1) / kChunkTile;
  const int64_t stride = (int64_t)gridDim.x * kWaves;
  int64_t t = (int64_t)blockIdx.x * kWaves + wave;

  // Columns past the end (and tiles past the last) reload the last chunk, so
  // the loads stay unconditional and the compiler waits on exactly the head it
  // is about to use. Those scores are not stored.
  auto load_head = [&](int64_t tile, int h, uint4 (&buf)[kCB][kKSteps]) {
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      int64_t c = tile * kChunkTile + cb * 16 + col;
      c = c < n_chunks ? c : n_chunks - 1;
      const uint4* src = KR + (c * kHeads + h) * (kDim / 8) + grp;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) buf[cb][ks] = src[4 * ks];
    }
  };

  // A ring of kRing head buffers over the (tile, head) sequence: a buffer is
  // refilled with the step kRing ahead as soon as its head has been used.
  uint4 kb[kRing][kCB][kKSteps];

  // ---- stage q̂: thread = (A row tid / 8, head tid % 8), 128 dims each
  {
    const int r = tid >> 3, h = tid & 7;
    const int ty = 4 * blockIdx.y + arow_group(r);
    const int u = arow_pos(r);
    // Segments span nr_u = min(M, 16) slots. A query's last part may hold
    // fewer rows: its spare slots repeat the part's last row under MAX (the
    // max is unchanged) and stay zero under MEAN (q̂ = 0 adds nothing).
    bool ok = ty < g.n_tiles;
    int64_t row = 0;
    if (ok) {
      const TileRows tr = tile_rows_of(g, ty);
      const int s = u / nr_u;
      int m = u % nr_u;
      ok = s < tr.nq;
      if (m >= tr.nr) {
        ok = ok && token_reduce != MSA_TOKEN_REDUCE_MEAN;
        m = tr.nr - 1;
      }
      row = (int64_t)(tr.b0 + s) * g.M + tr.m0 + m;
    }
    if (!ok) row = 0;   // loaded (always in bounds) and zeroed below
    uint4 raw[16];
    const uint4* src = reinterpret_cast<const uint4*>(QR + (row * kHeads + h) * kDim);
#pragma unroll
    for (int i = 0; i < 16; ++i) raw[i] = src[i];
    // this wave's first key loads fly while q̂ is prepared (the scheduling
    // barriers keep the row loads ahead of them, so waiting for the rows does
    // not wait for the keys)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < kRing; ++k) load_head(t, k, kb[k]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (!ok) raw[i] = make_uint4(0, 0, 0, 0);
    // squares of bf16 values are exact in fp32; the sum runs in fp64
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = bf16lo(w[j]), b = bf16hi(w[j]);
        ss += (double)(a * a) + (double)(b * b);
      }
    }
    const double nrm = sqrt(ss);
    const float inv = (float)(1.0 / (nrm > (double)kNormEps ? nrm : (double)kNormEps));
    const int rb = r >> 4;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // dims [8i, 8i+8): k-step i/4, k group i%4 → lane (r % 16) + 16·(i % 4)
      const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
      uint32_t hw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        hw[j] = pack2(f2bf(bf16lo(w[j]) * inv), f2bf(bf16hi(w[j]) * inv));
      const int frag = (h * 4 + rb) * kKSteps + (i >> 2);
      qs[frag * 64 + (r & 15) + 16 * (i & 3)] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    }
  }
  __syncthreads();

  // ---- this lane group's segment: queries [b0, b0 + nq) × nr_u rows each
  const int ty = 4 * blockIdx.y + grp;
  TileRows tr = {0, 0, 0, 0, 1};
  if (ty < g.n_tiles) tr = tile_rows_of(g, ty);
  const bool mean = token_reduce == MSA_TOKEN_REDUCE_MEAN;
  const float fin = (mean && g.parts == 1) ? 0.125f / (float)g.M : 0.125f;   // with the head mean
  const float eps2 = kNormEps * kNormEps;

  if (t >= n_ct) return;

  f32x4_t tot[kCB][4];
  auto head = [&](int h, const uint4 (&kb)[kCB][kKSteps]) {
    // The q̂ fragments do not change from tile to tile; without this compiler
    // barrier all 128 of them (512 registers) get hoisted out of the tile loop.
    asm volatile("" ::: "memory");
    // this head's 16 fragments are read first, so their LDS latency overlaps
    // the wait for the head's key loads; each serves both column blocks
    uint4 qa[4][kKSteps];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) qa[rb][ks] = qs[((h * 4 + rb) * kKSteps + ks) * 64 + lane];
    __builtin_amdgcn_sched_barrier(0);
    float inv_k[kCB];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      float nk = 0.0f;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        nk = dot2(kb[cb][ks].x, kb[cb][ks].x, nk);
        nk = dot2(kb[cb][ks].y, kb[cb][ks].y, nk);
        nk = dot2(kb[cb][ks].z, kb[cb][ks].z, nk);
        nk = dot2(kb[cb][ks].w, kb[cb][ks].w, nk);
      }
      nk += __shfl_xor(nk, 16);
      nk += __shfl_xor(nk, 32);
      inv_k[cb] = __builtin_amdgcn_rsqf(fmaxf(nk, eps2));
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[rb][ks]),
                                                        as_bf16x8(kb[cb][ks]), acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[cb][rb][i] = fmaf(acc[i], inv_k[cb], tot[cb][rb][i]);
      }
  };

  // Token reduction of each query of this lane group, then store.
  //   One token per query with 16-byte aligned rows (the batched decode case):
  //   no reduction; a 4×4 transpose within each lane quad (two DPP exchange
  //   steps) gives lane j of a quad four consecutive chunk scores of query
  //   4·rb + j, so each query row of the tile is written as two full 64-byte
  //   runs by 16-byte stores.
  //   Otherwise each column block is parked in the wave's LDS slice
  //   ([group][position][column]) and every query is reduced with an ordinary
  //   loop; a wave's LDS accesses run in order, so no barrier is needed.
  float* wl = reinterpret_cast<float*>(qs + kFrags * 64) + wave * (kRows * 16) +
              grp * (kSegRows * 16) + col;
  const bool vec_rows =
      nr_u == 1 && (n_chunks & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  const int j0 = lane & 1, j1 = (lane >> 1) & 1;
  auto finish = [&](int64_t tile) {
    const int64_t c0 = tile * kChunkTile;
    if (vec_rows && c0 + kChunkTile <= n_chunks) {
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          // register i of lane j (in the quad) holds (query 4rb+i, chunk j)
          float v0 = tot[cb][rb][0], v1 = tot[cb][rb][1];
          float v2 = tot[cb][rb][2], v3 = tot[cb][rb][3];
          // swap bit 0 of the register index with bit 0 of the lane index
          float s0 = j0 ? v0 : v1, s1 = j0 ? v2 : v3;
          s0 = dpp_f<0xB1>(s0);
          s1 = dpp_f<0xB1>(s1);
          if (j0) { v0 = s0; v2 = s1; } else { v1 = s0; v3 = s1; }
          // swap bit 1 of the register index with bit 1 of the lane index
          s0 = j1 ? v0 : v2;
          s1 = j1 ? v1 : v3;
          s0 = dpp_f<0x4E>(s0);
          s1 = dpp_f<0x4E>(s1);
          if (j1) { v0 = s0; v1 = s1; } else { v2 = s0; v3 = s1; }
          // lane (4a + j) now holds query 4rb + j, chunks 4a .. 4a + 3
          const int u = 4 * rb + (lane & 3);
          if (u < tr.nq) {
            float4* dst = reinterpret_cast<float4*>(
                out + (int64_t)(tr.b0 + u) * n_chunks + c0 + cb * 16 + 4 * ((lane >> 2) & 3));
            *dst = make_float4(v0 * fin, v1 * fin, v2 * fin, v3 * fin);
          }
        }
      return;
    }
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
#pragma unroll
      for (int u = 0; u < kSegRows; ++u) wl[u * 16] = tot[cb][u >> 2][u & 3];
      const int64_t c = c0 + cb * 16 + col;
      if (c < n_chunks) {
        float* p = out + ((int64_t)tr.part * g.B + tr.b0) * n_chunks + c;
        for (int q = 0; q < tr.nq; ++q) {
          const float* r = wl + q * nr_u * 16;
          float run = r[0];
          for (int m = 1; m < nr_u; ++m) {
            const float x = r[m * 16];
            run = mean ? run + x : nan_max(run, x);
          }
          p[(int64_t)q * n_chunks] = run * fin;
        }
      }
    }
  };

  while (true) {
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) tot[cb][rb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int64_t tn = t + stride;
#pragma unroll
    for (int h = 0; h < kHeads; ++h) {
      head(h, kb[h % kRing]);
      if (h + kRing < kHeads)
        load_head(t, h + kRing, kb[h % kRing]);
      else
        load_head(tn, h + kRing - kHeads, kb[h % kRing]);
    }
    finish(t);
    t = tn;
    if (t >= n_ct) break;
  }
}

}  // namespace

int launch_scan_mfma(const uint16_t* QR, const RouteGeom& g, const uint16_t* KRbar,
                     int64_t n_chunks, int32_t token_reduce, float* out, hipStream_t s) {
  if (n_chunks == 0 || g.n_tiles == 0) return MSA_OK;
  if (g.tile_rows != kSegRows) return fail(MSA_ERR_UNSUPPORTED, "MFMA scan needs 16-row segments");
  const int64_t n_ct = (n_chunks + kChunkTile - 1) / kChunkTile;
  const int n_ty = (g.n_tiles + 3) / 4;   // four segments per workgroup
  // one resident workgroup per CU (160 KiB of LDS); its waves stride over tiles
  int64_t wg = 256 / n_ty;
  if (wg < 1) wg = 1;
  const int64_t wg_max = (n_ct + kWaves - 1) / kWaves;
  if (wg > wg_max) wg = wg_max;
  // more than 64 KiB of dynamic LDS has to be allowed (set on every launch,
  // so the library keeps no state between calls)
  MSA_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(scan_mfma_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes));
  hipLaunchKernelGGL(scan_mfma_kernel, dim3((unsigned)wg, (unsigned)n_ty), dim3(kThreads),
                     kLdsBytes, s, QR, g, reinterpret_cast<const uint4*>(KRbar), n_chunks,
                     token_reduce, out);
  MSA_LAUNCH_CHECK("scan_mfma_kernel launch");
  return MSA_OK;
}

}  // namespace msa
