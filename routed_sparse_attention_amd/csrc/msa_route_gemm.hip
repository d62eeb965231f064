// msa_route_score for long query blocks: the cosine scan as one tiled bf16
// contraction over all router heads.
//
// Method (portal.techblg.uk IRMaD reading, section M, routing bullet):
//   S_tc = mean_h cos(Q^R_{t,h}, K̄^R_{c,h}),  S_c = max_t S_tc (or mean_t).
// With q̂ = q / max(‖q‖, eps) and k̂ = k / max(‖k‖, eps) per head, the head sum
// of cosines is a plain sum of products over all 8 × 128 router dims, so a
// query's scores are one [rows × 1024] · [1024 × chunks] product followed by
// a max (or sum) over each query's rows (section M, Memory Parallel bullet:
// the score matrix is computed in tiles and never held whole).
//
// Used when M is a multiple of 128: 256-row tiles when M is a multiple of
// 256, else 128-row tiles (every row tile then belongs to one query; a
// 256-row tile over a 128-token query would leave half its products unused).
// The kernels below are written for 256-row tiles; with 128-row tiles each
// wave has two 32-row blocks instead of four, and nothing else changes.
// Design:
//   - qhat_rows_kernel writes q̂ once per call (fp64 norm per (row, head),
//     the scaled value formed in fp32 and rounded to bf16);
//   - scan_gemm_kernel: a workgroup of 8 waves owns 256 query rows × kCols
//     chunks and walks the 8 heads as the contraction's k-steps (128 dims
//     each). Each step's q̂ rows and key rows are staged through registers
//     into LDS while the previous step's products run; the threads that stage
//     a key row normalise it on the way (‖k‖ from the values they hold, a DPP
//     sum over the 16 lanes sharing the row, then k̂ rounded to bf16). Rounding
//     k̂ as well as q̂ to bf16 moves a score by ~1e-4 at most, inside the 1e-3
//     score tolerance;
//   - wave (wr, wc) computes rows 128·wr .. +128 × a quarter of the chunks with
//     v_mfma_f32_32x32x16_bf16 (A = q̂ rows, B = k̂ rows, both read from LDS as
//     one 16-byte fragment per lane; rows padded to 136 bf16 so the reads are
//     bank-conflict free), accumulating all heads in one register tile;
//   - epilogue: each wave reduces its 128 rows per chunk column (registers,
//     then one exchange between the two lane halves) and the workgroup's two
//     row halves are merged through LDS, so a 256-token query needs no second
//     pass (longer queries write one partial per 256 rows);
//   - with 4 or more row tiles (and 256-chunk tiles) the staged form below
//     takes over: k̂ written once per call, q̂ and k̂ rows moved by DMA into
//     two 64-dim LDS stages, one in flight while the other is multiplied
//     (bit-identical scores: the same products in the same order);
//   - workgroup order is XCD-aware (consecutive workgroups go to the 8 XCDs in
//     turn). With 4 or more row tiles, each XCD runs blocks of 4 row tiles ×
//     8 chunk tiles, 32 workgroups at a time, and its next block keeps the
//     same row tiles while the eight XCDs walk the same chunk blocks: an XCD's
//     q̂ rows stay in its L2 and each key block is fetched while all eight read
//     it (32 queries × 256 tokens over 157K chunks: 10.4 → 3.8 GB of L2
//     misses, 3.57 → 3.31 ms). With fewer row tiles, workgroup L runs chunk
//     tile (L % 8) + 8·(L / 8 / Y) for row tile (L / 8) % Y.
#include "msa_internal.h"

namespace msa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kGWaves = 8;
constexpr int kGThreads = 64 * kGWaves;
constexpr int kGRows = 256;          // query rows per workgroup tile
constexpr int kGPitch = 136;         // bf16 per LDS row (128 + 8: conflict-free fragment reads)

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// Reduces each chunk column's 32·kRB rows of a wave tile: this lane's 16·kRB
// accumulator values of the column (row blocks 0..kRB-1 × 16, in that order),
// then the other lane half's through one exchange. A sum for the mean
// reduction; for the max, a maximum that is NaN when any value is. The max
// takes fmaxf (which skips NaN) and carries a NaN through a running sum of
// the same values: the values are finite or NaN (head sums of products of
// unit vectors, |value| <= 8 up to rounding), so that sum is NaN exactly when
// one of them is. Both branches are straight-line code (the branch is
// uniform), so the epilogue costs one or two VALU operations per value.
template <int kRB, int kNcb>
__device__ __forceinline__ void reduce_columns(const f32x16_t (&acc)[kRB][kNcb], bool mean,
                                               int half, float (&red)[kNcb]) {
  if (mean) {
#pragma unroll
    for (int cb = 0; cb < kNcb; ++cb) {
      float r = acc[0][cb][0];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int v = (rb == 0 ? 1 : 0); v < 16; ++v) r += acc[rb][cb][v];
      const float o = __shfl_xor(r, 32);
      red[cb] = half == 0 ? r + o : o + r;
    }
  } else {
#pragma unroll
    for (int cb = 0; cb < kNcb; ++cb) {
      float r = acc[0][cb][0], z = r;
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int v = (rb == 0 ? 1 : 0); v < 16; ++v) {
          r = fmaxf(r, acc[rb][cb][v]);
          z += acc[rb][cb][v];
        }
      r = z != z ? z : r;
      const float o = __shfl_xor(r, 32);
      red[cb] = half == 0 ? nan_max(r, o) : nan_max(o, r);
    }
  }
}
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// q̂ rows: one thread per (row, head), 128 dims. Same arithmetic as the
// batched scan's staging: fp64 sum of squares, inv = 1 / max(‖q‖, eps)
// rounded to fp32, q̂ = bf16(q · inv) formed in fp32.
__global__ __launch_bounds__(256) void qhat_rows_kernel(const uint16_t* __restrict__ QR,
                                                         int64_t n_rows, uint16_t* __restrict__ Qh) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // row * 8 + head
  if (i >= n_rows * kHeads) return;
  const uint4* src = reinterpret_cast<const uint4*>(QR) + i * (kDim / 8);
  uint4 raw[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) raw[k] = src[k];
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const uint32_t w[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = bf16lo(w[j]), b = bf16hi(w[j]);
      ss += (double)(a * a) + (double)(b * b);
    }
  }
  const double nrm = sqrt(ss);
  const float inv = (float)(1.0 / (nrm > (double)kNormEps ? nrm : (double)kNormEps));
  uint4* dst = reinterpret_cast<uint4*>(Qh) + i * (kDim / 8);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const uint32_t w[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack2(f2bf(bf16lo(w[j]) * inv), f2bf(bf16hi(w[j]) * inv));
    dst[k] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

struct GemmGeom {
  int32_t B, M;
  int64_t n_rows;        // B · M
  int32_t n_row_tiles;   // n_rows / tile rows (256, or 128 when M is an odd multiple of 128)
  int32_t n_col_tiles;   // ceil(n_chunks / kCols)
  int32_t parts;         // row tiles per query (1: final scores)
};

template <int kRows, int kCols>
__global__ __launch_bounds__(kGThreads) void scan_gemm_kernel(const uint16_t* __restrict__ Qh,
                                                              GemmGeom g,
                                                              const uint4* __restrict__ KR,
                                                              int64_t n_chunks,
                                                              int32_t token_reduce,
                                                              float* __restrict__ out) {
  constexpr int kNcb = kCols / 128;                 // 32-chunk column blocks per wave
  constexpr int kRB = kRows / 64;                   // 32-row blocks per wave
  constexpr int kQPass = kRows / 32;                // staging passes of the q̂ tile
  constexpr int kBPass = kCols / 32;                // staging passes of the key tile
  extern __shared__ uint4 lds4[];
  uint16_t* As = reinterpret_cast<uint16_t*>(lds4);          // [kRows][kGPitch] q̂ of one head
  uint16_t* Bs = As + kRows * kGPitch;                        // [kCols][kGPitch] k̂ of one head

  const int L = blockIdx.x;
  const int Y = g.n_row_tiles;
  const int xcd = L & 7, slot = L >> 3;
  int x, y;
  if (Y >= 4) {
    // blocks of 4 row tiles × 8 chunk tiles, one block per 32 consecutive
    // workgroups of an XCD; an XCD's next block keeps its row tiles
    const int blk = (slot >> 5) * 8 + xcd;
    const int j = slot & 31;
    const int RB = (Y + 3) / 4;
    y = 4 * (blk % RB) + (j >> 3);
    x = 8 * (blk / RB) + (j & 7);
    if (y >= Y) return;
  } else {
    x = xcd + 8 * (slot / Y);   // chunk tile
    y = slot % Y;               // row tile
  }
  if (x >= g.n_col_tiles) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int wr = wave & 1;                  // row half (kRows / 2 rows)
  const int wc = wave >> 1;                 // column quarter

  // staging: thread (r0, p) = (tid / 16, tid % 16) moves 16-byte piece p of
  // rows r0 + 32·i; the 16 lanes of one row are one DPP row
  const int p = tid & 15;
  const int r0 = tid >> 4;
  const int64_t c_base = (int64_t)x * kCols;
  const int64_t row_base = (int64_t)y * kRows;
  // Each load is the tile's base (uniform) plus a 32-bit per-thread offset
  // (a tile spans at most 512 KiB). Chunks past the end read the last chunk
  // (clamped); their results are not stored.
  constexpr int kRowV = kHeads * kDim / 8;                   // 16-byte vectors per row
  const u32x4_t* qtile = reinterpret_cast<const u32x4_t*>(Qh) + row_base * kRowV;
  const u32x4_t* ktile = reinterpret_cast<const u32x4_t*>(KR) + c_base * kRowV;
  const int k_rows = (int)min((int64_t)kCols, n_chunks - c_base);   // >= 1
  int koff[kBPass];
#pragma unroll
  for (int i = 0; i < kBPass; ++i) koff[i] = min(r0 + 32 * i, k_rows - 1) * kRowV + p;
  u32x4_t qreg[kQPass], kreg[kBPass];
  auto load = [&](int h) {
    const u32x4_t* qh = qtile + h * (kDim / 8);
    const u32x4_t* kh = ktile + h * (kDim / 8);
#pragma unroll
    for (int i = 0; i < kQPass; ++i) qreg[i] = qh[(r0 + 32 * i) * kRowV + p];
#pragma unroll
    for (int i = 0; i < kBPass; ++i) kreg[i] = kh[koff[i]];
  };
  const float eps2 = kNormEps * kNormEps;
  // k̂ = k / max(‖k‖, eps) per key row, in registers
  auto normalise = [&]() {
#pragma unroll
    for (int i = 0; i < kBPass; ++i) {
      const u32x4_t w = kreg[i];
      float nk = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) nk = dot2(w[j], w[j], nk);
      const float inv = __builtin_amdgcn_rsqf(fmaxf(row_sum16(nk), eps2));
      u32x4_t o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = cvt_pk_bf16(bf16lo(w[j]) * inv, bf16hi(w[j]) * inv);
      kreg[i] = o;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < kQPass; ++i)
      *reinterpret_cast<u32x4_t*>(As + (r0 + 32 * i) * kGPitch + p * 8) = qreg[i];
#pragma unroll
    for (int i = 0; i < kBPass; ++i)
      *reinterpret_cast<u32x4_t*>(Bs + (r0 + 32 * i) * kGPitch + p * 8) = kreg[i];
  };

  f32x16_t acc[kRB][kNcb];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
    for (int cb = 0; cb < kNcb; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0.0f;

  load(0);
  normalise();
  store();
  __syncthreads();

  // fragment rows of this wave: A rows (kRows/2)·wr + 32·rb + col, B rows
  // (chunks) wc·(kCols/4) + 32·cb + col; k slice 16·ks + 8·half
  const uint16_t* a_base = As + (wr * (kRows / 2) + col) * kGPitch + half * 8;
  const uint16_t* b_base = Bs + (wc * (kCols / 4) + col) * kGPitch + half * 8;

  for (int h = 0; h < kHeads; ++h) {
    if (h + 1 < kHeads) load(h + 1);
#pragma unroll
    for (int ks = 0; ks < kDim / 16; ++ks) {
      // the next head's keys are normalised half way through this head's
      // products, so their VALU work overlaps the MFMA pipeline
      if (ks == kDim / 32 && h + 1 < kHeads) normalise();
      u32x4_t a[kRB], b[kNcb];
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
        a[rb] = *reinterpret_cast<const u32x4_t*>(a_base + rb * 32 * kGPitch + ks * 16);
#pragma unroll
      for (int cb = 0; cb < kNcb; ++cb)
        b[cb] = *reinterpret_cast<const u32x4_t*>(b_base + cb * 32 * kGPitch + ks * 16);
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int cb = 0; cb < kNcb; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[rb]), as_bf16x8(b[cb]),
                                                                acc[rb][cb], 0, 0, 0);
    }
    __syncthreads();              // every wave is done with this head's tiles
    if (h + 1 < kHeads) {
      store();
      __syncthreads();
    }
  }

  // ---- epilogue: reduce this wave's kRows / 2 rows per chunk column
  const bool mean = token_reduce == MSA_TOKEN_REDUCE_MEAN;
  float red[kNcb];
  reduce_columns<kRB, kNcb>(acc, mean, half, red);
  // the two row halves are one query: half 1 hands its values to half 0,
  // which writes the tile's part (query y / parts, part y % parts)
  const float fin = (mean && g.parts == 1) ? 0.125f / (float)g.M : 0.125f;   // with the head mean
  float* xch = reinterpret_cast<float*>(lds4);        // [4 column quarters][kNcb][32]
  if (wr == 1 && half == 0) {
#pragma unroll
    for (int cb = 0; cb < kNcb; ++cb) xch[(wc * kNcb + cb) * 32 + col] = red[cb];
  }
  __syncthreads();
  if (wr == 0 && half == 0) {
    const int64_t b = y / g.parts, part = y % g.parts;
#pragma unroll
    for (int cb = 0; cb < kNcb; ++cb) {
      const int64_t c = c_base + wc * (kCols / 4) + cb * 32 + col;
      const float o = xch[(wc * kNcb + cb) * 32 + col];
      if (c < n_chunks) out[(part * g.B + b) * n_chunks + c] = (mean ? red[cb] + o : nan_max(red[cb], o)) * fin;
    }
  }
}

// ---------------------------------------------------------------------------
// Staged form for many row tiles. k̂ is written once per call by
// khat_rows_kernel (the same arithmetic as the staging threads' normalise
// above, so a key's k̂ is bit-identical), and the contraction then reads q̂
// and k̂ rows by DMA (global_load_lds, 1 KiB per instruction) into two LDS
// stage buffers of 64 dims each: stage s + 1 is in flight while stage s is
// multiplied, with no register staging and no normalisation in the loop.
// The k-steps run over the same dims in the same order as the kernel above,
// so the scores are bit-identical to it.
//
// Stage layout (per buffer): q̂ rows 0..255 then key rows 0..kCols-1, 128
// bytes (8 pieces of 16 bytes) each, in blocks of 8 rows per KiB; piece p of
// row r sits at slot 8·(r % 8) + (p ^ ((r >> 1) & 7)) of its block, so the
// MFMA fragment reads (32 rows × one piece) hit 16 different bank groups
// per 16 lanes. Each wave fills 8 of the blocks.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void khat_rows_kernel(const uint4* __restrict__ KR,
                                                         int64_t n_rows,
                                                         uint4* __restrict__ Kh) {
  // thread (row, p): piece p of (chunk, head) row `row`; a row is one DPP row
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = t >> 4;
  const int p = (int)(t & 15);
  const bool ok = row < n_rows;
  u32x4_t w = {0u, 0u, 0u, 0u};
  if (ok) w = reinterpret_cast<const u32x4_t*>(KR)[row * 16 + p];
  float nk = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) nk = dot2(w[j], w[j], nk);
  const float inv = __builtin_amdgcn_rsqf(fmaxf(row_sum16(nk), kNormEps * kNormEps));
  u32x4_t o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = cvt_pk_bf16(bf16lo(w[j]) * inv, bf16hi(w[j]) * inv);
  if (ok) reinterpret_cast<u32x4_t*>(Kh)[row * 16 + p] = o;
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gmem_void_t;
constexpr int kSDims = 64;                          // dims per stage
constexpr int kSRowBytes = kSDims * 2;              // 128 B per row per stage
constexpr int kStages = kHeads * kDim / kSDims;     // 16
// s_waitcnt: vmcnt(N) only / lgkmcnt(0) only (gfx9 field layout)
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}
// Workgroup barrier that keeps memory accesses on their side of it in the
// compiler (the barrier intrinsic alone orders none). Not a memory-model
// fence: a release fence would also wait for this wave's stage loads in
// flight (they count as LDS writes); the explicit vmcnt / lgkmcnt waits
// around each barrier give the ordering the hardware needs.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int kCols>
__global__ __launch_bounds__(kGThreads) void scan_gemm_dma_kernel(const uint16_t* __restrict__ Qh,
                                                                  GemmGeom g,
                                                                  const uint16_t* __restrict__ Kh,
                                                                  int64_t n_chunks,
                                                                  int32_t token_reduce,
                                                                  float* __restrict__ out) {
  constexpr int kNcb = kCols / 128;                 // 32-chunk column blocks per wave
  constexpr int kBlocks = (kGRows + kCols) / 8;     // 1 KiB blocks per stage
  constexpr int kBlocksPerWave = kBlocks / kGWaves;
  constexpr int kBufBytes = kBlocks * 1024;
  __shared__ __attribute__((aligned(16))) uint8_t buf0[kBufBytes];
  __shared__ __attribute__((aligned(16))) uint8_t buf1[kBufBytes];

  const int L = blockIdx.x;
  const int Y = g.n_row_tiles;
  const int xcd = L & 7, slot = L >> 3;
  int x, y;
  if (Y >= 4) {
    const int blk = (slot >> 5) * 8 + xcd;
    const int j = slot & 31;
    const int RB = (Y + 3) / 4;
    y = 4 * (blk % RB) + (j >> 3);
    x = 8 * (blk / RB) + (j & 7);
    if (y >= Y) return;
  } else {
    x = xcd + 8 * (slot / Y);
    y = slot % Y;
  }
  if (x >= g.n_col_tiles) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int wr = wave & 1;
  const int wc = wave >> 1;
  const int64_t c_base = (int64_t)x * kCols;
  const int64_t row_base = (int64_t)y * kGRows;

  // this lane's source row and piece in each of its wave's blocks (the
  // same for every stage; the stage adds 64 dims)
  const uint16_t* src[kBlocksPerWave];
#pragma unroll
  for (int bi = 0; bi < kBlocksPerWave; ++bi) {
    const int blk = wave * kBlocksPerWave + bi;
    const int slot_l = lane;                     // LDS slot of this lane in the block
    const int rl = slot_l >> 3;                  // row within the block
    if (blk < kGRows / 8) {
      const int r = 8 * blk + rl;
      const int p = (slot_l & 7) ^ ((r >> 1) & 7);
      src[bi] = Qh + (row_base + r) * kRowElems + 8 * p;
    } else {
      const int r = 8 * (blk - kGRows / 8) + rl;
      const int p = (slot_l & 7) ^ ((r >> 1) & 7);
      int64_t c = c_base + r;
      c = c < n_chunks ? c : n_chunks - 1;       // in bounds; not stored
      src[bi] = Kh + c * kRowElems + 8 * p;
    }
  }
  auto issue = [&](int st, uint8_t* buf) {
#pragma unroll
    for (int bi = 0; bi < kBlocksPerWave; ++bi)
      __builtin_amdgcn_global_load_lds((gmem_void_t*)(src[bi] + st * kSDims),
                                       (lds_void_t*)(buf + (wave * kBlocksPerWave + bi) * 1024),
                                       16, 0, 0);
  };

  f32x16_t acc[4][kNcb];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < kNcb; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0.0f;

  // fragment byte offsets within a stage buffer (k-step ks adds pieces 2ks)
  int a_off[4], b_off[kNcb];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int R = 128 * wr + 32 * rb + col;
    a_off[rb] = 1024 * (R >> 3) + 16 * (8 * (R & 7));
  }
#pragma unroll
  for (int cb = 0; cb < kNcb; ++cb) {
    const int R = (kCols / 4) * wc + 32 * cb + col;
    b_off[cb] = kGRows * kSRowBytes + 1024 * (R >> 3) + 16 * (8 * (R & 7));
  }
  int a_sw[4], b_sw[kNcb];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) a_sw[rb] = ((128 * wr + 32 * rb + col) >> 1) & 7;
#pragma unroll
  for (int cb = 0; cb < kNcb; ++cb) b_sw[cb] = (((kCols / 4) * wc + 32 * cb + col) >> 1) & 7;
  // (a macro, not a lambda: the reads must name buf0 / buf1 themselves, so
  // the compiler waits only for the DMA of the buffer being read)
#define MSA_GEMM_STAGE(BUF)                                                              \
  _Pragma("unroll") for (int ks = 0; ks < kSDims / 16; ++ks) {                             \
    const int P = 2 * ks + half;                                                           \
    u32x4_t a[4], b[kNcb];                                                                 \
    _Pragma("unroll") for (int rb = 0; rb < 4; ++rb)                                       \
      a[rb] = *reinterpret_cast<const u32x4_t*>(&BUF[a_off[rb] + 16 * (P ^ a_sw[rb])]);    \
    _Pragma("unroll") for (int cb = 0; cb < kNcb; ++cb)                                    \
      b[cb] = *reinterpret_cast<const u32x4_t*>(&BUF[b_off[cb] + 16 * (P ^ b_sw[cb])]);    \
    _Pragma("unroll") for (int rb = 0; rb < 4; ++rb)                                       \
      _Pragma("unroll") for (int cb = 0; cb < kNcb; ++cb)                                  \
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                             \
            as_bf16x8(a[rb]), as_bf16x8(b[cb]), acc[rb][cb], 0, 0, 0);                     \
  }

  issue(0, buf0);
  issue(1, buf1);
  // whole ring turns with no branch inside: stages st (buf0) and st + 1
  // (buf1), refilling each buffer with the stage two ahead once read
  for (int st = 0; st + 2 < kStages; st += 2) {
    wait_vm<kBlocksPerWave>();          // stage st landed (st + 1 may be in flight)
    lds_barrier();
    MSA_GEMM_STAGE(buf0)
    wait_lgkm0();
    lds_barrier();       // every wave is done reading buf0
    issue(st + 2, buf0);
    wait_vm<kBlocksPerWave>();          // stage st + 1 landed
    lds_barrier();
    MSA_GEMM_STAGE(buf1)
    wait_lgkm0();
    lds_barrier();
    issue(st + 3, buf1);
  }
  // the last two stages
  wait_vm<kBlocksPerWave>();
  lds_barrier();
  MSA_GEMM_STAGE(buf0)
  wait_vm<0>();
  lds_barrier();
  MSA_GEMM_STAGE(buf1)
  wait_lgkm0();
  lds_barrier();

#undef MSA_GEMM_STAGE

  // ---- epilogue: as in scan_gemm_kernel
  const bool mean = token_reduce == MSA_TOKEN_REDUCE_MEAN;
  float red[kNcb];
  reduce_columns<4, kNcb>(acc, mean, half, red);
  const float fin = (mean && g.parts == 1) ? 0.125f / (float)g.M : 0.125f;
  float* xch = reinterpret_cast<float*>(buf0);
  if (wr == 1 && half == 0) {
#pragma unroll
    for (int cb = 0; cb < kNcb; ++cb) xch[(wc * kNcb + cb) * 32 + col] = red[cb];
  }
  __syncthreads();
  if (wr == 0 && half == 0) {
    const int64_t b = y / g.parts, part = y % g.parts;
#pragma unroll
    for (int cb = 0; cb < kNcb; ++cb) {
      const int64_t c = c_base + wc * (kCols / 4) + cb * 32 + col;
      const float o = xch[(wc * kNcb + cb) * 32 + col];
      if (c < n_chunks) out[(part * g.B + b) * n_chunks + c] = (mean ? red[cb] + o : nan_max(red[cb], o)) * fin;
    }
  }
}

template <int kRows, int kCols>
constexpr size_t gemm_lds_bytes() {
  return (size_t)(kRows + kCols) * kGPitch * 2;
}

}  // namespace

template <int kRows, int kCols>
static int launch_tiles(dim3 grid, const uint16_t* qhat, const GemmGeom& g, const uint4* kr,
                        int64_t n_chunks, int32_t token_reduce, float* out, hipStream_t s) {
  const void* fn = reinterpret_cast<const void*>(scan_gemm_kernel<kRows, kCols>);
  constexpr size_t lds = gemm_lds_bytes<kRows, kCols>();
  MSA_HIP(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
  hipLaunchKernelGGL((scan_gemm_kernel<kRows, kCols>), grid, dim3(kGThreads), lds, s, qhat, g, kr,
                     n_chunks, token_reduce, out);
  MSA_LAUNCH_CHECK("scan_gemm_kernel launch");
  return MSA_OK;
}

// Row tiles of 256 when M is a multiple of 256, else 128 (a 128-row tile has
// half the products per key byte, but a 256-row tile would leave half of its
// products unused).
static int32_t gemm_tile_rows(int32_t M) { return M % kGRows == 0 ? kGRows : kGRows / 2; }

bool scan_gemm_fits(int32_t M) { return M >= kGRows / 2 && M % (kGRows / 2) == 0; }

int32_t scan_gemm_parts(int32_t M) { return M / gemm_tile_rows(M); }

// The staged form is used from kKhatMinTiles row tiles on: its k̂ pass
// (a read and a write of the key store) then costs a few percent of the
// contraction, while for one or two 256-row tiles it would cost as much.
constexpr int32_t kKhatMinTiles = 4;
static bool gemm_staged(int32_t B, int32_t M) {
  return M % kGRows == 0 && (int64_t)B * M / kGRows >= kKhatMinTiles;
}

size_t scan_gemm_ws_bytes(int32_t B, int32_t M, int64_t n_chunks) {
  size_t b = align_up((size_t)B * M * kHeads * kDim * 2, 256);
  if (gemm_staged(B, M)) b += align_up((size_t)n_chunks * kRowElems * 2, 256);
  return b;
}

int launch_scan_gemm(const uint16_t* QR, int32_t B, int32_t M, const uint16_t* KRbar,
                     int64_t n_chunks, int32_t token_reduce, float* out, void* ws,
                     hipStream_t s) {
  uint16_t* qhat = static_cast<uint16_t*>(ws);
  if (n_chunks == 0 || B == 0) return MSA_OK;
  if (!scan_gemm_fits(M)) return fail(MSA_ERR_UNSUPPORTED, "tiled scan needs M a multiple of 128");
  const int32_t rows = gemm_tile_rows(M);
  GemmGeom g;
  g.B = B;
  g.M = M;
  g.n_rows = (int64_t)B * M;
  if (g.n_rows / rows > 0x7fffffffLL) return fail(MSA_ERR_SHAPE, "tiled scan: too many rows");
  g.n_row_tiles = (int32_t)(g.n_rows / rows);
  g.parts = scan_gemm_parts(M);
  const int64_t qthreads = g.n_rows * kHeads;
  // one-wave workgroups: a 256-token query's 2,048 (row, head) threads spread
  // over 32 CUs instead of 8 (each thread's loads are 16 strided 16-byte reads)
  hipLaunchKernelGGL(qhat_rows_kernel, dim3((unsigned)((qthreads + 63) / 64)), dim3(64), 0, s,
                     QR, g.n_rows, qhat);
  MSA_LAUNCH_CHECK("qhat_rows_kernel launch");
  // 256-chunk tiles when they give at least two workgroups per CU, else 128
  const int64_t tiles256 = (n_chunks + 255) / 256;
  const bool wide = tiles256 * g.n_row_tiles >= 512;
  const int cols = wide ? 256 : 128;
  g.n_col_tiles = (int32_t)((n_chunks + cols - 1) / cols);
  int64_t n_wg = 8 * (((int64_t)g.n_col_tiles + 7) / 8) * g.n_row_tiles;
  if (g.n_row_tiles >= 4) {
    const int64_t blocks = (((int64_t)g.n_row_tiles + 3) / 4) * (((int64_t)g.n_col_tiles + 7) / 8);
    n_wg = 8 * 32 * ((blocks + 7) / 8);
  }
  if (n_wg > 0x7fffffffLL) return fail(MSA_ERR_SHAPE, "tiled scan: grid too large");
  const uint4* kr = reinterpret_cast<const uint4*>(KRbar);
  if (gemm_staged(B, M) && wide) {
    uint16_t* khat = qhat + align_up((size_t)g.n_rows * kHeads * kDim * 2, 256) / 2;
    const int64_t krows = n_chunks * kHeads;
    hipLaunchKernelGGL(khat_rows_kernel, dim3((unsigned)((krows * 16 + 255) / 256)), dim3(256), 0,
                       s, kr, krows, reinterpret_cast<uint4*>(khat));
    MSA_LAUNCH_CHECK("khat_rows_kernel launch");
    hipLaunchKernelGGL(scan_gemm_dma_kernel<256>, dim3((unsigned)n_wg), dim3(kGThreads), 0, s,
                       qhat, g, khat, n_chunks, token_reduce, out);
    MSA_LAUNCH_CHECK("scan_gemm_dma_kernel launch");
    return MSA_OK;
  }
  const dim3 grid((unsigned)n_wg);
  if (rows == kGRows)
    return wide ? launch_tiles<kGRows, 256>(grid, qhat, g, kr, n_chunks, token_reduce, out, s)
                : launch_tiles<kGRows, 128>(grid, qhat, g, kr, n_chunks, token_reduce, out, s);
  return wide ? launch_tiles<kGRows / 2, 256>(grid, qhat, g, kr, n_chunks, token_reduce, out, s)
              : launch_tiles<kGRows / 2, 128>(grid, qhat, g, kr, n_chunks, token_reduce, out, s);
}

}  // namespace msa
