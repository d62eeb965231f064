// msa_gather_attend: context assembly, global RoPE and sparse attention
// (MSA stage 3).
//
// Method (portal.techblg.uk IRMaD reading, section M, routing bullet and
// positional-encoding bullet):
//   K_ctx = [{K̄_i}_{i∈I}; K_q],  V_ctx = [{V̄_i}_{i∈I}; V_q],
//   Output = Attention(Q_q, K_ctx, V_ctx),
// and the active context (query and generated tokens) carries global RoPE with
// positions offset from k (also zhichai.net "关键技术细节" 1, chooseai.io 2.2).
// Readings: local token v sits at pos0 + v with pos0 = n_sel by default; the
// M query tokens are the last M local tokens; memory chunks are fully visible
// and local keys causal; logits scale 1/sqrt(128); q head h reads KV head
// h / (Hq / 8); memory chunks enter in rank order.
//
// Pipeline (one stream, three launches):
//   prep      block 0 turns the selected ids into the list of memory chunk
//             rows (and n_mem); the other blocks rotate Q and K_loc into the
//             workspace (bf16), one thread per rotation pair;
//   attn      flash attention, one wave per (32 query rows of one KV group,
//             KV head, key split), about 2048 waves. Each 32-key tile of K
//             and V is read with one 256-byte row per 16 lanes (coalesced,
//             and large PCIe reads when K̄/V̄ sit in pinned host memory —
//             they are read in place, with no staging copy) and staged in
//             LDS: K row-major, V transposed (a lane holds 8 consecutive keys,
//             so each dim's keys go out as one 16-byte store), so both MFMA B
//             fragments are 16-byte LDS reads. Row maxima and sums use DPP
//             within 16-lane rows and one exchange between rows.
//             S = Q·K^T and O += P·V use v_mfma_f32_32x32x16_bf16; the online
//             softmax runs in fp32 in the exp2 domain; P is re-laid out from
//             the accumulator layout to the A-operand layout through LDS;
//   combine   merges the key splits (log-sum-exp weights computed once per
//             row in LDS, then one independent load per split and dim) and
//             writes bf16 (and optionally fp32) output.
#include "msa_internal.h"

namespace msa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kKeyTile = 32;
constexpr int kRowTile = 32;
constexpr int kMaxSplits = 256;
constexpr float kLog2e = 1.4426950408889634f;

struct AttnWs {
  int32_t* mem_rows;   // [max_sel_chunks]
  int32_t* n_mem;      // [1]
  uint16_t* Qr;        // [M][Hq][128]
  uint16_t* Kr;        // [M_loc][8][128]
  float* Opart;        // [n_splits][M*Hq][128]
  float* ML;           // [n_splits][M*Hq][2]
};

struct PrepArgs {
  const int32_t* sel_ids; const int32_t* n_sel; int32_t top_k;
  const int64_t* dco; int32_t n_docs; int64_t n_chunks; int64_t max_sel; int64_t pos0;
  const uint16_t* Q; int32_t M; int32_t Hq;
  const uint16_t* Kl; int32_t M_loc; int32_t rotate_k; double theta;
  int32_t* mem_rows; int32_t* n_mem; uint16_t* Qr; uint16_t* Kr;
};

__device__ __forceinline__ int clamp_nsel(const int32_t* n_sel, int top_k) {
  int ns = *n_sel;
  return ns < 0 ? 0 : (ns > top_k ? top_k : ns);
}

__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
  if (blockIdx.x == 0) {
    // ---- chunk list of the selected documents, in rank order
    if (threadIdx.x >= 64) return;
    const int lane = threadIdx.x;
    const int ns = clamp_nsel(a.n_sel, a.top_k);
    int64_t start = 0, cnt = 0;
    if (lane < ns) {
      const int32_t id = a.sel_ids[lane];
      if (id >= 0 && id < a.n_docs) {
        int64_t c0 = a.dco[id], c1 = a.dco[id + 1];
        c0 = max((int64_t)0, min(c0, a.n_chunks));
        c1 = max(c0, min(c1, a.n_chunks));
        start = c0;
        cnt = c1 - c0;
      }
    }
    int64_t incl = cnt;
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    const int64_t off = incl - cnt;
    const int64_t total = __shfl(incl, 63);
    for (int64_t j = 0; j < cnt && off + j < a.max_sel; ++j)
      a.mem_rows[off + j] = (int32_t)(start + j);
    if (lane == 0) *a.n_mem = (int32_t)(total < a.max_sel ? total : a.max_sel);
    return;
  }
  // ---- global RoPE: Q rows u·Hq + h at pos0 + (M_loc − M) + u; K rows v·8 + g at pos0 + v
  const int64_t q_pairs = (int64_t)a.M * a.Hq * 64;
  const int64_t k_pairs = a.rotate_k ? (int64_t)a.M_loc * kHeads * 64 : 0;
  const int64_t idx = (int64_t)(blockIdx.x - 1) * blockDim.x + threadIdx.x;
  if (idx >= q_pairs + k_pairs) return;
  const int64_t pos0 = a.pos0 < 0 ? (int64_t)clamp_nsel(a.n_sel, a.top_k) : a.pos0;
  const uint16_t* src;
  uint16_t* dst;
  int64_t pos;
  int m;
  if (idx < q_pairs) {
    const int64_t row = idx / 64;
    m = (int)(idx % 64);
    pos = pos0 + (a.M_loc - a.M) + row / a.Hq;
    src = a.Q + row * kDim;
    dst = a.Qr + row * kDim;
  } else {
    const int64_t k = idx - q_pairs;
    const int64_t row = k / 64;
    m = (int)(k % 64);
    pos = pos0 + row / kHeads;
    src = a.Kl + row * kDim;
    dst = a.Kr + row * kDim;
  }
  const double om = pow(a.theta, -2.0 * (double)m / (double)kDim);
  double sn, cs;
  sincos((double)pos * om, &sn, &cs);
  const double x = bf16f(src[m]), y = bf16f(src[m + 64]);
  dst[m] = d2bf(x * cs - y * sn);
  dst[m + 64] = d2bf(y * cs + x * sn);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// LDS pitches (bf16 elements)
constexpr int kKPitch = 136;  // K tile [32 keys][128 dims]
constexpr int kVPitch = 40;   // V^T tile [128 dims][32 keys]
constexpr int kPPitch = 40;   // P tile [32 rows][32 keys]

__global__ __launch_bounds__(64) void attn_kernel(const uint16_t* __restrict__ Qr, int32_t M,
                                                  int32_t Hq, const uint16_t* __restrict__ Kloc,
                                                  const uint16_t* __restrict__ Vloc,
                                                  int32_t M_loc, const uint16_t* Kbar,
                                                  const uint16_t* Vbar,
                                                  const int32_t* __restrict__ mem_rows,
                                                  const int32_t* __restrict__ n_mem_p,
                                                  int32_t key_split, float qk_scale_log2,
                                                  float* __restrict__ Opart,
                                                  float* __restrict__ ML) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kKeyTile * kKPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kDim * kVPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Ps[kRowTile * kPPitch];

  const int lane = threadIdx.x;
  const int col = lane & 31;      // MFMA column lane (key / dim)
  const int half = lane >> 5;     // which 8-wide k slice this lane holds
  const int rb = blockIdx.x;      // row block within the KV group
  const int g = blockIdx.y;       // KV head
  const int split = blockIdx.z;
  const int G = Hq / kHeads;      // query heads per KV head
  const int rows_g = M * G;
  const int n_mem = *n_mem_p;
  const int n_keys = n_mem + M_loc;
  const int k_begin = split * key_split;
  const int k_end = min(k_begin + key_split, n_keys);
  const int64_t n_rows_tot = (int64_t)M * Hq;

  // A fragments of this lane's query row (row = lane % 32 of the block)
  uint4 qa[8];
  {
    const int r = rb * kRowTile + col;
    if (r < rows_g) {
      const int u = r / G, h = g * G + r % G;
      const uint4* qrow = reinterpret_cast<const uint4*>(Qr + ((int64_t)u * Hq + h) * kDim);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qa[ks] = qrow[ks * 2 + half];
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qa[ks] = make_uint4(0, 0, 0, 0);
    }
  }
  // Accumulator rows held by this lane: r(v) = base_r + off(v), with
  // off(v) = 8(v/4) + v%4 a constant; row r is valid while off(v) < rem.
  const int base_r = rb * kRowTile + 4 * half;
  const int rem = rows_g - base_r;

  f32x16_t O[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) O[db][v] = 0.0f;
  float mrow[16], lpart[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) { mrow[v] = -INFINITY; lpart[v] = 0.0f; }

  // Load layout: lane (sub, dv) = (lane / 16, lane % 16) reads the 16-byte
  // vector dv of keys 8·sub .. 8·sub + 7 (one instruction covers 4 keys' 256-byte
  // head rows, 16 lanes each), so a lane holds 8 consecutive keys of the same
  // 8 dims and writes each dim's 8 keys of V^T as one 16-byte store.
  const int sub = lane >> 4;
  const int dv = lane & 15;
  for (int kt = k_begin; kt < k_end; kt += kKeyTile) {
    // ---- K and V tiles. Keys past the split are clamped to its last key (a
    //      real row, so finite) and masked out of the softmax below.
    uint4 kx[8], vx[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int j = min(kt + sub * 8 + it, k_end - 1);
      const bool mem = j < n_mem;
      const int64_t off = mem ? ((int64_t)mem_rows[j] * kHeads + g) * kDim
                              : ((int64_t)(j - n_mem) * kHeads + g) * kDim;
      kx[it] = reinterpret_cast<const uint4*>((mem ? Kbar : Kloc) + off)[dv];
      vx[it] = reinterpret_cast<const uint4*>((mem ? Vbar : Vloc) + off)[dv];
    }
#pragma unroll
    for (int it = 0; it < 8; ++it)
      *reinterpret_cast<uint4*>(&Ks[(sub * 8 + it) * kKPitch + dv * 8]) = kx[it];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // dim dv·8 + e of keys 8·sub .. 8·sub + 7
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4& a = vx[2 * q];
        const uint4& b = vx[2 * q + 1];
        const uint32_t wa = (e >> 1) == 0 ? a.x : (e >> 1) == 1 ? a.y : (e >> 1) == 2 ? a.z : a.w;
        const uint32_t wb = (e >> 1) == 0 ? b.x : (e >> 1) == 1 ? b.y : (e >> 1) == 2 ? b.z : b.w;
        w[q] = (e & 1) ? ((wa >> 16) | (wb & 0xffff0000u)) : ((wa & 0xffffu) | (wb << 16));
      }
      *reinterpret_cast<uint4*>(&Vt[(dv * 8 + e) * kVPitch + sub * 8]) =
          make_uint4(w[0], w[1], w[2], w[3]);
    }
    __syncthreads();

    // ---- S = Q K^T (rows × 32 keys)
    f32x16_t S;
#pragma unroll
    for (int v = 0; v < 16; ++v) S[v] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint4 kb = *reinterpret_cast<const uint4*>(&Ks[col * kKPitch + ks * 16 + half * 8]);
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qa[ks]), as_bf16x8(kb), S, 0, 0, 0);
    }

    // ---- mask, scale to the log2 domain, online softmax
    const int j = kt + col;
    const bool key_ok = j < k_end;
    // causal: local key vloc is visible to query token u = r / G iff
    // u >= vloc - (M_loc - M), i.e. r >= (vloc - (M_loc - M))·G
    const int lim_off = j < n_mem ? -(1 << 30) : (j - n_mem - (M_loc - M)) * G - base_r;
    float p[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int off = 8 * (v >> 2) + (v & 3);
      const bool ok = key_ok && off < rem && off >= lim_off;
      const float s = ok ? S[v] * qk_scale_log2 : -INFINITY;
      // max over the row's 32 key lanes: four DPP steps within each 16-lane
      // row, then one exchange between the two rows of this half
      float t = s;
      t = fmaxf(t, dpp_f<0xB1>(t));    // quad_perm [1,0,3,2]
      t = fmaxf(t, dpp_f<0x4E>(t));    // quad_perm [2,3,0,1]
      t = fmaxf(t, dpp_f<0x141>(t));   // row_half_mirror
      t = fmaxf(t, dpp_f<0x140>(t));   // row_mirror
      t = fmaxf(t, __shfl_xor(t, 16));
      const float mn = fmaxf(mrow[v], t);
      const float alpha = (mn == -INFINITY) ? 1.0f : exp2f(mrow[v] - mn);
      p[v] = (mn == -INFINITY) ? 0.0f : exp2f(s - mn);
      lpart[v] = lpart[v] * alpha + p[v];
      mrow[v] = mn;
#pragma unroll
      for (int db = 0; db < 4; ++db) O[db][v] *= alpha;
    }
    // ---- P -> LDS [row][key] as bf16, then A fragments (16 keys per k-step)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = 8 * (v >> 2) + 4 * half + (v & 3);
      Ps[i * kPPitch + col] = f2bf(p[v]);
    }
    __syncthreads();
    uint4 pa[2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
      pa[k2] = *reinterpret_cast<const uint4*>(&Ps[col * kPPitch + k2 * 16 + half * 8]);
    // ---- O += P V : B fragment = 8 keys of one dim, contiguous in V^T
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const uint4 vb =
            *reinterpret_cast<const uint4*>(&Vt[(db * 32 + col) * kVPitch + k2 * 16 + half * 8]);
        O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(pa[k2]), as_bf16x8(vb), O[db],
                                                        0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- row sums of p over the 32 key lanes, then write the partials
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float t = row_sum16(lpart[v]);
    t += __shfl_xor(t, 16);
    lpart[v] = t;
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int off = 8 * (v >> 2) + (v & 3);
    if (off >= rem) continue;
    const int r = base_r + off;
    const int u = r / G, h = g * G + r % G;
    const int64_t grow = (int64_t)split * n_rows_tot + (int64_t)u * Hq + h;
#pragma unroll
    for (int db = 0; db < 4; ++db) Opart[grow * kDim + db * 32 + col] = O[db][v];
    if (col == 0) {
      ML[grow * 2] = mrow[v];
      ML[grow * 2 + 1] = lpart[v];
    }
  }
}

__global__ __launch_bounds__(128) void combine_kernel(const float* __restrict__ Opart,
                                                      const float* __restrict__ ML,
                                                      int32_t n_splits, int64_t n_rows,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ out_f32) {
  __shared__ float ms[kMaxSplits], ls[kMaxSplits];
  const int64_t row = blockIdx.x;
  const int d = threadIdx.x;
  for (int s = d; s < n_splits; s += blockDim.x) {
    ms[s] = ML[((int64_t)s * n_rows + row) * 2];
    ls[s] = ML[((int64_t)s * n_rows + row) * 2 + 1];
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int s = 0; s < n_splits; ++s) mx = fmaxf(mx, ms[s]);
  float L = 0.0f, acc = 0.0f;
  if (mx != -INFINITY) {
    for (int s0 = 0; s0 < n_splits; s0 += 8) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int s = s0 + u;
        x[u] = (s < n_splits && ms[s] != -INFINITY) ? Opart[((int64_t)s * n_rows + row) * kDim + d]
                                                    : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int s = s0 + u;
        if (s < n_splits && ms[s] != -INFINITY) {
          const float w = exp2f(ms[s] - mx);
          L += w * ls[s];
          acc += w * x[u];
        }
      }
    }
  }
  const float o = L > 0.0f ? acc / L : 0.0f;
  out[row * kDim + d] = f2bf(o);
  if (out_f32) out_f32[row * kDim + d] = o;
}

struct AttnPlan {
  int32_t row_blocks, key_split, n_splits;
  size_t off_rows, off_nmem, off_qr, off_kr, off_opart, off_ml, total;
};

AttnPlan attn_plan(int32_t M, int32_t M_loc, int32_t Hq, int64_t max_sel) {
  AttnPlan p;
  const int32_t G = Hq / kHeads;
  p.row_blocks = (M * G + kRowTile - 1) / kRowTile;
  const int64_t max_keys = max_sel + M_loc;
  // aim for >= 2048 waves (8 per CU: one tile's loads of each in flight while
  // the others compute), at most kMaxSplits splits
  int64_t want = 2048 / ((int64_t)p.row_blocks * kHeads);
  if (want < 1) want = 1;
  const int64_t tiles = (max_keys + kKeyTile - 1) / kKeyTile;
  int64_t tiles_per_split = (tiles + want - 1) / want;
  if (tiles_per_split < 1) tiles_per_split = 1;
  if ((tiles + tiles_per_split - 1) / tiles_per_split > kMaxSplits)
    tiles_per_split = (tiles + kMaxSplits - 1) / kMaxSplits;
  p.key_split = (int32_t)(tiles_per_split * kKeyTile);
  p.n_splits = (int32_t)((max_keys + p.key_split - 1) / p.key_split);
  if (p.n_splits < 1) p.n_splits = 1;
  // The partials are sized for the most splits any key count up to max_keys
  // can produce: ceil(t / ceil(t / want)) <= want, and <= t, and <= kMaxSplits.
  // (The split count is not monotonic in t, and a workspace sized at the
  // capacity is reused for smaller contexts, e.g. across interleave rounds.)
  int64_t ws_splits = want < kMaxSplits ? want : kMaxSplits;
  if (ws_splits > tiles) ws_splits = tiles;
  if (ws_splits < p.n_splits) ws_splits = p.n_splits;
  size_t o = 0;
  p.off_rows = o; o = align_up(o + sizeof(int32_t) * (size_t)(max_sel > 0 ? max_sel : 1), 256);
  p.off_nmem = o; o = align_up(o + sizeof(int32_t), 256);
  p.off_qr = o; o = align_up(o + 2 * (size_t)M * Hq * kDim, 256);
  p.off_kr = o; o = align_up(o + 2 * (size_t)M_loc * kHeads * kDim, 256);
  p.off_opart = o; o = align_up(o + 4 * (size_t)ws_splits * M * Hq * kDim, 256);
  p.off_ml = o; o = align_up(o + 4 * 2 * (size_t)ws_splits * M * Hq, 256);
  p.total = o;
  return p;
}

}  // namespace

size_t attend_workspace(int32_t M, int32_t M_loc, int32_t n_q_heads, int64_t max_sel_chunks) {
  return attn_plan(M, M_loc, n_q_heads, max_sel_chunks).total;
}

int launch_attend(const AttendArgs& a, void* ws, size_t ws_bytes, hipStream_t s) {
  const AttnPlan p = attn_plan(a.M, a.M_loc, a.n_q_heads, a.max_sel_chunks);
  if (ws_bytes < p.total) return fail(MSA_ERR_WORKSPACE, "attend workspace too small");
  char* base = static_cast<char*>(ws);
  AttnWs w;
  w.mem_rows = reinterpret_cast<int32_t*>(base + p.off_rows);
  w.n_mem = reinterpret_cast<int32_t*>(base + p.off_nmem);
  w.Qr = reinterpret_cast<uint16_t*>(base + p.off_qr);
  w.Kr = reinterpret_cast<uint16_t*>(base + p.off_kr);
  w.Opart = reinterpret_cast<float*>(base + p.off_opart);
  w.ML = reinterpret_cast<float*>(base + p.off_ml);

  PrepArgs pa;
  pa.sel_ids = a.sel_ids; pa.n_sel = a.n_sel; pa.top_k = a.top_k;
  pa.dco = a.dco; pa.n_docs = a.n_docs; pa.n_chunks = a.n_chunks;
  pa.max_sel = a.max_sel_chunks; pa.pos0 = a.pos0;
  pa.Q = a.Q; pa.M = a.M; pa.Hq = a.n_q_heads;
  pa.Kl = a.K_loc; pa.M_loc = a.M_loc; pa.rotate_k = a.k_loc_rotated ? 0 : 1; pa.theta = a.theta;
  pa.mem_rows = w.mem_rows; pa.n_mem = w.n_mem; pa.Qr = w.Qr; pa.Kr = w.Kr;
  const int64_t pairs = (int64_t)a.M * a.n_q_heads * 64 +
                        (pa.rotate_k ? (int64_t)a.M_loc * kHeads * 64 : 0);
  hipLaunchKernelGGL(prep_kernel, dim3((unsigned)(1 + (pairs + 255) / 256)), dim3(256), 0, s, pa);
  MSA_LAUNCH_CHECK("prep_kernel launch");

  const uint16_t* kloc = pa.rotate_k ? w.Kr : a.K_loc;
  const float scale = (float)(1.0 / sqrt((double)kDim)) * kLog2e;
  hipLaunchKernelGGL(attn_kernel, dim3(p.row_blocks, kHeads, p.n_splits), dim3(64), 0, s, w.Qr,
                     a.M, a.n_q_heads, kloc, a.V_loc, a.M_loc, a.Kbar, a.Vbar, w.mem_rows, w.n_mem,
                     p.key_split, scale, w.Opart, w.ML);
  MSA_LAUNCH_CHECK("attn_kernel launch");

  const int64_t n_rows = (int64_t)a.M * a.n_q_heads;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)n_rows), dim3(kDim), 0, s, w.Opart, w.ML,
                     p.n_splits, n_rows, a.out, a.out_f32);
  MSA_LAUNCH_CHECK("combine_kernel launch");
  return MSA_OK;
}

}  // namespace msa
