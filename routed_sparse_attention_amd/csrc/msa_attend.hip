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
// Pipeline (one stream, two launches) for up to 32 query rows per KV head
// (decode; several queries of a batch share the launches):
//   attn      flash attention, one wave per (32 query rows of one KV group,
//             KV head, key split), about 2048 waves. Each wave first builds
//             the chunk list of the selected documents itself (their ranges
//             and a prefix sum in registers, the offsets in LDS; a key's
//             chunk row is a 6-step binary search), issues its first tile's
//             loads, and while they are in flight rotates its own query rows
//             in registers from an LDS table of (cos, sin) per position and
//             frequency. Angles are reduced to [-1/2, 1/2] revolutions in fp64
//             (positions reach 2^20), then take the hardware fp32 cos/sin.
//             Each 32-key tile of K and V is read with one 256-byte row per
//             16 lanes (coalesced; K̄/V̄ in pinned host memory are read in
//             place over PCIe, with no staging copy), at most two K/V row
//             pairs of a wave in flight, and staged in LDS: K row-major, V
//             transposed (a lane holds 8 consecutive keys, so each dim's keys
//             go out as one 16-byte store), so both MFMA B fragments are
//             16-byte LDS reads. Local keys of a single row block are rotated
//             in LDS (lane = frequency; the angle-addition recurrence over the
//             tile's keys). Row maxima and sums use DPP within 16-lane rows and
//             one exchange between rows. S = Q·K^T and O += P·V use
//             v_mfma_f32_32x32x16_bf16; the online softmax runs in fp32 in the
//             exp2 domain; P is re-laid out from the accumulator layout to the
//             A-operand layout through LDS. The workgroup is one wave, so LDS
//             hand-offs need only a compiler barrier;
//   combine   merges the key splits: every split's partial and (m, l) are
//             loaded in one round, weighted by exp2(m_s − max) and summed in
//             split order; writes bf16 (and optionally fp32) output.
#include <cmath>

#include "msa_internal.h"

namespace msa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
// plain vector type for 16-byte moves (a HIP_vector_type copy is a memcpy,
// which can leave the K/V tile registers in scratch)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u32x4 gu32x4;
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kKeyTile = 32;
constexpr int kRowTile = 32;
constexpr int kMaxSplits = 256;
constexpr float kLog2e = 1.4426950408889634f;

// Base-2 exponential of the online softmax: the hardware instruction alone.
// Its arguments are scores minus the running row maximum (<= 0), so a result
// below fp32's normal range (a weight under 2^-126 of the row's largest) is
// flushed to zero instead of being scaled through the denormal range, which
// a bf16 output cannot see.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Keys per split. The launch fixes the number of splits from the largest
// context the call allows (max_sel chunks + the local keys); each workgroup
// cuts the context actually selected into that many runs of whole tiles, so
// a selection far below the capacity still spreads over every split. Every
// workgroup of a query derives the same count from the same chunk list.
__device__ __forceinline__ int split_keys(int n_keys, int n_splits, int tile) {
  const int tiles = (n_keys + tile - 1) / tile;
  return ((tiles + n_splits - 1) / n_splits) * tile;
}

// rotation frequencies omega_m = theta^(-2m/128) (host-made)
struct RopeTab {
  double om[kDim / 2];
};

struct AttnArgs {
  const uint16_t* Q; int32_t M; int32_t Hq;
  const uint16_t* Kloc; const uint16_t* Vloc; int32_t M_loc;
  int32_t rot_inline;             // rotate local keys in the attention waves
  const uint16_t* Kbar; const uint16_t* Vbar; int64_t n_chunks;
  const int64_t* dco; int32_t n_docs;
  const int32_t* sel_ids; const int32_t* n_sel; int32_t top_k;
  int64_t max_sel; int64_t pos0;
  float qk_scale_log2;
  float* Opart; float* ML;
  // queries of a batch: blockIdx.z = query · n_splits + split; per-query
  // element strides of Q, the local keys and values, the partials and the
  // (m, l) pairs (selection: top_k ids and one n_sel per query)
  int32_t n_splits;
  int64_t q_stride, kl_stride, op_stride, ml_stride;
  RopeTab rt;
};

__device__ __forceinline__ int clamp_nsel(const int32_t* n_sel, int top_k) {
  int ns = *n_sel;
  return ns < 0 ? 0 : (ns > top_k ? top_k : ns);
}

// The attention workgroup is one wave: LDS traffic between its lanes is
// ordered by the wave's in-order LDS queue, so a compiler-level barrier
// suffices. (__syncthreads would also wait for every global load in flight,
// which is exactly what the first tile's loads must not do.)
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A pointer field of the by-value argument struct, materialised in scalar
// registers. (Left as struct fields, `mem ? a.Kbar : a.Kloc` becomes a
// per-lane load of the selected field's address: a dependent memory round
// before every K/V load.)
typedef const __attribute__((address_space(1))) uint16_t gbf16;   // global memory
__device__ __forceinline__ gbf16* uniform_ptr(const uint16_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<gbf16*>(((uint64_t)hi << 32) | lo);
}

// (cos, sin) of an fp64 angle: reduced to [-1/2, 1/2] revolutions in fp64,
// then the hardware fp32 cos/sin (which take revolutions). Positions reach
// 2^20 and more, so the reduction must not happen in fp32.
__device__ __forceinline__ float2 cis_hw(double angle) {
  double rev = angle * 0.15915494309189535;   // 1 / (2 pi)
  rev -= rint(rev);
  const float rf = (float)rev;
  return make_float2(__builtin_amdgcn_cosf(rf), __builtin_amdgcn_sinf(rf));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16lo(w[i]);
    f[2 * i + 1] = bf16hi(w[i]);
  }
}

__device__ __forceinline__ uint4 pack8(const float* f) {
  return make_uint4(cvt_pk_bf16(f[0], f[1]), cvt_pk_bf16(f[2], f[3]), cvt_pk_bf16(f[4], f[5]),
                    cvt_pk_bf16(f[6], f[7]));
}

// LDS layout (bytes): K tile [32 keys][136] bf16, V^T tile [128 dims][40] bf16,
// P tile [32 rows][40] bf16. Before the key loop the K and V^T tiles hold
// the query rotation table [position][64 frequencies] of (cos, sin) fp32.
constexpr int kKPitch = 136;
constexpr int kVPitch = 40;
constexpr int kPPitch = 40;
constexpr int kKsBytes = kKeyTile * kKPitch * 2;
constexpr int kVtBytes = kDim * kVPitch * 2;
constexpr int kPsBytes = kRowTile * kPPitch * 2;
static_assert(kRowTile * (kDim / 2) * 8 <= kKsBytes + kVtBytes, "rotation table fits");
constexpr int kMaxSel = 64;   // top_k bound
// s_waitcnt immediate: vmcnt(2), expcnt and lgkmcnt at their maxima (no wait)
// (fields: vmcnt bits 3:0 and 15:14, expcnt bits 6:4, lgkmcnt bits 11:8)
constexpr int kWaitVm2 = 2 | (7 << 4) | (15 << 8);

// HOST_KV: K̄/V̄ are read from pinned host memory over PCIe. Those reads are
// throttled (below) and the kernel keeps its full register budget; with
// device memory the loads are not throttled and the kernel is held to two
// waves per SIMD (measured: a 128-token query over 2K selected chunks 85 ->
// 60 us; decode unchanged).
template <bool HOST_KV>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(HOST_KV ? 1 : 2)))
void attn_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kKsBytes + kVtBytes + kPsBytes];
  __shared__ int32_t s_off[kMaxSel];
  __shared__ int64_t s_start[kMaxSel];
  __shared__ int32_t s_rows[kKeyTile];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(lds);
  uint16_t* Vt = reinterpret_cast<uint16_t*>(lds + kKsBytes);
  uint16_t* Ps = reinterpret_cast<uint16_t*>(lds + kKsBytes + kVtBytes);
  float2* trig = reinterpret_cast<float2*>(lds);

  const int lane = threadIdx.x;
  const int col = lane & 31;      // MFMA column lane (key / dim)
  const int half = lane >> 5;     // which 8-wide k slice this lane holds
  const int rb = blockIdx.x;      // row block within the KV group
  const int g = blockIdx.y;       // KV head
  const int qb = blockIdx.z / a.n_splits;          // query of the batch
  const int split = blockIdx.z - qb * a.n_splits;
  const int G = a.Hq / kHeads;    // query heads per KV head
  const int rows_g = a.M * G;
  const int64_t n_rows_tot = (int64_t)a.M * a.Hq;
  // this query's rows, local context, selection and partials (uniform)
  const uint16_t* Qq = a.Q + qb * a.q_stride;
  const int32_t* sel_ids = a.sel_ids + (int64_t)qb * a.top_k;
  const int32_t* n_sel = a.n_sel + qb;
  float* Opart = a.Opart + qb * a.op_stride;
  float* MLq = a.ML + qb * a.ml_stride;
  gbf16* Kbar = uniform_ptr(a.Kbar);
  gbf16* Vbar = uniform_ptr(a.Vbar);
  gbf16* Kloc = uniform_ptr(a.Kloc + qb * a.kl_stride);
  gbf16* Vloc = uniform_ptr(a.Vloc + qb * a.kl_stride);

  // the query rows are loaded first: their loads overlap the chunk-list ones
  uint4 qa[8];
  const int r = rb * kRowTile + col;
  if (r < rows_g) {
    const int u = r / G, h = g * G + r % G;
    const uint4* qrow = reinterpret_cast<const uint4*>(Qq + ((int64_t)u * a.Hq + h) * kDim);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qa[ks] = qrow[ks * 2 + half];
  } else {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qa[ks] = make_uint4(0, 0, 0, 0);
  }

  // this lane's rotation frequency (lane = m below), loaded in the first round
  const double om = a.rt.om[lane];

  // ---- chunk ranges of the selected documents, in rank order: lane i holds
  //      document i's range; a key's place in the memory part is the prefix
  //      sum of the ranges before it, cut at max_sel
  const int32_t id = lane < a.top_k ? sel_ids[lane] : -1;   // loaded with n_sel
  const int ns = clamp_nsel(n_sel, a.top_k);
  int64_t start = 0, cnt = 0;
  if (lane < ns) {
    if (id >= 0 && id < a.n_docs) {
      int64_t c0 = a.dco[id], c1 = a.dco[id + 1];
      c0 = max((int64_t)0, min(c0, a.n_chunks));
      c1 = max(c0, min(c1, a.n_chunks));
      start = c0;
      cnt = c1 - c0;
    }
  }
  int64_t incl = cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  const int64_t total = __shfl(incl, 63);
  const int n_mem = (int)min(total, a.max_sel);
  if (lane < ns) {
    s_off[lane] = (int)min(incl - cnt, a.max_sel);
    s_start[lane] = start;
  }
  const int n_keys = n_mem + a.M_loc;
  const int key_split = split_keys(n_keys, a.n_splits, kKeyTile);
  const int k_begin = split * key_split;
  const int k_end = min(k_begin + key_split, n_keys);
  const int64_t pos0 = a.pos0 < 0 ? (int64_t)ns : a.pos0;

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
  // (cos, sin) table at the block's query positions, lane = frequency m; it
  // sits where the K / V^T tiles go
  const int u_first = rb * kRowTile / G;
  if (k_begin < k_end) {
    const int r_last = min(rb * kRowTile + kRowTile, rows_g) - 1;
    const int n_pos = r_last / G - u_first + 1;
    const int64_t p_first = pos0 + (a.M_loc - a.M) + u_first;
    for (int i = 0; i < n_pos; ++i) trig[i * 64 + lane] = cis_hw((double)(p_first + i) * om);
  }
  // the chunk offsets and the table are read below by other lanes
  wave_sync();
  for (int kt = k_begin; kt < k_end; kt += kKeyTile) {
    // ---- K and V rows of the tile. Keys past the split are clamped to its
    //      last key (a real row, so finite) and masked out of the softmax
    //      below. A memory key's chunk row is found by binary search: the
    //      last document whose offset is <= j (offsets are non-decreasing; an
    //      empty range is skipped because the next offset equals its own).
    if (kt < n_mem) {
      if (lane < kKeyTile) {
        const int j = kt + lane;
        int row = 0;
        if (j < n_mem) {
          int d = 0;
#pragma unroll
          for (int step = kMaxSel / 2; step > 0; step >>= 1) {
            const int t = d + step;
            if (t < ns && s_off[t] <= j) d = t;
          }
          row = (int)(s_start[d] + (j - s_off[d]));
        }
        s_rows[lane] = row;
      }
      wave_sync();
    }
    // (the 8 row reads go out before any load; a local key's read is unused)
    int crow[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) crow[it] = s_rows[min(kt + sub * 8 + it, k_end - 1) - kt];
    u32x4 kx[8], vx[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int j = min(kt + sub * 8 + it, k_end - 1);
      const bool mem = j < n_mem;
      const int64_t off = mem ? ((int64_t)crow[it] * kHeads + g) * kDim
                              : ((int64_t)(j - n_mem) * kHeads + g) * kDim;
      kx[it] = reinterpret_cast<gu32x4*>((mem ? Kbar : Kloc) + off)[dv];
      vx[it] = reinterpret_cast<gu32x4*>((mem ? Vbar : Vloc) + off)[dv];
      // host K̄/V̄: at most two K/V pairs of a wave in flight. With all
      // sixteen issued at once by every wave, reads of pinned host memory
      // over PCIe measured slower (decode, 16 documents: 63.5 vs 58.0 us per
      // call); from device memory all sixteen go out at once (256 query
      // tokens over 2K chunks: 146 -> 132 us per call)
      if (HOST_KV) __builtin_amdgcn_s_waitcnt(kWaitVm2);
    }

    // ---- first tile: the A fragments of this lane's query row (row =
    //      lane % 32 of the block) are rotated to the row's global position
    //      while the tile's loads are in flight. A lane holds dims
    //      16·ks + 8·half + e; the rotation pairs (m, m + 64) are ks and
    //      ks + 4 of the same lane.
    if (kt == k_begin) {
      if (r < rows_g) {
        const float4* tr = reinterpret_cast<const float4*>(trig + (r / G - u_first) * 64);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          float x[8], y[8], cs8[8], sn8[8];
          unpack8(qa[ks], x);
          unpack8(qa[ks + 4], y);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 t = tr[(16 * ks + 8 * half) / 2 + q];
            cs8[2 * q] = t.x; sn8[2 * q] = t.y;
            cs8[2 * q + 1] = t.z; sn8[2 * q + 1] = t.w;
          }
          float xo[8], yo[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            xo[e] = x[e] * cs8[e] - y[e] * sn8[e];
            yo[e] = y[e] * cs8[e] + x[e] * sn8[e];
          }
          qa[ks] = pack8(xo);
          qa[ks + 4] = pack8(yo);
        }
      }
      wave_sync();   // the table's LDS becomes the K / V^T tiles
    }

#pragma unroll
    for (int it = 0; it < 8; ++it)
      *reinterpret_cast<u32x4*>(&Ks[(sub * 8 + it) * kKPitch + dv * 8]) = kx[it];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // dim dv·8 + e of keys 8·sub .. 8·sub + 7
      u32x4 w;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t wa = vx[2 * q][e >> 1];
        const uint32_t wb = vx[2 * q + 1][e >> 1];
        w[q] = (e & 1) ? ((wa >> 16) | (wb & 0xffff0000u)) : ((wa & 0xffffu) | (wb << 16));
      }
      *reinterpret_cast<u32x4*>(&Vt[(dv * 8 + e) * kVPitch + sub * 8]) = w;
    }
    wave_sync();
    // ---- local keys of this tile at pos0 + v, rotated in LDS: lane = m;
    //      (cos, sin) at the first local key, then the angle-addition
    //      recurrence over the tile's keys (fp32, at most 31 steps)
    if (a.rot_inline && kt + kKeyTile > n_mem) {
      const int t0 = max(0, n_mem - kt);
      const int m = lane;
      float2 cs = cis_hw((double)(pos0 + (kt + t0 - n_mem)) * om);
      const float2 step = cis_hw(om);
      // groups of 8 keys: the group's 16 LDS reads go out together
      for (int tg = t0 & ~7; tg < kKeyTile; tg += 8) {
        uint16_t xr[8], yr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          xr[i] = Ks[(tg + i) * kKPitch + m];
          yr[i] = Ks[(tg + i) * kKPitch + m + 64];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (tg + i < t0) continue;
          const float x = bf16f(xr[i]), y = bf16f(yr[i]);
          Ks[(tg + i) * kKPitch + m] = f2bf(x * cs.x - y * cs.y);
          Ks[(tg + i) * kKPitch + m + 64] = f2bf(y * cs.x + x * cs.y);
          cs = make_float2(cs.x * step.x - cs.y * step.y, cs.y * step.x + cs.x * step.y);
        }
      }
      wave_sync();
    }

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
    const int lim_off = j < n_mem ? -(1 << 30) : (j - n_mem - (a.M_loc - a.M)) * G - base_r;
    float p[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int off = 8 * (v >> 2) + (v & 3);
      const bool ok = key_ok && off < rem && off >= lim_off;
      const float sv = ok ? S[v] * a.qk_scale_log2 : -INFINITY;
      // max over the row's 32 key lanes: four DPP steps within each 16-lane
      // row, then one exchange between the two rows of this half
      float t = sv;
      t = fmaxf(t, dpp_f<0xB1>(t));    // quad_perm [1,0,3,2]
      t = fmaxf(t, dpp_f<0x4E>(t));    // quad_perm [2,3,0,1]
      t = fmaxf(t, dpp_f<0x141>(t));   // row_half_mirror
      t = fmaxf(t, dpp_f<0x140>(t));   // row_mirror
      t = fmaxf(t, __shfl_xor(t, 16));
      const float mn = fmaxf(mrow[v], t);
      const float alpha = (mn == -INFINITY) ? 1.0f : exp2_hw(mrow[v] - mn);
      p[v] = (mn == -INFINITY) ? 0.0f : exp2_hw(sv - mn);
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
    wave_sync();
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
    wave_sync();
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
    const int64_t grow = (int64_t)split * n_rows_tot + (int64_t)u * a.Hq + h;
#pragma unroll
    for (int db = 0; db < 4; ++db) Opart[grow * kDim + db * 32 + col] = O[db][v];
    if (col == 0) {
      MLq[grow * 2] = mrow[v];
      MLq[grow * 2 + 1] = lpart[v];
    }
  }
}

// One workgroup per output row, a thread per dim. Every split's (m, l) and
// partial are loaded in one round (a split with no keys has m = -inf and a
// zero partial, so its weight exp2(-inf - max) = 0 drops it); the sum runs
// in split order.
constexpr int kCombineBatch = 64;
__global__ __launch_bounds__(128) void combine_kernel(const float* __restrict__ Opart_all,
                                                      const float* __restrict__ ML_all,
                                                      int32_t n_splits, int64_t n_rows,
                                                      int64_t op_stride, int64_t ml_stride,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ out_f32) {
  // one workgroup per output row of a batch of queries (n_rows each); query
  // qb's partials at qb·op_stride / qb·ml_stride, its rows after the
  // previous queries'
  __shared__ float ms[kMaxSplits], ls[kMaxSplits];
  const int64_t row_all = blockIdx.x;
  const int64_t qb = row_all / n_rows;
  const int64_t row = row_all - qb * n_rows;
  const float* Opart = Opart_all + qb * op_stride;
  const float* ML = ML_all + qb * ml_stride;
  const int d = threadIdx.x;
  float x[kCombineBatch];
#pragma unroll
  for (int u = 0; u < kCombineBatch; ++u)
    if (u < n_splits) x[u] = Opart[((int64_t)u * n_rows + row) * kDim + d];
  for (int s = d; s < n_splits; s += blockDim.x) {
    ms[s] = ML[((int64_t)s * n_rows + row) * 2];
    ls[s] = ML[((int64_t)s * n_rows + row) * 2 + 1];
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int s = 0; s < n_splits; ++s) mx = fmaxf(mx, ms[s]);
  float L = 0.0f, acc = 0.0f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      if (u < n_splits) {
        const float w = exp2f(ms[u] - mx);
        L += w * ls[u];
        acc += w * x[u];
      }
    }
    for (int s = kCombineBatch; s < n_splits; ++s) {
      const float w = exp2f(ms[s] - mx);
      L += w * ls[s];
      acc += w * Opart[((int64_t)s * n_rows + row) * kDim + d];
    }
  }
  const float o = L > 0.0f ? acc / L : 0.0f;
  out[row_all * kDim + d] = f2bf(o);
  if (out_f32) out_f32[row_all * kDim + d] = o;
}

// ---------------------------------------------------------------------------
// Multi-token queries (more than 32 query rows per KV head): one workgroup of
// four waves per (128 query rows of one KV group, KV head, key split). The
// waves share each 64-key tile of K and V, staged in LDS in two buffers (the
// next tile's loads are in flight while the current one is multiplied), so a
// tile is read from memory once per 128 rows instead of once per 32.
//
// Each wave computes S^T = K · Q^T for its 32 rows: the accumulator of
// v_mfma_f32_32x32x16_bf16 then puts one query row in each lane (32 lanes ×
// 2 halves), so the row maximum and sum need no cross-lane reduction beyond
// one exchange between the halves, and the softmax weights P^T are already
// the B operand of O^T += V^T · P^T. For that, the sixteen weights a lane
// holds for a 32-key block must be keys 16s + 8·half + 0..7 (s = 0, 1), so K
// is stored in LDS with bits 2 and 3 of each key's row swapped; V^T keeps
// the natural key order and is written with one 16-byte store per dim and 8
// keys. O^T keeps one row per lane, so the online-softmax rescale is
// lane-local, and it is skipped when no row maximum moved.
//
// Q arrives rotated and pre-scaled by log2(e)/sqrt(128) and the local keys
// rotated (rot_qk_kernel), so the tile loop has no trigonometry. Each
// workgroup writes its split's partial (O, m, l per row); combine_rows_kernel
// merges the splits. (Merging in the last workgroup to finish would need a
// device-scope release per workgroup, which on this chip writes back the
// whole L2 of the workgroup's XCD: measured 3× slower than the extra pass.)
// ---------------------------------------------------------------------------
constexpr int kMtWaves = 4;
constexpr int kMtThreads = 64 * kMtWaves;
constexpr int kMtRows = 32 * kMtWaves;          // query rows per workgroup
constexpr int kMtKeys = 64;                     // keys per tile
constexpr int kMtKPitch = 136;                  // bf16 per K row in LDS
constexpr int kMtVPitch = 72;                   // bf16 per V^T row in LDS
constexpr int kMtKElems = kMtKeys * kMtKPitch;
constexpr int kMtVElems = kDim * kMtVPitch;
constexpr int kMtBufElems = kMtKElems + kMtVElems;

struct MtArgs {
  const uint16_t* Qr; int32_t M; int32_t Hq;     // rotated, pre-scaled queries [M, Hq, 128]
  const uint16_t* Kr; const uint16_t* Vloc; int32_t M_loc;   // rotated local keys
  const uint16_t* Kbar; const uint16_t* Vbar; int64_t n_chunks;
  const int64_t* dco; int32_t n_docs;
  const int32_t* sel_ids; const int32_t* n_sel; int32_t top_k;
  int64_t max_sel;
  uint16_t* Opart; float* ML;     // per split: O / l in bf16, and (m, l)
  // queries of a batch: blockIdx.z = query · n_splits + split; per-query
  // element strides of Qr, Kr, Vloc, the partials and the (m, l) pairs
  int32_t n_splits;
  int64_t qr_stride, kr_stride, v_stride, op_stride, ml_stride;
};

// Rotates the query rows (at pos0 + M_loc - M + u, then scaled by qscale) and,
// when Kr != nullptr, the local keys (at pos0 + v) into the workspace. One
// wave per (token, group of 8 heads), lane m = rotation pair (m, m + 64): the
// angle depends on the token's position and m only, so a wave forms its
// (cos, sin) once — the angle reduced to [-1/2, 1/2] revolutions in fp64,
// hardware fp32 cos/sin — and applies it to its 8 heads (each head's two
// loads are one 128-byte run per wave); bf16 results.
constexpr int kRotHeads = 8;
__global__ __launch_bounds__(256) void rot_qk_kernel(const uint16_t* __restrict__ Q, int32_t M,
                                                     int32_t Hq, const uint16_t* __restrict__ Kl,
                                                     int32_t M_loc, const int32_t* __restrict__ n_sel,
                                                     int32_t top_k, int64_t pos0_arg, RopeTab rt,
                                                     float qscale, uint16_t* __restrict__ Qr,
                                                     uint16_t* __restrict__ Kr, int32_t nb,
                                                     int64_t q_stride, int64_t kl_stride) {
  // nb queries: query b's Q at Q + b·q_stride, its local keys at
  // Kl + b·kl_stride, its n_sel at n_sel[b]; outputs packed per query.
  // Units: per query, M tokens × Hq / 8 query head groups, then (with Kr)
  // M_loc tokens of 8 KV heads.
  const int64_t unit = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int m = threadIdx.x & 63;
  const int n_qg = Hq / kRotHeads;
  const int64_t nq = (int64_t)M * n_qg;
  const int64_t nk = Kr ? (int64_t)M_loc : 0;
  if (unit >= (nq + nk) * nb) return;
  const uint16_t* src;
  uint16_t* dst;
  int64_t row0, pos;
  int b;
  float sc = 1.0f;
  const bool is_q = unit < nq * nb;
  if (is_q) {
    b = (int)(unit / nq);
    const int64_t j = unit - (int64_t)b * nq;
    const int64_t tok = j / n_qg;
    row0 = tok * Hq + (j % n_qg) * kRotHeads;      // first of the group's rows
    src = Q + b * q_stride;
    dst = Qr + (int64_t)b * M * Hq * kDim;
    sc = qscale;
    pos = (M_loc - M) + tok;
  } else {
    const int64_t j0 = unit - nq * nb;
    b = (int)(j0 / nk);
    const int64_t tok = j0 - (int64_t)b * nk;
    row0 = tok * kHeads;
    src = Kl + b * kl_stride;
    dst = Kr + (int64_t)b * M_loc * kHeads * kDim;
    pos = tok;
  }
  pos += pos0_arg < 0 ? (int64_t)clamp_nsel(n_sel + b, top_k) : pos0_arg;
  const float2 cs = cis_hw((double)pos * rt.om[m]);
  float x[kRotHeads], y[kRotHeads];
#pragma unroll
  for (int h = 0; h < kRotHeads; ++h) {
    x[h] = bf16f(src[(row0 + h) * kDim + m]);
    y[h] = bf16f(src[(row0 + h) * kDim + m + 64]);
  }
#pragma unroll
  for (int h = 0; h < kRotHeads; ++h) {
    dst[(row0 + h) * kDim + m] = f2bf((x[h] * cs.x - y[h] * cs.y) * sc);
    dst[(row0 + h) * kDim + m + 64] = f2bf((y[h] * cs.x + x[h] * cs.y) * sc);
  }
}

// LDS row of key q (0..63) of a tile in the K buffer: bits 2 and 3 swapped.
__device__ __forceinline__ int k_row(int q) {
  return (q & ~12) | ((q & 4) << 1) | ((q & 8) >> 1);
}

template <bool HOST_KV>
__global__ __launch_bounds__(kMtThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attn_mt_kernel(const MtArgs args) {
  // this workgroup's query of the batch: its own rows, local keys, selection
  // and partials (uniform pointer arithmetic)
  const int qb = blockIdx.z / args.n_splits;
  MtArgs a = args;
  a.Qr += qb * args.qr_stride;
  a.Kr += qb * args.kr_stride;
  a.Vloc += qb * args.v_stride;
  a.sel_ids += (int64_t)qb * args.top_k;
  a.n_sel += qb;
  a.Opart += qb * args.op_stride;
  a.ML += qb * args.ml_stride;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kMtBufElems];
  __shared__ int32_t s_off[kMaxSel];
  __shared__ int64_t s_start[kMaxSel];
  __shared__ int32_t s_rows[2][kMtKeys];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int rg = blockIdx.x;
  const int g = blockIdx.y;
  const int split = blockIdx.z - qb * args.n_splits;
  const int G = a.Hq / kHeads;
  const int rows_g = a.M * G;
  const int64_t n_rows_tot = (int64_t)a.M * a.Hq;
  gbf16* Kbar = uniform_ptr(a.Kbar);
  gbf16* Vbar = uniform_ptr(a.Vbar);
  gbf16* Kloc = uniform_ptr(a.Kr);
  gbf16* Vloc = uniform_ptr(a.Vloc);

  // ---- this lane's query row (B operand of S^T = K Q^T): dims 16ks + 8·half
  const int r = rg * kMtRows + wave * 32 + col;
  const bool row_ok = r < rows_g;
  const int u = row_ok ? r / G : 0;
  const int hq = g * G + (row_ok ? r % G : 0);
  uint4 qa[8];
  {
    const uint4* qrow = reinterpret_cast<const uint4*>(a.Qr + ((int64_t)u * a.Hq + hq) * kDim);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qa[ks] = row_ok ? qrow[ks * 2 + half] : make_uint4(0, 0, 0, 0);
  }

  // ---- chunk ranges of the selected documents in rank order (every wave
  //      computes the prefix sum; wave 0 keeps it in LDS)
  const int32_t id = lane < a.top_k ? a.sel_ids[lane] : -1;
  const int ns = clamp_nsel(a.n_sel, a.top_k);
  int64_t start = 0, cnt = 0;
  if (lane < ns && id >= 0 && id < a.n_docs) {
    int64_t c0 = a.dco[id], c1 = a.dco[id + 1];
    c0 = max((int64_t)0, min(c0, a.n_chunks));
    c1 = max(c0, min(c1, a.n_chunks));
    start = c0;
    cnt = c1 - c0;
  }
  int64_t incl = cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  const int64_t total = __shfl(incl, 63);
  const int n_mem = (int)min(total, a.max_sel);
  if (wave == 0 && lane < ns) {
    s_off[lane] = (int)min(incl - cnt, a.max_sel);
    s_start[lane] = start;
  }

  // ---- keys of this split, cut where the workgroup's last token stops
  //      seeing local keys (causal)
  const int n_keys = n_mem + a.M_loc;
  const int key_split = split_keys(n_keys, a.n_splits, kMtKeys);
  const int k_begin = split * key_split;
  const int r_last = min(rows_g, (rg + 1) * kMtRows) - 1;
  const int u_first = min(rg * kMtRows, rows_g - 1) / G;
  const int lim_wg_hi = n_mem + (a.M_loc - a.M) + r_last / G;    // last key any row sees
  const int lim_wg_lo = n_mem + (a.M_loc - a.M) + u_first;       // last key every row sees
  const int k_end = min(min(k_begin + key_split, n_keys), lim_wg_hi + 1);
  const int n_tiles = k_end > k_begin ? (k_end - k_begin + kMtKeys - 1) / kMtKeys : 0;
  const int lim_row = n_mem + (a.M_loc - a.M) + u;               // last key this row sees

  // key j of the context -> chunk row (>= 0) or -(v + 1) for local key v
  auto key_row = [&](int j) -> int {
    if (j < n_mem) {
      int d = 0;
#pragma unroll
      for (int step = kMaxSel / 2; step > 0; step >>= 1) {
        const int t = d + step;
        if (t < ns && s_off[t] <= j) d = t;
      }
      return (int)(s_start[d] + (j - s_off[d]));
    }
    return -(j - n_mem + 1);
  };

  // Loads of one tile: waves 0-1 read V as 8 consecutive keys × one 16-byte
  // vector (lane (c, dv) = (t % 8, t / 8): keys 8c .. 8c + 7, vector dv), so
  // each dim's 8 keys leave as one 16-byte V^T store; waves 2-3 read K rows
  // (lane (q0, dv) = (t / 16, t % 16): keys q0 + 8i, vector dv). Either way
  // each load instruction covers whole 128- or 256-byte runs of rows.
  const bool is_v = wave < 2;
  const int tt = tid & 127;
  const int vc = tt & 7, vdv = tt >> 3;
  const int kq0 = tt >> 4, kdv = tt & 15;
  // this wave's two sources (pooled memory, local context) and lane vector
  gbf16* const src_mem = is_v ? Vbar : Kbar;
  gbf16* const src_loc = is_v ? Vloc : Kloc;
  const int my_dv = is_v ? vdv : kdv;
  const int q_base = is_v ? 8 * vc : kq0;
  const int q_step = is_v ? 1 : 8;
  u32x4 xv[8];
  auto load_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rk = s_rows[buf][q_base + q_step * i];
      const bool mem = rk >= 0;
      const int64_t off = ((int64_t)(mem ? rk : -rk - 1) * kHeads + g) * kDim + my_dv * 8;
      xv[i] = *reinterpret_cast<gu32x4*>((mem ? src_mem : src_loc) + off);
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* Ks = lds + buf * kMtBufElems;
    uint16_t* Vt = Ks + kMtKElems;
    if (is_v) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // dim vdv·8 + e of keys 8vc .. 8vc + 7
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t wa = xv[2 * q][e >> 1];
          const uint32_t wb = xv[2 * q + 1][e >> 1];
          w[q] = (e & 1) ? ((wa >> 16) | (wb & 0xffff0000u)) : ((wa & 0xffffu) | (wb << 16));
        }
        *reinterpret_cast<u32x4*>(&Vt[(vdv * 8 + e) * kMtVPitch + 8 * vc]) = w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<u32x4*>(&Ks[k_row(kq0 + 8 * i) * kMtKPitch + kdv * 8]) = xv[i];
    }
  };
  auto rows_of = [&](int buf, int t) {
    if (tid < kMtKeys) s_rows[buf][tid] = key_row(min(k_begin + t * kMtKeys + tid, k_end - 1));
  };

  f32x16_t O[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) O[db][v] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  __syncthreads();   // chunk list in LDS
  if (n_tiles > 0) rows_of(0, 0);
  __syncthreads();
  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
    if (n_tiles > 1) rows_of(1, 1);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int b = t & 1;
    if (t + 1 < n_tiles) load_tile(b ^ 1);
    const uint16_t* Ks = lds + b * kMtBufElems;
    const uint16_t* Vt = Ks + kMtKElems;
    const int tile0 = k_begin + t * kMtKeys;

    // ---- S^T = K Q^T for the tile's two 32-key blocks (log2 domain: Q
    //      carries the scale)
    f32x16_t S[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) S[kb][v] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const uint4 ka =
            *reinterpret_cast<const uint4*>(&Ks[(kb * 32 + col) * kMtKPitch + ks * 16 + half * 8]);
        S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka), as_bf16x8(qa[ks]), S[kb],
                                                         0, 0, 0);
      }
    }

    // ---- mask (only tiles that reach past the split's end or into keys
    //      some row must not see); register v of block kb holds key
    //      32kb + 16(v / 8) + 8·half + v % 8
    const bool full = tile0 + kMtKeys <= k_end && tile0 + kMtKeys - 1 <= lim_wg_lo;
    if (!full) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = tile0 + kb * 32 + 16 * (v >> 3) + 8 * half + (v & 7);
          const bool ok = j < k_end && (j < n_mem || j <= lim_row);
          S[kb][v] = ok ? S[kb][v] : -INFINITY;
        }
    }
    float mx = S[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, S[kb][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const bool live = m_new != -INFINITY;
    // rescale only when some row's maximum moved (the common case after the
    // first tiles is that none did)
    if (__any(m_new != m_run)) {
      const float alpha = live ? exp2_hw(m_run - m_new) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) O[db][v] *= alpha;
    }
    m_run = m_new;
    // a row with every key so far masked has m = -inf and S = -inf: its
    // weights are exp2(-inf - 0) = 0
    const float m_use = live ? m_new : 0.0f;
    float psum = 0.0f;
    uint4 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int sg = 0; sg < 2; ++sg) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = exp2_hw(S[kb][8 * sg + e] - m_use);
          psum += p[e];
        }
        pb[kb][sg] = pack8(p);
      }
    l_run += psum;

    // ---- O^T += V^T P^T: k-step (kb, sg) covers keys 32kb + 16sg + 8·half + 0..7
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) {
          const uint4 va = *reinterpret_cast<const uint4*>(
              &Vt[(db * 32 + col) * kMtVPitch + kb * 32 + sg * 16 + half * 8]);
          O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), as_bf16x8(pb[kb][sg]),
                                                          O[db], 0, 0, 0);
        }

    if (t + 1 < n_tiles) {
      store_tile(b ^ 1);
      if (t + 2 < n_tiles) rows_of(b, t + 2);
    }
    __syncthreads();
  }

  // ---- this split's partial: lane (row, half) holds dims 32db + 8a + 4·half + 0..3.
  //      The partial is stored normalised, O / l, in bf16 (half the bytes of
  //      fp32 for the merge to move); (m, l) stay fp32.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (row_ok) {
    const int64_t grow = (int64_t)split * n_rows_tot + (int64_t)u * a.Hq + hq;
    uint16_t* dst = a.Opart + grow * kDim;
    const float inv_l = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<uint2*>(dst + db * 32 + 8 * q + 4 * half) =
            make_uint2(cvt_pk_bf16(O[db][4 * q] * inv_l, O[db][4 * q + 1] * inv_l),
                       cvt_pk_bf16(O[db][4 * q + 2] * inv_l, O[db][4 * q + 3] * inv_l));
    if (half == 0) {
      a.ML[grow * 2] = m_run;
      a.ML[grow * 2 + 1] = l_tot;
    }
  }
}

// Merges the key splits of the multi-token kernel: 32 threads per output
// row, 4 dims each (8-byte loads of the bf16 partials O_s / l_s); the
// partials are weighted by exp2(m_s - max) · l_s and summed in split order.
// The (m, l) pairs and partials of the first kCombRegs splits are loaded
// together, before the maximum is known, so the merge waits for one memory
// round trip instead of two; later splits (more than the multi-token plan
// makes at its usual shapes) are read in a second loop.
constexpr int kCombRows = 8;
constexpr int kCombRegs = 8;
__global__ __launch_bounds__(256) void combine_rows_kernel(const uint16_t* __restrict__ Opart_all,
                                                           const float* __restrict__ ML_all,
                                                           int32_t n_splits, int64_t n_rows,
                                                           int32_t nb, int64_t op_stride,
                                                           int64_t ml_stride,
                                                           uint16_t* __restrict__ out_all,
                                                           float* __restrict__ out_f32_all) {
  // nb queries of n_rows rows each; query b's partials at b·op_stride /
  // b·ml_stride, its output rows after the previous queries'
  const int64_t grow_all = (int64_t)blockIdx.x * kCombRows + (threadIdx.x >> 5);
  if (grow_all >= n_rows * nb) return;
  const int64_t qb = grow_all / n_rows;
  const int64_t row = grow_all - qb * n_rows;
  const uint16_t* Opart = Opart_all + qb * op_stride;
  const float* ML = ML_all + qb * ml_stride;
  uint16_t* out = out_all + qb * n_rows * kDim;
  float* out_f32 = out_f32_all ? out_f32_all + qb * n_rows * kDim : nullptr;
  const int d = (threadIdx.x & 31) * 4;
  float2 ml[kCombRegs];
  uint2 xs[kCombRegs];
#pragma unroll
  for (int s = 0; s < kCombRegs; ++s) {
    if (s < n_splits) {
      const int64_t gr = (int64_t)s * n_rows + row;
      ml[s] = *reinterpret_cast<const float2*>(ML + gr * 2);
      xs[s] = *reinterpret_cast<const uint2*>(Opart + gr * kDim + d);
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < kCombRegs; ++s)
    if (s < n_splits) mx = fmaxf(mx, ml[s].x);
  for (int s = kCombRegs; s < n_splits; ++s) mx = fmaxf(mx, ML[((int64_t)s * n_rows + row) * 2]);
  float L = 0.0f;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  auto add = [&](float m, float l, uint2 x) {
    const float w = exp2f(m - mx) * l;
    L += w;
    acc.x += w * bf16lo(x.x);
    acc.y += w * bf16hi(x.x);
    acc.z += w * bf16lo(x.y);
    acc.w += w * bf16hi(x.y);
  };
  if (mx != -INFINITY) {
#pragma unroll
    for (int s = 0; s < kCombRegs; ++s)
      if (s < n_splits) add(ml[s].x, ml[s].y, xs[s]);
    for (int s = kCombRegs; s < n_splits; ++s) {
      const int64_t gr = (int64_t)s * n_rows + row;
      add(ML[gr * 2], ML[gr * 2 + 1], *reinterpret_cast<const uint2*>(Opart + gr * kDim + d));
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const float o[4] = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
  *reinterpret_cast<uint2*>(out + row * kDim + d) =
      make_uint2(pack2(f2bf(o[0]), f2bf(o[1])), pack2(f2bf(o[2]), f2bf(o[3])));
  if (out_f32) *reinterpret_cast<float4*>(out_f32 + row * kDim + d) = make_float4(o[0], o[1], o[2], o[3]);
}

struct AttnPlan {
  bool multi;                 // the multi-token kernel (more than 32 rows per KV head)
  int32_t row_blocks, key_split, n_splits;
  size_t off_kr, off_qr, off_opart, off_ml, total;
  int64_t kr_q, qr_q, op_q, ml_q;   // per-query elements of each workspace part
};

// The split plan is that of one query whatever nb is (so each query of a
// batch computes exactly what it would alone); the workspace holds nb
// queries' rotated rows and partials.
AttnPlan attn_plan(int32_t M, int32_t M_loc, int32_t Hq, int64_t max_sel, int32_t nb = 1) {
  AttnPlan p;
  const int32_t G = Hq / kHeads;
  const int32_t rows_g = M * G;
  p.multi = rows_g > kRowTile;
  const int32_t block_rows = p.multi ? kMtRows : kRowTile;
  const int32_t tile_keys = p.multi ? kMtKeys : kKeyTile;
  // (the one-wave kernel serves up to 32 rows per KV head: one row block,
  // so each local key is read, and rotated, by one wave per KV head)
  p.row_blocks = (rows_g + block_rows - 1) / block_rows;
  const int64_t max_keys = max_sel + M_loc;
  // one-wave kernel: aim for >= 2048 waves (8 per CU: one tile's loads of
  // each in flight while the others compute); multi-token kernel: about one
  // four-wave workgroup per CU (256 tokens: 4 splits; 2 per CU measured
  // slower, more split partials for no more overlap). At most kMaxSplits
  // splits either way.
  const int64_t target = p.multi ? 256 : 2048;
  int64_t want = target / ((int64_t)p.row_blocks * kHeads);
  if (want < 1) want = 1;
  const int64_t tiles = (max_keys + tile_keys - 1) / tile_keys;
  int64_t tiles_per_split = (tiles + want - 1) / want;
  if (tiles_per_split < 1) tiles_per_split = 1;
  if ((tiles + tiles_per_split - 1) / tiles_per_split > kMaxSplits)
    tiles_per_split = (tiles + kMaxSplits - 1) / kMaxSplits;
  p.key_split = (int32_t)(tiles_per_split * tile_keys);
  p.n_splits = (int32_t)((max_keys + p.key_split - 1) / p.key_split);
  if (p.n_splits < 1) p.n_splits = 1;
  // The partials are sized for the most splits any key count up to max_keys
  // can produce: ceil(t / ceil(t / want)) <= want, and <= t, and <= kMaxSplits.
  // (The split count is not monotonic in t, and a workspace sized at the
  // capacity is reused for smaller contexts, e.g. across interleave rounds.)
  int64_t ws_splits = want < kMaxSplits ? want : kMaxSplits;
  if (ws_splits > tiles) ws_splits = tiles;
  if (ws_splits < p.n_splits) ws_splits = p.n_splits;
  p.kr_q = (int64_t)M_loc * kHeads * kDim;
  p.qr_q = p.multi ? (int64_t)M * Hq * kDim : 0;
  p.op_q = ws_splits * M * Hq * kDim;
  p.ml_q = 2 * ws_splits * M * Hq;
  size_t o = 0;
  p.off_kr = o; o = align_up(o + 2 * (size_t)nb * p.kr_q, 256);
  p.off_qr = o; o = align_up(o + 2 * (size_t)nb * p.qr_q, 256);
  // partials: bf16 O / l for the multi-token kernel, fp32 O otherwise
  p.off_opart = o; o = align_up(o + (p.multi ? 2 : 4) * (size_t)nb * p.op_q, 256);
  p.off_ml = o; o = align_up(o + 4 * (size_t)nb * p.ml_q, 256);
  p.total = o;
  return p;
}

// omega_m = theta^(-2m/128), made for each call
RopeTab rope_tab(double theta) {
  RopeTab t;
  for (int m = 0; m < kDim / 2; ++m) t.om[m] = std::pow(theta, -2.0 * (double)m / (double)kDim);
  return t;
}

}  // namespace

size_t attend_workspace(int32_t M, int32_t M_loc, int32_t n_q_heads, int64_t max_sel_chunks,
                        int32_t nb) {
  return attn_plan(M, M_loc, n_q_heads, max_sel_chunks, nb).total;
}


int launch_attend(const AttendArgs& a, void* ws, size_t ws_bytes, hipStream_t s,
                  const AttendBatch* batch) {
  const int32_t nb = batch ? batch->nb : 1;
  const AttnPlan p = attn_plan(a.M, a.M_loc, a.n_q_heads, a.max_sel_chunks, nb);
  if (ws_bytes < p.total) return fail(MSA_ERR_WORKSPACE, "attend workspace too small");
  if (nb > 1 && batch->q_stride != (int64_t)a.M * a.n_q_heads * kDim)
    return fail(MSA_ERR_UNSUPPORTED, "batched attention: packed queries only");
  if ((int64_t)p.n_splits * nb > 65535)
    return fail(MSA_ERR_SHAPE, "batched attention: %d queries x %d key splits exceed the grid",
                nb, p.n_splits);
  char* base = static_cast<char*>(ws);
  uint16_t* Kr = reinterpret_cast<uint16_t*>(base + p.off_kr);
  float* Opart = reinterpret_cast<float*>(base + p.off_opart);
  float* ML = reinterpret_cast<float*>(base + p.off_ml);
  const float qk_scale_log2 = (float)(1.0 / sqrt((double)kDim)) * kLog2e;
  const RopeTab rt = rope_tab(a.theta);

  if (p.multi) {
    uint16_t* Qr = reinterpret_cast<uint16_t*>(base + p.off_qr);
    uint16_t* kr_dst = a.k_loc_rotated ? nullptr : Kr;
    const int64_t q_stride = batch ? batch->q_stride : 0;
    const int64_t kl_stride = batch ? batch->kv_stride : 0;
    // one wave (64 lanes) per token and group of 8 heads
    const int64_t waves =
        ((int64_t)a.M * (a.n_q_heads / kRotHeads) + (kr_dst ? (int64_t)a.M_loc : 0)) * nb;
    hipLaunchKernelGGL(rot_qk_kernel, dim3((unsigned)((waves * 64 + 255) / 256)), dim3(256), 0, s,
                       a.Q, a.M, a.n_q_heads, a.K_loc, a.M_loc, a.n_sel, a.top_k, a.pos0, rt,
                       qk_scale_log2, Qr, kr_dst, nb, q_stride, kl_stride);
    MSA_LAUNCH_CHECK("rot_qk_kernel launch");
    MtArgs k;
    k.Qr = Qr; k.M = a.M; k.Hq = a.n_q_heads;
    k.Kr = a.k_loc_rotated ? a.K_loc : Kr; k.Vloc = a.V_loc; k.M_loc = a.M_loc;
    k.Kbar = a.Kbar; k.Vbar = a.Vbar; k.n_chunks = a.n_chunks;
    k.dco = a.dco; k.n_docs = a.n_docs;
    k.sel_ids = a.sel_ids; k.n_sel = a.n_sel; k.top_k = a.top_k;
    k.max_sel = a.max_sel_chunks;
    k.Opart = reinterpret_cast<uint16_t*>(base + p.off_opart); k.ML = ML;
    k.n_splits = p.n_splits;
    k.qr_stride = p.qr_q;
    k.kr_stride = a.k_loc_rotated ? kl_stride : p.kr_q;
    k.v_stride = kl_stride;
    k.op_stride = p.op_q;
    k.ml_stride = p.ml_q;
    const dim3 grid(p.row_blocks, kHeads, p.n_splits * nb);
    if (a.kv_on_host)
      hipLaunchKernelGGL(attn_mt_kernel<true>, grid, dim3(kMtThreads), 0, s, k);
    else
      hipLaunchKernelGGL(attn_mt_kernel<false>, grid, dim3(kMtThreads), 0, s, k);
    MSA_LAUNCH_CHECK("attn_mt_kernel launch");
    const int64_t n_rows = (int64_t)a.M * a.n_q_heads;
    hipLaunchKernelGGL(combine_rows_kernel,
                       dim3((unsigned)((n_rows * nb + kCombRows - 1) / kCombRows)), dim3(256), 0,
                       s, k.Opart, ML, p.n_splits, n_rows, nb, p.op_q, p.ml_q, a.out, a.out_f32);
    MSA_LAUNCH_CHECK("combine_rows_kernel launch");
    return MSA_OK;
  } else {
    AttnArgs k;
    k.Q = a.Q; k.M = a.M; k.Hq = a.n_q_heads;
    k.Kloc = a.K_loc; k.Vloc = a.V_loc; k.M_loc = a.M_loc;
    k.rot_inline = a.k_loc_rotated ? 0 : 1;
    k.Kbar = a.Kbar; k.Vbar = a.Vbar; k.n_chunks = a.n_chunks;
    k.dco = a.dco; k.n_docs = a.n_docs;
    k.sel_ids = a.sel_ids; k.n_sel = a.n_sel; k.top_k = a.top_k;
    k.max_sel = a.max_sel_chunks; k.pos0 = a.pos0;
    k.qk_scale_log2 = qk_scale_log2;
    k.Opart = Opart;
    k.ML = ML;
    k.n_splits = p.n_splits;
    k.q_stride = batch ? batch->q_stride : 0;
    k.kl_stride = batch ? batch->kv_stride : 0;
    k.op_stride = p.op_q;
    k.ml_stride = p.ml_q;
    k.rt = rt;
    const dim3 grid(p.row_blocks, kHeads, p.n_splits * nb);
    if (a.kv_on_host)
      hipLaunchKernelGGL(attn_kernel<true>, grid, dim3(64), 0, s, k);
    else
      hipLaunchKernelGGL(attn_kernel<false>, grid, dim3(64), 0, s, k);
    MSA_LAUNCH_CHECK("attn_kernel launch");
  }

  const int64_t n_rows = (int64_t)a.M * a.n_q_heads;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(n_rows * nb)), dim3(kDim), 0, s, Opart, ML,
                     p.n_splits, n_rows, p.op_q, p.ml_q, a.out, a.out_f32);
  MSA_LAUNCH_CHECK("combine_kernel launch");
  return MSA_OK;
}

}  // namespace msa
