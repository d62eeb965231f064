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
// Pipeline (one stream, two launches; three when several row blocks share
// the local keys):
//   rot_k     (only then) rotates K_loc into the workspace, one thread per
//             rotation pair, so that each local key is rotated once;
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
  int32_t key_split; float qk_scale_log2;
  float* Opart; float* ML;
  RopeTab rt;
};

__device__ __forceinline__ int clamp_nsel(const int32_t* n_sel, int top_k) {
  int ns = *n_sel;
  return ns < 0 ? 0 : (ns > top_k ? top_k : ns);
}

// Local keys rotated once into the workspace: K rows v·8 + g at pos0 + v.
__global__ __launch_bounds__(256) void rot_k_kernel(const uint16_t* __restrict__ Kl, int32_t M_loc,
                                                    const int32_t* __restrict__ n_sel,
                                                    int32_t top_k, int64_t pos0_arg, RopeTab rt,
                                                    uint16_t* __restrict__ Kr) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)M_loc * kHeads * (kDim / 2)) return;
  const int64_t pos0 = pos0_arg < 0 ? (int64_t)clamp_nsel(n_sel, top_k) : pos0_arg;
  const int64_t row = idx / (kDim / 2);
  const int m = (int)(idx % (kDim / 2));
  double sn, cs;
  sincos((double)(pos0 + row / kHeads) * rt.om[m], &sn, &cs);
  const uint16_t* src = Kl + row * kDim;
  const double x = bf16f(src[m]), y = bf16f(src[m + 64]);
  Kr[row * kDim + m] = d2bf(x * cs - y * sn);
  Kr[row * kDim + m + 64] = d2bf(y * cs + x * sn);
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
  return make_uint4(pack2(f2bf(f[0]), f2bf(f[1])), pack2(f2bf(f[2]), f2bf(f[3])),
                    pack2(f2bf(f[4]), f2bf(f[5])), pack2(f2bf(f[6]), f2bf(f[7])));
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
  const int split = blockIdx.z;
  const int G = a.Hq / kHeads;    // query heads per KV head
  const int rows_g = a.M * G;
  const int64_t n_rows_tot = (int64_t)a.M * a.Hq;
  gbf16* Kbar = uniform_ptr(a.Kbar);
  gbf16* Vbar = uniform_ptr(a.Vbar);
  gbf16* Kloc = uniform_ptr(a.Kloc);
  gbf16* Vloc = uniform_ptr(a.Vloc);

  // the query rows are loaded first: their loads overlap the chunk-list ones
  uint4 qa[8];
  const int r = rb * kRowTile + col;
  if (r < rows_g) {
    const int u = r / G, h = g * G + r % G;
    const uint4* qrow = reinterpret_cast<const uint4*>(a.Q + ((int64_t)u * a.Hq + h) * kDim);
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
  const int32_t id = lane < a.top_k ? a.sel_ids[lane] : -1;   // loaded with n_sel
  const int ns = clamp_nsel(a.n_sel, a.top_k);
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
  const int k_begin = split * a.key_split;
  const int k_end = min(k_begin + a.key_split, n_keys);
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
      const float alpha = (mn == -INFINITY) ? 1.0f : exp2f(mrow[v] - mn);
      p[v] = (mn == -INFINITY) ? 0.0f : exp2f(sv - mn);
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
    for (int db = 0; db < 4; ++db) a.Opart[grow * kDim + db * 32 + col] = O[db][v];
    if (col == 0) {
      a.ML[grow * 2] = mrow[v];
      a.ML[grow * 2 + 1] = lpart[v];
    }
  }
}

// One workgroup per output row, a thread per dim. Every split's (m, l) and
// partial are loaded in one round (a split with no keys has m = -inf and a
// zero partial, so its weight exp2(-inf - max) = 0 drops it); the sum runs
// in split order.
constexpr int kCombineBatch = 64;
__global__ __launch_bounds__(128) void combine_kernel(const float* __restrict__ Opart,
                                                      const float* __restrict__ ML,
                                                      int32_t n_splits, int64_t n_rows,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ out_f32) {
  __shared__ float ms[kMaxSplits], ls[kMaxSplits];
  const int64_t row = blockIdx.x;
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
  out[row * kDim + d] = f2bf(o);
  if (out_f32) out_f32[row * kDim + d] = o;
}

struct AttnPlan {
  int32_t row_blocks, key_split, n_splits;
  bool rot_inline;
  size_t off_kr, off_opart, off_ml, total;
};

AttnPlan attn_plan(int32_t M, int32_t M_loc, int32_t Hq, int64_t max_sel) {
  AttnPlan p;
  const int32_t G = Hq / kHeads;
  p.row_blocks = (M * G + kRowTile - 1) / kRowTile;
  // with one row block every local key is read by one wave per KV head, so
  // it is rotated where it is read; otherwise once, by rot_k_kernel
  p.rot_inline = p.row_blocks == 1;
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
  p.off_kr = o; o = align_up(o + 2 * (size_t)M_loc * kHeads * kDim, 256);
  p.off_opart = o; o = align_up(o + 4 * (size_t)ws_splits * M * Hq * kDim, 256);
  p.off_ml = o; o = align_up(o + 4 * 2 * (size_t)ws_splits * M * Hq, 256);
  p.total = o;
  return p;
}

// omega_m = theta^(-2m/128), kept for the last theta used
const RopeTab& rope_tab(double theta) {
  static thread_local RopeTab t;
  static thread_local double last = -1.0;
  if (theta != last) {
    for (int m = 0; m < kDim / 2; ++m) t.om[m] = std::pow(theta, -2.0 * (double)m / (double)kDim);
    last = theta;
  }
  return t;
}

}  // namespace

size_t attend_workspace(int32_t M, int32_t M_loc, int32_t n_q_heads, int64_t max_sel_chunks) {
  return attn_plan(M, M_loc, n_q_heads, max_sel_chunks).total;
}

int launch_attend(const AttendArgs& a, void* ws, size_t ws_bytes, hipStream_t s) {
  const AttnPlan p = attn_plan(a.M, a.M_loc, a.n_q_heads, a.max_sel_chunks);
  if (ws_bytes < p.total) return fail(MSA_ERR_WORKSPACE, "attend workspace too small");
  char* base = static_cast<char*>(ws);
  uint16_t* Kr = reinterpret_cast<uint16_t*>(base + p.off_kr);
  AttnArgs k;
  k.Q = a.Q; k.M = a.M; k.Hq = a.n_q_heads;
  k.Kloc = a.K_loc; k.Vloc = a.V_loc; k.M_loc = a.M_loc;
  k.rot_inline = (!a.k_loc_rotated && p.rot_inline) ? 1 : 0;
  k.Kbar = a.Kbar; k.Vbar = a.Vbar; k.n_chunks = a.n_chunks;
  k.dco = a.dco; k.n_docs = a.n_docs;
  k.sel_ids = a.sel_ids; k.n_sel = a.n_sel; k.top_k = a.top_k;
  k.max_sel = a.max_sel_chunks; k.pos0 = a.pos0;
  k.key_split = p.key_split;
  k.qk_scale_log2 = (float)(1.0 / sqrt((double)kDim)) * kLog2e;
  k.Opart = reinterpret_cast<float*>(base + p.off_opart);
  k.ML = reinterpret_cast<float*>(base + p.off_ml);
  k.rt = rope_tab(a.theta);
  if (!a.k_loc_rotated && !p.rot_inline) {
    const int64_t pairs = (int64_t)a.M_loc * kHeads * (kDim / 2);
    hipLaunchKernelGGL(rot_k_kernel, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0, s,
                       a.K_loc, a.M_loc, a.n_sel, a.top_k, a.pos0, k.rt, Kr);
    MSA_LAUNCH_CHECK("rot_k_kernel launch");
    k.Kloc = Kr;
  }
  if (a.kv_on_host)
    hipLaunchKernelGGL(attn_kernel<true>, dim3(p.row_blocks, kHeads, p.n_splits), dim3(64), 0, s, k);
  else
    hipLaunchKernelGGL(attn_kernel<false>, dim3(p.row_blocks, kHeads, p.n_splits), dim3(64), 0, s, k);
  MSA_LAUNCH_CHECK("attn_kernel launch");

  const int64_t n_rows = (int64_t)a.M * a.n_q_heads;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)n_rows), dim3(kDim), 0, s, k.Opart, k.ML,
                     p.n_splits, n_rows, a.out, a.out_f32);
  MSA_LAUNCH_CHECK("combine_kernel launch");
  return MSA_OK;
}

}  // namespace msa
