// msa_pool: chunk mean-pooling with document-wise RoPE (MSA stage 1).
//
// Method (portal.techblg.uk IRMaD reading, section M, routing bullet and
// positional-encoding bullet): K̄ = φ(K), V̄ = φ(V), K̄^R = φ(K^R) where φ is the
// mean over each 64-token chunk of a document, and K carries RoPE whose
// positions restart at 0 in every document. Readings: K is rotated at its
// document-local token position before the mean (TOKEN mode) or the pooled
// mean is rotated at its chunk index (CHUNK mode); rotate-half pairs
// (m, m+64) with ω_m = θ^(-2m/128); a partial last chunk is divided by its own
// token count; output is rounded to bf16 (the caches are BF16).
//
// Design (HBM-bound stream, 6 KiB read per token):
//   - each wave pools kChunksPerWave consecutive chunks of one tensor; V and
//     K^R go through a plain-mean instantiation and K through the RoPE one,
//     so the plain pass keeps its register count (and occupancy) low;
//   - lane (h, p) = (lane/8, lane%8) owns dims [8p, 8p+8) and [64+8p, 64+8p+8)
//     of head h: both halves of every rotation pair it needs arrive in its own
//     two 16-byte loads, so RoPE needs no cross-lane exchange;
//   - sums are fp64: on gfx950 an fp64 add issues at the rate of a non-packed
//     fp32 add, and fp64 makes the bf16 result the correctly rounded mean
//     (the fp32 error of a 64-term sum can exceed one bf16 ulp when the mean
//     is near zero);
//   - cos/sin of t·ω advance by an fp64 angle-addition step per token; the
//     host supplies cos ω_m, sin ω_m in fp64, and a chunk that does not
//     continue the previous one (a wave's first chunk, CHUNK mode) reaches its
//     angle by square-and-multiply of that one-step rotation;
//   - token loads are branch-free (clamped indices, masked values) and go
//     into two register sets taken in turn (4 tokens per group plain, 2 with
//     RoPE): one group is summed while the next is in flight.
#include <cmath>

#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kChunksPerWave = 2;   // (1, 2, 4, 8, 16 measured: 2 is fastest)
constexpr int kWavesPerWG = 4;

// Largest i in [0, n_docs-1] with dco[i] <= c (document holding chunk c).
__device__ int find_doc(const int64_t* dco, int n_docs, int64_t c) {
  int lo = 0, hi = n_docs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (dco[mid] <= c) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// (cos, sin) of n·ω from (cos ω, sin ω) by square-and-multiply (n >= 0).
__device__ __forceinline__ void rot_pow(double c1, double s1, int64_t n, double& c, double& s) {
  c = 1.0;
  s = 0.0;
  double bc = c1, bs = s1;
  while (n > 0) {
    if (n & 1) {
      const double t = c * bc - s * bs;
      s = s * bc + c * bs;
      c = t;
    }
    const double t = bc * bc - bs * bs;
    bs = 2.0 * bc * bs;
    bc = t;
    n >>= 1;
  }
}

__device__ __forceinline__ void unpack8(const uint4& x, double* v) {
  v[0] = bf16lo(x.x); v[1] = bf16hi(x.x);
  v[2] = bf16lo(x.y); v[3] = bf16hi(x.y);
  v[4] = bf16lo(x.z); v[5] = bf16hi(x.z);
  v[6] = bf16lo(x.w); v[7] = bf16hi(x.w);
}

__device__ __forceinline__ uint4 pack8(const double* m) {
  uint4 r;
  r.x = pack2(d2bf(m[0]), d2bf(m[1]));
  r.y = pack2(d2bf(m[2]), d2bf(m[3]));
  r.z = pack2(d2bf(m[4]), d2bf(m[5]));
  r.w = pack2(d2bf(m[6]), d2bf(m[7]));
  return r;
}

// One wave pools kChunksPerWave consecutive chunks of one tensor. ROPE: the
// tensor is K and carries document RoPE (TOKEN or CHUNK mode); otherwise a
// plain mean (V, K^R). Lane (h, p) = (lane/8, lane%8) owns dims [8p, 8p+8)
// and [64+8p, 64+8p+8) of head h.
template <bool ROPE, int kUnroll>
__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a, int32_t first_tensor) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 3, p = lane & 7;
  const int idx0 = h * 16 + p;        // 16-byte vector holding dims 8p..8p+7
  const int idx1 = idx0 + 8;          // dims 64+8p..64+8p+7
  const int tensor = first_tensor + (int)blockIdx.y;   // 0: K, 1: V, 2: K^R
  const uint16_t* src = tensor == 0 ? a.K : (tensor == 1 ? a.V : a.KR);
  uint16_t* dst = tensor == 0 ? a.Kbar : (tensor == 1 ? a.Vbar : a.KRbar);
  if (dst == nullptr) return;
  const int64_t c_first = ((int64_t)blockIdx.x * kWavesPerWG + wave) * kChunksPerWave;
  if (c_first >= a.n_chunks) return;
  const int64_t c_begin = a.chunk_base + c_first;
  const int64_t c_end = a.chunk_base + min(c_first + (int64_t)kChunksPerWave, a.n_chunks);
  const bool tok_rope = ROPE && a.rope_mode == MSA_DOC_ROPE_TOKEN;
  const bool chunk_rope = ROPE && a.rope_mode == MSA_DOC_ROPE_CHUNK;

  // the one-step rotation (cos ω, sin ω) of this lane's 8 pairs, and the
  // running rotation (cs, sn) of the current token
  double cw[8], sw[8], cs[8], sn[8];
  if (ROPE) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      cw[e] = a.cw[8 * p + e];
      sw[e] = a.sw[8 * p + e];
      cs[e] = 1.0; sn[e] = 0.0;
    }
  }

  int doc = find_doc(a.dco, a.n_docs, c_begin);
  int64_t next_pos = -1;  // document position at which (cs, sn) is valid
  const uint4* src4 = reinterpret_cast<const uint4*>(src);
  uint4* dst4 = reinterpret_cast<uint4*>(dst);

  for (int64_t c = c_begin; c < c_end; ++c) {
    while (doc + 1 < a.n_docs && a.dco[doc + 1] <= c) { ++doc; next_pos = -1; }
    int64_t j = c - a.dco[doc];
    if (j < 0) j = 0;
    int64_t t0 = a.dto[doc] + j * a.chunk;
    int64_t t1 = min(t0 + (int64_t)a.chunk, a.dto[doc + 1]);
    t0 = max((int64_t)0, min(t0, a.n_tokens));
    t1 = max(t0, min(t1, a.n_tokens));
    const int n = (int)(t1 - t0);
    const int64_t pos = j * a.chunk;

    if (tok_rope && pos != next_pos) {
      for (int e = 0; e < 8; ++e) rot_pow(cw[e], sw[e], pos, cs[e], sn[e]);
    }

    double acc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0;

    // Branch-free loads: token indices past the chunk's end are clamped to
    // its last token (always in bounds) and their values masked out. Two
    // register sets take turns: a group of kUnroll tokens is summed while the
    // next group's loads are in flight. An empty chunk (malformed offsets can
    // place it at t0 = n_tokens) reads the last token instead, masked out.
    const uint4* row = src4 + min(t0, a.n_tokens - 1) * kRowVec;
    const int last = n > 0 ? n - 1 : 0;
    auto load = [&](int t, uint4* x0, uint4* x1) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t tt = min(t + u, last);
        x0[u] = load_stream(row + tt * kRowVec + idx0);
        x1[u] = load_stream(row + tt * kRowVec + idx1);
      }
    };
    auto consume = [&](int t, const uint4* x0, const uint4* x1) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        // a clamped duplicate contributes +0 (its words are zeroed)
        const uint32_t m = (t + u < n) ? 0xffffffffu : 0u;
        const uint4 y0 = make_uint4(x0[u].x & m, x0[u].y & m, x0[u].z & m, x0[u].w & m);
        const uint4 y1 = make_uint4(x1[u].x & m, x1[u].y & m, x1[u].z & m, x1[u].w & m);
        double lo[8], hi[8];
        unpack8(y0, lo);
        unpack8(y1, hi);
        if (tok_rope) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            acc[e] = fma(lo[e], cs[e], fma(-hi[e], sn[e], acc[e]));
            acc[8 + e] = fma(hi[e], cs[e], fma(lo[e], sn[e], acc[8 + e]));
            const double c2 = cs[e] * cw[e] - sn[e] * sw[e];
            sn[e] = sn[e] * cw[e] + cs[e] * sw[e];
            cs[e] = c2;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            acc[e] += lo[e];
            acc[8 + e] += hi[e];
          }
        }
      }
    };
    uint4 xa[kUnroll], xb[kUnroll], ya[kUnroll], yb[kUnroll];
    load(0, xa, xb);
    for (int t = 0;;) {
      load(t + kUnroll, ya, yb);
      consume(t, xa, xb);
      t += kUnroll;
      if (t >= n) break;
      load(t + kUnroll, xa, xb);
      consume(t, ya, yb);
      t += kUnroll;
      if (t >= n) break;
    }
    if (tok_rope) {
      // the recurrence advanced past the chunk's end by the masked tail steps;
      // it stays valid only when the chunk was full (the next chunk continues)
      next_pos = (n % kUnroll == 0) ? pos + n : -1;
    }

    double mean[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) mean[e] = n > 0 ? acc[e] / (double)n : 0.0;
    if (chunk_rope) {
      for (int e = 0; e < 8; ++e) {
        double c_, s_;
        rot_pow(cw[e], sw[e], j, c_, s_);
        const double x = mean[e], y = mean[8 + e];
        mean[e] = x * c_ - y * s_;
        mean[8 + e] = y * c_ + x * s_;
      }
    }
    dst4[c * kRowVec + idx0] = pack8(mean);
    dst4[c * kRowVec + idx1] = pack8(mean + 8);
  }
}

}  // namespace

int launch_pool(const PoolArgs& args, hipStream_t s) {
  if (args.n_chunks == 0) return MSA_OK;
  PoolArgs a = args;
  for (int m = 0; m < 64; ++m) {
    const double om = std::pow(a.theta, -2.0 * (double)m / (double)kDim);
    a.cw[m] = std::cos(om);
    a.sw[m] = std::sin(om);
  }
  const int64_t per_wg = (int64_t)kChunksPerWave * kWavesPerWG;
  const unsigned n_wg = (unsigned)((a.n_chunks + per_wg - 1) / per_wg);
  // V and K^R (plain means), then K (document RoPE): separate instantiations
  // so the plain pass does not carry the rotation state's registers
  if (a.Vbar || a.KRbar) {
    hipLaunchKernelGGL((pool_kernel<false, 4>), dim3(n_wg, 2), dim3(256), 0, s, a, 1);
    MSA_LAUNCH_CHECK("pool_kernel<plain> launch");
  }
  if (a.Kbar) {
    hipLaunchKernelGGL((pool_kernel<true, 2>), dim3(n_wg, 1), dim3(256), 0, s, a, 0);
    MSA_LAUNCH_CHECK("pool_kernel<rope> launch");
  }
  return MSA_OK;
}

}  // namespace msa
