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
//   - one workgroup of 3 waves handles kChunksPerWG consecutive chunks; wave 0
//     pools K, wave 1 V, wave 2 K^R, so no wave diverges;
//   - lane (h, p) = (lane/8, lane%8) owns dims [8p, 8p+8) and [64+8p, 64+8p+8)
//     of head h: both halves of every rotation pair it needs arrive in its own
//     two 16-byte loads, so RoPE needs no cross-lane exchange;
//   - sums are fp64: on gfx950 an fp64 add issues at the rate of a non-packed
//     fp32 add, and fp64 makes the bf16 result the correctly rounded mean
//     (the fp32 error of a 64-term sum can exceed one bf16 ulp when the mean
//     is near zero);
//   - cos/sin of t·ω advance by an fp64 angle-addition step per token; only a
//     workgroup's first chunk (if it starts mid-document) needs a sincos.
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kChunksPerWG = 8;
constexpr int kUnroll = 4;

// Largest i in [0, n_docs-1] with dco[i] <= c (document holding chunk c).
__device__ int find_doc(const int64_t* dco, int n_docs, int64_t c) {
  int lo = 0, hi = n_docs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (dco[mid] <= c) lo = mid; else hi = mid - 1;
  }
  return lo;
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

__global__ __launch_bounds__(192) void pool_kernel(PoolArgs a) {
  const int wave = threadIdx.x >> 6;  // 0: K, 1: V, 2: K^R
  const int lane = threadIdx.x & 63;
  const int h = lane >> 3, p = lane & 7;
  const int idx0 = h * 16 + p;        // 16-byte vector holding dims 8p..8p+7
  const int idx1 = idx0 + 8;          // dims 64+8p..64+8p+7
  const uint16_t* src = wave == 0 ? a.K : (wave == 1 ? a.V : a.KR);
  uint16_t* dst = wave == 0 ? a.Kbar : (wave == 1 ? a.Vbar : a.KRbar);
  if (dst == nullptr) return;
  const int64_t c_begin = (int64_t)blockIdx.x * kChunksPerWG;
  if (c_begin >= a.n_chunks) return;
  const int64_t c_end = min(c_begin + (int64_t)kChunksPerWG, a.n_chunks);
  const bool tok_rope = (wave == 0) && a.rope_mode == MSA_DOC_ROPE_TOKEN;
  const bool chunk_rope = (wave == 0) && a.rope_mode == MSA_DOC_ROPE_CHUNK;

  // ω_m for this lane's 8 pairs, and the one-step rotation (cos ω, sin ω).
  double om[8], cw[8], sw[8], cs[8], sn[8];
  if (wave == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      om[e] = pow(a.theta, -2.0 * (double)(8 * p + e) / (double)kDim);
      sincos(om[e], &sw[e], &cw[e]);
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
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (pos == 0) { cs[e] = 1.0; sn[e] = 0.0; }
        else sincos((double)pos * om[e], &sn[e], &cs[e]);
      }
    }

    double acc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0;

    const uint4* row = src4 + t0 * kRowVec;
    for (int t = 0; t < n; t += kUnroll) {
      uint4 x0[kUnroll], x1[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (t + u < n) {
          x0[u] = load_stream(row + (int64_t)(t + u) * kRowVec + idx0);
          x1[u] = load_stream(row + (int64_t)(t + u) * kRowVec + idx1);
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (t + u < n) {
          double lo[8], hi[8];
          unpack8(x0[u], lo);
          unpack8(x1[u], hi);
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
            for (int e = 0; e < 8; ++e) { acc[e] += lo[e]; acc[8 + e] += hi[e]; }
          }
        }
      }
    }
    next_pos = pos + n;

    double mean[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) mean[e] = n > 0 ? acc[e] / (double)n : 0.0;
    if (chunk_rope) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        double s_, c_;
        sincos((double)j * om[e], &s_, &c_);
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

int launch_pool(const PoolArgs& a, hipStream_t s) {
  if (a.n_chunks == 0) return MSA_OK;
  const int64_t n_wg = (a.n_chunks + kChunksPerWG - 1) / kChunksPerWG;
  hipLaunchKernelGGL(pool_kernel, dim3((unsigned)n_wg), dim3(192), 0, s, a);
  MSA_LAUNCH_CHECK("pool_kernel launch");
  return MSA_OK;
}

}  // namespace msa
