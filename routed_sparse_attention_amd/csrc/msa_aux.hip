// Router supervision: the auxiliary contrastive loss and its gradient.
//
// Method (portal.techblg.uk IRMaD reading, section M, training bullet):
//   L_aux = −(1/|P|) Σ_{i∈P} log[ exp(s_i/τ) / (exp(s_i/τ) + Σ_{j∉P} exp(s_j/τ)) ]
// over the query's routing document scores s (section M, routing bullet:
// s_i = max_j max_t mean_h cos(Q^R_{t,h}, K̄^R_{ij,h})), supervising every
// layer's router. Readings: the negatives of every positive are all other
// documents of the store; τ is a parameter; the gradient reaches the first
// maximising chunk of each document and, in it, the first maximising token.
//
// Pipeline (deterministic: fixed reduction orders, no atomics):
//   msa_route_scores   chunk scores S [B, C] (the routing scan kernels);
//   qnorm              max(‖q_{b,t,h}‖, eps) per query row and head;
//   doc_argmax         c* = the first chunk of each document reaching its max;
//   aux_doc_fwd        one wave per document, looping over the queries: the
//                      first token t* maximising the head-mean cosine at c*,
//                      recomputed in fp32 (the exact bf16 products), which is
//                      also the s_i the loss uses, and the per-head cosines;
//   aux_weights        one workgroup per query: loss and ∂L/∂s_k for every
//                      document (max-shifted exponentials, fp32);
//   aux_dk             one wave per document: every chunk row of dK̄^R is
//                      written once — the sum over queries (in order) of
//                      (w/8)(q̂ − cos·k̂)/‖k‖ where that query chose the chunk;
//   aux_dq_partial/final  dQ^R[b,t] = (U − q̂·A)/(8‖q‖) per head with
//                      U = Σ w k̂, A = Σ w cos over the documents whose t* is
//                      t: partial sums over fixed document ranges, then an
//                      in-order sum of the partials.
// Row layout in a wave: lane l holds elements [16l, 16l+16) of a 1024-element
// (8 heads × 128) row, so the 8 lanes of head l/8 reduce with three DPP steps.
#include <cmath>

#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kAuxMaxPos = 256;

__device__ __forceinline__ void load_row16(const uint16_t* row, int lane, float* x) {
  const uint4* p = reinterpret_cast<const uint4*>(row) + 2 * lane;
  const uint4 a = p[0], b = p[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = bf16lo(w[i]);
    x[2 * i + 1] = bf16hi(w[i]);
  }
}

// sum over the 8 lanes of this lane's head (every one of them gets it)
__device__ __forceinline__ float head_sum8(float v) {
  v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);   // row_half_mirror: the other quad of the 8
  return v;
}

// sum over the 8 heads of a value that is uniform within each head's lanes
__device__ __forceinline__ float heads_total(float v) {
  v += dpp_f<0x140>(v);   // row_mirror: heads 2r and 2r+1 of the 16-lane row
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ void clamp_range(const int64_t* dco, int k, int64_t C, int64_t& c0,
                                            int64_t& c1) {
  c0 = dco[k];
  c1 = dco[k + 1];
  c0 = c0 < 0 ? 0 : (c0 > C ? C : c0);
  c1 = c1 < c0 ? c0 : (c1 > C ? C : c1);
}

// max(‖q_{b,t,h}‖, eps): one wave per query row
__global__ __launch_bounds__(256) void qnorm_kernel(const uint16_t* __restrict__ QR, int64_t rows,
                                                    float* __restrict__ qn) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  float x[16];
  load_row16(QR + r * kRowElems, lane, x);
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) ss = fmaf(x[e], x[e], ss);
  ss = head_sum8(ss);
  if ((lane & 7) == 0) qn[r * kHeads + (lane >> 3)] = fmaxf(sqrtf(ss), kNormEps);
}

// c*: the first chunk of document k reaching its maximum chunk score. The
// 256 documents of a block own one contiguous chunk range, streamed through
// an LDS tile with coalesced loads; each thread scans its own chunks there.
constexpr int kArgTile = 4096;
__global__ __launch_bounds__(256) void doc_argmax_kernel(const float* __restrict__ S, int64_t C,
                                                         const int64_t* __restrict__ dco,
                                                         int32_t N, int32_t* __restrict__ cstar) {
  __shared__ float tile[kArgTile];
  const int b = blockIdx.y;
  const int64_t d0 = (int64_t)blockIdx.x * 256;
  const int64_t d1 = d0 + 256 < N ? d0 + 256 : N;
  const int64_t k = d0 + threadIdx.x;
  int64_t r0, r1, tmp, c0 = 0, c1 = 0;
  clamp_range(dco, (int)d0, C, r0, tmp);
  clamp_range(dco, (int)(d1 - 1), C, tmp, r1);
  if (r1 < r0) r1 = r0;
  if (k < N) clamp_range(dco, (int)k, C, c0, c1);
  const float* Sb = S + (int64_t)b * C;
  float best = -INFINITY;
  int64_t arg = c0 < C ? c0 : (C > 0 ? C - 1 : 0);
  for (int64_t t0 = r0; t0 < r1; t0 += kArgTile) {
    const int n = (int)(r1 - t0 < kArgTile ? r1 - t0 : kArgTile);
    float v[kArgTile / 256];
#pragma unroll
    for (int u = 0; u < kArgTile / 256; ++u) {
      const int i = (int)threadIdx.x + u * 256;
      v[u] = Sb[t0 + (i < n ? i : n - 1)];
    }
#pragma unroll
    for (int u = 0; u < kArgTile / 256; ++u) tile[threadIdx.x + u * 256] = v[u];
    __syncthreads();
    const int64_t a = c0 > t0 ? c0 : t0, e = c1 < t0 + n ? c1 : t0 + n;
    for (int64_t c = a; c < e; ++c) {
      const float x = tile[c - t0];
      if (x > best) { best = x; arg = c; }
    }
    __syncthreads();
  }
  if (k < N) cstar[(int64_t)b * N + k] = (int32_t)arg;
}

// t*, the exact s_k and the per-head cosines at (t*, c*): one wave per doc
__global__ __launch_bounds__(256) void aux_doc_fwd_kernel(
    const uint16_t* __restrict__ QR, int32_t B, int32_t M, const float* __restrict__ qn,
    const uint16_t* __restrict__ KR, int32_t N, const int32_t* __restrict__ cstar,
    float* __restrict__ s_out, int32_t* __restrict__ tstar, float* __restrict__ cosv) {
  const int lane = threadIdx.x & 63;
  const int k = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (k >= N) return;
  const int h = lane >> 3;
  for (int b = 0; b < B; ++b) {
    const int64_t bk = (int64_t)b * N + k;
    float kx[16];
    load_row16(KR + (int64_t)cstar[bk] * kRowElems, lane, kx);
    float kk = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) kk = fmaf(kx[e], kx[e], kk);
    const float nk = fmaxf(sqrtf(head_sum8(kk)), kNormEps);
    float best = -INFINITY, best_cos = 0.0f;
    int tb = 0;
    for (int t = 0; t < M; ++t) {
      const int64_t row = (int64_t)b * M + t;
      float qx[16];
      load_row16(QR + row * kRowElems, lane, qx);
      float d = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) d = fmaf(qx[e], kx[e], d);
      const float cs = head_sum8(d) / (qn[row * kHeads + h] * nk);
      const float S = heads_total(cs) * 0.125f;
      if (S > best) {   // uniform over the wave; strict: the first maximum wins
        best = S;
        best_cos = cs;
        tb = t;
      }
    }
    if (lane == 0) {
      s_out[bk] = best;
      tstar[bk] = tb;
    }
    if ((lane & 7) == 0) cosv[bk * kHeads + h] = best_cos;
  }
}

// loss[b] and w[b,k] = ∂L/∂s_k: one workgroup per query
constexpr int kWThreads = 1024;
__global__ __launch_bounds__(kWThreads) void aux_weights_kernel(
    const float* __restrict__ s, int32_t N, const int32_t* __restrict__ pos_ids,
    const int32_t* __restrict__ n_pos, int32_t max_pos, float tau, float* __restrict__ loss,
    float* __restrict__ w) {
  __shared__ int pid[kAuxMaxPos];
  __shared__ int n_p;
  __shared__ float red[kWThreads / 64];
  __shared__ float zpos[kAuxMaxPos], tpos[kAuxMaxPos];
  __shared__ float m_sh, zneg_sh, rsum_sh;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* sb = s + (int64_t)b * N;
  float* wb = w + (int64_t)b * N;
  const float inv_tau = 1.0f / tau;

  // distinct valid positives, in list order
  if (tid == 0) {
    int np = n_pos[b];
    np = np < 0 ? 0 : (np > max_pos ? max_pos : np);
    int cnt = 0;
    for (int i = 0; i < np; ++i) {
      const int id = pos_ids[(int64_t)b * max_pos + i];
      if (id < 0 || id >= N) continue;
      bool seen = false;
      for (int j = 0; j < cnt; ++j) seen = seen || pid[j] == id;
      if (!seen) pid[cnt++] = id;
    }
    n_p = cnt;
  }
  __syncthreads();
  const int P = n_p;
  auto is_pos = [&](int k) {
    bool r = false;
    for (int j = 0; j < P; ++j) r = r || pid[j] == k;
    return r;
  };
  if (P == 0) {
    for (int k = tid; k < N; k += kWThreads) wb[k] = 0.0f;
    if (tid == 0) loss[b] = 0.0f;
    return;
  }
  // m = max_k s_k/τ (the shift of every exponential)
  float m = -INFINITY;
  for (int k = tid; k < N; k += kWThreads) m = fmaxf(m, sb[k] * inv_tau);
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (tid == 0) {
    float x = red[0];
    for (int i = 1; i < kWThreads / 64; ++i) x = fmaxf(x, red[i]);
    m_sh = x;
  }
  __syncthreads();
  m = m_sh;
  // Z_neg = Σ over negatives of exp(s/τ − m): strided partials, then a fixed tree
  float z = 0.0f;
  for (int k = tid; k < N; k += kWThreads)
    if (!is_pos(k)) z += expf(sb[k] * inv_tau - m);
  for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
  __syncthreads();
  if (lane == 0) red[wave] = z;
  __syncthreads();
  if (tid == 0) {
    float x = 0.0f;
    for (int i = 0; i < kWThreads / 64; ++i) x += red[i];
    zneg_sh = x;
  }
  __syncthreads();
  const float zneg = zneg_sh;
  // per positive: Z_i and −log(e_i / Z_i)
  if (tid < P) {
    const float a = sb[pid[tid]] * inv_tau - m;
    const float zi = expf(a) + zneg;
    zpos[tid] = zi;
    tpos[tid] = logf(zi) - a;
  }
  __syncthreads();
  if (tid == 0) {
    float l = 0.0f, r = 0.0f;
    for (int j = 0; j < P; ++j) {
      l += tpos[j];
      r += 1.0f / zpos[j];
    }
    loss[b] = l / (float)P;
    rsum_sh = r;
  }
  __syncthreads();
  const float rsum = rsum_sh;
  const float scale = inv_tau / (float)P;
  for (int k = tid; k < N; k += kWThreads) {
    const float e = expf(sb[k] * inv_tau - m);
    int j = -1;
    for (int q = 0; q < P; ++q) j = (j < 0 && pid[q] == k) ? q : j;
    wb[k] = j >= 0 ? -(1.0f - e / zpos[j]) * scale : e * rsum * scale;
  }
}

// every chunk row of dK̄^R, once: one wave per document. The queries'
// (chunk, weight, token) for this document are loaded once, one query per
// lane (64 at a time); per chunk a ballot picks the queries that chose it.
__global__ __launch_bounds__(256) void aux_dk_kernel(
    const uint16_t* __restrict__ QR, int32_t B, int32_t M, const float* __restrict__ qn,
    const uint16_t* __restrict__ KR, int64_t C, const int64_t* __restrict__ dco, int32_t N,
    const int32_t* __restrict__ cstar, const int32_t* __restrict__ tstar,
    const float* __restrict__ cosv, const float* __restrict__ w, float* __restrict__ dK) {
  const int lane = threadIdx.x & 63;
  const int k = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (k >= N) return;
  const int h = lane >> 3;
  int64_t c0, c1;
  clamp_range(dco, k, C, c0, c1);
  const int n_groups = (B + 63) / 64;
  int my_c = -1, my_t = 0;
  float my_w = 0.0f;
  auto load_group = [&](int g) {
    const int b = g * 64 + lane;
    my_c = -1;
    my_w = 0.0f;
    my_t = 0;
    if (b < B) {
      const int64_t bk = (int64_t)b * N + k;
      my_w = w[bk];
      my_c = my_w != 0.0f ? cstar[bk] : -1;
      my_t = tstar[bk];
    }
  };
  if (n_groups == 1) load_group(0);
  for (int64_t c = c0; c < c1; ++c) {
    float acc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
    bool have_k = false;
    float kx[16], nk = 0.0f;
    for (int g = 0; g < n_groups; ++g) {
      if (n_groups > 1) load_group(g);
      uint64_t mask = __ballot(my_c == (int)c);
      while (mask) {   // queries in ascending order: a fixed summation order
        const int j = __builtin_ctzll(mask);
        mask &= mask - 1;
        const int b = g * 64 + j;
        const float wk = __shfl(my_w, j);
        const int t = __shfl(my_t, j);
        if (!have_k) {
          load_row16(KR + c * kRowElems, lane, kx);
          float kk = 0.0f;
#pragma unroll
          for (int e = 0; e < 16; ++e) kk = fmaf(kx[e], kx[e], kk);
          nk = fmaxf(sqrtf(head_sum8(kk)), kNormEps);
          have_k = true;
        }
        const int64_t row = (int64_t)b * M + t;
        float qx[16];
        load_row16(QR + row * kRowElems, lane, qx);
        const float nq = qn[row * kHeads + h];
        const float cs = cosv[((int64_t)b * N + k) * kHeads + h];
        const float gk = wk * 0.125f / nk;
        // (q̂ − cos·k̂)/‖k‖, or q̂/eps when ‖k‖ is at the clamp
        const bool proj = nk > kNormEps;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float qh = qx[e] / nq, kh = kx[e] / nk;
          acc[e] = fmaf(gk, proj ? qh - cs * kh : qh, acc[e]);
        }
      }
    }
    float4* dst = reinterpret_cast<float4*>(dK + c * kRowElems) + 4 * lane;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dst[i] = make_float4(acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]);
  }
}

// partial U = Σ w k̂ and A_h = Σ w cos_h over documents [k0, k1) with t* = t
constexpr int kPartStride = kRowElems + kHeads;
__global__ __launch_bounds__(256) void aux_dq_partial_kernel(
    int32_t M, const uint16_t* __restrict__ KR, int32_t N, const int32_t* __restrict__ cstar,
    const int32_t* __restrict__ tstar, const float* __restrict__ cosv, const float* __restrict__ w,
    int32_t n_parts, float* __restrict__ part) {
  __shared__ float red[4][kPartStride];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bt = blockIdx.x, p = blockIdx.y;
  const int b = bt / M, t = bt % M;
  const int h = lane >> 3;
  const int64_t per = ((int64_t)N + n_parts - 1) / n_parts;
  const int64_t k0 = (int64_t)p * per;
  const int64_t k1 = k0 + per < N ? k0 + per : N;
  float U[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) U[e] = 0.0f;
  float A = 0.0f;
  for (int64_t k = k0 + wave; k < k1; k += 4) {
    const int64_t bk = (int64_t)b * N + k;
    if (tstar[bk] != t) continue;
    const float wk = w[bk];
    if (wk == 0.0f) continue;
    float kx[16];
    load_row16(KR + (int64_t)cstar[bk] * kRowElems, lane, kx);
    float kk = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) kk = fmaf(kx[e], kx[e], kk);
    const float g = wk / fmaxf(sqrtf(head_sum8(kk)), kNormEps);
#pragma unroll
    for (int e = 0; e < 16; ++e) U[e] = fmaf(g, kx[e], U[e]);
    A = fmaf(wk, cosv[bk * kHeads + h], A);
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) red[wave][16 * lane + e] = U[e];
  if ((lane & 7) == 0) red[wave][kRowElems + h] = A;
  __syncthreads();
  float* dst = part + ((int64_t)bt * n_parts + p) * kPartStride;
  for (int i = threadIdx.x; i < kPartStride; i += 256)
    dst[i] = ((red[0][i] + red[1][i]) + red[2][i]) + red[3][i];
}

// dQ^R[b,t] = (U − q̂·A)/(8‖q‖) per head, or U/(8 eps) at the clamp
__global__ __launch_bounds__(64) void aux_dq_final_kernel(const uint16_t* __restrict__ QR,
                                                          const float* __restrict__ qn,
                                                          const float* __restrict__ part,
                                                          int32_t n_parts,
                                                          float* __restrict__ dQ) {
  const int lane = threadIdx.x;
  const int64_t bt = blockIdx.x;
  const int h = lane >> 3;
  float U[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) U[e] = 0.0f;
  float A = 0.0f;
  for (int p = 0; p < n_parts; ++p) {
    const float* src = part + (bt * n_parts + p) * kPartStride;
#pragma unroll
    for (int e = 0; e < 16; ++e) U[e] += src[16 * lane + e];
    A += src[kRowElems + h];
  }
  float qx[16];
  load_row16(QR + bt * kRowElems, lane, qx);
  const float nq = qn[bt * kHeads + h];
  const bool proj = nq > kNormEps;
  const float inv = 0.125f / nq;
  float4* dst = reinterpret_cast<float4*>(dQ + bt * kRowElems) + 4 * lane;
  float o[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) o[e] = inv * (proj ? U[e] - (qx[e] / nq) * A : U[e]);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
}

struct AuxPlan {
  size_t off_route, route_bytes, off_S, off_cstar, off_s, off_tstar, off_cos, off_w, off_qn,
      off_part, total;
  int32_t n_parts;
};

AuxPlan aux_plan(const msa_dims* d, int32_t B, int32_t M, int64_t C, int32_t N) {
  AuxPlan p;
  size_t o = 0;
  p.route_bytes = msa_route_scores_workspace(d, B, M, C);
  p.off_route = o; o = align_up(o + p.route_bytes, 256);
  const size_t bn = (size_t)B * N;
  p.off_S = o; o = align_up(o + 4 * (size_t)B * C, 256);
  p.off_cstar = o; o = align_up(o + 4 * bn, 256);
  p.off_s = o; o = align_up(o + 4 * bn, 256);
  p.off_tstar = o; o = align_up(o + 4 * bn, 256);
  p.off_cos = o; o = align_up(o + 4 * bn * kHeads, 256);
  p.off_w = o; o = align_up(o + 4 * bn, 256);
  p.off_qn = o; o = align_up(o + 4 * (size_t)B * M * kHeads, 256);
  int64_t parts = (2048 + (int64_t)B * M - 1) / ((int64_t)B * M);
  const int64_t by_docs = ((int64_t)N + 63) / 64;
  if (parts > by_docs) parts = by_docs;
  if (parts > 64) parts = 64;
  if (parts < 1) parts = 1;
  p.n_parts = (int32_t)parts;
  p.off_part = o; o = align_up(o + 4 * (size_t)B * M * parts * kPartStride, 256);
  p.total = o;
  return p;
}

}  // namespace
}  // namespace msa

using namespace msa;

extern "C" {

size_t msa_route_aux_loss_workspace(const msa_dims* d, int32_t B, int32_t M, int64_t n_chunks,
                                    int32_t n_docs) {
  if (check_dims(d) || B < 1 || M < 1 || n_docs < 1 || n_chunks < n_docs) return 0;
  return aux_plan(d, B, M, n_chunks, n_docs).total;
}

int32_t msa_route_aux_loss(const msa_dims* d, const msa_bf16* QR, int32_t B, int32_t M,
                           const msa_bf16* KRbar, const int64_t* dco, int32_t n_docs,
                           int64_t n_chunks, const int32_t* pos_ids, const int32_t* n_pos,
                           int32_t max_pos, float tau, float* loss, float* dQR, float* dKRbar,
                           float* doc_scores, int32_t* best_chunk, int32_t* best_token, void* ws,
                           size_t ws_bytes, void* stream) {
  clear_error();
  int rc = check_dims(d);
  if (rc) return rc;
  if (d->token_reduce != MSA_TOKEN_REDUCE_MAX)
    return fail(MSA_ERR_UNSUPPORTED, "aux_loss: only the MAX token reduction is differentiated");
  if (!QR || !KRbar || !dco || !pos_ids || !n_pos || !loss || !dQR || !dKRbar)
    return fail(MSA_ERR_INVALID_ARG, "aux_loss: NULL pointer argument");
  if (!(tau > 0.0f) || !std::isfinite(tau))
    return fail(MSA_ERR_INVALID_ARG, "aux_loss: tau must be finite and > 0");
  if (B < 1 || M < 1 || B > 65535 || (int64_t)B * M > (1 << 20))
    return fail(MSA_ERR_SHAPE, "aux_loss: B=%d M=%d out of range", B, M);
  if (max_pos < 1 || max_pos > kAuxMaxPos)
    return fail(MSA_ERR_SHAPE, "aux_loss: max_pos=%d must be in [1, %d]", max_pos, kAuxMaxPos);
  MSA_A16("aux_loss", QR);
  MSA_A16("aux_loss", KRbar);
  if (n_docs < 1 || n_chunks < n_docs || n_chunks >= ((int64_t)1 << 31))
    return fail(MSA_ERR_SHAPE, "aux_loss: n_docs=%d, n_chunks=%lld out of range", n_docs,
                (long long)n_chunks);
  const AuxPlan p = aux_plan(d, B, M, n_chunks, n_docs);
  if (ws == nullptr || ws_bytes < p.total)
    return fail(MSA_ERR_WORKSPACE, "aux_loss workspace: need %zu bytes, got %zu", p.total,
                ws_bytes);
  char* base = static_cast<char*>(ws);
  float* S = reinterpret_cast<float*>(base + p.off_S);
  int32_t* cstar = best_chunk ? best_chunk : reinterpret_cast<int32_t*>(base + p.off_cstar);
  float* s = doc_scores ? doc_scores : reinterpret_cast<float*>(base + p.off_s);
  int32_t* tstar = best_token ? best_token : reinterpret_cast<int32_t*>(base + p.off_tstar);
  float* cosv = reinterpret_cast<float*>(base + p.off_cos);
  float* w = reinterpret_cast<float*>(base + p.off_w);
  float* qn = reinterpret_cast<float*>(base + p.off_qn);
  float* part = reinterpret_cast<float*>(base + p.off_part);
  hipStream_t st = static_cast<hipStream_t>(stream);

  rc = msa_route_scores(d, QR, B, M, KRbar, n_chunks, S, base + p.off_route, p.route_bytes, stream);
  if (rc) return rc;
  clear_error();
  const int64_t rows = (int64_t)B * M;
  hipLaunchKernelGGL(qnorm_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, QR, rows, qn);
  MSA_LAUNCH_CHECK("qnorm_kernel launch");
  hipLaunchKernelGGL(doc_argmax_kernel, dim3((unsigned)((n_docs + 255) / 256), (unsigned)B),
                     dim3(256), 0, st, S, n_chunks, dco, n_docs, cstar);
  MSA_LAUNCH_CHECK("doc_argmax_kernel launch");
  const unsigned doc_blocks = (unsigned)((n_docs + 3) / 4);
  hipLaunchKernelGGL(aux_doc_fwd_kernel, dim3(doc_blocks), dim3(256), 0, st, QR, B, M, qn, KRbar,
                     n_docs, cstar, s, tstar, cosv);
  MSA_LAUNCH_CHECK("aux_doc_fwd_kernel launch");
  hipLaunchKernelGGL(aux_weights_kernel, dim3((unsigned)B), dim3(kWThreads), 0, st, s, n_docs,
                     pos_ids, n_pos, max_pos, tau, loss, w);
  MSA_LAUNCH_CHECK("aux_weights_kernel launch");
  hipLaunchKernelGGL(aux_dk_kernel, dim3(doc_blocks), dim3(256), 0, st, QR, B, M, qn, KRbar,
                     n_chunks, dco, n_docs, cstar, tstar, cosv, w, dKRbar);
  MSA_LAUNCH_CHECK("aux_dk_kernel launch");
  hipLaunchKernelGGL(aux_dq_partial_kernel, dim3((unsigned)rows, (unsigned)p.n_parts), dim3(256),
                     0, st, M, KRbar, n_docs, cstar, tstar, cosv, w, p.n_parts, part);
  MSA_LAUNCH_CHECK("aux_dq_partial_kernel launch");
  hipLaunchKernelGGL(aux_dq_final_kernel, dim3((unsigned)rows), dim3(64), 0, st, QR, qn, part,
                     p.n_parts, dQR);
  MSA_LAUNCH_CHECK("aux_dq_final_kernel launch");
  return MSA_OK;
}

}  // extern "C"
