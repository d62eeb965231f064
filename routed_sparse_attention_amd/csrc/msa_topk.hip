// msa_doc_reduce + msa_topk: chunk -> document max and top-k selection
// (MSA stage 2, second half).
//
// Method (portal.techblg.uk IRMaD reading, section M, routing bullet):
//   s_i = max_j S_ij over document i's chunks, I = Top-k({s_i}), k = 16.
// Readings: ties go to the lowest document id; with fewer than k documents
// all are selected; a NaN score ranks below every number.
//
// Design. Every document score becomes one unique 64-bit key
//   (order-preserving uint32 of the score) << 32 | (0xFFFFFFFF − id),
// so "larger key" means "better document", equal scores fall back to the
// lower id, and selection is a plain descending sort of integers — the result
// is deterministic and independent of thread order.
//   stage 1: one workgroup per (slice of 1024 documents, query): each thread
//     max-reduces its documents' chunk ranges, max-merges with the previous
//     scores when accumulating, writes the document scores, and the workgroup
//     sorts its 1024 keys (bitonic, in LDS) and keeps its k best;
//   stage 2: one workgroup per query merges the slices' candidates the same
//     way and writes ids, scores and n_sel.
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kSortN = 1024;
constexpr int kThreads = 256;

// Sorts 1024 keys in LDS into descending order (all 256 threads take part).
__device__ void bitonic_desc_1024(uint64_t* s) {
  const int tid = threadIdx.x;
  for (int k = 2; k <= kSortN; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
#pragma unroll
      for (int p = tid; p < kSortN / 2; p += kThreads) {
        const int i = 2 * j * (p / j) + (p % j);
        const int l = i + j;
        const bool desc = (i & k) == 0;
        const uint64_t x = s[i], y = s[l];
        if (desc ? (x < y) : (x > y)) {
          s[i] = y;
          s[l] = x;
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ uint64_t doc_key(float s, int32_t i) {
  return ((uint64_t)ord_key(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
}

__global__ __launch_bounds__(256) void doc_topk1_kernel(const float* __restrict__ S, int64_t C,
                                                        const int64_t* __restrict__ dco,
                                                        int32_t n_docs,
                                                        float* __restrict__ doc_scores,
                                                        int32_t accumulate, int32_t K,
                                                        uint64_t* __restrict__ cand,
                                                        int32_t n_slices) {
  __shared__ uint64_t keys[kSortN];
  const int tid = threadIdx.x;
  const int b = blockIdx.y;
  const int slice = blockIdx.x;
  for (int q = 0; q < kSortN / kThreads; ++q) {
    const int64_t i = (int64_t)slice * kSortN + q * kThreads + tid;
    uint64_t key = 0;
    if (i < n_docs) {
      int64_t c0 = dco[i], c1 = dco[i + 1];
      c0 = max((int64_t)0, min(c0, C));
      c1 = max(c0, min(c1, C));
      float s = -INFINITY;
      const float* Sb = S + (int64_t)b * C;
      for (int64_t c = c0; c < c1; ++c) s = (c == c0) ? Sb[c] : nan_max(s, Sb[c]);
      float* ds = doc_scores + (int64_t)b * n_docs + i;
      if (accumulate) s = nan_max(*ds, s);
      *ds = s;
      key = doc_key(s, (int32_t)i);
    }
    keys[q * kThreads + tid] = key;
  }
  __syncthreads();
  bitonic_desc_1024(keys);
  if (tid < K) cand[((int64_t)b * n_slices + slice) * K + tid] = keys[tid];
}

__global__ __launch_bounds__(256) void doc_topk2_kernel(const uint64_t* __restrict__ cand,
                                                        int32_t n_slices, int32_t K,
                                                        int32_t n_docs,
                                                        int32_t* __restrict__ topk_ids,
                                                        float* __restrict__ topk_scores,
                                                        int32_t* __restrict__ n_sel) {
  __shared__ uint64_t keys[kSortN];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int64_t total = (int64_t)n_slices * K;
  const uint64_t* src = cand + (int64_t)b * total;
  if (tid < K) keys[tid] = 0;
  const int fresh = kSortN - K;
  for (int64_t base = 0; base < total || base == 0; base += fresh) {
    for (int j = K + tid; j < kSortN; j += kThreads) {
      const int64_t idx = base + (j - K);
      keys[j] = idx < total ? src[idx] : 0;
    }
    __syncthreads();
    bitonic_desc_1024(keys);
    if (base + fresh >= total) break;
  }
  const int ns = n_docs < K ? n_docs : K;
  if (tid < K) {
    const uint64_t key = keys[tid];
    if (tid < ns) {
      topk_ids[(int64_t)b * K + tid] = (int32_t)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu));
      topk_scores[(int64_t)b * K + tid] = ord_val((uint32_t)(key >> 32));
    } else {
      topk_ids[(int64_t)b * K + tid] = -1;
      topk_scores[(int64_t)b * K + tid] = -INFINITY;
    }
  }
  if (tid == 0) n_sel[b] = ns;
}

__global__ void fill_f32_kernel(float* p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

}  // namespace

size_t doc_topk_workspace(int32_t B, int32_t n_docs, int32_t top_k) {
  const int64_t n_slices = (n_docs + kSortN - 1) / kSortN;
  return align_up((size_t)B * n_slices * top_k * sizeof(uint64_t), 256);
}

int launch_doc_topk(const float* S, int32_t B, int64_t n_chunks, const int64_t* dco,
                    int32_t n_docs, float* doc_scores, int32_t accumulate, int32_t top_k,
                    uint64_t* cand, int32_t* topk_ids, float* topk_scores, int32_t* n_sel,
                    hipStream_t s) {
  const int32_t n_slices = (n_docs + kSortN - 1) / kSortN;
  hipLaunchKernelGGL(doc_topk1_kernel, dim3(n_slices, B), dim3(kThreads), 0, s, S, n_chunks, dco,
                     n_docs, doc_scores, accumulate, top_k, cand, n_slices);
  MSA_LAUNCH_CHECK("doc_topk1_kernel launch");
  hipLaunchKernelGGL(doc_topk2_kernel, dim3(B), dim3(kThreads), 0, s, cand, n_slices, top_k,
                     n_docs, topk_ids, topk_scores, n_sel);
  MSA_LAUNCH_CHECK("doc_topk2_kernel launch");
  return MSA_OK;
}

int launch_fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  if (n == 0) return MSA_OK;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
  MSA_LAUNCH_CHECK("fill_f32_kernel launch");
  return MSA_OK;
}

}  // namespace msa
