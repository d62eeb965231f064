// msa_doc_reduce + msa_topk: chunk -> document max and top-k selection
// (MSA stage 2, second half).
//
// Method (portal.techblg.uk IRMaD reading, section M, routing bullet):
//   s_i = max_j S_ij over document i's chunks, I = Top-k({s_i}), k = 16.
// Readings: ties go to the lowest document id; with fewer than k documents
// all are selected; a NaN score ranks below every number.
//
// Design.
//   doc_max: a workgroup per (64 documents, query). The documents' chunk
//     range is contiguous; it streams through a 16 KiB LDS tile with
//     coalesced loads (all 16 loads of a thread in flight), then four threads
//     per document max-reduce its chunks from LDS and combine by DPP (NaN
//     propagates, as numpy's max does), max-merge with the previous score
//     when accumulating, and write the document score and the best key of
//     the 64 documents. (Looping a workgroup over several queries, with the
//     next query's loads in flight, measured slower: fewer workgroups.)
//   topk_select: one 1024-thread workgroup per query. Each document becomes
//     the unique 64-bit key (order-preserving uint32 of the score) << 32 |
//     (0xFFFFFFFF − id), so larger key = better document and equal scores
//     fall back to the lower id (NaN maps to the lowest scores).
//     Up to 2048 documents: all keys are sorted. Beyond: the best key of
//     every block of bs documents (bs the largest power of two <= 256 that
//     leaves at least k blocks; combined from doc_max's 64-document maxima),
//     and T = the k-th best block
//     maximum is reached by at least k documents; only blocks whose maximum
//     reaches T — exactly k of them, block maxima being distinct — can hold
//     a key >= T; those keys are ballot-compacted into LDS and sorted, and
//     the head of the list is the answer. Keys are distinct (the id is part
//     of the key), so lists of up to 256 keys are sorted in one step by rank
//     counting (each key's rank = number of larger keys); longer ones by a
//     bitonic network.
//     Fallback (massive ties at T, or more than 2048 blocks):
//     radix select on the uint32 score keys. Four passes
//     over 8-bit digits, most significant first, histogram the keys that
//     share the digits fixed so far (one LDS histogram per wave, rows padded
//     so waves hit different banks) and fix the digit holding the k-th best;
//     after the last pass T is the k-th best key exactly. Every key above T is
//     selected, then the lowest-index keys equal to T (a ballot scan over
//     rounds of 1024 consecutive indices fixes that order). The k
//     winners are ranked by (key desc, id asc) with a k×k comparison, so the
//     output does not depend on thread timing.
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kMaxThreads = 256;
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kHistPitch = 257;
constexpr int kMaxK = 64;
constexpr int kCandCap = 2048;
constexpr int kMaxHot = 512;

__device__ __forceinline__ uint64_t doc_key(float score, int64_t i) {
  return ((uint64_t)ord_key(score) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)x, m);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(x >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

// The 64 documents of a block own one contiguous chunk range (the chunk
// plan keeps documents contiguous). The block streams that range through an
// LDS tile with coalesced loads (all of a thread's loads in flight); four
// threads then share each document, striding over its chunks in the tile,
// and combine with two DPP steps.
constexpr int kDocsPerBlock = 64;
constexpr int kDocTile = 4096;   // chunk scores per LDS tile (16 KiB: 8 blocks per CU)
constexpr int kDocLoads = kDocTile / kMaxThreads;   // 16 loads per thread

__global__ __launch_bounds__(256) void doc_max_kernel(const float* __restrict__ S, int64_t C,
                                                      const int64_t* __restrict__ dco,
                                                      int32_t n_docs,
                                                      float* __restrict__ doc_scores,
                                                      int32_t accumulate,
                                                      uint64_t* __restrict__ bmax) {
  __shared__ float tile[kDocTile];
  __shared__ uint64_t wbest[kMaxThreads / 64];
  const int b = blockIdx.y;
  const int64_t d0 = (int64_t)blockIdx.x * kDocsPerBlock;
  const int64_t d1 = min(d0 + kDocsPerBlock, (int64_t)n_docs);
  const int sub = threadIdx.x & 3;
  const int64_t i = d0 + (threadIdx.x >> 2);
  auto clampc = [&](int64_t c) { return max((int64_t)0, min(c, C)); };
  const int64_t r0 = clampc(dco[d0]), r1 = max(r0, clampc(dco[d1]));
  int64_t c0 = 0, c1 = 0;
  if (i < n_docs) {
    c0 = clampc(dco[i]);
    c1 = max(c0, clampc(dco[i + 1]));
  }
  const float* Sb = S + (int64_t)b * C;
  float s = -INFINITY;
  for (int64_t t0 = r0; t0 < r1; t0 += kDocTile) {
    const int n = (int)min((int64_t)kDocTile, r1 - t0);
    // every load is issued before any store waits on one; slots past the
    // range are neither loaded nor read back
    float v[kDocLoads];
#pragma unroll
    for (int u = 0; u < kDocLoads; ++u) {
      const int c = (int)threadIdx.x + u * kMaxThreads;
      if (c < n) v[u] = Sb[t0 + c];
    }
#pragma unroll
    for (int u = 0; u < kDocLoads; ++u) {
      const int c = (int)threadIdx.x + u * kMaxThreads;
      if (c < n) tile[c] = v[u];
    }
    __syncthreads();
    const int a = (int)(max(c0, t0) - t0), e = (int)(min(c1, t0 + n) - t0);
#pragma unroll 4
    for (int c = a + sub; c < e; c += 4) s = nan_max(s, tile[c]);
    __syncthreads();
  }
  s = nan_max(s, dpp_f<0xB1>(s));   // the document's four threads (a lane quad)
  s = nan_max(s, dpp_f<0x4E>(s));
  uint64_t key = 0;
  if (i < n_docs && sub == 0) {
    float* ds = doc_scores + (int64_t)b * n_docs + i;
    if (accumulate) s = nan_max(*ds, s);
    *ds = s;
    key = doc_key(s, i);
  }
  // the best key of these 64 documents, for the top-k threshold
#pragma unroll
  for (int o = 4; o < 64; o <<= 1) {
    const uint64_t y = shfl_xor_u64(key, o);
    key = y > key ? y : key;
  }
  if ((threadIdx.x & 63) == 0) wbest[threadIdx.x >> 6] = key;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t best = 0;
    for (int w = 0; w < kMaxThreads / 64; ++w) best = wbest[w] > best ? wbest[w] : best;
    bmax[(int64_t)b * gridDim.x + blockIdx.x] = best;
  }
}

// Radix-select fallback: fills sel[0..Ks) with the Ks best 64-bit keys (any
// order). All 1024 threads must call it.
__device__ void radix_select(const float* __restrict__ s, int N, int Ks, uint32_t* hist,
                             uint32_t* tot, uint32_t* wave_eq, uint64_t* sel, int* sel_n,
                             uint32_t* scratch) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  uint32_t& s_digit = scratch[0];
  uint32_t& s_krem = scratch[1];
  uint32_t& n_eq = scratch[2];
  uint32_t prefix = 0;           // digits fixed so far
  uint32_t krem = (uint32_t)Ks;  // how many still to take at or below the prefix
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < kSelWaves * kHistPitch; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < N; i += kSelThreads) {
      const uint32_t key = ord_key(s[i]);
      const bool match = pass == 0 || (key >> (shift + 8)) == prefix;
      if (match) atomicAdd(&hist[wave * kHistPitch + ((key >> shift) & 255u)], 1u);
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t c = 0;
      for (int w = 0; w < kSelWaves; ++w) c += hist[w * kHistPitch + tid];
      tot[tid] = c;
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t acc = 0;
      int d = 255;
      for (; d > 0; --d) {
        if (acc + tot[d] >= krem) break;
        acc += tot[d];
      }
      s_digit = (uint32_t)d;
      s_krem = krem - acc;
    }
    __syncthreads();
    prefix = (prefix << 8) | s_digit;
    krem = s_krem;
    __syncthreads();
  }
  const uint32_t T = prefix;  // the Ks-th best score key; take `krem` of the keys equal to T

  // Keys above T are all taken. Keys equal to T: usually exactly `krem`
  // exist and all are taken; if more tie, the lowest indices win, found by an
  // ordered ballot scan over rounds of 1024 consecutive indices.
  if (tid == 0) { *sel_n = 0; n_eq = 0; }
  __syncthreads();
  for (int i = tid; i < N; i += kSelThreads) {
    const uint32_t key = ord_key(s[i]);
    if (key > T) {
      const int slot = atomicAdd(sel_n, 1);
      if (slot < kMaxK) sel[slot] = ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
    }
    const uint64_t eqm = __ballot(key == T);
    if (lane == 0 && eqm) atomicAdd(&n_eq, (uint32_t)__popcll(eqm));
  }
  __syncthreads();
  const bool all_ties = n_eq <= krem;
  uint32_t carry = 0;
  for (int base = 0; base < N && carry < krem; base += kSelThreads) {
    const int i = base + tid;
    const uint32_t key = i < N ? ord_key(s[i]) : 0u;
    const bool eq = i < N && key == T;
    const uint64_t m = __ballot(eq);
    if (lane == 0) wave_eq[wave] = (uint32_t)__popcll(m);
    __syncthreads();
    uint32_t before = carry, total = 0;
    for (int w = 0; w < kSelWaves; ++w) {
      if (w < wave) before += wave_eq[w];
      total += wave_eq[w];
    }
    before += (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
    if (eq && (all_ties || before < krem)) {
      const int slot = atomicAdd(sel_n, 1);
      if (slot < kMaxK) sel[slot] = ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
    }
    carry += total;
    __syncthreads();
  }
  __syncthreads();
}

// Bitonic sort of n2 (a power of two, <= kCandCap) keys in LDS, descending.
__device__ void bitonic_desc(uint64_t* a, int n2) {
  const int tid = threadIdx.x;
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int p = tid; p < n2 / 2; p += kSelThreads) {
        const int i = 2 * j * (p / j) + (p % j);
        const int l = i + j;
        const bool desc = (i & k) == 0;
        const uint64_t x = a[i], y = a[l];
        if (desc ? (x < y) : (x > y)) { a[i] = y; a[l] = x; }
      }
      __syncthreads();
    }
  }
}

// Sorts n <= kRankMax distinct keys of a[] descending into out[] (a and out
// must not overlap): a key's rank is the number of larger keys. The four
// threads of a lane quad share a key, each counting every fourth key, so the
// serial LDS loop is n / 4 long.
constexpr int kRankMax = kSelThreads / 4;
__device__ void rank_sort_desc(const uint64_t* a, uint64_t* out, int n) {
  const int i = threadIdx.x >> 2, q = threadIdx.x & 3;
  uint64_t x = 0;
  int r = 0;
  if (i < n) {
    x = a[i];
#pragma unroll 8
    for (int j = q; j < n; j += 4) r += a[j] > x ? 1 : 0;
  }
  r += __shfl_xor(r, 1);
  r += __shfl_xor(r, 2);
  if (i < n && q == 0) out[r] = x;
  __syncthreads();
}

// Sorts cand[0..n) descending in place (cand has room for kCandCap keys;
// rank sorting uses the upper half as its output).
__device__ void sort_cand_desc(uint64_t* cand, int n) {
  if (n <= kRankMax) {
    rank_sort_desc(cand, cand + kCandCap / 2, n);
    if (threadIdx.x < n) cand[threadIdx.x] = cand[kCandCap / 2 + threadIdx.x];
    __syncthreads();
    return;
  }
  int n2 = 1;
  while (n2 < n) n2 <<= 1;
  for (int i = n + threadIdx.x; i < n2; i += kSelThreads) cand[i] = 0;
  __syncthreads();
  bitonic_desc(cand, n2);
}

__global__ __launch_bounds__(1024) void topk_select_kernel(const float* __restrict__ doc_scores,
                                                           const uint64_t* __restrict__ bmax64,
                                                           int32_t bs, int32_t N, int32_t K,
                                                           int32_t* __restrict__ topk_ids,
                                                           float* __restrict__ topk_scores,
                                                           int32_t* __restrict__ n_sel) {
  __shared__ uint64_t cand[kCandCap];
  __shared__ uint32_t hist[kSelWaves * kHistPitch];
  __shared__ uint32_t tot[256];
  __shared__ uint32_t wave_eq[kSelWaves];
  __shared__ uint32_t scratch[4];
  __shared__ int hot[kMaxHot];
  __shared__ int n_cand;

  const int tid = threadIdx.x, lane = tid & 63;
  const int b = blockIdx.x;
  const float* s = doc_scores + (int64_t)b * N;
  const int Ks = N < K ? N : K;
  const int n_blocks = (N + bs - 1) / bs;
  const int wave = tid >> 6;

  int cnt = kCandCap + 1;  // forces the fallback unless the fast path applies
  if (N > kCandCap && n_blocks >= K && n_blocks <= kCandCap) {
    // ---- T = K-th best block maximum: at least K documents reach it, and a
    //      document at or above T can only sit in a block whose maximum does
    // block maxima over blocks of bs documents: from doc_max's maxima of 64
    // documents when bs is a multiple of 64, else one wave per block
    const int nb64 = (N + kDocsPerBlock - 1) / kDocsPerBlock;
    const uint64_t* bm = bmax64 + (int64_t)b * nb64;
    const int r = bs / kDocsPerBlock;
    if (r >= 1) {
      for (int j = tid; j < n_blocks; j += kSelThreads) {
        uint64_t key = 0;
#pragma unroll
        for (int q = 0; q < kMaxThreads / kDocsPerBlock; ++q) {
          const int x = j * r + q;
          const uint64_t y = (q < r && x < nb64) ? bm[x] : 0ull;
          key = y > key ? y : key;
        }
        cand[j] = key;
      }
    } else for (int j = wave; j < n_blocks; j += kSelWaves) {
      uint64_t key = 0;
      for (int i = lane; i < bs; i += 64) {
        const int d = j * bs + i;
        if (d < N) {
          const uint64_t k2 = doc_key(s[d], d);
          key = k2 > key ? k2 : key;
        }
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint64_t y = shfl_xor_u64(key, o);
        key = y > key ? y : key;
      }
      if (lane == 0) cand[j] = key;
    }
    if (tid == 0) n_cand = 0;
    __syncthreads();
    sort_cand_desc(cand, n_blocks);
    const uint64_t T = cand[K - 1];
    // block maxima are distinct, so exactly the first K blocks reach T
    const int n_hot = K;
    if (tid < n_hot) hot[tid] = (int)((0xFFFFFFFFu - (uint32_t)(cand[tid] & 0xFFFFFFFFu)) / bs);
    __syncthreads();
    // ---- gather keys >= T from the hot blocks (bs documents each); every
    //      load of a thread is issued before the compaction
    constexpr int kPer = kMaxK * kMaxThreads / kSelThreads;   // bs <= kMaxThreads
    const int total = n_hot * bs;
    uint64_t kk[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int j = u * kSelThreads + tid;
      kk[u] = 0;
      if (j < total) {
        const int64_t i = (int64_t)hot[j / bs] * bs + (j % bs);
        if (i < N) kk[u] = doc_key(s[i], i);
      }
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const bool c = kk[u] >= T && kk[u] != 0;   // kk = 0 past `total`
      const uint64_t m = __ballot(c);
      if (m) {
        int pos0 = 0;
        if (lane == 0) pos0 = atomicAdd(&n_cand, (int)__popcll(m));
        pos0 = __shfl(pos0, 0);
        const int pos = pos0 + (int)__popcll(m & ((1ull << lane) - 1ull));
        if (c && pos < kCandCap / 2) cand[pos] = kk[u];
      }
    }
    __syncthreads();
    cnt = n_cand <= kCandCap / 2 ? n_cand : kCandCap + 1;
  } else if (N <= kCandCap) {
    for (int i = tid; i < N; i += kSelThreads) cand[i] = doc_key(s[i], i);
    cnt = N;
    __syncthreads();
  }
  if (cnt <= kCandCap) {
    sort_cand_desc(cand, cnt);
  } else {
    // massive ties at the threshold (or an unusual shape): radix select into
    // cand[kMaxK..), then rank into cand[0..Ks)
    radix_select(s, N, Ks, hist, tot, wave_eq, cand + kMaxK, &n_cand, scratch);
    if (tid < Ks) {
      const uint64_t e = cand[kMaxK + tid];
      int rank = 0;
      for (int j = 0; j < Ks; ++j) rank += cand[kMaxK + j] > e ? 1 : 0;
      cand[rank] = e;
    }
    __syncthreads();
  }
  if (tid < K) {
    int32_t* ids = topk_ids + (int64_t)b * K;
    float* sc = topk_scores + (int64_t)b * K;
    if (tid < Ks) {
      const uint64_t e = cand[tid];
      ids[tid] = (int32_t)(0xFFFFFFFFu - (uint32_t)(e & 0xFFFFFFFFu));
      sc[tid] = ord_val((uint32_t)(e >> 32));
    } else {
      ids[tid] = -1;
      sc[tid] = -INFINITY;
    }
  }
  if (tid == 0) n_sel[b] = Ks;
}

__global__ void fill_f32_kernel(float* p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

}  // namespace

size_t doc_topk_workspace(int32_t B, int32_t n_docs, int32_t top_k) {
  (void)top_k;
  const int64_t nb64 = (n_docs + kDocsPerBlock - 1) / kDocsPerBlock;
  return align_up((size_t)B * nb64 * sizeof(uint64_t), 256);
}

int launch_doc_topk(const float* S, int32_t B, int64_t n_chunks, const int64_t* dco,
                    int32_t n_docs, float* doc_scores, int32_t accumulate, int32_t top_k,
                    uint64_t* cand, int32_t* topk_ids, float* topk_scores, int32_t* n_sel,
                    hipStream_t s) {
  if (top_k > kMaxK) return fail(MSA_ERR_UNSUPPORTED, "top_k > %d", kMaxK);
  const unsigned blocks = (unsigned)((n_docs + kDocsPerBlock - 1) / kDocsPerBlock);
  hipLaunchKernelGGL(doc_max_kernel, dim3(blocks, B), dim3(kMaxThreads), 0, s, S, n_chunks, dco,
                     n_docs, doc_scores, accumulate, cand);
  MSA_LAUNCH_CHECK("doc_max_kernel launch");
  // threshold blocks: the largest power of two <= 256 documents that still
  // gives at least top_k blocks
  int bs = kMaxThreads;
  while (bs > 1 && (n_docs + bs - 1) / bs < top_k) bs >>= 1;
  hipLaunchKernelGGL(topk_select_kernel, dim3(B), dim3(kSelThreads), 0, s, doc_scores, cand, bs,
                     n_docs, top_k, topk_ids, topk_scores, n_sel);
  MSA_LAUNCH_CHECK("topk_select_kernel launch");
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
