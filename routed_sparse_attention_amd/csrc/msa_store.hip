// Streaming memory update: a pooled store that grows by whole documents, and
// its files.
//
// Method: pooling is per document (portal.techblg.uk IRMaD reading, section
// M, routing bullet: each document's chunks are pooled on their own), so the
// store of a corpus is the concatenation of its documents' pooled rows, and
// new documents can be appended without re-encoding the others. The pages
// name the re-encoding cost of a changing knowledge base as a limitation and
// incremental encoding as a future direction (paper.rainbus.top, limitations
// and future-directions sections).
//
// Design (host code; the pooling itself is pool_kernel):
//   - append plans the new documents' chunks on the host, writes their
//     absolute chunk offsets into the host mirror and uploads them after the
//     store's current offsets, then pools straight into the store's tail
//     rows (pool_kernel takes absolute offsets and a chunk base), so nothing
//     is staged or copied;
//   - files stream through the caller's staging buffer with synchronous
//     copies; a save goes to "<path>.tmp" and is renamed into place, so a
//     reader never sees a half-written store.
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "msa_internal.h"

namespace msa {
namespace {

constexpr char kMagic[8] = {'M', 'S', 'A', 'S', 'T', 'O', 'R', '1'};
constexpr uint32_t kVersion = 1;
constexpr uint32_t kTensorKR = 1, kTensorK = 2, kTensorV = 4;
constexpr size_t kRowBytes = (size_t)kRowElems * sizeof(uint16_t);
constexpr size_t kMinStaging = (size_t)1 << 20;

struct FileHeader {   // 64 bytes, little-endian
  char magic[8];
  uint32_t version;
  uint32_t header_bytes;
  int32_t n_docs;
  int32_t chunk;
  int64_t n_chunks;
  int32_t heads;
  int32_t head_dim;
  uint32_t tensors;
  int32_t doc_rope_mode;
  float rope_theta;
  uint8_t reserved[12];
};
static_assert(sizeof(FileHeader) == 64, "the store file header is 64 bytes");

struct FileCloser {
  FILE* f = nullptr;
  ~FileCloser() {
    if (f) std::fclose(f);
  }
};

int check_store(const msa_store* st, const char* who) {
  if (st == nullptr) return fail(MSA_ERR_INVALID_ARG, "%s: store is NULL", who);
  if (!st->doc_chunk_offsets || !st->doc_chunk_offsets_h)
    return fail(MSA_ERR_INVALID_ARG, "%s: store offsets are NULL", who);
  if (st->cap_docs < 0 || st->cap_chunks < 0 || st->n_docs < 0 || st->n_chunks < 0 ||
      st->n_docs > st->cap_docs || st->n_chunks > st->cap_chunks)
    return fail(MSA_ERR_SHAPE, "%s: store fill (%d docs, %lld chunks) outside its capacity "
                "(%d, %lld)", who, st->n_docs, (long long)st->n_chunks, st->cap_docs,
                (long long)st->cap_chunks);
  if (st->doc_chunk_offsets_h[st->n_docs] != st->n_chunks)
    return fail(MSA_ERR_SHAPE, "%s: store offsets end at %lld, not at n_chunks=%lld", who,
                (long long)st->doc_chunk_offsets_h[st->n_docs], (long long)st->n_chunks);
  return MSA_OK;
}

uint32_t store_mask(const msa_store* st) {
  return (st->KRbar ? kTensorKR : 0u) | (st->Kbar ? kTensorK : 0u) | (st->Vbar ? kTensorV : 0u);
}

int read_header(FILE* f, const char* path, FileHeader* h) {
  if (std::fread(h, sizeof(*h), 1, f) != 1)
    return fail(MSA_ERR_IO, "store file %s: cannot read the header", path);
  if (std::memcmp(h->magic, kMagic, sizeof(kMagic)) != 0)
    return fail(MSA_ERR_IO, "store file %s: not an MSA store (bad magic)", path);
  if (h->version != kVersion || h->header_bytes != sizeof(FileHeader))
    return fail(MSA_ERR_IO, "store file %s: unsupported version %u / header %u bytes", path,
                h->version, h->header_bytes);
  if (h->n_docs < 0 || h->n_chunks < h->n_docs || h->chunk < 1 || h->heads < 1 ||
      h->head_dim < 1 || (h->tensors & ~7u) != 0)
    return fail(MSA_ERR_IO, "store file %s: malformed header", path);
  return MSA_OK;
}

// The present tensors in file order, with their store pointers.
struct TensorSlot {
  uint32_t bit;
  const char* name;
};
constexpr TensorSlot kOrder[3] = {{kTensorKR, "KRbar"}, {kTensorK, "Kbar"}, {kTensorV, "Vbar"}};

msa_bf16* slot_ptr(const msa_store* st, uint32_t bit) {
  return bit == kTensorKR ? st->KRbar : (bit == kTensorK ? st->Kbar : st->Vbar);
}

}  // namespace
}  // namespace msa

using namespace msa;

extern "C" {

int32_t msa_store_reset(msa_store* st, void* stream) {
  clear_error();
  if (st == nullptr) return fail(MSA_ERR_INVALID_ARG, "store_reset: store is NULL");
  if (!st->doc_chunk_offsets || !st->doc_chunk_offsets_h)
    return fail(MSA_ERR_INVALID_ARG, "store_reset: store offsets are NULL");
  if (st->cap_docs < 0 || st->cap_chunks < 0)
    return fail(MSA_ERR_SHAPE, "store_reset: negative capacity");
  st->doc_chunk_offsets_h[0] = 0;
  MSA_HIP(hipMemcpyAsync(st->doc_chunk_offsets, st->doc_chunk_offsets_h, sizeof(int64_t),
                         hipMemcpyHostToDevice, static_cast<hipStream_t>(stream)));
  st->n_docs = 0;
  st->n_chunks = 0;
  return MSA_OK;
}

int32_t msa_store_append(const msa_dims* d, msa_store* st, const msa_bf16* K, const msa_bf16* V,
                         const msa_bf16* KR, const int64_t* dto, const int64_t* dto_h,
                         int32_t n_new, int64_t n_new_tokens, void* stream) {
  clear_error();
  int rc = check_dims(d);
  if (rc) return rc;
  rc = check_store(st, "store_append");
  if (rc) return rc;
  if ((st->Kbar && !K) || (st->Vbar && !V) || (st->KRbar && !KR))
    return fail(MSA_ERR_INVALID_ARG, "store_append: the store keeps a tensor whose raw input "
                "is NULL");
  if (!dto || !dto_h) return fail(MSA_ERR_INVALID_ARG, "store_append: NULL token offsets");
  MSA_A16("store_append", K);
  MSA_A16("store_append", V);
  MSA_A16("store_append", KR);
  MSA_A16("store_append", st->Kbar);
  MSA_A16("store_append", st->Vbar);
  MSA_A16("store_append", st->KRbar);
  if (n_new < 1) return fail(MSA_ERR_SHAPE, "store_append: n_new=%d must be >= 1", n_new);
  if (dto_h[0] != 0 || dto_h[n_new] != n_new_tokens)
    return fail(MSA_ERR_SHAPE, "store_append: token offsets must run from 0 to n_new_tokens=%lld",
                (long long)n_new_tokens);
  std::vector<int64_t> rel((size_t)n_new + 1);
  rc = msa_plan_chunks(dto_h, n_new, d->chunk, rel.data());
  if (rc) return rc;
  const int64_t new_chunks = rel[(size_t)n_new];
  if ((int64_t)st->n_docs + n_new > st->cap_docs || st->n_chunks + new_chunks > st->cap_chunks)
    return fail(MSA_ERR_SHAPE, "store_append: %d documents / %lld chunks do not fit (store holds "
                "%d / %lld of %d / %lld)", n_new, (long long)new_chunks, st->n_docs,
                (long long)st->n_chunks, st->cap_docs, (long long)st->cap_chunks);
  if ((st->n_chunks + new_chunks) / 8 >= ((int64_t)1 << 31))
    return fail(MSA_ERR_SHAPE, "store_append: too many chunks");
  const void* kb = nullptr;
  const void* vb = nullptr;
  if (st->Kbar && (rc = resolve_any(st->Kbar, &kb, "store Kbar"))) return rc;
  if (st->Vbar && (rc = resolve_any(st->Vbar, &vb, "store Vbar"))) return rc;

  // absolute offsets of the new documents, after the store's current ones
  int64_t* mirror = st->doc_chunk_offsets_h + st->n_docs;
  for (int32_t i = 0; i <= n_new; ++i) mirror[i] = st->n_chunks + rel[(size_t)i];
  hipStream_t s = static_cast<hipStream_t>(stream);
  MSA_HIP(hipMemcpyAsync(st->doc_chunk_offsets + st->n_docs, mirror,
                         ((size_t)n_new + 1) * sizeof(int64_t), hipMemcpyHostToDevice, s));
  PoolArgs a;
  a.K = K; a.V = V; a.KR = KR;
  a.dto = dto;
  a.dco = st->doc_chunk_offsets + st->n_docs;
  a.n_docs = n_new; a.n_tokens = n_new_tokens; a.n_chunks = new_chunks; a.chunk = d->chunk;
  a.chunk_base = st->n_chunks;
  a.theta = (double)d->rope_theta; a.rope_mode = d->doc_rope_mode;
  a.Kbar = static_cast<uint16_t*>(const_cast<void*>(kb));
  a.Vbar = static_cast<uint16_t*>(const_cast<void*>(vb));
  a.KRbar = st->KRbar;
  rc = launch_pool(a, s);
  if (rc) return rc;
  st->n_docs += n_new;
  st->n_chunks += new_chunks;
  return MSA_OK;
}

int32_t msa_store_file_info(const char* path, int32_t* n_docs, int64_t* n_chunks,
                            uint32_t* tensor_mask) {
  clear_error();
  if (!path) return fail(MSA_ERR_INVALID_ARG, "store_file_info: path is NULL");
  FileCloser fc;
  fc.f = std::fopen(path, "rb");
  if (!fc.f) return fail(MSA_ERR_IO, "store file %s: cannot open", path);
  FileHeader h;
  const int rc = read_header(fc.f, path, &h);
  if (rc) return rc;
  if (n_docs) *n_docs = h.n_docs;
  if (n_chunks) *n_chunks = h.n_chunks;
  if (tensor_mask) *tensor_mask = h.tensors;
  return MSA_OK;
}

int32_t msa_store_save(const msa_dims* d, const msa_store* st, const char* path, void* staging_h,
                       size_t staging_bytes) {
  clear_error();
  int rc = check_dims(d);
  if (rc) return rc;
  rc = check_store(st, "store_save");
  if (rc) return rc;
  if (!path) return fail(MSA_ERR_INVALID_ARG, "store_save: path is NULL");
  if (!staging_h || staging_bytes < kMinStaging)
    return fail(MSA_ERR_INVALID_ARG, "store_save: staging buffer of at least 1 MiB required");
  MSA_HIP(hipDeviceSynchronize());   // every pending write to the store has landed

  FileHeader h;
  std::memset(&h, 0, sizeof(h));
  std::memcpy(h.magic, kMagic, sizeof(kMagic));
  h.version = kVersion;
  h.header_bytes = sizeof(FileHeader);
  h.n_docs = st->n_docs;
  h.chunk = d->chunk;
  h.n_chunks = st->n_chunks;
  h.heads = kHeads;
  h.head_dim = kDim;
  h.tensors = store_mask(st);
  h.doc_rope_mode = d->doc_rope_mode;
  h.rope_theta = d->rope_theta;

  std::string tmp = std::string(path) + ".tmp";
  {
    FileCloser fc;
    fc.f = std::fopen(tmp.c_str(), "wb");
    if (!fc.f) return fail(MSA_ERR_IO, "store file %s: cannot create", tmp.c_str());
    if (std::fwrite(&h, sizeof(h), 1, fc.f) != 1 ||
        std::fwrite(st->doc_chunk_offsets_h, sizeof(int64_t), (size_t)st->n_docs + 1, fc.f) !=
            (size_t)st->n_docs + 1)
      return fail(MSA_ERR_IO, "store file %s: write failed", tmp.c_str());
    const size_t bytes = (size_t)st->n_chunks * kRowBytes;
    for (const TensorSlot& ts : kOrder) {
      const char* src = reinterpret_cast<const char*>(slot_ptr(st, ts.bit));
      if (!src) continue;
      for (size_t off = 0; off < bytes; off += staging_bytes) {
        const size_t n = bytes - off < staging_bytes ? bytes - off : staging_bytes;
        MSA_HIP(hipMemcpy(staging_h, src + off, n, hipMemcpyDefault));
        if (std::fwrite(staging_h, 1, n, fc.f) != n)
          return fail(MSA_ERR_IO, "store file %s: write failed (%s)", tmp.c_str(), ts.name);
      }
    }
    const int closed = std::fclose(fc.f);
    fc.f = nullptr;
    if (closed != 0) return fail(MSA_ERR_IO, "store file %s: close failed", tmp.c_str());
  }
  if (std::rename(tmp.c_str(), path) != 0)
    return fail(MSA_ERR_IO, "store file %s: cannot rename into place", path);
  return MSA_OK;
}

int32_t msa_store_load(const msa_dims* d, msa_store* st, const char* path, void* staging_h,
                       size_t staging_bytes) {
  clear_error();
  int rc = check_dims(d);
  if (rc) return rc;
  rc = check_store(st, "store_load");
  if (rc) return rc;
  if (!path) return fail(MSA_ERR_INVALID_ARG, "store_load: path is NULL");
  if (!staging_h || staging_bytes < kMinStaging)
    return fail(MSA_ERR_INVALID_ARG, "store_load: staging buffer of at least 1 MiB required");
  FileCloser fc;
  fc.f = std::fopen(path, "rb");
  if (!fc.f) return fail(MSA_ERR_IO, "store file %s: cannot open", path);
  FileHeader h;
  rc = read_header(fc.f, path, &h);
  if (rc) return rc;
  if (h.chunk != d->chunk || h.heads != kHeads || h.head_dim != kDim)
    return fail(MSA_ERR_SHAPE, "store file %s: chunk %d, %d heads × %d does not match the dims",
                path, h.chunk, h.heads, h.head_dim);
  const uint32_t want = store_mask(st);
  if ((want & ~h.tensors) != 0)
    return fail(MSA_ERR_SHAPE, "store file %s: holds tensors 0x%x, the store wants 0x%x", path,
                h.tensors, want);
  if (st->Kbar && (h.doc_rope_mode != d->doc_rope_mode || h.rope_theta != d->rope_theta))
    return fail(MSA_ERR_SHAPE, "store file %s: K̄ was pooled with doc_rope_mode %d, theta %g",
                path, h.doc_rope_mode, (double)h.rope_theta);
  if (h.n_docs > st->cap_docs || h.n_chunks > st->cap_chunks)
    return fail(MSA_ERR_SHAPE, "store file %s: %d documents / %lld chunks exceed the capacity",
                path, h.n_docs, (long long)h.n_chunks);
  std::vector<int64_t> offs((size_t)h.n_docs + 1);
  if (std::fread(offs.data(), sizeof(int64_t), offs.size(), fc.f) != offs.size())
    return fail(MSA_ERR_IO, "store file %s: truncated offsets", path);
  if (offs[0] != 0 || offs[(size_t)h.n_docs] != h.n_chunks)
    return fail(MSA_ERR_IO, "store file %s: offsets do not run from 0 to n_chunks", path);
  for (int32_t i = 0; i < h.n_docs; ++i)
    if (offs[(size_t)i + 1] <= offs[(size_t)i])
      return fail(MSA_ERR_IO, "store file %s: document %d has no chunk", path, i);
  MSA_HIP(hipDeviceSynchronize());   // nothing in flight still uses the store

  // From here on the store's rows are overwritten: a failure leaves it empty.
  st->n_docs = 0;
  st->n_chunks = 0;
  st->doc_chunk_offsets_h[0] = 0;
  const size_t bytes = (size_t)h.n_chunks * kRowBytes;
  for (const TensorSlot& ts : kOrder) {
    if (!(h.tensors & ts.bit)) continue;
    char* dst = reinterpret_cast<char*>(slot_ptr(st, ts.bit));
    if (!(want & ts.bit)) {
      if (std::fseek(fc.f, (long)bytes, SEEK_CUR) != 0)
        return fail(MSA_ERR_IO, "store file %s: truncated (%s)", path, ts.name);
      continue;
    }
    for (size_t off = 0; off < bytes; off += staging_bytes) {
      const size_t n = bytes - off < staging_bytes ? bytes - off : staging_bytes;
      if (std::fread(staging_h, 1, n, fc.f) != n)
        return fail(MSA_ERR_IO, "store file %s: truncated (%s)", path, ts.name);
      MSA_HIP(hipMemcpy(dst + off, staging_h, n, hipMemcpyDefault));
    }
  }
  std::memcpy(st->doc_chunk_offsets_h, offs.data(), offs.size() * sizeof(int64_t));
  MSA_HIP(hipMemcpy(st->doc_chunk_offsets, offs.data(), offs.size() * sizeof(int64_t),
                    hipMemcpyHostToDevice));
  st->n_docs = h.n_docs;
  st->n_chunks = h.n_chunks;
  return MSA_OK;
}

}  // extern "C"
