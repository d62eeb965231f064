"""MI355X-native hot path of Memory Sparse Attention (MSA).

The compute lives in ``libmsa.so`` (hand-written HIP for gfx950, C ABI in
``include/msa.h``); this package is its ctypes binding. Stages:
``encode_pool`` (chunk mean-pooling with document RoPE), ``route_topk``
(cosine routing, document max, top-k), ``sparse_attend`` (assembly, global
RoPE, GQA attention), ``Interleave`` (Memory Interleave rounds), ``InterleaveBatch`` (rounds of
several queries with one batched routing scan),
``Store`` (a pooled store that grows by whole documents, with save/load) and
``route_aux_loss`` (the router's auxiliary contrastive loss and its gradient).
"""
from ._lib import (  # noqa: F401
    DOC_ROPE_CHUNK, DOC_ROPE_TOKEN, EXPORTED, LIB_PATH, NOALLOC_SCRATCH_BYTES, STORE_K, STORE_KR, STORE_V,
    TOKEN_REDUCE_MAX, TOKEN_REDUCE_MEAN, Dims, Interleave, InterleaveBatch, MsaError, Store, dims, encode_pool,
    lib, plan_chunks, route_aux_loss, route_topk, route_topk_noalloc, route_scores, route_topk_workspace, select_topk, sparse_attend,
    sparse_attend_batch, sparse_attend_workspace, store_file_info,
)
