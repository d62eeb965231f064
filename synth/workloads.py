"""Seeded synthetic workloads shaped like the MSA pages' inference setting.

Shapes follow the method's stated hyper-parameters (MSA explainer at
portal.techblg.uk, section M "Materials & Methods", architecture bullet):
64-token chunks, top-16 documents, 8 heads of dimension 128, 18 routed layers,
BF16 caches. Query heads (32, GQA group 4) and every size below follow the five
workloads this library is measured on. The pages evaluate on public QA and
needle suites; none of their items are reproduced here. Random tensors with a
planted "needle" stand in for them.

Nothing here computes any step of the method. Planting works by *layout*: every
token of one chunk of a planted document gets the same router-key vector u, so
the chunk's mean is u itself, and the planted query tokens are u plus Gaussian
noise. Pooled stores (the 16M and 100M workloads) are drawn directly with the
distribution that pooling 64 N(0,1) tokens yields, N(0, 1/64).

All randomness comes from ``torch.Generator`` (tensor values) and
``numpy.random.default_rng`` (lengths and planted ids) seeded from
(seed, stream), so a workload is bit-reproducible on a given torch build.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

H_KV = 8      # KV heads per routed layer
H_R = 8       # router heads
H_Q = 32      # query heads (GQA group of 4)
D = 128       # head dimension
CHUNK = 64    # pooling chunk length P
TOP_K = 16    # documents selected per query
N_LAYERS = 18  # routed layers in the 100M-token store

__all__ = [
    "H_KV", "H_R", "H_Q", "D", "CHUNK", "TOP_K", "N_LAYERS",
    "RawMemory", "PooledMemory", "AttendInputs", "RouteQuery",
    "torch_gen", "np_rng", "randn_bf16", "offsets_from_lengths",
    "lengths_fixed", "lengths_uniform_n", "lengths_until", "counts_until",
    "raw_memory", "pooled_store", "route_query_planted_raw",
    "route_queries_planted_pooled", "attend_inputs",
    "cfg1_tiny", "cfg2_1m", "cfg3_batched", "cfg4_100m", "cfg5_memory",
    "cfg5_round",
]


# ----------------------------------------------------------------------------
# seeding helpers
# ----------------------------------------------------------------------------
def torch_gen(seed: int, stream: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(stream)) & 0x7FFF_FFFF_FFFF)
    return g


def np_rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


def randn_bf16(shape, gen: torch.Generator, device="cpu", std: float = 1.0,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """N(0, std^2) values rounded to bf16, filled in slabs to bound temporaries."""
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    slab = 1 << 28
    for s in range(0, flat.numel(), slab):
        part = flat[s:s + slab]
        tmp = torch.empty(part.shape, dtype=torch.float32, device=out.device)
        tmp.normal_(0.0, std, generator=gen)
        part.copy_(tmp)
        del tmp
    return out


# ----------------------------------------------------------------------------
# ragged document layouts
# ----------------------------------------------------------------------------
def offsets_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=out[1:])
    return out


def lengths_fixed(n_docs: int, length: int) -> np.ndarray:
    return np.full(n_docs, length, dtype=np.int64)


def lengths_uniform_n(rng, n_docs: int, lo: int, hi: int, step: int = 1) -> np.ndarray:
    """n_docs lengths drawn uniformly from {lo, lo+step, ..., hi}."""
    k = (hi - lo) // step + 1
    return lo + step * rng.integers(0, k, size=n_docs, dtype=np.int64)


def lengths_until(rng, total: int, lo: int, hi: int, step: int = 1) -> np.ndarray:
    """Draw lengths uniformly from {lo, lo+step, ..., hi} until ``total`` is
    reached; the last length is trimmed so the lengths sum to ``total``."""
    out = []
    acc = 0
    k = (hi - lo) // step + 1
    while acc < total:
        n = int(lo + step * rng.integers(0, k))
        n = min(n, total - acc)
        out.append(n)
        acc += n
    return np.asarray(out, dtype=np.int64)


def counts_until(rng, total: int, lo: int, hi: int) -> np.ndarray:
    return lengths_until(rng, total, lo, hi, 1)


# ----------------------------------------------------------------------------
# containers
# ----------------------------------------------------------------------------
@dataclass
class RawMemory:
    """Per-token K, V, K^R of a document collection, token-major [T, 8, 128]."""
    K: torch.Tensor
    V: torch.Tensor
    KR: torch.Tensor
    doc_token_offsets: np.ndarray             # int64 [N+1]
    planted: dict = field(default_factory=dict)  # doc -> (chunk in doc, u [8,128] bf16 cpu)

    @property
    def n_docs(self) -> int:
        return len(self.doc_token_offsets) - 1

    @property
    def n_tokens(self) -> int:
        return int(self.doc_token_offsets[-1])


@dataclass
class PooledMemory:
    """A pooled store drawn directly: K̄^R (and optionally K̄, V̄) [C, 8, 128]."""
    KRbar: torch.Tensor                       # [C,8,128] or [layers, C, 8, 128]
    doc_chunk_offsets: np.ndarray             # int64 [N+1]
    Kbar: torch.Tensor | None = None
    Vbar: torch.Tensor | None = None

    @property
    def n_docs(self) -> int:
        return len(self.doc_chunk_offsets) - 1

    @property
    def n_chunks(self) -> int:
        return int(self.doc_chunk_offsets[-1])


@dataclass
class RouteQuery:
    QR: torch.Tensor                          # [B, M, 8, 128]
    planted_docs: list                        # per query: list of doc ids


@dataclass
class AttendInputs:
    Q: torch.Tensor                           # [M, 32, 128]
    K_loc: torch.Tensor                       # [M_loc, 8, 128]
    V_loc: torch.Tensor                       # [M_loc, 8, 128]


# ----------------------------------------------------------------------------
# generic generators
# ----------------------------------------------------------------------------
def raw_memory(lengths, seed: int, device="cpu", n_plant: int = 0,
               plant_docs=None, std: float = 1.0) -> RawMemory:
    """Raw K, V, K^R ~ N(0, std^2) in bf16 for documents of the given lengths.

    ``n_plant`` documents (or the given ``plant_docs``) get one seeded chunk in
    which every K^R token equals one vector u ~ N(0,1)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    offs = offsets_from_lengths(lengths)
    T = int(offs[-1])
    g = torch_gen(seed, 1, device)
    K = randn_bf16((T, H_KV, D), g, device, std)
    V = randn_bf16((T, H_KV, D), g, device, std)
    KR = randn_bf16((T, H_R, D), g, device, std)
    rng = np_rng(seed, 2)
    if plant_docs is None:
        plant_docs = rng.choice(len(lengths), size=n_plant, replace=False) if n_plant else []
    planted = {}
    gu = torch_gen(seed, 3, "cpu")
    for d in [int(x) for x in plant_docs]:
        n_chunks_doc = (int(lengths[d]) + CHUNK - 1) // CHUNK
        c = int(rng.integers(0, n_chunks_doc))
        u = randn_bf16((H_R, D), gu, "cpu")
        t0 = int(offs[d]) + c * CHUNK
        t1 = min(t0 + CHUNK, int(offs[d + 1]))
        KR[t0:t1] = u.to(device).unsqueeze(0)
        planted[d] = (c, u)
    return RawMemory(K, V, KR, offs, planted)


def pooled_store(chunk_counts, seed: int, device="cpu", n_layers: int | None = None,
                 kv_device=None, with_kv: bool = False, kv_pinned: bool = False) -> PooledMemory:
    """K̄^R ~ N(0, 1/64) bf16 drawn directly (optionally one slab per layer)."""
    counts = np.asarray(chunk_counts, dtype=np.int64)
    offs = offsets_from_lengths(counts)
    C = int(offs[-1])
    g = torch_gen(seed, 11, device)
    shape = (C, H_R, D) if n_layers is None else (n_layers, C, H_R, D)
    KRbar = torch.empty(shape, dtype=torch.bfloat16, device=device)
    if n_layers is None:
        randn_bf16(shape, g, device, 0.125, out=KRbar)
    else:
        for l in range(n_layers):
            randn_bf16((C, H_R, D), g, device, 0.125, out=KRbar[l])
    Kbar = Vbar = None
    if with_kv:
        kvd = device if kv_device is None else kv_device
        gk = torch_gen(seed, 12, device)
        Kbar = torch.empty((C, H_KV, D), dtype=torch.bfloat16, device=kvd, pin_memory=kv_pinned)
        Vbar = torch.empty((C, H_KV, D), dtype=torch.bfloat16, device=kvd, pin_memory=kv_pinned)
        slab = 1 << 17
        for dst in (Kbar, Vbar):
            for s in range(0, C, slab):
                e = min(C, s + slab)
                dst[s:e].copy_(randn_bf16((e - s, H_KV, D), gk, device, 0.125))
    return PooledMemory(KRbar, offs, Kbar, Vbar)


def route_query_planted_raw(mem: RawMemory, M: int, seed: int, device="cpu",
                            block: int | None = None, noise: float = 0.3) -> RouteQuery:
    """One query of M router tokens ~ N(0,1); for the b-th planted document a
    block of ``block`` tokens (default M // n_planted) is u_b + noise·N(0,1)."""
    g = torch_gen(seed, 21, "cpu")
    QR = randn_bf16((1, M, H_R, D), g, "cpu")
    docs = sorted(mem.planted.keys())
    if docs:
        blk = block if block is not None else M // len(docs)
        if blk * len(docs) > M:
            raise ValueError("planted blocks do not fit in the query")
        # contiguous blocks from a seeded base offset
        base = int(np_rng(seed, 22).integers(0, M - blk * len(docs) + 1))
        starts = [base + b * blk for b in range(len(docs))]
        for b, d in enumerate(docs):
            u = mem.planted[d][1].float()
            n = torch.empty((blk, H_R, D), dtype=torch.float32)
            n.normal_(0.0, 1.0, generator=g)
            QR[0, starts[b]:starts[b] + blk] = (u.unsqueeze(0) + noise * n).to(torch.bfloat16)
    return RouteQuery(QR.to(device), [docs])


def route_queries_planted_pooled(store: PooledMemory, B: int, per_query: int, seed: int,
                                 device="cpu", layer: int | None = None,
                                 noise: float = 0.3) -> RouteQuery:
    """B single-token queries; query b = sum of ``per_query`` seeded pooled
    router keys (one chunk of each of its planted docs) + noise·N(0,1)."""
    rng = np_rng(seed, 31)
    g = torch_gen(seed, 32, "cpu")
    N = store.n_docs
    offs = store.doc_chunk_offsets
    KR = store.KRbar if layer is None else store.KRbar[layer]
    QR = torch.empty((B, 1, H_R, D), dtype=torch.bfloat16)
    planted = []
    for b in range(B):
        docs = [int(x) for x in rng.choice(N, size=per_query, replace=False)]
        acc = torch.zeros((H_R, D), dtype=torch.float32)
        for d in docs:
            c = int(offs[d]) + int(rng.integers(0, int(offs[d + 1] - offs[d])))
            acc += KR[c].float().cpu()
        n = torch.empty((H_R, D), dtype=torch.float32)
        n.normal_(0.0, 1.0, generator=g)
        QR[b, 0] = (acc + noise * n).to(torch.bfloat16)
        planted.append(sorted(docs))
    return RouteQuery(QR.to(device), planted)


def attend_inputs(M: int, M_loc: int, seed: int, device="cpu", stream: int = 41) -> AttendInputs:
    g = torch_gen(seed, stream, device)
    Q = randn_bf16((M, H_Q, D), g, device)
    K_loc = randn_bf16((M_loc, H_KV, D), g, device)
    V_loc = randn_bf16((M_loc, H_KV, D), g, device)
    return AttendInputs(Q, K_loc, V_loc)


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------
def cfg1_tiny(device="cpu", seed: int = 1):
    """64 docs × 512 tokens (32,768 tokens, 512 chunks), 1 layer; a 64-token
    query (32 Q heads) with 4 planted docs, 16 router tokens each."""
    mem = raw_memory(lengths_fixed(64, 512), seed, device, n_plant=4)
    q = route_query_planted_raw(mem, 64, seed, device)
    att = attend_inputs(64, 64, seed, device)
    return mem, q, att


def cfg2_1m(device="cpu", seed: int = 2, exact_1m: bool = False):
    """1500 docs, lengths uniform on {256, 320, ..., 4096} (≈3.26M tokens), or
    docs drawn from the same law until exactly 2^20 tokens; one needle doc and
    a 128-token query whose seeded 32-token block points at it."""
    rng = np_rng(seed, 0)
    if exact_1m:
        lengths = lengths_until(rng, 1 << 20, 256, 4096, 64)
    else:
        lengths = lengths_uniform_n(rng, 1500, 256, 4096, 64)
    mem = raw_memory(lengths, seed, device, n_plant=1)
    q = route_query_planted_raw(mem, 128, seed, device, block=32)
    att = attend_inputs(128, 128, seed, device)
    return mem, q, att


def cfg3_batched(device="cpu", seed: int = 3, n_chunks: int = 250_000, B: int = 64):
    """250K pooled chunks (docs of 4..64 chunks), 64 single-token queries with
    2 planted docs each."""
    rng = np_rng(seed, 0)
    counts = counts_until(rng, n_chunks, 4, 64)
    store = pooled_store(counts, seed, device)
    q = route_queries_planted_pooled(store, B, 2, seed, device)
    return store, q


def cfg4_100m(device="cpu", seed: int = 4, n_chunks: int = 1_562_500, n_layers: int = N_LAYERS,
              kv_pinned: bool = True, M_loc: int = 129):
    """100M memory tokens: 1,562,500 pooled chunks per layer, router keys for
    ``n_layers`` layers resident on ``device``; K̄/V̄ of one layer (reused by
    every layer) in pinned host memory; one needle per layer; a single decode
    token (32 Q heads) with 128 tokens of history."""
    rng = np_rng(seed, 0)
    counts = counts_until(rng, n_chunks, 4, 64)
    on_gpu = str(device).startswith("cuda")
    store = pooled_store(counts, seed, device, n_layers=n_layers, with_kv=True,
                         kv_device="cpu" if (kv_pinned and on_gpu) else device,
                         kv_pinned=kv_pinned and on_gpu)
    queries = [route_queries_planted_pooled(store, 1, 1, seed + 100 * l, device, layer=l)
               for l in range(n_layers)]
    atts = [attend_inputs(1, M_loc, seed + 100 * l, device) for l in range(n_layers)]
    return store, queries, atts


def cfg5_memory(device="cpu", seed: int = 5, n_tokens: int = 10_000_000, n_queries: int = 32,
                hops: int = 3):
    """10M raw tokens (docs uniform on [256, 8192]); ``n_queries`` × ``hops``
    distinct planted chain documents."""
    rng = np_rng(seed, 0)
    lengths = lengths_until(rng, n_tokens, 256, 8192, 1)
    n_plant = min(n_queries * hops, len(lengths))
    mem = raw_memory(lengths, seed, device, n_plant=n_plant)
    docs = list(mem.planted.keys())
    chains = [docs[q * hops:(q + 1) * hops] for q in range(n_queries)]
    return mem, chains


def cfg5_round(mem: RawMemory, chain_doc: int, query: int, rnd: int, seed: int = 5,
               device="cpu", M_new: int = 256, block: int = 64, noise: float = 0.3):
    """New tokens of one interleave round: Q, K, V, Q^R ~ N(0,1) except one
    seeded 64-token block of Q^R that is u_(chain doc) + noise·N(0,1)."""
    s = seed * 10_000 + query * 10 + rnd
    g = torch_gen(s, 51, "cpu")
    QR = randn_bf16((M_new, H_R, D), g, "cpu")
    rng = np_rng(s, 52)
    t0 = int(rng.integers(0, M_new - block + 1))
    u = mem.planted[chain_doc][1].float()
    n = torch.empty((block, H_R, D), dtype=torch.float32)
    n.normal_(0.0, 1.0, generator=g)
    QR[t0:t0 + block] = (u.unsqueeze(0) + noise * n).to(torch.bfloat16)
    att = attend_inputs(M_new, M_new, s, "cpu", stream=53)
    return (QR.to(device), att.Q.to(device), att.K_loc.to(device), att.V_loc.to(device))
