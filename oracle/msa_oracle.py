"""MSA oracle: a plain, slow, fp64 CPU implementation of the MSA inference path.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It imports nothing
from the HIP library or its binding, and the library never imports it.

Sources (the pages describing "MSA: Memory Sparse Attention", arXiv 2603.23516):
  [rainbus]  paper.rainbus.top/paper/2603.23516 — "方法步骤详情" (method steps)
             and "核心方法" (core method) sections.
  [techblg]  portal.techblg.uk IRMaD reading — section "M. Materials & Methods":
             the architecture bullet (P=64, top-16, 8 heads × 128, 18 layers),
             the routing/sparse-attention bullet (the only explicit formulas),
             the positional-encoding bullet (document-wise and global RoPE),
             the three-stage inference bullet, the Memory Parallel bullet
             (BF16 caches) and the Memory Interleave bullet.
  [chooseai] chooseai.io/news/2962 — sections 2.1 (mechanism), 2.2 (document
             RoPE), 2.3 (KV compression), 2.4 (Memory Interleave).
  [zhichai]  zhichai.net/topic/177169529 — "关键技术细节" 1 (Parallel/Global RoPE).

Everything is float64 (bf16 inputs are decoded exactly). Where the pages leave
a step open, the reading taken is stated at the function; the same list is
kept with the design notes of the repository.

Array conventions: bf16 tensors are numpy ``uint16`` bit patterns, token-major
``[T, H, 128]``; pooled tensors are ``[C, H, 128]``; offsets are int64 CSR.
"""
from __future__ import annotations

import math

import numpy as np

# Hyper-parameters fixed by the pages ([techblg] §M architecture bullet;
# [rainbus] method steps: chunk P=64, k=16).
CHUNK = 64
TOP_K = 16
N_KV_HEADS = 8
N_ROUTER_HEADS = 8
HEAD_DIM = 128
N_ROUTED_LAYERS = 18
# Not on the pages (readings): 32 query heads (GQA group 4) from the measured
# workloads, RoPE base 1e6, cosine norm clamp 1e-6.
N_Q_HEADS = 32
ROPE_THETA = 1.0e6
NORM_EPS = 1.0e-6

TOKEN_REDUCE_MAX = 0
TOKEN_REDUCE_MEAN = 1
DOC_ROPE_TOKEN = 0
DOC_ROPE_CHUNK = 1


# ----------------------------------------------------------------------------
# bf16 <-> float64 (the caches are BF16: [techblg] §M Memory Parallel bullet)
# ----------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """Exact decode: a bf16 pattern is the top half of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """Round float64 to the nearest bf16 (8 significant bits), ties to even.

    Written from the definition: x = m·2^e with 0.5 <= |m| < 1, keep 8 bits of
    m with round-half-even (``np.rint``), all exact in float64. Below the
    smallest normal (2^-126) the quantum is fixed at 2^-133 (subnormals).
    Values beyond the largest finite bf16 become ±inf; NaN stays NaN."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    m, e = np.frexp(x)
    normal = np.abs(x) >= 2.0 ** -126
    out[normal] = np.ldexp(np.rint(np.ldexp(m[normal], 8)), e[normal] - 8)
    sub = ~normal
    out[sub] = np.rint(x[sub] * 2.0 ** 133) * 2.0 ** -133
    max_bf16 = (2.0 - 2.0 ** -7) * 2.0 ** 127
    out = np.where(np.abs(out) > max_bf16, np.copysign(np.inf, out), out)
    out = np.where(np.isnan(x), np.nan, out)
    f32 = out.astype(np.float32)          # exact: every value is a bf16 value
    return (f32.view(np.uint32) >> 16).astype(np.uint16)


def bf16_ord(bits) -> np.ndarray:
    """Monotone integer map of bf16 patterns (for ulp distances)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    return np.where(b & 0x8000, 0x8000 - b, b)


# ----------------------------------------------------------------------------
# step 1: chunk plan — each document split into fixed 64-token chunks
# ([chooseai] §2.1 "分块压缩"; [techblg] lay summary ③)
# ----------------------------------------------------------------------------
def plan_chunks(doc_token_offsets, chunk: int = CHUNK) -> np.ndarray:
    """doc_chunk_offsets: document i owns chunks [dco[i], dco[i+1]); it has
    ceil(n_i / chunk) chunks (the last may be partial). A chunk never spans
    two documents. Every document must hold at least one token."""
    offs = np.asarray(doc_token_offsets, dtype=np.int64)
    n = np.diff(offs)
    if np.any(n < 1):
        raise ValueError("every document needs at least one token")
    counts = [(int(L) + chunk - 1) // chunk for L in n]
    out = np.zeros(len(counts) + 1, dtype=np.int64)
    out[1:] = np.cumsum(counts)
    return out


# ----------------------------------------------------------------------------
# RoPE ([techblg] §M positional-encoding bullet; [zhichai] 关键技术细节 1)
# Reading: rotate-half pairs (m, m+64), frequency ω_m = θ^(-2m/128).
# ----------------------------------------------------------------------------
def rope_rotate(x, positions, theta: float = ROPE_THETA) -> np.ndarray:
    """Rotate every head of x [n, H, D] (float64) by its token's position.

    Pair (x_m, x_{m+D/2}) at position t turns by the angle t·ω_m:
        x'_m       = x_m·cos(tω_m) − x_{m+D/2}·sin(tω_m)
        x'_{m+D/2} = x_{m+D/2}·cos(tω_m) + x_m·sin(tω_m)
    """
    x = np.asarray(x, dtype=np.float64)
    n, H, Dh = x.shape
    half = Dh // 2
    omega = theta ** (-2.0 * np.arange(half, dtype=np.float64) / Dh)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * omega[None, :]  # [n, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


# ----------------------------------------------------------------------------
# step 2+3: document RoPE and chunk mean-pooling φ
# ([techblg] §M routing bullet: K̄=φ(K), V̄=φ(V), K̄^R=φ(K^R);
#  [techblg] §M positional bullet: positions restart at 0 in every document;
#  [rainbus] method steps Stage 1: chunk mean-pooling with P=64)
# Readings: K is rotated at its document-local token position before pooling
# (DOC_ROPE_TOKEN) — or, as the switchable alternative, the pooled chunk is
# rotated at its chunk index (DOC_ROPE_CHUNK). V and K^R are not rotated.
# A partial last chunk is divided by its own token count. Output rounds to
# bf16 (the caches are BF16).
# ----------------------------------------------------------------------------
def pool(K, V, KR, doc_token_offsets, chunk: int = CHUNK, theta: float = ROPE_THETA,
         doc_rope_mode: int = DOC_ROPE_TOKEN, docs=None):
    """Returns (Kbar, Vbar, KRbar) as bf16 patterns [C, H, D] and the chunk
    offsets. ``docs`` restricts the work to a subset of documents (their
    chunks are returned in document order, with matching offsets)."""
    offs = np.asarray(doc_token_offsets, dtype=np.int64)
    dco_all = plan_chunks(offs, chunk)
    doc_list = range(len(offs) - 1) if docs is None else list(docs)
    outs = ([], [], [])
    sub_offs = [0]
    for i in doc_list:
        t0, t1 = int(offs[i]), int(offs[i + 1])
        k = bf16_to_f64(K[t0:t1])
        v = bf16_to_f64(V[t0:t1])
        kr = bf16_to_f64(KR[t0:t1])
        local_pos = np.arange(t1 - t0)
        if doc_rope_mode == DOC_ROPE_TOKEN:
            k = rope_rotate(k, local_pos, theta)
        n_ch = int(dco_all[i + 1] - dco_all[i])
        for c in range(n_ch):
            a, b = c * chunk, min((c + 1) * chunk, t1 - t0)
            kbar = k[a:b].sum(axis=0) / (b - a)
            if doc_rope_mode == DOC_ROPE_CHUNK:
                kbar = rope_rotate(kbar[None], np.array([c]), theta)[0]
            outs[0].append(f64_to_bf16(kbar))
            outs[1].append(f64_to_bf16(v[a:b].sum(axis=0) / (b - a)))
            outs[2].append(f64_to_bf16(kr[a:b].sum(axis=0) / (b - a)))
        sub_offs.append(sub_offs[-1] + n_ch)
    H, Dh = np.asarray(K).shape[1:]
    stack = [np.stack(o) if o else np.zeros((0, H, Dh), np.uint16) for o in outs]
    dco = dco_all if docs is None else np.asarray(sub_offs, dtype=np.int64)
    return stack[0], stack[1], stack[2], dco


# ----------------------------------------------------------------------------
# step 4+5: cosine routing score per chunk
# ([techblg] §M routing bullet: S_ij = max_t( mean_h cos((Q^R_h)_t, K̄^R_ij,h) );
#  [rainbus] core method: per-head router keys, cosine relevance)
# Readings: a norm is clamped at 1e-6 before dividing; the token reduction is
# the max (the explicit formula) or, switchably, the mean.
# ----------------------------------------------------------------------------
def _unit(x):
    n = np.sqrt((x * x).sum(axis=-1, keepdims=True))
    return x / np.maximum(n, NORM_EPS)


def token_chunk_scores(QR, KRbar) -> np.ndarray:
    """S_tc = mean over heads of cos(Q^R_{t,h}, K̄^R_{c,h}); QR [M,H,D],
    KRbar [C,H,D] (bf16 patterns) → float64 [M, C]."""
    q = _unit(bf16_to_f64(QR))            # [M,H,D]
    k = _unit(bf16_to_f64(KRbar))         # [C,H,D]
    H = q.shape[1]
    cos = np.einsum("mhd,chd->mch", q, k)  # per-head cosines
    return cos.sum(axis=-1) / H


def chunk_scores(QR, KRbar, token_reduce: int = TOKEN_REDUCE_MAX) -> np.ndarray:
    """S_c: reduce S_tc over the query's tokens (max, or mean)."""
    S = token_chunk_scores(QR, KRbar)
    if token_reduce == TOKEN_REDUCE_MAX:
        return S.max(axis=0)
    return S.mean(axis=0)


# ----------------------------------------------------------------------------
# step 6: chunk -> document ([techblg] §M routing bullet: s_i = max_j S_ij)
# ----------------------------------------------------------------------------
def doc_scores(S_c, doc_chunk_offsets) -> np.ndarray:
    dco = np.asarray(doc_chunk_offsets, dtype=np.int64)
    S_c = np.asarray(S_c, dtype=np.float64)
    return np.array([S_c[dco[i]:dco[i + 1]].max() for i in range(len(dco) - 1)],
                    dtype=np.float64)


# ----------------------------------------------------------------------------
# step 7: Top-k ([techblg] §M routing bullet: I = Top-k({s_i}), k = 16)
# Readings: ties go to the lowest document id; with N < k all N are taken;
# a NaN score ranks after every number.
# ----------------------------------------------------------------------------
def topk(s, k: int = TOP_K):
    """Returns (ids int64 [n_sel], scores float64 [n_sel], margins float64
    [n_sel]) where margins[r] = s_(r) − s_(r+1) (inf past the last doc)."""
    s = np.asarray(s, dtype=np.float64)
    order = sorted(range(len(s)), key=lambda i: (bool(np.isnan(s[i])), -s[i] if not np.isnan(s[i]) else 0.0, i))
    n_sel = min(k, len(s))
    ids = np.array(order[:n_sel], dtype=np.int64)
    ranked = s[np.array(order, dtype=np.int64)] if len(order) else np.zeros(0)
    margins = np.empty(n_sel, dtype=np.float64)
    for r in range(n_sel):
        margins[r] = ranked[r] - ranked[r + 1] if r + 1 < len(ranked) else np.inf
    return ids, ranked[:n_sel].copy(), margins


def route_topk(QR, KRbar, doc_chunk_offsets, k: int = TOP_K,
               token_reduce: int = TOKEN_REDUCE_MAX, prev_doc_scores=None):
    """Stage 2 for one query: chunk scores → doc scores (max-merged into
    ``prev_doc_scores`` when given) → Top-k. Returns (doc_scores, ids, scores, margins)."""
    s = doc_scores(chunk_scores(QR, KRbar, token_reduce), doc_chunk_offsets)
    if prev_doc_scores is not None:
        s = np.maximum(np.asarray(prev_doc_scores, dtype=np.float64), s)
    ids, sc, mg = topk(s, k)
    return s, ids, sc, mg


# ----------------------------------------------------------------------------
# steps 8-10: context assembly, global RoPE, sparse attention
# ([techblg] §M routing bullet: K_ctx=[{K̄_i}_{i∈I}; K_q], V_ctx likewise,
#  Output = Attention(Q_q, K_ctx, V_ctx);
#  [techblg] §M positional bullet: the active context uses global RoPE with
#  query positions offset from k, the number of Top-k compressed entries;
#  [chooseai] §2.2; [zhichai] 关键技术细节 1 "start index offset k")
# Readings: pos0 = n_sel (k, or N when N < k); local token v sits at pos0+v;
# the M query tokens are the last M of the M_loc local tokens; memory chunks
# are fully visible, local keys causal; scale 1/sqrt(D); q head h reads KV
# head h // (Hq/Hkv); memory chunks enter in rank order.
# ----------------------------------------------------------------------------
def assemble(Kbar, Vbar, doc_chunk_offsets, sel_ids):
    dco = np.asarray(doc_chunk_offsets, dtype=np.int64)
    rows = np.concatenate([np.arange(dco[i], dco[i + 1]) for i in sel_ids]) if len(sel_ids) \
        else np.zeros(0, dtype=np.int64)
    return np.asarray(Kbar)[rows], np.asarray(Vbar)[rows], rows


def sparse_attend(Q, K_loc, V_loc, Kbar, Vbar, doc_chunk_offsets, sel_ids, pos0=None,
                  k_loc_rotated: bool = False, theta: float = ROPE_THETA) -> np.ndarray:
    """Q [M,Hq,D], K_loc/V_loc [M_loc,Hkv,D], Kbar/Vbar [C,Hkv,D] (bf16
    patterns) → output float64 [M, Hq, D]."""
    M, Hq, Dh = np.asarray(Q).shape
    M_loc, Hkv, _ = np.asarray(K_loc).shape
    if M > M_loc:
        raise ValueError("the query tokens must be part of the local context")
    sel_ids = list(sel_ids)
    if pos0 is None:
        pos0 = len(sel_ids)
    kmem, vmem, _ = assemble(Kbar, Vbar, doc_chunk_offsets, sel_ids)
    kmem = bf16_to_f64(kmem) if len(kmem) else np.zeros((0, Hkv, Dh))
    vmem = bf16_to_f64(vmem) if len(vmem) else np.zeros((0, Hkv, Dh))
    q_local_idx = np.arange(M_loc - M, M_loc)
    q = rope_rotate(bf16_to_f64(Q), pos0 + q_local_idx, theta)
    kl = bf16_to_f64(K_loc)
    if not k_loc_rotated:
        kl = rope_rotate(kl, pos0 + np.arange(M_loc), theta)
    vl = bf16_to_f64(V_loc)
    group = Hq // Hkv
    scale = 1.0 / math.sqrt(Dh)
    out = np.zeros((M, Hq, Dh), dtype=np.float64)
    for u in range(M):
        n_vis = q_local_idx[u] + 1               # local keys 0..j_u
        for h in range(Hq):
            g = h // group
            keys = np.concatenate([kmem[:, g, :], kl[:n_vis, g, :]], axis=0)
            vals = np.concatenate([vmem[:, g, :], vl[:n_vis, g, :]], axis=0)
            logits = keys @ q[u, h] * scale
            p = np.exp(logits - logits.max())
            p /= p.sum()
            out[u, h] = p @ vals
    return out


# ----------------------------------------------------------------------------
# step 11: Memory Interleave ([techblg] §M Memory Interleave bullet;
# [rainbus] method steps; [chooseai] §2.4)
# The pages loop route → assemble → generate, appending new context each
# round. Reading: the appended tokens join the active context; the running
# document scores are max-merged with the new tokens' scores (equal to
# re-routing every active token under the max reduction); then top-k and
# attention for the new tokens over [selected memory; all local tokens].
# ----------------------------------------------------------------------------
class InterleaveState:
    def __init__(self, n_docs: int, Hkv: int = N_KV_HEADS, Dh: int = HEAD_DIM):
        self.doc_scores = np.full(n_docs, -np.inf)
        self.K_loc = np.zeros((0, Hkv, Dh), dtype=np.uint16)
        self.V_loc = np.zeros((0, Hkv, Dh), dtype=np.uint16)
        self.QR_all = None


def interleave_step(state: InterleaveState, Q_new, K_new, V_new, QR_new, KRbar, Kbar, Vbar,
                    doc_chunk_offsets, k: int = TOP_K, theta: float = ROPE_THETA):
    s, ids, sc, mg = route_topk(QR_new, KRbar, doc_chunk_offsets, k,
                                TOKEN_REDUCE_MAX, prev_doc_scores=state.doc_scores)
    state.doc_scores = s
    state.K_loc = np.concatenate([state.K_loc, np.asarray(K_new)], axis=0)
    state.V_loc = np.concatenate([state.V_loc, np.asarray(V_new)], axis=0)
    state.QR_all = np.asarray(QR_new) if state.QR_all is None else \
        np.concatenate([state.QR_all, np.asarray(QR_new)], axis=0)
    out = sparse_attend(Q_new, state.K_loc, state.V_loc, Kbar, Vbar, doc_chunk_offsets,
                        ids, None, False, theta)
    return ids, sc, mg, out


# ----------------------------------------------------------------------------
# sizing ([techblg] §M Memory Parallel bullet: 100M tokens, P=64, 8 heads ×
# 128, 18 layers, BF16)
# ----------------------------------------------------------------------------
def store_bytes(n_tokens: int, chunk: int = CHUNK, heads: int = N_ROUTER_HEADS,
                head_dim: int = HEAD_DIM, layers: int = N_ROUTED_LAYERS, bytes_per: int = 2) -> int:
    """Bytes of one pooled tensor (K̄, V̄ or K̄^R) over all routed layers."""
    return (n_tokens // chunk) * heads * head_dim * bytes_per * layers


# ----------------------------------------------------------------------------
# Router supervision: the auxiliary contrastive loss and its gradient
# ([techblg] §M training-data bullet: L_aux = −(1/|P|) Σ_i log[ exp(s_i⁺/τ) /
#  (exp(s_i⁺/τ) + Σ_j exp(s_ij⁻/τ)) ] supervises every layer's router; the
#  temperature τ is fixed but its value is not given).
# Readings: s are the query's routing document scores (step 6: max over a
# document's chunks of the max over query tokens of the head-mean cosine); P
# is the query's set of positive documents and the negatives of every
# positive are all other documents of the store; τ is a parameter. Through
# the two maxima the gradient reaches one (chunk, token) pair per document:
# the first chunk (lowest index) attaining the document score and, in it, the
# first token (lowest index) attaining the chunk score. A norm at or below the
# clamp contributes x / eps, so its gradient is the plain k̂ / eps (or q̂ / eps).
# ----------------------------------------------------------------------------
def aux_loss_f64(q, k, doc_chunk_offsets, positives, tau: float, eps: float = NORM_EPS,
                 choice=None):
    """One query on float64 arrays: q [M,H,D] (its router tokens), k [C,H,D]
    (the pooled router keys). Returns (loss, dq [M,H,D], dk [C,H,D], s [N],
    c_star [N], t_star [N], gaps [N]) where gaps[i] is the smaller of the
    margins that fix c_star[i] and t_star[i] (inf where unique by size).
    ``choice`` = (c_star, t_star) evaluates the loss and gradient at given
    (chunk, token) pairs instead of the first maxima (s_i is then the score
    at that pair) — another element of the subgradient where maxima tie."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    dco = np.asarray(doc_chunk_offsets, dtype=np.int64)
    M, H, _ = q.shape
    N = len(dco) - 1
    rq = np.sqrt((q * q).sum(axis=-1))                  # [M,H]
    rk = np.sqrt((k * k).sum(axis=-1))                  # [C,H]
    nq, nk = np.maximum(rq, eps), np.maximum(rk, eps)
    qh, kh = q / nq[..., None], k / nk[..., None]
    cos = np.einsum("mhd,chd->mch", qh, kh)              # [M,C,H]
    S = cos.sum(axis=-1) / H                             # [M,C]
    Sc = S.max(axis=0)                                   # [C]
    s = np.empty(N)
    c_star = np.empty(N, dtype=np.int64)
    t_star = np.empty(N, dtype=np.int64)
    gaps = np.full(N, np.inf)
    for i in range(N):
        seg = Sc[dco[i]:dco[i + 1]]
        j = int(np.argmax(seg))                          # first maximum
        c = int(dco[i]) + j
        t = int(np.argmax(S[:, c]))                      # first maximum
        if choice is not None:
            c, t = int(choice[0][i]), int(choice[1][i])
        s[i], c_star[i], t_star[i] = S[t, c], c, t
        if len(seg) > 1:
            gaps[i] = min(gaps[i], seg[j] - np.max(np.delete(seg, j)))
        if M > 1:
            gaps[i] = min(gaps[i], S[t, c] - np.max(np.delete(S[:, c], t)))
    P = sorted(set(int(x) for x in positives))
    neg = np.ones(N, dtype=bool)
    neg[P] = False
    a = s / tau
    e = np.exp(a - a.max())                              # shared shift
    z_neg = e[neg].sum()
    loss = 0.0
    ds = np.zeros(N)
    for i in P:
        z = e[i] + z_neg
        loss -= math.log(e[i] / z)
        ds[i] -= (1.0 - e[i] / z) / tau
        ds[neg] += e[neg] / z / tau
    loss /= len(P)
    ds /= len(P)
    # chain rule: ds_i → the head-mean cosine at (t*, c*) → each head's cosine
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    for i in range(N):
        g = ds[i] / H
        c, t = c_star[i], t_star[i]
        ch = cos[t, c]                                   # [H]
        gq = np.where((rq[t] > eps)[:, None], kh[c] - ch[:, None] * qh[t], kh[c]) / nq[t][:, None]
        gk = np.where((rk[c] > eps)[:, None], qh[t] - ch[:, None] * kh[c], qh[t]) / nk[c][:, None]
        dq[t] += g * gq
        dk[c] += g * gk
    return loss, dq, dk, s, c_star, t_star, gaps


def route_aux_loss(QR, KRbar, doc_chunk_offsets, positives, tau: float, choice=None):
    """B queries: QR [B,M,H,D] and KRbar [C,H,D] bf16 patterns, positives[b]
    the positive document ids of query b (``choice`` = (c_star [B,N],
    t_star [B,N]) as in aux_loss_f64). Returns (loss [B], dQR [B,M,H,D],
    dKRbar [C,H,D] summed over the queries, s [B,N], c_star [B,N],
    t_star [B,N], gaps [B,N])."""
    QR = np.asarray(QR)
    k = bf16_to_f64(KRbar)
    B = QR.shape[0]
    outs = [aux_loss_f64(bf16_to_f64(QR[b]), k, doc_chunk_offsets, positives[b], tau,
                         choice=None if choice is None else (choice[0][b], choice[1][b]))
            for b in range(B)]
    loss = np.array([o[0] for o in outs])
    dQ = np.stack([o[1] for o in outs])
    dK = np.sum([o[2] for o in outs], axis=0)
    return (loss, dQ, dK, np.stack([o[3] for o in outs]), np.stack([o[4] for o in outs]),
            np.stack([o[5] for o in outs]), np.stack([o[6] for o in outs]))
