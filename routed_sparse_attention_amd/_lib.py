"""ctypes binding of libmsa.so (C ABI declared in include/msa.h).

Argument marshalling only: every step of the MSA path runs in the HIP
library. PyTorch supplies device memory, pinned host memory, workspaces and
the current stream. If the library is not built the calls raise; there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsa.so")

MSA_OK = 0
STATUS = {0: "MSA_OK", -1: "MSA_ERR_INVALID_ARG", -2: "MSA_ERR_SHAPE", -3: "MSA_ERR_WORKSPACE",
          -4: "MSA_ERR_HIP", -5: "MSA_ERR_UNSUPPORTED", -6: "MSA_ERR_IO"}
TOKEN_REDUCE_MAX, TOKEN_REDUCE_MEAN = 0, 1
DOC_ROPE_TOKEN, DOC_ROPE_CHUNK = 0, 1

# every symbol include/msa.h declares
EXPORTED = [
    "msa_default_dims", "msa_last_error", "msa_abi_version", "msa_plan_chunks",
    "msa_encode_pool_workspace", "msa_encode_pool", "msa_route_topk_workspace", "msa_route_topk",
    "msa_route_scores_workspace", "msa_route_scores", "msa_select_topk_workspace", "msa_select_topk",
    "msa_sparse_attend_workspace", "msa_sparse_attend", "msa_interleave_reset",
    "msa_interleave_step_workspace", "msa_interleave_step", "msa_store_reset", "msa_store_append",
    "msa_store_save", "msa_store_load", "msa_store_file_info", "msa_route_aux_loss_workspace",
    "msa_route_aux_loss", "msa_route_topk_noalloc", "msa_interleave_batch_reset",
    "msa_interleave_batch_step_workspace", "msa_interleave_batch_step",
    "msa_sparse_attend_batch_workspace", "msa_sparse_attend_batch",
]
NOALLOC_SCRATCH_BYTES = 16 << 20   # MSA_NOALLOC_SCRATCH_BYTES
STORE_KR, STORE_K, STORE_V = 1, 2, 4   # tensor bits of a store file


class MsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [("n_kv_heads", ctypes.c_int32), ("n_router_heads", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("token_reduce", ctypes.c_int32),
                ("doc_rope_mode", ctypes.c_int32)]


class InterleaveStateC(ctypes.Structure):
    _fields_ = [("doc_scores", ctypes.c_void_p), ("K_loc", ctypes.c_void_p),
                ("V_loc", ctypes.c_void_p), ("cap_loc", ctypes.c_int32),
                ("n_loc", ctypes.c_int32), ("topk_ids", ctypes.c_void_p),
                ("topk_scores", ctypes.c_void_p), ("n_sel", ctypes.c_void_p),
                ("pos0", ctypes.c_int64)]


class InterleaveBatchC(ctypes.Structure):
    _fields_ = [("doc_scores", ctypes.c_void_p), ("K_loc", ctypes.c_void_p),
                ("V_loc", ctypes.c_void_p), ("B", ctypes.c_int32), ("cap_loc", ctypes.c_int32),
                ("n_loc", ctypes.c_int32), ("topk_ids", ctypes.c_void_p),
                ("topk_scores", ctypes.c_void_p), ("n_sel", ctypes.c_void_p),
                ("pos0", ctypes.c_int64)]


class StoreC(ctypes.Structure):
    _fields_ = [("Kbar", ctypes.c_void_p), ("Vbar", ctypes.c_void_p), ("KRbar", ctypes.c_void_p),
                ("doc_chunk_offsets", ctypes.c_void_p), ("doc_chunk_offsets_h", ctypes.c_void_p),
                ("cap_chunks", ctypes.c_int64), ("cap_docs", ctypes.c_int32),
                ("n_docs", ctypes.c_int32), ("n_chunks", ctypes.c_int64)]


_lib = None
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_DP = ctypes.POINTER(Dims)


def lib() -> ctypes.CDLL:
    """Loads libmsa.so (raises ImportError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(hipcc, gfx950); the MSA path has no other implementation")
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "msa_default_dims": (None, [_DP]),
        "msa_last_error": (ctypes.c_char_p, []),
        "msa_abi_version": (_i32, []),
        "msa_plan_chunks": (_i32, [_vp, _i32, _i32, _vp]),
        "msa_encode_pool_workspace": (_sz, [_DP, _i32, _i64]),
        "msa_encode_pool": (_i32, [_DP, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64, _vp, _vp, _vp,
                                   _vp, _sz, _vp]),
        "msa_route_topk_workspace": (_sz, [_DP, _i32, _i32, _i64, _i32]),
        "msa_route_topk": (_i32, [_DP, _vp, _i32, _i32, _vp, _vp, _i32, _i64, _vp, _i32, _vp, _vp,
                                  _vp, _vp, _sz, _vp]),
        "msa_route_scores_workspace": (_sz, [_DP, _i32, _i32, _i64]),
        "msa_route_scores": (_i32, [_DP, _vp, _i32, _i32, _vp, _i64, _vp, _vp, _sz, _vp]),
        "msa_select_topk_workspace": (_sz, [_DP, _i32, _i32]),
        "msa_select_topk": (_i32, [_DP, _vp, _i32, _vp, _i32, _i64, _vp, _i32, _vp, _vp, _vp, _vp,
                                   _sz, _vp]),
        "msa_sparse_attend_workspace": (_sz, [_DP, _i32, _i32, _i64]),
        "msa_sparse_attend": (_i32, [_DP, _vp, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _i32, _i64,
                                     _vp, _i32, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _sz, _vp]),
        "msa_sparse_attend_batch_workspace": (_sz, [_DP, _i32, _i32, _i32, _i64]),
        "msa_sparse_attend_batch": (_i32, [_DP, _vp, _i32, _i32, _vp, _vp, _i32, _i32, _vp, _vp,
                                           _i32, _i64, _vp, _i32, _vp, _vp, _i64, _i64, _vp, _vp,
                                           _vp, _sz, _vp]),
        "msa_interleave_reset": (_i32, [ctypes.POINTER(InterleaveStateC), _i32, _vp]),
        "msa_interleave_step_workspace": (_sz, [_DP, _i32, _i32, _i64, _i32, _i64]),
        "msa_interleave_step": (_i32, [_DP, ctypes.POINTER(InterleaveStateC), _vp, _vp, _vp, _vp,
                                       _i32, _vp, _vp, _vp, _i32, _i64, _vp, _i32, _i64, _vp, _vp,
                                       _sz, _vp]),
        "msa_interleave_batch_reset": (_i32, [ctypes.POINTER(InterleaveBatchC), _i32, _vp]),
        "msa_interleave_batch_step_workspace": (_sz, [_DP, _i32, _i32, _i32, _i64, _i32, _i64]),
        "msa_interleave_batch_step": (_i32, [_DP, ctypes.POINTER(InterleaveBatchC), _vp, _vp, _vp,
                                             _vp, _i32, _vp, _vp, _vp, _i32, _i64, _vp, _i32, _i64,
                                             _vp, _vp, _sz, _vp]),
        "msa_store_reset": (_i32, [ctypes.POINTER(StoreC), _vp]),
        "msa_store_append": (_i32, [_DP, ctypes.POINTER(StoreC), _vp, _vp, _vp, _vp, _vp, _i32, _i64,
                                    _vp]),
        "msa_store_save": (_i32, [_DP, ctypes.POINTER(StoreC), ctypes.c_char_p, _vp, _sz]),
        "msa_store_load": (_i32, [_DP, ctypes.POINTER(StoreC), ctypes.c_char_p, _vp, _sz]),
        "msa_store_file_info": (_i32, [ctypes.c_char_p, ctypes.POINTER(_i32), ctypes.POINTER(_i64),
                                       ctypes.POINTER(ctypes.c_uint32)]),
        "msa_route_topk_noalloc": (_i32, [_DP, _vp, _i32, _i32, _vp, _vp, _i32, _i64, _vp, _i32,
                                          _vp, _vp, _vp, _vp]),
        "msa_route_aux_loss_workspace": (_sz, [_DP, _i32, _i32, _i64, _i32]),
        "msa_route_aux_loss": (_i32, [_DP, _vp, _i32, _i32, _vp, _vp, _i32, _i64, _vp, _vp, _i32,
                                      ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(rc: int):
    if rc != MSA_OK:
        raise MsaError(rc, lib().msa_last_error().decode(errors="replace"))


def dims(**kw) -> Dims:
    d = Dims()
    lib().msa_default_dims(ctypes.byref(d))
    for k, v in kw.items():
        if not hasattr(d, k):
            raise TypeError(f"unknown dims field {k}")
        setattr(d, k, v)
    return d


def _p(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor, name: str, dtype, device_kind: str | None = "cuda", ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device_kind is not None and t.device.type != device_kind:
        raise ValueError(f"{name} must be on {device_kind}, got {t.device}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got shape {tuple(t.shape)}")


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
def plan_chunks(doc_token_offsets, chunk: int = 64) -> np.ndarray:
    dto = np.ascontiguousarray(np.asarray(doc_token_offsets, dtype=np.int64))
    out = np.zeros_like(dto)
    _check(lib().msa_plan_chunks(dto.ctypes.data, len(dto) - 1, chunk, out.ctypes.data))
    return out


def encode_pool(K, V, KR, doc_token_offsets, doc_chunk_offsets, n_chunks: int, d: Dims | None = None,
                outputs=("K", "V", "KR"), out=None):
    """Stage-1 pooling: returns (Kbar, Vbar, KRbar) bf16 [n_chunks, 8, 128]
    (None for outputs not requested)."""
    d = d or dims()
    for t, n in ((K, "K"), (V, "V"), (KR, "KR")):
        _need(t, n, torch.bfloat16, ndim=3)
    _need(doc_token_offsets, "doc_token_offsets", torch.int64)
    _need(doc_chunk_offsets, "doc_chunk_offsets", torch.int64)
    n_docs = doc_token_offsets.numel() - 1
    if out is None:
        mk = lambda: torch.empty((n_chunks, K.shape[1], K.shape[2]), dtype=torch.bfloat16, device=K.device)
        out = tuple(mk() if name in outputs else None for name in ("K", "V", "KR"))
    Kb, Vb, Rb = out
    ws = lib().msa_encode_pool_workspace(ctypes.byref(d), n_docs, n_chunks)
    w = _workspace(ws, K.device)
    _check(lib().msa_encode_pool(ctypes.byref(d), _p(K), _p(V), _p(KR), _p(doc_token_offsets),
                                 _p(doc_chunk_offsets), n_docs, K.shape[0], n_chunks, _p(Kb), _p(Vb),
                                 _p(Rb), _p(w), ws, _stream()))
    return Kb, Vb, Rb


def route_topk_workspace(B: int, M: int, n_chunks: int, n_docs: int, d: Dims | None = None) -> int:
    d = d or dims()
    return lib().msa_route_topk_workspace(ctypes.byref(d), B, M, n_chunks, n_docs)


def route_topk(QR, KRbar, doc_chunk_offsets, d: Dims | None = None, doc_scores=None,
               accumulate: bool = False, ws=None, outs=None):
    """Stage-2 routing for B queries: returns (doc_scores [B,N] f32,
    topk_ids [B,k] i32, topk_scores [B,k] f32, n_sel [B] i32)."""
    d = d or dims()
    _need(QR, "QR", torch.bfloat16, ndim=4)
    _need(KRbar, "KRbar", torch.bfloat16, ndim=3)
    _need(doc_chunk_offsets, "doc_chunk_offsets", torch.int64)
    B, M = QR.shape[0], QR.shape[1]
    n_docs = doc_chunk_offsets.numel() - 1
    C = KRbar.shape[0]
    dev = QR.device
    if doc_scores is None:
        if accumulate:
            raise ValueError("accumulate needs doc_scores")
        doc_scores = torch.empty((B, n_docs), dtype=torch.float32, device=dev)
    if outs is None:
        outs = (torch.empty((B, d.top_k), dtype=torch.int32, device=dev),
                torch.empty((B, d.top_k), dtype=torch.float32, device=dev),
                torch.empty((B,), dtype=torch.int32, device=dev))
    ids, sc, ns = outs
    need = lib().msa_route_topk_workspace(ctypes.byref(d), B, M, C, n_docs)
    if ws is None or ws.numel() < need:
        ws = _workspace(need, dev)
    _check(lib().msa_route_topk(ctypes.byref(d), _p(QR), B, M, _p(KRbar), _p(doc_chunk_offsets),
                                n_docs, C, _p(doc_scores), int(bool(accumulate)), _p(ids), _p(sc),
                                _p(ns), _p(ws), ws.numel(), _stream()))
    return doc_scores, ids, sc, ns


def route_topk_noalloc(QR, KRbar, doc_chunk_offsets, d: Dims | None = None, doc_scores=None,
                       accumulate: bool = False, outs=None):
    """route_topk through the entry point that takes no workspace (the
    library's fixed device scratch); the caller still passes the outputs."""
    d = d or dims()
    _need(QR, "QR", torch.bfloat16, ndim=4)
    _need(KRbar, "KRbar", torch.bfloat16, ndim=3)
    _need(doc_chunk_offsets, "doc_chunk_offsets", torch.int64)
    B, M = QR.shape[0], QR.shape[1]
    n_docs = doc_chunk_offsets.numel() - 1
    dev = QR.device
    if doc_scores is None:
        if accumulate:
            raise ValueError("accumulate needs doc_scores")
        doc_scores = torch.empty((B, n_docs), dtype=torch.float32, device=dev)
    if outs is None:
        outs = (torch.empty((B, d.top_k), dtype=torch.int32, device=dev),
                torch.empty((B, d.top_k), dtype=torch.float32, device=dev),
                torch.empty((B,), dtype=torch.int32, device=dev))
    ids, sc, ns = outs
    _check(lib().msa_route_topk_noalloc(ctypes.byref(d), _p(QR), B, M, _p(KRbar),
                                        _p(doc_chunk_offsets), n_docs, KRbar.shape[0],
                                        _p(doc_scores), int(bool(accumulate)), _p(ids), _p(sc),
                                        _p(ns), _stream()))
    return doc_scores, ids, sc, ns


def route_scores(QR, KRbar, d: Dims | None = None, out=None, ws=None):
    """Chunk scores S_c [B, n_chunks] fp32 (first half of route_topk)."""
    d = d or dims()
    _need(QR, "QR", torch.bfloat16, ndim=4)
    _need(KRbar, "KRbar", torch.bfloat16, ndim=3)
    B, M, C = QR.shape[0], QR.shape[1], KRbar.shape[0]
    if out is None:
        out = torch.empty((B, C), dtype=torch.float32, device=QR.device)
    need = lib().msa_route_scores_workspace(ctypes.byref(d), B, M, C)
    if need and (ws is None or ws.numel() < need):
        ws = _workspace(need, QR.device)
    _check(lib().msa_route_scores(ctypes.byref(d), _p(QR), B, M, _p(KRbar), C, _p(out), _p(ws),
                                  0 if ws is None else ws.numel(), _stream()))
    return out


def select_topk(chunk_scores, doc_chunk_offsets, d: Dims | None = None, doc_scores=None,
                accumulate: bool = False, ws=None, outs=None):
    """Document max + top-k from chunk scores [B, n_chunks] (second half of
    route_topk): returns (doc_scores, topk_ids, topk_scores, n_sel)."""
    d = d or dims()
    _need(chunk_scores, "chunk_scores", torch.float32, ndim=2)
    _need(doc_chunk_offsets, "doc_chunk_offsets", torch.int64)
    B, C = chunk_scores.shape
    n_docs = doc_chunk_offsets.numel() - 1
    dev = chunk_scores.device
    if doc_scores is None:
        if accumulate:
            raise ValueError("accumulate needs doc_scores")
        doc_scores = torch.empty((B, n_docs), dtype=torch.float32, device=dev)
    if outs is None:
        outs = (torch.empty((B, d.top_k), dtype=torch.int32, device=dev),
                torch.empty((B, d.top_k), dtype=torch.float32, device=dev),
                torch.empty((B,), dtype=torch.int32, device=dev))
    ids, sc, ns = outs
    need = lib().msa_select_topk_workspace(ctypes.byref(d), B, n_docs)
    if ws is None or ws.numel() < need:
        ws = _workspace(need, dev)
    _check(lib().msa_select_topk(ctypes.byref(d), _p(chunk_scores), B, _p(doc_chunk_offsets), n_docs,
                                 C, _p(doc_scores), int(bool(accumulate)), _p(ids), _p(sc), _p(ns),
                                 _p(ws), ws.numel(), _stream()))
    return doc_scores, ids, sc, ns


def sparse_attend_workspace(M: int, M_loc: int, max_sel_chunks: int, d: Dims | None = None) -> int:
    d = d or dims()
    return lib().msa_sparse_attend_workspace(ctypes.byref(d), M, M_loc, max_sel_chunks)


def sparse_attend(Q, K_loc, V_loc, Kbar, Vbar, doc_chunk_offsets, sel_ids, n_sel,
                  max_sel_chunks: int, pos0: int = -1, k_loc_rotated: bool = False,
                  d: Dims | None = None, want_f32: bool = False, ws=None, out=None):
    """Stage-3 sparse attention for one query: returns out bf16 [M, Hq, 128]
    (and fp32 when want_f32). Kbar/Vbar may be pinned host tensors."""
    d = d or dims()
    _need(Q, "Q", torch.bfloat16, ndim=3)
    _need(K_loc, "K_loc", torch.bfloat16, ndim=3)
    _need(V_loc, "V_loc", torch.bfloat16, ndim=3)
    on_host = Kbar.device.type == "cpu"
    for t, n in ((Kbar, "Kbar"), (Vbar, "Vbar")):
        _need(t, n, torch.bfloat16, device_kind=None, ndim=3)
        if (t.device.type == "cpu") != on_host:
            raise ValueError("Kbar and Vbar must both be on the GPU or both in pinned host memory")
        if on_host and not t.is_pinned():
            raise ValueError(f"{n}: host memory must be pinned")
    _need(doc_chunk_offsets, "doc_chunk_offsets", torch.int64)
    _need(sel_ids, "sel_ids", torch.int32)
    _need(n_sel, "n_sel", torch.int32)
    M, M_loc = Q.shape[0], K_loc.shape[0]
    dev = Q.device
    if out is None:
        out = torch.empty(Q.shape, dtype=torch.bfloat16, device=dev)
    of = torch.empty(Q.shape, dtype=torch.float32, device=dev) if want_f32 else None
    need = lib().msa_sparse_attend_workspace(ctypes.byref(d), M, M_loc, max_sel_chunks)
    if ws is None or ws.numel() < need:
        ws = _workspace(need, dev)
    _check(lib().msa_sparse_attend(ctypes.byref(d), _p(Q), M, _p(K_loc), _p(V_loc), M_loc,
                                   int(bool(k_loc_rotated)), _p(Kbar), _p(Vbar), int(on_host),
                                   Kbar.shape[0], _p(doc_chunk_offsets),
                                   doc_chunk_offsets.numel() - 1, _p(sel_ids), _p(n_sel),
                                   max_sel_chunks, pos0, _p(out), _p(of), _p(ws), ws.numel(),
                                   _stream()))
    return (out, of) if want_f32 else out


def sparse_attend_batch(Q, K_loc, V_loc, Kbar, Vbar, doc_chunk_offsets, sel_ids, n_sel,
                        max_sel_chunks: int, pos0: int = -1, k_loc_rotated: bool = False,
                        d: Dims | None = None, want_f32: bool = False, ws=None, out=None):
    """Stage-3 sparse attention for B queries of one shape in one set of
    launches: Q [B, M, Hq, 128], K_loc / V_loc [B, M_loc, 8, 128], sel_ids
    [B, top_k], n_sel [B]; returns out bf16 [B, M, Hq, 128] (and fp32 when
    want_f32). Each query's result equals sparse_attend's for it alone."""
    d = d or dims()
    _need(Q, "Q", torch.bfloat16, ndim=4)
    _need(K_loc, "K_loc", torch.bfloat16, ndim=4)
    _need(V_loc, "V_loc", torch.bfloat16, ndim=4)
    on_host = Kbar.device.type == "cpu"
    for t, n in ((Kbar, "Kbar"), (Vbar, "Vbar")):
        _need(t, n, torch.bfloat16, device_kind=None, ndim=3)
        if (t.device.type == "cpu") != on_host:
            raise ValueError("Kbar and Vbar must both be on the GPU or both in pinned host memory")
        if on_host and not t.is_pinned():
            raise ValueError(f"{n}: host memory must be pinned")
    _need(doc_chunk_offsets, "doc_chunk_offsets", torch.int64)
    _need(sel_ids, "sel_ids", torch.int32, ndim=2)
    _need(n_sel, "n_sel", torch.int32)
    B, M, M_loc = Q.shape[0], Q.shape[1], K_loc.shape[1]
    if K_loc.shape[0] != B or V_loc.shape[:2] != K_loc.shape[:2] or sel_ids.shape[0] != B \
            or n_sel.numel() != B:
        raise ValueError("sparse_attend_batch: every input needs the same batch size B")
    dev = Q.device
    if out is None:
        out = torch.empty(Q.shape, dtype=torch.bfloat16, device=dev)
    of = torch.empty(Q.shape, dtype=torch.float32, device=dev) if want_f32 else None
    need = lib().msa_sparse_attend_batch_workspace(ctypes.byref(d), B, M, M_loc, max_sel_chunks)
    if ws is None or ws.numel() < need:
        ws = _workspace(need, dev)
    _check(lib().msa_sparse_attend_batch(
        ctypes.byref(d), _p(Q), B, M, _p(K_loc), _p(V_loc), M_loc, int(bool(k_loc_rotated)),
        _p(Kbar), _p(Vbar), int(on_host), Kbar.shape[0], _p(doc_chunk_offsets),
        doc_chunk_offsets.numel() - 1, _p(sel_ids), _p(n_sel), max_sel_chunks, pos0, _p(out),
        _p(of), _p(ws), ws.numel(), _stream()))
    return (out, of) if want_f32 else out


class Interleave:
    """Memory Interleave state for one query (caller-owned device buffers)."""

    def __init__(self, n_docs: int, cap_loc: int, device="cuda", d: Dims | None = None,
                 pos0: int = -1):
        self.d = d or dims()
        self.n_docs = n_docs
        self.doc_scores = torch.empty((n_docs,), dtype=torch.float32, device=device)
        self.K_loc = torch.zeros((cap_loc, 8, 128), dtype=torch.bfloat16, device=device)
        self.V_loc = torch.zeros((cap_loc, 8, 128), dtype=torch.bfloat16, device=device)
        self.topk_ids = torch.empty((self.d.top_k,), dtype=torch.int32, device=device)
        self.topk_scores = torch.empty((self.d.top_k,), dtype=torch.float32, device=device)
        self.n_sel = torch.empty((1,), dtype=torch.int32, device=device)
        self.st = InterleaveStateC(_p(self.doc_scores), _p(self.K_loc), _p(self.V_loc), cap_loc, 0,
                                   _p(self.topk_ids), _p(self.topk_scores), _p(self.n_sel), pos0)
        self.reset()

    def reset(self):
        """Forget every round: running scores to -inf, no local tokens."""
        _check(lib().msa_interleave_reset(ctypes.byref(self.st), self.n_docs, _stream()))

    @property
    def n_loc(self) -> int:
        return self.st.n_loc

    def step(self, Q_new, K_new, V_new, QR_new, KRbar, Kbar, Vbar, doc_chunk_offsets,
             max_sel_chunks: int, ws=None, out=None):
        d = self.d
        for t, n in ((Q_new, "Q_new"), (K_new, "K_new"), (V_new, "V_new"), (QR_new, "QR_new")):
            _need(t, n, torch.bfloat16, ndim=3)
        _need(KRbar, "KRbar", torch.bfloat16, ndim=3)
        on_host = Kbar.device.type == "cpu"
        M_new = Q_new.shape[0]
        dev = Q_new.device
        if out is None:
            out = torch.empty(Q_new.shape, dtype=torch.bfloat16, device=dev)
        need = lib().msa_interleave_step_workspace(ctypes.byref(d), M_new, self.st.cap_loc,
                                                   KRbar.shape[0], self.n_docs, max_sel_chunks)
        if ws is None or ws.numel() < need:
            ws = _workspace(need, dev)
        _check(lib().msa_interleave_step(ctypes.byref(d), ctypes.byref(self.st), _p(Q_new),
                                         _p(K_new), _p(V_new), _p(QR_new), M_new, _p(KRbar),
                                         _p(Kbar), _p(Vbar), int(on_host), KRbar.shape[0],
                                         _p(doc_chunk_offsets), self.n_docs, max_sel_chunks,
                                         _p(out), _p(ws), ws.numel(), _stream()))
        return out


class InterleaveBatch:
    """Memory Interleave state for B queries that advance together
    (msa_interleave_batch_*; caller-owned device buffers, contiguous per query)."""

    def __init__(self, B: int, n_docs: int, cap_loc: int, device="cuda", d: Dims | None = None,
                 pos0: int = -1):
        self.d = d or dims()
        self.B = B
        self.n_docs = n_docs
        self.doc_scores = torch.empty((B, n_docs), dtype=torch.float32, device=device)
        self.K_loc = torch.zeros((B, cap_loc, 8, 128), dtype=torch.bfloat16, device=device)
        self.V_loc = torch.zeros((B, cap_loc, 8, 128), dtype=torch.bfloat16, device=device)
        self.topk_ids = torch.empty((B, self.d.top_k), dtype=torch.int32, device=device)
        self.topk_scores = torch.empty((B, self.d.top_k), dtype=torch.float32, device=device)
        self.n_sel = torch.empty((B,), dtype=torch.int32, device=device)
        self.st = InterleaveBatchC(_p(self.doc_scores), _p(self.K_loc), _p(self.V_loc), B, cap_loc,
                                   0, _p(self.topk_ids), _p(self.topk_scores), _p(self.n_sel), pos0)
        self.reset()

    def reset(self):
        """Forget every round: running scores to -inf, no local tokens."""
        _check(lib().msa_interleave_batch_reset(ctypes.byref(self.st), self.n_docs, _stream()))

    @property
    def n_loc(self) -> int:
        return self.st.n_loc

    def workspace_bytes(self, M_new: int, n_chunks: int, max_sel_chunks: int) -> int:
        return lib().msa_interleave_batch_step_workspace(ctypes.byref(self.d), self.B, M_new,
                                                         self.st.cap_loc, n_chunks, self.n_docs,
                                                         max_sel_chunks)

    def step(self, Q_new, K_new, V_new, QR_new, KRbar, Kbar, Vbar, doc_chunk_offsets,
             max_sel_chunks: int, ws=None, out=None):
        """One round: Q_new [B, M_new, n_q_heads, 128], K_new/V_new/QR_new
        [B, M_new, 8, 128]; returns out [B, M_new, n_q_heads, 128]."""
        d = self.d
        for t, n in ((Q_new, "Q_new"), (K_new, "K_new"), (V_new, "V_new"), (QR_new, "QR_new")):
            _need(t, n, torch.bfloat16, ndim=4)
            if t.shape[0] != self.B:
                raise ValueError(f"{n} has {t.shape[0]} queries, the state {self.B}")
        _need(KRbar, "KRbar", torch.bfloat16, ndim=3)
        on_host = Kbar.device.type == "cpu"
        M_new = Q_new.shape[1]
        dev = Q_new.device
        if out is None:
            out = torch.empty(Q_new.shape, dtype=torch.bfloat16, device=dev)
        need = self.workspace_bytes(M_new, KRbar.shape[0], max_sel_chunks)
        if ws is None or ws.numel() < need:
            ws = _workspace(need, dev)
        _check(lib().msa_interleave_batch_step(ctypes.byref(d), ctypes.byref(self.st), _p(Q_new),
                                               _p(K_new), _p(V_new), _p(QR_new), M_new, _p(KRbar),
                                               _p(Kbar), _p(Vbar), int(on_host), KRbar.shape[0],
                                               _p(doc_chunk_offsets), self.n_docs, max_sel_chunks,
                                               _p(out), _p(ws), ws.numel(), _stream()))
        return out


# ---------------------------------------------------------------------------
def store_file_info(path: str) -> tuple[int, int, int]:
    """(n_docs, n_chunks, tensor bits) from a store file's header."""
    n_docs, n_chunks, mask = _i32(), _i64(), ctypes.c_uint32()
    _check(lib().msa_store_file_info(os.fsencode(path), ctypes.byref(n_docs), ctypes.byref(n_chunks),
                                     ctypes.byref(mask)))
    return n_docs.value, n_chunks.value, mask.value


class Store:
    """A pooled memory store that grows by whole documents (msa_store_*).

    Buffers are allocated here for the given capacity; ``tensors`` picks which
    of K̄ ("K"), V̄ ("V") and K̄^R ("KR") are kept; ``kv_on_host`` puts K̄/V̄ in
    pinned host memory (the host tier). Views of the filled part: ``Kbar``,
    ``Vbar``, ``KRbar``, ``doc_chunk_offsets`` (device) and ``offsets_h``."""

    def __init__(self, cap_docs: int, cap_chunks: int, d: Dims | None = None,
                 tensors=("K", "V", "KR"), kv_on_host: bool = False, device="cuda"):
        self.d = d or dims()
        self.device = torch.device(device)
        shape = (cap_chunks, 8, 128)

        def alloc(name, host):
            if name not in tensors:
                return None
            if host:
                return torch.empty(shape, dtype=torch.bfloat16, pin_memory=True)
            return torch.empty(shape, dtype=torch.bfloat16, device=self.device)

        self._K = alloc("K", kv_on_host)
        self._V = alloc("V", kv_on_host)
        self._KR = alloc("KR", False)
        self._dco = torch.zeros((cap_docs + 1,), dtype=torch.int64, device=self.device)
        self._dco_h = torch.zeros((cap_docs + 1,), dtype=torch.int64, pin_memory=True)
        self.st = StoreC(_p(self._K), _p(self._V), _p(self._KR), _p(self._dco), _p(self._dco_h),
                         cap_chunks, cap_docs, 0, 0)
        self.reset()

    def reset(self):
        _check(lib().msa_store_reset(ctypes.byref(self.st), _stream()))

    @property
    def n_docs(self) -> int:
        return self.st.n_docs

    @property
    def n_chunks(self) -> int:
        return self.st.n_chunks

    def _view(self, t):
        return None if t is None else t[: self.n_chunks]

    @property
    def Kbar(self):
        return self._view(self._K)

    @property
    def Vbar(self):
        return self._view(self._V)

    @property
    def KRbar(self):
        return self._view(self._KR)

    @property
    def doc_chunk_offsets(self) -> torch.Tensor:
        return self._dco[: self.n_docs + 1]

    @property
    def offsets_h(self) -> np.ndarray:
        return self._dco_h[: self.n_docs + 1].numpy().copy()

    def append(self, K, V, KR, doc_token_offsets) -> range:
        """Pools and appends documents given by their raw states and token
        offsets (from 0); returns the new documents' ids."""
        dto_h = np.ascontiguousarray(np.asarray(doc_token_offsets, dtype=np.int64))
        n_new = len(dto_h) - 1
        for t, n in ((K, "K"), (V, "V"), (KR, "KR")):
            if t is not None:
                _need(t, n, torch.bfloat16, ndim=3)
        dto = torch.from_numpy(dto_h).to(self.device)
        first = self.n_docs
        T = int(dto_h[-1]) if n_new >= 0 else 0
        _check(lib().msa_store_append(ctypes.byref(self.d), ctypes.byref(self.st),
                                      _p(K if self._K is not None else None),
                                      _p(V if self._V is not None else None),
                                      _p(KR if self._KR is not None else None), _p(dto),
                                      dto_h.ctypes.data, n_new, T, _stream()))
        self._keep = (dto, dto_h)   # the uploads read these until the stream catches up
        return range(first, self.n_docs)

    def _staging(self, nbytes: int):
        return torch.empty((max(int(nbytes), 1 << 20),), dtype=torch.uint8, pin_memory=True)

    def save(self, path: str, staging_bytes: int = 64 << 20):
        stg = self._staging(staging_bytes)
        _check(lib().msa_store_save(ctypes.byref(self.d), ctypes.byref(self.st), os.fsencode(path),
                                    _p(stg), stg.numel()))

    def load(self, path: str, staging_bytes: int = 64 << 20):
        stg = self._staging(staging_bytes)
        _check(lib().msa_store_load(ctypes.byref(self.d), ctypes.byref(self.st), os.fsencode(path),
                                    _p(stg), stg.numel()))


# ---------------------------------------------------------------------------
def route_aux_loss(QR, KRbar, doc_chunk_offsets, positives, tau: float, d: Dims | None = None,
                   ws=None):
    """The router's auxiliary contrastive loss and its gradient for B queries
    (msa_route_aux_loss). ``positives[b]`` lists query b's positive document
    ids. Returns (loss [B], dQR [B,M,8,128], dKRbar [C,8,128], doc_scores
    [B,N], best_chunk [B,N], best_token [B,N])."""
    d = d or dims()
    _need(QR, "QR", torch.bfloat16, ndim=4)
    _need(KRbar, "KRbar", torch.bfloat16, ndim=3)
    _need(doc_chunk_offsets, "doc_chunk_offsets", torch.int64)
    B, M, C = QR.shape[0], QR.shape[1], KRbar.shape[0]
    N = doc_chunk_offsets.numel() - 1
    dev = QR.device
    max_pos = max(1, max(len(p) for p in positives))
    pos = torch.full((B, max_pos), -1, dtype=torch.int32)
    for b, p in enumerate(positives):
        if len(p):
            pos[b, :len(p)] = torch.tensor(list(p), dtype=torch.int32)
    pos = pos.to(dev)
    n_pos = torch.tensor([len(p) for p in positives], dtype=torch.int32, device=dev)
    loss = torch.empty((B,), dtype=torch.float32, device=dev)
    dQR = torch.empty((B, M, 8, 128), dtype=torch.float32, device=dev)
    dKR = torch.empty((C, 8, 128), dtype=torch.float32, device=dev)
    ds = torch.empty((B, N), dtype=torch.float32, device=dev)
    bc = torch.empty((B, N), dtype=torch.int32, device=dev)
    bt = torch.empty((B, N), dtype=torch.int32, device=dev)
    need = lib().msa_route_aux_loss_workspace(ctypes.byref(d), B, M, C, N)
    if ws is None or ws.numel() < need:
        ws = _workspace(need, dev)
    _check(lib().msa_route_aux_loss(ctypes.byref(d), _p(QR), B, M, _p(KRbar), _p(doc_chunk_offsets),
                                    N, C, _p(pos), _p(n_pos), max_pos, float(tau), _p(loss),
                                    _p(dQR), _p(dKR), _p(ds), _p(bc), _p(bt), _p(ws), ws.numel(),
                                    _stream()))
    return loss, dQR, dKR, ds, bc, bt
