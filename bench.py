#!/usr/bin/env python3
"""Throughput of the MSA hot path on one MI355X.

Default workload ("100M"): a 100M-token memory — 1,562,500 pooled chunks per
routed layer — with the router keys of all 18 routed layers resident in HBM
(57.6 GB, bf16) and the pooled K̄/V̄ of one layer (6.4 GB) in pinned host
memory, read by every layer; documents of 4–64 chunks; one planted needle per
layer; one decode query (32 Q heads, 128 tokens of history + itself).

One step = one decode query through all 18 layers, each layer running the
whole hot path on the current stream:
    msa_route_scores  (cosine scan of the layer's 1,562,500 router keys)
    msa_select_topk   (chunk -> document max, top-16)
    msa_sparse_attend (chunk list, global RoPE, GQA attention over the
                       selected chunks read in place from pinned host memory
                       plus the local KV)
value = memory tokens routed per second per query = 18 × 100M / step time.

The JSON line also carries the roofline of the dominant kernel (the routing
scan: 2048 algorithmic bytes per chunk, timed with HIP events around its own
launches in the timed region) and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
SCAN_BYTES_PER_CHUNK = 8 * 128 * 2          # one pooled router-key row
TOKENS_PER_CHUNK = 64


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=18)
    ap.add_argument("--chunks", type=int, default=1_562_500)
    ap.add_argument("--kv", choices=["host", "device"], default="host")
    ap.add_argument("--cpu-sample-chunks", type=int, default=400_000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quiet", action="store_true")
    return ap.parse_args()


def log(args, msg):
    if not args.quiet:
        print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def stored_traffic(kernel_src):
    """HBM bytes per scan launch measured with rocprofv3 counters (see
    profiles/), valid only while the kernel source is unchanged."""
    p = os.path.join(ROOT, "profiles", "traffic_route_scan.json")
    if not os.path.exists(p):
        return None
    t = json.load(open(p))
    if t.get("source_sha256") != source_sha(kernel_src):
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(args, store, n_layers, dev_query, att0):
    """The oracle, untouched, on a bounded sample of the same workload."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from oracle import msa_oracle as O

    u16 = lambda t: t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    C = store.n_chunks
    sample = min(args.cpu_sample_chunks, C)
    block = 100_000
    qr = u16(dev_query.QR[0])
    with threadpool_limits(limits=1):
        t_route = 0.0
        done = 0
        while done < sample:
            n = min(block, sample - done)
            kr = u16(store.KRbar[0, done:done + n])
            t0 = time.perf_counter()
            O.chunk_scores(qr, kr)
            t_route += time.perf_counter() - t0
            done += n
        rng = np.random.default_rng(0)
        S = rng.standard_normal(C)
        t0 = time.perf_counter()
        s = O.doc_scores(S, store.doc_chunk_offsets)
        O.topk(s, 16)
        t_select = time.perf_counter() - t0
        # a fixed selection (documents 0..15) gives the same amount of work
        sel = list(range(16))
        dco = store.doc_chunk_offsets
        rows = np.concatenate([np.arange(dco[i], dco[i + 1]) for i in sel])
        kbar = u16(store.Kbar[torch.from_numpy(rows)])
        vbar = u16(store.Vbar[torch.from_numpy(rows)])
        sub_dco = np.concatenate([[0], np.cumsum([dco[i + 1] - dco[i] for i in sel])])
        t0 = time.perf_counter()
        O.sparse_attend(u16(att0.Q), u16(att0.K_loc), u16(att0.V_loc), kbar, vbar, sub_dco,
                        list(range(16)))
        t_attend = time.perf_counter() - t0
    t_layer = t_route * (C / sample) + t_select + t_attend
    value = n_layers * C * TOKENS_PER_CHUNK / (n_layers * t_layer)
    return {
        "value": value, "unit": "tokens/s", "cores": 1, "kind": "oracle",
        "sample": (f"oracle routing over {sample:,} of {C:,} chunks of layer 0 "
                   f"({t_route:.2f} s, scaled to the full layer), document max + top-16 over "
                   f"{store.n_docs:,} documents ({t_select:.2f} s) and sparse attention for one "
                   f"decode token over 16 documents ({t_attend:.2f} s); per-layer time × "
                   f"{n_layers} layers; numpy fp64, 1 thread"),
        "seconds_measured": t_route + t_select + t_attend,
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this MSA build measures one GPU; multi-GPU runs are not "
                          "part of it (see the sharding notes in DESIGN.md)",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import routed_sparse_attention_amd as msa
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"
    L = args.layers
    t_gen = time.perf_counter()
    log(args, f"generating {L} layers × {args.chunks:,} chunks of router keys on the GPU, "
              f"K̄/V̄ of one layer on the {args.kv}")
    store, queries, atts = synth.cfg4_100m(dev, n_chunks=args.chunks, n_layers=L,
                                           kv_pinned=(args.kv == "host"))
    torch.cuda.synchronize()
    log(args, f"generated in {time.perf_counter() - t_gen:.1f} s; docs={store.n_docs:,}")
    C, N = store.n_chunks, store.n_docs
    d = msa.dims()
    dco = torch.from_numpy(store.doc_chunk_offsets).to(dev)
    max_doc = int(np.diff(store.doc_chunk_offsets).max())
    max_sel = d.top_k * max_doc
    QR = [q.QR for q in queries]
    S = torch.empty((1, C), dtype=torch.float32, device=dev)
    ds = torch.empty((1, N), dtype=torch.float32, device=dev)
    ids = torch.empty((1, d.top_k), dtype=torch.int32, device=dev)
    sc = torch.empty((1, d.top_k), dtype=torch.float32, device=dev)
    ns = torch.empty((1,), dtype=torch.int32, device=dev)
    ws_sel = torch.empty(max(1, msa.lib().msa_select_topk_workspace(ctypes.byref(d), 1, N)),
                         dtype=torch.uint8, device=dev)
    ws_att = torch.empty(msa.sparse_attend_workspace(1, atts[0].K_loc.shape[0], max_sel, d),
                         dtype=torch.uint8, device=dev)
    outs = [torch.empty((1, 32, 128), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    Kb, Vb = store.Kbar, store.Vbar

    ev = lambda: torch.cuda.Event(enable_timing=True)
    timing = {"scan": [], "select": [], "attend": []}

    def step(record):
        for l in range(L):
            e = [ev() for _ in range(4)] if record else None
            if record:
                e[0].record()
            msa.route_scores(QR[l], store.KRbar[l], d, out=S)
            if record:
                e[1].record()
            msa.select_topk(S, dco, d, doc_scores=ds, ws=ws_sel, outs=(ids, sc, ns))
            if record:
                e[2].record()
            msa.sparse_attend(atts[l].Q, atts[l].K_loc, atts[l].V_loc, Kb, Vb, dco, ids[0], ns,
                              max_sel, d=d, ws=ws_att, out=outs[l])
            if record:
                e[3].record()
                timing["scan"].append((e[0], e[1]))
                timing["select"].append((e[1], e[2]))
                timing["attend"].append((e[2], e[3]))

    # correctness guard on the measured configuration: every layer's needle
    step(False)
    torch.cuda.synchronize()
    for l in range(L):
        msa.route_scores(QR[l], store.KRbar[l], d, out=S)
        msa.select_topk(S, dco, d, doc_scores=ds, ws=ws_sel, outs=(ids, sc, ns))
        got = set(ids[0].cpu().tolist())
        assert set(queries[l].planted_docs[0]) <= got, f"layer {l}: needle not selected"
    log(args, "needles found in every layer")

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0, t1 = ev(), ev()
    t0.record()
    wall0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps
    avg = {k: sum(a.elapsed_time(b) for a, b in v) / len(v) * 1e3 for k, v in timing.items()}  # µs

    tokens = C * TOKENS_PER_CHUNK
    value = L * tokens / (ms_step * 1e-3)
    scan_bytes = C * SCAN_BYTES_PER_CHUNK
    achieved = scan_bytes / (avg["scan"] * 1e-6) / 1e9
    traffic = stored_traffic(os.path.join(ROOT, "routed_sparse_attention_amd", "csrc",
                                          "msa_route.hip"))
    result = {
        "metric": "memory tokens routed/sec per query",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{tokens / 1e6:.0f}M-token memory, {L} routed layers, one decode query "
                        f"per step",
            "memory_tokens": tokens, "chunks_per_layer": C, "documents": N, "layers": L,
            "top_k": d.top_k, "chunk": 64, "heads": 8, "head_dim": 128, "q_heads": 32,
            "local_tokens": int(atts[0].K_loc.shape[0]),
            "router_keys_bytes": L * scan_bytes,
            "kv_tier": "pinned host (read in place over PCIe)" if args.kv == "host" else "HBM",
        },
        "route_scan_us_per_layer": avg["scan"],
        "select_topk_us_per_layer": avg["select"],
        "sparse_attend_us_per_query_layer": avg["attend"],
        "route_tokens_per_s_per_layer": tokens / (avg["scan"] * 1e-6),
        "roofline": {
            "bound": "hbm", "kernel": "scan_valu_kernel (msa_route_scores)",
            "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
            "bytes_per_launch": scan_bytes,
        },
        "wall_s_timed": wall,
    }
    if not args.no_cpu_baseline:
        log(args, "timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(args, store, L, queries[0], atts[0])
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
