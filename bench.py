"""Benchmark of the centroid-masked sparse LM head on one MI355X.

Workload: the greedy sweep (d=256, V=262144, Nc=2048 equal clusters of 128,
K=32, bf16 inputs, synthetic seeded data).  A step is one ``top_tokens`` call
(centroid projection, top-K, deduplicated slab gather, sparse dot, argmax) at
B=64 for the headline ``value``, issued straight through the C ABI (four
kernel launches).  Each sweep row also reports the same call replayed from a
captured HIP graph (the pages' sequencing; on ROCm a graph launch costs more
host and device time than the four launches it replaces) and the device time
per call with eight calls captured in one graph.  The line also carries every
batch size of the sweep, the masked full-vocabulary output (forward), the
fused top-m (also with log-probabilities over the row's candidates), the
fused draft step and FP8 slabs at B in {1, 16, 64} (eager
calls; forward also as graph replays), the skewed head (Zipf clusters,
correlated rows) at B=64, and the wide head with its dense comparison
path.

Cold HBM: every step uses a different copy of the weights (``--copies``,
default 8, about 1 GiB) and, for B < 64, a different group of hidden rows, so
the bytes touched across one rotation exceed twice the 256 MiB Infinity Cache.
Warm replays (one copy, one row group) are reported separately.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_MFMA_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
MIN_SECONDS = 0.1   # every row but the headline is timed for at least this long
METRIC = "sparse-head draft rows/sec at B=1..64 + achieved HBM GB/s vs peak (1 MI355X)"

# HBM bytes per launch of the dominant kernel (gather, top_tokens, B=64) from
# two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE in KiB per dispatch), each
# scaled by what the counter reads for a plain 128 MiB copy (fetch x2.00,
# write x1.00); see profiles/gather_kernel_sweep_B64.md.  Valid only for the
# kernel source it was measured on: any other source reports null.
TRAFFIC_RECORD = {
    "kernels_sha256_prefix": "0ce68a787527410b",
    "fetch_kib": 41437.8, "fetch_scale": 2.00, "write_kib": 128, "write_scale": 1.00,
}


def _traffic_bytes():
    import hashlib
    src = os.path.join(ROOT, "centroid_masked_sparse_amd", "csrc", "ce_kernels.hip")
    with open(src, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    r = TRAFFIC_RECORD
    if not digest.startswith(r["kernels_sha256_prefix"]):
        return None
    return int((r["fetch_kib"] * r["fetch_scale"] + r["write_kib"] * r["write_scale"]) * 1024)


def _to_device(a, dtype, torch):
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to("cuda:0")


def _union_bytes(topk: np.ndarray, sizes: np.ndarray, d: int, elem: int) -> tuple[int, int]:
    """(gathered slab bytes, clusters) of the union of the rows' selected centroids."""
    u = np.unique(topk.reshape(-1))
    return int(sizes[u].sum()) * d * elem, len(u)


def _time_replays(torch, graphs, steps, warmup, stream_handle, min_s=MIN_SECONDS):
    """Average ms per launch cycling through ``graphs``, timed for at least
    ``min_s`` seconds."""
    n = len(graphs)
    for i in range(warmup):
        graphs[i % n].launch(stream_handle)
    torch.cuda.synchronize()

    def issue(i0, k):
        for i in range(i0, i0 + k):
            graphs[i % n].launch(stream_handle)
    return _timed(torch, issue, steps, min_s) * 1e-3


def _timed(torch, issue, steps, min_s):
    """Microseconds per call: batches of ``steps`` calls (``issue(i0, n)``
    enqueues calls i0 .. i0+n-1), each bracketed by events, repeated until
    ``min_s`` seconds of calls have been timed, so that a row's figure does
    not depend on how few steps were asked for."""
    total_ms, n, i0 = 0.0, 0, 0
    while True:
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record()
        issue(i0, steps)
        ev1.record()
        torch.cuda.synchronize()
        total_ms += ev0.elapsed_time(ev1)
        n += steps
        i0 += steps
        if total_ms * 1e-3 >= min_s:
            return total_ms * 1e3 / n


def _time_calls(torch, calls, steps, warmup, min_s=MIN_SECONDS):
    """Microseconds per call of eager C-ABI calls cycling through ``calls``
    ((function, args, keep-alive...) tuples), timed for at least ``min_s``
    seconds; every distinct call is run (and its status checked) during
    warm-up."""
    n = len(calls)
    for i in range(max(warmup, n)):
        f, a = calls[i % n][0], calls[i % n][1]
        st = f(*a)
        if st != 0:
            raise RuntimeError(f"{f.__name__} failed with status {st}")
    torch.cuda.synchronize()

    def issue(i0, k):
        for i in range(i0, i0 + k):
            f, a = calls[i % n][0], calls[i % n][1]
            f(*a)
    return _timed(torch, issue, steps, min_s)


def _eager_us_per_call(torch, heads, hs, K, B, steps, warmup, stream, min_s=MIN_SECONDS):
    """Cold eager calls: ce_top_tokens straight through the C ABI (four kernel
    launches), rotating weight copies and row groups like the graph replays;
    timed for at least ``min_s`` seconds (0: exactly ``steps`` calls)."""
    from centroid_masked_sparse_amd import OP_TOP_TOKENS
    calls = []
    for s_ in range(len(hs)):
        for head in heads:
            out = torch.empty((B,), dtype=torch.int32, device="cuda:0")
            ws = head._workspace(B, K, OP_TOP_TOKENS)
            calls.append((head._lib.ce_top_tokens,
                          (head._handle, hs[s_].data_ptr(), B, K, out.data_ptr(), None,
                           ws.data_ptr(), ws.numel(), stream), out))
    n = len(calls)
    for i in range(max(warmup, n)):
        f, a, _ = calls[i % n]
        st = f(*a)
        if st != 0:
            raise RuntimeError(f"ce_top_tokens failed with status {st}")
    torch.cuda.synchronize()

    def issue(i0, k):
        for i in range(i0, i0 + k):
            f, a, _ = calls[i % n]
            f(*a)
    return _timed(torch, issue, steps, min_s)


def _device_us_per_call(torch, heads, hs, K, B, steps, warmup, per_graph=8):
    """Cold calls per microsecond of device time: ``per_graph`` consecutive calls
    (rotating weight copies and row groups) captured into one graph, so the
    host cost of a graph launch is spread over them."""
    dev = "cuda:0"
    graphs, keep = [], []
    for r in range(len(heads)):
        outs = [torch.empty((B,), dtype=torch.int32, device=dev) for _ in range(per_graph)]
        calls = [(heads[(r + m) % len(heads)], hs[(r * per_graph + m) % len(hs)], outs[m])
                 for m in range(per_graph)]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for head, hg, o in calls:   # first use allocates each head's workspace
                head.top_tokens(hg, K, out=o)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for head, hg, o in calls:
                head.top_tokens(hg, K, out=o)
        graphs.append(g)
        keep.append(outs)
    n = max(20, steps // per_graph)
    for i in range(max(2, warmup // per_graph)):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n):
        graphs[i % len(graphs)].replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (n * per_graph)


EMB_DIM = 2560   # backbone width of the embedding table (assumed: the pages give none)


def _stream_read_probe(torch, lib, stream, log, nbytes=2 << 30, calls=20):
    """Streaming read rate of this GPU: `ce_probe_stream_read` over a 2 GiB
    buffer (8 times the Infinity Cache), each launch bracketed by events on the
    stream it runs on; GB/s over the mean launch time."""
    from centroid_masked_sparse_amd import _ffi
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    for _ in range(3):
        _ffi.check(lib.ce_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), stream),
                   "ce_probe_stream_read")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(calls)]
    for a, b in ev:
        a.record()
        _ffi.check(lib.ce_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), stream),
                   "ce_probe_stream_read")
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    out = {"GB_s": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes": nbytes, "us_per_launch": round(ms * 1e3, 2),
           "frac_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    log(f"[bench] streaming read probe: {out}")
    del buf, sink
    torch.cuda.empty_cache()
    return out


def _draft_section(torch, heads, groups, K, args, stream, log):
    """The fused draft step (final RMSNorm, head, next step's scaled embedding:
    four launches) against the same step unfused (PyTorch RMSNorm in float32,
    ce_top_tokens, PyTorch embedding lookup and scale), at B in {1, 16, 64}.
    Seeded synthetic norm weight and embedding table; the 64 hidden rows of
    the sweep workload serve as the rows before the norm."""
    from centroid_masked_sparse_amd import OP_DRAFT_STEP
    dev = "cuda:0"
    V, d = heads[0].V, heads[0].d
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    nw = (1.0 + 0.1 * torch.randn(d, generator=g, device=dev)).to(torch.bfloat16)
    table = torch.randn((V, EMB_DIM), generator=g, device=dev).to(torch.bfloat16)
    normalizer = float(EMB_DIM) ** 0.5
    n32 = torch.tensor(normalizer, dtype=torch.float32, device=dev)
    eps = 1e-6
    rows = []
    for B in (1, 16, 64):
        hs = groups(B)
        calls, keep = [], []
        for s_ in range(len(hs)):
            for head in heads:
                h_out = torch.empty_like(hs[s_])
                tok = torch.empty((B,), dtype=torch.int32, device=dev)
                emb = torch.empty((B, EMB_DIM), dtype=torch.bfloat16, device=dev)
                ws = head._workspace(B, K, OP_DRAFT_STEP)
                calls.append((head._lib.ce_draft_step,
                              (head._handle, hs[s_].data_ptr(), nw.data_ptr(), ctypes.c_float(eps),
                               B, K, h_out.data_ptr(), tok.data_ptr(), table.data_ptr(), EMB_DIM,
                               ctypes.c_float(normalizer), emb.data_ptr(), None, ws.data_ptr(),
                               ws.numel(), stream)))
                keep.append((h_out, tok, emb))
        fused = _time_calls(torch, calls, args.steps, args.warmup)

        def unfused(i):
            head = heads[i % len(heads)]
            x = hs[(i // len(heads)) % len(hs)]
            xf = x.float()
            h = (xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + eps)).to(torch.bfloat16) * nw
            tok = head.top_tokens(h, K)
            return table[tok.long()] * n32

        for i in range(max(args.warmup, 2 * len(heads))):
            unfused(i)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        n = max(50, args.steps // 4)
        a.record()
        for i in range(n):
            unfused(i)
        b.record()
        torch.cuda.synchronize()
        unf = a.elapsed_time(b) * 1e3 / n
        row = {"B": B, "emb_dim": EMB_DIM, "us_per_call": round(fused, 3),
               "rows_per_s": round(B / (fused * 1e-6), 1), "unfused_us_per_call": round(unf, 3)}
        rows.append(row)
        log(f"[bench] draft_step: {row}")
    del table
    torch.cuda.empty_cache()
    return rows


def _fp8_section(torch, heads, groups, H, w, K, args, stream, log):
    """Top tokens with FP8 (E4M3) slabs: one FP8 head quantised at prepare
    time from each bf16 weight copy, timed like the headline (eager C-ABI
    calls, rotating copies and row groups) at B in {1, 16, 64}.  Bytes are
    the union of selected clusters' codes and float32 row scales plus the bf16
    centroids.  Also: how often the FP8 argmax equals the bf16 argmax on the
    64 rows, and the FP8 gather kernel alone at B=64."""
    from centroid_masked_sparse_amd import Head, _ffi
    dev = "cuda:0"
    d, Nc, sizes = w.d, w.Nc, w.sizes
    fheads = [Head(h._keep[0], h._keep[1], w.tos, max_B=64, max_K=K, slabs="fp8",
                   projection=args.projection) for h in heads]
    torch.cuda.synchronize()
    rows = []
    slab64 = None
    for B in (1, 16, 64):
        hs = groups(B)
        topk = torch.empty((B, K), dtype=torch.int32, device=dev)
        ub = []
        for hg in hs:
            heads[0].top_tokens(hg, K, topk_out=topk)
            torch.cuda.synchronize()
            ub.append(_union_bytes(topk.cpu().numpy(), sizes, d + 4, 1)[0])
        slab = float(np.mean(ub))
        unique = Nc * d * 2 + slab
        us = _eager_us_per_call(torch, fheads, hs, K, B, args.steps, args.warmup, stream)
        row = {"B": B, "us_per_call": round(us, 3), "rows_per_s": round(B / (us * 1e-6), 1),
               "unique_MiB": round(unique / 2**20, 2), "GB_s": round(unique / (us * 1e-6) / 1e9, 1)}
        rows.append(row)
        log(f"[bench] fp8 top_tokens B={B}: {row}")
        if B == 64:
            slab64 = slab
    tb = heads[0].top_tokens(H, K)
    tf = fheads[0].top_tokens(H, K)
    agree = float((tb == tf).float().mean().item())
    n = args.probe_calls
    start_ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    stop_ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in start_ev + stop_ev:
        e.record()                      # creates the HIP events
    torch.cuda.synchronize()
    out = torch.empty((64,), dtype=torch.int32, device=dev)
    for i in range(n):
        _ffi.check(fheads[0]._lib.ce_probe_gather_events(start_ev[i].cuda_event, stop_ev[i].cuda_event),
                   "ce_probe_gather_events")
        fheads[i % len(fheads)].top_tokens(H, K, out=out)
    torch.cuda.synchronize()
    g_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(start_ev, stop_ev)]))
    res = {"format": "OCP E4M3 codes + fp32 row scale", "argmax_agreement_with_bf16": round(agree, 4),
           "sweep": rows, "gather_us_B64": round(g_ms * 1e3, 3),
           "gather_GB_s_B64": round(slab64 / (g_ms * 1e-3) / 1e9, 1)}
    log(f"[bench] fp8 slabs: agreement {agree:.4f}, gather B=64 {g_ms * 1e3:.2f} us, "
        f"{res['gather_GB_s_B64']} GB/s")
    for h in fheads:
        h.close()
    del fheads
    torch.cuda.empty_cache()
    return res


def _skewed_section(torch, args, stream, log):
    """The skewed head at B=64 (d=512, V=262144, Nc=2048 Zipf(1.1) clusters of
    10 .. 44,286 tokens, K=32, rows around 8 anchor directions): top_tokens
    through the C ABI, cold over two weight copies (512 MiB), with the
    gather alone.  Stresses the dedup (overlapping row sets: the line gives
    their mean pairwise Jaccard) and the load balance (tiles that many rows
    selected; the line gives the largest selected cluster, in tokens)."""
    from centroid_masked_sparse_amd import Head, OP_TOP_TOKENS, _ffi
    from workloads import make_workload
    w = make_workload("skewed")
    d, Nc, K, B = w.d, w.Nc, w.K, 64
    C0 = _to_device(w.C, w.dtype, torch)
    E0 = _to_device(w.E, w.dtype, torch)
    H = _to_device(w.h, w.dtype, torch)[:B].contiguous()
    heads = [Head(C0 if m == 0 else C0.clone(), E0 if m == 0 else E0.clone(), w.tos, w.offsets,
                  max_B=B, max_K=K, projection=args.projection) for m in range(2)]
    topk = torch.empty((B, K), dtype=torch.int32, device="cuda:0")
    heads[0].top_tokens(H, K, topk_out=topk)
    torch.cuda.synchronize()
    sel = topk.cpu().numpy()
    slab, clusters = _union_bytes(sel, w.sizes, d, 2)
    unique = Nc * d * 2 + slab
    # overlap of the rows' selections: mean pairwise Jaccard, and the largest
    # cluster any row selected
    sets = [set(r.tolist()) for r in sel]
    jac = [len(sets[i] & sets[j]) / len(sets[i] | sets[j]) for i in range(B) for j in range(i + 1, B)]
    largest = int(max(w.sizes[c] for c in set().union(*sets)))
    us = _eager_us_per_call(torch, heads, [H], K, B, args.steps, args.warmup, stream)
    n = max(20, args.probe_calls // 4)
    start_ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    stop_ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in start_ev + stop_ev:
        e.record()
    torch.cuda.synchronize()
    o = torch.empty((B,), dtype=torch.int32, device="cuda:0")
    for i in range(n):
        _ffi.check(heads[0]._lib.ce_probe_gather_events(start_ev[i].cuda_event, stop_ev[i].cuda_event),
                   "ce_probe_gather_events")
        heads[i % 2].top_tokens(H, K, out=o)
    torch.cuda.synchronize()
    g_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(start_ev, stop_ev)]))
    out = {"workload": f"skewed head d={d} V={w.V} Nc={Nc} Zipf(1.1) CSR, K={K} bf16, B={B}, "
                       f"correlated rows, cold (2 weight copies)",
           "us_per_call": round(us, 3), "rows_per_s": round(B / (us * 1e-6), 1),
           "union_clusters": clusters, "mean_jaccard": round(float(np.mean(jac)), 4),
           "largest_cluster_in_union": largest, "unique_MiB": round(unique / 2**20, 2),
           "GB_s": round(unique / (us * 1e-6) / 1e9, 1),
           "frac_peak": round(unique / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
           "gather_us": round(g_ms * 1e3, 3), "gather_GB_s": round(slab / (g_ms * 1e-3) / 1e9, 1)}
    log(f"[bench] skewed: {out}")
    for h in heads:
        h.close()
    del heads, E0, C0
    torch.cuda.empty_cache()
    return out


def _wide_section(torch, args, stream, log):
    """The wide head at B=64: the sparse head at K=64 and at K=Nc (every
    centroid: the exact dense argmax), beside a dense comparison path, the
    vendor bf16 GEMM (fp32 output) of all V logits followed by an argmax.
    Cold over two weight copies."""
    from centroid_masked_sparse_amd import OP_TOP_TOKENS, Head, _ffi
    from workloads import make_workload
    w = make_workload("wide")
    d, V, Nc, K, B = w.d, w.V, w.Nc, w.K, 64
    sizes = w.sizes
    ncopy = 2
    C0 = _to_device(w.C, w.dtype, torch)
    E0 = _to_device(w.E, w.dtype, torch)
    H = _to_device(w.h, w.dtype, torch)[:B].contiguous()
    heads = [Head(C0 if m == 0 else C0.clone(), E0 if m == 0 else E0.clone(), w.tos,
                  max_B=B, max_K=Nc, projection=args.projection) for m in range(ncopy)]
    out = {"workload": f"wide head d={d} V={V} Nc={Nc} bf16, B={B}, cold ({ncopy} weight copies)"}
    for k in (K, Nc):
        topk = torch.empty((B, k), dtype=torch.int32, device="cuda:0")
        heads[0].top_tokens(H, k, topk_out=topk)
        torch.cuda.synchronize()
        slab, _ = _union_bytes(topk.cpu().numpy(), sizes, d, 2)
        unique = Nc * d * 2 + slab
        calls = []
        for hd in heads:
            o = torch.empty((B,), dtype=torch.int32, device="cuda:0")
            ws = hd._workspace(B, k, OP_TOP_TOKENS)
            calls.append((hd._lib.ce_top_tokens, (hd._handle, H.data_ptr(), B, k, o.data_ptr(), None,
                                                  ws.data_ptr(), ws.numel(), stream), o))
        # rows whose top-K boundary needed recomputed canonical keys (MFMA
        # projection), over 20 calls of each copy
        rc0 = [hd.repair_counts() for hd in heads]
        for _ in range(20):
            for f, a, _o in calls:
                f(*a)
        rc1 = [hd.repair_counts() for hd in heads]
        repaired = sum(r1[0] - r0[0] + r1[1] - r0[1] for r0, r1 in zip(rc0, rc1)) / (20 * len(heads))
        us = _time_calls(torch, calls, max(20, args.steps // 8), max(5, args.warmup // 8))
        # the gather alone (HIP events around its launch), and its matrix-core
        # throughput on the useful multiply-adds: d per (row, candidate token)
        n = max(20, args.probe_calls // 4)
        start_ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        stop_ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in start_ev + stop_ev:
            e.record()
        torch.cuda.synchronize()
        for i in range(n):
            _ffi.check(heads[0]._lib.ce_probe_gather_events(start_ev[i].cuda_event, stop_ev[i].cuda_event),
                       "ce_probe_gather_events")
            f, a_, _o = calls[i % len(calls)]
            f(*a_)
        torch.cuda.synchronize()
        g_us = float(np.mean([x.elapsed_time(y) for x, y in zip(start_ev, stop_ev)])) * 1e3
        cand = int(sum(sizes[c] for row in topk.cpu().numpy() for c in row))
        tflops = 2.0 * d * cand / (g_us * 1e-6) / 1e12
        out[f"sparse_K{k}"] = {"us_per_call": round(us, 3), "rows_per_s": round(B / (us * 1e-6), 1),
                               "unique_MiB": round(unique / 2**20, 2),
                               "GB_s": round(unique / (us * 1e-6) / 1e9, 1),
                               "frac_peak": round(unique / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                               "repaired_rows_per_call": round(repaired, 2),
                               "gather_us": round(g_us, 3),
                               "gather_GB_s": round(slab / (g_us * 1e-6) / 1e9, 1),
                               "gather_mfma_useful_TFLOP_s": round(tflops, 1),
                               "gather_mfma_frac_of_bf16_dense_peak": round(tflops / PEAK_MFMA_BF16_TFLOPS, 4),
                               "calls": "eager C-ABI calls"}
        log(f"[bench] wide sparse K={k}: {out[f'sparse_K{k}']}")
    # dense comparison: E in token order, logits^T = E_tok @ h^T (fp32 out)
    inv = torch.from_numpy(np.argsort(w.tos).astype(np.int64)).to("cuda:0")
    E_tok = [E0.index_select(0, inv).contiguous()]
    E_tok.append(E_tok[0].clone())
    hT = H.t().contiguous()
    del heads, E0, C0
    torch.cuda.empty_cache()

    def dense(e):
        return torch.argmax(torch.mm(e, hT, out_dtype=torch.float32), dim=0)

    for i in range(3):
        dense(E_tok[i % 2])
    torch.cuda.synchronize()
    n = max(20, args.steps // 20)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n):
        dense(E_tok[i % 2])
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / n
    dense_bytes = V * d * 2
    out["dense_gemm_argmax"] = {
        "us_per_call": round(us, 3), "rows_per_s": round(B / (us * 1e-6), 1),
        "bytes_MiB": round(dense_bytes / 2**20, 1), "GB_s": round(dense_bytes / (us * 1e-6) / 1e9, 1),
        "tflops": round(2.0 * B * d * V / (us * 1e-6) / 1e12, 2),
        "path": "vendor bf16 GEMM (torch.mm, fp32 out) of all V logits + argmax; eager, not captured"}
    log(f"[bench] wide dense comparison: {out['dense_gemm_argmax']}")
    del E_tok
    torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--batches", default="1,2,4,8,16,32,64")
    ap.add_argument("--copies", type=int, default=8)
    ap.add_argument("--no-masked", action="store_true")
    ap.add_argument("--no-wide", action="store_true")
    ap.add_argument("--no-top-m", action="store_true")
    ap.add_argument("--no-draft", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-skewed", action="store_true")
    ap.add_argument("--probe-calls", type=int, default=200)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--projection", choices=("auto", "exact", "mfma"), default="auto",
                    help="centroid projection of the fused calls (auto: the bf16-MFMA one with "
                         "its certified top-K for bf16 heads)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: the head runs on one GPU; --gpus above 1 is not supported "
              "(no collective path is built).", file=sys.stderr)
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: launched with WORLD_SIZE > 1; only one GPU is supported.", file=sys.stderr)
        return 2

    import torch

    from centroid_masked_sparse_amd import OP_MASKED_LOGITS, OP_TOP_TOKENS, Head, _ffi
    from workloads import CONFIGS, make_workload

    w = make_workload("sweep")
    d, V, Nc, K = w.d, w.V, w.Nc, w.K
    elem = 2
    sizes = w.sizes
    batches = [int(b) for b in args.batches.split(",") if b]
    dev = "cuda:0"
    stream = torch.cuda.current_stream(dev).cuda_stream
    log = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731

    # weight copies for cold-HBM rotation
    C0 = _to_device(w.C, w.dtype, torch)
    E0 = _to_device(w.E, w.dtype, torch)
    heads = []
    for m in range(args.copies):
        C = C0 if m == 0 else C0.clone()
        E = E0 if m == 0 else E0.clone()
        heads.append(Head(C, E, w.tos, max_B=64, max_K=K, projection=args.projection))
    H = _to_device(w.h, w.dtype, torch)          # the 64 drawn rows
    torch.cuda.synchronize()
    log(f"[bench] {args.copies} weight copies ready "
        f"({args.copies * (E0.numel() + C0.numel()) * elem / 2**20:.0f} MiB)")

    def groups(B):
        return [H[s * B:(s + 1) * B].contiguous() for s in range(64 // B)]

    probe = _stream_read_probe(torch, heads[0]._lib, stream, log)

    # ------------------------------------------------------------ sweep (top_tokens)
    sweep = []
    head_row = None
    for B in batches:
        hs = groups(B)
        outs, graphs_cold, graphs_warm = [], [], None
        topk = torch.empty((B, K), dtype=torch.int32, device=dev)
        ub = []
        for hg in hs:
            heads[0].top_tokens(hg, K, topk_out=topk)
            torch.cuda.synchronize()
            ub.append(_union_bytes(topk.cpu().numpy(), sizes, d, elem))
        slab_bytes = float(np.mean([u[0] for u in ub]))
        clusters = float(np.mean([u[1] for u in ub]))
        unique = Nc * d * elem + slab_bytes
        per_copy = []
        for m, head in enumerate(heads):
            gl = []
            for hg in hs:
                out = torch.empty((B,), dtype=torch.int32, device=dev)
                outs.append(out)
                gl.append(head.capture(OP_TOP_TOKENS, hg, K, out))
            per_copy.append(gl)
        # rotate copies fastest, then row groups
        for s in range(len(hs)):
            for m in range(len(heads)):
                graphs_cold.append(per_copy[m][s])
        graphs_warm = [per_copy[0][0]]
        ms_cold = _time_replays(torch, graphs_cold, args.steps, args.warmup, stream)
        ms_warm = _time_replays(torch, graphs_warm, args.steps, args.warmup, stream)
        graph_us = ms_cold * 1e3
        dev_us = _device_us_per_call(torch, heads, hs, K, B, args.steps, args.warmup)
        us = _eager_us_per_call(torch, heads, hs, K, B, args.steps, args.warmup, stream)
        row = {
            "B": B, "us_per_call": round(us, 3), "rows_per_s": round(B / (us * 1e-6), 1),
            "unique_MiB": round(unique / 2**20, 2), "union_clusters": round(clusters, 1),
            "GB_s": round(unique / (us * 1e-6) / 1e9, 1),
            "frac_peak": round(unique / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "frac_probe": round(unique / (us * 1e-6) / 1e9 / probe["GB_s"], 4),
            "graph_us_per_call": round(graph_us, 3),
            "graph_warm_us_per_call": round(ms_warm * 1e3, 3),
            "device_us_per_call": round(dev_us, 3),
            "row_groups": len(hs), "copies": len(heads),
        }
        if B == max(batches):
            # the headline: exactly --steps calls after --warmup, as asked
            us_k = _eager_us_per_call(torch, heads, hs, K, B, args.steps, args.warmup, stream,
                                      min_s=0.0)
            row["headline_us_per_call"] = round(us_k, 3)
            head_row = row
            head_slab = slab_bytes
            head_unique = unique
            head_groups = hs
        sweep.append(row)
        log(f"[bench] top_tokens B={B}: {row}")
        for gl in per_copy:
            for g in gl:
                g.close()

    # ------------------------------------------------------------ gather kernel probe
    Bp = head_row["B"]
    hp = head_groups[0]
    start_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.probe_calls)]
    stop_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.probe_calls)]
    for e in start_ev + stop_ev:
        e.record()
    torch.cuda.synchronize()
    out = torch.empty((Bp,), dtype=torch.int32, device=dev)
    for i in range(args.probe_calls):
        _ffi.check(heads[0]._lib.ce_probe_gather_events(start_ev[i].cuda_event, stop_ev[i].cuda_event),
                   "ce_probe_gather_events")
        heads[i % len(heads)].top_tokens(hp, K, out=out)
    torch.cuda.synchronize()
    gather_ms = float(np.mean([s.elapsed_time(e) for s, e in zip(start_ev, stop_ev)]))
    gather_gbs = head_slab / (gather_ms * 1e-3) / 1e9
    log(f"[bench] gather kernel B={Bp}: {gather_ms * 1e3:.2f} us, {head_slab / 2**20:.1f} MiB slabs,"
        f" {gather_gbs:.0f} GB/s")

    # ------------------------------------------------------------ masked logits (forward)
    masked = []
    if not args.no_masked:
        for B in [b for b in CONFIGS["masked"].batches if b in (1, 16, 64)]:
            hs = groups(B)
            topk = torch.empty((B, K), dtype=torch.int32, device=dev)
            ub = []
            for hg in hs:
                heads[0].masked_logits(hg, K, topk_out=topk)
                torch.cuda.synchronize()
                ub.append(_union_bytes(topk.cpu().numpy(), sizes, d, elem)[0])
            unique = Nc * d * elem + float(np.mean(ub)) + B * V * 4
            per_copy = []
            for head in heads:
                gl = []
                for hg in hs:
                    o = torch.empty((B, V), dtype=torch.float32, device=dev)
                    gl.append((head.capture(OP_MASKED_LOGITS, hg, K, o), o))
                per_copy.append(gl)
            cold = [per_copy[m][s][0] for s in range(len(hs)) for m in range(len(heads))]
            steps = max(50, args.steps // 4)
            ms = _time_replays(torch, cold, steps, max(10, args.warmup // 4), stream)
            graph_us = ms * 1e3
            # eager C-ABI calls (the fill then runs beside the projection and
            # top-K on the library's side stream), same rotation
            calls = []
            for s_ in range(len(hs)):
                for m_, head in enumerate(heads):
                    o = per_copy[m_][s_][1]
                    ws = head._workspace(B, K, OP_MASKED_LOGITS)
                    calls.append((head._lib.ce_masked_logits,
                                  (head._handle, hs[s_].data_ptr(), B, K, o.data_ptr(), None,
                                   ws.data_ptr(), ws.numel(), stream)))
            us = _time_calls(torch, calls, steps, max(10, args.warmup // 4))
            row = {"B": B, "us_per_call": round(us, 3), "rows_per_s": round(B / (us * 1e-6), 1),
                   "bytes_MiB": round(unique / 2**20, 2),
                   "GB_s": round(unique / (us * 1e-6) / 1e9, 1),
                   "frac_peak": round(unique / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                   "graph_us_per_call": round(graph_us, 3)}
            masked.append(row)
            log(f"[bench] masked_logits B={B}: {row}")
            for gl in per_copy:
                for g, _o in gl:
                    g.close()
            del per_copy
            torch.cuda.empty_cache()

    # ------------------------------------------------------------ fused top-m
    top_m = []
    if not args.no_top_m:
        from centroid_masked_sparse_amd import OP_TOP_M, OP_TOP_M_LOG_SOFTMAX
        m = 8

        def top_m_us(B, hs, op, fn):
            calls = []
            for s_ in range(len(hs)):
                for head in heads:
                    tok = torch.empty((B, m), dtype=torch.int32, device=dev)
                    val = torch.empty((B, m), dtype=torch.float32, device=dev)
                    ws = head._workspace(B, K, op)
                    calls.append((getattr(head._lib, fn),
                                  (head._handle, hs[s_].data_ptr(), B, K, m, tok.data_ptr(),
                                   val.data_ptr(), None, ws.data_ptr(), ws.numel(), stream),
                                  tok, val))
            return _time_calls(torch, calls, args.steps, args.warmup)

        for B in (1, 16, 64):
            hs = groups(B)
            us = top_m_us(B, hs, OP_TOP_M, "ce_top_m")
            # the same with log-probabilities over the row's candidates
            us_ls = top_m_us(B, hs, OP_TOP_M_LOG_SOFTMAX, "ce_top_m_log_softmax")
            row = {"B": B, "m": m, "us_per_call": round(us, 3), "rows_per_s": round(B / (us * 1e-6), 1),
                   "log_softmax_us_per_call": round(us_ls, 3)}
            top_m.append(row)
            log(f"[bench] top_m: {row}")

    # ------------------------------------------------------------ fused draft step
    draft = []
    if not args.no_draft:
        draft = _draft_section(torch, heads, groups, K, args, stream, log)

    # ------------------------------------------------------------ FP8 slabs
    fp8 = None
    if not args.no_fp8:
        fp8 = _fp8_section(torch, heads, groups, H, w, K, args, stream, log)

    # ------------------------------------------------------------ skewed clusters (config 5)
    skewed = None
    if not args.no_skewed:
        skewed = _skewed_section(torch, args, stream, log)

    # ------------------------------------------------------------ wide head (d=1024, Nc=4096)
    wide = None
    if not args.no_wide:
        wide = _wide_section(torch, args, stream, log)

    # ------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        hrows = w.h[:Bp]
        t0 = time.perf_counter()
        calls = 0
        while True:
            oracle.top_tokens(hrows, w.C, w.E, w.offsets, w.tos, K, w.dtype)
            calls += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        secs = time.perf_counter() - t0
        cpu = {"value": round(calls * Bp / secs, 2), "unit": "rows/s", "cores": 1, "kind": "oracle",
               # the headline's unique bytes (centroids and the rows' slab
               # union) per oracle call of the same rows
               "GB_s": round(calls * head_unique / secs / 1e9, 5),
               "sample": f"{calls} oracle top_tokens call(s) of the first {Bp} rows of the sweep "
                         f"workload, {secs:.1f} s single-threaded numpy (float64 canonical dots); "
                         f"host has {len(os.sched_getaffinity(0))} usable of {os.cpu_count()} cores; "
                         f"numpy {np.__version__}"}
        log(f"[bench] cpu oracle: {cpu}")

    us = head_row["headline_us_per_call"]
    line = {
        "metric": METRIC,
        "value": round(head_row["B"] / (us * 1e-6), 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": f"greedy sweep d={d} V={V} Nc={Nc} K={K} bf16, B={Bp}, cold HBM "
                               f"({len(heads)} weight copies, {head_row['row_groups']} row groups)",
                   "B": Bp, "d": d, "V": V, "Nc": Nc, "K": K, "inputs": "bf16",
                   "calls": "eager C-ABI calls (graph replays reported per row)",
                   "accumulate": "f64 canonical chain, fp32 results"},
        "hbm_GB_s": round(head_unique / (us * 1e-6) / 1e9, 1),
        "hbm_frac_peak": round(head_unique / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        "roofline": {"bound": "hbm", "kernel": "gather_kernel<bf16,argmax>",
                     "scope": "the dominant kernel alone (candidate gather + sparse dot + "
                              "argmax); the whole call's fraction is whole_call_frac",
                     "whole_call_frac": round(head_unique / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                     "achieved": round(gather_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gather_gbs / PEAK_HBM_GBS, 4), "traffic": _traffic_bytes(),
                     "bytes_per_launch": int(head_slab), "us_per_launch": round(gather_ms * 1e3, 3),
                     "probe_GB_s": probe["GB_s"], "frac_probe": round(gather_gbs / probe["GB_s"], 4)},
        "stream_read_probe": probe,
        "cpu_baseline": cpu,
        "sweep": sweep,
        "masked": masked,
        "top_m": top_m,
        "draft_step": draft,
        "fp8_slabs": fp8,
        "skewed": skewed,
        "wide": wide,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
