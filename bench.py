"""Benchmark of the DSA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode] [--no-bwd] [--no-dense] [--no-cpu-baseline]

A step is one pass of the whole prefill path (indexer -> top-k -> sparse GQA attention) over
the 128K-token prefill workload (batch 1, L = 131072 causal, k = 2048, 64 indexer heads of
dim 128, 32 query / 4 KV heads of dim 128, keys in 16-token blocks), with every input already
resident in HBM.  The timed step is the fused dsa_prefill call; the same chunk schedule is then
driven through the C ABI's separate entry points with HIP events on the launch stream around
every kernel, which gives the per-kernel times (and the rooflines) beside it.  The attention
step runs with adjacent-query dedup (merged index sets of 8-row blocks); the fused call is also
timed with a workspace too small for the merged sets, which attends per row.  The same prefill
on inputs whose neighbouring queries select overlapping sets follows (with and without dedup).
The decode step (batch 32 over 131072-token caches, k = 2048) is timed after the prefill, eagerly
and captured in a HIP graph, then the torch.topk-shaped top-k on the decode scores, the backward
of the sparse attention and the indexer's warm-up step (target, KL and the indexer backward) on
the 32K prefill, and dense causal GQA attention on the prefill and decode shapes through torch's
fused SDPA (context lines beside the headline value).

One JSON line is printed last.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s

PREFILL = "c3_prefill_128k"
DECODE = "c4_decode_b32_128k"


def counter_traffic(kernel_key):
    """HBM bytes per launch (read + write, calibrated) from the committed counter runs, or None
    when the kernel source changed since they were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        data = json.load(open(path))
        ent = data["kernels"][kernel_key]
        cur = hashlib.sha256(open(os.path.join(ROOT, ent["source"]), "rb").read()).hexdigest()[:16]
        if cur != ent["sha256_16"]:
            return None
        return (ent["read_gb_per_launch"] + ent["write_gb_per_launch"]) * 1e9
    except (OSError, KeyError, ValueError):
        return None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default=PREFILL)
    ap.add_argument("--decode-workload", default=DECODE)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-correlated", action="store_true", help="skip the correlated-query prefill context line")
    ap.add_argument("--bwd-workload", default="c2_prefill_32k")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-attention context line")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle baseline sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for counter calibration) and exit")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n, "launches": 3}))


class Timer:
    """HIP events on torch's current stream (the stream every library call is enqueued on)."""

    def __init__(self):
        import torch
        self.torch = torch
        self.pending = {}
        self.total = {}
        self.count = {}

    def start(self, name):
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record()
        return (name, ev)

    def stop(self, tok):
        name, ev0 = tok
        ev1 = self.torch.cuda.Event(enable_timing=True)
        ev1.record()
        self.pending.setdefault(name, []).append((ev0, ev1))

    def collect(self):
        self.torch.cuda.synchronize()
        for name, evs in self.pending.items():
            for a, b in evs:
                self.total[name] = self.total.get(name, 0.0) + a.elapsed_time(b)
                self.count[name] = self.count.get(name, 0) + 1
        self.pending = {}

    def reset(self):
        self.pending, self.total, self.count = {}, {}, {}


def prefill_bench(args, dsa, inp):
    import torch
    spec = inp.WORKLOADS[args.workload]
    assert spec["kind"] == "prefill"
    t0 = time.time()
    pi = inp.workload(args.workload)
    log(f"generated {args.workload} inputs in {time.time() - t0:.1f}s")
    dev = dsa.upload_prefill_inputs(pi)
    lens = [int(x) for x in pi.seq_lens]
    total = sum(lens)
    hq, d = pi.q.shape[1], pi.q.shape[2]
    hkv = pi.k.shape[1]
    h_idx, d_idx = pi.q_idx.shape[1], pi.q_idx.shape[2]
    k = pi.top_k
    max_seqlen = max(lens)
    ld = (max_seqlen + 3) // 4 * 4
    cu = pi.cu_seqlens
    ws_bytes = dsa.dsa_prefill_workspace_size(len(lens), total, max_seqlen, hq, hkv, d, h_idx, d_idx, k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    chunk = min(total, 2048)   # the default chunk dsa_prefill_workspace_size provides for
    # A workspace with room for the chunk only: dsa_prefill then attends per row (no dedup).
    ws_chunk_bytes = (chunk * ld * 4 + 255) // 256 * 256 + dsa.dsa_topk_workspace_size(chunk, ld, k)
    # The dedup attention's merged sets (blocks of 8 rows, as dsa_prefill builds them).
    ublk = 8
    nb, cap = dsa.dsa_query_union_size(total, k, ublk)
    u_counts = torch.empty(nb, dtype=torch.int32, device="cuda")
    u_rows = torch.empty((nb, cap), dtype=torch.int32, device="cuda")
    u_masks = torch.empty((nb, cap), dtype=torch.int16, device="cuda")
    scores = ws.view(torch.float32)[: chunk * ld].view(chunk, ld)
    # Same carving as dsa_prefill: the chunk's scores, then the top-k scratch (256-byte aligned).
    topk_off = (chunk * ld * 4 + 255) // 256 * 256
    topk_ws = ws[topk_off:]
    out = torch.empty_like(dev["q"])
    lse = torch.empty(total, hq, dtype=torch.float32, device="cuda")
    idx = torch.empty(total, k, dtype=torch.int32, device="cuda")
    row_len = torch.from_numpy(np.concatenate([np.arange(1, n + 1) for n in lens]).astype(np.int32)).cuda()
    timer = Timer()

    def step():
        for b in range(len(lens)):
            o, e = int(cu[b]), int(cu[b + 1])
            for c0 in range(o, e, chunk):
                c1 = min(e, c0 + chunk)
                tok = timer.start("indexer")
                dsa.dsa_index_scores(dev["q_idx"], dev["k_idx"], dev["w"], cu, c0, c1 - c0, scores, ld=ld)
                timer.stop(tok)
                tok = timer.start("topk")
                dsa.dsa_topk(scores, row_len[c0:c1], k, idx[c0:c1], workspace=topk_ws, ld=ld)
                timer.stop(tok)
        # The attention step as dsa_prefill runs it (top-k sets never repeat a position, so every
        # 8-row block is attended from its merged set): merged sets, then the merged-set kernel.
        tok = timer.start("query_union")
        dsa.dsa_query_union(idx, dev["cu"], u_counts, u_rows, u_masks, ublk)
        timer.stop(tok)
        tok = timer.start("sparse_attn")
        dsa.dsa_sparse_gqa_attn_union(dev["q"], dev["k"], dev["v"], u_counts, u_rows, u_masks, out, lse,
                                      block_rows=ublk)
        timer.stop(tok)

    def fused(workspace=ws):
        dsa.dsa_prefill(dev["q"], dev["k"], dev["v"], dev["q_idx"], dev["k_idx"], dev["w"], dev["cu"], cu,
                        max_seqlen, k, out, lse, idx, workspace)

    # Timed region: the fused entry point, inputs already resident.
    for _ in range(args.warmup):
        fused()
    torch.cuda.synchronize()
    log(f"prefill warmup done; timing {args.steps} steps")
    t_start = time.perf_counter()
    for _ in range(args.steps):
        fused()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t_start) * 1e3 / args.steps

    # Attribution: the same schedule through the separate entry points, HIP events per kernel.
    step()
    timer.collect()
    timer.reset()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    sep_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    timer.collect()
    kern = {n: timer.total[n] / args.steps for n in timer.total}            # ms per step
    launches = {n: timer.count[n] / args.steps for n in timer.count}
    log(f"prefill {ms_per_step:.1f} ms/step (separate entry points {sep_ms:.1f}); kernels {kern}")

    # The same fused call with a workspace too small for the merged sets: attention per row.
    ws_chunk = ws[:ws_chunk_bytes]
    fused(ws_chunk)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fused(ws_chunk)
    torch.cuda.synchronize()
    no_dedup_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    out_nd = out.clone()
    fused()
    torch.cuda.synchronize()
    dd_err = (out.float() - out_nd.float()).abs()
    log(f"prefill without dedup {no_dedup_ms:.1f} ms/step; |O dedup - O per row| max {float(dd_err.max()):.2e}")

    # Algorithmic work per step.
    pairs = sum(n * (n + 1) // 2 for n in lens)
    idx_flops = pairs * 2 * h_idx * d_idx
    sel_pairs = sum(sum(min(t + 1, k) for t in range(n)) for n in lens)
    attn_bytes = sel_pairs * (2 * hkv * d * 2 + 4) + total * (2 * hq * d * 2 + 4 * hq)
    counts = u_counts.cpu().numpy().astype(np.int64)
    merged = int(counts.sum())
    padded = int(((counts + 31) // 32 * 32).sum())
    # Merged-set attention: each merged KV row's key and value rows of every group once, the
    # merged lists (int32 row + uint16 mask, padded to 32), Q in, O and lse out.
    merged_bytes = merged * hkv * d * 2 * 2 + padded * 6 + total * (2 * hq * d * 2 + 4 * hq)
    # Its MFMA work: per merged KV row and group, S^T and O^T over 8 rows x G heads (plus the row
    # sums on a ones operand, not counted).
    merged_flops = merged * hkv * 2 * (2 * ublk * (hq // hkv) * d)
    union_bytes = total * k * 4 + padded * 6
    topk_bytes = pairs * 4 + total * k * 4   # one pass over each row's scores + index write
    idx_tflops = idx_flops / (kern["indexer"] * 1e-3) / 1e12
    attn_gbs = merged_bytes / (kern["sparse_attn"] * 1e-3) / 1e9
    attn_tflops = merged_flops / (kern["sparse_attn"] * 1e-3) / 1e12
    union_gbs = union_bytes / (kern["query_union"] * 1e-3) / 1e9
    topk_gbs = topk_bytes / (kern["topk"] * 1e-3) / 1e9
    stats16 = {}
    nb16, cap16 = dsa.dsa_query_union_size(total, k, 16)
    c16 = torch.empty(nb16, dtype=torch.int32, device="cuda")
    r16 = torch.empty((nb16, cap16), dtype=torch.int32, device="cuda")
    m16 = torch.empty((nb16, cap16), dtype=torch.int16, device="cuda")
    dsa.dsa_query_union(idx, dev["cu"], c16, r16, m16, 16)
    c16 = c16.cpu().numpy()
    for t in (8192, 32768, 65536, total - 16):
        stats16[str(t)] = int(c16[min(t // 16, nb16 - 1)])
    dedup = {"block_rows": ublk, "merged_rows_per_block_mean": float(counts.mean()),
             "index_slots_per_block": ublk * k, "merged_fraction": merged / float(total * k),
             "prefill_ms_without_dedup": no_dedup_ms, "max_abs_out_vs_per_row": float(dd_err.max()),
             "union16_at_t": stats16, "union16_mean": float(c16.mean())}
    del r16, m16

    res = dict(
        pi=pi, rows_total=total, ms_per_step=ms_per_step, sep_ms=sep_ms, kern=kern, launches=launches,
        idx_flops=idx_flops, idx_tflops=idx_tflops, attn_bytes=attn_bytes, attn_gbs=attn_gbs, topk_bytes=topk_bytes,
        topk_gbs=topk_gbs, pairs=pairs, sel_pairs=sel_pairs, merged_bytes=merged_bytes,
        merged_flops=merged_flops, attn_tflops=attn_tflops, union_gbs=union_gbs, union_bytes=union_bytes, dedup=dedup,
    )
    del dev, ws, scores, out, lse, idx, u_rows, u_masks
    torch.cuda.empty_cache()
    return res


def correlated_bench(args, dsa, inp):
    """The fused prefill on the 128K workload whose neighbouring queries select overlapping sets,
    with and without dedup (the workspace decides), plus the merged-set sizes of 16-row blocks
    (the pages report about 8000 of 32768 at 128K on real inputs: context, not a target)."""
    import torch
    name = "c3q_prefill_128k_qblocks16"
    t0 = time.time()
    pi = inp.workload(name)
    log(f"generated {name} inputs in {time.time() - t0:.1f}s")
    dev = dsa.upload_prefill_inputs(pi)
    lens = [int(x) for x in pi.seq_lens]
    total, k = sum(lens), pi.top_k
    hq, d, hkv = pi.q.shape[1], pi.q.shape[2], pi.k.shape[1]
    h_idx, d_idx = pi.q_idx.shape[1], pi.q_idx.shape[2]
    max_seqlen = max(lens)
    ld = (max_seqlen + 3) // 4 * 4
    ws = torch.empty(dsa.dsa_prefill_workspace_size(1, total, max_seqlen, hq, hkv, d, h_idx, d_idx, k),
                     dtype=torch.uint8, device="cuda")
    chunk = min(total, 2048)
    ws_chunk = ws[:(chunk * ld * 4 + 255) // 256 * 256 + dsa.dsa_topk_workspace_size(chunk, ld, k)]
    out = torch.empty_like(dev["q"])
    lse = torch.empty(total, hq, dtype=torch.float32, device="cuda")
    idx = torch.empty(total, k, dtype=torch.int32, device="cuda")
    cu = pi.cu_seqlens
    res = {}
    for label, w in (("with_dedup", ws), ("without_dedup", ws_chunk)):
        dsa.dsa_prefill(dev["q"], dev["k"], dev["v"], dev["q_idx"], dev["k_idx"], dev["w"], dev["cu"], cu,
                        max_seqlen, k, out, lse, idx, w)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dsa.dsa_prefill(dev["q"], dev["k"], dev["v"], dev["q_idx"], dev["k_idx"], dev["w"], dev["cu"], cu,
                            max_seqlen, k, out, lse, idx, w)
        torch.cuda.synchronize()
        res[label] = (time.perf_counter() - t0) * 1e3 / args.steps
        if label == "with_dedup":
            out_dd = out.clone()
    err = (out_dd.float() - out.float()).abs()
    nb16, cap16 = dsa.dsa_query_union_size(total, k, 16)
    c16 = torch.empty(nb16, dtype=torch.int32, device="cuda")
    r16 = torch.empty((nb16, cap16), dtype=torch.int32, device="cuda")
    m16 = torch.empty((nb16, cap16), dtype=torch.int16, device="cuda")
    dsa.dsa_query_union(idx, dev["cu"], c16, r16, m16, 16)
    c16 = c16.cpu().numpy()
    out_j = {"workload": f"{name}: the 128K prefill with the indexer queries of each 16-token block sharing "
                         f"content (q_noise {pi.meta['q_noise']})",
             "prefill_ms_with_dedup": res["with_dedup"], "prefill_ms_without_dedup": res["without_dedup"],
             "tokens_per_s_with_dedup": total / (res["with_dedup"] * 1e-3),
             "union16_mean": float(c16.mean()),
             "union16_at_t": {str(t): int(c16[min(t // 16, nb16 - 1)]) for t in (8192, 32768, 65536, total - 16)},
             "pages_union16_at_128k_real_inputs": 8000,
             "max_abs_out_dedup_vs_per_row": float(err.max())}
    log(f"correlated-query prefill: {out_j}")
    del dev, ws, out, lse, idx, r16, m16
    torch.cuda.empty_cache()
    return out_j


def decode_bench(args, dsa, inp):
    import torch
    t0 = time.time()
    di = inp.workload(args.decode_workload)
    log(f"generated {args.decode_workload} inputs in {time.time() - t0:.1f}s")
    dev = dsa.upload_decode_inputs(di)
    batch, hq, d = di.q.shape
    s_max, hkv = di.k_cache.shape[1], di.k_cache.shape[2]
    h_idx, d_idx = di.q_idx.shape[1], di.q_idx.shape[2]
    k = di.top_k
    ws = torch.empty(dsa.dsa_decode_workspace_size(batch, s_max, hq, hkv, d, h_idx, d_idx, k), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(dev["q"])
    lse = torch.empty(batch, hq, dtype=torch.float32, device="cuda")
    idx = torch.empty(batch, k, dtype=torch.int32, device="cuda")
    max_len = int(di.seq_lens.max())

    def step():
        dsa.dsa_decode(dev["q"], dev["q_idx"], dev["w"], dev["k_cache"], dev["v_cache"], dev["k_idx_cache"],
                       dev["seq_lens"], max_len, k, out, lse, idx, ws)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    n_iter = max(20, args.steps * 4)
    evs = []
    for _ in range(n_iter):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    times = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    us_median = times[len(times) // 2]
    us_min = times[0]
    lens = di.seq_lens.astype(np.int64)
    bytes_step = int((lens * d_idx * 2).sum() + (lens * 4 * 2).sum()
                     + (np.minimum(lens, k) * (2 * hkv * d * 2 + 4)).sum() + batch * hq * d * 2 * 2)
    log(f"decode median {us_median:.1f} us (min {us_min:.1f})")

    # The same step captured once in a HIP graph and replayed: no host launch work per step.
    eager = (out.clone(), lse.clone(), idx.clone())
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    gevs = []
    for _ in range(n_iter):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        gevs.append((a, b))
    torch.cuda.synchronize()
    gtimes = sorted(a.elapsed_time(b) * 1e3 for a, b in gevs)
    graph_same = bool(torch.equal(out, eager[0]) and torch.equal(lse, eager[1]) and torch.equal(idx, eager[2]))
    graph_us = {"median": gtimes[len(gtimes) // 2], "min": gtimes[0], "same_outputs_as_eager": graph_same}
    log(f"decode in a HIP graph: median {graph_us['median']:.1f} us (min {graph_us['min']:.1f}); "
        f"outputs equal to the eager call: {graph_same}")
    del graph

    # The torch.topk-shaped top-k on the decode step's own scores (the first region of the decode
    # workspace, left there by the last step), beside the ascending form.
    ld = (s_max + 3) // 4 * 4
    scores = ws.view(torch.float32)[: batch * ld].view(batch, ld)
    row_len = dev["seq_lens"]
    tk_ws = torch.empty(dsa.dsa_topk_workspace_size(batch, ld, k), dtype=torch.uint8, device="cuda")
    idx_s = torch.empty(batch, k, dtype=torch.int32, device="cuda")
    val_s = torch.empty(batch, k, dtype=torch.float32, device="cuda")
    timing = {}
    for name, fn in (("ascending", dsa.dsa_topk), ("sorted", dsa.dsa_topk_sorted)):
        for _ in range(3):
            fn(scores, row_len, k, idx_s, val_s, workspace=tk_ws)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(20):
            fn(scores, row_len, k, idx_s, val_s, workspace=tk_ws)
        b.record()
        torch.cuda.synchronize()
        timing[name] = a.elapsed_time(b) * 1e3 / 20
        if name == "ascending":
            asc_i = idx_s.cpu().numpy().copy()
    # The sorted form holds the ascending form's set, by descending value (equal values by position).
    got_i = idx_s.cpu().numpy()
    got_v = val_s.cpu().numpy()
    ok = True
    for j in range(batch):
        order_ok = bool(np.all((got_v[j, :-1] > got_v[j, 1:]) |
                               ((got_v[j, :-1] == got_v[j, 1:]) & (got_i[j, :-1] < got_i[j, 1:]))))
        ok = ok and order_ok and bool(np.array_equal(np.sort(got_i[j]), asc_i[j]))
    topk_sorted = {"rows": batch, "row_len": int(lens.max()), "k": k, "us_sorted": timing["sorted"],
                   "us_ascending": timing["ascending"], "same_set_as_ascending_form_and_ordered": ok}
    log(f"torch.topk-shaped top-k {timing['sorted']:.1f} us (ascending form {timing['ascending']:.1f} us); "
        f"same set as the ascending form, ordered: {ok}")
    del dev, ws, tk_ws
    torch.cuda.empty_cache()
    return dict(us_median=us_median, us_min=us_min, graph_us=graph_us, bytes_step=bytes_step,
                gbs=bytes_step / (us_median * 1e-6) / 1e9, batch=batch, s_max=s_max,
                topk_sorted=topk_sorted)


def attn_bwd_bench(args, dsa, inp):
    """Backward of the sparse attention on the 32K prefill (training side), after one fused
    prefill that provides O, lse and the index sets; dO is synthetic."""
    import torch
    pi = inp.workload(args.bwd_workload)
    dev = dsa.upload_prefill_inputs(pi)
    k = pi.top_k
    out, lse, idx = dsa.prefill(dev["q"], dev["k"], dev["v"], dev["q_idx"], dev["k_idx"], dev["w"],
                                pi.cu_seqlens, k)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    dout = torch.randn(out.shape, generator=g, device="cuda").to(torch.bfloat16)
    dq = torch.empty(out.shape, dtype=torch.float32, device="cuda")
    dk = torch.empty(dev["k"].shape, dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)

    def run():
        dsa.dsa_sparse_gqa_attn_bwd(dev["q"], dev["k"], dev["v"], out, lse, dout, idx, dev["cu"], dq, dk, dv)

    run()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(3):
        run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 3
    a.record()
    dsa.dsa_sparse_gqa_attn(dev["q"], dev["k"], dev["v"], idx, dev["cu"], out, lse)
    b.record()
    torch.cuda.synchronize()
    fwd_ms = a.elapsed_time(b)
    lens = [int(x) for x in pi.seq_lens]
    hkv, d = pi.k.shape[1], pi.k.shape[2]
    sel_pairs = sum(sum(min(t + 1, k) for t in range(n)) for n in lens)
    # per selected (row, KV group): K and V rows gathered (2 x 256 B) and 2 x 128 fp32 atomics
    algo_bytes = sel_pairs * hkv * (2 * d * 2 + 2 * d * 4)
    total = sum(lens)
    log(f"attention backward {ms:.1f} ms (forward {fwd_ms:.1f} ms) on {args.bwd_workload}")
    del dev, dq, dk, dv, dout, out, lse, idx
    torch.cuda.empty_cache()
    return {"workload": args.bwd_workload, "ms": ms, "forward_ms": fwd_ms, "tokens_per_s": total / (ms * 1e-3),
            "algorithmic_gb_per_s": algo_bytes / (ms * 1e-3) / 1e9,
            "note": "dq, dk, dv from dO; dk/dv scattered with fp32 atomics (bound by L2 atomic throughput)"}


def warmup_bench(args, dsa, inp):
    """The indexer's dense warm-up step on the 32K prefill: per chunk of 2048 rows the indexer
    scores, the head-mean causal attention target, the per-row KL with its gradient, and that
    gradient's backward through the indexer (dq_idx, dw, dk_idx)."""
    import torch
    pi = inp.workload(args.bwd_workload)
    dev = dsa.upload_prefill_inputs(pi)
    lens = [int(x) for x in pi.seq_lens]
    total = sum(lens)
    hq, d = pi.q.shape[1], pi.q.shape[2]
    ld = (max(lens) + 3) // 4 * 4
    chunk = min(total, 2048)
    scores = torch.empty(chunk, ld, dtype=torch.float32, device="cuda")
    probs = torch.empty(chunk, ld, dtype=torch.float32, device="cuda")
    lse = torch.empty(chunk, hq, dtype=torch.float32, device="cuda")
    loss = torch.empty(total, dtype=torch.float32, device="cuda")
    row_len = torch.from_numpy(np.concatenate([np.arange(1, n + 1) for n in lens]).astype(np.int32)).cuda()
    cu = pi.cu_seqlens
    h_idx, d_idx = pi.q_idx.shape[1], pi.q_idx.shape[2]
    dq = torch.empty(total, h_idx, d_idx, dtype=torch.float32, device="cuda")
    dw = torch.empty(total, h_idx, dtype=torch.float32, device="cuda")
    dk = torch.empty(total, d_idx, dtype=torch.float32, device="cuda")
    t_target = []
    t_bwd = []

    def timed(fn, into):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        into.append((a, b))

    def step():
        dk.zero_()
        for c0 in range(0, total, chunk):
            n = min(chunk, total - c0)
            dsa.dsa_index_scores(dev["q_idx"], dev["k_idx"], dev["w"], cu, c0, n, scores, ld=ld)
            timed(lambda: dsa.dsa_attn_head_mean(dev["q"], dev["k"], cu, c0, n, probs, lse, ld=ld), t_target)
            dsa.dsa_indexer_kl(scores, probs, row_len[c0:c0 + n], loss[c0:c0 + n], scores, ld=ld)
            timed(lambda: dsa.dsa_index_scores_bwd(dev["q_idx"], dev["k_idx"], dev["w"], cu, c0, n, scores, dq, dw, dk,
                                                   ld=ld), t_bwd)

    step()
    torch.cuda.synchronize()
    t_target.clear()
    t_bwd.clear()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    target_ms = sum(a.elapsed_time(b) for a, b in t_target)
    bwd_ms = sum(a.elapsed_time(b) for a, b in t_bwd)
    pairs = sum(n * (n + 1) // 2 for n in lens)
    target_flops = 2 * pairs * 2 * hq * d          # two passes of the causal Q K^T, all heads
    bwd_flops = 3 * pairs * 2 * h_idx * d_idx      # recompute c, then u (-> dq, dw) and dk
    log(f"indexer warm-up step {ms:.1f} ms per pass (target {target_ms:.1f} ms, "
        f"{target_flops / (target_ms * 1e-3) / 1e12:.0f} TFLOP/s; indexer backward {bwd_ms:.1f} ms, "
        f"{bwd_flops / (bwd_ms * 1e-3) / 1e12:.0f} TFLOP/s)")
    del dev, scores, probs, lse, loss, dq, dw, dk
    torch.cuda.empty_cache()
    return {"workload": args.bwd_workload, "ms": ms, "tokens_per_s": total / (ms * 1e-3), "target_ms": target_ms,
            "target_tflops": target_flops / (target_ms * 1e-3) / 1e12,
            "indexer_bwd_ms": bwd_ms, "indexer_bwd_tflops": bwd_flops / (bwd_ms * 1e-3) / 1e12,
            "note": "indexer scores + head-mean dense attention target + per-row KL and d loss / d scores + "
                    "the indexer backward (dq_idx, dw, dk_idx); backward TFLOP/s counts 3 x 2 H_I d_I flop per "
                    "causal pair"}


def measured_peaks(dsa):
    """What the box reaches on the two priced resources (the library's probe kernels): an
    MFMA-only loop of 16x16x32 and of 32x32x16 bf16 instructions, and a streaming read of 4 GiB.
    Best of several timed launches each."""
    import torch

    def best_ms(fn, reps):
        fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b))
        return min(out)

    grid, iters = 2048, 20000
    sink = torch.zeros(1 << 16, dtype=torch.float32, device="cuda")
    res = {}
    for shape in (16, 32):
        flops = dsa.dsa_probe_mfma_bf16(shape, grid, iters, sink)
        ms = best_ms(lambda: dsa.dsa_probe_mfma_bf16(shape, grid, iters, sink), 5)
        res[f"mfma_bf16_{shape}x{shape}x{512 // shape}_tflops"] = flops / (ms * 1e-3) / 1e12
    buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    best = {g: buf.numel() / (best_ms(lambda: dsa.dsa_probe_stream_read(buf, g, sink), 6) * 1e-3) / 1e9
            for g in (2048, 8192, 16384, 32768, 65536)}
    res["stream_read_gbs"] = max(best.values())
    res["stream_read_gbs_by_grid"] = best
    del buf, sink
    torch.cuda.empty_cache()
    log(f"measured peaks: {res}")
    return res


def _sdpa_first_backend(torch, fn):
    """Run fn under the first fused SDPA backend that accepts it (flash, then memory-efficient;
    never the math backend, which would materialise the score matrix).  Returns (name, result)."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    for name, backend in (("flash", SDPBackend.FLASH_ATTENTION), ("efficient", SDPBackend.EFFICIENT_ATTENTION)):
        try:
            with sdpa_kernel([backend]):
                res = fn()
            torch.cuda.synchronize()
            return name, res
        except RuntimeError as e:
            log(f"torch SDPA backend {name} refused: {str(e).splitlines()[0][:160]}")
    return None, None


def dense_bench(args, dsa, inp, dsa_prefill_ms, dsa_decode_us):
    """Dense causal GQA attention on the same shapes through torch's fused SDPA (context for the
    sparse path's ratio to full attention; not a path of this library)."""
    import math
    import torch
    import torch.nn.functional as F

    def timed_ms(fn, n):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    res = {"what": "torch.nn.functional.scaled_dot_product_attention on the benchmark shapes (K/V heads "
                   "repeated per query head in prefill; the query heads of a group as query rows in decode)"}
    pi = inp.workload(args.workload)
    q = dsa.to_device_bf16(pi.q)
    total, hq, d = q.shape
    hkv = pi.k.shape[1]
    grp = hq // hkv
    scale = 1.0 / math.sqrt(d)
    qh = q.permute(1, 0, 2).unsqueeze(0).contiguous()
    kh = dsa.to_device_bf16(pi.k).permute(1, 0, 2).repeat_interleave(grp, dim=0).unsqueeze(0).contiguous()
    vh = dsa.to_device_bf16(pi.v).permute(1, 0, 2).repeat_interleave(grp, dim=0).unsqueeze(0).contiguous()
    fn = lambda: F.scaled_dot_product_attention(qh, kh, vh, is_causal=True, scale=scale)  # noqa: E731
    backend, o = _sdpa_first_backend(torch, fn)
    if backend is not None:
        # Cross-check on the rows whose top-k keeps every position (t < k): there the sparse
        # attention is the dense one.
        k_sel = pi.top_k
        n = min(k_sel, total)
        pos = torch.arange(k_sel, dtype=torch.int32, device="cuda")
        idx = torch.where(pos[None, :] <= pos[:n, None], pos[None, :], torch.full_like(pos[None, :], -1))
        cu = torch.tensor([0, n], dtype=torch.int32, device="cuda")
        o_sp = torch.empty((n, hq, d), dtype=torch.bfloat16, device="cuda")
        dsa.dsa_sparse_gqa_attn(q[:n].contiguous(), dsa.to_device_bf16(pi.k[:n]), dsa.to_device_bf16(pi.v[:n]),
                                idx.contiguous(), cu, o_sp, softmax_scale=scale)
        o_dense = o[0].permute(1, 0, 2)[:n].float()
        ms = timed_ms(fn, 3)
        causal_flops = 4.0 * hq * d * total * (total + 1) / 2
        floor_ms = causal_flops / (PEAK_BF16_TFLOPS * 1e12) * 1e3
        res["prefill"] = {"backend": backend, "ms": ms, "tflops": causal_flops / (ms * 1e-3) / 1e12,
                          "dsa_prefill_over_dense": dsa_prefill_ms / ms,
                          "dense_floor_ms_at_bf16_peak": floor_ms,
                          "dsa_prefill_over_dense_floor": dsa_prefill_ms / floor_ms,
                          "max_abs_vs_sparse_attn_all_positions_rows_below_k": float((o_dense - o_sp.float()).abs().max())}
        log(f"dense prefill ({backend}): {ms:.1f} ms; DSA prefill / dense = {dsa_prefill_ms / ms:.3f}")
    del q, qh, kh, vh, o
    torch.cuda.empty_cache()

    if dsa_decode_us is not None:
        di = inp.workload(args.decode_workload)
        batch, s_max = di.k_cache.shape[0], di.k_cache.shape[1]
        qd = dsa.to_device_bf16(di.q).view(batch, hkv, grp, d)
        kd = dsa.to_device_bf16(di.k_cache).permute(0, 2, 1, 3).contiguous()
        vd = dsa.to_device_bf16(di.v_cache).permute(0, 2, 1, 3).contiguous()
        fn = lambda: F.scaled_dot_product_attention(qd, kd, vd, scale=scale)  # noqa: E731
        backend, _ = _sdpa_first_backend(torch, fn)
        if backend is not None:
            us = timed_ms(fn, 20) * 1e3
            nbytes = 2 * kd.numel() * 2
            floor_us = nbytes / (PEAK_HBM_GBS * 1e9) * 1e6
            res["decode"] = {"backend": backend, "us": us, "gbs": nbytes / (us * 1e-6) / 1e9,
                             "dsa_decode_over_dense": dsa_decode_us / us,
                             "dense_floor_us_at_hbm_peak": floor_us,
                             "dsa_decode_over_dense_floor": dsa_decode_us / floor_us}
            log(f"dense decode ({backend}): {us:.1f} us; DSA decode / dense = {dsa_decode_us / us:.3f}")
        del qd, kd, vd
        torch.cuda.empty_cache()
    return res


def cpu_baseline(args, pi):
    """The oracle as it stands, on a bounded sample of rows of the same workload (the only leg of
    the benchmark that runs it)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import dsa_testlib as tl
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    total = sum(int(x) for x in pi.seq_lens)
    rng = np.random.default_rng(123)
    rows = rng.integers(0, total, 4096).tolist()
    done = 0
    t0 = time.perf_counter()
    while done < len(rows) and time.perf_counter() - t0 < args.cpu_seconds:
        tl.oracle_prefill_rows_lazy(pi, rows[done:done + 4])
        done += 4
    el = time.perf_counter() - t0
    work_sample = sum(r + 1 for r in rows[:done])           # indexer work grows with the prefix length
    work_all = total * (total + 1) / 2
    rows_per_s = done / el
    tokens_per_s = total / (el * work_all / work_sample)     # whole-job rate, extrapolated by work
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} uniformly drawn rows of the 128K prefill in {el:.1f}s ({rows_per_s:.2f} rows/s); "
                      f"whole-job rate extrapolated by causal work (sum of t+1)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported (the library has no "
              f"multi-GPU path; the sharding it would take is described in the design notes)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch
    import sparse_long_context_lightning_amd as dsa
    from sparse_long_context_lightning_amd import inputs as inp

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dsa.load()
    pre = prefill_bench(args, dsa, inp)
    peaks = measured_peaks(dsa)
    corr = None if args.no_correlated else correlated_bench(args, dsa, inp)
    dec = None if args.no_decode else decode_bench(args, dsa, inp)
    bwd = None if args.no_bwd else attn_bwd_bench(args, dsa, inp)
    wup = None if args.no_bwd else warmup_bench(args, dsa, inp)
    dense = None if args.no_dense else dense_bench(args, dsa, inp, pre["ms_per_step"],
                                                   None if dec is None else dec["us_median"])
    cpu = None if args.no_cpu_baseline else cpu_baseline(args, pre["pi"])

    total = pre["rows_total"]
    value = total / (pre["ms_per_step"] * 1e-3)
    kern = pre["kern"]
    line = {
        "metric": "DSA prefill tokens/s at 128K (k=2048) + decode µs/step; % HBM/MFMA peak",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill_128k_blocks16: batch 1, L=131072 causal, k=2048, indexer 64x128 bf16, "
                               "GQA 32q/4kv heads x 128",
                   "global_batch": 1, "seq_len": total, "top_k": 2048},
        "separate_entry_points_ms_per_step": pre["sep_ms"],
        "kernel_ms_per_step": kern,
        "kernel_launches_per_step": pre["launches"],
        "roofline": {"bound": "mfma", "kernel": "indexer_prefill", "achieved": pre["idx_tflops"],
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": pre["idx_tflops"] / PEAK_BF16_TFLOPS,
                     "traffic": counter_traffic("indexer_prefill_kernel@prefill_128k"),
                     "traffic_unit": "bytes per launch (HBM read+write, rocprofv3 FETCH_SIZE/WRITE_SIZE, calibrated)",
                     "algorithmic_flops_per_launch": pre["idx_flops"] / pre["launches"]["indexer"],
                     "measured_peak": peaks["mfma_bf16_16x16x32_tflops"],
                     "frac_of_measured_peak": pre["idx_tflops"] / peaks["mfma_bf16_16x16x32_tflops"],
                     "avg_launch_ms": pre["kern"]["indexer"] / pre["launches"]["indexer"]},
        "roofline_sparse_attn": {"bound": "hbm", "kernel": "sparse_attn_union (8-row blocks)",
                                 "achieved": pre["attn_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                 "frac": pre["attn_gbs"] / PEAK_HBM_GBS,
                                 "measured_peak": peaks["stream_read_gbs"],
                                 "frac_of_measured_peak": pre["attn_gbs"] / peaks["stream_read_gbs"],
                                 "traffic": counter_traffic("sparse_attn_union_kernel@prefill_128k"),
                                 "algorithmic_bytes_per_launch": pre["merged_bytes"],
                                 "mfma_tflops": pre["attn_tflops"], "mfma_frac": pre["attn_tflops"] / PEAK_BF16_TFLOPS,
                                 "bytes_without_dedup": pre["attn_bytes"]},
        "roofline_query_union": {"bound": "hbm", "achieved": pre["union_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                 "frac": pre["union_gbs"] / PEAK_HBM_GBS,
                                 "algorithmic_bytes_per_launch": pre["union_bytes"]},
        "measured_peaks": peaks,
        "dedup": pre["dedup"],
        "prefill_correlated_queries": corr,
        "roofline_topk": {"bound": "hbm", "achieved": pre["topk_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": pre["topk_gbs"] / PEAK_HBM_GBS},
        "cpu_baseline": cpu,
    }
    if dec is not None:
        line["decode_us_per_step"] = dec["us_median"]
        line["decode_us_min"] = dec["us_min"]
        line["decode_us_per_step_hip_graph"] = dec["graph_us"]
        line["decode_config"] = {"workload": "decode_b32_128k: batch 32, 131072-token caches, k=2048"}
        line["roofline_decode"] = {"bound": "hbm", "achieved": dec["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": dec["gbs"] / PEAK_HBM_GBS,
                                   "frac_of_measured_peak": dec["gbs"] / peaks["stream_read_gbs"]}
        line["topk_sorted_decode_scores"] = dec["topk_sorted"]
    if bwd is not None:
        line["sparse_attn_backward"] = bwd
    if wup is not None:
        line["indexer_warmup_objective"] = wup
    if dense is not None:
        line["dense_attention_context"] = dense
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
