"""Benchmark of the DSA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode] [--no-extra] [--no-bwd] [--no-dense]
                    [--no-correlated] [--no-cpu-baseline]

A step is one pass of the whole prefill path (indexer -> top-k -> sparse GQA attention) over
the 128K-token prefill workload (batch 1, L = 131072 causal, k = 2048, 64 indexer heads of
dim 128, 32 query / 4 KV heads of dim 128, keys in 16-token blocks), with every input already
resident in HBM.  The timed step is the fused dsa_prefill call; the same call is then repeated
with the library's launch timing on (dsa_timing_enable: two HIP events on the launch stream
around each of its launches), which gives the per-kernel times of that very schedule (and the
rooflines) beside it.  The attention step runs with adjacent-query dedup (merged index sets of
8-row blocks); the fused call is also timed with a workspace too small for the merged sets,
which attends per row.

Each sparse-attention kernel is read three ways: its HBM traffic from the committed rocprofv3
counter runs (FETCH_SIZE + WRITE_SIZE, calibrated) over its time against the 8 TB/s peak, its
algorithmic gather bytes over its time (an "effective" rate that L2 and last-level-cache reuse
can push past the peak), and against a gather probe (libdsa_probes.so) that reads exactly the
same key and value rows in the same work order with no arithmetic, the achievable ceiling of
that access pattern on the box.

Also timed: the decode step (batch 32 over 131072-token caches, k = 2048), eagerly, per kernel
through the separate entry points, and captured in a HIP graph; the 256K long-video mix (packed
262144 + 65536 + 8192-token prefill, then batch-8 decode over 262144-token caches) and the 32K
prefill as extra fields; the correlated-query 128K prefill with and without dedup; the
torch.topk-shaped top-k on the decode scores; the backward of the sparse attention and the
indexer's warm-up step on the 32K prefill; dense causal GQA attention on the prefill and decode
shapes through torch's fused SDPA (context); and the CPU oracle on sampled rows of the same
128K workload (its rate, and its agreement with the timed run's outputs on those rows and on
every decode row).

One JSON line is printed last.
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
MAX_ENGINE_CLOCK_GHZ = 2.4    # the engine clock at which that peak is quoted

PREFILL = "c3_prefill_128k"
DECODE = "c4_decode_b32_128k"
EXTRA_PREFILL = ("c5_video_mix_prefill", "c2_prefill_32k")
EXTRA_DECODE = ("c5_video_mix_decode",)
CPU_SAMPLE_ROWS = 4096       # candidate rows of the oracle sample (drawn before the timed run)


def counter_entry(kernel_key):
    """Committed counter-run figures of one kernel on one workload (profiles/counters.json), or
    None when the kernel's source changed since they were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        data = json.load(open(path))
        ent = data["kernels"][kernel_key]
        cur = hashlib.sha256(open(os.path.join(ROOT, ent["source"]), "rb").read()).hexdigest()[:16]
        if cur != ent["sha256_16"]:
            return None
        return ent
    except (OSError, KeyError, ValueError):
        return None


def counter_traffic(kernel_key):
    """HBM bytes per launch (read + write, calibrated) from the committed counter runs, or None."""
    ent = counter_entry(kernel_key)
    return None if ent is None else (ent["read_gb_per_launch"] + ent["write_gb_per_launch"]) * 1e9


def hbm_roofline(kernel, kernel_key, avg_launch_ms, algorithmic_bytes, ceiling=None, **extra):
    """An HBM-bound kernel read against the 8 TB/s peak: achieved = counter bytes per launch over
    the launch's average time (null when no current counter run exists), beside the algorithmic
    bytes' effective rate and, where given, the gather probe's ceiling on the same rows."""
    traffic = counter_traffic(kernel_key)
    achieved = None if traffic is None else traffic / (avg_launch_ms * 1e-3) / 1e9
    r = {"bound": "hbm", "kernel": kernel, "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
         "frac": None if achieved is None else achieved / PEAK_HBM_GBS, "traffic": traffic,
         "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated; FETCH_SIZE counts L2 "
                         "misses, Infinity Cache hits included)",
         "avg_launch_ms": avg_launch_ms, "algorithmic_bytes_per_launch": algorithmic_bytes,
         "effective_algorithmic_gbs": algorithmic_bytes / (avg_launch_ms * 1e-3) / 1e9}
    if ceiling is not None:
        r["gather_ceiling"] = dict(ceiling, frac_of_ceiling=ceiling["ms"] / avg_launch_ms)
    r.update(extra)
    return r


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
    ap.add_argument("--no-extra", action="store_true", help="skip the 256K video-mix and 32K extra fields")
    ap.add_argument("--no-correlated", action="store_true", help="skip the correlated-query prefill context line")
    ap.add_argument("--bwd-workload", default="c2_prefill_32k")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-attention context line")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle baseline sample")
    ap.add_argument("--training-only", action="store_true",
                    help="run only the training-side sections (attention backward, indexer warm-up) and print them")
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


def best_ms(fn, reps=3):
    """Best of `reps` event-timed calls (after one untimed call)."""
    import torch
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


def gather_ceiling(dsa, k, v, idx, nsplits=(1,), row_stride=0, group_fastest=False):
    """The gather probe over the same key / value rows in the same work order, with both load
    shapes (64-byte pieces of 16 rows per instruction, or 4 whole rows per instruction), 1, 2 and 4
    chunks in flight per wave and each given number of index ranges per row (one wave each): the
    best time is the achievable ceiling of that access pattern."""
    import torch
    rows = idx.shape[0]
    hkv = k.shape[1]
    wgs = ((rows * hkv * max(nsplits) + 3) // 4 + 7) // 8 * 8
    sink = torch.zeros(wgs, dtype=torch.int32, device="cuda")
    by_cfg = {}
    for whole in (False, True):
        for nsplit in nsplits:
            for depth in (1, 2, 4):
                by_cfg[f"{'whole_rows' if whole else 'row_pieces'}_nsplit{nsplit}_depth{depth}"] = best_ms(
                    lambda: dsa.dsa_probe_gather(k, v, idx, sink, nsplit=nsplit, row_stride=row_stride,
                                                 group_fastest=group_fastest, depth=depth, whole_rows=whole))
    best = min(by_cfg, key=by_cfg.get)
    return {"ms": by_cfg[best], "config": best, "ms_by_config": by_cfg,
            "what": "dsa_probe_gather: the same K and V rows, same work order, no arithmetic"}


def prefill_section(args, dsa, inp, name, steps, warmup, full):
    """The fused prefill on workload `name` (the timed step), then the same fused call with the
    library's launch timing on (HIP events on the launch stream around each of its launches) for
    per-kernel times and rooflines.  `full` adds the prefill without dedup, the 16-row merged-set
    statistics, the gather ceilings and the rows kept for the oracle's check."""
    import torch
    t0 = time.time()
    pi = inp.workload(name)
    log(f"generated {name} inputs in {time.time() - t0:.1f}s")
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
    # Same carving as dsa_prefill: the chunk's score rows, then the top-k scratch (256-byte aligned;
    # per row a threshold, a candidate count and a redo flag, then the candidate lists).
    topk_off = (chunk * ld * 4 + 255) // 256 * 256
    out = torch.empty_like(dev["q"])
    lse = torch.empty(total, hq, dtype=torch.float32, device="cuda")
    idx = torch.empty(total, k, dtype=torch.int32, device="cuda")

    def fused(workspace=ws):
        dsa.dsa_prefill(dev["q"], dev["k"], dev["v"], dev["q_idx"], dev["k_idx"], dev["w"], dev["cu"], cu,
                        max_seqlen, k, out, lse, idx, workspace)

    # Timed region: the fused entry point, inputs already resident.
    for _ in range(warmup):
        fused()
    torch.cuda.synchronize()
    log(f"{name}: prefill warmup done; timing {steps} steps")
    t_start = time.perf_counter()
    for _ in range(steps):
        fused()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t_start) * 1e3 / steps

    samples = None
    if full:
        # The timed run's outputs on the rows the oracle may check (drawn before it runs).
        cand = np.random.default_rng(123).integers(0, total, CPU_SAMPLE_ROWS)
        sel = torch.from_numpy(cand.astype(np.int64)).cuda()
        samples = {"rows": cand.tolist(), "idx": idx[sel].cpu().numpy(), "out": out[sel].float().cpu().numpy(),
                   "lse": lse[sel].cpu().numpy()}

    # Attribution: the same fused call with the library's launch timing on (two HIP events on the
    # launch stream around each launch, summed per launch name); the timed region ran with it off.
    dsa.dsa_timing_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        fused()
    torch.cuda.synchronize()
    timing_on_ms = (time.perf_counter() - t0) * 1e3 / steps
    rec = dsa.dsa_timing_read()
    dsa.dsa_timing_enable(False)
    kern = {n: ms / steps for n, (ms, c) in rec.items()}            # ms per step
    launches = {n: c / steps for n, (ms, c) in rec.items()}
    log(f"{name}: prefill {ms_per_step:.1f} ms/step (with launch timing {timing_on_ms:.1f}); kernels "
        + ", ".join(f"{n} {v:.2f}" for n, v in kern.items()))

    # The fused top-k's candidate counts of the last chunk: the chunk-only workspace leaves the
    # top-k scratch intact (the merged sets of the dedup attention would reuse it).
    fused(ws[:ws_chunk_bytes])
    torch.cuda.synchronize()
    last_rows = (lens[-1] - 1) % chunk + 1
    cnt = ws[topk_off + 4 * chunk: topk_off + 8 * chunk].view(torch.int32)[:last_rows].cpu().numpy()
    last_n = np.arange(lens[-1] - last_rows + 1, lens[-1] + 1)
    cand_mean = float(cnt[last_n > k].mean()) if (last_n > k).any() else 0.0

    res = {"name": name, "pi": pi, "rows_total": total, "ms_per_step": ms_per_step, "timing_on_ms": timing_on_ms,
           "kern": kern, "launches": launches, "samples": samples, "candidates_per_row_mean": cand_mean}
    if full:
        # The same fused call with a workspace too small for the merged sets: attention per row.
        ws_chunk = ws[:ws_chunk_bytes]
        fused(ws_chunk)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fused(ws_chunk)
        torch.cuda.synchronize()
        res["no_dedup_ms"] = (time.perf_counter() - t0) * 1e3 / steps
        out_nd = out.clone()
        # the per-row kernel alone on the same sets, for its own gather ceiling
        res["per_row_attn_ms"] = best_ms(lambda: dsa.dsa_sparse_gqa_attn(dev["q"], dev["k"], dev["v"], idx, dev["cu"],
                                                                         out_nd, None))
        dsa.dsa_sparse_gqa_attn(dev["q"], dev["k"], dev["v"], idx, dev["cu"], out_nd, None)
        fused()
        torch.cuda.synchronize()
        res["max_abs_out_vs_per_row"] = float((out.float() - out_nd.float()).abs().max())
        log(f"{name}: prefill without dedup {res['no_dedup_ms']:.1f} ms/step; per-row attention kernel "
            f"{res['per_row_attn_ms']:.1f} ms; |O dedup - O per row| max {res['max_abs_out_vs_per_row']:.2e}")
        del out_nd
        # Gather ceilings: the per-row kernel's rows (every selected position of every row, KV
        # group slowest) and the merged-set kernel's rows (every merged KV row of every 8-row
        # block), each through the gather probe.
        if len(lens) == 1:
            res["ceiling_per_row"] = gather_ceiling(dsa, dev["k"], dev["v"], idx)
            dsa.dsa_query_union(idx, dev["cu"], u_counts, u_rows, u_masks, ublk)
            merged_idx = torch.where(torch.arange(cap, device="cuda")[None, :] < u_counts[:, None], u_rows,
                                     torch.full_like(u_rows, -1))
            res["ceiling_merged"] = gather_ceiling(dsa, dev["k"], dev["v"], merged_idx)
            del merged_idx
            log(f"{name}: gather ceilings per row {res['ceiling_per_row']['ms']:.1f} ms, merged sets "
                f"{res['ceiling_merged']['ms']:.1f} ms")

    # Algorithmic work per step.
    pairs = sum(n * (n + 1) // 2 for n in lens)
    idx_flops = pairs * 2 * h_idx * d_idx
    sel_pairs = sum(sum(min(t + 1, k) for t in range(n)) for n in lens)
    attn_bytes = sel_pairs * (2 * hkv * d * 2 + 4) + total * (2 * hq * d * 2 + 4 * hq)
    dsa.dsa_query_union(idx, dev["cu"], u_counts, u_rows, u_masks, ublk)
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
    # The fused top-k (indexer_emit is the indexer itself; its candidate appends are counted here):
    # per row with more than k positions, 2048 sample floats written and read and its candidates
    # (key, position) written and read; every row's k indices written.
    ikey = "indexer_emit" if "indexer_emit" in kern else "indexer"
    topk_parts = [n for n in ("indexer_sample", "topk_threshold", "topk_select", "indexer_rescore", "topk_redo",
                              "topk") if n in kern]
    rows_long = sum(max(0, n - k) for n in lens)
    topk_bytes = rows_long * (2048 * 4 * 2 + cand_mean * 8 * 2) + total * k * 4
    topk_ms = sum(kern[n] for n in topk_parts)
    res.update(pairs=pairs, idx_flops=idx_flops, sel_pairs=sel_pairs, attn_bytes=attn_bytes, merged=merged,
               merged_bytes=merged_bytes, merged_flops=merged_flops, union_bytes=union_bytes, topk_bytes=topk_bytes,
               indexer_key=ikey, topk_parts=topk_parts, topk_ms=topk_ms,
               idx_tflops=idx_flops / (kern[ikey] * 1e-3) / 1e12,
               attn_tflops=merged_flops / (kern["sparse_attn_union"] * 1e-3) / 1e12,
               union_gbs=union_bytes / (kern["query_union"] * 1e-3) / 1e9,
               topk_gbs=topk_bytes / (topk_ms * 1e-3) / 1e9,
               merged_fraction=merged / float(sel_pairs), block_rows=ublk,
               merged_rows_per_block_mean=float(counts.mean()))
    if full:
        stats16 = {}
        nb16, cap16 = dsa.dsa_query_union_size(total, k, 16)
        c16 = torch.empty(nb16, dtype=torch.int32, device="cuda")
        r16 = torch.empty((nb16, cap16), dtype=torch.int32, device="cuda")
        m16 = torch.empty((nb16, cap16), dtype=torch.int16, device="cuda")
        dsa.dsa_query_union(idx, dev["cu"], c16, r16, m16, 16)
        c16 = c16.cpu().numpy()
        for t in (8192, 32768, 65536, total - 16):
            stats16[str(t)] = int(c16[min(t // 16, nb16 - 1)])
        res["union16_at_t"] = stats16
        res["union16_mean"] = float(c16.mean())
        del r16, m16
    del dev, ws, out, lse, idx, u_rows, u_masks
    torch.cuda.empty_cache()
    return res


def indexer_roofline(pre, counter_key=None):
    ik = pre["indexer_key"]
    r = {"bound": "mfma", "kernel": "indexer_prefill_kernel<64, 128, 4, 2> (the fused top-k's emitting pass)"
                                    if ik == "indexer_emit" else "indexer_prefill_kernel",
         "achieved": pre["idx_tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
         "frac": pre["idx_tflops"] / PEAK_BF16_TFLOPS,
         "algorithmic_flops_per_launch": pre["idx_flops"] / pre["launches"][ik],
         "avg_launch_ms": pre["kern"][ik] / pre["launches"][ik]}
    if counter_key:
        r["traffic"] = counter_traffic(counter_key)
        r["traffic_unit"] = "bytes per launch (HBM read+write, rocprofv3 FETCH_SIZE/WRITE_SIZE, calibrated)"
        ent = counter_entry(counter_key)
        if ent is not None and "shader_clock_ghz" in ent:
            # The 2.5 PFLOP/s peak holds at the 2.4 GHz maximum engine clock; the committed clock
            # pass measures the clock this kernel actually runs at (power-limited below 2.4 GHz).
            clk = ent["shader_clock_ghz"]
            r["shader_clock_ghz_by_counters"] = clk
            r["peak_at_that_clock"] = PEAK_BF16_TFLOPS * clk / MAX_ENGINE_CLOCK_GHZ
            r["frac_at_that_clock"] = pre["idx_tflops"] / r["peak_at_that_clock"]
    return r


def prefill_summary(pre):
    """Extra-field summary of a prefill section (the 256K mix, the 32K prefill)."""
    kern = pre["kern"]
    return {"workload": pre["name"], "tokens": pre["rows_total"], "ms_per_step": pre["ms_per_step"],
            "tokens_per_s": pre["rows_total"] / (pre["ms_per_step"] * 1e-3),
            "ms_per_step_with_launch_timing": pre["timing_on_ms"], "kernel_ms_per_step": kern,
            "roofline_indexer": indexer_roofline(pre),
            "sparse_attn_effective_algorithmic_gbs": pre["merged_bytes"] / (kern["sparse_attn_union"] * 1e-3) / 1e9,
            "indexer_plus_topk_ms_per_step": kern[pre["indexer_key"]] + pre["topk_ms"],
            "merged_rows_per_8_row_block_mean": pre["merged_rows_per_block_mean"],
            "topk_gbs": pre["topk_gbs"]}


def decode_section(args, dsa, inp, name, full):
    """The decode step on workload `name`: eager median, per kernel through the separate entry points
    (decode indexer, top-k, decode attention), the attention's gather ceiling; `full` adds the step
    captured in a HIP graph and the torch.topk-shaped top-k on the step's scores."""
    import torch
    t0 = time.time()
    di = inp.workload(name)
    log(f"generated {name} inputs in {time.time() - t0:.1f}s")
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

    def timed_median(fn, n_iter):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        evs = []
        for _ in range(n_iter):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        times = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        return times[len(times) // 2], times[0]

    n_iter = max(20, args.steps * 4)
    us_median, us_min = timed_median(step, n_iter)
    samples = {"idx": idx.cpu().numpy(), "out": out.float().cpu().numpy(), "lse": lse.cpu().numpy()}
    lens = di.seq_lens.astype(np.int64)
    idx_bytes = int((lens * d_idx * 2).sum())
    score_bytes = int((lens * 4).sum())
    attn_bytes = int((np.minimum(lens, k) * (2 * hkv * d * 2 + 4)).sum() + batch * hq * d * 2 * 2)
    bytes_step = idx_bytes + 2 * score_bytes + attn_bytes
    log(f"{name}: decode median {us_median:.1f} us (min {us_min:.1f})")

    # Per kernel through the separate entry points (same kernels, same order, same buffers).
    ld = (s_max + 3) // 4 * 4
    scores = torch.empty(batch, ld, dtype=torch.float32, device="cuda")
    tk_ws = torch.empty(dsa.dsa_topk_workspace_size(batch, ld, k), dtype=torch.uint8, device="cuda")
    at_ws_n = dsa.dsa_sparse_gqa_attn_decode_workspace_size(batch, hq, hkv, k)
    at_ws = torch.empty(max(at_ws_n, 16), dtype=torch.uint8, device="cuda")
    idx2 = torch.empty_like(idx)
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    per = {}
    per["indexer"] = timed_median(lambda: dsa.dsa_decode_index_scores(dev["q_idx"], dev["w"], dev["k_idx_cache"],
                                                                       dev["seq_lens"], max_len, scores), n_iter)[0]
    per["topk"] = timed_median(lambda: dsa.dsa_topk(scores, dev["seq_lens"], k, idx2, workspace=tk_ws), n_iter)[0]
    per["attention"] = timed_median(lambda: dsa.dsa_sparse_gqa_attn_decode(dev["q"], dev["k_cache"], dev["v_cache"],
                                                                          idx2, dev["seq_lens"], out2, lse2,
                                                                          workspace=at_ws), n_iter)[0]
    torch.cuda.synchronize()
    same = bool(torch.equal(idx, idx2) and torch.equal(out.view(torch.int16), out2.view(torch.int16)))
    ceiling = gather_ceiling(dsa, dev["k_cache"].view(batch * s_max, hkv, d), dev["v_cache"].view(batch * s_max, hkv, d),
                             idx2, nsplits=(1, 2, 4, 8, 16, 32), row_stride=s_max, group_fastest=True)
    log(f"{name}: decode kernels (us) {per}; separate entry points equal the fused step: {same}; attention gather "
        f"ceiling {ceiling['ms'] * 1e3:.1f} us")
    res = dict(name=name, us_median=us_median, us_min=us_min, bytes_step=bytes_step,
               gbs=bytes_step / (us_median * 1e-6) / 1e9, batch=batch, s_max=s_max, kernel_us=per,
               separate_entry_points_equal_fused=same, idx_bytes=idx_bytes, attn_bytes=attn_bytes,
               score_bytes=score_bytes, attn_ceiling=ceiling, samples=samples, di=di)

    if full:
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
        g_med, g_min = timed_median(graph.replay, n_iter)
        graph_same = bool(torch.equal(out, eager[0]) and torch.equal(lse, eager[1]) and torch.equal(idx, eager[2]))
        res["graph_us"] = {"median": g_med, "min": g_min, "same_outputs_as_eager": graph_same}
        log(f"{name}: decode in a HIP graph: median {g_med:.1f} us (min {g_min:.1f}); outputs equal: {graph_same}")
        del graph

        # The torch.topk-shaped top-k on the decode step's scores, beside the ascending form.
        idx_s = torch.empty(batch, k, dtype=torch.int32, device="cuda")
        val_s = torch.empty(batch, k, dtype=torch.float32, device="cuda")
        timing = {}
        for nm, fn in (("ascending", dsa.dsa_topk), ("sorted", dsa.dsa_topk_sorted)):
            timing[nm] = timed_median(lambda: fn(scores, dev["seq_lens"], k, idx_s, val_s, workspace=tk_ws),
                                      n_iter)[0]
            if nm == "ascending":
                asc_i = idx_s.cpu().numpy().copy()
        got_i = idx_s.cpu().numpy()
        got_v = val_s.cpu().numpy()
        ok = True
        for j in range(batch):
            order_ok = bool(np.all((got_v[j, :-1] > got_v[j, 1:]) |
                                   ((got_v[j, :-1] == got_v[j, 1:]) & (got_i[j, :-1] < got_i[j, 1:]))))
            ok = ok and order_ok and bool(np.array_equal(np.sort(got_i[j]), asc_i[j]))
        res["topk_sorted"] = {"rows": batch, "row_len": int(lens.max()), "k": k, "us_sorted": timing["sorted"],
                              "us_ascending": timing["ascending"], "same_set_as_ascending_form_and_ordered": ok}
        log(f"{name}: torch.topk-shaped top-k {timing['sorted']:.1f} us (ascending {timing['ascending']:.1f} us); "
            f"ordered: {ok}")
    del dev, ws, tk_ws, scores, at_ws
    torch.cuda.empty_cache()
    return res


def decode_rooflines(dec):
    us = dec["kernel_us"]
    return {
        "roofline_decode_step": {"bound": "hbm", "achieved": dec["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                 "frac": dec["gbs"] / PEAK_HBM_GBS, "algorithmic_bytes_per_step": dec["bytes_step"]},
        "roofline_decode_indexer": hbm_roofline("indexer_decode_coop_kernel",
                                                f"indexer_decode_coop_kernel<64, 128, 2>@{dec['name']}", us["indexer"] * 1e-3,
                                                dec["idx_bytes"] + dec["score_bytes"]),
        "roofline_decode_attn": hbm_roofline("decode sparse attention (split partials + combine)",
                                             f"sparse_attn_kernel@{dec['name']}", us["attention"] * 1e-3,
                                             dec["attn_bytes"], ceiling=dec["attn_ceiling"],
                                             note="each cache row is read by one query, so physical bytes equal "
                                                  "algorithmic bytes: effective_algorithmic_gbs is the HBM rate"),
    }


def decode_summary(dec):
    r = {"workload": dec["name"], "batch": dec["batch"], "s_max": dec["s_max"], "us_per_step": dec["us_median"],
         "us_min": dec["us_min"], "kernel_us_separate_entry_points": dec["kernel_us"]}
    r.update(decode_rooflines(dec))
    return r


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


def attn_bwd_bench(args, dsa, inp):
    """Backward of the sparse attention on the 32K prefill (training side), after one fused
    prefill that provides O, lse and the index sets; dO is synthetic.  Both forms: per row (one
    float atomic per selected (row, KV head, dim) for dk / dv) and with dk / dv summed over the
    merged sets of blocks of adjacent rows first (one atomic per merged position)."""
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
    total, hq = out.shape[0], out.shape[1]
    hkv, d = pi.k.shape[1], pi.k.shape[2]
    ws = torch.empty(max(dsa.dsa_sparse_gqa_attn_bwd_dedup_workspace_size(total, k, hq, hkv), 16),
                     dtype=torch.uint8, device="cuda")

    def per_row():
        dsa.dsa_sparse_gqa_attn_bwd(dev["q"], dev["k"], dev["v"], out, lse, dout, idx, dev["cu"], dq, dk, dv)

    def dedup():
        dsa.dsa_sparse_gqa_attn_bwd_dedup(dev["q"], dev["k"], dev["v"], out, lse, dout, idx, dev["cu"], dq, dk, dv,
                                          workspace=ws)

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    ms_row = timed(per_row)
    ref = (dq.clone(), dk.clone(), dv.clone())
    ms = timed(dedup)
    # the two forms agree up to the order of the float additions
    agree = {n: float((x - y).abs().max() / y.abs().max().clamp_min(1e-30))
             for n, x, y in zip(("dq", "dk", "dv"), (dq, dk, dv), ref)}
    # merged-set sizes: the workspace begins with the per-block counts (int32)
    rows_per_block = 16 if hq // hkv == 16 else 32
    n_blocks = (total + rows_per_block - 1) // rows_per_block
    merged = int(ws[:4 * n_blocks].view(torch.int32).to(torch.int64).sum().item())
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    dsa.dsa_sparse_gqa_attn(dev["q"], dev["k"], dev["v"], idx, dev["cu"], out, lse)
    b.record()
    torch.cuda.synchronize()
    fwd_ms = a.elapsed_time(b)
    lens = [int(x) for x in pi.seq_lens]
    sel_pairs = sum(sum(min(t + 1, k) for t in range(n)) for n in lens)
    atomics_row = sel_pairs * hkv * 2 * d
    atomics_dedup = merged * hkv * 2 * d
    # per selected (row, KV group): K and V rows gathered (2 x 256 B) and 2 x 128 fp32 atomics
    algo_bytes = sel_pairs * hkv * (2 * d * 2 + 2 * d * 4)
    log(f"attention backward {ms:.1f} ms with merged sets of {rows_per_block} rows (per row {ms_row:.1f} ms, "
        f"forward {fwd_ms:.1f} ms) on {args.bwd_workload}; merged positions {merged / sel_pairs:.3f} of the "
        f"selected pairs; agreement {agree}")
    del dev, dq, dk, dv, dout, out, lse, idx, ws, ref
    torch.cuda.empty_cache()
    return {"workload": args.bwd_workload, "ms": ms, "per_row_ms": ms_row, "forward_ms": fwd_ms,
            "tokens_per_s": total / (ms * 1e-3), "merged_block_rows": rows_per_block,
            "merged_positions_per_selected_pair": merged / sel_pairs,
            "float_atomic_adds": {"per_row": atomics_row, "merged_sets": atomics_dedup},
            "atomic_adds_per_s": {"per_row": atomics_row / (ms_row * 1e-3),
                                  "merged_sets": atomics_dedup / (ms * 1e-3)},
            "dedup_vs_per_row_max_rel_diff": agree,
            "algorithmic_gb_per_s_per_row_form": algo_bytes / (ms_row * 1e-3) / 1e9,
            "note": "dq, dk, dv from dO; dk/dv with fp32 atomics, whose device rate (measured_peaks: the "
                    "same for 64 or 16 consecutive floats per row and instruction) bounds both forms; the "
                    "merged-set form issues one atomic per merged position and dim instead of one per "
                    "selected pair"}


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


def measured_peaks(dsa):
    """What the box reaches on the priced resources (the probe library): an MFMA-only loop of
    16x16x32 and of 32x32x16 bf16 instructions, a streaming read of 4 GiB, and float-atomic adds in
    the attention backward's two scatter shapes.  Best of several timed launches each."""
    import torch

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
    del buf
    # float atomics over 134 MB (the 32K backward's dk + dv), 64 or 16 consecutive floats per row piece
    abuf = torch.zeros(262144, 128, dtype=torch.float32, device="cuda")
    for w in (64, 16):
        adds = dsa.dsa_probe_atomic_add(abuf, w, 8192, 256)
        res[f"float_atomic_adds_per_s_{w}_per_row"] = adds / (best_ms(lambda: dsa.dsa_probe_atomic_add(abuf, w, 8192,
                                                                                                     256), 3) * 1e-3)
    del abuf, sink
    torch.cuda.empty_cache()
    log(f"measured peaks: {res}")
    return res


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(args, pre, dec):
    """The oracle as it stands, on a bounded sample of rows of the same 128K workload (the only leg of
    the benchmark that runs it): its whole-job rate extrapolated by causal work, and its agreement
    with the timed run's outputs on those rows (index mismatches, max / mean absolute O error, lse
    error), plus every row of the timed decode step."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import dsa_testlib as tl
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    pi = pre["pi"]
    smp = pre["samples"]
    total = sum(int(x) for x in pi.seq_lens)
    rows = smp["rows"]
    done = 0
    idx_rows_bad = idx_slots_bad = 0
    err_max = err_sum = lse_max = 0.0
    n_err = 0
    t0 = time.perf_counter()
    while done < len(rows) and time.perf_counter() - t0 < args.cpu_seconds:
        want = tl.oracle_prefill_rows_lazy(pi, rows[done:done + 4])
        got_i = smp["idx"][done:done + 4]
        bad = got_i != want["idx"]
        idx_rows_bad += int(bad.any(axis=1).sum())
        idx_slots_bad += int(bad.sum())
        e = np.abs(smp["out"][done:done + 4].astype(np.float64) - want["out"])
        err_max = max(err_max, float(e.max()))
        err_sum += float(e.sum())
        n_err += e.size
        lse_max = max(lse_max, float(np.abs(smp["lse"][done:done + 4] - want["lse"]).max()))
        done += 4
    el = time.perf_counter() - t0
    work_sample = sum(r + 1 for r in rows[:done])           # indexer work grows with the prefix length
    work_all = total * (total + 1) / 2
    rows_per_s = done / el
    tokens_per_s = total / (el * work_all / work_sample)     # whole-job rate, extrapolated by work
    res = {"value": tokens_per_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{done} uniformly drawn rows of the 128K prefill in {el:.1f}s ({rows_per_s:.2f} rows/s); "
                     f"whole-job rate extrapolated by causal work (sum of t+1)",
           "host_cpu_count": os.cpu_count(), "cpu_model": _cpu_model(),
           "parity_vs_timed_prefill": {"rows": done, "index_mismatch_rows": idx_rows_bad,
                                       "index_mismatch_slots": idx_slots_bad, "out_max_abs": err_max,
                                       "out_mean_abs": err_sum / max(1, n_err), "lse_max_abs": lse_max,
                                       "tolerance": {"out_max_abs": tl.MAX_ABS, "out_mean_abs": tl.MEAN_ABS,
                                                     "lse_max_abs": tl.LSE_ABS}}}
    if dec is not None:
        t1 = time.perf_counter()
        di = dec["di"]
        batch = di.q.shape[0]
        want = tl.oracle_decode_rows_lazy(di, range(batch))
        got = dec["samples"]
        bad = got["idx"] != np.asarray(want["idx"])
        e = np.abs(got["out"].astype(np.float64) - np.asarray(want["out"]))
        res["parity_vs_timed_decode"] = {
            "workload": dec["name"], "rows": batch, "index_mismatch_rows": int(bad.any(axis=1).sum()),
            "index_mismatch_slots": int(bad.sum()), "out_max_abs": float(e.max()), "out_mean_abs": float(e.mean()),
            "lse_max_abs": float(np.abs(got["lse"] - np.asarray(want["lse"])).max()),
            "oracle_s": time.perf_counter() - t1}
    log(f"cpu baseline: {res}")
    return res


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
    if args.training_only:
        print(json.dumps({"sparse_attn_backward": attn_bwd_bench(args, dsa, inp),
                          "indexer_warmup_objective": warmup_bench(args, dsa, inp)}))
        return
    pre = prefill_section(args, dsa, inp, args.workload, args.steps, args.warmup, full=True)
    peaks = measured_peaks(dsa)
    corr = None if args.no_correlated else correlated_bench(args, dsa, inp)
    dec = None if args.no_decode else decode_section(args, dsa, inp, args.decode_workload, full=True)
    extra = {}
    if not args.no_extra:
        for name in EXTRA_PREFILL:
            extra[name] = prefill_summary(prefill_section(args, dsa, inp, name, min(args.steps, 5), 1, full=False))
        if not args.no_decode:
            for name in EXTRA_DECODE:
                extra[name] = decode_summary(decode_section(args, dsa, inp, name, full=False))
    bwd = None if args.no_bwd else attn_bwd_bench(args, dsa, inp)
    if bwd is not None:
        ceiling = peaks.get("float_atomic_adds_per_s_16_per_row")
        bwd["atomic_adds_per_s"]["probe_ceiling"] = ceiling
        if ceiling:
            bwd["atomic_frac_of_probe"] = {k: v / ceiling for k, v in bwd["atomic_adds_per_s"].items()
                                           if k != "probe_ceiling"}
    wup = None if args.no_bwd else warmup_bench(args, dsa, inp)
    dense = None if args.no_dense else dense_bench(args, dsa, inp, pre["ms_per_step"],
                                                   None if dec is None else dec["us_median"])
    cpu = None if args.no_cpu_baseline else cpu_baseline(args, pre, dec)

    total = pre["rows_total"]
    value = total / (pre["ms_per_step"] * 1e-3)
    kern = pre["kern"]
    attn_ms = kern["sparse_attn_union"] / pre["launches"]["sparse_attn_union"]
    roof = indexer_roofline(pre, f"indexer_prefill_kernel<64, 128, 4, 2>@{pre['name']}")
    roof["measured_peak"] = peaks["mfma_bf16_16x16x32_tflops"]
    roof["frac_of_measured_peak"] = pre["idx_tflops"] / peaks["mfma_bf16_16x16x32_tflops"]
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
        "ms_per_step_with_launch_timing": pre["timing_on_ms"],
        "kernel_ms_per_step": kern,
        "kernel_launches_per_step": pre["launches"],
        "roofline": roof,
        "roofline_sparse_attn": hbm_roofline(
            "sparse_attn_union_kernel (8-row merged sets)", f"sparse_attn_union_kernel<8, 2, 2>@{pre['name']}", attn_ms,
            pre["merged_bytes"], ceiling=pre.get("ceiling_merged"),
            mfma_tflops=pre["attn_tflops"], mfma_frac=pre["attn_tflops"] / PEAK_BF16_TFLOPS,
            bytes_without_dedup=pre["attn_bytes"],
            note="merged K/V rows are re-read by neighbouring blocks through L2 and the Infinity Cache, so the "
                 "effective algorithmic rate can exceed the HBM peak; the counter rate is the L2-miss traffic"),
        "roofline_sparse_attn_per_row": hbm_roofline(
            "sparse_attn_kernel (per row, the path without dedup)", f"sparse_attn_kernel@{pre['name']}",
            pre["per_row_attn_ms"], pre["attn_bytes"], ceiling=pre.get("ceiling_per_row")),
        "roofline_query_union": {"bound": "hbm", "achieved": pre["union_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                 "frac": pre["union_gbs"] / PEAK_HBM_GBS,
                                 "algorithmic_bytes_per_launch": pre["union_bytes"]},
        "roofline_topk": {"bound": "hbm", "achieved": pre["topk_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": pre["topk_gbs"] / PEAK_HBM_GBS, "kernels": pre["topk_parts"],
                          "ms_per_step": pre["topk_ms"], "algorithmic_bytes_per_step": pre["topk_bytes"],
                          "candidates_per_row_mean": pre["candidates_per_row_mean"],
                          "note": "fused top-k: no score is written or re-read; the bytes are the sample, the "
                                  "candidate lists (written by the emitting indexer, read by the select) and the "
                                  "index rows, so the kernels are latency-bound rather than HBM-bound"},
        "indexer_plus_topk_ms_per_step": kern[pre["indexer_key"]] + pre["topk_ms"],
        "measured_peaks": peaks,
        "dedup": {"block_rows": pre["block_rows"], "merged_rows_per_block_mean": pre["merged_rows_per_block_mean"],
                  "index_slots_per_block": pre["block_rows"] * 2048, "merged_fraction": pre["merged_fraction"],
                  "prefill_ms_without_dedup": pre["no_dedup_ms"],
                  "max_abs_out_vs_per_row": pre["max_abs_out_vs_per_row"],
                  "union16_at_t": pre["union16_at_t"], "union16_mean": pre["union16_mean"]},
        "prefill_correlated_queries": corr,
        "cpu_baseline": cpu,
    }
    if dec is not None:
        line["decode_us_per_step"] = dec["us_median"]
        line["decode_us_min"] = dec["us_min"]
        line["decode_us_per_step_hip_graph"] = dec["graph_us"]
        line["decode_config"] = {"workload": "decode_b32_128k: batch 32, 131072-token caches, k=2048"}
        line["decode_kernel_us_separate_entry_points"] = dec["kernel_us"]
        dr = decode_rooflines(dec)
        line["roofline_decode"] = dict(dr["roofline_decode_step"],
                                       frac_of_measured_peak=dec["gbs"] / peaks["stream_read_gbs"])
        line["roofline_decode_indexer"] = dr["roofline_decode_indexer"]
        line["roofline_decode_attn"] = dr["roofline_decode_attn"]
        line["topk_sorted_decode_scores"] = dec["topk_sorted"]
    for name, summary in extra.items():
        line[name] = summary
    if bwd is not None:
        line["sparse_attn_backward"] = bwd
    if wup is not None:
        line["indexer_warmup_objective"] = wup
    if dense is not None:
        line["dense_attention_context"] = dense
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
