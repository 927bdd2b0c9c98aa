"""Shared helpers of the GPU parity tests: upload synthetic inputs, run the oracle on the same
bf16 values, and compare (indices bit for bit, outputs within the stated tolerance)."""

from __future__ import annotations

import numpy as np

from oracle import dsa_oracle as orc
from sparse_long_context_lightning_amd import inputs as inp

# Attention outputs: bf16 in, fp32 accumulate, bf16 out.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
LSE_ABS = 2e-3


def f64(bits):
    return inp.bf16_bits_to_f32(bits).astype(np.float64)


def upload_prefill(pi, device="cuda"):
    from sparse_long_context_lightning_amd import upload_prefill_inputs
    return upload_prefill_inputs(pi, device)


def upload_decode(di, device="cuda"):
    from sparse_long_context_lightning_amd import upload_decode_inputs
    return upload_decode_inputs(di, device)


def bf16_tensor_to_f64(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def oracle_prefill_rows(pi, rows):
    return orc.prefill(f64(pi.q), f64(pi.k), f64(pi.v), f64(pi.q_idx), f64(pi.k_idx), pi.w.astype(np.float64),
                       pi.cu_seqlens, pi.top_k, rows=rows)


def oracle_prefill_rows_lazy(pi, rows, keep_scores=False):
    """Oracle on sampled rows of a large workload without widening whole tensors up front.  With
    keep_scores, also each row's indexer scores (exact in fp32 for the integer indexer inputs, so
    kept as float32 to halve the memory; the cast is checked to be exact)."""
    cu = [int(x) for x in pi.cu_seqlens]
    hq, d = pi.q.shape[1], pi.q.shape[2]
    scale = orc.default_softmax_scale(d)
    out = {"idx": [], "out": [], "lse": [], "wsum": []}
    scores = []
    for r in rows:
        b = max(i for i in range(len(cu) - 1) if cu[i] <= r)
        o, t = cu[b], r - cu[b]
        sc = orc.index_scores_row(f64(pi.q_idx[r]), pi.w[r].astype(np.float64), f64(pi.k_idx[o:o + t + 1]))
        if keep_scores:
            sc32 = sc.astype(np.float32)
            assert np.array_equal(sc32.astype(np.float64), sc), "scores not exact in fp32"
            scores.append(sc32)
        sel = orc.select_topk_row(sc, pi.top_k)
        valid = sel[sel >= 0]
        # only the selected key/value rows are widened
        kk = np.zeros((t + 1,) + pi.k.shape[1:], dtype=np.float64)
        vv = np.zeros_like(kk)
        kk[valid] = f64(pi.k[o + valid])
        vv[valid] = f64(pi.v[o + valid])
        oo, ll, ws = orc.sparse_gqa_attention_row(f64(pi.q[r]), kk, vv, sel, scale)
        out["idx"].append(sel)
        out["out"].append(oo)
        out["lse"].append(ll)
        out["wsum"].append(ws)
    res = {k: np.asarray(v) for k, v in out.items()}
    if keep_scores:
        res["scores"] = scores
    return res


def oracle_decode_rows_lazy(di, batch_rows):
    hq, d = di.q.shape[1], di.q.shape[2]
    scale = orc.default_softmax_scale(d)
    out = {"idx": [], "out": [], "lse": [], "scores": []}
    for b in batch_rows:
        n = int(di.seq_lens[b])
        sc = orc.index_scores_row(f64(di.q_idx[b]), di.w[b].astype(np.float64), f64(di.k_idx_cache[b, :n]))
        sel = orc.select_topk_row(sc, di.top_k)
        valid = sel[sel >= 0]
        kk = np.zeros((n,) + di.k_cache.shape[2:], dtype=np.float64)
        vv = np.zeros_like(kk)
        kk[valid] = f64(di.k_cache[b, valid])
        vv[valid] = f64(di.v_cache[b, valid])
        oo, ll, _ = orc.sparse_gqa_attention_row(f64(di.q[b]), kk, vv, sel, scale)
        out["idx"].append(sel)
        out["out"].append(oo)
        out["lse"].append(ll)
        out["scores"].append(sc)
    return out


def assert_attn_close(got, want, what=""):
    err = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(want, dtype=np.float64))
    assert err.max() <= MAX_ABS, f"{what}: max-abs error {err.max():.3e} > {MAX_ABS}"
    assert err.mean() <= MEAN_ABS, f"{what}: mean-abs error {err.mean():.3e} > {MEAN_ABS}"


def assert_idx_equal(got, want, rows=None, what=""):
    got = np.asarray(got)
    want = np.asarray(want)
    if not np.array_equal(got, want):
        bad = np.nonzero((got != want).any(axis=-1))[0]
        r0 = bad[0]
        label = rows[r0] if rows is not None else r0
        diff = np.nonzero(got[r0] != want[r0])[0][:5]
        raise AssertionError(f"{what}: {len(bad)} rows differ; first row {label}, slots {diff.tolist()}: "
                             f"got {got[r0][diff].tolist()} want {want[r0][diff].tolist()}")


def check_index_structure(idx, row_lens, k):
    """Every row: ascending, unique, in range, count = min(len, k), -1 padding after."""
    idx = np.asarray(idx)
    row_lens = np.asarray(row_lens)
    cnt = np.minimum(row_lens, k)
    pos = np.arange(k)[None, :]
    valid = pos < cnt[:, None]
    assert np.all(idx[~valid] == -1), "padding must be -1"
    v = np.where(valid, idx, 0)
    assert np.all(v >= 0) and np.all(v < row_lens[:, None]), "index out of range"
    d = np.diff(idx, axis=1)
    both = valid[:, 1:]
    assert np.all(d[both] > 0), "indices must be strictly ascending"


def check_index_structure_device(idx, row_lens, k):
    """check_index_structure on the device, for index sets too large to copy to the host."""
    import torch
    row_lens = row_lens.to(idx.device).to(torch.int64)
    cnt = torch.clamp(row_lens, max=k)
    pos = torch.arange(k, device=idx.device)[None, :]
    valid = pos < cnt[:, None]
    assert bool((idx[~valid] == -1).all()), "padding must be -1"
    v = idx.to(torch.int64)
    assert bool(((v >= 0) & (v < row_lens[:, None]) | ~valid).all()), "index out of range"
    d = v[:, 1:] - v[:, :-1]
    assert bool(((d > 0) | ~valid[:, 1:]).all()), "indices must be strictly ascending"


def sample_rows(cu_seqlens, k, n_random, seed, period=None):
    """Deterministic row sample of a packed prefill: row 0, the first and last row of each
    sequence, rows k-2 .. k+1 of each sequence, the text/frame boundaries of the first and last
    periods when `period` is given (32 text tokens then a frame), and n_random rows drawn from
    PCG64(seed + 100)."""
    cu = [int(x) for x in cu_seqlens]
    rows = {0}
    for b in range(len(cu) - 1):
        o, n = cu[b], cu[b + 1] - cu[b]
        if n == 0:
            continue
        rows |= {o, o + n - 1}
        rows |= {o + t for t in (k - 2, k - 1, k, k + 1) if 0 <= t < n}
        if period:
            last = (n - 1) // period
            for j in (0, 1, last // 2, last):
                rows |= {o + j * period + t for t in (31, 32, period - 1) if j * period + t < n}
    rng = np.random.default_rng(seed + 100)
    rows |= set(int(x) for x in rng.integers(0, cu[-1], n_random))
    return sorted(rows)
