"""Backward of the indexer scores (dsa_index_scores_bwd) through the C ABI against the oracle's
index_scores_row_grad.  GPU only.

Tolerance, from the arithmetic: the ReLU mask [c > 0] is exact on both sides (the integer
indexer inputs make c exact in fp32), and the one rounding is g [c > 0] (for dk_idx
g w [c > 0], w a power of two) to bf16 (relative 2^-9 per term) ahead of fp32 accumulation.  So each
output differs from the float64 oracle by at most 2^-9 times the sum of the absolute values of
its terms, plus fp32 accumulation error; the tests allow 2^-8 times that sum, computed here
from the same inputs with every factor replaced by its absolute value."""

import numpy as np
import pytest

from oracle import dsa_oracle as orc
from sparse_long_context_lightning_amd import inputs as inp

import dsa_testlib as tl

pytestmark = pytest.mark.gpu

H, DI = 64, 128


def _grad_input(lens, ld, seed):
    """Seeded gradient of the scores: N(0, 1) / length on each row's prefix, NaN past it (never
    read by the kernels)."""
    rng = np.random.default_rng(seed)
    total = sum(lens)
    g = np.full((total, ld), np.nan, dtype=np.float32)
    r = 0
    for n in lens:
        for t in range(n):
            g[r, :t + 1] = (rng.standard_normal(t + 1) / (t + 1)).astype(np.float32)
            r += 1
    return g


def _oracle(pi, g, row_range=None):
    """Oracle gradients of the packed rows in row_range (all rows if None) and the per-element
    bounds on their rounding error (sums of |terms|)."""
    q, k, w = tl.f64(pi.q_idx), tl.f64(pi.k_idx), pi.w.astype(np.float64)
    total = q.shape[0]
    dq = np.zeros_like(q)
    dw = np.zeros_like(w)
    dk = np.zeros_like(k)
    bq = np.zeros_like(q)
    bw = np.zeros_like(w)
    bk = np.zeros_like(k)
    cu = pi.cu_seqlens
    for b in range(len(cu) - 1):
        o = int(cu[b])
        for t in range(int(cu[b + 1]) - o):
            r = o + t
            if row_range is not None and r not in row_range:
                continue
            kp = k[o:o + t + 1]
            gr = g[r, :t + 1].astype(np.float64)
            gq, gw, gk = orc.index_scores_row_grad(q[r], w[r], kp, gr)
            dq[r], dw[r] = gq, gw
            dk[o:o + t + 1] += gk
            m = (q[r] @ kp.T) > 0
            ag = np.abs(gr)[None, :] * m                      # |g| [c > 0], [H, n]
            ua = ag @ np.abs(kp)                              # [H, DI]
            bq[r] = np.abs(w[r])[:, None] * ua
            bw[r] = np.sum(np.abs(q[r]) * ua, axis=1)
            bk[o:o + t + 1] += ag.T @ (np.abs(w[r])[:, None] * np.abs(q[r]))
    return (dq, dw, dk), (bq, bw, bk)


def _run(dsa, pi, g, chunks):
    import torch
    dev = tl.upload_prefill(pi)
    total = pi.q_idx.shape[0]
    g_t = torch.from_numpy(g).cuda()
    dq = torch.full((total, H, DI), float("nan"), dtype=torch.float32, device="cuda")
    dw = torch.full((total, H), float("nan"), dtype=torch.float32, device="cuda")
    dk = torch.zeros((total, DI), dtype=torch.float32, device="cuda")
    for r0, n in chunks:
        dsa.dsa_index_scores_bwd(dev["q_idx"], dev["k_idx"], dev["w"], pi.cu_seqlens, r0, n, g_t[r0:r0 + n], dq, dw,
                                 dk)
    torch.cuda.synchronize()
    return dq.cpu().numpy().astype(np.float64), dw.cpu().numpy().astype(np.float64), \
        dk.cpu().numpy().astype(np.float64)


def _check(name, got, want, bound, rows=None):
    if rows is not None:
        got, want, bound = got[rows], want[rows], bound[rows]
    err = np.abs(got - want)
    tol = 2.0 ** -8 * bound + 1e-6
    bad = err > tol
    assert not np.any(np.isnan(got)), f"{name}: NaN in the checked rows"
    assert not np.any(bad), f"{name}: {int(bad.sum())} elements off, worst {float((err - tol).max()):.3e} over " \
                            f"tolerance at {np.unravel_index(np.argmax(err - tol), err.shape)}"
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
    assert rel < 1e-2, f"{name}: relative error {rel:.2e}"
    print(f"{name}: max abs err {err.max():.3e}, relative {rel:.2e}")


@pytest.mark.parametrize("lens,chunks", [
    ([300], [(0, 300)]),                                   # one call; the keys are split (atomics)
    ([130, 333], [(0, 150), (150, 150), (300, 163)]),      # chunks across a sequence boundary
    ([1, 5, 64, 65], [(0, 135)]),                          # tiny and tile-edge sequences
    ([1100], [(0, 1100)]),                                 # enough row blocks for unsplit keys
])
def test_indexer_bwd_matches_oracle(dsa, lens, chunks):
    pi = inp.prefill_inputs(lens, H, DI, 8, 2, 128, 64, seed=sum(lens) + 11)
    ld = (max(lens) + 3) // 4 * 4
    g = _grad_input(lens, ld, seed=len(lens) + 5)
    print(f"lens {lens} chunks {chunks}", flush=True)
    got = _run(dsa, pi, g, chunks)
    want, bound = _oracle(pi, g)
    for name, a, b, c in zip(("dq", "dw", "dk"), got, want, bound):
        _check(name, a, b, c)


def test_indexer_bwd_leaves_other_rows_untouched(dsa):
    lens = [200, 90]
    pi = inp.prefill_inputs(lens, H, DI, 8, 2, 128, 64, seed=7)
    g = _grad_input(lens, 200, seed=8)
    dq, dw, dk = _run(dsa, pi, g, [(120, 100)])
    rows = np.r_[0:120, 220:290]
    assert np.all(np.isnan(dq[rows])) and np.all(np.isnan(dw[rows]))
    # rows 120..219 reach keys 0..199 of sequence 0 and keys 0..19 of sequence 1 only
    assert np.all(dk[220:290] == 0.0)
    (wq, ww, wk), (bq, bw, bk) = _oracle(pi, g, row_range=range(120, 220))
    _check("dq", dq, wq, bq, rows=np.r_[120:220])
    _check("dw", dw, ww, bw, rows=np.r_[120:220])
    _check("dk", dk, wk, bk)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_indexer_bwd_full_32k_chunked(dsa):
    """The 32K prefill in the benchmark's launch configuration (16 calls of 2048 rows, dk_I
    accumulated over them): dq_I and dw on sampled rows recomputed by the oracle one by one, and
    dk_I of the last 16 keys, which only the last 16 rows reach, recomputed from those rows."""
    import torch
    pi = inp.workload("c2_prefill_32k")
    total = int(pi.cu_seqlens[-1])
    dev = tl.upload_prefill(pi)
    rng = np.random.default_rng(31)
    chunk = 2048
    # Seeded gradient rows N(0, 1)/(t+1) on each prefix, generated per chunk on the host.
    dq = torch.full((total, H, DI), float("nan"), dtype=torch.float32, device="cuda")
    dw = torch.full((total, H), float("nan"), dtype=torch.float32, device="cuda")
    dk = torch.zeros((total, DI), dtype=torch.float32, device="cuda")
    g_rows = {}
    check = [0, 1, 2047, 2048, 9000, 20001, total - 17, total - 1] + list(range(total - 16, total))
    buf = np.zeros((chunk, total), dtype=np.float32)
    for c0 in range(0, total, chunk):
        n = min(chunk, total - c0)
        buf[:] = 0.0
        for i in range(n):
            t = c0 + i
            buf[i, :t + 1] = (rng.standard_normal(t + 1) / (t + 1)).astype(np.float32)
            if t in check:
                g_rows[t] = buf[i, :t + 1].astype(np.float64).copy()
        g_t = torch.from_numpy(buf[:n]).cuda()
        dsa.dsa_index_scores_bwd(dev["q_idx"], dev["k_idx"], dev["w"], pi.cu_seqlens, c0, n, g_t, dq, dw, dk)
    torch.cuda.synchronize()
    q, k, w = tl.f64(pi.q_idx), tl.f64(pi.k_idx), pi.w.astype(np.float64)
    got_q, got_w, got_k = dq.cpu().numpy(), dw.cpu().numpy(), dk.cpu().numpy()
    want_k = np.zeros((16, DI))
    bound_k = np.zeros((16, DI))
    for t in sorted(set(check)):
        kp = k[:t + 1]
        gq, gw, gk = orc.index_scores_row_grad(q[t], w[t], kp, g_rows[t])
        m = (q[t] @ kp.T) > 0
        ag = np.abs(g_rows[t])[None, :] * m
        ua = ag @ np.abs(kp)
        _check(f"dq row {t}", got_q[t][None], gq[None], (np.abs(w[t])[:, None] * ua)[None])
        _check(f"dw row {t}", got_w[t][None], gw[None], np.sum(np.abs(q[t]) * ua, axis=1)[None])
        if t >= total - 16:
            s0 = total - 16          # row t reaches keys s0 .. t
            want_k[:t + 1 - s0] += gk[s0:]
            bound_k[:t + 1 - s0] += (ag.T @ (np.abs(w[t])[:, None] * np.abs(q[t])))[s0:]
    _check("dk last 16 keys", got_k[total - 16:], want_k, bound_k)
