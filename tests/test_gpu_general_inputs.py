"""Indexer inputs outside the exact-score workloads (any finite bf16 q_idx / k_idx, any finite fp32
w, negative weights included; reading R19), through the C ABI against the oracle.  GPU only.

Scores: the kernel's fp32 sums differ from the float64 oracle by rounding only.  A score is a
d_I-term dot product per head, a product with w and an H_I-term sum, so the classic bound for
recursive fp32 summation allows (d_I + H_I + 2) * 2^-24 times the sum of the absolute values
of its terms, sum_j |w_j| sum_d |q_jd k_d|.  Top-k: where scores are not exact the
index set is not unique up to rounding, so it is checked by value: every selected position's
oracle score is at least the oracle's k-th largest score minus that row's tolerance, and the
set has the right size, ascending order and range."""

import numpy as np
import pytest

from oracle import dsa_oracle as orc
from sparse_long_context_lightning_amd import inputs as inp

import dsa_testlib as tl

pytestmark = pytest.mark.gpu


def _general_inputs(lens, h_idx, d_idx, seed):
    rng = np.random.default_rng(seed)
    total = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = inp.f32_to_bf16_bits(rng.standard_normal((total, h_idx, d_idx)).astype(np.float32))
    k = inp.f32_to_bf16_bits(rng.standard_normal((total, d_idx)).astype(np.float32))
    w = (rng.standard_normal((total, h_idx)) * 0.3).astype(np.float32)  # signed weights
    return cu, q, k, w


@pytest.mark.parametrize("lens,h_idx,d_idx", [([700], 64, 128), ([130, 517], 64, 128), ([300], 4, 64)])
def test_scores_general_inputs_within_rounding(dsa, lens, h_idx, d_idx):
    import torch
    from sparse_long_context_lightning_amd import to_device_bf16
    cu, q, k, w = _general_inputs(lens, h_idx, d_idx, seed=sum(lens) + h_idx)
    total = int(cu[-1])
    ld = (max(lens) + 3) // 4 * 4
    scores = torch.full((total, ld), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa_index_scores(to_device_bf16(q), to_device_bf16(k), torch.from_numpy(w).cuda(), cu, 0, total, scores)
    got = scores.cpu().numpy().astype(np.float64)
    qf, kf, wf = tl.f64(q), tl.f64(k), w.astype(np.float64)
    want = orc.index_scores(qf, kf, wf, cu)
    for b in range(len(lens)):
        o = int(cu[b])
        for t in range(lens[b]):
            r = o + t
            bound = (d_idx + h_idx + 2) * 2.0 ** -24 * (np.abs(wf[r]) @ (np.abs(qf[r]) @ np.abs(kf[o:o + t + 1]).T))
            err = np.abs(got[r, :t + 1] - want[r])
            assert np.all(err <= bound), f"row {r}: worst {np.max(err - bound):.3e}"
            assert np.all(np.isnan(got[r, t + 1:]))


def test_topk_general_inputs_by_value(dsa):
    import torch
    from sparse_long_context_lightning_amd import to_device_bf16
    lens = [3000]
    top_k = 256
    cu, q, k, w = _general_inputs(lens, 64, 128, seed=77)
    total = int(cu[-1])
    ld = total
    scores = torch.empty((total, ld), dtype=torch.float32, device="cuda")
    dsa.dsa_index_scores(to_device_bf16(q), to_device_bf16(k), torch.from_numpy(w).cuda(), cu, 0, total, scores)
    row_len = torch.arange(1, total + 1, dtype=torch.int32, device="cuda")
    idx = torch.empty((total, top_k), dtype=torch.int32, device="cuda")
    ws = torch.empty(dsa.dsa_topk_workspace_size(total, ld, top_k), dtype=torch.uint8, device="cuda")
    dsa.dsa_topk(scores, row_len, top_k, idx, workspace=ws)
    got = idx.cpu().numpy()
    tl.check_index_structure(got, np.arange(1, total + 1), top_k)
    qf, kf, wf = tl.f64(q), tl.f64(k), w.astype(np.float64)
    for t in list(range(0, total, 97)) + [top_k - 1, top_k, total - 1]:
        want = orc.index_scores_row(qf[t], wf[t], kf[:t + 1])
        n = min(t + 1, top_k)
        sel = got[t, :n]
        if t + 1 <= top_k:
            assert np.array_equal(sel, np.arange(t + 1))
            continue
        kth = np.sort(want)[::-1][top_k - 1]
        tol = 2 * (128 + 64 + 2) * 2.0 ** -24 * np.max(np.abs(wf[t]) @ (np.abs(qf[t]) @ np.abs(kf[:t + 1]).T))
        assert np.all(want[sel] >= kth - tol), f"row {t}: a selected score is below the k-th largest"


def test_fused_prefill_general_inputs_equals_composition(dsa):
    """The prefill's fused top-k (sampled threshold, candidates compared as floats in the indexer
    pass) on general inputs with signed weights, where scores and, for rows a little longer than k,
    the thresholds themselves are negative: its index sets equal dsa_topk over dsa_index_scores of
    the same rows (the same fp32 scores, one tie rule), in both of the sequence's chunks."""
    import torch
    from sparse_long_context_lightning_amd import to_device_bf16
    lens = [3000]
    top_k = 256
    cu, qi, ki, w = _general_inputs(lens, 64, 128, seed=313)
    total = int(cu[-1])
    rng = np.random.default_rng(314)
    q, k, v = (inp.f32_to_bf16_bits(rng.standard_normal(s).astype(np.float32))
               for s in ((total, 32, 128), (total, 4, 128), (total, 4, 128)))
    dq, dk, dv, dqi, dki = (to_device_bf16(x) for x in (q, k, v, qi, ki))
    dw = torch.from_numpy(w).cuda()
    out, lse, idx = dsa.prefill(dq, dk, dv, dqi, dki, dw, cu, top_k)
    scores = torch.empty((total, total), dtype=torch.float32, device="cuda")
    dsa.dsa_index_scores(dqi, dki, dw, cu, 0, total, scores)
    row_len = torch.arange(1, total + 1, dtype=torch.int32, device="cuda")
    ref = torch.empty((total, top_k), dtype=torch.int32, device="cuda")
    dsa.dsa_topk(scores, row_len, top_k, ref)
    got, want = idx.cpu().numpy(), ref.cpu().numpy()
    assert np.array_equal(got, want), f"first differing row {int(np.argmax((got != want).any(axis=1)))}"
    # the rows just past k select with a negative k-th score
    sc = scores.cpu().numpy()
    kth = np.array([np.sort(sc[t, :t + 1])[::-1][top_k - 1] for t in range(top_k, 700)])
    assert (kth < 0).sum() > 50
