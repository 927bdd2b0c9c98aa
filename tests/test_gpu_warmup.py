"""The indexer's dense warm-up pieces through the C ABI against the oracle: the head-mean causal
attention target (dsa_attn_head_mean) and the per-row KL divergence with its gradient
(dsa_indexer_kl).  GPU only.

Tolerances: the target's logits are fp32 sums of exact bf16 products, so the probabilities
differ from float64 only by fp32 rounding and the exp2 approximation (checked at 2e-6 absolute,
2e-4 relative); the KL loss is an fp32 sum over up to a few thousand terms (relative 1e-4) and
its gradient r - p is checked at 2e-6 absolute."""

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import dsa_oracle as orc
from sparse_long_context_lightning_amd import inputs as inp

import dsa_testlib as tl

pytestmark = pytest.mark.gpu


def _target_case(dsa, lens, hq, hkv, row_begin=0, row_count=None, seed=0):
    import torch
    pi = inp.prefill_inputs(lens, 4, 64, hq, hkv, 128, 64, seed=seed)
    dev = tl.upload_prefill(pi)
    total = sum(lens)
    row_count = total - row_begin if row_count is None else row_count
    ld = (max(lens) + 3) // 4 * 4
    probs = torch.full((row_count, ld), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((row_count, hq), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa_attn_head_mean(dev["q"], dev["k"], pi.cu_seqlens, row_begin, row_count, probs, lse)
    torch.cuda.synchronize()
    return pi, probs.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("lens,hq,hkv", [([300, 70], 32, 4), ([200], 16, 1), ([129, 3], 16, 4), ([150], 32, 8),
                                         ([170, 40], 48, 4), ([90], 12, 1), ([260], 24, 2)])
def test_head_mean_target_matches_oracle(dsa, lens, hq, hkv):
    pi, probs, lse = _target_case(dsa, lens, hq, hkv, seed=sum(lens) + hq)
    q, k = tl.f64(pi.q), tl.f64(pi.k)
    scale = orc.default_softmax_scale(128)
    cu = pi.cu_seqlens
    g = hq // hkv
    for b in range(len(lens)):
        o = int(cu[b])
        for t in range(lens[b]):
            r = o + t
            want = orc.attention_head_mean_row(q[r], k[o:o + t + 1], scale)
            np.testing.assert_allclose(probs[r, :t + 1], want, atol=2e-6, rtol=2e-4, err_msg=f"row {r}")
            assert np.all(np.isnan(probs[r, t + 1:])), "entries past the prefix must stay untouched"
            z = scale * np.einsum("shd,hd->hs", np.repeat(k[o:o + t + 1], g, axis=1), q[r])
            np.testing.assert_allclose(lse[r], logsumexp(z, axis=1), atol=1e-4, rtol=1e-5)


@pytest.mark.parametrize("hq,hkv", [(32, 4), (16, 1), (32, 8), (64, 4), (48, 4), (4, 1)])
def test_head_mean_target_with_split_keys(dsa, hq, hkv):
    """Rows whose prefixes span several 2048-key splits (the kernel's key split: per-split
    statistics merged into lse, per-split probabilities): a window of a 5000-token sequence packed
    after a 700-token one that crosses the 4096-key split boundary, and a window across the two
    sequences' boundary; probabilities, untouched entries past each prefix and lse."""
    lens = [700, 5000]
    o = lens[0]
    for row_begin, row_count in ((o + 4060, 70), (o - 6, 12), (o + 2040, 17)):
        pi, probs, lse = _target_case(dsa, lens, hq, hkv, row_begin=row_begin, row_count=row_count,
                                      seed=hq + 7 * hkv + row_begin)
        q, k = tl.f64(pi.q), tl.f64(pi.k)
        scale = orc.default_softmax_scale(128)
        g = hq // hkv
        for i in range(row_count):
            r = row_begin + i
            b = 0 if r < o else 1
            t = r - (0 if b == 0 else o)
            kp = k[(0 if b == 0 else o):r + 1]
            want = orc.attention_head_mean_row(q[r], kp, scale)
            np.testing.assert_allclose(probs[i, :t + 1], want, atol=2e-6, rtol=2e-4, err_msg=f"row {r}")
            assert np.all(np.isnan(probs[i, t + 1:])), f"row {r}: entries past the prefix must stay untouched"
            z = scale * np.einsum("shd,hd->hs", np.repeat(kp, g, axis=1), q[r])
            np.testing.assert_allclose(lse[i], logsumexp(z, axis=1), atol=1e-4, rtol=1e-5, err_msg=f"lse of row {r}")


def test_head_mean_target_row_window(dsa):
    pi, probs, lse = _target_case(dsa, [260], 32, 4, row_begin=100, row_count=90, seed=3)
    q, k = tl.f64(pi.q), tl.f64(pi.k)
    scale = orc.default_softmax_scale(128)
    for i in range(90):
        t = 100 + i
        want = orc.attention_head_mean_row(q[t], k[:t + 1], scale)
        np.testing.assert_allclose(probs[i, :t + 1], want, atol=2e-6, rtol=2e-4)


def test_indexer_kl_matches_oracle(dsa):
    import torch
    rng = np.random.default_rng(12)
    lens = np.array([1, 2, 7, 64, 257, 1000, 3000])
    rows, ld = len(lens), 3000
    scores = np.zeros((rows, ld), dtype=np.float32)
    target = np.zeros((rows, ld), dtype=np.float32)
    for i, n in enumerate(lens):
        scores[i, :n] = (rng.standard_normal(n) * (3.0 if i % 2 else 40.0)).astype(np.float32)
        p = rng.random(n) ** 4
        p[rng.random(n) < 0.2] = 0.0
        p[0] = max(p[0], 1e-3)
        target[i, :n] = (p / p.sum()).astype(np.float32)
    s_t = torch.from_numpy(scores).cuda()
    p_t = torch.from_numpy(target).cuda()
    rl = torch.from_numpy(lens.astype(np.int32)).cuda()
    loss = torch.empty(rows, dtype=torch.float32, device="cuda")
    grad = torch.empty_like(s_t)
    dsa.dsa_indexer_kl(s_t, p_t, rl, loss, grad)
    dsa.dsa_indexer_kl(s_t, p_t, rl, loss, s_t)          # in place over the scores
    torch.cuda.synchronize()
    got_l, got_g, got_inplace = loss.cpu().numpy(), grad.cpu().numpy(), s_t.cpu().numpy()
    for i, n in enumerate(lens):
        want_l, want_g = orc.indexer_kl_row(scores[i, :n].astype(np.float64), target[i, :n].astype(np.float64))
        assert abs(got_l[i] - want_l) <= 1e-4 * max(1.0, abs(want_l)), (i, got_l[i], want_l)
        np.testing.assert_allclose(got_g[i, :n], want_g, atol=2e-6)
        np.testing.assert_array_equal(got_inplace[i, :n], got_g[i, :n])


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_head_mean_target_full_32k(dsa):
    """The 32K prefill's target in the benchmark's launch configuration (2048-row windows):
    sampled rows of the first and the last window recomputed by the oracle one by one."""
    import torch
    pi = inp.workload("c2_prefill_32k")
    total = int(pi.cu_seqlens[-1])
    hq = pi.q.shape[1]
    dev = tl.upload_prefill(pi)
    q, k = tl.f64(pi.q), tl.f64(pi.k)
    scale = orc.default_softmax_scale(128)
    chunk = 2048
    probs = torch.empty(chunk, total, dtype=torch.float32, device="cuda")
    lse = torch.empty(chunk, hq, dtype=torch.float32, device="cuda")
    for c0, rows in ((0, [0, 1, 777, 2047]), (total - chunk, [total - chunk, total - 1000, total - 1])):
        dsa.dsa_attn_head_mean(dev["q"], dev["k"], pi.cu_seqlens, c0, chunk, probs, lse, ld=total)
        torch.cuda.synchronize()
        got = probs.cpu().numpy().astype(np.float64)
        got_lse = lse.cpu().numpy().astype(np.float64)
        g = hq // k.shape[1]
        for r in rows:
            want = orc.attention_head_mean_row(q[r], k[:r + 1], scale)
            np.testing.assert_allclose(got[r - c0, :r + 1], want, atol=2e-6, rtol=2e-4, err_msg=f"row {r}")
            z = scale * np.einsum("shd,hd->hs", np.repeat(k[:r + 1], g, axis=1), q[r])
            np.testing.assert_allclose(got_lse[r - c0], logsumexp(z, axis=1), atol=1e-4, rtol=1e-5,
                                       err_msg=f"lse of row {r}")
