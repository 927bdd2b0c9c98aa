"""Pins of the CPU oracle against things other than itself: hand-worked examples, closed
forms, library routines (integer matmul, torch.topk, torch SDPA, scipy logsumexp) and brute
force on tiny inputs.  CPU only."""

import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import dsa_oracle as orc
from sparse_long_context_lightning_amd import inputs as inp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- indexer scores

def test_scores_hand_worked_example():
    g = _load("indexer_worked_example.json")
    q = np.array(g["q_idx"], dtype=np.float64)
    k = np.array(g["k_idx"], dtype=np.float64)
    w = np.array(g["w"], dtype=np.float64)
    got = orc.index_scores(q, k, w, [0, 3])
    for row, want in zip(got, g["scores"]):
        assert row.tolist() == want


def test_scores_single_head_unit_weight_is_relu_of_integer_matmul():
    rng = np.random.default_rng(11)
    t, d = 37, 16
    q = rng.integers(-3, 4, size=(t, 1, d))
    k = rng.integers(-3, 4, size=(t, d))
    w = np.ones((t, 1))
    full = np.maximum(q[:, 0, :].astype(np.int64) @ k.astype(np.int64).T, 0)  # textbook matmul on int64
    got = orc.index_scores(q, k, w, [0, t])
    for r in range(t):
        assert np.array_equal(got[r], full[r, : r + 1].astype(np.float64))


def test_scores_relu_sign_identity():
    # ReLU(-x) - ReLU(x) = -x, so I(-q) - I(q) = -sum_j w_j <q_j, k_s>: catches a dropped or
    # mis-signed ReLU and a wrong weight/head pairing.
    rng = np.random.default_rng(12)
    t, h, d = 23, 3, 8
    q = rng.integers(-3, 4, size=(t, h, d)).astype(np.float64)
    k = rng.integers(-3, 4, size=(t, d)).astype(np.float64)
    w = rng.choice([0.125, 0.25, 0.5, 1.0, -0.5], size=(t, h))
    pos = orc.index_scores(q, k, w, [0, t])
    neg = orc.index_scores(-q, k, w, [0, t])
    lin = np.einsum("tj,tjd,sd->ts", w, q, k)
    for r in range(t):
        assert np.array_equal(neg[r] - pos[r], -lin[r, : r + 1])


def test_scores_weight_belongs_to_query_row():
    rng = np.random.default_rng(13)
    t, h, d = 17, 4, 8
    q = rng.integers(-3, 4, size=(t, h, d)).astype(np.float64)
    k = rng.integers(-3, 4, size=(t, d)).astype(np.float64)
    w = rng.choice([0.125, 0.25, 0.5, 1.0], size=(t, h))
    base = orc.index_scores(q, k, w, [0, t])
    w2 = w.copy()
    w2[9] *= 2.0
    moved = orc.index_scores(q, k, w2, [0, t])
    for r in range(t):
        assert np.array_equal(moved[r], base[r] * (2.0 if r == 9 else 1.0))


def test_scores_are_causal_and_sequence_local():
    rng = np.random.default_rng(14)
    lens = [5, 9, 3]
    tot = sum(lens)
    q = rng.integers(-3, 4, size=(tot, 2, 4)).astype(np.float64)
    k = rng.integers(-3, 4, size=(tot, 4)).astype(np.float64)
    w = np.ones((tot, 2))
    got = orc.index_scores(q, k, w, [0, 5, 14, 17])
    assert [len(r) for r in got] == [t + 1 for n in lens for t in range(n)]
    # brute force with explicit loops for the second sequence
    for t in range(9):
        r = 5 + t
        for s in range(t + 1):
            want = 0.0
            for j in range(2):
                dot = sum(q[r, j, c] * k[5 + s, c] for c in range(4))
                want += w[r, j] * max(0.0, dot)
            assert got[r][s] == want


def test_scores_exact_for_workload_value_ranges():
    # Worst case of the large workloads: 64 heads * 128 dims * 9 per product, in 1/8 steps,
    # stays below 2**24 units, so float32 represents every score exactly.
    worst = 64 * 128 * 9
    assert worst * 8 < 2 ** 24
    pi = inp.prefill_inputs([300], 64, 128, 8, 2, 128, 64, seed=5)
    q = inp.bf16_bits_to_f32(pi.q_idx).astype(np.float64)
    k = inp.bf16_bits_to_f32(pi.k_idx).astype(np.float64)
    rows = orc.index_scores(q, k, pi.w.astype(np.float64), pi.cu_seqlens)
    for r in rows[::37]:
        assert np.array_equal(r.astype(np.float32).astype(np.float64), r)
        assert np.array_equal(r * 8, np.round(r * 8))


# ---------------------------------------------------------------- top-k selection

def _brute_topk(scores, k):
    n = len(scores)
    if n <= k:
        return list(range(n)) + [-1] * (k - n)
    ranked = sorted(range(n), key=lambda s: (-scores[s], s))
    return sorted(ranked[:k])


def test_topk_hand_worked_example():
    g = _load("indexer_worked_example.json")
    for kk, want_rows in g["topk"].items():
        for sc, want in zip(g["scores"], want_rows):
            assert orc.select_topk_row(np.array(sc), int(kk)).tolist() == want
    for case in g["tie_rows"]:
        assert orc.select_topk_row(np.array(case["scores"]), case["k"]).tolist() == case["idx"]


@pytest.mark.parametrize("seed", range(6))
def test_topk_equals_bruteforce_sort_with_ties(seed):
    rng = np.random.default_rng(100 + seed)
    for _ in range(60):
        n = int(rng.integers(1, 70))
        k = int(rng.integers(1, 40))
        sc = rng.integers(-2, 4, size=n) / 8.0          # heavy ties
        assert orc.select_topk_row(sc, k).tolist() == _brute_topk(sc.tolist(), k)


def test_topk_special_rows():
    n, k = 50, 8
    assert orc.select_topk_row(np.zeros(n), k).tolist() == list(range(k))
    assert orc.select_topk_row(np.arange(n, 0, -1.0), k).tolist() == list(range(k))
    assert orc.select_topk_row(np.arange(n, dtype=np.float64), k).tolist() == list(range(n - k, n))
    assert orc.select_topk_row(np.arange(5.0), k).tolist() == [0, 1, 2, 3, 4, -1, -1, -1]
    assert orc.select_topk_row(np.arange(8.0), 8).tolist() == list(range(8))


def test_topk_matches_torch_topk_without_ties():
    rng = np.random.default_rng(7)
    for n, k in [(100, 10), (1000, 256), (4097, 2048)]:
        sc = rng.permutation(n).astype(np.float64) * 0.5 - 17.0
        ref = torch.topk(torch.from_numpy(sc), k).indices.sort().values.numpy()
        assert np.array_equal(orc.select_topk_row(sc, k), ref)


def _brute_topk_sorted(scores, k):
    """Pure-Python ranking by (-score, position), kept in rank order, padded with -1 / -inf."""
    n = len(scores)
    ranked = sorted(range(n), key=lambda s: (-scores[s], s))[:k]
    return ranked + [-1] * (k - len(ranked)), [scores[s] for s in ranked] + [-math.inf] * (k - len(ranked))


@pytest.mark.parametrize("seed", range(4))
def test_topk_sorted_equals_bruteforce_ranking_with_ties(seed):
    rng = np.random.default_rng(300 + seed)
    for _ in range(60):
        n = int(rng.integers(1, 70))
        k = int(rng.integers(1, 40))
        sc = rng.integers(-2, 4, size=n) / 8.0          # heavy ties
        idx, val = orc.select_topk_sorted_row(sc, k)
        want_idx, want_val = _brute_topk_sorted(sc.tolist(), k)
        assert idx.tolist() == want_idx
        assert val.tolist() == want_val


def test_topk_sorted_matches_torch_topk_sorted_without_ties():
    rng = np.random.default_rng(8)
    for n, k in [(100, 10), (1000, 256), (4097, 2048)]:
        sc = rng.permutation(n).astype(np.float64) * 0.25 - 3.0
        ref = torch.topk(torch.from_numpy(sc), k, sorted=True)
        idx, val = orc.select_topk_sorted_row(sc, k)
        assert np.array_equal(idx, ref.indices.numpy())
        assert np.array_equal(val, ref.values.numpy())


def test_topk_sorted_keeps_the_same_set_as_the_ascending_form():
    rng = np.random.default_rng(9)
    for n, k in [(3, 8), (64, 64), (500, 37), (3000, 2048)]:
        sc = rng.integers(-5, 6, size=n) / 4.0
        idx, val = orc.select_topk_sorted_row(sc, k)
        asc = orc.select_topk_row(sc, k)
        assert np.array_equal(np.sort(idx[idx >= 0]), asc[asc >= 0])
        assert np.all(np.diff(val[idx >= 0]) <= 0)
        assert np.all(idx[min(n, k):] == -1) and np.all(np.isneginf(val[min(n, k):]))


# ---------------------------------------------------------------- sparse attention

def test_attention_hand_worked_example():
    g = _load("attention_worked_example.json")
    o, lse, ws = orc.sparse_gqa_attention_row(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]),
                                              np.array(g["idx"]), g["scale"])
    np.testing.assert_allclose(o, np.array(g["out"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(g["lse"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(ws, 1.0, atol=1e-12)


def _sdpa_masked(q, k, v, mask, scale):
    """torch SDPA in float64 on the CPU; q [T,Hq,D], k/v [S,Hkv,D], mask [T,S] bool (True = keep)."""
    hq, hkv = q.shape[1], k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0)
    kt = torch.from_numpy(k).repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2).unsqueeze(0).contiguous()
    vt = torch.from_numpy(v).repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2).unsqueeze(0).contiguous()
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask),
                                                           scale=scale)
    return out[0].permute(1, 0, 2).numpy()


def _rand_attn(seed, t, hq, hkv, d):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((t, hq, d)), rng.standard_normal((t, hkv, d)), rng.standard_normal((t, hkv, d)))


def test_attention_with_k_at_least_length_is_dense_causal_gqa():
    t, hq, hkv, d, h_i, d_i = 40, 8, 2, 16, 2, 8
    q, k, v = _rand_attn(21, t, hq, hkv, d)
    rng = np.random.default_rng(22)
    qi = rng.integers(-3, 4, size=(t, h_i, d_i)).astype(np.float64)
    ki = rng.integers(-3, 4, size=(t, d_i)).astype(np.float64)
    w = np.ones((t, h_i))
    scale = 1 / math.sqrt(d)
    res = orc.prefill(q, k, v, qi, ki, w, [0, t], top_k=t, softmax_scale=scale)
    ref = _sdpa_masked(q, k, v, np.tril(np.ones((t, t), dtype=bool)), scale)
    np.testing.assert_allclose(res["out"], ref, atol=1e-12)


def test_attention_equals_sdpa_with_index_mask():
    t, hq, hkv, d = 60, 4, 2, 8
    q, k, v = _rand_attn(31, t, hq, hkv, d)
    rng = np.random.default_rng(32)
    scale = 0.3
    mask = np.zeros((t, t), dtype=bool)
    for r in range(t):
        n = int(rng.integers(1, r + 2))
        sel = np.sort(rng.choice(r + 1, size=n, replace=False))
        mask[r, sel] = True
        idx = np.full(t, -1)
        idx[:n] = sel
        o, lse, ws = orc.sparse_gqa_attention_row(q[r], k, v, idx, scale)
        ref = _sdpa_masked(q[r:r + 1], k, v, mask[r:r + 1], scale)[0]
        np.testing.assert_allclose(o, ref, atol=1e-12)
        np.testing.assert_allclose(ws, 1.0, atol=1e-12)
        for h in range(hq):
            z = scale * (k[sel, h // (hq // hkv)] @ q[r, h])
            assert abs(lse[h] - logsumexp(z)) < 1e-12


def test_attention_unit_values_and_single_position():
    t, hq, hkv, d = 12, 6, 3, 8
    q, k, v = _rand_attn(41, t, hq, hkv, d)
    ones = np.ones_like(v)
    idx = np.array([0, 3, 7, 11, -1, -1])
    o, _, _ = orc.sparse_gqa_attention_row(q[11], k, ones, idx, 0.5)
    np.testing.assert_allclose(o, 1.0, atol=1e-14)
    o1, lse1, _ = orc.sparse_gqa_attention_row(q[0], k, v, np.array([0, -1]), 0.5)
    for h in range(hq):
        assert np.array_equal(o1[h], v[0, h // 2])
        assert abs(lse1[h] - 0.5 * (k[0, h // 2] @ q[0, h])) < 1e-14


def test_attention_index_order_is_irrelevant():
    t, hq, hkv, d = 30, 4, 1, 8
    q, k, v = _rand_attn(51, t, hq, hkv, d)
    idx = np.array([2, 5, 11, 29, 17, -1])
    a = orc.sparse_gqa_attention_row(q[29], k, v, idx, 0.4)
    b = orc.sparse_gqa_attention_row(q[29], k, v, idx[[4, 0, 5, 3, 1, 2]], 0.4)
    np.testing.assert_allclose(a[0], b[0], atol=1e-13)


# ---------------------------------------------------------------- adjacent-query dedup

def test_union_hand_worked_example():
    g = _load("dedup_worked_example.json")
    got = orc.adjacent_query_union(np.array(g["idx"]), g["cu_seqlens"], block_rows=g["block_rows"])
    assert len(got) == len(g["blocks"])
    for (kv, m), want in zip(got, g["blocks"]):
        assert kv.tolist() == want["kv_rows"]
        assert m.tolist() == want["masks"]


def _random_index_lists(rng, cu, k, p_bad=0.1):
    """Index lists with repeats, negative entries and entries past the causal prefix."""
    total = cu[-1]
    idx = np.empty((total, k), dtype=np.int64)
    for b in range(len(cu) - 1):
        for t in range(cu[b + 1] - cu[b]):
            row = rng.integers(0, t + 1, size=k)
            bad = rng.random(k) < p_bad
            row[bad] = rng.choice([-1, -7, t + 1, t + 40], size=int(bad.sum()))
            idx[cu[b] + t] = row
    return idx


@pytest.mark.parametrize("block_rows", [16, 5])
def test_union_masks_rebuild_every_rows_distinct_valid_set(block_rows):
    rng = np.random.default_rng(61)
    cu = [0, 37, 38, 90]
    idx = _random_index_lists(rng, cu, 12)
    blocks = orc.adjacent_query_union(idx, cu, block_rows=block_rows)
    assert len(blocks) == (cu[-1] + block_rows - 1) // block_rows
    for b, (kv, m) in enumerate(blocks):
        assert np.all(np.diff(kv) > 0) and np.all(m > 0) and np.all(m < (1 << block_rows))
        for j in range(block_rows):
            r = b * block_rows + j
            mine = set(kv[((m >> j) & 1) == 1].tolist())
            if r >= cu[-1]:
                assert not mine
                continue
            s = max(i for i in range(len(cu) - 1) if cu[i] <= r)
            t = r - cu[s]
            assert mine == {cu[s] + int(p) for p in idx[r] if 0 <= p <= t}, (b, j)
        want = np.unique(np.concatenate([kv[((m >> j) & 1) == 1] for j in range(block_rows)] + [kv[:0]]))
        assert np.array_equal(kv, want)


def test_union_size_matches_independent_inclusion_probability():
    # Rows that draw k distinct positions uniformly from their prefixes [0, t_j] include a given
    # position s with probability k / (t_j + 1), independently of each other, so the expected
    # union size of a block is sum_s (1 - prod_j (1 - [s <= t_j] k / (t_j + 1))).
    rng = np.random.default_rng(62)
    t0, n_blocks, k = 600, 40, 64
    total = t0 + 16 * n_blocks
    idx = np.full((total, k), -1, dtype=np.int64)
    for t in range(t0, total):
        idx[t] = rng.choice(t + 1, size=k, replace=False)
    blocks = orc.adjacent_query_union(idx, [0, total], blocks=range(t0 // 16 + 1, total // 16))
    got = np.mean([len(kv) for kv, _ in blocks])
    want = []
    for b in range(t0 // 16 + 1, total // 16):
        ts = np.arange(16 * b, 16 * b + 16)
        s = np.arange(ts[-1] + 1)[:, None]
        miss = np.where(s <= ts[None, :], 1.0 - k / (ts[None, :] + 1.0), 1.0)
        want.append(float(np.sum(1.0 - np.prod(miss, axis=1))))
    want = float(np.mean(want))
    assert abs(got - want) < 0.01 * want, (got, want)


def test_union_attention_equals_per_row_attention_over_distinct_positions():
    hq, hkv, d = 4, 2, 8
    cu = [0, 21, 40]
    rng = np.random.default_rng(63)
    q, k, v = _rand_attn(64, cu[-1], hq, hkv, d)
    idx = _random_index_lists(rng, cu, 6)
    for b, (kv, m) in enumerate(orc.adjacent_query_union(idx, cu, block_rows=8)):
        n = min(8, cu[-1] - 8 * b)
        o, lse = orc.sparse_gqa_attention_union(q, k, v, kv, m, 8 * b, n, 0.3)
        for j in range(n):
            r = 8 * b + j
            s = 0 if r < cu[1] else 1
            t = r - cu[s]
            sel = np.unique([p for p in idx[r] if 0 <= p <= t]).astype(np.int64)
            o_ref, l_ref, _ = orc.sparse_gqa_attention_row(q[r], k[cu[s]:cu[s + 1]], v[cu[s]:cu[s + 1]], sel, 0.3)
            np.testing.assert_allclose(o[j], o_ref, atol=1e-13)
            np.testing.assert_allclose(lse[j], l_ref, atol=1e-13)


# ---------------------------------------------------------------- composition

# ---------------------------------------------------------------- sparse attention backward

def _sparse_loss(q, k, v, idx, cu, dout, scale):
    """sum(dout * O) through the oracle forward: its gradient is what the backward returns."""
    total = 0.0
    for b in range(len(cu) - 1):
        o = cu[b]
        for t in range(cu[b + 1] - o):
            r = o + t
            sel = np.asarray([i for i in idx[r] if 0 <= i <= t])
            out, _, _ = orc.sparse_gqa_attention_row(q[r], k[o:o + t + 1], v[o:o + t + 1], sel, scale)
            total += float((out * dout[r]).sum())
    return total


def test_attention_grad_matches_central_differences():
    rng = np.random.default_rng(31)
    lens, hq, hkv, d, k_sel = [5, 4], 4, 2, 6, 3
    cu = [0, 5, 9]
    total = sum(lens)
    q, k, v = _rand_attn(32, total, hq, hkv, d)
    dout = rng.standard_normal((total, hq, d))
    idx = np.full((total, k_sel), -1, dtype=np.int64)
    for b in range(2):
        for t in range(lens[b]):
            n = int(rng.integers(1, min(t + 1, k_sel) + 1))
            idx[cu[b] + t, :n] = rng.choice(t + 1, size=n, replace=False)
    idx[6, 1] = 7 if idx[6, 1] < 0 else idx[6, 1]     # an out-of-prefix entry (t = 1) is ignored
    scale = 0.37
    dq, dk, dv = orc.sparse_attention_grad(q, k, v, idx, cu, dout, scale)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for pos in np.ndindex(*x.shape):
            old = x[pos]
            x[pos] = old + eps
            lp = _sparse_loss(q, k, v, idx, cu, dout, scale)
            x[pos] = old - eps
            lm = _sparse_loss(q, k, v, idx, cu, dout, scale)
            x[pos] = old
            num[pos] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, num, atol=1e-7, rtol=1e-6, err_msg=name)


def test_attention_grad_with_all_positions_is_dense_causal_gqa_autograd():
    t, hq, hkv, d = 24, 8, 2, 16
    q, k, v = _rand_attn(33, t, hq, hkv, d)
    dout = np.random.default_rng(34).standard_normal((t, hq, d))
    idx = np.full((t, t), -1, dtype=np.int64)
    for r in range(t):
        idx[r, :r + 1] = np.arange(r + 1)
    scale = 1 / math.sqrt(d)
    dq, dk, dv = orc.sparse_attention_grad(q, k, v, idx, [0, t], dout, scale)
    qt = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0).requires_grad_(True)
    kt = torch.from_numpy(k).permute(1, 0, 2).unsqueeze(0).requires_grad_(True)
    vt = torch.from_numpy(v).permute(1, 0, 2).unsqueeze(0).requires_grad_(True)
    g = hq // hkv
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(g, dim=1), vt.repeat_interleave(g, dim=1), is_causal=True, scale=scale)
    out.backward(torch.from_numpy(dout).permute(1, 0, 2).unsqueeze(0))
    np.testing.assert_allclose(dq, qt.grad[0].permute(1, 0, 2).numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad[0].permute(1, 0, 2).numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad[0].permute(1, 0, 2).numpy(), atol=1e-12)


def test_attention_grad_single_position_closed_form():
    # one selected key: p = 1, so dq = 0, dk = 0 and dv = sum of the group's dO rows
    t, hq, hkv, d = 3, 4, 2, 5
    q, k, v = _rand_attn(35, t, hq, hkv, d)
    dout = np.random.default_rng(36).standard_normal((t, hq, d))
    idx = np.array([[0], [0], [2]])
    dq, dk, dv = orc.sparse_attention_grad(q, k, v, idx, [0, t], dout, 0.5)
    assert np.all(dq == 0) and np.all(dk == 0)
    want = np.zeros_like(v)
    for r, s in ((0, 0), (1, 0), (2, 2)):
        for h in range(hq):
            want[s, h // 2] += dout[r, h]
    np.testing.assert_allclose(dv, want, atol=1e-14)


# ---------------------------------------------------------------- indexer warm-up (KL) loss

def _torch_warmup(q, k, qi, ki, w, lens, scale):
    """The warm-up loss written with torch ops (masked dense matrices, autograd for the gradients)."""
    out_loss, grads = [], []
    qi_t = torch.from_numpy(qi).requires_grad_(True)
    ki_t = torch.from_numpy(ki).requires_grad_(True)
    w_t = torch.from_numpy(w).requires_grad_(True)
    total = 0
    o = 0
    loss_sum = torch.zeros((), dtype=torch.float64)
    for n in lens:
        qs, ks = torch.from_numpy(q[o:o + n]), torch.from_numpy(k[o:o + n])
        g = qs.shape[1] // ks.shape[1]
        causal = torch.tril(torch.ones(n, n, dtype=torch.bool))
        logits = scale * torch.einsum("thd,shd->hts", qs, ks.repeat_interleave(g, dim=1))
        logits = logits.masked_fill(~causal, float("-inf"))
        target = torch.softmax(logits, dim=-1).mean(dim=0)                       # [t, s]
        c = torch.einsum("tjd,sd->tjs", qi_t[o:o + n], ki_t[o:o + n])
        scores = (w_t[o:o + n, :, None] * torch.relu(c)).sum(dim=1)              # [t, s]
        log_r = torch.log_softmax(scores.masked_fill(~causal, float("-inf")), dim=-1)
        safe = torch.where(target > 0, target, torch.ones_like(target))
        kl = torch.where(target > 0, target * (torch.log(safe) - log_r), torch.zeros_like(target)).sum(dim=-1)
        out_loss.append(kl.detach().numpy())
        loss_sum = loss_sum + kl.sum()
        o += n
    loss_sum.backward()
    return np.concatenate(out_loss), qi_t.grad.numpy(), ki_t.grad.numpy(), w_t.grad.numpy()


def test_warmup_loss_and_grads_match_torch_autograd():
    rng = np.random.default_rng(41)
    lens, hq, hkv, d, h_i, d_i = [9, 5], 4, 2, 8, 3, 6
    total = sum(lens)
    q, k, _ = _rand_attn(42, total, hq, hkv, d)
    qi = rng.standard_normal((total, h_i, d_i))
    ki = rng.standard_normal((total, d_i))
    w = rng.standard_normal((total, h_i))                 # signed weights: both branches of ReLU matter
    scale = 0.3
    got = orc.indexer_warmup_loss_grads(q, k, qi, ki, w, [0, 9, 14], scale)
    want = _torch_warmup(q, k, qi, ki, w, lens, scale)
    for name, a, b in zip(("loss", "dq_idx", "dk_idx", "dw"), got, want):
        np.testing.assert_allclose(a, b, atol=1e-12, err_msg=name)


def test_warmup_grads_match_central_differences():
    rng = np.random.default_rng(43)
    lens, hq, hkv, d, h_i, d_i = [6], 2, 1, 4, 2, 3
    q, k, _ = _rand_attn(44, 6, hq, hkv, d)
    qi = rng.standard_normal((6, h_i, d_i))
    ki = rng.standard_normal((6, d_i))
    w = rng.standard_normal((6, h_i))
    _, dq, dk, dw = orc.indexer_warmup_loss_grads(q, k, qi, ki, w, [0, 6], 0.5)

    def total_loss():
        return orc.indexer_warmup_loss_grads(q, k, qi, ki, w, [0, 6], 0.5)[0].sum()

    eps = 1e-6
    for name, x, g in (("q_idx", qi, dq), ("k_idx", ki, dk), ("w", w, dw)):
        num = np.zeros_like(x)
        for pos in np.ndindex(*x.shape):
            old = x[pos]
            x[pos] = old + eps
            lp = total_loss()
            x[pos] = old - eps
            lm = total_loss()
            x[pos] = old
            num[pos] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, num, atol=1e-7, rtol=1e-6, err_msg=name)


def test_kl_is_zero_when_the_indexer_matches_the_target_and_positive_otherwise():
    rng = np.random.default_rng(45)
    p = rng.random(50)
    p /= p.sum()
    loss, grad = orc.indexer_kl_row(np.log(p) + 3.0, p)
    assert abs(loss) < 1e-12 and np.max(np.abs(grad)) < 1e-12
    loss2, grad2 = orc.indexer_kl_row(rng.standard_normal(50), p)
    assert loss2 > 0 and abs(grad2.sum()) < 1e-12
    # a target with zeros: those terms add nothing to the loss
    p0 = p.copy()
    p0[:10] = 0
    p0 /= p0.sum()
    sc = rng.standard_normal(50)
    r = np.exp(sc - sc.max())
    r /= r.sum()
    want = float(np.sum(p0[10:] * (np.log(p0[10:]) - np.log(r[10:]))))
    assert abs(orc.indexer_kl_row(sc, p0)[0] - want) < 1e-12


def test_head_mean_target_is_a_distribution_and_single_head_softmax():
    q, k, _ = _rand_attn(46, 7, 4, 2, 8)
    for t in range(7):
        p = orc.attention_head_mean_row(q[t], k[:t + 1], 0.4)
        assert p.shape == (t + 1,) and abs(p.sum() - 1) < 1e-12 and np.all(p > 0)
    q1, k1, _ = _rand_attn(47, 5, 1, 1, 8)
    z = 0.4 * (k1[:, 0] @ q1[4, 0])
    np.testing.assert_allclose(orc.attention_head_mean_row(q1[4], k1, 0.4), np.exp(z) / np.exp(z).sum(), atol=1e-15)


def test_packed_prefill_equals_separate_sequences():
    lens = [20, 7, 13]
    pi = inp.prefill_inputs(lens, 2, 8, 4, 2, 16, 6, seed=9)
    f = inp.bf16_bits_to_f32
    arrs = [f(pi.q), f(pi.k), f(pi.v), f(pi.q_idx), f(pi.k_idx), pi.w]
    packed = orc.prefill(*arrs, pi.cu_seqlens, top_k=6)
    o = 0
    for n in lens:
        part = orc.prefill(*[a[o:o + n] for a in arrs], [0, n], top_k=6)
        assert np.array_equal(packed["idx"][o:o + n], part["idx"])
        np.testing.assert_allclose(packed["out"][o:o + n], part["out"], atol=1e-13)
        o += n


def test_decode_equals_last_prefill_row():
    s, hq, hkv, d, h_i, d_i, kk = 50, 4, 2, 8, 2, 8, 10
    pi = inp.prefill_inputs([s], h_i, d_i, hq, hkv, d, kk, seed=10)
    f = inp.bf16_bits_to_f32
    q, k, v, qi, ki = f(pi.q), f(pi.k), f(pi.v), f(pi.q_idx), f(pi.k_idx)
    pre = orc.prefill(q, k, v, qi, ki, pi.w, pi.cu_seqlens, top_k=kk, rows=[s - 1])
    dec = orc.decode(q[s - 1:s], qi[s - 1:s], pi.w[s - 1:s], k[None], v[None], ki[None],
                     np.array([s]), top_k=kk)
    assert np.array_equal(pre["idx"][0], dec["idx"][0])
    np.testing.assert_allclose(pre["out"][0], dec["out"][0], atol=1e-13)


# ---------------------------------------------------------------- synthetic inputs

def test_inputs_are_deterministic_and_in_range():
    a = inp.prefill_inputs([64, 32], 4, 64, 8, 2, 128, 16, seed=3, structure="blocks16")
    b = inp.prefill_inputs([64, 32], 4, 64, 8, 2, 128, 16, seed=3, structure="blocks16")
    for x, y in [(a.q, b.q), (a.k_idx, b.k_idx), (a.w, b.w), (a.k, b.k)]:
        assert np.array_equal(x, y)
    vals = inp.bf16_bits_to_f32(a.q_idx)
    assert set(np.unique(vals).tolist()) <= set(range(-3, 4))
    assert set(np.unique(inp.bf16_bits_to_f32(a.k_idx)).tolist()) <= set(range(-3, 4))
    assert set(np.unique(a.w).tolist()) <= {1.0, 0.5, 0.25, 0.125}


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10 ** rng.uniform(-3, 3, 100000)).astype(np.float32)
    ours = inp.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(inp.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())
