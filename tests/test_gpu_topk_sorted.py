"""The torch.topk-shaped top-k (dsa_topk_sorted) against the oracle's ranking, through the C ABI,
on both selection paths (with and without scratch).  GPU only."""

import numpy as np
import pytest

from oracle import dsa_oracle as orc

pytestmark = pytest.mark.gpu


def _run_sorted(dsa, scores_np, lens, k):
    import torch
    rows, ld = scores_np.shape
    s = torch.from_numpy(np.ascontiguousarray(scores_np, dtype=np.float32)).cuda()
    rl = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    res = []
    for with_ws in (True, False):
        idx = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
        val = torch.full((rows, k), float("nan"), dtype=torch.float32, device="cuda")
        ws = None
        if with_ws:
            ws = torch.empty(max(dsa.dsa_topk_workspace_size(rows, ld, k), 16), dtype=torch.uint8, device="cuda")
        dsa.dsa_topk_sorted(s, rl, k, idx, val, workspace=ws)
        res.append((idx.cpu().numpy(), val.cpu().numpy()))
    assert np.array_equal(res[0][0], res[1][0]), "the two selection paths disagree"
    assert np.array_equal(res[0][1], res[1][1])
    return res[0]


def _check(scores_np, lens, k, idx, val):
    for r in range(scores_np.shape[0]):
        n = int(lens[r])
        want_idx, want_val = orc.select_topk_sorted_row(scores_np[r, :n].astype(np.float64), k)
        assert np.array_equal(idx[r], want_idx), f"row {r} (len {n}): first diff at {np.argmax(idx[r] != want_idx)}"
        assert np.array_equal(val[r].astype(np.float64), want_val), f"row {r} values"


@pytest.mark.parametrize("seed", [0, 1])
def test_topk_sorted_random_rows_with_ties(dsa, seed):
    rng = np.random.default_rng(40 + seed)
    rows, ld, k = 64, 9000, 256
    scores = (rng.integers(-40, 400, size=(rows, ld)) / 8.0).astype(np.float32)
    lens = rng.integers(1, ld + 1, size=rows)
    lens[:4] = [k - 1, k, k + 1, ld]
    idx, val = _run_sorted(dsa, scores, lens, k)
    _check(scores, lens, k, idx, val)


def test_topk_sorted_special_rows_and_sizes(dsa):
    n = 5000
    rows = [np.zeros(n), np.arange(n, 0, -1.0), np.arange(n, dtype=np.float64)]
    z = np.zeros(n)
    z[1::2] = -0.0                                    # -0 == +0: ranked by position
    rows.append(z)
    r = np.full(n, 3.0)
    r[::7] = 5.0
    rows.append(r)
    r = np.full(n, -1.0)
    r[4000] = np.inf
    r[10] = -np.inf
    rows.append(r)
    scores = np.stack(rows).astype(np.float32)
    for k in (1, 5, 2048):
        lens = [n] * len(rows)
        idx, val = _run_sorted(dsa, scores, lens, k)
        _check(scores, lens, k, idx, val)
    # rows shorter than k keep everything, best first, then -1 / -inf
    short = np.random.default_rng(2).integers(-3, 4, size=(6, 64)).astype(np.float32)
    idx, val = _run_sorted(dsa, short, [1, 2, 10, 33, 63, 64], 64)
    _check(short, [1, 2, 10, 33, 63, 64], 64, idx, val)


def test_topk_sorted_long_rows_same_set_as_ascending_form(dsa):
    import torch
    rng = np.random.default_rng(11)
    ld, k = 131072, 2048
    scores = (rng.integers(0, 6000, size=(3, ld)) / 8.0).astype(np.float32)
    lens = [ld, 100000, 70001]
    idx, val = _run_sorted(dsa, scores, lens, k)
    _check(scores, lens, k, idx, val)
    s = torch.from_numpy(scores).cuda()
    rl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    asc = torch.empty(3, k, dtype=torch.int32, device="cuda")
    dsa.dsa_topk(s, rl, k, asc)
    assert np.array_equal(np.sort(idx, axis=1), asc.cpu().numpy())
