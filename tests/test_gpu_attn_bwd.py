"""Backward of the sparse GQA attention (dsa_sparse_gqa_attn_bwd, and dsa_sparse_gqa_attn_bwd_dedup,
which sums dk / dv over the merged sets of blocks of adjacent rows) against the oracle's float64
gradients on the same bf16 inputs, through the C ABI.  GPU only.

Tolerance: the kernel rounds p and dz to bf16 as MFMA operands (relative 2^-9) and takes
D = <dO, O> from the bf16 forward output, with fp32 accumulation; each gradient entry is a sum
of such terms, so its error is a small multiple of 2^-9 times the sum of the absolute terms.
The checks use the error relative to the largest reference magnitude of each tensor
(max 1e-2) and to its mean magnitude (mean 5e-3)."""

from collections import defaultdict

import numpy as np
import pytest

from oracle import dsa_oracle as orc
from sparse_long_context_lightning_amd import inputs as inp

import dsa_testlib as tl

pytestmark = pytest.mark.gpu

REL_MAX = 1e-2
REL_MEAN = 5e-3


def _case(lens, hq, hkv, k_sel, seed, mode="random", bad_entries=False):
    pi = inp.prefill_inputs(lens, 4, 64, hq, hkv, 128, k_sel, seed=seed)
    rng = np.random.default_rng(seed + 1)
    total = sum(lens)
    idx = np.full((total, k_sel), -1, dtype=np.int32)
    cu = pi.cu_seqlens
    anchor = {}
    for b in range(len(lens)):
        for t in range(lens[b]):
            r = cu[b] + t
            if mode == "all":
                sel = np.arange(min(t + 1, k_sel))
            elif mode == "overlap":
                # adjacent rows share most positions: a set drawn once per 32 rows from the
                # positions all of them can see, the row's own latest positions, a few of its own
                t0 = t - t % 32
                if (b, t0) not in anchor:
                    anchor[(b, t0)] = rng.choice(t0 + 1, size=min(t0 + 1, k_sel), replace=False)
                own = np.concatenate([np.arange(max(0, t - 7), t + 1), rng.choice(t + 1, size=min(t + 1, 3))])
                sel = np.unique(np.concatenate([anchor[(b, t0)][:max(0, k_sel - 11)], own]))[:k_sel]
            elif mode == "iid":
                sel = np.sort(rng.choice(t + 1, size=min(t + 1, k_sel), replace=False))
            else:
                n = int(rng.integers(1, min(t + 1, k_sel) + 1))
                sel = np.sort(rng.choice(t + 1, size=n, replace=False))
            idx[r, :len(sel)] = sel
            if bad_entries and len(sel) < k_sel:
                idx[r, len(sel)] = t + 1 + int(rng.integers(0, 5))   # outside the prefix: ignored
    dout = inp.f32_to_bf16_bits(rng.standard_normal((total, hq, 128)).astype(np.float32))
    return pi, idx, dout


def _run(dsa, pi, idx, dout_bits, dedup=False):
    import torch
    dev = tl.upload_prefill(pi)
    idx_t = torch.from_numpy(idx).cuda()
    total, hq, d = dev["q"].shape
    hkv = dev["k"].shape[1]
    out = torch.empty_like(dev["q"])
    lse = torch.empty(total, hq, dtype=torch.float32, device="cuda")
    dsa.dsa_sparse_gqa_attn(dev["q"], dev["k"], dev["v"], idx_t, dev["cu"], out, lse)
    dout = torch.from_numpy(dout_bits.view(np.int16)).cuda().view(torch.bfloat16)
    dq = torch.full((total, hq, d), float("nan"), dtype=torch.float32, device="cuda")
    dk = torch.full((total, hkv, d), float("nan"), dtype=torch.float32, device="cuda")
    dv = torch.full((total, hkv, d), float("nan"), dtype=torch.float32, device="cuda")
    bwd = dsa.dsa_sparse_gqa_attn_bwd_dedup if dedup else dsa.dsa_sparse_gqa_attn_bwd
    bwd(dev["q"], dev["k"], dev["v"], out, lse, dout, idx_t, dev["cu"], dq, dk, dv)
    torch.cuda.synchronize()
    return dq.cpu().numpy().astype(np.float64), dk.cpu().numpy().astype(np.float64), dv.cpu().numpy().astype(np.float64)


def _check(name, got, want):
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - want)
    scale_max = max(np.abs(want).max(), 1e-30)
    scale_mean = max(np.abs(want).mean(), 1e-30)
    print(f"{name}: max err / max |ref| = {err.max() / scale_max:.2e}, mean err / mean |ref| = {err.mean() / scale_mean:.2e}")
    assert err.max() <= REL_MAX * scale_max, f"{name}: max err {err.max():.3e} vs max |ref| {scale_max:.3e}"
    assert err.mean() <= REL_MEAN * scale_mean, f"{name}: mean err {err.mean():.3e} vs mean |ref| {scale_mean:.3e}"


CASES = [([300, 45, 700], 32, 4, 64), ([500], 16, 1, 100), ([90, 200], 4, 4, 33), ([257], 8, 2, 256)]


@pytest.mark.parametrize("dedup", [False, True])
@pytest.mark.parametrize("lens,hq,hkv,k_sel", CASES)
def test_attn_bwd_matches_oracle(dsa, lens, hq, hkv, k_sel, dedup):
    pi, idx, dout = _case(lens, hq, hkv, k_sel, seed=sum(lens) + hq, bad_entries=True)
    dq, dk, dv = _run(dsa, pi, idx, dout, dedup=dedup)
    want = orc.sparse_attention_grad(tl.f64(pi.q), tl.f64(pi.k), tl.f64(pi.v), idx, pi.cu_seqlens, tl.f64(dout))
    for name, g, w in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        _check(name, g, w)


# Merged-set backward: sets that overlap heavily between adjacent rows (the case it is for), blocks
# of 32 rows that straddle sequence starts, a last block of a few rows, group sizes 4, 8 and 16.
@pytest.mark.parametrize("lens,hq,hkv,k_sel", [([600, 37, 300], 32, 4, 64), ([161, 33, 70, 5], 8, 2, 40),
                                               ([400], 16, 1, 96), ([64, 64], 16, 2, 128)])
def test_attn_bwd_dedup_overlapping_sets_match_oracle(dsa, lens, hq, hkv, k_sel):
    pi, idx, dout = _case(lens, hq, hkv, k_sel, seed=3 * sum(lens) + hq, mode="overlap", bad_entries=True)
    dq, dk, dv = _run(dsa, pi, idx, dout, dedup=True)
    want = orc.sparse_attention_grad(tl.f64(pi.q), tl.f64(pi.k), tl.f64(pi.v), idx, pi.cu_seqlens, tl.f64(dout))
    for name, g, w in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        _check(name, g, w)


def test_attn_bwd_dedup_repeated_entries_count_per_occurrence(dsa):
    """A block in which a row lists a position twice is done per row, where each entry counts:
    the oracle adds that position's contribution twice."""
    lens, hq, hkv, k_sel = [300], 32, 4, 48
    pi, idx, dout = _case(lens, hq, hkv, k_sel, seed=21, mode="overlap")
    for r in (40, 41, 200):   # rows in blocks 1 and 6: repeat their first entry in a spare slot
        n = int((idx[r] >= 0).sum())
        if n < k_sel:
            idx[r, n] = idx[r, 0]
        else:
            idx[r, -1] = idx[r, 0]
    dq, dk, dv = _run(dsa, pi, idx, dout, dedup=True)
    want = orc.sparse_attention_grad(tl.f64(pi.q), tl.f64(pi.k), tl.f64(pi.v), idx, pi.cu_seqlens, tl.f64(dout))
    for name, g, w in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        _check(name, g, w)


def _oracle_rows(pi, idx, dout, rows):
    """dq of `rows` and their summed dk / dv contributions per packed position, from the oracle's
    per-row gradient with each row's in-prefix entries taken as a small key list (entry j of the
    list is key j), so that long prefixes need not be widened."""
    cu = [int(x) for x in pi.cu_seqlens]
    scale = orc.default_softmax_scale(pi.q.shape[2])
    dq, dk, dv = {}, defaultdict(float), defaultdict(float)
    for i, r in enumerate(rows):
        if i % 50 == 0:
            print(f"oracle row gradients: {i} of {len(rows)}", flush=True)
        b = max(i for i in range(len(cu) - 1) if cu[i] <= r)
        o, t = cu[b], r - cu[b]
        ent = np.asarray([int(p) for p in idx[r] if 0 <= int(p) <= t], dtype=np.int64)
        kk, vv = tl.f64(pi.k[o + ent]), tl.f64(pi.v[o + ent])
        gq, gk, gv = orc.sparse_gqa_attention_row_grad(tl.f64(pi.q[r]), kk, vv, np.arange(len(ent)), scale,
                                                       tl.f64(dout[r]))
        dq[r] = gq
        for j, p in enumerate(ent):
            dk[o + int(p)] = dk[o + int(p)] + gk[j]
            dv[o + int(p)] = dv[o + int(p)] + gv[j]
    return dq, dk, dv


def _check_sampled(pi, idx, dout, got, sample_rows, sample_keys):
    """Oracle values of dq on sample_rows and of dk / dv on sample_keys (every row that selected
    one of them taken into account)."""
    dq, dk, dv = got
    want_dq, _, _ = _oracle_rows(pi, idx, dout, sample_rows)
    rows_of_keys = np.nonzero(np.isin(idx, np.asarray(sample_keys)).any(axis=1))[0]
    _, want_dk, want_dv = _oracle_rows(pi, idx, dout, rows_of_keys)
    _check("dq (sampled rows)", dq[sample_rows], np.stack([want_dq[r] for r in sample_rows]))
    zero = np.zeros(dk.shape[1:])
    _check("dk (sampled keys)", dk[sample_keys], np.stack([want_dk.get(s, zero) for s in sample_keys]))
    _check("dv (sampled keys)", dv[sample_keys], np.stack([want_dv.get(s, zero) for s in sample_keys]))


def test_attn_bwd_dedup_past_one_bitmap_window(dsa):
    """A 33000-row sequence: the merged sets of its last blocks span more positions than one pass of
    the 32-bit-per-position builder covers (32768), so they are built in two windows."""
    lens, hq, hkv, k_sel = [33000], 4, 1, 32
    pi, idx, dout = _case(lens, hq, hkv, k_sel, seed=33, mode="overlap")
    got = _run(dsa, pi, idx, dout, dedup=True)
    rows = [0, 5, 31, 32, 1000, 32767, 32768, 32800, 32990, 32999]
    keys = [0, 17, 32500, 32767, 32768, 32790, 32995, 32999]
    _check_sampled(pi, idx, dout, got, rows, keys)


def test_attn_bwd_dedup_full_size_iid_sets(dsa):
    """The 32K shape (32 query heads, 4 KV heads, k = 2048) with i.i.d. index sets (the least
    overlap between adjacent rows): sampled rows and keys against the oracle, and the whole
    result against the per-row backward."""
    lens, hq, hkv, k_sel = [32768], 32, 4, 2048
    pi, idx, dout = _case(lens, hq, hkv, k_sel, seed=77, mode="iid")
    print("index sets drawn", flush=True)
    got = _run(dsa, pi, idx, dout, dedup=True)
    rows = [0, 2047, 2048, 9000, 20001, 32735, 32767]
    keys = [32300, 32700, 32767]   # ~30 rows select one of them: each costs a full oracle row (0.3 s)
    _check_sampled(pi, idx, dout, got, rows, keys)
    per_row = _run(dsa, pi, idx, dout, dedup=False)
    for name, g, w in zip(("dq", "dk", "dv"), got, per_row):
        _check(name + " (dedup vs per row)", g, w)


@pytest.mark.parametrize("dedup", [False, True])
def test_attn_bwd_all_positions_is_dense_causal_gqa_backward(dsa, dedup):
    import torch
    lens, hq, hkv = [160], 8, 2
    pi, idx, dout = _case(lens, hq, hkv, 160, seed=5, mode="all")
    dq, dk, dv = _run(dsa, pi, idx, dout, dedup=dedup)
    q = torch.from_numpy(tl.f64(pi.q)).permute(1, 0, 2).unsqueeze(0).requires_grad_(True)
    k = torch.from_numpy(tl.f64(pi.k)).permute(1, 0, 2).unsqueeze(0).requires_grad_(True)
    v = torch.from_numpy(tl.f64(pi.v)).permute(1, 0, 2).unsqueeze(0).requires_grad_(True)
    o = torch.nn.functional.scaled_dot_product_attention(q, k.repeat_interleave(hq // hkv, dim=1),
                                                         v.repeat_interleave(hq // hkv, dim=1), is_causal=True,
                                                         scale=orc.default_softmax_scale(128))
    o.backward(torch.from_numpy(tl.f64(dout)).permute(1, 0, 2).unsqueeze(0))
    _check("dq", dq, q.grad[0].permute(1, 0, 2).numpy())
    _check("dk", dk, k.grad[0].permute(1, 0, 2).numpy())
    _check("dv", dv, v.grad[0].permute(1, 0, 2).numpy())


@pytest.mark.parametrize("dedup", [False, True])
def test_attn_bwd_positions_never_selected_get_zero(dsa, dedup):
    lens, hq, hkv, k_sel = [400], 8, 2, 16
    pi, idx, dout = _case(lens, hq, hkv, k_sel, seed=9)
    dq, dk, dv = _run(dsa, pi, idx, dout, dedup=dedup)
    used = np.zeros(400, dtype=bool)
    used[idx[idx >= 0]] = True
    assert np.all(dk[~used] == 0) and np.all(dv[~used] == 0)
    assert np.any(dk[used] != 0) and np.any(dv[used] != 0)
