"""Parity at the full sizes of the five synthetic workloads, in the launch configuration the
benchmark times (dsa_prefill with its default 2048-row workspace, dsa_decode over whole
caches).  Sampled prefill rows are recomputed by the oracle one by one: indexer scores and
indices bit for bit, outputs and log-sum-exp within tolerance.  Every row's index set is checked
for structure (ascending, unique, in range, min(t+1, k) entries, -1 padding).  Decode batches are
checked in full, the decode indexer's scores bit for bit.  GPU only; each test takes seconds to
about a minute (the oracle's rows dominate)."""

import numpy as np
import pytest

from sparse_long_context_lightning_amd import inputs as inp

import dsa_testlib as tl

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(600)]

# Random rows per prefill workload on top of the deterministic ones (oracle cost grows with t).
N_RANDOM = {"c2_prefill_32k": 512, "c3_prefill_128k": 256, "c5_video_mix_prefill": 256}


def _run_prefill(dsa, name, period=None):
    import torch
    pi = inp.workload(name)
    print(f"[full-size] {name}: T={int(pi.cu_seqlens[-1])} k={pi.top_k}", flush=True)
    dev = tl.upload_prefill(pi)
    out, lse, idx = dsa.prefill(dev["q"], dev["k"], dev["v"], dev["q_idx"], dev["k_idx"], dev["w"],
                                pi.cu_seqlens, pi.top_k)
    torch.cuda.synchronize()
    row_lens = torch.cat([torch.arange(1, n + 1, dtype=torch.int32) for n in pi.seq_lens])
    tl.check_index_structure_device(idx, row_lens, pi.top_k)
    rows = tl.sample_rows(pi.cu_seqlens, pi.top_k, N_RANDOM[name], pi.meta["seed"], period)
    print(f"[full-size] {name}: oracle on {len(rows)} sampled rows", flush=True)
    want = tl.oracle_prefill_rows_lazy(pi, rows, keep_scores=True)
    # The indexer's scores of every sampled row (one-row windows: each score is one workgroup's
    # own dot products, so the window does not change it), bit for bit.
    ld = (max(int(x) for x in pi.seq_lens) + 3) // 4 * 4
    buf = torch.full((1, ld), float("nan"), dtype=torch.float32, device="cuda")
    for r, want_sc in zip(rows, want["scores"]):
        dsa.dsa_index_scores(dev["q_idx"], dev["k_idx"], dev["w"], pi.cu_seqlens, r, 1, buf)
        got = buf[0, :len(want_sc)].cpu().numpy()
        assert np.array_equal(got, want_sc), f"{name}: scores of row {r} differ"
    sel = torch.tensor(rows, dtype=torch.int64, device="cuda")
    tl.assert_idx_equal(idx[sel].cpu().numpy(), want["idx"], rows, f"{name} idx")
    tl.assert_attn_close(tl.bf16_tensor_to_f64(out[sel]), want["out"], f"{name} O")
    assert np.max(np.abs(lse[sel].cpu().numpy() - want["lse"])) <= tl.LSE_ABS
    assert np.all(np.abs(np.asarray(want["wsum"]) - 1.0) < 1e-12)


def _run_decode(dsa, name):
    import torch
    pi = inp.workload(name)
    print(f"[full-size] {name}: B={pi.q.shape[0]} S={pi.s_max} k={pi.top_k}", flush=True)
    dev = tl.upload_decode(pi)
    out, lse, idx = dsa.decode(dev["q"], dev["q_idx"], dev["w"], dev["k_cache"], dev["v_cache"],
                               dev["k_idx_cache"], dev["seq_lens"], pi.top_k)
    batch = pi.q.shape[0]
    want = tl.oracle_decode_rows_lazy(pi, range(batch))
    ld = (pi.s_max + 3) // 4 * 4
    scores = torch.full((batch, ld), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa_decode_index_scores(dev["q_idx"], dev["w"], dev["k_idx_cache"], dev["seq_lens"], pi.s_max, scores)
    got = scores.cpu().numpy()
    for b in range(batch):
        n = int(pi.seq_lens[b])
        assert np.array_equal(got[b, :n].astype(np.float64), want["scores"][b]), f"{name}: scores of sequence {b}"
    tl.assert_idx_equal(idx.cpu().numpy(), np.asarray(want["idx"]), what=f"{name} idx")
    tl.assert_attn_close(tl.bf16_tensor_to_f64(out), np.asarray(want["out"]), f"{name} O")
    assert np.max(np.abs(lse.cpu().numpy() - np.asarray(want["lse"]))) <= tl.LSE_ABS


def test_full_c2_prefill_32k(dsa):
    _run_prefill(dsa, "c2_prefill_32k")


def test_full_c3_prefill_128k(dsa):
    _run_prefill(dsa, "c3_prefill_128k")


def test_full_c4_decode_b32_128k(dsa):
    _run_decode(dsa, "c4_decode_b32_128k")


def test_full_c5_video_mix_prefill(dsa):
    _run_prefill(dsa, "c5_video_mix_prefill", period=288)


def test_full_c5_video_mix_decode(dsa):
    _run_decode(dsa, "c5_video_mix_decode")
