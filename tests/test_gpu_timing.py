"""The library's launch timing and launch log on a fused prefill (GPU only): one entry per launch
name with the launch counts of the chunk schedule, results unchanged with timing on, nothing
recorded once it is off."""

import numpy as np
import pytest

from sparse_long_context_lightning_amd import inputs as inp

import dsa_testlib as tl

pytestmark = pytest.mark.gpu


def test_launch_timing_of_the_fused_prefill(dsa):
    import torch
    lens = [3000]
    pi = inp.prefill_inputs(lens, 64, 128, 32, 4, 128, 512, seed=5)
    dev = tl.upload_prefill(pi)

    def run():
        return dsa.prefill(dev["q"], dev["k"], dev["v"], dev["q_idx"], dev["k_idx"], dev["w"], pi.cu_seqlens,
                           pi.top_k)

    out0, lse0, idx0 = run()
    dsa.dsa_timing_enable(True)
    out1, lse1, idx1 = run()
    rec = dsa.dsa_timing_read()
    dsa.dsa_timing_enable(False)
    # two chunks of at most 2048 rows ([0, 2048), [2048, 3000)), both on the fused top-k path
    for name in ("indexer_sample", "topk_threshold", "indexer_emit", "topk_select", "indexer_rescore",
                 "topk_redo"):
        ms, n = rec[name]
        assert n == 2 and ms > 0, (name, rec[name])
    for name in ("query_union", "sparse_attn_union"):
        ms, n = rec[name]
        assert n == 1 and ms > 0, (name, rec[name])
    assert "indexer" not in rec and "topk" not in rec
    # the emitting indexer does the prefill's indexer work: the largest entry of the top-k side
    assert rec["indexer_emit"][0] > rec["topk_select"][0]
    assert torch.equal(idx0, idx1) and torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(lse0, lse1)
    # off: nothing more is recorded
    run()
    torch.cuda.synchronize()
    assert all(n == 0 and ms == 0.0 for ms, n in dsa.dsa_timing_read().values())
    want = tl.oracle_prefill_rows_lazy(pi, [2999, 2048, 600])
    tl.assert_idx_equal(idx1.cpu().numpy()[[2999, 2048, 600]], want["idx"], [2999, 2048, 600], "idx")
    assert np.isfinite(lse1.cpu().numpy()).all()


def test_launch_log_of_the_fused_prefill(dsa):
    """DSA_LOG=1: besides the call line, one stderr line per kernel launch, in launch order (a
    child process, since the variable is read once per process)."""
    import os
    import subprocess
    import sys
    code = (
        "import torch\n"
        "import sparse_long_context_lightning_amd as dsa\n"
        "from sparse_long_context_lightning_amd import inputs as inp\n"
        "pi = inp.prefill_inputs([1000], 64, 128, 32, 4, 128, 256, seed=9)\n"
        "dev = dsa.upload_prefill_inputs(pi)\n"
        "dsa.prefill(dev['q'], dev['k'], dev['v'], dev['q_idx'], dev['k_idx'], dev['w'], pi.cu_seqlens, pi.top_k)\n"
        "torch.cuda.synchronize()\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300,
                         env=dict(os.environ, DSA_LOG="1"))
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l.strip() for l in res.stderr.splitlines() if l.startswith("[dsa]")]
    assert any(l.startswith("[dsa] dsa_prefill(batch=1 total=1000") for l in lines), lines
    launches = [l.split("launch ", 1)[1] for l in lines if "launch " in l]
    # one chunk of all 1000 rows on the fused top-k path, then the attention with dedup
    assert launches == ["indexer_sample", "topk_threshold", "indexer_emit", "topk_select", "indexer_rescore",
                        "topk_redo", "query_union", "sparse_attn_union", "sparse_attn"], launches


def test_launch_timing_of_the_decode_step(dsa):
    """The decode step's launches by name: the decode indexer, the top-k (one entry for its
    threshold / collect / select), the split attention and its combine — one each per step."""
    import torch
    seq = [3000, 1, 700, 2049, 2999]
    di = inp.decode_inputs(len(seq), 3000, seq, 64, 128, 32, 4, 128, 512, seed=21)
    dev = tl.upload_decode(di)

    def run():
        return dsa.decode(dev["q"], dev["q_idx"], dev["w"], dev["k_cache"], dev["v_cache"], dev["k_idx_cache"],
                          dev["seq_lens"], 512, max_seq_len=max(seq))

    out0, lse0, idx0 = run()
    dsa.dsa_timing_enable(True)
    out1, lse1, idx1 = run()
    out2, lse2, idx2 = run()
    rec = dsa.dsa_timing_read()
    dsa.dsa_timing_enable(False)
    assert set(rec) >= {"indexer_decode", "topk", "sparse_attn_decode", "attn_combine"}, rec
    for name in ("indexer_decode", "topk", "sparse_attn_decode", "attn_combine"):
        ms, n = rec[name]
        assert n == 2 and ms > 0, (name, rec[name])
    for o, l, i in ((out1, lse1, idx1), (out2, lse2, idx2)):
        assert torch.equal(i, idx0) and torch.equal(o.view(torch.int16), out0.view(torch.int16))
        assert torch.equal(l, lse0)
