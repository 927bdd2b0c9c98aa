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
