"""The fused entry points captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library enqueues kernels only (no allocation, no memset, no synchronisation), so a captured
dsa_decode / dsa_prefill replays the same work.  Each test replays the graph several times, with
new input values copied into the captured buffers and eager calls of the same entry point (on
other buffers) and synchronisations in between, and checks every replay bit for bit against an
eager call on the same values.  GPU only."""

import numpy as np
import pytest

from sparse_long_context_lightning_amd import inputs as inp

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # first call outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_decode_graph_replays_match_eager(dsa):
    torch = _torch()
    seq = [3000, 1, 700, 512, 513, 2999, 1234, 64]
    s_max, k = 3000, 512
    dis = [inp.decode_inputs(len(seq), s_max, seq, 64, 128, 32, 4, 128, k, seed=s) for s in (901, 902, 903)]
    devs = [dsa.upload_decode_inputs(di) for di in dis]
    batch, hq, d = dis[0].q.shape
    nbytes = dsa.dsa_decode_workspace_size(batch, s_max, hq, 4, d, 64, 128, k)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    cap = {name: t.clone() for name, t in devs[0].items()}
    out = torch.empty_like(cap["q"])
    lse = torch.empty(batch, hq, dtype=torch.float32, device="cuda")
    idx = torch.empty(batch, k, dtype=torch.int32, device="cuda")

    def step():
        dsa.dsa_decode(cap["q"], cap["q_idx"], cap["w"], cap["k_cache"], cap["v_cache"], cap["k_idx_cache"],
                       cap["seq_lens"], max(seq), k, out, lse, idx, ws)

    g = _capture(torch, step)
    for rep in range(6):
        dev = devs[rep % 3]
        for name, t in dev.items():
            cap[name].copy_(t)
        g.replay()
        torch.cuda.synchronize()
        got = (out.clone(), lse.clone(), idx.clone())
        # eager work of the same entry point between replays (own buffers)
        e_out, e_lse, e_idx = dsa.decode(dev["q"], dev["q_idx"], dev["w"], dev["k_cache"], dev["v_cache"],
                                         dev["k_idx_cache"], dev["seq_lens"], k, max_seq_len=max(seq))
        torch.cuda.synchronize()
        assert torch.equal(got[2], e_idx), f"replay {rep}: idx"
        assert torch.equal(got[0], e_out), f"replay {rep}: out"
        assert torch.equal(got[1], e_lse), f"replay {rep}: lse"


@pytest.mark.parametrize("lens", [[2600], [700, 64, 1500]])
def test_prefill_graph_replays_match_eager(dsa, lens):
    """dsa_prefill with dedup (the default workspace) captured whole, chunk loop included."""
    torch = _torch()
    k = 256
    pis = [inp.prefill_inputs(lens, 64, 128, 32, 4, 128, k, seed=s, structure="blocks16") for s in (911, 912)]
    devs = [dsa.upload_prefill_inputs(pi) for pi in pis]
    cu = pis[0].cu_seqlens
    total = sum(lens)
    max_len = max(lens)
    nbytes = dsa.dsa_prefill_workspace_size(len(lens), total, max_len, 32, 4, 128, 64, 128, k)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    cap = {name: t.clone() for name, t in devs[0].items()}
    out = torch.empty_like(cap["q"])
    lse = torch.empty(total, 32, dtype=torch.float32, device="cuda")
    idx = torch.empty(total, k, dtype=torch.int32, device="cuda")

    def step():
        dsa.dsa_prefill(cap["q"], cap["k"], cap["v"], cap["q_idx"], cap["k_idx"], cap["w"], cap["cu"], cu, max_len,
                        k, out, lse, idx, ws)

    g = _capture(torch, step)
    for rep in range(4):
        dev = devs[rep % 2]
        for name, t in dev.items():
            cap[name].copy_(t)
        g.replay()
        torch.cuda.synchronize()
        got = (out.clone(), lse.clone(), idx.clone())
        e_out, e_lse, e_idx = dsa.prefill(dev["q"], dev["k"], dev["v"], dev["q_idx"], dev["k_idx"], dev["w"], cu, k)
        torch.cuda.synchronize()
        assert torch.equal(got[2], e_idx), f"replay {rep}: idx"
        assert torch.equal(got[0], e_out), f"replay {rep}: out"
        assert torch.equal(got[1], e_lse), f"replay {rep}: lse"
    # the two input sets really differ
    assert not np.array_equal(pis[0].q_idx, pis[1].q_idx)
