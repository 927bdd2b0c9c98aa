"""The measurement probes (libdsa_probes.so) run, report their work, and leave their sink
untouched.  GPU only."""

import pytest

pytestmark = pytest.mark.gpu


def test_probes_run_and_store_nothing(dsa):
    import torch
    sink = torch.zeros(4096, dtype=torch.float32, device="cuda")
    flops16 = dsa.dsa_probe_mfma_bf16(16, 512, 100, sink)
    flops32 = dsa.dsa_probe_mfma_bf16(32, 512, 100, sink)
    assert flops16 == 512 * 4 * 100 * 8 * 16 * 16 * 32 * 2
    assert flops32 == 512 * 4 * 100 * 4 * 32 * 32 * 16 * 2
    buf = torch.arange(1 << 20, dtype=torch.int32, device="cuda")
    dsa.dsa_probe_stream_read(buf, 4096, sink)
    dsa.dsa_probe_stream_read(buf[:1000], 7, sink)  # ragged: fewer pieces than threads
    torch.cuda.synchronize()
    assert torch.count_nonzero(sink).item() == 0


@pytest.mark.parametrize("depth,group_fastest,nsplit,whole", [(1, False, 1, False), (2, True, 4, True),
                                                              (4, False, 2, True), (2, False, 3, False)])
def test_gather_probe_runs_and_stores_nothing(dsa, depth, group_fastest, nsplit, whole):
    import torch
    n_pos, hkv, rows, k_sel = 5000, 4, 300, 100   # ragged: 100 entries = 3 chunks + 4
    k = torch.randn(n_pos, hkv, 128, device="cuda").to(torch.bfloat16)
    v = torch.randn(n_pos, hkv, 128, device="cuda").to(torch.bfloat16)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    # positions past n_pos and negative entries are both legal (they read row 0 / nothing)
    idx = torch.randint(-10, n_pos + 10, (rows, k_sel), generator=g, device="cuda", dtype=torch.int32)
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    dsa.dsa_probe_gather(k, v, idx, sink, nsplit=nsplit, group_fastest=group_fastest, depth=depth, whole_rows=whole)
    # decode layout: row r reads positions r * row_stride + p
    idx_d = torch.randint(0, 16, (rows, k_sel), generator=g, device="cuda", dtype=torch.int32)
    dsa.dsa_probe_gather(k, v, idx_d, sink, nsplit=nsplit, row_stride=16, group_fastest=group_fastest, depth=depth,
                         whole_rows=whole)
    torch.cuda.synchronize()
    assert torch.count_nonzero(sink).item() == 0


@pytest.mark.parametrize("floats_per_row", [16, 64])
def test_atomic_probe_adds_exactly_its_count(dsa, floats_per_row):
    import torch
    buf = torch.zeros(5000, 128, dtype=torch.float32, device="cuda")
    adds = dsa.dsa_probe_atomic_add(buf, floats_per_row, 96, 7)
    assert adds == 96 * 4 * 7 * 64
    torch.cuda.synchronize()
    # each float receives a small integer count: the sum is exact
    assert int(buf.double().sum().item()) == adds
