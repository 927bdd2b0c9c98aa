"""The measurement probes run, report their work, and leave their sink untouched.  GPU only."""

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
