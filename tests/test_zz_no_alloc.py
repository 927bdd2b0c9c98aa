"""dsa_decode_noalloc (the decode step on the library's static per-device scratch) against
dsa_decode with a caller workspace: the same kernels, so outputs must be equal bit for bit.  Two
calls in a row on the same scratch, the second smaller than the first; a step too large for the
scratch is refused before anything runs.  Called through the C ABI with ctypes.  GPU only.  Named
to be collected last (it shares the device's one scratch array with nothing else, and must pass
after every other test as well as alone)."""

import ctypes
import math

import numpy as np
import pytest

from sparse_long_context_lightning_amd import inputs as inp

import dsa_testlib as tl

pytestmark = pytest.mark.gpu


def _noalloc(dsa, dev, seq_lens, max_len, top_k):
    import torch
    lib = dsa.load()
    batch, hq, d = dev["q"].shape
    s_max, hkv = dev["k_cache"].shape[1], dev["k_cache"].shape[2]
    h_idx, d_idx = dev["q_idx"].shape[1], dev["q_idx"].shape[2]
    out = torch.full_like(dev["q"], float("nan"))
    lse = torch.full((batch, hq), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((batch, top_k), -99, dtype=torch.int32, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = lib.dsa_decode_noalloc(p(dev["q"]), p(dev["q_idx"]), p(dev["w"]), p(dev["k_cache"]), p(dev["v_cache"]), p(dev["k_idx_cache"]),
            p(seq_lens), ctypes.c_int(batch), ctypes.c_int(s_max), ctypes.c_int(max_len), ctypes.c_int(hq),
            ctypes.c_int(hkv), ctypes.c_int(d), ctypes.c_int(h_idx), ctypes.c_int(d_idx), ctypes.c_int(top_k),
            ctypes.c_float(1.0 / math.sqrt(d)), p(out), p(lse), p(idx),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, out, lse, idx


@pytest.mark.parametrize("first,second", [
    # (batch, s_max, seq_lens, top_k): a larger step, then a smaller one on the same scratch
    ((8, 65536, [65536, 1, 40000, 2049, 2048, 65535, 777, 30000], 2048), (3, 5000, [5000, 129, 1], 256)),
    ((32, 131072, None, 2048), (4, 131072, [131072, 131071, 2048, 1], 2048)),
])
def test_noalloc_decode_equals_decode_twice(dsa, first, second):
    import torch
    for seed, (batch, s_max, seq, k) in enumerate((first, second)):
        seq = [s_max] * batch if seq is None else seq
        print(f"[no-alloc] batch {batch} s_max {s_max} k {k}", flush=True)
        di = inp.decode_inputs(batch, s_max, seq, 64, 128, 32, 4, 128, k, seed=600 + seed)
        dev = tl.upload_decode(di)
        st, out, lse, idx = _noalloc(dsa, dev, dev["seq_lens"], max(seq), k)
        assert st == dsa.DSA_OK, dsa.dsa_last_error()
        ref_out, ref_lse, ref_idx = dsa.decode(dev["q"], dev["q_idx"], dev["w"], dev["k_cache"], dev["v_cache"],
                                               dev["k_idx_cache"], dev["seq_lens"], k, max_seq_len=max(seq))
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx)
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        assert torch.equal(lse, ref_lse)
        if batch <= 8:   # and against the oracle on the small steps
            want = tl.oracle_decode_rows_lazy(di, range(batch))
            tl.assert_idx_equal(idx.cpu().numpy(), np.asarray(want["idx"]), what="no-alloc decode idx")
            tl.assert_attn_close(tl.bf16_tensor_to_f64(out), np.asarray(want["out"]), "no-alloc decode O")
        del dev


def test_noalloc_decode_refuses_a_step_beyond_its_scratch(dsa):
    import torch
    lib = dsa.load()
    # 64 sequences of 262144 positions need 64 MiB of scores alone: refused on the host, nothing runs
    need = dsa.dsa_decode_workspace_size(64, 262144, 32, 4, 128, 64, 128, 2048)
    assert need > (32 << 20)
    fake = ctypes.c_void_p(1 << 20)
    st = lib.dsa_decode_noalloc(*([fake] * 7), 64, 262144, 262144, 32, 4, 128, 64, 128, 2048, 0.1, fake, None, fake,
                                None)
    assert st == dsa.DSA_ERR_WORKSPACE
    assert "static scratch" in dsa.dsa_last_error()
    torch.cuda.synchronize()
