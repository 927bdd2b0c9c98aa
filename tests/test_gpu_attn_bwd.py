"""Backward of the sparse GQA attention (dsa_sparse_gqa_attn_bwd) against the oracle's float64
gradients on the same bf16 inputs, through the C ABI.  GPU only.

Tolerance: the kernel rounds p and dz to bf16 as MFMA operands (relative 2^-9) and takes
D = <dO, O> from the bf16 forward output, with fp32 accumulation; each gradient entry is a sum
of such terms, so its error is a small multiple of 2^-9 times the sum of the absolute terms.
The checks use the error relative to the largest reference magnitude of each tensor
(max 1e-2) and to its mean magnitude (mean 5e-3)."""

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
    for b in range(len(lens)):
        for t in range(lens[b]):
            r = cu[b] + t
            if mode == "all":
                sel = np.arange(min(t + 1, k_sel))
            else:
                n = int(rng.integers(1, min(t + 1, k_sel) + 1))
                sel = np.sort(rng.choice(t + 1, size=n, replace=False))
            idx[r, :len(sel)] = sel
            if bad_entries and len(sel) < k_sel:
                idx[r, len(sel)] = t + 1 + int(rng.integers(0, 5))   # outside the prefix: ignored
    dout = inp.f32_to_bf16_bits(rng.standard_normal((total, hq, 128)).astype(np.float32))
    return pi, idx, dout


def _run(dsa, pi, idx, dout_bits):
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
    dsa.dsa_sparse_gqa_attn_bwd(dev["q"], dev["k"], dev["v"], out, lse, dout, idx_t, dev["cu"], dq, dk, dv)
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


@pytest.mark.parametrize("lens,hq,hkv,k_sel", [([300, 45, 700], 32, 4, 64), ([500], 16, 1, 100),
                                               ([90, 200], 4, 4, 33), ([257], 8, 2, 256)])
def test_attn_bwd_matches_oracle(dsa, lens, hq, hkv, k_sel):
    pi, idx, dout = _case(lens, hq, hkv, k_sel, seed=sum(lens) + hq, bad_entries=True)
    dq, dk, dv = _run(dsa, pi, idx, dout)
    want = orc.sparse_attention_grad(tl.f64(pi.q), tl.f64(pi.k), tl.f64(pi.v), idx, pi.cu_seqlens, tl.f64(dout))
    for name, g, w in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        _check(name, g, w)


def test_attn_bwd_all_positions_is_dense_causal_gqa_backward(dsa):
    import torch
    lens, hq, hkv = [160], 8, 2
    pi, idx, dout = _case(lens, hq, hkv, 160, seed=5, mode="all")
    dq, dk, dv = _run(dsa, pi, idx, dout)
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


def test_attn_bwd_positions_never_selected_get_zero(dsa):
    lens, hq, hkv, k_sel = [400], 8, 2, 16
    pi, idx, dout = _case(lens, hq, hkv, k_sel, seed=9)
    dq, dk, dv = _run(dsa, pi, idx, dout)
    used = np.zeros(400, dtype=bool)
    used[idx[idx >= 0]] = True
    assert np.all(dk[~used] == 0) and np.all(dv[~used] == 0)
    assert np.any(dk[used] != 0) and np.any(dv[used] != 0)
