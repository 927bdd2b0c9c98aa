"""ctypes binding of libdsa.so (the C ABI in include/dsa.h).

Argument marshalling only: every step of the path runs in the HIP library.  Tensors are torch
device tensors; the call is enqueued on torch's current stream.  There is no fallback: if
the library is missing or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsa.so")
PROBES_LIB_PATH = os.path.join(_PKG, "libdsa_probes.so")

DSA_OK = 0
DSA_ERR_INVALID_ARG = 1
DSA_ERR_UNSUPPORTED = 2
DSA_ERR_WORKSPACE = 3
DSA_ERR_HIP = 4
DSA_MAX_TOP_K = 2048

EXPORTED = (
    "dsa_abi_version", "dsa_status_string", "dsa_last_error", "dsa_index_scores", "dsa_decode_index_scores",
    "dsa_topk_workspace_size", "dsa_topk", "dsa_topk_sorted", "dsa_sparse_gqa_attn", "dsa_sparse_gqa_attn_bwd",
    "dsa_prefill_workspace_size", "dsa_prefill", "dsa_decode_workspace_size", "dsa_decode", "dsa_attn_head_mean",
    "dsa_indexer_kl", "dsa_index_scores_bwd", "dsa_query_union_size", "dsa_query_union",
    "dsa_sparse_gqa_attn_union", "dsa_sparse_gqa_attn_dedup_workspace_size", "dsa_sparse_gqa_attn_dedup",
    "dsa_decode_noalloc", "dsa_sparse_gqa_attn_decode_workspace_size", "dsa_sparse_gqa_attn_decode",
    "dsa_sparse_gqa_attn_bwd_dedup_workspace_size", "dsa_sparse_gqa_attn_bwd_dedup",
    "dsa_timing_enable", "dsa_timing_count", "dsa_timing_entry",
)
# The measurement probes (include/dsa_probes.h), a separate library used by the benchmark.
PROBES_EXPORTED = ("dsa_probe_last_error", "dsa_probe_mfma_bf16", "dsa_probe_stream_read", "dsa_probe_gather",
                   "dsa_probe_atomic_add")


class DsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t


def load():
    """Load libdsa.so (built in-tree by build.py); raises if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sparse_long_context_lightning_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "dsa_abi_version": ([], _I),
        "dsa_status_string": ([_I], ctypes.c_char_p),
        "dsa_last_error": ([], ctypes.c_char_p),
        "dsa_timing_enable": ([_I], _I),
        "dsa_timing_count": ([ctypes.POINTER(_I)], _I),
        "dsa_timing_entry": ([_I, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                              ctypes.POINTER(_I64)], _I),
        "dsa_index_scores": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _I64, _P], _I),
        "dsa_decode_index_scores": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _I64, _P], _I),
        "dsa_topk_workspace_size": ([_I, _I64, _I, ctypes.POINTER(_SZ)], _I),
        "dsa_topk": ([_P, _I64, _I, _P, _I, _P, _P, _P, _SZ, _P], _I),
        "dsa_topk_sorted": ([_P, _I64, _I, _P, _I, _P, _P, _P, _SZ, _P], _I),
        "dsa_attn_head_mean": ([_P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P, _I64, _P, _P], _I),
        "dsa_indexer_kl": ([_P, _P, _I64, _I, _P, _P, _P, _P], _I),
        "dsa_index_scores_bwd": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _I64, _P, _P, _P, _P], _I),
        "dsa_sparse_gqa_attn": ([_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _F, _P, _P, _P], _I),
        "dsa_sparse_gqa_attn_bwd": ([_P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P],
                                    _I),
        "dsa_sparse_gqa_attn_bwd_dedup_workspace_size": ([_I, _I, _I, _I, ctypes.POINTER(_SZ)], _I),
        "dsa_sparse_gqa_attn_bwd_dedup": ([_P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _F, _P, _P, _P,
                                           _P, _SZ, _P], _I),
        "dsa_query_union_size": ([_I, _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I)], _I),
        "dsa_query_union": ([_P, _I, _P, _I, _I, _I, _I, _P, _P, _P, _P], _I),
        "dsa_sparse_gqa_attn_union": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P], _I),
        "dsa_sparse_gqa_attn_dedup_workspace_size": ([_I, _I, _I, _I, ctypes.POINTER(_SZ)], _I),
        "dsa_sparse_gqa_attn_dedup": ([_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _F, _P, _P, _P, _SZ, _P], _I),
        "dsa_prefill_workspace_size": ([_I, _I, _I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(_SZ)], _I),
        "dsa_prefill": ([_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P,
                         _SZ, _P], _I),
        "dsa_decode_workspace_size": ([_I, _I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(_SZ)], _I),
        "dsa_decode": ([_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _SZ,
                        _P], _I),
        "dsa_sparse_gqa_attn_decode_workspace_size": ([_I, _I, _I, _I, ctypes.POINTER(_SZ)], _I),
        "dsa_sparse_gqa_attn_decode": ([_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _F, _P, _P, _P, _SZ, _P], _I),
        "dsa_decode_noalloc": ([_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P],
                               _I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


_probes = None


def load_probes():
    """Load libdsa_probes.so (the measurement probes, built beside libdsa.so); raises if absent."""
    global _probes
    if _probes is not None:
        return _probes
    if not os.path.exists(PROBES_LIB_PATH):
        raise RuntimeError(f"{PROBES_LIB_PATH} is missing: build it with `python -m sparse_long_context_lightning_amd.build`")
    lib = ctypes.CDLL(PROBES_LIB_PATH)
    sig = {
        "dsa_probe_last_error": ([], ctypes.c_char_p),
        "dsa_probe_mfma_bf16": ([_I, _I, _I, _P, ctypes.POINTER(ctypes.c_longlong), _P], _I),
        "dsa_probe_stream_read": ([_P, _SZ, _I, _P, _P], _I),
        "dsa_probe_gather": ([_P, _P, _I64, _I, _P, _I, _I, _I, _I64, _I, _I, _I, _P, _I64, _P], _I),
        "dsa_probe_atomic_add": ([_P, _I64, _I, _I, _I, ctypes.POINTER(ctypes.c_longlong), _P], _I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _probes = lib
    return lib


def _check_probe(status: int):
    if status != 0:
        raise DsaError(status, load_probes().dsa_probe_last_error().decode())


def _status_name(status: int) -> str:
    return {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED", 3: "DSA_ERR_WORKSPACE",
            4: "DSA_ERR_HIP"}.get(status, f"status {status}")


def _check(status: int):
    if status != DSA_OK:
        raise DsaError(status, load().dsa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _host_i32(x):
    arr = np.ascontiguousarray(np.asarray(x if not hasattr(x, "cpu") else x.cpu().numpy(), dtype=np.int32))
    return arr, arr.ctypes.data_as(ctypes.c_void_p)


# ----------------------------------------------------------------------------- raw entry points

def dsa_abi_version() -> int:
    return load().dsa_abi_version()


def dsa_status_string(status: int) -> str:
    return load().dsa_status_string(status).decode()


def dsa_last_error() -> str:
    return load().dsa_last_error().decode()


def dsa_timing_enable(on: bool):
    """Clear the launch-timing record and turn per-launch timing on or off."""
    _check(load().dsa_timing_enable(1 if on else 0))


def dsa_timing_read() -> dict:
    """Wait for the timed launches and return {name: (total_ms, launches)}."""
    lib = load()
    n = _I(0)
    _check(lib.dsa_timing_count(ctypes.byref(n)))
    out = {}
    for i in range(n.value):
        name = ctypes.c_char_p()
        ms = ctypes.c_double()
        cnt = _I64()
        _check(lib.dsa_timing_entry(i, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(cnt)))
        out[name.value.decode()] = (ms.value, int(cnt.value))
    return out


def dsa_index_scores(q_idx, k_idx, w, cu_seqlens_host, row_begin, row_count, scores, ld=None, stream=None):
    """Indexer scores of packed rows [row_begin, row_begin + row_count) into scores[row_count, ld]."""
    cu, cu_p = _host_i32(cu_seqlens_host)
    total, h_idx, d_idx = q_idx.shape
    ld = scores.shape[1] if ld is None else ld
    _check(load().dsa_index_scores(_ptr(q_idx), _ptr(k_idx), _ptr(w), cu_p, len(cu) - 1, total, h_idx, d_idx,
                                   row_begin, row_count, _ptr(scores), ld, _stream(stream)))


def dsa_decode_index_scores(q_idx, w, k_idx_cache, seq_lens, max_seq_len, scores, ld=None, stream=None):
    """Indexer scores of each sequence's new token against its cached keys into scores[batch, ld]
    (entries at positions >= seq_lens[b] untouched)."""
    batch, h_idx, d_idx = q_idx.shape
    s_max = k_idx_cache.shape[1]
    ld = scores.shape[1] if ld is None else ld
    _check(load().dsa_decode_index_scores(_ptr(q_idx), _ptr(w), _ptr(k_idx_cache), _ptr(seq_lens), batch, s_max,
                                          max_seq_len, h_idx, d_idx, _ptr(scores), ld, _stream(stream)))


def dsa_attn_head_mean(q, k, cu_seqlens_host, row_begin, row_count, probs, lse, softmax_scale=None, ld=None,
                       stream=None):
    """Head-mean causal attention distribution (warm-up target) of packed rows into probs[row_count, ld],
    and the dense per-head log-sum-exp into lse[row_count, hq]."""
    cu, cu_p = _host_i32(cu_seqlens_host)
    total, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    ld = probs.shape[1] if ld is None else ld
    _check(load().dsa_attn_head_mean(_ptr(q), _ptr(k), cu_p, len(cu) - 1, total, hq, hkv, d, scale, row_begin,
                                     row_count, _ptr(probs), ld, _ptr(lse), _stream(stream)))


def dsa_indexer_kl(scores, target, row_len, row_loss, grad, ld=None, stream=None):
    """Per-row KL(target || softmax(scores)) and its gradient r - p (grad may be scores itself)."""
    rows = scores.shape[0]
    ld = scores.shape[1] if ld is None else ld
    _check(load().dsa_indexer_kl(_ptr(scores), _ptr(target), ld, rows, _ptr(row_len), _ptr(row_loss), _ptr(grad),
                                 _stream(stream)))


def dsa_index_scores_bwd(q_idx, k_idx, w, cu_seqlens_host, row_begin, row_count, dscores, dq_idx, dw, dk_idx,
                         ld=None, stream=None):
    """Backward of dsa_index_scores for packed rows [row_begin, row_begin + row_count): dq_idx and dw of
    those rows are written, dk_idx is added to.  dscores[row_count, ld] is the gradient of their scores."""
    cu, cu_p = _host_i32(cu_seqlens_host)
    total, h_idx, d_idx = q_idx.shape
    ld = dscores.shape[1] if ld is None else ld
    _check(load().dsa_index_scores_bwd(_ptr(q_idx), _ptr(k_idx), _ptr(w), cu_p, len(cu) - 1, total, h_idx, d_idx,
                                       row_begin, row_count, _ptr(dscores), ld, _ptr(dq_idx), _ptr(dw),
                                       _ptr(dk_idx), _stream(stream)))


def dsa_topk_workspace_size(rows, ld, k) -> int:
    n = _SZ(0)
    _check(load().dsa_topk_workspace_size(rows, ld, k, ctypes.byref(n)))
    return n.value


def dsa_topk(scores, row_len, k, idx_out, values_out=None, workspace=None, ld=None, stream=None):
    """Per-row top-k of scores[rows, ld] with valid lengths row_len[rows] (int32, device)."""
    rows = scores.shape[0]
    ld = scores.shape[1] if ld is None else ld
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().dsa_topk(_ptr(scores), ld, rows, _ptr(row_len), k, _ptr(idx_out), _ptr(values_out),
                           _ptr(workspace), ws_bytes, _stream(stream)))


def dsa_topk_sorted(scores, row_len, k, idx_out, values_out=None, workspace=None, ld=None, stream=None):
    """dsa_topk in torch.topk(sorted=True) order: descending score, equal scores by position."""
    rows = scores.shape[0]
    ld = scores.shape[1] if ld is None else ld
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().dsa_topk_sorted(_ptr(scores), ld, rows, _ptr(row_len), k, _ptr(idx_out), _ptr(values_out),
                                  _ptr(workspace), ws_bytes, _stream(stream)))


def dsa_sparse_gqa_attn(q, k, v, idx, cu_seqlens, out, lse=None, softmax_scale=None, stream=None):
    """Sparse GQA attention of every packed row over idx[row, :] (device cu_seqlens)."""
    total, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    _check(load().dsa_sparse_gqa_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), idx.shape[1], _ptr(cu_seqlens),
                                      cu_seqlens.shape[0] - 1, total, hq, hkv, d, scale, _ptr(out), _ptr(lse),
                                      _stream(stream)))


def dsa_sparse_gqa_attn_decode_workspace_size(batch, hq, hkv, k_sel) -> int:
    n = _SZ(0)
    _check(load().dsa_sparse_gqa_attn_decode_workspace_size(batch, hq, hkv, k_sel, ctypes.byref(n)))
    return n.value


def dsa_sparse_gqa_attn_decode(q, k_cache, v_cache, idx, seq_lens, out, lse=None, softmax_scale=None, workspace=None,
                               stream=None):
    """Sparse GQA attention of each sequence's new token over idx[b, :] positions of its cache;
    allocates the workspace when none is given."""
    import torch
    batch, hq, d = q.shape
    s_max, hkv = k_cache.shape[1], k_cache.shape[2]
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    if workspace is None:
        nbytes = dsa_sparse_gqa_attn_decode_workspace_size(batch, hq, hkv, idx.shape[1])
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _check(load().dsa_sparse_gqa_attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(idx), idx.shape[1],
                                             _ptr(seq_lens), batch, s_max, hq, hkv, d, scale, _ptr(out), _ptr(lse),
                                             _ptr(workspace), workspace.numel() * workspace.element_size(),
                                             _stream(stream)))


def dsa_query_union_size(total_tokens, k_sel, block_rows=16):
    """(n_blocks, cap): blocks of block_rows (8 or 16) packed rows and the per-block entry capacity."""
    nb, cap = _I(0), _I(0)
    _check(load().dsa_query_union_size(total_tokens, k_sel, block_rows, ctypes.byref(nb), ctypes.byref(cap)))
    return nb.value, cap.value


def dsa_query_union(idx, cu_seqlens, counts, kv_rows, masks, block_rows=16, stream=None):
    """Merged index sets of blocks of block_rows adjacent packed rows: counts [n_blocks] int32, kv_rows
    [n_blocks, cap] int32 (ascending packed KV rows), masks [n_blocks, cap] int16 (bit j = row R b + j)."""
    total, k_sel = idx.shape
    _check(load().dsa_query_union(_ptr(idx), k_sel, _ptr(cu_seqlens), cu_seqlens.shape[0] - 1, total, block_rows,
                                  kv_rows.shape[1], _ptr(counts), _ptr(kv_rows), _ptr(masks), _stream(stream)))


def dsa_sparse_gqa_attn_union(q, k, v, counts, kv_rows, masks, out, lse=None, softmax_scale=None, block_rows=16,
                              stream=None):
    """Sparse GQA attention of every packed row from the merged sets of dsa_query_union."""
    total, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    _check(load().dsa_sparse_gqa_attn_union(_ptr(q), _ptr(k), _ptr(v), _ptr(counts), _ptr(kv_rows), _ptr(masks),
                                            block_rows, kv_rows.shape[1], total, hq, hkv, d, scale, _ptr(out),
                                            _ptr(lse), _stream(stream)))


def dsa_sparse_gqa_attn_dedup_workspace_size(total_tokens, k_sel, hq, hkv):
    n = _SZ(0)
    _check(load().dsa_sparse_gqa_attn_dedup_workspace_size(total_tokens, k_sel, hq, hkv, ctypes.byref(n)))
    return n.value


def dsa_sparse_gqa_attn_dedup(q, k, v, idx, cu_seqlens, out, lse=None, softmax_scale=None, workspace=None,
                              stream=None):
    """dsa_sparse_gqa_attn with adjacent-query dedup (merged sets of 8-row blocks); allocates the
    workspace when none is given."""
    import torch
    total, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    if workspace is None:
        nbytes = dsa_sparse_gqa_attn_dedup_workspace_size(total, idx.shape[1], hq, hkv)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _check(load().dsa_sparse_gqa_attn_dedup(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), idx.shape[1], _ptr(cu_seqlens),
                                            cu_seqlens.shape[0] - 1, total, hq, hkv, d, scale, _ptr(out), _ptr(lse),
                                            _ptr(workspace), workspace.numel() * workspace.element_size(),
                                            _stream(stream)))


def dsa_sparse_gqa_attn_bwd(q, k, v, out, lse, dout, idx, cu_seqlens, dq, dk, dv, softmax_scale=None, stream=None):
    """Backward of dsa_sparse_gqa_attn: dq written, dk / dv zeroed and accumulated (float32)."""
    total, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    _check(load().dsa_sparse_gqa_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(idx),
                                          idx.shape[1], _ptr(cu_seqlens), cu_seqlens.shape[0] - 1, total, hq, hkv, d,
                                          scale, _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream)))


def dsa_sparse_gqa_attn_bwd_dedup_workspace_size(total_tokens, k_sel, hq, hkv):
    n = _SZ(0)
    _check(load().dsa_sparse_gqa_attn_bwd_dedup_workspace_size(total_tokens, k_sel, hq, hkv, ctypes.byref(n)))
    return n.value


def dsa_sparse_gqa_attn_bwd_dedup(q, k, v, out, lse, dout, idx, cu_seqlens, dq, dk, dv, softmax_scale=None,
                                  workspace=None, stream=None):
    """dsa_sparse_gqa_attn_bwd with dk / dv summed over the merged sets of blocks of adjacent rows
    before they are added; allocates the workspace when none is given."""
    import torch
    total, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    if workspace is None:
        nbytes = dsa_sparse_gqa_attn_bwd_dedup_workspace_size(total, idx.shape[1], hq, hkv)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _check(load().dsa_sparse_gqa_attn_bwd_dedup(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                                                _ptr(idx), idx.shape[1], _ptr(cu_seqlens), cu_seqlens.shape[0] - 1,
                                                total, hq, hkv, d, scale, _ptr(dq), _ptr(dk), _ptr(dv),
                                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                                _stream(stream)))


def dsa_prefill_workspace_size(batch, total_tokens, max_seqlen, hq, hkv, head_dim, h_idx, d_idx, top_k) -> int:
    n = _SZ(0)
    _check(load().dsa_prefill_workspace_size(batch, total_tokens, max_seqlen, hq, hkv, head_dim, h_idx, d_idx,
                                             top_k, ctypes.byref(n)))
    return n.value


def dsa_prefill(q, k, v, q_idx, k_idx, w, cu_seqlens, cu_seqlens_host, max_seqlen, top_k, out, lse, idx_out,
                workspace, softmax_scale=None, stream=None):
    cu, cu_p = _host_i32(cu_seqlens_host)
    total, hq, d = q.shape
    hkv = k.shape[1]
    h_idx, d_idx = q_idx.shape[1], q_idx.shape[2]
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().dsa_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(cu_seqlens), cu_p,
                              len(cu) - 1, total, max_seqlen, hq, hkv, d, h_idx, d_idx, top_k, scale, _ptr(out),
                              _ptr(lse), _ptr(idx_out), _ptr(workspace), ws_bytes, _stream(stream)))


def dsa_decode_workspace_size(batch, s_max, hq, hkv, head_dim, h_idx, d_idx, top_k) -> int:
    n = _SZ(0)
    _check(load().dsa_decode_workspace_size(batch, s_max, hq, hkv, head_dim, h_idx, d_idx, top_k, ctypes.byref(n)))
    return n.value


def dsa_decode(q, q_idx, w, k_cache, v_cache, k_idx_cache, seq_lens, max_seq_len, top_k, out, lse, idx_out,
               workspace, softmax_scale=None, stream=None):
    batch, hq, d = q.shape
    s_max, hkv = k_cache.shape[1], k_cache.shape[2]
    h_idx, d_idx = q_idx.shape[1], q_idx.shape[2]
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().dsa_decode(_ptr(q), _ptr(q_idx), _ptr(w), _ptr(k_cache), _ptr(v_cache), _ptr(k_idx_cache),
                             _ptr(seq_lens), batch, s_max, max_seq_len, hq, hkv, d, h_idx, d_idx, top_k, scale,
                             _ptr(out), _ptr(lse), _ptr(idx_out), _ptr(workspace), ws_bytes, _stream(stream)))


# ----------------------------------------------------------------------------- allocating helpers

def prefill(q, k, v, q_idx, k_idx, w, cu_seqlens_host, top_k, softmax_scale=None, workspace=None, stream=None):
    """Allocate outputs and run dsa_prefill.  Returns (out, lse, idx)."""
    import torch
    dev = q.device
    cu = np.asarray(cu_seqlens_host, dtype=np.int32)
    total, hq, d = q.shape
    max_seqlen = int(np.max(np.diff(cu))) if len(cu) > 1 else 0
    cu_dev = torch.from_numpy(cu).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty(total, hq, dtype=torch.float32, device=dev)
    idx = torch.empty(total, top_k, dtype=torch.int32, device=dev)
    if workspace is None:
        nbytes = dsa_prefill_workspace_size(len(cu) - 1, total, max_seqlen, hq, k.shape[1], d, q_idx.shape[1],
                                            q_idx.shape[2], top_k)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    dsa_prefill(q, k, v, q_idx, k_idx, w, cu_dev, cu, max_seqlen, top_k, out, lse, idx, workspace, softmax_scale,
                stream)
    return out, lse, idx


def decode(q, q_idx, w, k_cache, v_cache, k_idx_cache, seq_lens, top_k, max_seq_len=None, softmax_scale=None,
           workspace=None, stream=None):
    """Allocate outputs and run dsa_decode.  Returns (out, lse, idx)."""
    import torch
    dev = q.device
    batch, hq, d = q.shape
    s_max = k_cache.shape[1]
    if max_seq_len is None:
        max_seq_len = s_max
    out = torch.empty_like(q)
    lse = torch.empty(batch, hq, dtype=torch.float32, device=dev)
    idx = torch.empty(batch, top_k, dtype=torch.int32, device=dev)
    if workspace is None:
        nbytes = dsa_decode_workspace_size(batch, s_max, hq, k_cache.shape[2], d, q_idx.shape[1], q_idx.shape[2],
                                           top_k)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    dsa_decode(q, q_idx, w, k_cache, v_cache, k_idx_cache, seq_lens, max_seq_len, top_k, out, lse, idx, workspace,
               softmax_scale, stream)
    return out, lse, idx


def to_device_bf16(bits: np.ndarray, device="cuda"):
    """Upload bf16 bit patterns (uint16 numpy) as a torch.bfloat16 device tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def upload_prefill_inputs(pi, device="cuda"):
    """Device tensors of a prefill workload (`inputs.PrefillInputs`): q, k, v, q_idx, k_idx as
    bf16, w as float32, cu (cu_seqlens) as int32."""
    import torch
    return dict(
        q=to_device_bf16(pi.q, device), k=to_device_bf16(pi.k, device), v=to_device_bf16(pi.v, device),
        q_idx=to_device_bf16(pi.q_idx, device), k_idx=to_device_bf16(pi.k_idx, device),
        w=torch.from_numpy(np.ascontiguousarray(pi.w)).to(device),
        cu=torch.from_numpy(pi.cu_seqlens).to(device),
    )


def upload_decode_inputs(di, device="cuda"):
    """Device tensors of a decode workload (`inputs.DecodeInputs`): q, q_idx and the three caches
    as bf16, w as float32, seq_lens as int32."""
    import torch
    return dict(
        q=to_device_bf16(di.q, device), q_idx=to_device_bf16(di.q_idx, device),
        w=torch.from_numpy(np.ascontiguousarray(di.w)).to(device),
        k_cache=to_device_bf16(di.k_cache, device), v_cache=to_device_bf16(di.v_cache, device),
        k_idx_cache=to_device_bf16(di.k_idx_cache, device),
        seq_lens=torch.from_numpy(di.seq_lens.astype(np.int32)).to(device),
    )


def dsa_probe_mfma_bf16(shape, grid, iters, sink, stream=None) -> int:
    """Enqueue the MFMA-only probe; returns the flops it executes."""
    flops = ctypes.c_longlong(0)
    _check_probe(load_probes().dsa_probe_mfma_bf16(shape, grid, iters, _ptr(sink), ctypes.byref(flops),
                                                   _stream(stream)))
    return flops.value


def dsa_probe_stream_read(src, grid, sink, stream=None):
    """Enqueue the streaming-read probe over the whole of `src`."""
    _check_probe(load_probes().dsa_probe_stream_read(_ptr(src), src.numel() * src.element_size(), grid, _ptr(sink),
                                                     _stream(stream)))


def dsa_probe_atomic_add(buf, floats_per_row, grid, iters, stream=None):
    """Enqueue the float-atomic probe over buf [n_rows, 128] float32; returns the adds it makes."""
    n = ctypes.c_longlong(0)
    _check_probe(load_probes().dsa_probe_atomic_add(_ptr(buf), buf.shape[0], floats_per_row, grid, iters,
                                                    ctypes.byref(n), _stream(stream)))
    return n.value


def dsa_probe_gather(k, v, idx, sink, nsplit=1, row_stride=0, group_fastest=False, depth=2, whole_rows=False,
                     stream=None):
    """Enqueue the gather probe: the key and value rows the sparse attention reads for index sets
    idx[rows, k_sel] over k, v [n_pos, hkv, 128] (position row * row_stride + p)."""
    n_pos, hkv = k.shape[0], k.shape[1]
    rows, k_sel = idx.shape
    _check_probe(load_probes().dsa_probe_gather(_ptr(k), _ptr(v), n_pos, hkv, _ptr(idx), k_sel, rows, nsplit,
                                                row_stride, int(bool(group_fastest)), depth, int(bool(whole_rows)),
                                                _ptr(sink), sink.numel(), _stream(stream)))
