"""The C ABI on a host without a GPU: the library loads, exports every declared symbol, and
rejects bad arguments with the documented status before anything is enqueued."""

import ctypes
import os
import re

import pytest

import sparse_long_context_lightning_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")
PROBES_HEADER = os.path.join(ROOT, "include", "dsa_probes.h")

P = ctypes.c_void_p
FAKE = P(1 << 20)            # aligned, never dereferenced by host validation
MISALIGNED = P((1 << 20) + 2)


def _declared(header=HEADER):
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(dsa_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = dsa.load()
    names = _declared()
    assert len(names) == 30
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(dsa.EXPORTED)
    # the measurement probes live in their own library, not in the product ABI
    assert not any(n.startswith("dsa_probe") for n in names)
    assert not hasattr(lib, "dsa_probe_mfma_bf16")


def test_probe_library_exports_every_declared_symbol():
    lib = dsa.load_probes()
    names = _declared(PROBES_HEADER)
    assert set(names) == set(dsa.PROBES_EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_launch_timing_record_without_launches():
    # Turning the timing on or off and reading an empty record make no HIP call.
    lib = dsa.load()
    dsa.dsa_timing_enable(True)
    dsa.dsa_timing_enable(False)
    assert dsa.dsa_timing_read() == {}
    n = ctypes.c_int(-1)
    assert lib.dsa_timing_count(None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_timing_count(ctypes.byref(n)) == dsa.DSA_OK and n.value == 0
    name, ms, cnt = ctypes.c_char_p(), ctypes.c_double(), ctypes.c_int64()
    assert lib.dsa_timing_entry(0, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(cnt)) == dsa.DSA_ERR_INVALID_ARG
    assert "outside" in dsa.dsa_last_error()


def test_version_and_status_strings():
    assert dsa.dsa_abi_version() == 1
    assert dsa.dsa_status_string(0) == "DSA_OK"
    assert dsa.dsa_status_string(3) == "DSA_ERR_WORKSPACE"
    assert dsa.dsa_status_string(99) == "DSA_ERR_UNKNOWN"


def _cu(vals):
    arr = (ctypes.c_int32 * len(vals))(*vals)
    return arr, ctypes.cast(arr, P)


def _prefill(lib, **over):
    cu_arr, cu_p = _cu([0, 100, 300])
    args = dict(q=FAKE, k=FAKE, v=FAKE, q_idx=FAKE, k_idx=FAKE, w=FAKE, cu=FAKE, cu_host=cu_p, batch=2, total=300,
                max_seqlen=200, hq=32, hkv=4, d=128, h_idx=64, d_idx=128, top_k=2048, scale=0.1, out=FAKE, lse=None,
                idx=FAKE, ws=FAKE, ws_bytes=1 << 30, stream=None)
    args.update(over)
    return lib.dsa_prefill(*args.values())


@pytest.mark.parametrize("over,status", [
    (dict(q=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(idx=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(cu_host=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(k=MISALIGNED), dsa.DSA_ERR_INVALID_ARG),
    (dict(hq=30, hkv=4), dsa.DSA_ERR_INVALID_ARG),
    (dict(d=64), dsa.DSA_ERR_UNSUPPORTED),
    (dict(hq=64, hkv=2), dsa.DSA_ERR_UNSUPPORTED),
    (dict(h_idx=8), dsa.DSA_ERR_UNSUPPORTED),
    (dict(top_k=0), dsa.DSA_ERR_UNSUPPORTED),
    (dict(top_k=4096), dsa.DSA_ERR_UNSUPPORTED),
    (dict(total=299), dsa.DSA_ERR_INVALID_ARG),
    (dict(max_seqlen=150), dsa.DSA_ERR_INVALID_ARG),
    (dict(ws_bytes=1000), dsa.DSA_ERR_WORKSPACE),
    (dict(ws=None), dsa.DSA_ERR_WORKSPACE),
])
def test_prefill_rejects_bad_arguments(over, status):
    lib = dsa.load()
    assert _prefill(lib, **over) == status
    assert dsa.dsa_last_error() != ""


def test_prefill_rejects_bad_cu_seqlens():
    lib = dsa.load()
    for vals in ([1, 100, 300], [0, 200, 100], [0, 100, 301]):
        arr, p = _cu(vals)
        assert _prefill(lib, cu_host=p) == dsa.DSA_ERR_INVALID_ARG


def test_other_entry_points_reject_bad_arguments():
    lib = dsa.load()
    cu_arr, cu_p = _cu([0, 64])
    # index scores: ld not a multiple of 4, row range outside, unsupported shape
    assert lib.dsa_index_scores(FAKE, FAKE, FAKE, cu_p, 1, 64, 64, 128, 0, 64, FAKE, 66, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_index_scores(FAKE, FAKE, FAKE, cu_p, 1, 64, 64, 128, 10, 60, FAKE, 64, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_index_scores(FAKE, FAKE, FAKE, cu_p, 1, 64, 64, 128, 0, 64, FAKE, 32, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_index_scores(FAKE, FAKE, FAKE, cu_p, 1, 64, 8, 128, 0, 64, FAKE, 64, None) == dsa.DSA_ERR_UNSUPPORTED
    # top-k
    assert lib.dsa_topk(FAKE, 64, 4, FAKE, 0, FAKE, None, None, 0, None) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_topk(FAKE, 63, 4, FAKE, 8, FAKE, None, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk(None, 64, 4, FAKE, 8, FAKE, None, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk(FAKE, 64, 4, None, 8, FAKE, None, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk_sorted(FAKE, 64, 4, FAKE, 4096, FAKE, None, None, 0, None) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_topk_sorted(FAKE, 62, 4, FAKE, 8, FAKE, None, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk_sorted(FAKE, 64, 4, FAKE, 8, None, None, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    # sparse attention
    assert lib.dsa_sparse_gqa_attn(FAKE, FAKE, FAKE, FAKE, 0, FAKE, 1, 64, 8, 2, 128, ctypes.c_float(0.1), FAKE, None,
                                   None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_sparse_gqa_attn(FAKE, FAKE, FAKE, FAKE, 16, FAKE, 1, 64, 8, 3, 128, ctypes.c_float(0.1), FAKE,
                                   None, None) == dsa.DSA_ERR_INVALID_ARG
    # decode
    args = [FAKE] * 7 + [4, 1000, 1000, 32, 4, 128, 64, 128, 2048, ctypes.c_float(0.1), FAKE, None, FAKE, FAKE, 10,
                         None]
    assert lib.dsa_decode(*args) == dsa.DSA_ERR_WORKSPACE
    args2 = list(args)
    args2[9] = 1001  # max_seq_len > s_max
    assert lib.dsa_decode(*args2) == dsa.DSA_ERR_INVALID_ARG
    # decode indexer scores: ld below s_max or not a multiple of 4, bad max_seq_len, unsupported shape
    d = lambda **o: [FAKE, FAKE, FAKE, FAKE, o.get("batch", 4), 1000, o.get("mx", 1000), o.get("h", 64), 128, FAKE,
                     o.get("ld", 1000), None]
    assert lib.dsa_decode_index_scores(*d(ld=996)) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_decode_index_scores(*d(ld=1002)) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_decode_index_scores(*d(mx=1001)) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_decode_index_scores(*d(mx=0)) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_decode_index_scores(*d(batch=0)) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_decode_index_scores(*d(h=8)) == dsa.DSA_ERR_UNSUPPORTED


def test_probe_validation():
    lib = dsa.load_probes()
    bad = 1  # DSA_PROBE_ERR_INVALID_ARG
    flops = ctypes.c_longlong(0)
    assert lib.dsa_probe_mfma_bf16(8, 64, 10, FAKE, ctypes.byref(flops), None) == bad
    assert lib.dsa_probe_mfma_bf16(16, 0, 10, FAKE, ctypes.byref(flops), None) == bad
    assert lib.dsa_probe_mfma_bf16(16, 64, 0, FAKE, ctypes.byref(flops), None) == bad
    assert lib.dsa_probe_mfma_bf16(32, 64, 10, None, ctypes.byref(flops), None) == bad
    assert lib.dsa_probe_last_error() != b""
    assert lib.dsa_probe_stream_read(MISALIGNED, 1 << 20, 64, FAKE, None) == bad
    assert lib.dsa_probe_stream_read(FAKE, (1 << 20) + 8, 64, FAKE, None) == bad
    assert lib.dsa_probe_stream_read(FAKE, 0, 64, FAKE, None) == bad
    assert lib.dsa_probe_stream_read(FAKE, 1 << 20, 0, FAKE, None) == bad
    assert lib.dsa_probe_stream_read(FAKE, 1 << 20, 64, None, None) == bad

    def gather(**o):
        a = dict(k=FAKE, v=FAKE, n_pos=1024, hkv=4, idx=FAKE, k_sel=64, rows=100, nsplit=1, row_stride=0,
                 group_fastest=0, depth=2, whole_rows=0, sink=FAKE, sink_len=1 << 20, stream=None)
        a.update(o)
        return lib.dsa_probe_gather(*a.values())

    assert gather(k=MISALIGNED) == bad
    assert gather(idx=None) == bad
    assert gather(depth=3) == bad
    assert gather(rows=0) == bad
    assert gather(row_stride=-1) == bad
    adds = ctypes.c_longlong(0)
    assert lib.dsa_probe_atomic_add(None, 1024, 64, 64, 10, ctypes.byref(adds), None) == bad
    assert lib.dsa_probe_atomic_add(FAKE, 0, 64, 64, 10, ctypes.byref(adds), None) == bad
    assert lib.dsa_probe_atomic_add(FAKE, 1024, 32, 64, 10, ctypes.byref(adds), None) == bad
    assert lib.dsa_probe_atomic_add(FAKE, 1024, 16, 0, 10, ctypes.byref(adds), None) == bad
    assert lib.dsa_probe_atomic_add(FAKE, 1024, 16, 64, 0, ctypes.byref(adds), None) == bad
    assert gather(sink_len=99) == bad     # 100 rows x 4 groups / 4 waves = 100 workgroups, padded to 104


def test_query_union_validation():
    lib = dsa.load()
    assert dsa.dsa_query_union_size(300, 2048) == (19, 32768)
    assert dsa.dsa_query_union_size(300, 2048, 8) == (38, 16384)
    assert dsa.dsa_query_union_size(16, 3) == (1, 64)
    with pytest.raises(dsa.DsaError):
        dsa.dsa_query_union_size(16, 3, 4)
    ok_cap = 32768
    args = lambda **o: [o.get("idx", FAKE), 2048, FAKE, 1, o.get("total", 300), o.get("rows", 16), o.get("cap", ok_cap),
                        FAKE, o.get("kv", FAKE), o.get("masks", FAKE), None]
    assert lib.dsa_query_union(*args(idx=None)) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_query_union(*args(kv=MISALIGNED)) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_query_union(*args(masks=MISALIGNED)) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_query_union(*args(cap=ok_cap - 32)) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_query_union(*args(cap=ok_cap + 16)) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_query_union(*args(rows=12)) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_query_union(*args(rows=8, cap=16384 - 32)) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_query_union(*args(rows=8, cap=16384, total=0)) == dsa.DSA_OK
    assert lib.dsa_query_union(*args(total=0)) == dsa.DSA_OK
    sc = ctypes.c_float(0.1)
    # merged-set attention: group sizes 4, 8, 16 only; cap a multiple of 32; blocks of 8 or 16 rows
    u = lambda **o: [FAKE, FAKE, FAKE, o.get("counts", FAKE), FAKE, FAKE, o.get("rows", 16), o.get("cap", ok_cap),
                     o.get("total", 300), o.get("hq", 32), 4, o.get("d", 128), sc, FAKE, None, None]
    assert lib.dsa_sparse_gqa_attn_union(*u(hq=8)) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_sparse_gqa_attn_union(*u(d=64)) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_sparse_gqa_attn_union(*u(rows=4)) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_sparse_gqa_attn_union(*u(cap=48)) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_sparse_gqa_attn_union(*u(counts=None)) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_sparse_gqa_attn_union(*u(total=0)) == dsa.DSA_OK


def test_dedup_attention_validation():
    lib = dsa.load()
    sc = ctypes.c_float(0.1)
    need = dsa.dsa_sparse_gqa_attn_dedup_workspace_size(300, 64, 32, 4)
    base = [FAKE, FAKE, FAKE, FAKE, 64, FAKE, 1, 300, 32, 4, 128, sc, FAKE, None]
    assert lib.dsa_sparse_gqa_attn_dedup(*base, None, 0, None) == dsa.DSA_ERR_WORKSPACE
    assert lib.dsa_sparse_gqa_attn_dedup(*base, FAKE, need - 1, None) == dsa.DSA_ERR_WORKSPACE
    assert lib.dsa_sparse_gqa_attn_dedup(*base, MISALIGNED, need, None) == dsa.DSA_ERR_INVALID_ARG
    bad = list(base)
    bad[3] = None
    assert lib.dsa_sparse_gqa_attn_dedup(*bad, FAKE, need, None) == dsa.DSA_ERR_INVALID_ARG
    bad = list(base)
    bad[8], bad[9] = 30, 4
    assert lib.dsa_sparse_gqa_attn_dedup(*bad, FAKE, need, None) == dsa.DSA_ERR_INVALID_ARG
    zero = list(base)
    zero[7] = 0
    assert lib.dsa_sparse_gqa_attn_dedup(*zero, FAKE, need, None) == dsa.DSA_OK
    # the merged-set kernel addresses K / V with 32-bit byte offsets: total_tokens * hkv < 2^24
    assert dsa.dsa_sparse_gqa_attn_dedup_workspace_size((1 << 22) - 1, 64, 32, 4) > 0
    assert dsa.dsa_sparse_gqa_attn_dedup_workspace_size(1 << 22, 64, 32, 4) == 0
    assert dsa.dsa_sparse_gqa_attn_dedup_workspace_size(1 << 22, 64, 16, 2) > 0


def test_dedup_backward_validation_and_workspace_size():
    lib = dsa.load()
    sc = ctypes.c_float(0.1)

    def _bwd_union(total, k, rows):   # per block: count, flag, rows x k int32 KV rows and uint32 masks
        nb, cap = (total + rows - 1) // rows, (rows * k + 31) // 32 * 32
        r = lambda x: (x + 255) // 256 * 256
        return 2 * r(nb * 4) + 2 * r(nb * cap * 4)
    assert dsa.dsa_sparse_gqa_attn_bwd_dedup_workspace_size(32768, 2048, 32, 4) == _bwd_union(32768, 2048, 32)
    assert dsa.dsa_sparse_gqa_attn_bwd_dedup_workspace_size(300, 64, 8, 2) == _bwd_union(300, 64, 32)
    assert dsa.dsa_sparse_gqa_attn_bwd_dedup_workspace_size(300, 64, 16, 1) == _bwd_union(300, 64, 16)
    # group sizes without the merged-set backward: the per-row backward, no workspace
    assert dsa.dsa_sparse_gqa_attn_bwd_dedup_workspace_size(300, 64, 4, 4) == 0
    assert dsa.dsa_sparse_gqa_attn_bwd_dedup_workspace_size(300, 64, 12, 4) == 0
    need = dsa.dsa_sparse_gqa_attn_bwd_dedup_workspace_size(300, 64, 32, 4)
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, 1, 300, 32, 4, 128, sc, FAKE, FAKE, FAKE]
    assert lib.dsa_sparse_gqa_attn_bwd_dedup(*base, None, 0, None) == dsa.DSA_ERR_WORKSPACE
    assert lib.dsa_sparse_gqa_attn_bwd_dedup(*base, FAKE, need - 1, None) == dsa.DSA_ERR_WORKSPACE
    assert lib.dsa_sparse_gqa_attn_bwd_dedup(*base, MISALIGNED, need, None) == dsa.DSA_ERR_INVALID_ARG
    for i in (4, 5, 6, 15, 16, 17):    # lse, dout, idx, dq, dk, dv are required
        bad = list(base)
        bad[i] = None
        assert lib.dsa_sparse_gqa_attn_bwd_dedup(*bad, FAKE, need, None) == dsa.DSA_ERR_INVALID_ARG, i
    bad = list(base)
    bad[15] = MISALIGNED
    assert lib.dsa_sparse_gqa_attn_bwd_dedup(*bad, FAKE, need, None) == dsa.DSA_ERR_INVALID_ARG
    bad = list(base)
    bad[13] = 64
    assert lib.dsa_sparse_gqa_attn_bwd_dedup(*bad, FAKE, need, None) == dsa.DSA_ERR_UNSUPPORTED
    zero = list(base)
    zero[10] = 0
    assert lib.dsa_sparse_gqa_attn_bwd_dedup(*zero, FAKE, need, None) == dsa.DSA_OK
    per_row = list(base)
    per_row[12] = 32   # group size 1: no workspace needed, the per-row path (nothing enqueued: total 0)
    per_row[10] = 0
    assert lib.dsa_sparse_gqa_attn_bwd_dedup(*per_row, None, 0, None) == dsa.DSA_OK


def test_head_mean_rejects_group_sizes_that_are_not_multiples_of_4():
    lib = dsa.load()
    cu_arr, cu_p = _cu([0, 300])
    sc = ctypes.c_float(0.1)
    call = lambda hq, hkv: lib.dsa_attn_head_mean(FAKE, FAKE, cu_p, 1, 300, hq, hkv, 128, sc, 0, 0, FAKE, 300, FAKE,
                                                  None)
    for hq, hkv in ((24, 4), (20, 4), (12, 2), (6, 1), (8, 4), (64, 16)):
        assert call(hq, hkv) == dsa.DSA_ERR_UNSUPPORTED, (hq, hkv)
    for hq, hkv in ((16, 4), (32, 4), (48, 4), (64, 4), (12, 1)):
        assert call(hq, hkv) == dsa.DSA_OK, (hq, hkv)   # zero rows: validated, nothing enqueued


def test_zero_sized_calls_are_no_ops():
    lib = dsa.load()
    cu_arr, cu_p = _cu([0, 64])
    assert lib.dsa_index_scores(FAKE, FAKE, FAKE, cu_p, 1, 64, 64, 128, 0, 0, FAKE, 64, None) == dsa.DSA_OK
    assert lib.dsa_topk(FAKE, 64, 0, FAKE, 8, FAKE, None, None, 0, None) == dsa.DSA_OK


def _topk_scratch(rows):
    head = (rows * 12 + 255) // 256 * 256
    return (head + rows * 8192 * 8 + 255) // 256 * 256


def test_workspace_sizes():
    # top-k: per-row threshold, counter and redo flag, then an 8192-entry (key, position) list per row;
    # rows longer than 262144 have only the scratch-free path
    assert dsa.dsa_topk_workspace_size(100, 4096, 2048) == _topk_scratch(100)
    assert dsa.dsa_topk_workspace_size(100, 262148, 2048) == 0
    # prefill: the larger of a 2048-row chunk of 131072 float scores plus its top-k scratch and the
    # merged index sets of the dedup attention (per 8-row block: count, flag, 8 k int32 KV rows,
    # 8 k uint16 masks, each array 256-byte aligned)
    def _union(total, k):
        nb, cap = (total + 7) // 8, (8 * k + 31) // 32 * 32
        r = lambda x: (x + 255) // 256 * 256
        return 2 * r(nb * 4) + r(nb * cap * 4) + r(nb * cap * 2)
    chunk = 2048 * 131072 * 4 + _topk_scratch(2048)
    assert _union(131072, 2048) > chunk
    assert dsa.dsa_prefill_workspace_size(1, 131072, 131072, 32, 4, 128, 64, 128, 2048) == _union(131072, 2048)
    assert dsa.dsa_sparse_gqa_attn_dedup_workspace_size(131072, 2048, 32, 4) == _union(131072, 2048)
    # group size 3 has no merged-set kernel: no dedup workspace, the chunk alone
    assert dsa.dsa_sparse_gqa_attn_dedup_workspace_size(131072, 2048, 12, 4) == 0
    assert dsa.dsa_prefill_workspace_size(1, 131072, 131072, 12, 4, 128, 64, 128, 2048) == chunk
    # small problems use the whole row count
    small = (100 * 100 * 4 + 255) // 256 * 256 + _topk_scratch(100)
    assert small > _union(100, 16)
    assert dsa.dsa_prefill_workspace_size(1, 100, 100, 8, 2, 128, 4, 64, 16) == small
    n = dsa.dsa_decode_workspace_size(32, 131072, 32, 4, 128, 64, 128, 2048)
    assert n >= 32 * 131072 * 4 + _topk_scratch(32)
    with pytest.raises(dsa.DsaError):
        dsa.dsa_decode_workspace_size(32, 131072, 32, 4, 64, 64, 128, 2048)


def test_topk_rejects_short_workspace():
    lib = dsa.load()
    need = dsa.dsa_topk_workspace_size(4, 64, 8)
    assert lib.dsa_topk(FAKE, 64, 4, FAKE, 8, FAKE, None, FAKE, need - 1, None) == dsa.DSA_ERR_WORKSPACE
    assert lib.dsa_topk(FAKE, 64, 4, FAKE, 8, FAKE, None, MISALIGNED, need, None) == dsa.DSA_ERR_INVALID_ARG


def test_index_scores_bwd_validation():
    lib = dsa.load()
    cu_arr, cu_p = _cu([0, 100, 300])

    def call(**over):
        a = dict(q=FAKE, k=FAKE, w=FAKE, cu=cu_p, batch=2, total=300, h=64, d=128, r0=80, rows=50, g=FAKE, ld=200,
                 dq=FAKE, dw=FAKE, dk=FAKE, stream=None)
        a.update(over)
        return lib.dsa_index_scores_bwd(*a.values())

    assert call(h=4, d=64) == dsa.DSA_ERR_UNSUPPORTED
    assert call(h=32, d=128) == dsa.DSA_ERR_UNSUPPORTED
    assert call(ld=198) == dsa.DSA_ERR_INVALID_ARG      # not a multiple of 4
    assert call(ld=28) == dsa.DSA_ERR_INVALID_ARG       # shorter than row 129's prefix (30)
    assert call(rows=300) == dsa.DSA_ERR_INVALID_ARG    # past total_tokens
    assert call(dq=MISALIGNED) == dsa.DSA_ERR_INVALID_ARG
    assert call(dk=None) == dsa.DSA_ERR_INVALID_ARG
    assert call(rows=0) == dsa.DSA_OK


def test_valid_call_without_a_gpu_reports_a_hip_error():
    """On a host without a usable GPU a call that passes validation fails at its first launch with
    DSA_ERR_HIP and the HIP message, instead of crashing (the pointers are never dereferenced: the
    launch is refused before any kernel runs).  Runs in a child process so that no HIP state of this
    process is touched."""
    import subprocess
    import sys
    code = r"""
import ctypes, sys
sys.path.insert(0, %r)
import sparse_long_context_lightning_amd as dsa
lib = dsa.load()
cu = (ctypes.c_int32 * 2)(0, 64)
st = lib.dsa_index_scores(ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 20),
                          ctypes.cast(cu, ctypes.c_void_p), 1, 64, 64, 128, 0, 64, ctypes.c_void_p(1 << 20), 64, None)
print(st, dsa.dsa_last_error())
""" % ROOT
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, res.stderr
    status, _, msg = res.stdout.strip().partition(" ")
    assert int(status) == dsa.DSA_ERR_HIP, res.stdout
    assert msg.startswith("indexer launch:"), msg


def test_dsa_log_reports_calls_and_rejections():
    """DSA_LOG=1: one stderr line per entry-point call (name and sizes) and one per rejection."""
    import subprocess
    import sys
    code = r"""
import ctypes, sys
sys.path.insert(0, %r)
import sparse_long_context_lightning_amd as dsa
lib = dsa.load()
lib.dsa_topk(ctypes.c_void_p(1 << 20), 64, 4, ctypes.c_void_p(1 << 20), 0, ctypes.c_void_p(1 << 20), None, None, 0, None)
""" % ROOT
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         env=dict(os.environ, DSA_LOG="1"), timeout=120)
    assert res.returncode == 0, res.stderr
    lines = [l for l in res.stderr.splitlines() if l.startswith("[dsa]")]
    assert lines[0] == "[dsa] dsa_topk(rows=4 ld=64 k=0 ws=0)", lines
    assert lines[1].startswith("[dsa] -> status 2: top_k 0 outside"), lines
    quiet = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                           env={k: v for k, v in os.environ.items() if k != "DSA_LOG"}, timeout=120)
    assert "[dsa]" not in quiet.stderr


def test_noalloc_decode_validation_without_a_gpu():
    """dsa_decode_noalloc checks its arguments on the host like dsa_decode, and refuses a step whose
    scratch need exceeds the library's static scratch before touching any device."""
    lib = dsa.load()
    f = ctypes.c_float(0.1)
    big = [FAKE] * 7 + [64, 262144, 262144, 32, 4, 128, 64, 128, 2048, f, FAKE, None, FAKE, None]
    assert lib.dsa_decode_noalloc(*big) == dsa.DSA_ERR_WORKSPACE
    assert "static scratch" in dsa.dsa_last_error()
    bad_shape = [FAKE] * 7 + [4, 1000, 1000, 32, 4, 64, 64, 128, 2048, f, FAKE, None, FAKE, None]
    assert lib.dsa_decode_noalloc(*bad_shape) == dsa.DSA_ERR_UNSUPPORTED
    assert dsa.dsa_decode_workspace_size(32, 131072, 32, 4, 128, 64, 128, 2048) <= (32 << 20)
    assert dsa.dsa_decode_workspace_size(8, 262144, 32, 4, 128, 64, 128, 2048) <= (32 << 20)
