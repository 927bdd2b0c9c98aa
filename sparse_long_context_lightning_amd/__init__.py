"""DSA (lightning indexer -> top-k -> sparse GQA attention) for AMD MI355X.

The compute runs in libdsa.so (hand-written HIP for gfx950) behind the C ABI declared in
include/dsa.h; this package only binds it.  The benchmark's measurement probes are a separate
library, libdsa_probes.so (include/dsa_probes.h).  Build the library with
`python -m sparse_long_context_lightning_amd.build`.
"""

from ._lib import (  # noqa: F401
    DSA_ERR_HIP,
    DSA_ERR_INVALID_ARG,
    DSA_ERR_UNSUPPORTED,
    DSA_ERR_WORKSPACE,
    DSA_MAX_TOP_K,
    DSA_OK,
    EXPORTED,
    LIB_PATH,
    PROBES_EXPORTED,
    PROBES_LIB_PATH,
    DsaError,
    decode,
    dsa_abi_version,
    dsa_decode,
    dsa_decode_index_scores,
    dsa_decode_workspace_size,
    dsa_attn_head_mean,
    dsa_index_scores,
    dsa_index_scores_bwd,
    dsa_indexer_kl,
    dsa_last_error,
    dsa_prefill,
    dsa_prefill_workspace_size,
    dsa_probe_gather,
    dsa_probe_mfma_bf16,
    dsa_probe_stream_read,
    dsa_query_union,
    dsa_query_union_size,
    dsa_sparse_gqa_attn,
    dsa_sparse_gqa_attn_bwd,
    dsa_sparse_gqa_attn_dedup,
    dsa_sparse_gqa_attn_dedup_workspace_size,
    dsa_sparse_gqa_attn_union,
    dsa_status_string,
    dsa_topk,
    dsa_topk_sorted,
    dsa_topk_workspace_size,
    load,
    load_probes,
    prefill,
    to_device_bf16,
    upload_decode_inputs,
    upload_prefill_inputs,
)
