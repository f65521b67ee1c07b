"""Indexer-selected sparse attention over pooled block keys, MI355X (gfx950).

The computation lives in libqsa.so (hand-written HIP, C ABI in
include/qsa.h); ``qsa`` is its thin binding and ``pipeline`` chains the
calls into a decode layer and a tiled prefill chunk.
"""
from . import qsa  # noqa: F401
from .qsa import (  # noqa: F401
    ATTN_A, ATTN_B, KEYS_BF16, KEYS_FP8, SEL_A, SEL_A_FP8, SEL_B, SEL_B_FP8, AttnCfg, QsaError, SelCfg, decode_layer_workspace,
    FP8_MLA_ROW, KV_BF16, KV_FP8_MLA, fp8_keys_empty, make_kv, qsa_fp8_keys_bytes, qsa_quantize_keys,
    qsa_quantize_latent,
    qsa_decode_layer, qsa_decode_layer_noalloc, qsa_decode_layer_workspace_bytes, qsa_decode_layer_latent,
    qsa_decode_layer_latent_workspace_bytes, decode_layer_latent_workspace, qsa_index_scores,
    qsa_index_topk, qsa_index_topk_workspace_bytes, index_topk_workspace, qsa_index_lists,
    qsa_kv_append, qsa_lse_merge, qsa_pool_keys, qsa_sparse_decode, qsa_sparse_prefill, qsa_sparse_prefill_merge,
    qsa_topk_blocks,
    qsa_topk_workspace_bytes, qsa_version, topk_workspace, decode_layer_error, check_decode_layer_error,
    qsa_index_topk_prefill, qsa_index_topk_prefill_workspace_bytes, index_topk_prefill_workspace,
    qsa_row_cache_bytes, qsa_decode_cached_plan_bytes, row_cache_empty, qsa_row_cache_step, qsa_sparse_decode_cached,
)
