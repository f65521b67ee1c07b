"""Algorithmic bytes and FLOPs of the hot path (host-side arithmetic only).

Decode unit = one query (one sequence) in one layer: the pooled-key scan
(every complete block's key), the indexer query, the gathered K/V rows of
the selected tokens, the query and the bf16 output. Scores and selections
are intermediates and are not counted. ("3090x3で 314 万コンテキスト": the
K/V read per layer is |S| x head_dim x 2 B x 2 (K and V) x kv heads, section
"なぜ"; the scan reads blocks x 128 x 2 B per layer, section
"VRAM に残す必要があるもの".)
"""
from __future__ import annotations

BF16 = 2


def attended_tokens(ctx: int, block: int = 4, topk: int = 512) -> int:
    nblk = ctx // block
    return ctx if nblk <= topk else topk * block + ctx % block


def scan_bytes(ctx: int, block: int = 4, idx_dim: int = 128) -> int:
    return (ctx // block) * idx_dim * BF16


def scan_bytes_fp8(ctx: int, block: int = 4, idx_dim: int = 128) -> int:
    """FP8 keys: idx_dim one-byte codes plus a 4-byte scale per key
    ("GLM-5.3 ...", footnote 3: 132 bytes for a 128-value key)."""
    return (ctx // block) * (idx_dim + 4)


def kv_bytes(n_tokens: int, hkv: int = 2, d: int = 256) -> int:
    return n_tokens * hkv * d * BF16 * 2


def decode_unit_bytes(ctx: int, block: int = 4, topk: int = 512, idx_dim: int = 128, hq: int = 16,
                      hkv: int = 2, d: int = 256) -> int:
    s = attended_tokens(ctx, block, topk)
    return (scan_bytes(ctx, block, idx_dim) + idx_dim * BF16 + kv_bytes(s, hkv, d)
            + hq * d * BF16 + hq * d * BF16)


def decode_unit_bytes_fp8(ctx: int, block: int = 4, topk: int = 512, idx_dim: int = 128, hq: int = 16,
                          hkv: int = 2, d: int = 256) -> int:
    """decode_unit_bytes with FP8 pooled keys (the K/V rows stay bf16)."""
    return decode_unit_bytes(ctx, block, topk, idx_dim, hq, hkv, d) - scan_bytes(ctx, block, idx_dim) \
        + scan_bytes_fp8(ctx, block, idx_dim)


def decode_unit_flops(ctx: int, block: int = 4, topk: int = 512, idx_dim: int = 128, hq: int = 16,
                      d: int = 256) -> int:
    s = attended_tokens(ctx, block, topk)
    return 2 * idx_dim * (ctx // block) + 2 * hq * s * (d + d)


def prefill_flops(ctxs, block: int = 4, topk: int = 512, idx_dim: int = 128, hq: int = 16, dk: int = 256,
                  dv: int = 256) -> dict:
    """Useful FLOPs of a prefill chunk: attention over each query's selected
    tokens plus the indexer scores of every candidate block."""
    att = sum(2 * hq * attended_tokens(c, block, topk) * (dk + dv) for c in ctxs)
    idx = sum(2 * idx_dim * (c // block) for c in ctxs)
    return {"attention": att, "indexer": idx, "total": att + idx}


def per_token_bytes(layers: int = 12, idx_dim: int = 128, block: int = 4, hkv: int = 2, d: int = 256) -> dict:
    """Memory per context token over all sparse layers: the pooled key
    (kept next to the GPU) and the K, V and raw indexer key rows."""
    pooled = layers * idx_dim * BF16 / block
    rows = layers * (2 * hkv * d * BF16 + idx_dim * BF16)
    return {"pooled": pooled, "kv_and_raw_keys": rows}


# Shared-latent variant ("GLM-5.3 最適化 第2部", section "PCP" and footnote 1):
# token-level indexer of idx_heads x idx_dim, top-2048 tokens, 64 query heads
# over one 576-wide latent row per token (V = its first 512 columns).

def mla_decode_unit_bytes(ctx: int, topk: int = 2048, idx_dim: int = 64, idx_heads: int = 4, hq: int = 64,
                          dk: int = 576, dv: int = 512) -> int:
    """One query in one layer: every earlier token's indexer key, the indexer
    query and head weights, the selected latent rows, the query and the bf16
    output."""
    s = attended_tokens(ctx, 1, topk)
    return (ctx * idx_dim * BF16 + idx_heads * idx_dim * BF16 + idx_heads * 4 + s * dk * BF16
            + hq * dk * BF16 + hq * dv * BF16)


FP8_MLA_ROW = 656  # "GLM-5.3 ...", footnote 1: 512 FP8 values + 4 scales + 64 bf16 rotary values


def mla_decode_unit_bytes_fp8_rows(ctx: int, topk: int = 2048, idx_dim: int = 64, idx_heads: int = 4,
                                   hq: int = 64, dk: int = 576, dv: int = 512) -> int:
    """mla_decode_unit_bytes with the selected latent rows in the 656-byte
    FP8 format (indexer keys bf16)."""
    s = attended_tokens(ctx, 1, topk)
    return mla_decode_unit_bytes(ctx, topk, idx_dim, idx_heads, hq, dk, dv) - s * dk * BF16 + s * FP8_MLA_ROW


def mla_decode_unit_bytes_fp8(ctx: int, topk: int = 2048, idx_dim: int = 64, idx_heads: int = 4, hq: int = 64,
                              dk: int = 576, dv: int = 512) -> int:
    """FP8 token keys (idx_dim codes + a 4-byte scale) and FP8 sparse-MLA rows."""
    return mla_decode_unit_bytes_fp8_rows(ctx, topk, idx_dim, idx_heads, hq, dk, dv) - ctx * idx_dim * BF16 \
        + ctx * (idx_dim + 4)


def mla_prefill_flops(ctxs, topk: int = 2048, idx_dim: int = 64, idx_heads: int = 4, hq: int = 64,
                      dk: int = 576, dv: int = 512) -> dict:
    """Useful FLOPs of a prefill chunk of the shared-latent variant."""
    att = sum(2 * hq * attended_tokens(c, 1, topk) * (dk + dv) for c in ctxs)
    idx = sum(2 * idx_heads * idx_dim * c for c in ctxs)
    return {"attention": att, "indexer": idx, "total": att + idx}
