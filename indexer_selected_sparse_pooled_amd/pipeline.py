"""The hot path as a chain of libqsa calls.

A decode layer is A2 -> A3 -> A4 -> A5 (scores, top-k, split attention,
merge): one qsa_decode_layer call for the pooled-block variant, one
qsa_decode_layer_latent call for the shared latent, or the separate calls; a prefill chunk is A2 -> A3 -> A6 per history tile -> A5. Buffers
are allocated once with torch and reused; every step runs in libqsa's
kernels, enqueued on one stream with no host synchronisation, so a whole
layer or chunk can be captured in a HIP graph.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import qsa


@dataclass
class DecodeBuffers:
    scores: torch.Tensor    # [nq, max_ctx / block] fp32 (or None: see decode_buffers)
    sel: torch.Tensor       # [nq, topk] int32
    n_sel: torch.Tensor     # [nq] int32
    ws: torch.Tensor        # top-k workspace (or None)
    itk_ws: torch.Tensor    # zero-filled workspace of qsa_index_topk / qsa_index_lists (or None)
    layer_ws: torch.Tensor  # zero-filled workspace of qsa_decode_layer (or None)
    o_part: torch.Tensor    # [n_split, nq, hq, dv] fp32
    lse_part: torch.Tensor  # [n_split, nq, hq] fp32
    o: torch.Tensor         # [nq, hq, dv] fp32
    o_bf16: torch.Tensor    # [nq, hq, dv] bf16
    lse: torch.Tensor       # [nq, hq] fp32
    n_split: int
    latent_ws: torch.Tensor = None  # workspace of qsa_decode_layer_latent (or None)


def default_n_split(nq: int, hkv: int, budget_tokens: int) -> int:
    """Splits per (query, kv head): about 128 work-groups in all (fewer
    splits mean fewer partials to merge; the gathered rows are a small part
    of a decode step's bytes), or about 256 for the shared latent (one kv
    head, 64 heads per work-group: measured best at batch 8), at least 128
    tokens each (64 for the shared latent)."""
    target, least = (256, 64) if hkv == 1 else (128, 128)
    want = max(1, -(-target // max(1, nq * hkv)))
    most = max(1, budget_tokens // least)
    return int(min(want, most, 256))


def fused_select(sel_cfg) -> bool:
    """Whether qsa_index_topk covers this indexer (pooled 4-token blocks,
    one 128-d indexer head)."""
    return sel_cfg.block == 4 and sel_cfg.idx_dim == 128 and sel_cfg.idx_heads == 1


def fused_layer(sel_cfg, attn_cfg) -> bool:
    """Whether qsa_decode_layer covers this configuration."""
    return fused_select(sel_cfg) and (attn_cfg.hq, attn_cfg.hkv, attn_cfg.dk, attn_cfg.dv) == (16, 2, 256, 256)


def latent_layer(sel_cfg, attn_cfg) -> bool:
    """Whether qsa_decode_layer_latent covers this configuration (with bf16
    latent rows): the token-level 4-head indexer over the shared latent."""
    return ((sel_cfg.block, sel_cfg.idx_dim, sel_cfg.idx_heads) == (1, 64, 4) and sel_cfg.topk <= 2048
            and (attn_cfg.hq, attn_cfg.hkv, attn_cfg.dk, attn_cfg.dv) == (64, 1, 576, 512))


def decode_buffers(sel_cfg, attn_cfg, nq, max_ctx, n_split=None, device="cuda", keep_scores=True) -> DecodeBuffers:
    """Buffers of one decode layer. keep_scores=False: no score buffer (the
    one-call pooled-block layer then writes no scores; the separate calls
    need one)."""
    nmax = max(1, max_ctx // sel_cfg.block)
    if n_split is None:
        n_split = default_n_split(nq, attn_cfg.hkv, sel_cfg.topk * sel_cfg.block + sel_cfg.block - 1)
    f32 = dict(dtype=torch.float32, device=device)
    return DecodeBuffers(
        scores=torch.empty(nq, nmax, **f32) if keep_scores else None,
        sel=torch.empty(nq, sel_cfg.topk, dtype=torch.int32, device=device),
        n_sel=torch.empty(nq, dtype=torch.int32, device=device),
        ws=qsa.topk_workspace(sel_cfg, nq, max_ctx, device),
        itk_ws=qsa.index_topk_workspace(sel_cfg, nq, max_ctx, device) if fused_select(sel_cfg) else None,
        layer_ws=(qsa.decode_layer_workspace(sel_cfg, attn_cfg, nq, max_ctx, n_split, device)
                  if fused_layer(sel_cfg, attn_cfg) else None),
        o_part=torch.empty(n_split, nq, attn_cfg.hq, attn_cfg.dv, **f32),
        lse_part=torch.empty(n_split, nq, attn_cfg.hq, **f32),
        o=torch.empty(nq, attn_cfg.hq, attn_cfg.dv, **f32),
        o_bf16=torch.empty(nq, attn_cfg.hq, attn_cfg.dv, dtype=torch.bfloat16, device=device),
        lse=torch.empty(nq, attn_cfg.hq, **f32),
        n_split=n_split,
        latent_ws=(qsa.decode_layer_latent_workspace(sel_cfg, attn_cfg, nq, max_ctx, n_split, device)
                   if latent_layer(sel_cfg, attn_cfg) else None),
    )


def decode_layer(sel_cfg, attn_cfg, q_ctx, max_ctx, q_idx, keys, q, kv, bufs: DecodeBuffers,
                 q_seq=None, w_idx=None, stream=None, fused=False) -> None:
    """One decode layer for nq queries (one per sequence): results in bufs.o / o_bf16 / lse.
    fused=True issues the layer as one qsa_decode_layer call, or one
    qsa_decode_layer_latent call for the shared latent with bf16 rows (same
    results; the attention work-groups select their query's tokens
    themselves, so no selection is re-read in between)."""
    if fused and bufs.layer_ws is not None and w_idx is None and fused_layer(sel_cfg, attn_cfg):
        qsa.qsa_decode_layer(sel_cfg, attn_cfg, q_ctx, max_ctx, q_idx, keys, q, kv, bufs.scores, bufs.sel,
                             bufs.n_sel, bufs.n_split, bufs.layer_ws, o_out=bufs.o, o_out_bf16=bufs.o_bf16,
                             lse_out=bufs.lse, q_seq=q_seq, stream=stream)
        return
    if fused and bufs.latent_ws is not None and w_idx is not None and kv.format == qsa.KV_BF16:
        qsa.qsa_decode_layer_latent(sel_cfg, attn_cfg, q_ctx, max_ctx, q_idx, w_idx, keys, q, kv, bufs.scores,
                                    bufs.sel, bufs.n_sel, bufs.n_split, bufs.latent_ws, o_out=bufs.o,
                                    o_out_bf16=bufs.o_bf16, lse_out=bufs.lse, q_seq=q_seq, stream=stream)
        return
    if bufs.itk_ws is not None and w_idx is None:
        qsa.qsa_index_topk(sel_cfg, q_ctx, max_ctx, q_idx, keys, bufs.scores, bufs.sel, bufs.n_sel, bufs.itk_ws,
                           q_seq=q_seq, stream=stream)
    else:
        qsa.qsa_index_scores(sel_cfg, q_ctx, max_ctx, q_idx, keys, bufs.scores, q_seq=q_seq, w_idx=w_idx,
                             stream=stream)
        qsa.qsa_topk_blocks(sel_cfg, q_ctx, max_ctx, bufs.scores, bufs.sel, bufs.n_sel, bufs.ws, stream=stream)
    qsa.qsa_sparse_decode(sel_cfg, attn_cfg, q_ctx, max_ctx, q, kv, bufs.sel, bufs.n_sel, bufs.n_split,
                          bufs.o_part, bufs.lse_part, q_seq=q_seq, stream=stream)
    qsa.qsa_lse_merge(bufs.o_part, bufs.lse_part, o_out=bufs.o, o_out_bf16=bufs.o_bf16, lse_out=bufs.lse,
                      stream=stream)


@dataclass
class MicroBatch:
    """Sequences lo .. hi-1 of a decode batch, with their own buffers (one
    set per layer) and their slices of the batch's q_ctx / q_seq."""
    lo: int
    hi: int
    q_ctx: torch.Tensor
    q_seq: torch.Tensor
    bufs: list


def micro_batches(sel_cfg, attn_cfg, q_ctx, q_seq, max_ctx, n_layers, n_micro, n_split=None, device="cuda",
                  keep_scores=True):
    """Split a decode batch into n_micro contiguous micro-batches. Each keeps
    the batch's max_ctx and n_split (the whole batch's default unless given),
    so its layers run exactly the batch's kernels on its own sequences.
    keep_scores: as decode_buffers."""
    nq = int(q_ctx.numel())
    if not 1 <= n_micro <= nq:
        raise ValueError(f"n_micro {n_micro} not in [1, {nq}]")
    if n_split is None:
        n_split = default_n_split(nq, attn_cfg.hkv, sel_cfg.topk * sel_cfg.block + sel_cfg.block - 1)
    out = []
    for m in range(n_micro):
        lo, hi = m * nq // n_micro, (m + 1) * nq // n_micro
        out.append(MicroBatch(lo, hi, q_ctx[lo:hi].contiguous(), q_seq[lo:hi].contiguous(),
                              [decode_buffers(sel_cfg, attn_cfg, hi - lo, max_ctx, n_split=n_split, device=device,
                                              keep_scores=keep_scores)
                               for _ in range(n_layers)]))
    return out


def decode_step_streams(sel_cfg, attn_cfg, max_ctx, layers, micro, side_streams) -> None:
    """One decode step of a batch split into micro-batches: each micro-batch
    goes through the layers in order (one qsa_decode_layer call per layer)
    on a stream of its own, the first on the current stream and the others
    on side_streams (default priority); the current stream then waits for
    all of them. A micro-batch's layer l depends only on its own layer l - 1,
    so the streams' scans and attention tails can overlap. layers: one
    (q_idx, keys, q, kv) per layer, q_idx and q over the whole batch (their
    rows lo .. hi-1 go to each micro-batch); keys and kv are addressed by
    q_seq. Results land in each micro-batch's bufs[l]."""
    if len(side_streams) < len(micro) - 1:
        raise ValueError("need one side stream per micro-batch after the first")
    cur = torch.cuda.current_stream()
    for s in side_streams[:len(micro) - 1]:
        s.wait_stream(cur)

    streams = [cur] + list(side_streams[:len(micro) - 1])
    # issued layer by layer, alternating between the micro-batches, so that
    # the streams' work is submitted interleaved (a captured graph keeps
    # this order) rather than one micro-batch's whole chain first
    for l, (q_idx, keys, q, kv) in enumerate(layers):
        for s, mb in zip(streams, micro):
            with torch.cuda.stream(s):
                decode_layer(sel_cfg, attn_cfg, mb.q_ctx, max_ctx, q_idx[mb.lo:mb.hi], keys, q[mb.lo:mb.hi], kv,
                             mb.bufs[l], q_seq=mb.q_seq, fused=True)
    for s in side_streams[:len(micro) - 1]:
        cur.wait_stream(s)


@dataclass
class PrefillBuffers:
    scores: torch.Tensor      # [nq, max_ctx / block] fp32
    sel: torch.Tensor
    n_sel: torch.Tensor
    ws: torch.Tensor
    o_tiles: torch.Tensor     # [n_tiles, nq, hq, dv] fp32
    lse_tiles: torch.Tensor   # [n_tiles, nq, hq] fp32
    o: torch.Tensor
    o_bf16: torch.Tensor
    lse: torch.Tensor
    tiles: list
    sel_ws: torch.Tensor = None  # qsa_index_topk_prefill's workspace where that call applies


def history_tiles(ctx_max: int, tile: int):
    """[k*tile, (k+1)*tile) clipped to [0, ctx_max)."""
    return [(a, min(a + tile, ctx_max)) for a in range(0, ctx_max, tile)]


def single_tile_final(sel_cfg, attn_cfg, kv, n_tiles) -> bool:
    """Whether a chunk whose whole history is one tile takes its final
    result (O, lse and the bf16 copy) straight from the attention launch
    (qsa_sparse_prefill_merge as first and last tile): the shared latent with
    token-level selection and bf16 rows. No partials and no merge pass."""
    return (n_tiles == 1 and (attn_cfg.hq, attn_cfg.hkv, attn_cfg.dk, attn_cfg.dv) == (64, 1, 576, 512)
            and sel_cfg.block == 1 and kv.format == qsa.KV_BF16)


def running_tile_merge(attn_cfg) -> bool:
    """Whether qsa_sparse_prefill_merge covers this attention (the
    pooled-block variant): a chunk can then merge its history tiles as they
    complete instead of keeping per-tile partials (no partial buffers, no
    final merge; each tile reads the running result back, so it takes longer
    per tile)."""
    return (attn_cfg.hq, attn_cfg.hkv, attn_cfg.dk, attn_cfg.dv) == (16, 2, 256, 256)


def prefill_buffers(sel_cfg, attn_cfg, nq, max_ctx, tile, device="cuda", partials=True) -> PrefillBuffers:
    """partials: allocate per-tile partial results (o_tiles, lse_tiles);
    a chunk run with running_merge=True does without them."""
    nmax = max(1, max_ctx // sel_cfg.block)
    tiles = history_tiles(max_ctx, tile)
    f32 = dict(dtype=torch.float32, device=device)
    n_part = len(tiles) if partials else 0
    return PrefillBuffers(
        scores=torch.empty(nq, nmax, **f32),
        sel=torch.empty(nq, sel_cfg.topk, dtype=torch.int32, device=device),
        n_sel=torch.empty(nq, dtype=torch.int32, device=device),
        ws=qsa.topk_workspace(sel_cfg, nq, max_ctx, device),
        o_tiles=torch.empty(n_part, nq, attn_cfg.hq, attn_cfg.dv, **f32),
        lse_tiles=torch.empty(n_part, nq, attn_cfg.hq, **f32),
        o=torch.empty(nq, attn_cfg.hq, attn_cfg.dv, **f32),
        o_bf16=torch.empty(nq, attn_cfg.hq, attn_cfg.dv, dtype=torch.bfloat16, device=device),
        lse=torch.empty(nq, attn_cfg.hq, **f32),
        tiles=tiles,
        sel_ws=(qsa.index_topk_prefill_workspace(sel_cfg, nq, max_ctx, device)
                if sel_cfg.block == 1 and sel_cfg.idx_heads == 4 and nq >= 16 else None),
    )


def prefill_chunk(sel_cfg, attn_cfg, q_ctx, max_ctx, q_idx, keys, q, kv, bufs: PrefillBuffers,
                  w_idx=None, stream=None, fused_select=True, running_merge=False) -> None:
    """A chunk of queries of one sequence: selection, then the history tiles
    in the outer loop (one attention call per tile), then the merge of the
    per-tile partials; with running_merge (pooled-block variant), each tile
    is merged into the running result as it completes instead; a
    shared-latent chunk with one tile writes its result from the attention
    (single_tile_final). The
    token-level indexer selects in one call (qsa_index_topk_prefill) unless
    fused_select is False."""
    if fused_select and bufs.sel_ws is not None:
        qsa.qsa_index_topk_prefill(sel_cfg, q_ctx, max_ctx, q_idx, w_idx, keys, bufs.scores, bufs.sel, bufs.n_sel,
                                   bufs.sel_ws, stream=stream)
    else:
        qsa.qsa_index_scores(sel_cfg, q_ctx, max_ctx, q_idx, keys, bufs.scores, q_seq=None, w_idx=w_idx,
                             stream=stream)
        qsa.qsa_topk_blocks(sel_cfg, q_ctx, max_ctx, bufs.scores, bufs.sel, bufs.n_sel, bufs.ws, stream=stream)
    if running_merge:
        if not (running_tile_merge(attn_cfg) and kv.format == qsa.KV_BF16):
            raise ValueError("the running tile merge covers the pooled-block variant with bf16 K/V rows")
        # each tile merged into the running result as it completes
        last = len(bufs.tiles) - 1
        for t, (a, b) in enumerate(bufs.tiles):
            qsa.qsa_sparse_prefill_merge(sel_cfg, attn_cfg, q_ctx, max_ctx, q, kv, bufs.sel, bufs.n_sel, a, b,
                                         t == 0, t == last, bufs.o, bufs.lse, o_out_bf16=bufs.o_bf16, stream=stream)
        return
    if single_tile_final(sel_cfg, attn_cfg, kv, len(bufs.tiles)):
        a, b = bufs.tiles[0]
        qsa.qsa_sparse_prefill_merge(sel_cfg, attn_cfg, q_ctx, max_ctx, q, kv, bufs.sel, bufs.n_sel, a, b,
                                     True, True, bufs.o, bufs.lse, o_out_bf16=bufs.o_bf16, stream=stream)
        return
    if bufs.o_tiles.shape[0] != len(bufs.tiles):
        raise ValueError("prefill_buffers(..., partials=True) is needed for this attention")
    for t, (a, b) in enumerate(bufs.tiles):
        qsa.qsa_sparse_prefill(sel_cfg, attn_cfg, q_ctx, max_ctx, q, kv, bufs.sel, bufs.n_sel, a, b,
                               bufs.o_tiles[t], bufs.lse_tiles[t], stream=stream)
    qsa.qsa_lse_merge(bufs.o_tiles, bufs.lse_tiles, o_out=bufs.o, o_out_bf16=bufs.o_bf16, lse_out=bufs.lse,
                      stream=stream)
