"""CPU oracle: indexer-selected sparse attention over pooled block keys.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or
links this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library or its Python binding.

It is slow and plain on purpose: float64 numpy, with a matmul, a sort or a
partition as the only library steps, and no blocking, fusion or reordering
beyond what each definition states.

Sources (the method is described in prose only; no page prints a formula
or a worked example):

* [KVO] "3090x3で 314 万コンテキスト" (QSA K/V offload for exllamav3):
  section "なぜ" (why: budget 2048, compress ratio 4, threshold
  4*block_topk+3 = 2051, exactly 2048 tokens read per generated token),
  section "カーネルを書き換えずに済む" (the gather kernel addresses K/V as
  [token][kv_head][head_dim]), section "VRAM に残す必要があるもの" (one
  pooled key per block, 128 x bf16, scanned in full every step), section
  "ちなみにこの欠点" (prefill: history tiles in the outer loop, partial
  softmax results merged tile by tile, tile size changes nothing).
* [GLM] "GLM-5.3 最適化 第2部：16基のH200上でのPCP、DCP、およびHybrid
  HiSparse": section "PCP" (an indexer scores all earlier tokens and picks
  2,048 for sparse MLA; the latent is shared by all 64 heads), section "DCP"
  (partial attention results are combined with log-sum-exp), footnote 1
  (576-d QK, 512-d PV per latent row), section "試してみる" (prompts that fit
  the top-k would otherwise take the dense path: sparse equals dense there).
* [FLASH] "125B MoE を 3090 3 枚で運用する vLLM 最適化編", section 3.3
  (MoE block): top-k on packed keys where equal values go to the smaller id.
* [GLM] footnotes 1 and 3: the FP8 cache formats: an indexer key is 128
  FP8 values plus a 4-byte scale (132 bytes per token); a sparse-MLA row is
  656 bytes in the FP8 MLA format (the 512 latent values as FP8 with their
  scales, the 64 rotary values kept in 16-bit).
* OCP 8-bit floating point specification (E4M3): 1 sign bit, 4 exponent bits
  with bias 7, 3 mantissa bits; exponent field 0 holds subnormals; the
  pattern S.1111.111 is NaN; there are no infinities; the largest finite
  magnitude is 448.

Readings taken where the pages are silent:

R1  pooled key = exact mean of the block's raw keys, rounded once to bf16
    (round to nearest, ties to even).
R2  variant A score = plain dot product of the 128-d indexer query with the
    pooled key. Variant B score = sum over indexer heads h of
    w[h] * max(0, q_idx[h] . k[t]).
R3  one selection per query token, shared by every attention head.
R4  budget = the top `topk` complete blocks plus the 0..block-1 trailing
    tokens of the incomplete last block; when there are at most `topk`
    complete blocks every token is attended (full attention).
R5  a query at position p sees ctx = p + 1 tokens (its own included).
R6  no block is forced into the selection; the query's own complete block
    competes like any other.
R7  ranking order: score descending, then block index ascending
    (-0.0 equals +0.0; inputs are finite).
R8  selections are reported as ascending block indices.
R9  GQA: query head h reads kv head h // (hq // hkv).
R10 softmax scale is a parameter (1/16 for head_dim 256); lse is natural-log.
R11 an empty partial (no selected token in a tile) is (O = 0, lse = -inf).
R12 tiles are [k*T, (k+1)*T) in absolute token positions.
R17 FP8 values are OCP E4M3. A group of values (a whole indexer key, or 128
    consecutive latent values) shares one fp32 scale s = amax / 448 (fp32
    division of the group's largest magnitude); each value x is stored as
    the E4M3 code nearest to the fp32 quotient x / s (ties to even,
    magnitudes past 448 saturating to 448) and read back as code * s. An
    all-zero group has s = 0 and zero codes.
R18 the FP8 indexer key of a pooled block quantizes its bf16 pooled key
    (R1), one scale per key; the FP8 sparse-MLA row quantizes the first 512
    latent values in 4 groups of 128 and keeps the 64 rotary values as bf16.
"""
from __future__ import annotations

import math

import numpy as np

BF16_MAX = float.fromhex("0x1.fep127")


# ---------------------------------------------------------------- bf16 ----

def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """Round float64 values to bf16 bit patterns, nearest with ties to even.

    bf16 keeps 8 significant bits and fp32's exponent range: for
    |x| >= 2**-126 the spacing of bf16 values is 2**(e-8) with
    x = m * 2**e, 0.5 <= |m| < 1; below that the spacing is 2**-133.
    Rounding is done once, straight from float64.
    """
    x = np.atleast_1d(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    finite = np.isfinite(x)
    _, e = np.frexp(np.where(finite, x, 0.0))
    q = np.maximum(e - 8, -133)
    r = np.rint(np.ldexp(np.where(finite, x, 0.0), -q))  # ties to even
    y = np.ldexp(r, q)
    y = np.where(np.abs(y) > BF16_MAX, np.copysign(np.inf, x), y)
    y = np.where(finite, y, x)
    f = y.astype(np.float32)  # exact: y has at most 8 significant bits
    out[...] = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    out[nan] = 0x7FC0
    return out


# ------------------------------------------------------------ A1 pool ----

def _exact_sum_rows(v: np.ndarray) -> np.ndarray:
    """Sum along axis 1, checking with an error-free transformation that
    every float64 addition was exact (so the result is the exact sum)."""
    s = v[:, 0].copy()
    for j in range(1, v.shape[1]):
        b = v[:, j]
        t = s + b
        bb = t - s
        err = (s - (t - bb)) + (b - bb)
        if np.any(err != 0.0):
            raise ArithmeticError("block sum not exact in float64")
        s = t
    return s


def pool_keys(raw_bits: np.ndarray, block: int) -> np.ndarray:
    """A1: one pooled key per complete block of `block` tokens.

    pooled[b][d] = bf16( (1/block) * sum_{j<block} raw[block*b + j][d] )  (R1)

    [KVO] "VRAM に残す必要があるもの": the pooled key summarises a block's keys
    and is held as 128 bf16 values; the workload defines it as the mean.
    raw_bits: uint16 [n_tok][dim]. Returns uint16 [n_tok // block][dim].
    """
    raw = bf16_to_f64(raw_bits)
    n_tok, dim = raw.shape
    nblk = n_tok // block
    if nblk == 0:
        return np.zeros((0, dim), dtype=np.uint16)
    grp = raw[: nblk * block].reshape(nblk, block, dim)
    # sum over the block's tokens, per (block, dim) element
    flat = np.ascontiguousarray(grp.transpose(0, 2, 1)).reshape(nblk * dim, block)
    s = _exact_sum_rows(flat).reshape(nblk, dim)
    return f64_to_bf16(s / block)


# ----------------------------------------------------------- FP8 E4M3 ----

E4M3_MAX = 448.0


def e4m3_to_f64(codes) -> np.ndarray:
    """Exact value of OCP E4M3 codes (uint8) as float64.

    Exponent field e (bits 6..3), mantissa m (bits 2..0): e >= 1 is the
    normal number 2**(e-7) * (1 + m/8); e = 0 is the subnormal
    2**-6 * (m/8); S.1111.111 is NaN; bit 7 is the sign.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp((8 + m).astype(np.float64), e - 10))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where((c & 0x80) != 0, -mag, mag)


def f64_to_e4m3(x) -> np.ndarray:
    """Round finite values to E4M3 codes: nearest, ties to even, magnitudes
    above 448 saturate to 448. The sign of the input is kept (also for
    results that round to zero).

    Around a normal |x| = f * 2**e (0.5 <= f < 1) the format keeps 4
    significant bits, so its spacing is 2**(e-4); below 2**-6 the spacing
    is the subnormal step 2**-9.
    """
    x = np.atleast_1d(np.asarray(x, dtype=np.float64))
    if not np.all(np.isfinite(x)):
        raise ValueError("E4M3 rounding takes finite values")
    a = np.abs(x)
    _, e = np.frexp(a)
    q = np.maximum(e - 4, -9)
    y = np.minimum(np.ldexp(np.rint(np.ldexp(a, -q)), q), E4M3_MAX)  # rint: ties to even
    # encode the (now representable) magnitude y
    _, ey = np.frexp(y)
    normal = y >= 2.0 ** -6
    ef = np.where(normal, ey - 1 + 7, 0)
    mf = np.where(normal, np.ldexp(y, -(ey - 1)) * 8 - 8, np.ldexp(y, 9))
    code = (ef.astype(np.int64) << 3) | mf.astype(np.int64)
    code = code | np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8)


def quantize_e4m3(x, group: int):
    """R17: groups of `group` consecutive values along the last axis, each
    with one fp32 scale s = amax / 448 and codes = E4M3(x / s), both
    quotients in fp32. x must be exactly representable in fp32 (bf16 values
    are). Returns (codes uint8 [..., n], scales float32 [..., n / group])."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    if n % group:
        raise ValueError("the last axis must be a whole number of groups")
    xf = x.astype(np.float32)
    if not np.array_equal(xf.astype(np.float64), x):
        raise ValueError("values must be exact in fp32")
    g = xf.reshape(x.shape[:-1] + (n // group, group))
    amax = np.abs(g).max(axis=-1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)  # fp32 / fp32, correctly rounded
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    quot = (g / safe[..., None]).astype(np.float32)  # fp32 division per value
    codes = f64_to_e4m3(quot.astype(np.float64)).reshape(g.shape)
    codes = np.where(scale[..., None] > 0, codes, np.uint8(0)).astype(np.uint8)
    return codes.reshape(x.shape), scale


def dequantize_e4m3(codes, scales, group: int) -> np.ndarray:
    """code value * its group's scale, exact in float64 (4 + 24 significant bits)."""
    v = e4m3_to_f64(codes)
    sc = np.repeat(np.asarray(scales, dtype=np.float64), group, axis=-1)
    return v * sc


def fp8_keys(keys_bits):
    """R18: FP8 indexer keys, one scale per key (idx_dim codes + 4 bytes).
    [GLM] footnote 3: 128 FP8 values and a 4-byte scale per key.
    keys_bits: uint16 [n][dim] (bf16). Returns (codes [n][dim], scales [n])."""
    k = np.asarray(keys_bits, dtype=np.uint16)
    codes, scales = quantize_e4m3(bf16_to_f64(k), k.shape[-1])
    return codes, scales[..., 0]


def fp8_latent(latent_bits, n_quant: int = 512, group: int = 128):
    """R18: the FP8 sparse-MLA row: the first n_quant latent values in groups
    of `group` with one fp32 scale each, the rest (the rotary part) kept as
    bf16. [GLM] footnote 1: a 656-byte FP8 row (512 + 4*4 + 64*2 bytes).
    latent_bits: uint16 [n][576]. Returns (codes [n][512], scales [n][4],
    rope_bits [n][64])."""
    lat = np.asarray(latent_bits, dtype=np.uint16)
    codes, scales = quantize_e4m3(bf16_to_f64(lat[:, :n_quant]), group)
    return codes, scales, lat[:, n_quant:].copy()


def fp8_latent_values(codes, scales, rope_bits, group: int = 128) -> np.ndarray:
    """The float64 row an FP8 sparse-MLA row stands for: dequantized latent
    values, then the bf16 rotary values."""
    return np.concatenate([dequantize_e4m3(codes, scales, group), bf16_to_f64(rope_bits)], axis=-1)


# ---------------------------------------------------------- A2 scores ----

def index_scores(q_idx_bits: np.ndarray, keys_bits: np.ndarray, n: int) -> np.ndarray:
    """A2, variant A (R2): s[b] = q_idx . pooled[b] for b < n, in float64.

    [KVO] "VRAM に残す必要があるもの": every pooled key is scored each step.
    q_idx_bits: uint16 [dim]; keys_bits: uint16 [>= n][dim].
    """
    q = bf16_to_f64(q_idx_bits)
    k = bf16_to_f64(keys_bits[:n])
    return k @ q


def index_scores_relu(q_idx_bits: np.ndarray, w: np.ndarray, keys_bits: np.ndarray, n: int) -> np.ndarray:
    """A2, variant B (R2): s[t] = sum_h w[h] * max(0, q_idx[h] . k[t]).

    [GLM] "PCP": a token-level indexer scores every earlier token; the
    workload specifies several indexer heads combined by a ReLU-weighted sum.
    q_idx_bits: uint16 [heads][dim]; w: float32 [heads]; keys: uint16 [>= n][dim].
    """
    q = bf16_to_f64(q_idx_bits)
    k = bf16_to_f64(keys_bits[:n])
    per_head = k @ q.T  # [n][heads]
    return np.maximum(per_head, 0.0) @ np.asarray(w, dtype=np.float64)


def index_scores_fp8(q_idx_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray, n: int) -> np.ndarray:
    """A2, variant A with FP8 keys (R17, R18): s[b] = q_idx . (codes[b] * scales[b])."""
    q = bf16_to_f64(q_idx_bits)
    k = dequantize_e4m3(codes[:n], np.asarray(scales)[:n, None], codes.shape[-1])
    return k @ q


def index_scores_relu_fp8(q_idx_bits: np.ndarray, w: np.ndarray, codes: np.ndarray, scales: np.ndarray,
                          n: int) -> np.ndarray:
    """A2, variant B with FP8 token keys: the ReLU-weighted sum over the
    dequantized keys."""
    q = bf16_to_f64(q_idx_bits)
    k = dequantize_e4m3(codes[:n], np.asarray(scales)[:n, None], codes.shape[-1])
    return np.maximum(k @ q.T, 0.0) @ np.asarray(w, dtype=np.float64)


# ------------------------------------------------------------- A3 top-k ----

def n_candidates(ctx: int, block: int) -> int:
    """Number of complete blocks visible to a query with `ctx` tokens (R5)."""
    return ctx // block


def select_blocks(scores: np.ndarray, ctx: int, block: int, topk: int) -> np.ndarray:
    """A3 by full sort: ascending indices of the selected blocks (R4, R7, R8).

    [KVO] "なぜ": with more than topk complete blocks the indexer keeps a fixed
    budget; otherwise the whole history is read. [FLASH] 3.3: equal values go
    to the smaller index.
    """
    n = n_candidates(ctx, block)
    s = np.asarray(scores[:n], dtype=np.float64)
    if not np.all(np.isfinite(s)):
        raise ValueError("scores must be finite")
    if n <= topk:
        return np.arange(n, dtype=np.int64)
    order = np.lexsort((np.arange(n), -s))  # primary: -score; then index
    return np.sort(order[:topk])


def select_blocks_partition(scores: np.ndarray, ctx: int, block: int, topk: int) -> np.ndarray:
    """A3 a second way (selection, not sorting): find the topk-th largest
    value, keep everything above it, then fill with the lowest-indexed
    blocks equal to it."""
    n = n_candidates(ctx, block)
    s = np.asarray(scores[:n], dtype=np.float64)
    if n <= topk:
        return np.arange(n, dtype=np.int64)
    tau = np.partition(s, n - topk)[n - topk]
    above = np.flatnonzero(s > tau)
    equal = np.flatnonzero(s == tau)
    need = topk - above.size
    return np.sort(np.concatenate([above, equal[:need]]))


def selected_tokens(sel_blocks: np.ndarray, ctx: int, block: int) -> np.ndarray:
    """Token positions attended: each selected block's tokens, then the
    trailing tokens of the incomplete last block (R4). Ascending."""
    n = n_candidates(ctx, block)
    sel = np.asarray(sel_blocks, dtype=np.int64)
    toks = (sel[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    tail = np.arange(n * block, ctx, dtype=np.int64)
    return np.concatenate([toks, tail])


# ---------------------------------------------------------- A4 attend ----

def attend(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, tokens: np.ndarray,
           scale: float, dv: int = None):
    """A4: softmax attention of each query head over the given tokens.

    q_bits: uint16 [hq][dk]; k_bits: uint16 [n_tok][hkv][dk];
    v_bits: uint16 [n_tok][hkv][>= dv] (only the first dv columns are used,
    so the MLA latent can serve as both K and V).
    For head h with kv head g = h // (hq // hkv) (R9):
        z_j = scale * (q_h . k_{j,g}),  m = max z,  l = sum exp(z_j - m)
        O_h = sum exp(z_j - m) v_{j,g} / l,  lse_h = m + ln l
    An empty token set gives (O = 0, lse = -inf) (R11).
    [KVO] "なぜ" and "カーネルを書き換えずに済む": only the selected K/V rows are
    read, addressed per (token, kv head).
    Returns (O float64 [hq][dv], lse float64 [hq]).
    """
    return attend_values(q_bits, k_bits, v_bits, tokens, scale, dv, to_f64=bf16_to_f64)


def attend_values(q_bits, k_rows, v_rows, tokens, scale, dv=None, to_f64=None):
    """A4 over K/V rows given as float64 values (to_f64 None), or as any
    encoding that to_f64 turns into them (bf16 bits in attend). The FP8
    sparse-MLA rows enter here through fp8_latent_values."""
    conv = (lambda a: np.asarray(a, dtype=np.float64)) if to_f64 is None else to_f64
    hq, dk = q_bits.shape
    hkv = k_rows.shape[1]
    if dv is None:
        dv = v_rows.shape[2]
    group = hq // hkv
    q = bf16_to_f64(q_bits)
    out = np.zeros((hq, dv))
    lse = np.full(hq, -np.inf)
    tokens = np.asarray(tokens, dtype=np.int64)
    if tokens.size == 0:
        return out, lse
    for g in range(hkv):
        kg = conv(k_rows[tokens, g, :])
        vg = conv(v_rows[tokens, g, :dv])
        for h in range(g * group, (g + 1) * group):
            z = scale * (kg @ q[h])
            m = z.max()
            p = np.exp(z - m)
            l = p.sum()
            out[h] = (p @ vg) / l
            lse[h] = m + math.log(l)
    return out, lse


# ----------------------------------------------------------- A5 merge ----

def lse_merge(o_parts: np.ndarray, lse_parts: np.ndarray):
    """A5: combine partial softmax results.

    lse = M + ln sum_i exp(lse_i - M) with M = max_i lse_i;
    O = sum_i exp(lse_i - lse) O_i; partials with lse_i = -inf add nothing;
    if every partial is empty the result is (0, -inf).
    [GLM] "DCP": partial attention results are combined by log-sum-exp.
    [KVO] "ちなみにこの欠点": softmax partials are merged tile after tile.
    o_parts: [P][rows][dv]; lse_parts: [P][rows].
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    n_part, rows, dv = o_parts.shape
    out = np.zeros((rows, dv))
    lse = np.full(rows, -np.inf)
    for r in range(rows):
        li = lse_parts[:, r]
        live = np.isfinite(li)
        if not np.any(live):
            continue
        m = li[live].max()
        tot = m + math.log(np.exp(li[live] - m).sum())
        wts = np.exp(li[live] - tot)
        out[r] = wts @ o_parts[live, r, :]
        lse[r] = tot
    return out, lse


# --------------------------------------------------- decode, one query ----

def decode_query(q_bits, q_idx_bits, keys_bits, k_bits, v_bits, ctx, *, block=4, topk=512,
                 scale=1.0 / 16.0, w_idx=None, dv=None):
    """A2 -> A3 -> A4 for one query that sees `ctx` tokens of one sequence.

    Variant A (w_idx is None): keys_bits are pooled block keys.
    Variant B (w_idx given, block = 1): keys_bits are per-token indexer keys.
    Returns dict(scores, sel, tokens, o, lse).
    """
    n = n_candidates(ctx, block)
    if w_idx is None:
        s = index_scores(q_idx_bits, keys_bits, n)
    else:
        s = index_scores_relu(q_idx_bits, w_idx, keys_bits, n)
    sel = select_blocks(s, ctx, block, topk)
    toks = selected_tokens(sel, ctx, block)
    o, lse = attend(q_bits, k_bits, v_bits, toks, scale, dv)
    return {"scores": s, "sel": sel, "tokens": toks, "o": o, "lse": lse}


# ---------------------------------------------------- A6 tiled prefill ----

def tiles(ctx_max: int, tile: int):
    """History tiles [k*T, (k+1)*T) clipped to [0, ctx_max) (R12)."""
    return [(a, min(a + tile, ctx_max)) for a in range(0, ctx_max, tile)]


def prefill_tile(q_bits, k_bits, v_bits, tokens, tile_begin, tile_end, scale, dv=None):
    """A6 for one query and one tile: attention over S(q) intersected with
    [tile_begin, tile_end); an empty intersection gives (0, -inf)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    sub = tokens[(tokens >= tile_begin) & (tokens < tile_end)]
    return attend(q_bits, k_bits, v_bits, sub, scale, dv)


def prefill_query_tiled(q_bits, k_bits, v_bits, tokens, ctx_max, tile, scale, dv=None):
    """A6 + A5: loop over history tiles in order, merging partials.

    [KVO] "ちなみにこの欠点": history is cut into fixed-size tiles, every
    query is computed against a tile, and the softmax partials are merged
    before moving to the next tile.
    """
    parts = [prefill_tile(q_bits, k_bits, v_bits, tokens, a, b, scale, dv)
             for a, b in tiles(ctx_max, tile)]
    o_parts = np.stack([p[0] for p in parts])
    lse_parts = np.stack([p[1] for p in parts])
    o, lse = lse_merge(o_parts, lse_parts)
    return o, lse
