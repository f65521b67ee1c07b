"""Pins for the CPU oracle (no GPU needed).

Each test ties the oracle to something other than itself: values derived by
hand from the pages' definitions (tests/golden/), closed forms, library
routines for the special cases the method reduces to (torch's fp32->bf16
rounding, torch's scaled_dot_product_attention in float64), brute force on
tiny inputs, and invariants (budget count, tile-size invariance, partition
invariance of the log-sum-exp merge).
"""
import math
import os

import numpy as np
import pytest
import torch

import qsa_inputs as qi
from oracle import qsa_oracle as orc

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def _bits(seed, stream, shape):
    n = int(np.prod(shape))
    return qi.normal_bf16(seed, stream, 0, n).reshape(shape)


# ------------------------------------------------------------- bf16 ------

def test_f64_to_bf16_matches_torch_on_fp32_values():
    """For values exactly representable in fp32 the one-step rounding must
    equal torch's fp32 -> bf16 conversion (round to nearest even)."""
    rng = np.random.default_rng(1)
    u = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    # add exact halfway cases and the subnormal range
    halves = ((rng.integers(0, 2**16, 5000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    halves = halves[np.isfinite(halves)]
    f = np.concatenate([f, halves, np.float32([0.0, -0.0, 1e-40, -1e-40, 3.0e38, -3.0e38])])
    ours = orc.f64_to_bf16(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_roundtrip_exact():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    vals = orc.bf16_to_f64(bits)
    keep = np.isfinite(vals)
    assert np.array_equal(orc.f64_to_bf16(vals[keep]), bits[keep])


# ------------------------------------------------------------- pooling ---

def test_pool_golden_cases():
    for row in _golden_rows("pool_cases.txt"):
        raw = np.array([int(x, 16) for x in row[:4]], dtype=np.uint16).reshape(4, 1)
        want = int(row[4], 16)
        got = int(orc.pool_keys(raw, 4)[0, 0])
        assert got == want, (row, hex(got))


def test_pool_matches_torch_mean_when_fp32_is_exact():
    """Raw keys on a 2**-6 grid in [-4, 4]: their fp32 sum and mean are exact,
    so torch's fp32 mean followed by its bf16 rounding is the same quantity."""
    rng = np.random.default_rng(2)
    vals = rng.integers(-256, 257, size=(4 * 300, 128)).astype(np.float32) / np.float32(64)
    raw = torch.from_numpy(vals).to(torch.bfloat16)
    assert torch.equal(raw.float(), torch.from_numpy(vals))  # inputs exact in bf16
    ref = torch.from_numpy(vals).reshape(300, 4, 128).mean(dim=1).to(torch.bfloat16)
    ours = orc.pool_keys(raw.view(torch.int16).numpy().view(np.uint16), 4)
    assert np.array_equal(ours, ref.view(torch.int16).numpy().view(np.uint16))


def test_pool_constant_blocks_and_partial_tail():
    raw = np.repeat(_bits(5, 1, (10, 128)), 4, axis=0)  # each row repeated 4x
    raw = np.concatenate([raw, _bits(5, 2, (3, 128))])  # 3 trailing tokens
    pooled = orc.pool_keys(raw, 4)
    assert pooled.shape == (10, 128)
    assert np.array_equal(pooled, raw[0:40:4])


def test_pool_block_one_is_identity():
    raw = _bits(5, 3, (17, 64))
    assert np.array_equal(orc.pool_keys(raw, 1), raw)


# ------------------------------------------------------------- scores ----

def test_scores_one_hot_query_reads_one_dimension():
    raw = _bits(7, 1, (4 * 50, 128))
    pooled = orc.pool_keys(raw, 4)
    for d in (0, 5, 127):
        q = np.zeros(128, dtype=np.uint16)
        q[d] = 0x4000  # 2.0
        s = orc.index_scores(q, pooled, 50)
        assert np.array_equal(s, 2.0 * orc.bf16_to_f64(pooled[:, d]))


def test_scores_relu_weighted_hand_example():
    # 2 tokens, 4 heads, dim 2. Dots per head, token 0: (1, -1, 2, 0.5); token 1: (-3, 4, 0, 1).
    one, mone, two, half = 0x3F80, 0xBF80, 0x4000, 0x3F00
    k = np.array([[one, 0], [0, one]], dtype=np.uint16)
    q = np.array([[one, 0xC040], [mone, 0x4080], [two, 0], [half, one]], dtype=np.uint16)  # -3=C040, 4=4080
    w = np.array([1.0, -2.0, 0.5, 4.0], dtype=np.float32)
    s = orc.index_scores_relu(q, w, k, 2)
    # token 0: relu(1,-1,2,0.5)=(1,0,2,0.5) -> 1 + 0 + 1 + 2 = 4
    # token 1: relu(-3,4,0,1)=(0,4,0,1) -> 0 - 8 + 0 + 4 = -4
    assert s.tolist() == [4.0, -4.0]


# ----------------------------------------------------------- selection ---

def _brute_select(s, topk):
    n = len(s)
    rank = [sum(1 for j in range(n) if s[j] > s[i] or (s[j] == s[i] and j < i)) for i in range(n)]
    return [i for i in range(n) if rank[i] < topk]


@pytest.mark.parametrize("seed", range(40))
def test_select_brute_force_tiny(seed):
    n = 1 + seed % 37
    topk = 1 + (seed * 7) % 12
    s = qi.tie_heavy_f32(seed, 3, n, levels=5).astype(np.float64)
    ctx = n * 4 + seed % 4
    want = list(range(n)) if n <= topk else _brute_select(list(s), topk)
    assert orc.select_blocks(s, ctx, 4, topk).tolist() == want
    assert orc.select_blocks_partition(s, ctx, 4, topk).tolist() == want


@pytest.mark.parametrize("n", [513, 2048, 16024, 262080])
def test_select_sort_and_partition_agree(n):
    for kind in ("uniform", "ties"):
        if kind == "uniform":
            s = qi.uniform_f32(11, n, n).astype(np.float64)
        else:
            s = qi.tie_heavy_f32(11, n, n, levels=40).astype(np.float64)
        a = orc.select_blocks(s, 4 * n, 4, 512)
        b = orc.select_blocks_partition(s, 4 * n, 4, 512)
        assert np.array_equal(a, b)
        assert a.size == 512 and np.all(np.diff(a) > 0)
        # everything selected ranks at least as high as everything left out
        out = np.setdiff1d(np.arange(n), a)
        assert s[a].min() >= s[out].max()


def test_budget_counts_golden():
    for block, topk, ctx, want in (map(int, r) for r in _golden_rows("budget_counts.txt")):
        n = ctx // block
        s = qi.uniform_f32(3, ctx, n).astype(np.float64)
        sel = orc.select_blocks(s, ctx, block, topk)
        toks = orc.selected_tokens(sel, ctx, block)
        assert toks.size == want, (block, topk, ctx)
        assert np.unique(toks).size == toks.size
        assert toks.max(initial=-1) < ctx


def test_threshold_2051_is_full_attention_and_2052_drops_lowest():
    for ctx in range(2040, 2052):
        s = qi.uniform_f32(4, ctx, ctx // 4).astype(np.float64)
        toks = orc.selected_tokens(orc.select_blocks(s, ctx, 4, 512), ctx, 4)
        assert np.array_equal(toks, np.arange(ctx))
    s = qi.uniform_f32(4, 2052, 513).astype(np.float64)
    sel = orc.select_blocks(s, 2052, 4, 512)
    assert np.array_equal(sel, np.delete(np.arange(513), np.argmin(s)))


def test_planted_selection():
    """Raw keys of 512 chosen blocks get +8 on dim 0 and the indexer query is
    e0: the selection must be exactly the planted blocks."""
    nblk, dim = 4000, 128
    raw = _bits(9, 1, (4 * nblk, dim))
    rng = np.random.default_rng(3)
    planted = np.sort(rng.choice(nblk, 512, replace=False))
    vals = orc.bf16_to_f64(raw)
    for b in planted:
        vals[4 * b: 4 * b + 4, 0] += 8.0
    raw = orc.f64_to_bf16(vals).reshape(raw.shape)
    pooled = orc.pool_keys(raw, 4)
    q = np.zeros(dim, dtype=np.uint16)
    q[0] = 0x3F80
    s = orc.index_scores(q, pooled, nblk)
    assert np.array_equal(orc.select_blocks(s, 4 * nblk + 2, 4, 512), planted)


def test_ties_go_to_lower_index_and_signed_zero_ties():
    s = np.zeros(1000)
    s[::2] = -0.0
    assert np.array_equal(orc.select_blocks(s, 4000, 4, 512), np.arange(512))
    s = np.full(1000, 1.0)
    s[700:] = 2.0
    sel = orc.select_blocks(s, 4000, 4, 512)
    assert np.array_equal(sel, np.concatenate([np.arange(212), np.arange(700, 1000)]))


# ----------------------------------------------------------- attention ---

def _sdpa_ref(q_bits, k_bits, v_bits, tokens_mask, scale):
    """torch scaled_dot_product_attention in float64 over all tokens, with a
    boolean mask (True = attend); GQA by repeating kv heads."""
    hq = q_bits.shape[0]
    hkv = k_bits.shape[1]
    q = torch.from_numpy(orc.bf16_to_f64(q_bits))[None, :, None, :]
    k = torch.from_numpy(orc.bf16_to_f64(k_bits)).permute(1, 0, 2)
    v = torch.from_numpy(orc.bf16_to_f64(v_bits)).permute(1, 0, 2)
    k = k.repeat_interleave(hq // hkv, dim=0)[None]
    v = v.repeat_interleave(hq // hkv, dim=0)[None]
    mask = torch.from_numpy(tokens_mask)[None, None, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    return o[0, :, 0, :].numpy()


def _layer(seed, ctx, hq=16, hkv=2, d=256, idx_dim=128):
    q = _bits(seed, 1, (hq, d))
    k = _bits(seed, 2, (ctx, hkv, d))
    v = _bits(seed, 3, (ctx, hkv, d))
    raw = _bits(seed, 4, (ctx, idx_dim))
    qidx = _bits(seed, 5, (idx_dim,))
    return q, k, v, raw, qidx


@pytest.mark.parametrize("ctx", [1, 3, 4, 5, 777, 2051])
def test_short_context_equals_dense_attention(ctx):
    """At most 512 complete blocks: every token is attended, so the result is
    plain dense attention (torch SDPA in float64)."""
    q, k, v, raw, qidx = _layer(20 + ctx, ctx)
    pooled = orc.pool_keys(raw, 4)
    r = orc.decode_query(q, qidx, pooled, k, v, ctx)
    assert r["tokens"].size == ctx
    ref = _sdpa_ref(q, k, v, np.ones(ctx, dtype=bool), 1.0 / 16)
    assert np.max(np.abs(r["o"] - ref)) < 1e-12


@pytest.mark.parametrize("ctx", [2052, 2055, 5003])
def test_sparse_equals_masked_dense_attention(ctx):
    """Above the threshold the result equals dense attention with logits set
    to -inf outside the selected set (torch SDPA, boolean mask, float64)."""
    q, k, v, raw, qidx = _layer(30 + ctx, ctx)
    pooled = orc.pool_keys(raw, 4)
    r = orc.decode_query(q, qidx, pooled, k, v, ctx)
    assert r["tokens"].size == 2048 + ctx % 4
    mask = np.zeros(ctx, dtype=bool)
    mask[r["tokens"]] = True
    ref = _sdpa_ref(q, k, v, mask, 1.0 / 16)
    assert np.max(np.abs(r["o"] - ref)) < 1e-12


def test_attention_closed_forms():
    ctx = 3000
    q, k, v, raw, qidx = _layer(40, ctx)
    toks = np.sort(np.random.default_rng(5).choice(ctx, 700, replace=False))
    # constant V rows -> O equals that constant
    vc = np.full_like(v, 0x3FC0)  # 1.5
    o, lse = orc.attend(q, k, vc, toks, 1.0 / 16)
    assert np.max(np.abs(o - 1.5)) < 1e-13
    # K = 0 -> uniform weights: O = mean of the selected V rows, lse = ln |S|
    kz = np.zeros_like(k)
    o, lse = orc.attend(q, kz, v, toks, 1.0 / 16)
    vm = orc.bf16_to_f64(v[toks]).mean(axis=0)  # [hkv][d]
    for h in range(16):
        assert np.max(np.abs(o[h] - vm[h // 8])) < 1e-12
    assert np.allclose(lse, math.log(700), rtol=0, atol=1e-12)
    # one token -> O is its V row, lse is its logit
    o, lse = orc.attend(q, k, v, toks[:1], 1.0 / 16)
    t = toks[0]
    for h in range(16):
        assert np.array_equal(o[h], orc.bf16_to_f64(v[t, h // 8]))
        assert lse[h] == pytest.approx(float(orc.bf16_to_f64(k[t, h // 8]) @ orc.bf16_to_f64(q[h])) / 16, abs=1e-12)
    # empty set -> (0, -inf)
    o, lse = orc.attend(q, k, v, toks[:0], 1.0 / 16)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_dominant_logit_picks_its_row():
    ctx = 500
    q, k, v, raw, qidx = _layer(41, ctx)
    kk = k.copy()
    kk[123, :, :] = orc.f64_to_bf16(orc.bf16_to_f64(q[0]) * 4.0)  # aligned with head 0's query
    o, _ = orc.attend(q, kk, v, np.arange(ctx), 1.0)
    assert np.max(np.abs(o[0] - orc.bf16_to_f64(v[123, 0]))) < 1e-6


# -------------------------------------------------------------- merge ----

def test_merge_partition_invariance_and_identity():
    ctx = 4000
    q, k, v, raw, qidx = _layer(50, ctx)
    toks = np.sort(np.random.default_rng(6).choice(ctx, 2048, replace=False))
    o_all, lse_all = orc.attend(q, k, v, toks, 1.0 / 16)
    rng = np.random.default_rng(7)
    for n_part in (1, 2, 5, 33):
        lab = rng.integers(0, n_part, toks.size)
        parts = [orc.attend(q, k, v, toks[lab == i], 1.0 / 16) for i in range(n_part)]
        o, lse = orc.lse_merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        assert np.max(np.abs(o - o_all)) < 1e-12
        assert np.max(np.abs(lse - lse_all)) < 1e-12
    # merging with an empty partial changes nothing
    empty_o, empty_l = np.zeros_like(o_all), np.full_like(lse_all, -np.inf)
    o, lse = orc.lse_merge(np.stack([empty_o, o_all, empty_o]), np.stack([empty_l, lse_all, empty_l]))
    assert np.array_equal(o, o_all) and np.array_equal(lse, lse_all)
    # all partials empty -> empty
    o, lse = orc.lse_merge(np.stack([empty_o, empty_o]), np.stack([empty_l, empty_l]))
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_merge_two_partials_closed_form():
    o = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    lse = np.array([[0.0], [math.log(3.0)]])
    m, l = orc.lse_merge(o, lse)
    assert np.allclose(m, [[0.25, 0.75]], atol=1e-15)
    assert l[0] == pytest.approx(math.log(4.0), abs=1e-15)


# ------------------------------------------------------------- prefill ---

def test_prefill_tile_invariance_and_decode_equivalence():
    """A query at position p of a prefill chunk equals decode with ctx = p+1,
    whatever the history tile size."""
    hist, chunk = 5000, 40
    ctx_max = hist + chunk
    q_all = _bits(60, 1, (chunk, 16, 256))
    k = _bits(60, 2, (ctx_max, 2, 256))
    v = _bits(60, 3, (ctx_max, 2, 256))
    raw = _bits(60, 4, (ctx_max, 128))
    qidx = _bits(60, 5, (chunk, 128))
    pooled = orc.pool_keys(raw, 4)
    for i in (0, 1, 17, 38, 39):
        p = hist + i
        ctx = p + 1
        r = orc.decode_query(q_all[i], qidx[i], pooled, k, v, ctx)
        outs = [orc.prefill_query_tiled(q_all[i], k, v, r["tokens"], ctx_max, t, 1.0 / 16)
                for t in (8192, 1024, 333)]
        for o, lse in outs:
            assert np.max(np.abs(o - r["o"])) < 1e-12
            assert np.max(np.abs(lse - r["lse"])) < 1e-12


# ----------------------------------------------------------- variant B ---

def test_variant_b_threshold_and_count():
    hq, d_lat = 64, 576
    for ctx in (100, 2048, 2049, 3000):
        q = _bits(70, 1, (hq, d_lat))
        lat = _bits(70, 2, (ctx, 1, d_lat))
        keys = _bits(70, 3, (ctx, 64))
        qidx = _bits(70, 4, (4, 64))
        w = qi.uniform_f32(70, 5, 4)
        r = orc.decode_query(q, qidx, keys, lat, lat, ctx, block=1, topk=2048,
                             scale=1.0 / 24, w_idx=w, dv=512)
        assert r["tokens"].size == min(ctx, 2048)
        assert r["o"].shape == (hq, 512)
        if ctx <= 2048:
            ref = _sdpa_ref(q, lat, lat[:, :, :512], np.ones(ctx, dtype=bool), 1.0 / 24)
        else:
            mask = np.zeros(ctx, dtype=bool)
            mask[r["tokens"]] = True
            ref = _sdpa_ref(q, lat, lat[:, :, :512], mask, 1.0 / 24)
        assert np.max(np.abs(r["o"] - ref)) < 1e-12
