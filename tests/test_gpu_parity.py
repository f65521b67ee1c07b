"""GPU parity: libqsa (through its C ABI) against the CPU oracle.

Every GPU result is compared with the oracle on the same seeded inputs:
bit-exact for pooling and selection, within the stated tolerances for
scores and attention (see tests/qsa_cases.py).
"""
import numpy as np
import pytest
import torch

import qsa_inputs as qi
from oracle import qsa_oracle as orc
from tests import qsa_cases as qc

pytestmark = pytest.mark.gpu

gpu_ok = torch.cuda.is_available()


@pytest.fixture(scope="module")
def Q():
    if not gpu_ok:
        pytest.skip("no GPU")
    import indexer_selected_sparse_pooled_amd as pkg
    from indexer_selected_sparse_pooled_amd import pipeline
    pkg.qsa.lib()  # fails loudly if the library is missing
    return pkg, pipeline


def _print_case(name, **kw):
    print(f"[case] {name} {kw}", flush=True)


# ------------------------------------------------------------ generator ---

def test_gpu_generator_matches_host(Q):
    from qsa_inputs.gpu import fill_normal_bf16
    n = 1 << 20
    out = torch.empty(n + 5, dtype=torch.bfloat16, device="cuda")
    fill_normal_bf16(out, 77, 12345, start=3)
    torch.cuda.synchronize()
    want = qi.normal_bf16(77, 12345, 3, n + 5)
    assert np.array_equal(qc.from_dev_bits(out), want)


# ------------------------------------------------------------------ A1 ----

@pytest.mark.parametrize("n_tok", [4, 7, 1024, 8195])
def test_pool_bit_exact(Q, n_tok):
    pkg, _ = Q
    _print_case("pool", n_tok=n_tok)
    raw = np.stack([qc.bits(5, s, (n_tok, 128)) for s in range(3)])
    nb = n_tok // 4
    pooled = torch.zeros(3, max(nb, 1), 128, dtype=torch.bfloat16, device="cuda")
    pkg.qsa_pool_keys(qc.to_dev(raw), pooled, block=4)
    torch.cuda.synchronize()
    got = qc.from_dev_bits(pooled)
    for s in range(3):
        assert np.array_equal(got[s, :nb], orc.pool_keys(raw[s], 4))


def test_pool_golden_cases_on_gpu(Q):
    pkg, _ = Q
    rows = []
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "pool_cases.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append([int(x, 16) for x in line.split()])
    raw = np.zeros((len(rows) * 4, 8), dtype=np.uint16)
    for b, r in enumerate(rows):
        raw[4 * b: 4 * b + 4, 0] = r[:4]
    pooled = torch.zeros(1, len(rows), 8, dtype=torch.bfloat16, device="cuda")
    pkg.qsa_pool_keys(qc.to_dev(raw[None]), pooled, block=4)
    got = qc.from_dev_bits(pooled)[0, :, 0]
    assert got.tolist() == [r[4] for r in rows]


def test_pool_append_range(Q):
    """Pooling only [tok_begin, tok_end) leaves the other blocks untouched."""
    pkg, _ = Q
    raw = qc.bits(6, 1, (1, 4000, 128))
    pooled = torch.full((1, 1000, 128), 7, dtype=torch.int16, device="cuda")
    pkg.qsa_pool_keys(qc.to_dev(raw), pooled, tok_begin=400, tok_end=2003, block=4)
    got = qc.from_dev_bits(pooled)[0]
    ref = orc.pool_keys(raw[0], 4)
    assert np.array_equal(got[100:500], ref[100:500])
    assert np.all(got[:100] == 7) and np.all(got[500:] == 7)


# ------------------------------------------------------------------ A2 ----

@pytest.mark.parametrize("ctxs,q_seq", [([8195, 2051, 5000, 3], True), ([64096] * 20, False)])
def test_scores_variant_a(Q, ctxs, q_seq):
    pkg, _ = Q
    _print_case("scores_a", ctxs=ctxs[:4], q_seq=q_seq)
    nq = len(ctxs)
    max_ctx = max(ctxs)
    if q_seq:
        raws = np.stack([qc.bits(8, 100 + s, (max_ctx, 128)) for s in range(nq)])
    else:
        raws = qc.bits(8, 100, (1, max_ctx, 128))
        ctxs = [max_ctx - 40 * i for i in range(nq)]
    pooled_np = np.stack([orc.pool_keys(r, 4) for r in raws])
    q_idx = qc.bits(8, 7, (nq, 1, 128))
    scores = torch.full((nq, max_ctx // 4 + 3), float("nan"), device="cuda")
    pkg.qsa_index_scores(pkg.SEL_A, qc.i32(ctxs), max_ctx, qc.to_dev(q_idx), qc.to_dev(pooled_np), scores,
                         q_seq=qc.i32(range(nq)) if q_seq else None)
    got = scores.cpu().numpy()
    for i, ctx in enumerate(ctxs):
        s = i if q_seq else 0
        n = ctx // 4
        ref = orc.index_scores(q_idx[i, 0], pooled_np[s], n)
        tol = qc.score_tolerance(q_idx[i, 0], pooled_np[s], n)
        assert np.all(np.abs(got[i, :n] - ref) <= tol)
        assert np.all(np.isnan(got[i, n:])), "wrote past the candidates"


@pytest.mark.parametrize("chunk", [False, True])
def test_scores_variant_b(Q, chunk):
    pkg, _ = Q
    nq = 3 if not chunk else 40
    max_ctx = 5000
    keys = qc.bits(9, 1, (1 if chunk else nq, max_ctx, 64))
    q_idx = qc.bits(9, 2, (nq, 4, 64))
    w = np.stack([qi.uniform_f32(9, 10 + i, 4) for i in range(nq)])
    ctxs = [max_ctx - 7 * i for i in range(nq)]
    scores = torch.full((nq, max_ctx), float("nan"), device="cuda")
    pkg.qsa_index_scores(pkg.SEL_B, qc.i32(ctxs), max_ctx, qc.to_dev(q_idx), qc.to_dev(keys), scores,
                         q_seq=None if chunk else qc.i32(range(nq)), w_idx=torch.tensor(w, device="cuda"))
    got = scores.cpu().numpy()
    for i, ctx in enumerate(ctxs):
        s = 0 if chunk else i
        ref = orc.index_scores_relu(q_idx[i], w[i], keys[s], ctx)
        kd = orc.bf16_to_f64(keys[s][:ctx])
        qd = orc.bf16_to_f64(q_idx[i])
        tol = 64 * 2.0**-24 * (np.abs(kd) @ np.abs(qd).T) @ np.abs(w[i].astype(np.float64)) * 2 + 1e-30
        assert np.all(np.abs(got[i, :ctx] - ref) <= tol)
        assert np.all(np.isnan(got[i, ctx:]))


# ------------------------------------------------------------------ A3 ----

def _run_topk(pkg, cfg, scores_np, ctxs):
    nq = len(ctxs)
    max_ctx = max(ctxs)
    scores = torch.tensor(scores_np, device="cuda")
    sel = torch.full((nq, cfg.topk), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.full((nq,), -7, dtype=torch.int32, device="cuda")
    ws = pkg.topk_workspace(cfg, nq, max_ctx)
    pkg.qsa_topk_blocks(cfg, qc.i32(ctxs), max_ctx, scores, sel, n_sel, ws)
    return sel.cpu().numpy(), n_sel.cpu().numpy()


@pytest.mark.parametrize("n,kind", [(2048, "uniform"), (2049, "uniform"), (513, "ties"), (16024, "uniform"),
                                    (16024, "ties"), (32768, "ties"), (32769, "uniform"), (262080, "uniform"),
                                    (262080, "ties"), (100003, "sorted_desc"), (100003, "sorted_asc"),
                                    (70000, "all_equal"), (262080, "sampled_high")])
def test_topk_bit_exact(Q, n, kind):
    """Selection from fixed fp32 scores: the GPU must reproduce the oracle's
    ranking (score desc, index asc) exactly, on every path. "sampled_high"
    raises exactly the scores the threshold sample reads (256 runs of 16
    spread over the candidates), so the sampled threshold lies above all but
    a few scores and the exact fallback must run."""
    pkg, _ = Q
    _print_case("topk", n=n, kind=kind)
    nq = 3
    rows = []
    for i in range(nq):
        if kind == "uniform":
            s = qi.uniform_f32(21, 1000 * n + i, n)
        elif kind == "ties":
            s = qi.tie_heavy_f32(21, 1000 * n + i, n, levels=200)
        elif kind == "sorted_desc":
            s = np.sort(qi.uniform_f32(21, i, n))[::-1].copy()
        elif kind == "sorted_asc":
            s = np.sort(qi.uniform_f32(21, i, n))
        elif kind == "sampled_high":
            s = qi.uniform_f32(21, 1000 * n + i, n)
            for t in range(256):
                st = t * (n - 16) // 255
                s[st:st + 16] += np.float32(10.0)
        else:
            s = np.full(n, 0.5, dtype=np.float32)
        rows.append(s)
    scores = np.stack(rows).astype(np.float32)
    ctxs = [4 * n + 3, 4 * n, 4 * (n // 2) + 1]
    sel, n_sel = _run_topk(pkg, pkg.SEL_A, scores, ctxs)
    for i, ctx in enumerate(ctxs):
        want = orc.select_blocks(scores[i].astype(np.float64), ctx, 4, 512)
        assert n_sel[i] == want.size
        assert np.array_equal(sel[i, :n_sel[i]], want), f"query {i}"
        assert np.all(sel[i, n_sel[i]:] == -1)


def test_topk_small_and_empty_contexts(Q):
    pkg, _ = Q
    ctxs = [0, 1, 3, 4, 2051, 2052, 2055, 9]
    n = 600
    scores = np.stack([qi.uniform_f32(22, i, n) for i in range(len(ctxs))])
    sel, n_sel = _run_topk(pkg, pkg.SEL_A, scores, ctxs)
    for i, ctx in enumerate(ctxs):
        want = orc.select_blocks(scores[i].astype(np.float64), ctx, 4, 512)
        assert n_sel[i] == want.size and np.array_equal(sel[i, :n_sel[i]], want)
        assert np.all(sel[i, n_sel[i]:] == -1)


def test_topk_variant_b_large(Q):
    pkg, _ = Q
    n = 131072
    scores = np.stack([qi.uniform_f32(23, i, n) for i in range(2)])
    ctxs = [n, n - 5]
    sel, n_sel = _run_topk(pkg, pkg.SEL_B, scores, ctxs)
    for i, ctx in enumerate(ctxs):
        want = orc.select_blocks(scores[i].astype(np.float64), ctx, 1, 2048)
        assert np.array_equal(sel[i, :n_sel[i]], want)


# ------------------------------------------------------------- A4 + A5 ----

def _decode_with_sel(pkg, pipeline, case, sels, n_split):
    nq = case.nq
    max_ctx = max(case.ctxs)
    kv = pkg.make_kv(qc.to_dev(case.k), qc.to_dev(case.v))
    sel = torch.full((nq, 512), -1, dtype=torch.int32, device="cuda")
    n_sel = torch.zeros(nq, dtype=torch.int32, device="cuda")
    for i, s in enumerate(sels):
        sel[i, :len(s)] = torch.tensor(np.asarray(s, dtype=np.int32))
        n_sel[i] = len(s)
    o_part = torch.empty(n_split, nq, 16, 256, device="cuda")
    lse_part = torch.empty(n_split, nq, 16, device="cuda")
    pkg.qsa_sparse_decode(pkg.SEL_A, pkg.ATTN_A, qc.i32(case.ctxs), max_ctx, qc.to_dev(case.q), kv, sel, n_sel,
                          n_split, o_part, lse_part, q_seq=qc.i32(range(nq)))
    o = torch.empty(nq, 16, 256, device="cuda")
    ob = torch.empty(nq, 16, 256, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(nq, 16, device="cuda")
    pkg.qsa_lse_merge(o_part, lse_part, o_out=o, o_out_bf16=ob, lse_out=lse)
    torch.cuda.synchronize()
    return o.cpu().numpy(), qc.from_dev_bits(ob), lse.cpu().numpy(), o_part, lse_part


@pytest.mark.parametrize("n_split", [1, 3, 32, 64])
def test_decode_attention_with_oracle_selection(Q, n_split):
    pkg, pipeline = Q
    ctxs = [8195, 2051, 2052, 5001, 1, 0, 130]
    _print_case("decode_attn", n_split=n_split, ctxs=ctxs)
    case = qc.DecodeCase(31, ctxs)
    refs = case.oracle()
    o, ob, lse, _, _ = _decode_with_sel(pkg, pipeline, case, [r["sel"] for r in refs], n_split)
    for i, r in enumerate(refs):
        qc.check_attention(o[i], lse[i], r["o"], r["lse"], ob[i])


def test_decode_splits_match_oracle_partials(Q):
    """Each split's partial equals the oracle's attention over that split's
    part of the token list."""
    pkg, pipeline = Q
    case = qc.DecodeCase(32, [6003])
    r = case.oracle()[0]
    n_split = 5
    _, _, _, o_part, lse_part = _decode_with_sel(pkg, pipeline, case, [r["sel"]], n_split)
    toks = r["tokens"]
    L = toks.size
    for j in range(n_split):
        part = toks[j * L // n_split:(j + 1) * L // n_split]
        o_ref, lse_ref = orc.attend(case.q[0], case.k[0], case.v[0], part, 1.0 / 16)
        qc.check_attention(o_part[j, 0].cpu().numpy(), lse_part[j, 0].cpu().numpy(), o_ref, lse_ref)


@pytest.mark.parametrize("P,dv", [(7, 256), (33, 512), (7, 300), (20, 36)])
def test_merge_against_oracle(Q, P, dv):
    """Rows of 256, 512 (two 256-dim pieces per row), 300 (a partial second
    piece) and 36 dims; more partials than one batch of 16; an all-empty
    row; the bf16 copy equals the fp32 result rounded to bf16."""
    pkg, _ = Q
    rows = 33
    _print_case("merge", P=P, dv=dv)
    rng = np.random.default_rng(3)
    o = rng.standard_normal((P, rows, dv)).astype(np.float32)
    lse = (rng.standard_normal((P, rows)) * 3).astype(np.float32)
    lse[2, :] = -np.inf
    lse[:, 5] = -np.inf
    o[:, 5] = 0
    out = torch.empty(rows, dv, device="cuda")
    out_b = torch.empty(rows, dv, dtype=torch.bfloat16, device="cuda")
    out_l = torch.empty(rows, device="cuda")
    pkg.qsa_lse_merge(torch.tensor(o, device="cuda"), torch.tensor(lse, device="cuda"), o_out=out, o_out_bf16=out_b,
                      lse_out=out_l)
    ref_o, ref_l = orc.lse_merge(o, lse)
    got_o, got_l = out.cpu().numpy(), out_l.cpu().numpy()
    assert torch.equal(out_b, out.to(torch.bfloat16))
    assert np.isneginf(got_l[5]) and np.all(got_o[5] == 0)
    live = ~np.isneginf(ref_l)
    assert np.max(np.abs(got_o[live] - ref_o[live])) <= 1e-5 * np.max(np.abs(ref_o))
    assert np.max(np.abs(got_l[live] - ref_l[live])) <= 1e-5


# ------------------------------------------------------ decode end to end -

@pytest.mark.parametrize("ctxs", [[8192], [8195, 2051, 2052, 3, 40000]])
def test_decode_layer_end_to_end(Q, ctxs):
    pkg, pipeline = Q
    _print_case("decode_e2e", ctxs=ctxs)
    case = qc.DecodeCase(41, ctxs)
    refs = case.oracle()
    nq, max_ctx = case.nq, max(ctxs)
    raw = qc.to_dev(case.raw)
    pooled = torch.zeros(nq, max(1, case.cap // 4), 128, dtype=torch.bfloat16, device="cuda")
    pkg.qsa_pool_keys(raw, pooled, block=4)
    kv = pkg.make_kv(qc.to_dev(case.k), qc.to_dev(case.v))
    bufs = pipeline.decode_buffers(pkg.SEL_A, pkg.ATTN_A, nq, max_ctx)
    pipeline.decode_layer(pkg.SEL_A, pkg.ATTN_A, qc.i32(ctxs), max_ctx, qc.to_dev(case.q_idx[:, None, :]), pooled,
                          qc.to_dev(case.q), kv, bufs, q_seq=qc.i32(range(nq)))
    torch.cuda.synchronize()
    pooled_np = qc.from_dev_bits(pooled)
    sel, n_sel = bufs.sel.cpu().numpy(), bufs.n_sel.cpu().numpy()
    o, lse, ob = bufs.o.cpu().numpy(), bufs.lse.cpu().numpy(), qc.from_dev_bits(bufs.o_bf16)
    for i, r in enumerate(refs):
        nb = ctxs[i] // 4
        assert np.array_equal(pooled_np[i, :nb], r["pooled"])
        # every row's attention is checked: against the oracle's result, or
        # after a tolerated boundary swap against the oracle on the GPU's selection
        qc.check_row(sel[i], n_sel[i], o[i], lse[i], ob[i], r, ctxs[i], 4, 512, case.q[i], case.k[i], case.v[i],
                     1.0 / 16)


def test_decode_is_deterministic(Q):
    pkg, pipeline = Q
    case = qc.DecodeCase(42, [9000, 3001])
    nq, max_ctx = 2, 9000
    pooled = torch.zeros(nq, case.cap // 4, 128, dtype=torch.bfloat16, device="cuda")
    pkg.qsa_pool_keys(qc.to_dev(case.raw), pooled, block=4)
    kv = pkg.make_kv(qc.to_dev(case.k), qc.to_dev(case.v))
    outs = []
    for _ in range(3):
        bufs = pipeline.decode_buffers(pkg.SEL_A, pkg.ATTN_A, nq, max_ctx)
        pipeline.decode_layer(pkg.SEL_A, pkg.ATTN_A, qc.i32(case.ctxs), max_ctx,
                              qc.to_dev(case.q_idx[:, None, :]), pooled, qc.to_dev(case.q), kv, bufs,
                              q_seq=qc.i32(range(nq)))
        outs.append((bufs.o.cpu().numpy().tobytes(), bufs.sel.cpu().numpy().tobytes()))
    assert outs[0] == outs[1] == outs[2]


# ------------------------------------------------------------ A6 prefill --

@pytest.mark.parametrize("tile,running", [(8192, False), (1024, False), (332, False), (1024, True), (332, True)])
def test_prefill_chunk_tiled(Q, tile, running):
    """A prefill chunk of 48 queries after a 9000-token history: per-query
    selection, tiles in the outer loop, log-sum-exp merge (of the per-tile
    partials, or running, tile by tile); every row equals the oracle's
    decode at ctx = position + 1, whatever the tile size."""
    pkg, pipeline = Q
    hist, nq = 9000, 48
    ctx_max = hist + nq
    _print_case("prefill", tile=tile, hist=hist, nq=nq)
    seed = 51
    raw = qc.bits(seed, 1, (ctx_max, 128))
    k = qc.bits(seed, 2, (ctx_max, 2, 256))
    v = qc.bits(seed, 3, (ctx_max, 2, 256))
    q = qc.bits(seed, 4, (nq, 16, 256))
    q_idx = qc.bits(seed, 5, (nq, 1, 128))
    ctxs = [hist + i + 1 for i in range(nq)]
    pooled = torch.zeros(1, ctx_max // 4, 128, dtype=torch.bfloat16, device="cuda")
    pkg.qsa_pool_keys(qc.to_dev(raw[None]), pooled, block=4)
    kv = pkg.make_kv(qc.to_dev(k[None]), qc.to_dev(v[None]))
    bufs = pipeline.prefill_buffers(pkg.SEL_A, pkg.ATTN_A, nq, ctx_max, tile, partials=not running)
    pipeline.prefill_chunk(pkg.SEL_A, pkg.ATTN_A, qc.i32(ctxs), ctx_max, qc.to_dev(q_idx), pooled, qc.to_dev(q),
                           kv, bufs, running_merge=running)
    torch.cuda.synchronize()
    pooled_np = orc.pool_keys(raw, 4)
    sel, n_sel = bufs.sel.cpu().numpy(), bufs.n_sel.cpu().numpy()
    o, lse, ob = bufs.o.cpu().numpy(), bufs.lse.cpu().numpy(), qc.from_dev_bits(bufs.o_bf16)
    for i in range(nq):
        r = orc.decode_query(q[i], q_idx[i, 0], pooled_np, k, v, ctxs[i])
        qc.check_row(sel[i], n_sel[i], o[i], lse[i], ob[i], r, ctxs[i], 4, 512, q[i], k, v, 1.0 / 16)


def test_prefill_tile_partials_match_oracle(Q):
    """One tile call: each query's partial equals the oracle's attention over
    its tokens inside the tile (empty -> 0, -inf)."""
    pkg, pipeline = Q
    hist, nq = 6000, 16
    ctx_max = hist + nq
    k = qc.bits(52, 2, (ctx_max, 2, 256))
    v = qc.bits(52, 3, (ctx_max, 2, 256))
    q = qc.bits(52, 4, (nq, 16, 256))
    rng = np.random.default_rng(9)
    ctxs = [hist + i + 1 for i in range(nq)]
    sels = [np.sort(rng.choice(c // 4, 512, replace=False)) for c in ctxs]
    sels[3] = np.arange(0, 512)  # nothing inside the tile below
    sel = torch.tensor(np.stack(sels).astype(np.int32), device="cuda")
    n_sel = qc.i32([512] * nq)
    kv = pkg.make_kv(qc.to_dev(k[None]), qc.to_dev(v[None]))
    a, b = 4096, 5120
    o_p = torch.empty(nq, 16, 256, device="cuda")
    l_p = torch.empty(nq, 16, device="cuda")
    pkg.qsa_sparse_prefill(pkg.SEL_A, pkg.ATTN_A, qc.i32(ctxs), ctx_max, qc.to_dev(q), kv, sel, n_sel, a, b, o_p, l_p)
    torch.cuda.synchronize()
    o_p, l_p = o_p.cpu().numpy(), l_p.cpu().numpy()
    for i in range(nq):
        toks = orc.selected_tokens(sels[i], ctxs[i], 4)
        o_ref, l_ref = orc.prefill_tile(q[i], k, v, toks, a, b, 1.0 / 16)
        qc.check_attention(o_p[i], l_p[i], o_ref, l_ref)


def test_prefill_running_merge_matches_partials(Q):
    """qsa_sparse_prefill_merge over consecutive tiles (first / last flags,
    the running result in place) against qsa_sparse_prefill per tile plus
    qsa_lse_merge: equal within fp32 rounding of the merge order; lse
    -inf and O = 0 for a query with no token in any tile so far; the bf16
    output written by the last tile only."""
    pkg, pipeline = Q
    hist, nq = 9000, 24
    ctx_max = hist + nq
    k = qc.bits(54, 2, (ctx_max, 2, 256))
    v = qc.bits(54, 3, (ctx_max, 2, 256))
    q = qc.bits(54, 4, (nq, 16, 256))
    rng = np.random.default_rng(11)
    ctxs = [hist + i + 1 for i in range(nq)]
    sels = [np.sort(rng.choice(c // 4, 512, replace=False)) for c in ctxs]
    sels[5] = np.arange(1500, 2012)  # all inside one tile: empty before and after it
    sel = torch.tensor(np.stack(sels).astype(np.int32), device="cuda")
    n_sel = qc.i32([512] * nq)
    kv = pkg.make_kv(qc.to_dev(k[None]), qc.to_dev(v[None]))
    q_dev, q_ctx = qc.to_dev(q), qc.i32(ctxs)
    tiles = pipeline.history_tiles(ctx_max, 2048)
    o_p = torch.empty(len(tiles), nq, 16, 256, device="cuda")
    l_p = torch.empty(len(tiles), nq, 16, device="cuda")
    for t, (a, b) in enumerate(tiles):
        pkg.qsa_sparse_prefill(pkg.SEL_A, pkg.ATTN_A, q_ctx, ctx_max, q_dev, kv, sel, n_sel, a, b, o_p[t], l_p[t])
    o_ref = torch.empty(nq, 16, 256, device="cuda")
    l_ref = torch.empty(nq, 16, device="cuda")
    pkg.qsa_lse_merge(o_p, l_p, o_out=o_ref, lse_out=l_ref)
    o_run = torch.full((nq, 16, 256), float("nan"), device="cuda")
    l_run = torch.full((nq, 16), float("nan"), device="cuda")
    ob = torch.zeros(nq, 16, 256, dtype=torch.bfloat16, device="cuda")
    for t, (a, b) in enumerate(tiles):
        _print_case("prefill_running_merge", tile=t)
        pkg.qsa_sparse_prefill_merge(pkg.SEL_A, pkg.ATTN_A, q_ctx, ctx_max, q_dev, kv, sel, n_sel, a, b, t == 0,
                                     t == len(tiles) - 1, o_run, l_run, o_out_bf16=ob)
        torch.cuda.synchronize()
        if t == 0:
            # query 5 has no token in the first tile yet
            assert torch.all(torch.isneginf(l_run[5])) and torch.all(o_run[5] == 0)
        if t < len(tiles) - 1:
            assert torch.count_nonzero(ob.view(torch.int16)).item() == 0, "bf16 output before the last tile"
    o_run, l_run, o_r, l_r = o_run.cpu().numpy(), l_run.cpu().numpy(), o_ref.cpu().numpy(), l_ref.cpu().numpy()
    assert np.all(np.isfinite(l_run)) and np.max(np.abs(l_run - l_r)) <= 1e-5
    for i in range(nq):
        scale = np.max(np.abs(o_r[i]))
        assert np.max(np.abs(o_run[i] - o_r[i])) <= 1e-5 * scale, f"query {i}"
    obf = orc.bf16_to_f64(qc.from_dev_bits(ob))
    assert np.max(np.abs(obf - o_run)) <= 2.0**-8 * np.max(np.abs(o_run))
    # and against the oracle directly
    for i in (0, 5, nq - 1):
        toks = orc.selected_tokens(sels[i], ctxs[i], 4)
        o_o, l_o = orc.attend(q[i], k, v, toks, 1.0 / 16)
        qc.check_attention(o_run[i], l_run[i], o_o, l_o)


# --------------------------------------------------------------- errors ---

def test_argument_errors_raise(Q):
    pkg, _ = Q
    scores = torch.empty(2, 10, device="cuda")
    with pytest.raises(pkg.QsaError) as e:
        pkg.qsa_topk_blocks(pkg.SelCfg(4, 4096, 128, 1), qc.i32([40, 40]), 40, scores,
                            torch.empty(2, 4096, dtype=torch.int32, device="cuda"),
                            torch.empty(2, dtype=torch.int32, device="cuda"))
    assert e.value.status == 2
    with pytest.raises(pkg.QsaError) as e:
        pkg.qsa_topk_blocks(pkg.SEL_A, qc.i32([400, 40]), 400, scores,
                            torch.empty(2, 512, dtype=torch.int32, device="cuda"),
                            torch.empty(2, dtype=torch.int32, device="cuda"))
    assert e.value.status == 1  # ld_scores 10 < 100
