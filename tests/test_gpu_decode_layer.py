"""GPU parity of qsa_decode_layer (scan, top-k, attention and merge in one
launch) through the C ABI.

Checked against the oracle (selection bit-exact up to the boundary rule,
attention within the stated tolerances; where a tolerated swap occurred the
oracle attends over the GPU's selection) and against the separate calls
qsa_index_topk -> qsa_sparse_decode -> qsa_lse_merge on the same inputs
(scores, selection bit-exact; outputs within fp32 rounding). Cases: mixed
contexts (full attention, trailing tokens, empty), split counts 1..64, the
1,048,320-token batch-4 workload in the launch configuration the benchmark
times, repeated calls on one workspace, and HIP-graph replays.
"""
import numpy as np
import pytest
import torch

import qsa_inputs as qi
from oracle import qsa_oracle as orc
from tests import qsa_cases as qc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import indexer_selected_sparse_pooled_amd as pkg
    from indexer_selected_sparse_pooled_amd import pipeline
    pkg.qsa.lib()  # fails loudly if the library is missing
    return pkg, pipeline


def _print_case(name, **kw):
    print(f"[case] {name} {kw}", flush=True)


def _run(pkg, pipeline, ctxs, q_idx, pooled, q, kv, fused, n_split=None, bufs=None):
    nq, max_ctx = len(ctxs), max(max(ctxs), 4)
    if bufs is None:
        bufs = pipeline.decode_buffers(pkg.SEL_A, pkg.ATTN_A, nq, max_ctx, n_split=n_split)
        bufs.scores.fill_(float("nan"))
    pipeline.decode_layer(pkg.SEL_A, pkg.ATTN_A, qc.i32(ctxs), max_ctx, q_idx, pooled, q, kv, bufs,
                          q_seq=qc.i32(range(nq)), fused=fused)
    torch.cuda.synchronize()
    if fused:
        pkg.check_decode_layer_error(bufs.layer_ws)  # every bounded wait ended in time
    return bufs


def _same_as_separate(a, b, ctxs):
    """Fused and separate results on the same inputs: scores and selections
    bit-exact, outputs within fp32 rounding of the merge."""
    for i, ctx in enumerate(ctxs):
        n = ctx // 4
        assert torch.equal(a.scores[i, :n], b.scores[i, :n]), f"query {i}: scores"
    assert torch.equal(a.sel, b.sel) and torch.equal(a.n_sel, b.n_sel), "selection"
    la, lb = a.lse.cpu().numpy(), b.lse.cpu().numpy()
    assert np.array_equal(np.isneginf(la), np.isneginf(lb))
    live = ~np.isneginf(lb)
    assert np.max(np.abs(la[live] - lb[live]), initial=0.0) <= 1e-6
    oa, ob = a.o.cpu().numpy(), b.o.cpu().numpy()
    scale = np.max(np.abs(ob), axis=-1, keepdims=True) + 1e-30
    assert np.max(np.abs(oa - ob) / scale) <= 1e-5


def _check_against_oracle(bufs, refs, ctxs, q_bits, k_rows, v_rows):
    """refs[i]: oracle decode_query result; k_rows / v_rows(i, tokens) give
    the K / V rows of sequence i at those tokens."""
    sel, n_sel = bufs.sel.cpu().numpy(), bufs.n_sel.cpu().numpy()
    o, lse, ob = bufs.o.cpu().numpy(), bufs.lse.cpu().numpy(), qc.from_dev_bits(bufs.o_bf16)
    for i, r in enumerate(refs):
        if qc.check_selection(sel[i], n_sel[i], r["scores"], ctxs[i], 4, 512):
            o_ref, lse_ref = r["o"], r["lse"]
        else:  # tolerated boundary swap: attend over the GPU's selection
            toks = orc.selected_tokens(sel[i, :n_sel[i]], ctxs[i], 4)
            rows = np.arange(toks.size)
            o_ref, lse_ref = orc.attend(q_bits[i], k_rows(i, toks), v_rows(i, toks), rows, 1.0 / 16)
        qc.check_attention(o[i], lse[i], o_ref, lse_ref, ob[i])


@pytest.mark.parametrize("n_split", [1, 3, 32, 64])
def test_decode_layer_mixed_contexts(Q, n_split):
    """Full attention (ctx <= 2051), trailing tokens, an empty context and
    long contexts in one call."""
    pkg, pipeline = Q
    ctxs = [8195, 2051, 2052, 3, 0, 40000, 8192, 131071]
    _print_case("decode_layer_mixed", n_split=n_split)
    case = qc.DecodeCase(51, ctxs)
    refs = case.oracle()
    nq = case.nq
    pooled = torch.zeros(nq, case.cap // 4, 128, dtype=torch.bfloat16, device="cuda")
    pkg.qsa_pool_keys(qc.to_dev(case.raw), pooled, block=4)
    kv = pkg.make_kv(qc.to_dev(case.k), qc.to_dev(case.v))
    q_idx, q = qc.to_dev(case.q_idx[:, None, :]), qc.to_dev(case.q)
    fused = _run(pkg, pipeline, ctxs, q_idx, pooled, q, kv, True, n_split)
    assert fused.layer_ws is not None
    _check_against_oracle(fused, refs, ctxs, case.q, lambda i, t: case.k[i][t], lambda i, t: case.v[i][t])
    sep = _run(pkg, pipeline, ctxs, q_idx, pooled, q, kv, False, n_split)
    _same_as_separate(fused, sep, ctxs)
    assert torch.count_nonzero(fused.layer_ws[:64]).item() == 0, "control words not reset"


def _same_bits(a, b):
    for name in ("sel", "n_sel", "o", "o_bf16", "lse"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16_keys", "fp8_keys"])
def test_decode_layer_without_scores(Q, fp8):
    """qsa_decode_layer with no score buffer: the scan writes no scores, and
    every query whose selection does not come from the chunk lists (full
    attention, too few chunks for the union, ragged lengths) recomputes its
    scores from the keys, bit for bit the scan's. Results identical to the
    call with a score buffer; selections and outputs against the oracle
    (bf16 keys)."""
    pkg, pipeline = Q
    ctxs = [8195, 2051, 2052, 3, 0, 40000, 8192, 131071]
    _print_case("decode_layer_no_scores", ctxs=ctxs, fp8=fp8)
    case = qc.DecodeCase(51, ctxs)
    nq = case.nq
    pooled = torch.zeros(nq, case.cap // 4, 128, dtype=torch.bfloat16, device="cuda")
    pkg.qsa_pool_keys(qc.to_dev(case.raw), pooled, block=4)
    cfg = pkg.SEL_A_FP8 if fp8 else pkg.SEL_A
    keys = pooled
    if fp8:
        keys = pkg.fp8_keys_empty(nq, case.cap // 4, 128)
        pkg.qsa_quantize_keys(pooled, keys)
    kv = pkg.make_kv(qc.to_dev(case.k), qc.to_dev(case.v))
    q_idx, q = qc.to_dev(case.q_idx[:, None, :]), qc.to_dev(case.q)
    max_ctx = max(ctxs)
    out = []
    for keep in (True, False):
        bufs = pipeline.decode_buffers(cfg, pkg.ATTN_A, nq, max_ctx, keep_scores=keep)
        assert (bufs.scores is None) != keep
        pipeline.decode_layer(cfg, pkg.ATTN_A, qc.i32(ctxs), max_ctx, q_idx, keys, q, kv, bufs,
                              q_seq=qc.i32(range(nq)), fused=True)
        torch.cuda.synchronize()
        pkg.check_decode_layer_error(bufs.layer_ws)
        out.append(bufs)
    _same_bits(out[0], out[1])
    if not fp8:
        _check_against_oracle(out[1], case.oracle(), ctxs, case.q, lambda i, t: case.k[i][t],
                              lambda i, t: case.v[i][t])


@pytest.mark.parametrize("kind", ["tied_run", "graded_run"])
def test_decode_layer_without_scores_overflowing_lists(Q, kind):
    """Top blocks packed into a few chunks, so that a chunk's bound ranks
    above the 512th and the union check fails: with no score buffer the
    exact fallback recomputes the query's scores from the keys. Same bits as
    the call with a score buffer; the selection is the oracle's on the exact
    scores (the score is key dimension 0)."""
    pkg, pipeline = Q
    n_blk = 40000
    runs = {"tied_run": [(10003, 700, 8.0, 0.0)], "graded_run": [(5000, 600, 6.0, 2.0**-6)]}[kind]
    _print_case("decode_layer_no_scores_overflow", kind=kind)
    keys_np = qc.bits(47, 3, (n_blk, 128))
    for (b0, length, val, step) in runs:
        keys_np[b0:b0 + length, 0] = orc.f64_to_bf16(val + step * np.arange(length))
    keys = qc.to_dev(keys_np).unsqueeze(0)
    qv = np.zeros((1, 1, 128), dtype=np.uint16)
    qv[0, 0, 0] = 0x3F80  # 1.0: score = key dimension 0, exactly
    L = 4 * n_blk
    k = qc.to_dev(qc.bits(48, 1, (1, L, 2, 256)))
    v = qc.to_dev(qc.bits(48, 2, (1, L, 2, 256)))
    kv = pkg.make_kv(k, v)
    q = qc.to_dev(qc.bits(48, 3, (1, 16, 256)))
    out = []
    for keep in (True, False):
        bufs = pipeline.decode_buffers(pkg.SEL_A, pkg.ATTN_A, 1, L, keep_scores=keep)
        pipeline.decode_layer(pkg.SEL_A, pkg.ATTN_A, qc.i32([L]), L, qc.to_dev(qv), keys, q, kv, bufs,
                              q_seq=qc.i32([0]), fused=True)
        torch.cuda.synchronize()
        pkg.check_decode_layer_error(bufs.layer_ws)
        out.append(bufs)
    _same_bits(out[0], out[1])
    exact = orc.bf16_to_f64(keys_np[:, 0])
    want = orc.select_blocks(exact, L, 4, 512)
    assert np.array_equal(out[1].sel.cpu().numpy()[0], want)


def test_decode_layer_full_size_batch4(Q):
    """The 1,048,320-token, batch-4 workload in the benchmark's launch
    configuration (default split count). The layer's inputs (pooled keys,
    K, V, queries) come from the seeded generator on the GPU; the oracle
    regenerates them on the host (keys in full, K/V rows by index). Pooling
    itself is pinned bit-exact by its own tests."""
    pkg, pipeline = Q
    from qsa_inputs.gpu import fill_normal_bf16
    L, B = 1048320, 4
    nb = L // 4
    seed = qi.config_seed(3)
    _print_case("decode_layer_full", ctx=L, batch=B)
    keys = torch.empty(B, nb, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.empty(B, L, 2, 256, dtype=torch.bfloat16, device="cuda")
    v = torch.empty(B, L, 2, 256, dtype=torch.bfloat16, device="cuda")
    q = torch.empty(B, 16, 256, dtype=torch.bfloat16, device="cuda")
    q_idx = torch.empty(B, 1, 128, dtype=torch.bfloat16, device="cuda")
    for s in range(B):
        for t, kind in ((keys, "misc"), (k, "k"), (v, "v"), (q, "q"), (q_idx, "q_idx")):
            fill_normal_bf16(t[s], seed, qi.stream_id(0, s, kind))
    kv = pkg.make_kv(k, v)
    ctxs = [L] * B
    fused = _run(pkg, pipeline, ctxs, q_idx, keys, q, kv, True)
    assert fused.n_split == pipeline.default_n_split(B, 2, 512 * 4 + 3)

    def rows(i, toks, kind):
        idx = (toks[:, None, None] * 512 + np.arange(2)[None, :, None] * 256 + np.arange(256)[None, None, :])
        return qi.normal_bf16(seed, qi.stream_id(0, i, kind), 0, index=idx.reshape(-1).astype(np.uint64)).reshape(
            -1, 2, 256)

    refs, q_bits = [], []
    for s in range(B):
        keys_h = qi.normal_bf16(seed, qi.stream_id(0, s, "misc"), 0, nb * 128).reshape(nb, 128)
        qb = qi.normal_bf16(seed, qi.stream_id(0, s, "q"), 0, 16 * 256).reshape(16, 256)
        qib = qi.normal_bf16(seed, qi.stream_id(0, s, "q_idx"), 0, 128)
        sc = orc.index_scores(qib, keys_h, nb)
        sel = orc.select_blocks(sc, L, 4, 512)
        toks = orc.selected_tokens(sel, L, 4)
        o_ref, lse_ref = orc.attend(qb, rows(s, toks, "k"), rows(s, toks, "v"), np.arange(toks.size), 1.0 / 16)
        refs.append({"scores": sc, "o": o_ref, "lse": lse_ref})
        q_bits.append(qb)
        # the GPU's scores of this sequence against the fp64 oracle
        got = fused.scores[s, :nb].cpu().numpy().astype(np.float64)
        tol = qc.score_tolerance(qib, keys_h, nb)
        assert np.all(np.abs(got - sc) <= tol), f"sequence {s}: scores"
    _check_against_oracle(fused, refs, ctxs, q_bits, lambda i, t: rows(i, t, "k"), lambda i, t: rows(i, t, "v"))
    sep = _run(pkg, pipeline, ctxs, q_idx, keys, q, kv, False)
    _same_as_separate(fused, sep, ctxs)


def test_decode_layer_repeated_calls_and_graph(Q):
    """One workspace across calls with changing contexts (every counter
    resets itself), then the layer captured in a HIP graph and replayed
    with new contexts, eager work in between; each result equals the
    separate calls on the same inputs."""
    pkg, pipeline = Q
    cap = 300000
    case = qc.DecodeCase(53, [cap, cap, cap])
    nq = case.nq
    pooled = torch.zeros(nq, cap // 4, 128, dtype=torch.bfloat16, device="cuda")
    pkg.qsa_pool_keys(qc.to_dev(case.raw), pooled, block=4)
    kv = pkg.make_kv(qc.to_dev(case.k), qc.to_dev(case.v))
    q_idx, q = qc.to_dev(case.q_idx[:, None, :]), qc.to_dev(case.q)
    bufs = pipeline.decode_buffers(pkg.SEL_A, pkg.ATTN_A, nq, cap)
    rounds = [[cap, 250001, 2052], [9000, cap - 4, 100], [cap, cap, cap]]
    for rep, ctxs in enumerate(rounds):
        _print_case("decode_layer_repeat", rep=rep, ctxs=ctxs)
        pipeline.decode_layer(pkg.SEL_A, pkg.ATTN_A, qc.i32(ctxs), cap, q_idx, pooled, q, kv, bufs,
                              q_seq=qc.i32(range(nq)), fused=True)
        torch.cuda.synchronize()
        sep = _run(pkg, pipeline, ctxs, q_idx, pooled, q, kv, False)
        _same_as_separate(bufs, sep, ctxs)
        assert torch.count_nonzero(bufs.layer_ws[:64]).item() == 0, "control words not reset"

    q_ctx = qc.i32(rounds[0])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pipeline.decode_layer(pkg.SEL_A, pkg.ATTN_A, q_ctx, cap, q_idx, pooled, q, kv, bufs, q_seq=qc.i32(range(nq)),
                              fused=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    q_seq = qc.i32(range(nq))
    with torch.cuda.graph(g):
        pipeline.decode_layer(pkg.SEL_A, pkg.ATTN_A, q_ctx, cap, q_idx, pooled, q, kv, bufs, q_seq=q_seq, fused=True)
    for rep, ctxs in enumerate(rounds + rounds[:1]):
        _print_case("decode_layer_graph", rep=rep, ctxs=ctxs)
        q_ctx.copy_(qc.i32(ctxs))
        g.replay()
        torch.cuda.synchronize()
        sep = _run(pkg, pipeline, ctxs, q_idx, pooled, q, kv, False)  # eager work between replays
        _same_as_separate(bufs, sep, ctxs)
        assert torch.count_nonzero(bufs.layer_ws[:64]).item() == 0
    del g


def test_decode_layer_with_host_resident_kv(Q):
    """K/V rows in pinned host memory, read zero-copy over the host link
    (pooled keys stay in device memory): the same results, bit for bit, as
    with the K/V rows in device memory, for the one-call layer and for the
    separate calls."""
    pkg, pipeline = Q
    ctxs = [20000, 13333]
    _print_case("decode_layer_host_kv", ctxs=ctxs)
    case = qc.DecodeCase(31, ctxs)
    nq, max_ctx = len(ctxs), max(ctxs)
    pooled = torch.zeros(nq, case.cap // 4, 128, dtype=torch.bfloat16, device="cuda")
    pkg.qsa_pool_keys(qc.to_dev(case.raw), pooled, block=4)
    k_dev, v_dev = qc.to_dev(case.k), qc.to_dev(case.v)
    k_host = torch.empty(k_dev.shape, dtype=torch.bfloat16, pin_memory=True)
    v_host = torch.empty(v_dev.shape, dtype=torch.bfloat16, pin_memory=True)
    k_host.copy_(k_dev)
    v_host.copy_(v_dev)
    torch.cuda.synchronize()
    q_idx, q = qc.to_dev(case.q_idx[:, None, :]), qc.to_dev(case.q)
    for fused in (True, False):
        outs = []
        for kv in (pkg.make_kv(k_dev, v_dev), pkg.make_kv(k_host, v_host)):
            bufs = pipeline.decode_buffers(pkg.SEL_A, pkg.ATTN_A, nq, max_ctx)
            pipeline.decode_layer(pkg.SEL_A, pkg.ATTN_A, qc.i32(ctxs), max_ctx, q_idx, pooled, q, kv, bufs,
                                  q_seq=qc.i32(range(nq)), fused=fused)
            torch.cuda.synchronize()
            outs.append((bufs.sel.clone(), bufs.o.clone(), bufs.lse.clone()))
        for a, b in zip(*outs):
            assert torch.equal(a, b)


def test_host_kv_must_be_pinned(Q):
    pkg, _ = Q
    k = torch.zeros(1, 8, 2, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pkg.make_kv(k, k)


def test_two_stream_schedule_is_the_batch_step(Q):
    """The decode step as two micro-batches (sequences 0-1 and 2-3), each
    going through its layers in order on a stream of its own
    (pipeline.decode_step_streams), computes the batch-4 step: selections,
    outputs (fp32 and bf16) and lse bit-identical to one qsa_decode_layer
    call per layer over the whole batch. Checked eagerly and over graph
    replays with eager work between them."""
    pkg, pipeline = Q
    ctxs = [70000, 41003, 70000, 9002]
    cap = max(ctxs)
    n_layers, nq = 3, len(ctxs)
    layers, refs = [], []
    q_ctx, q_seq = qc.i32(ctxs), qc.i32(range(nq))
    for l in range(n_layers):
        case = qc.DecodeCase(90 + l, ctxs, cap=cap)
        pooled = torch.zeros(nq, case.cap // 4, 128, dtype=torch.bfloat16, device="cuda")
        pkg.qsa_pool_keys(qc.to_dev(case.raw), pooled, block=4)
        kv = pkg.make_kv(qc.to_dev(case.k), qc.to_dev(case.v))
        q_idx, q = qc.to_dev(case.q_idx[:, None, :]), qc.to_dev(case.q)
        layers.append((q_idx, pooled, q, kv))
        bf = pipeline.decode_buffers(pkg.SEL_A, pkg.ATTN_A, nq, cap)
        pipeline.decode_layer(pkg.SEL_A, pkg.ATTN_A, q_ctx, cap, q_idx, pooled, q, kv, bf, q_seq=q_seq, fused=True)
        refs.append(bf)
    torch.cuda.synchronize()
    n_split = refs[0].n_split
    micro = pipeline.micro_batches(pkg.SEL_A, pkg.ATTN_A, q_ctx, q_seq, cap, n_layers, 2, n_split=n_split)
    side = [torch.cuda.Stream()]

    def check(tag):
        for l, ref in enumerate(refs):
            for mb in micro:
                bf = mb.bufs[l]
                pkg.check_decode_layer_error(bf.layer_ws)
                for name in ("sel", "n_sel", "o", "o_bf16", "lse"):
                    got, want = getattr(bf, name), getattr(ref, name)[mb.lo:mb.hi]
                    assert torch.equal(got, want), f"{tag}: layer {l}, sequences {mb.lo}-{mb.hi - 1}: {name}"

    _print_case("two_stream_eager", ctxs=ctxs)
    pipeline.decode_step_streams(pkg.SEL_A, pkg.ATTN_A, cap, layers, micro, side)
    torch.cuda.synchronize()
    check("eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pipeline.decode_step_streams(pkg.SEL_A, pkg.ATTN_A, cap, layers, micro, side)
    for rep in range(3):
        _print_case("two_stream_graph", rep=rep)
        for mb in micro:
            for bf in mb.bufs:
                bf.o.zero_()
                bf.lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        check(f"graph replay {rep}")
        # eager work between replays: the batch call on layer 0 again
        pipeline.decode_layer(pkg.SEL_A, pkg.ATTN_A, q_ctx, cap, *layers[0], refs[0], q_seq=q_seq, fused=True)
        torch.cuda.synchronize()
    del g
