"""GPU checks of qsa_index_topk_prefill (A2 + A3 of a prefill chunk of the
token-level indexer without materialising the scores) through the C ABI.

The selections must equal those of qsa_index_scores + qsa_topk_blocks on the
same inputs, bit for bit (that path is checked against the oracle in the
other GPU tests; here a few rows are also checked against the oracle
directly). Cases: mixed contexts (empty, at most topk, at most the list
capacity, long), queries whose head weights are all negative (their best
scores are exact zeros, so the top-2048 is decided by index among ties),
FP8 keys, a chunk whose queries all fit the list and the largest context
the path takes (262,144 keys), repeated calls on one workspace, HIP-graph
replays, and inputs
planted so that the sampled threshold fails both ways: sampled keys that
score far above the rest (too few candidates) and unsampled keys that do
(too many). Those queries must take the regular path, and only their score
rows may be written (the buffer is pre-filled with NaN).
"""
import numpy as np
import pytest
import torch

import qsa_inputs as qi
from oracle import qsa_oracle as orc
from tests import qsa_cases as qc

pytestmark = pytest.mark.gpu

TOPK = 2048


@pytest.fixture(scope="module")
def Q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import indexer_selected_sparse_pooled_amd as pkg
    pkg.qsa.lib()  # fails loudly if the library is missing
    return pkg


def _print_case(name, **kw):
    print(f"[case] {name} {kw}", flush=True)


def _both(pkg, cfg, ctxs, max_ctx, q_idx, w, keys):
    """(fused sel, n_sel, scores after the fused call), (reference sel, n_sel)."""
    nq = len(ctxs)
    q_ctx = qc.i32(ctxs)
    scores = torch.full((nq, max_ctx), float("nan"), device="cuda")
    sel = torch.full((nq, TOPK), -7, dtype=torch.int32, device="cuda")
    n_sel = torch.full((nq,), -7, dtype=torch.int32, device="cuda")
    ws = pkg.index_topk_prefill_workspace(cfg, nq, max_ctx)
    assert ws is not None
    pkg.qsa_index_topk_prefill(cfg, q_ctx, max_ctx, q_idx, w, keys, scores, sel, n_sel, ws)
    torch.cuda.synchronize()
    fused = (sel.cpu().numpy(), n_sel.cpu().numpy(), scores.cpu().numpy())
    scores_r = torch.empty(nq, max_ctx, device="cuda")
    sel_r = torch.full((nq, TOPK), -7, dtype=torch.int32, device="cuda")
    n_sel_r = torch.full((nq,), -7, dtype=torch.int32, device="cuda")
    pkg.qsa_index_scores(cfg, q_ctx, max_ctx, q_idx, keys, scores_r, w_idx=w)
    pkg.qsa_topk_blocks(cfg, q_ctx, max_ctx, scores_r, sel_r, n_sel_r, pkg.topk_workspace(cfg, nq, max_ctx))
    torch.cuda.synchronize()
    return fused, (sel_r.cpu().numpy(), n_sel_r.cpu().numpy())


def _assert_same(fused, ref):
    assert np.array_equal(fused[1], ref[1]), "n_sel"
    assert np.array_equal(fused[0], ref[0]), "sel"


def _inputs(seed, nq, max_ctx, neg_rows=()):
    keys = qc.bits(seed, 1, (max_ctx, 64))
    q_idx = qc.bits(seed, 2, (nq, 4, 64))
    w = np.stack([qi.uniform_f32(seed, 100 + i, 4) for i in range(nq)])
    for i in neg_rows:
        w[i] = -np.abs(w[i]) - np.float32(0.01)
    return keys, q_idx, w.astype(np.float32)


def test_mixed_contexts_and_ties(Q):
    pkg = Q
    max_ctx = 40000
    rng = np.random.default_rng(5)
    ctxs = [0, 1, 100, 2047, 2048, 2049, 5000, 8192, 8193, 9001, 40000, 39999, 20000]
    ctxs += list(rng.integers(8200, 40001, 35))
    nq = len(ctxs)
    neg = (3, 9, 10, 20, 33)
    _print_case("prefill_select_mixed", nq=nq, max_ctx=max_ctx, neg_rows=neg)
    keys, q_idx, w = _inputs(71, nq, max_ctx, neg)
    fused, ref = _both(pkg, pkg.SEL_B, ctxs, max_ctx, qc.to_dev(q_idx), torch.tensor(w, device="cuda"),
                       qc.to_dev(keys[None]))
    _assert_same(fused, ref)
    for i in (9, 10, 11, 20, 40):  # direct oracle check (9, 10, 20 all-negative weights)
        sc = orc.index_scores_relu(q_idx[i], w[i], keys, ctxs[i])
        qc.check_selection(fused[0][i], fused[1][i], sc, ctxs[i], 1, TOPK)
    # no query here needed the regular path: no score row was written
    assert np.all(np.isnan(fused[2])), "scores were written"


def test_fp8_keys(Q):
    pkg = Q
    max_ctx = 30000
    ctxs = [30000 - 7 * i for i in range(24)] + [500, 9000]
    nq = len(ctxs)
    _print_case("prefill_select_fp8", nq=nq, max_ctx=max_ctx)
    keys, q_idx, w = _inputs(72, nq, max_ctx, (4,))
    kd = qc.to_dev(keys[None])
    k8 = pkg.fp8_keys_empty(1, max_ctx, 64)
    pkg.qsa_quantize_keys(kd, k8)
    fused, ref = _both(pkg, pkg.SEL_B_FP8, ctxs, max_ctx, qc.to_dev(q_idx), torch.tensor(w, device="cuda"), k8)
    _assert_same(fused, ref)
    # end to end: the oracle quantizes the bf16 keys itself, scores them and
    # selects; every query's selection must be the oracle's (boundary rule)
    codes, scales = orc.fp8_keys(keys)
    for i, ctx in enumerate(ctxs):
        sc = orc.index_scores_relu_fp8(q_idx[i], w[i], codes, scales, ctx)
        qc.check_selection(fused[0][i], fused[1][i], sc, ctx, 1, TOPK)


def _planted(seed, nq, max_ctx, sampled_high):
    """Keys whose dim 0 is +8 on the planted positions and -8 elsewhere, the
    rest small noise; queries with dim 0 = 4 in every head and positive
    weights: planted keys score about 32 x sum(w), the others exactly 0.
    Planted: the sampled positions (multiples of the sample stride) or the
    others."""
    step = -(-max_ctx // 4096)
    pos = np.arange(max_ctx)
    on = (pos % step == 0) if sampled_high else (pos % step != 0)
    kv = orc.bf16_to_f64(qc.bits(seed, 1, (max_ctx, 64))) * 0.1
    kv[:, 0] = np.where(on, 8.0, -8.0)
    qv = orc.bf16_to_f64(qc.bits(seed, 2, (nq, 4, 64))) * 0.1
    qv[:, :, 0] = 4.0
    w = np.stack([0.5 + 0.5 * qi.uniform_f32(seed, 100 + i, 4) ** 2 for i in range(nq)]).astype(np.float32)
    return orc.f64_to_bf16(kv), orc.f64_to_bf16(qv), w


@pytest.mark.parametrize("sampled_high", [True, False])
def test_threshold_failure_takes_the_regular_path(Q, sampled_high):
    pkg = Q
    max_ctx = 40000
    ctxs = [40000 - 3 * i for i in range(16)] + [3000, 7000]
    nq = len(ctxs)
    _print_case("prefill_select_fallback", sampled_high=sampled_high)
    keys, q_idx, w = _planted(73, nq, max_ctx, sampled_high)
    fused, ref = _both(pkg, pkg.SEL_B, ctxs, max_ctx, qc.to_dev(q_idx), torch.tensor(w, device="cuda"),
                       qc.to_dev(keys[None]))
    _assert_same(fused, ref)
    written = ~np.all(np.isnan(fused[2]), axis=1)
    # the long queries fail the sampled threshold; the two short ones keep every key
    assert written[:16].all() and not written[16:].any(), written
    sc = orc.index_scores_relu(q_idx[0], w[0], keys, ctxs[0])
    qc.check_selection(fused[0][0], fused[1][0], sc, ctxs[0], 1, TOPK)


def test_repeated_calls_and_graph_replays(Q):
    pkg = Q
    max_ctx = 20000
    ctxs = [20000 - 11 * i for i in range(32)]
    nq = len(ctxs)
    _print_case("prefill_select_graph", nq=nq)
    keys, q_idx, w = _inputs(74, nq, max_ctx, (0, 5))
    q_ctx, qd, wd, kd = qc.i32(ctxs), qc.to_dev(q_idx), torch.tensor(w, device="cuda"), qc.to_dev(keys[None])
    scores = torch.empty(nq, max_ctx, device="cuda")
    sel = torch.empty(nq, TOPK, dtype=torch.int32, device="cuda")
    n_sel = torch.empty(nq, dtype=torch.int32, device="cuda")
    ws = pkg.index_topk_prefill_workspace(pkg.SEL_B, nq, max_ctx)

    def call():
        pkg.qsa_index_topk_prefill(pkg.SEL_B, q_ctx, max_ctx, qd, wd, kd, scores, sel, n_sel, ws)

    call()
    torch.cuda.synchronize()
    want = (sel.clone(), n_sel.clone())
    call()
    torch.cuda.synchronize()
    assert torch.equal(sel, want[0]) and torch.equal(n_sel, want[1])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    for _ in range(3):
        sel.fill_(-5)
        n_sel.fill_(-5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sel, want[0]) and torch.equal(n_sel, want[1])
    del g


def test_argument_errors(Q):
    pkg = Q
    keys = torch.zeros(1, 1000, 64, dtype=torch.bfloat16, device="cuda")
    q_idx = torch.zeros(8, 4, 64, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(8, 4, device="cuda")
    scores = torch.empty(8, 1000, device="cuda")
    sel = torch.empty(8, TOPK, dtype=torch.int32, device="cuda")
    n_sel = torch.empty(8, dtype=torch.int32, device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(pkg.QsaError):  # fewer than 16 queries
        pkg.qsa_index_topk_prefill(pkg.SEL_B, qc.i32([1000] * 8), 1000, q_idx, w, keys, scores, sel, n_sel, ws)
    assert pkg.qsa_index_topk_prefill_workspace_bytes(pkg.SEL_B, 16, 300000) == 0
    assert pkg.qsa_index_topk_prefill_workspace_bytes(pkg.SEL_B, 16, 131072) > 0


@pytest.mark.parametrize("max_ctx,ctxs", [
    (3000, [3000 - 37 * i for i in range(16)]),             # every query's keys fit the list (stride 1)
    (262144, [262144 - 1000 * i for i in range(15)] + [9000]),  # the path's largest context (full bitmap)
])
def test_context_extremes(Q, max_ctx, ctxs):
    pkg = Q
    nq = len(ctxs)
    _print_case("prefill_select_extremes", max_ctx=max_ctx, nq=nq)
    keys, q_idx, w = _inputs(75, nq, max_ctx, (1,))
    fused, ref = _both(pkg, pkg.SEL_B, ctxs, max_ctx, qc.to_dev(q_idx), torch.tensor(w, device="cuda"),
                       qc.to_dev(keys[None]))
    _assert_same(fused, ref)
    assert np.all(np.isnan(fused[2])), "a query took the regular path"
    i = nq - 1
    sc = orc.index_scores_relu(q_idx[i], w[i], keys, ctxs[i])
    qc.check_selection(fused[0][i], fused[1][i], sc, ctxs[i], 1, TOPK)
