"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times, on sampled queries the oracle computes one by one.

* The pooled-key prefill chunk: 4096 queries after a 60,000-token history,
  8192-token history tiles; i.i.d. inputs, and the correlated-selection
  workload (indexer queries AR(1) over positions, neighbouring selections
  overlapping about 0.72 as the pages measured), whose mean overlap over
  all 4096 GPU selections must match the one recorded by
  tests/golden/correlated_overlap.py.
* The pooled-key prefill chunk at 1024-token history tiles (63 tiles).
* The shared-latent prefill chunk: 2048 queries at positions
  129,024..131,071, one history tile of 131,072 tokens.
* The shared-latent decode step: batch 8 at context 131,072, every query
  (one with all-negative indexer head weights).

Inputs come from the seeded generator on the GPU exactly as bench.py makes
them; the oracle regenerates the keys in full and the K/V (latent) rows of
each sampled query's selection by index.
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
    pkg.qsa.lib()
    return pkg, pipeline


def _print_case(name, **kw):
    print(f"[case] {name} {kw}", flush=True)


def _golden(key):
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "correlated_overlap.txt")
    for line in open(path):
        if line.startswith(key + " "):
            return float(line.split()[1])
    raise KeyError(key)


def _rows(seed, stream, toks, width):
    """Rows `toks` of a [tokens][width] bf16 tensor filled by the generator."""
    idx = (np.asarray(toks, dtype=np.int64)[:, None] * width + np.arange(width)[None, :]).reshape(-1)
    return qi.normal_bf16(seed, stream, 0, index=idx.astype(np.uint64)).reshape(len(toks), width)


@pytest.mark.parametrize("correlated,tile", [(False, 8192), (False, 1024), (True, 8192)])
def test_prefill_full_size_sampled(Q, correlated, tile):
    pkg, pipeline = Q
    from qsa_inputs.gpu import fill_normal_bf16
    H, C = 60000, 4096
    ctx_max = H + C
    seed = qi.config_seed(4)
    _print_case("prefill_full", correlated=correlated, tile=tile)
    S = lambda kind, salt=0: qi.stream_id(0, 0, kind, salt)
    raw = torch.empty(1, ctx_max, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.empty(1, ctx_max, 2, 256, dtype=torch.bfloat16, device="cuda")
    v = torch.empty(1, ctx_max, 2, 256, dtype=torch.bfloat16, device="cuda")
    q = torch.empty(C, 16, 256, dtype=torch.bfloat16, device="cuda")
    for t, kind in ((raw, "raw_key"), (k, "k"), (v, "v"), (q, "q")):
        fill_normal_bf16(t, seed, S(kind))
    if correlated:
        q_idx_np = qi.ar1_normal_bf16(seed, S("q_idx", 1), C, 128, _golden("rho"))
        q_idx = qc.to_dev(q_idx_np[:, None, :])
    else:
        q_idx = torch.empty(C, 1, 128, dtype=torch.bfloat16, device="cuda")
        fill_normal_bf16(q_idx, seed, S("q_idx"))
        q_idx_np = qi.normal_bf16(seed, S("q_idx"), 0, C * 128).reshape(C, 128)
    pooled = torch.empty(1, ctx_max // 4, 128, dtype=torch.bfloat16, device="cuda")
    pkg.qsa_pool_keys(raw, pooled, block=4)
    kv = pkg.make_kv(k, v)
    ctxs = list(range(H + 1, H + C + 1))
    bufs = pipeline.prefill_buffers(pkg.SEL_A, pkg.ATTN_A, C, ctx_max, tile)
    pipeline.prefill_chunk(pkg.SEL_A, pkg.ATTN_A, qc.i32(ctxs), ctx_max, q_idx, pooled, q, kv, bufs)
    torch.cuda.synchronize()
    sel, n_sel = bufs.sel.cpu().numpy(), bufs.n_sel.cpu().numpy()
    o, lse, ob = bufs.o.cpu().numpy(), bufs.lse.cpu().numpy(), qc.from_dev_bits(bufs.o_bf16)
    pooled_np = orc.pool_keys(qi.normal_bf16(seed, S("raw_key"), 0, ctx_max * 128).reshape(ctx_max, 128), 4)
    assert np.array_equal(qc.from_dev_bits(pooled[0]), pooled_np)
    for i in (0, 1, 777, 2048, 3001, 4094, 4095):
        ctx = ctxs[i]
        sc = orc.index_scores(q_idx_np[i], pooled_np, ctx // 4)
        qb = qi.normal_bf16(seed, S("q"), i * 4096, 4096).reshape(16, 256)

        def attend_ref(toks, qb=qb):
            kr = _rows(seed, S("k"), toks, 512).reshape(-1, 2, 256)
            vr = _rows(seed, S("v"), toks, 512).reshape(-1, 2, 256)
            return orc.attend(qb, kr, vr, np.arange(toks.size), 1.0 / 16)

        qc.check_row_with(sel[i], n_sel[i], o[i], lse[i], ob[i], sc, ctx, 4, 512, attend_ref)
    if correlated:
        ov = np.mean([np.intersect1d(sel[i], sel[i - 1]).size / 512 for i in range(1, C)])
        assert abs(ov - _golden("mean_overlap_previous")) <= 0.005, ov


def test_mla_prefill_full_size_sampled(Q):
    pkg, pipeline = Q
    from qsa_inputs.gpu import fill_normal_bf16
    L, C = 131072, 2048
    seed = qi.config_seed(5)
    _print_case("mla_prefill_full")
    S = lambda kind: qi.stream_id(1, 0, kind)
    lat = torch.empty(1, L, 1, 576, dtype=torch.bfloat16, device="cuda")
    keys = torch.empty(1, L, 64, dtype=torch.bfloat16, device="cuda")
    q = torch.empty(C, 64, 576, dtype=torch.bfloat16, device="cuda")
    q_idx = torch.empty(C, 4, 64, dtype=torch.bfloat16, device="cuda")
    for t, kind in ((lat, "latent"), (keys, "raw_key"), (q, "q"), (q_idx, "q_idx")):
        fill_normal_bf16(t, seed, S(kind))
    w_np = qi.uniform_f32(seed, S("w_idx"), C * 4).reshape(C, 4)
    w = torch.tensor(w_np, device="cuda")
    kv = pkg.make_kv(lat, lat)
    ctxs = list(range(L - C + 1, L + 1))
    bufs = pipeline.prefill_buffers(pkg.SEL_B, pkg.ATTN_B, C, L, L)
    pipeline.prefill_chunk(pkg.SEL_B, pkg.ATTN_B, qc.i32(ctxs), L, q_idx, keys, q, kv, bufs, w_idx=w)
    torch.cuda.synchronize()
    sel, n_sel = bufs.sel.cpu().numpy(), bufs.n_sel.cpu().numpy()
    o, lse, ob = bufs.o.cpu().numpy(), bufs.lse.cpu().numpy(), qc.from_dev_bits(bufs.o_bf16)
    keys_np = qi.normal_bf16(seed, S("raw_key"), 0, L * 64).reshape(L, 64)
    for i in (0, 1023, 2046, 2047):
        ctx = ctxs[i]
        qi_np = qi.normal_bf16(seed, S("q_idx"), i * 256, 256).reshape(4, 64)
        sc = orc.index_scores_relu(qi_np, w_np[i], keys_np, ctx)
        qb = qi.normal_bf16(seed, S("q"), i * 64 * 576, 64 * 576).reshape(64, 576)

        def attend_ref(toks, qb=qb):
            lr = _rows(seed, S("latent"), toks, 576)[:, None, :]
            return orc.attend(qb, lr, lr, np.arange(toks.size), 1.0 / 24, dv=512)

        qc.check_row_with(sel[i], n_sel[i], o[i], lse[i], ob[i], sc, ctx, 1, 2048, attend_ref)


@pytest.mark.parametrize("fused", [False, True], ids=["separate_calls", "one_call"])
def test_mla_decode_full_size(Q, fused):
    """The shared-latent decode step as the benchmark times it: batch 8 at
    context 131,072, layer 0 of the workload's inputs, in its launch
    configuration (32 splits): the separate calls, or one
    qsa_decode_layer_latent call (which selects from the union of its
    512-token chunk lists). Every query is checked
    against the oracle: the whole score row (131,072 tokens) and the top-2048
    from the oracle's own scores, then the attention over the selected latent
    rows regenerated by index. Query 5's indexer head weights are all
    negative (the workload's draw): its best scores are exact zeros and its
    selection is the 2,048 smallest-index zero-score tokens."""
    pkg, pipeline = Q
    from qsa_inputs.gpu import fill_normal_bf16
    L, B = 131072, 8
    seed = qi.config_seed(5)
    _print_case("mla_decode_full", ctx=L, batch=B, fused=fused)
    S = lambda s, kind: qi.stream_id(0, s, kind)
    lat = torch.empty(B, L, 1, 576, dtype=torch.bfloat16, device="cuda")
    keys = torch.empty(B, L, 64, dtype=torch.bfloat16, device="cuda")
    q = torch.empty(B, 64, 576, dtype=torch.bfloat16, device="cuda")
    q_idx = torch.empty(B, 4, 64, dtype=torch.bfloat16, device="cuda")
    for s in range(B):
        for t, kind in ((lat, "latent"), (keys, "raw_key"), (q, "q"), (q_idx, "q_idx")):
            fill_normal_bf16(t[s], seed, S(s, kind))
    w_np = np.stack([qi.uniform_f32(seed, S(s, "w_idx"), 4) for s in range(B)])
    assert np.all(w_np[5] < 0), "the workload's query 5 has all-negative head weights"
    kv = pkg.make_kv(lat, lat)
    q_ctx, q_seq = qc.i32([L] * B), qc.i32(range(B))
    bufs = pipeline.decode_buffers(pkg.SEL_B, pkg.ATTN_B, B, L)
    assert bufs.n_split == 32
    assert bufs.latent_ws is not None
    pipeline.decode_layer(pkg.SEL_B, pkg.ATTN_B, q_ctx, L, q_idx, keys, q, kv, bufs, q_seq=q_seq,
                          w_idx=torch.tensor(w_np, device="cuda"), fused=fused)
    torch.cuda.synchronize()
    sel, n_sel = bufs.sel.cpu().numpy(), bufs.n_sel.cpu().numpy()
    o, lse, ob = bufs.o.cpu().numpy(), bufs.lse.cpu().numpy(), qc.from_dev_bits(bufs.o_bf16)
    got_sc = bufs.scores.cpu().numpy()
    for i in range(B):
        keys_np = qi.normal_bf16(seed, S(i, "raw_key"), 0, L * 64).reshape(L, 64)
        qi_np = qi.normal_bf16(seed, S(i, "q_idx"), 0, 256).reshape(4, 64)
        sc = orc.index_scores_relu(qi_np, w_np[i], keys_np, L)
        # fp32 accumulation of 64 exact products per head, then 4 weighted terms
        bound = 70 * 2.0 ** -24 * ((np.abs(orc.bf16_to_f64(keys_np)) @ np.abs(orc.bf16_to_f64(qi_np)).T)
                                   @ np.abs(w_np[i].astype(np.float64))) + 1e-30
        assert np.all(np.abs(got_sc[i, :L] - sc) <= bound), f"query {i}: scores"
        qb = qi.normal_bf16(seed, S(i, "q"), 0, 64 * 576).reshape(64, 576)

        def attend_ref(toks, qb=qb, i=i):
            lr = _rows(seed, S(i, "latent"), toks, 576)[:, None, :]
            return orc.attend(qb, lr, lr, np.arange(toks.size), 1.0 / 24, dv=512)

        qc.check_row_with(sel[i], n_sel[i], o[i], lse[i], ob[i], sc, L, 1, 2048, attend_ref)
        if i == 5:  # ties at zero, decided by index
            assert np.all(sc[sel[i, :n_sel[i]]] == 0.0)
