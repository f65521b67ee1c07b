"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times, on sampled queries the oracle computes one by one.

* The pooled-key prefill chunk: 4096 queries after a 60,000-token history,
  8192-token history tiles; i.i.d. inputs, and the correlated-selection
  workload (indexer queries AR(1) over positions, neighbouring selections
  overlapping about 0.72 as the pages measured), whose mean overlap over
  all 4096 GPU selections must match the one recorded by
  tests/golden/correlated_overlap.py.
* The shared-latent prefill chunk: 2048 queries at positions
  129,024..131,071, one history tile of 131,072 tokens.

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


@pytest.mark.parametrize("correlated", [False, True])
def test_prefill_full_size_sampled(Q, correlated):
    pkg, pipeline = Q
    from qsa_inputs.gpu import fill_normal_bf16
    H, C = 60000, 4096
    ctx_max = H + C
    seed = qi.config_seed(4)
    _print_case("prefill_full", correlated=correlated)
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
    bufs = pipeline.prefill_buffers(pkg.SEL_A, pkg.ATTN_A, C, ctx_max, 8192)
    pipeline.prefill_chunk(pkg.SEL_A, pkg.ATTN_A, qc.i32(ctxs), ctx_max, q_idx, pooled, q, kv, bufs)
    torch.cuda.synchronize()
    sel, n_sel = bufs.sel.cpu().numpy(), bufs.n_sel.cpu().numpy()
    o, lse, ob = bufs.o.cpu().numpy(), bufs.lse.cpu().numpy(), qc.from_dev_bits(bufs.o_bf16)
    pooled_np = orc.pool_keys(qi.normal_bf16(seed, S("raw_key"), 0, ctx_max * 128).reshape(ctx_max, 128), 4)
    assert np.array_equal(qc.from_dev_bits(pooled[0]), pooled_np)
    for i in (0, 1, 777, 2048, 3001, 4094, 4095):
        ctx = ctxs[i]
        sc = orc.index_scores(q_idx_np[i], pooled_np, ctx // 4)
        qc.check_selection(sel[i], n_sel[i], sc, ctx, 4, 512)
        toks = orc.selected_tokens(sel[i, :n_sel[i]], ctx, 4)
        kr = _rows(seed, S("k"), toks, 512).reshape(-1, 2, 256)
        vr = _rows(seed, S("v"), toks, 512).reshape(-1, 2, 256)
        qb = qi.normal_bf16(seed, S("q"), i * 4096, 4096).reshape(16, 256)
        o_ref, lse_ref = orc.attend(qb, kr, vr, np.arange(toks.size), 1.0 / 16)
        qc.check_attention(o[i], lse[i], o_ref, lse_ref, ob[i])
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
        qc.check_selection(sel[i], n_sel[i], sc, ctx, 1, 2048)
        toks = orc.selected_tokens(sel[i, :n_sel[i]], ctx, 1)
        lr = _rows(seed, S("latent"), toks, 576)[:, None, :]
        qb = qi.normal_bf16(seed, S("q"), i * 64 * 576, 64 * 576).reshape(64, 576)
        o_ref, lse_ref = orc.attend(qb, lr, lr, np.arange(toks.size), 1.0 / 24, dv=512)
        qc.check_attention(o[i], lse[i], o_ref, lse_ref, ob[i])
