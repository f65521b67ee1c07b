"""GPU parity of the shared-latent variant (64 query heads over one 576-wide
bf16 latent row per token, V = its first 512 columns; token-level indexer of
4 heads x 64 dims with ReLU-weighted score sum, top 2,048 tokens) through
the C ABI, against the oracle.

Cases: attention on given selections with several split counts (full
attention at ctx <= 2048, one token, an empty context), the decode layer end
to end (scores, top-2048, attention, merge) through the separate calls and
through one qsa_decode_layer_latent call, a tiled prefill chunk whose
result must not depend on the tile size, and the single-tile chunk whose
result comes straight from the attention launch.
"""
import numpy as np
import pytest
import torch

import qsa_inputs as qi
from oracle import qsa_oracle as orc
from tests import qsa_cases as qc

pytestmark = pytest.mark.gpu

SCALE = 1.0 / 24.0  # 1 / sqrt(576)


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


class MlaCase:
    """nq sequences of one layer: latent rows, indexer keys, queries."""

    def __init__(self, seed, ctxs, cap=None):
        self.ctxs = list(ctxs)
        self.nq = len(ctxs)
        self.cap = (max(cap or max(ctxs), 8) + 7) // 8 * 8
        S = lambda s, kind: qi.stream_id(0, s, kind)
        self.latent = np.stack([qc.bits(seed, S(s, "latent"), (self.cap, 1, 576)) for s in range(self.nq)])
        self.keys = np.stack([qc.bits(seed, S(s, "raw_key"), (self.cap, 64)) for s in range(self.nq)])
        self.q = np.stack([qc.bits(seed, S(s, "q"), (64, 576)) for s in range(self.nq)])
        self.q_idx = np.stack([qc.bits(seed, S(s, "q_idx"), (4, 64)) for s in range(self.nq)])
        self.w = np.stack([qi.uniform_f32(seed, S(s, "w_idx"), 4) for s in range(self.nq)])

    def oracle(self, i):
        return orc.decode_query(self.q[i], self.q_idx[i], self.keys[i], self.latent[i], self.latent[i],
                                self.ctxs[i], block=1, topk=2048, scale=SCALE, w_idx=self.w[i], dv=512)


@pytest.mark.parametrize("n_split", [1, 5, 16, 32])
def test_mla_attention_on_given_selection(Q, n_split):
    pkg, _ = Q
    ctxs = [5000, 2048, 2049, 1, 0, 3001]
    _print_case("mla_attend", n_split=n_split)
    case = MlaCase(61, ctxs)
    nq = case.nq
    refs = [case.oracle(i) for i in range(nq)]
    sel = torch.full((nq, 2048), -1, dtype=torch.int32, device="cuda")
    n_sel = torch.zeros(nq, dtype=torch.int32, device="cuda")
    for i, r in enumerate(refs):
        sel[i, :r["sel"].size] = torch.tensor(r["sel"].astype(np.int32))
        n_sel[i] = int(r["sel"].size)
    lat = qc.to_dev(case.latent)
    kv = pkg.make_kv(lat, lat)
    o_part = torch.empty(n_split, nq, 64, 512, device="cuda")
    lse_part = torch.empty(n_split, nq, 64, device="cuda")
    pkg.qsa_sparse_decode(pkg.SEL_B, pkg.ATTN_B, qc.i32(ctxs), case.cap, qc.to_dev(case.q), kv, sel, n_sel, n_split,
                          o_part, lse_part, q_seq=qc.i32(range(nq)))
    o = torch.empty(nq, 64, 512, device="cuda")
    ob = torch.empty(nq, 64, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(nq, 64, device="cuda")
    pkg.qsa_lse_merge(o_part, lse_part, o_out=o, o_out_bf16=ob, lse_out=lse)
    torch.cuda.synchronize()
    o, lse, ob = o.cpu().numpy(), lse.cpu().numpy(), qc.from_dev_bits(ob)
    for i, r in enumerate(refs):
        qc.check_attention(o[i], lse[i], r["o"], r["lse"], ob[i])


def test_mla_decode_layer_end_to_end(Q):
    """Indexer scores (ReLU-weighted, 4 heads), top-2048 tokens, attention and
    merge through the pipeline's separate calls."""
    pkg, pipeline = Q
    ctxs = [20000, 2048, 2049, 7, 12345]
    _print_case("mla_decode_e2e", ctxs=ctxs)
    case = MlaCase(62, ctxs)
    nq = case.nq
    lat = qc.to_dev(case.latent)
    kv = pkg.make_kv(lat, lat)
    bufs = pipeline.decode_buffers(pkg.SEL_B, pkg.ATTN_B, nq, case.cap)
    assert bufs.layer_ws is None and bufs.latent_ws is not None
    pipeline.decode_layer(pkg.SEL_B, pkg.ATTN_B, qc.i32(ctxs), case.cap, qc.to_dev(case.q_idx), qc.to_dev(case.keys),
                          qc.to_dev(case.q), kv, bufs, q_seq=qc.i32(range(nq)),
                          w_idx=torch.tensor(case.w, device="cuda"))
    torch.cuda.synchronize()
    sel, n_sel = bufs.sel.cpu().numpy(), bufs.n_sel.cpu().numpy()
    o, lse, ob = bufs.o.cpu().numpy(), bufs.lse.cpu().numpy(), qc.from_dev_bits(bufs.o_bf16)
    for i in range(nq):
        r = case.oracle(i)
        qc.check_row(sel[i], n_sel[i], o[i], lse[i], ob[i], r, ctxs[i], 1, 2048, case.q[i], case.latent[i],
                     case.latent[i], SCALE, dv=512)


def _layer_both_ways(pkg, pipeline, case, n_split):
    """The decode layer through the separate calls and through one
    qsa_decode_layer_latent call, on the same inputs: both results."""
    nq = case.nq
    lat = qc.to_dev(case.latent)
    kv = pkg.make_kv(lat, lat)
    args = (qc.i32(case.ctxs), case.cap, qc.to_dev(case.q_idx), qc.to_dev(case.keys), qc.to_dev(case.q), kv)
    w = torch.tensor(case.w, device="cuda")
    out = []
    for fused in (False, True):
        bufs = pipeline.decode_buffers(pkg.SEL_B, pkg.ATTN_B, nq, case.cap, n_split=n_split)
        assert bufs.latent_ws is not None
        pipeline.decode_layer(pkg.SEL_B, pkg.ATTN_B, *args, bufs, q_seq=qc.i32(range(nq)), w_idx=w, fused=fused)
        torch.cuda.synchronize()
        out.append(dict(sel=bufs.sel.cpu().numpy(), n_sel=bufs.n_sel.cpu().numpy(), o=bufs.o.cpu().numpy(),
                        lse=bufs.lse.cpu().numpy(), ob=qc.from_dev_bits(bufs.o_bf16),
                        scores=bufs.scores.cpu().numpy()))
    return out


@pytest.mark.parametrize("n_split", [None, 3])
@pytest.mark.parametrize("which", ["short", "long"])
def test_mla_decode_layer_one_call(Q, which, n_split):
    """qsa_decode_layer_latent against the oracle and, bit for bit, against
    the separate calls, over every way its attention work-groups select:
    every token (ctx <= 2048), the register select straight over the scores
    (ctx <= 8192), the streamed select (too few chunk lists for the union),
    the union of the chunk lists (ctx > 65,024; one query ragged), and the
    fallback when a chunk's bound ranks above the union's 2048th (query with
    all-negative indexer weights: every score 0, ties decided by index)."""
    pkg, pipeline = Q
    ctxs = [0, 1, 2048, 2049, 8192, 8193, 20000] if which == "short" else [65536, 70001, 70001]
    _print_case("mla_decode_one_call", ctxs=ctxs, n_split=n_split)
    case = MlaCase(63, ctxs)
    if which == "long":
        case.w[2] = -np.abs(case.w[2]) - 0.125  # every score of query 2 is 0
    sep, one = _layer_both_ways(pkg, pipeline, case, n_split)
    for i, ctx in enumerate(ctxs):
        r = case.oracle(i)
        qc.check_row(one["sel"][i], one["n_sel"][i], one["o"][i], one["lse"][i], one["ob"][i], r, ctx, 1, 2048,
                     case.q[i], case.latent[i], case.latent[i], SCALE, dv=512)
        if which == "long" and i == 2:
            assert np.all(r["scores"][one["sel"][i, :2048]] == 0.0)
    for k in ("sel", "n_sel", "o", "lse", "ob"):
        assert np.array_equal(sep[k], one[k]), k
    for i, ctx in enumerate(ctxs):
        assert np.array_equal(sep["scores"][i, :ctx].view(np.uint32), one["scores"][i, :ctx].view(np.uint32))


@pytest.mark.parametrize("tile", [16384, 4096, 777])
def test_mla_prefill_chunk_tiled(Q, tile):
    """32 queries at positions 9000..9031 of one sequence: each selects its
    top-2048 among the tokens up to itself; history tiles in the outer loop,
    log-sum-exp merge; every row equals the oracle's decode at ctx = p + 1
    whatever the tile size."""
    pkg, pipeline = Q
    hist, nq = 9000, 32
    ctx_max = hist + nq
    _print_case("mla_prefill", tile=tile)
    seed = 63
    latent = qc.bits(seed, 1, (ctx_max, 1, 576))
    keys = qc.bits(seed, 2, (ctx_max, 64))
    q = qc.bits(seed, 3, (nq, 64, 576))
    q_idx = qc.bits(seed, 4, (nq, 4, 64))
    w = np.stack([qi.uniform_f32(seed, 100 + i, 4) for i in range(nq)])
    ctxs = [hist + i + 1 for i in range(nq)]
    lat = qc.to_dev(latent[None])
    kv = pkg.make_kv(lat, lat)
    bufs = pipeline.prefill_buffers(pkg.SEL_B, pkg.ATTN_B, nq, ctx_max, tile)
    pipeline.prefill_chunk(pkg.SEL_B, pkg.ATTN_B, qc.i32(ctxs), ctx_max, qc.to_dev(q_idx), qc.to_dev(keys[None]),
                           qc.to_dev(q), kv, bufs, w_idx=torch.tensor(w, device="cuda"))
    torch.cuda.synchronize()
    sel, n_sel = bufs.sel.cpu().numpy(), bufs.n_sel.cpu().numpy()
    o, lse, ob = bufs.o.cpu().numpy(), bufs.lse.cpu().numpy(), qc.from_dev_bits(bufs.o_bf16)
    for i in range(nq):
        r = orc.decode_query(q[i], q_idx[i], keys, latent, latent, ctxs[i], block=1, topk=2048, scale=SCALE,
                             w_idx=w[i], dv=512)
        qc.check_row(sel[i], n_sel[i], o[i], lse[i], ob[i], r, ctxs[i], 1, 2048, q[i], latent, latent, SCALE, dv=512)


def test_mla_prefill_single_tile_final(Q):
    """A chunk whose history is one tile takes O, lse and the bf16 copy
    straight from the attention (qsa_sparse_prefill_merge, first and last):
    bit for bit the result of qsa_sparse_prefill followed by a one-partial
    qsa_lse_merge. A shared-latent call that is not both first and last is
    refused."""
    pkg, pipeline = Q
    hist, nq = 5000, 24
    ctx_max = hist + nq
    _print_case("mla_prefill_single_tile", hist=hist, nq=nq)
    seed = 64
    latent = qc.bits(seed, 1, (ctx_max, 1, 576))
    keys = qc.bits(seed, 2, (ctx_max, 64))
    q = qc.to_dev(qc.bits(seed, 3, (nq, 64, 576)))
    q_idx = qc.to_dev(qc.bits(seed, 4, (nq, 4, 64)))
    w = torch.tensor(np.stack([qi.uniform_f32(seed, 100 + i, 4) for i in range(nq)]), device="cuda")
    q_ctx = qc.i32([hist + i + 1 for i in range(nq)])
    lat = qc.to_dev(latent[None])
    kv = pkg.make_kv(lat, lat)
    bufs = pipeline.prefill_buffers(pkg.SEL_B, pkg.ATTN_B, nq, ctx_max, ctx_max)
    assert len(bufs.tiles) == 1 and pipeline.single_tile_final(pkg.SEL_B, pkg.ATTN_B, kv, 1)
    pipeline.prefill_chunk(pkg.SEL_B, pkg.ATTN_B, q_ctx, ctx_max, q_idx, qc.to_dev(keys[None]), q, kv, bufs, w_idx=w)
    torch.cuda.synchronize()
    one = {k: getattr(bufs, k).clone() for k in ("o", "lse", "o_bf16")}
    a0, a1 = bufs.tiles[0]
    pkg.qsa_sparse_prefill(pkg.SEL_B, pkg.ATTN_B, q_ctx, ctx_max, q, kv, bufs.sel, bufs.n_sel, a0, a1,
                           bufs.o_tiles[0], bufs.lse_tiles[0])
    pkg.qsa_lse_merge(bufs.o_tiles, bufs.lse_tiles, o_out=bufs.o, o_out_bf16=bufs.o_bf16, lse_out=bufs.lse)
    torch.cuda.synchronize()
    for k, v in one.items():
        assert torch.equal(v, getattr(bufs, k)), k
    with pytest.raises(pkg.QsaError):
        pkg.qsa_sparse_prefill_merge(pkg.SEL_B, pkg.ATTN_B, q_ctx, ctx_max, q, kv, bufs.sel, bufs.n_sel, a0, a1,
                                     True, False, bufs.o, bufs.lse)
