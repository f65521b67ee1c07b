"""GPU parity of the FP8 indexer keys (OCP E4M3 codes with one fp32 scale
per key, stored in pages of 64) through the C ABI.

* qsa_quantize_keys writes the oracle's codes and scales bit for bit
  (fp8_keys: scale = amax / 448, code = nearest-even E4M3 of the fp32
  quotient), including all-zero keys, negative zeros, subnormal codes and
  saturating magnitudes, and nothing outside the requested key range.
* qsa_kv_append with FP8 pooled keys writes, for every completed block,
  the quantized pooled key bit for bit.
* qsa_index_scores (decode stream and prefill MFMA paths) agrees with the
  oracle's scores over the dequantized keys within the fp32 accumulation
  bound.
* qsa_index_topk, qsa_index_lists and qsa_decode_layer with FP8 keys: the
  same scores bit for bit as qsa_index_scores; on the 1,048,320-token
  batch-4 shape, end to end against the oracle, which quantizes the
  regenerated bf16 keys itself: its selection on its own scores (boundary
  rule) and its attention over the selected tokens.
"""
import numpy as np
import pytest
import torch

import qsa_inputs as qi
from oracle import qsa_oracle as orc
from tests import qsa_cases as qc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import indexer_selected_sparse_pooled_amd as p
    p.qsa.lib()
    return p


def _print_case(name, **kw):
    print(f"[case] {name} {kw}", flush=True)


def _special_keys(dim, seed):
    """N(0,1) keys with rows that reach the corners of the format."""
    k = qc.bits(seed, 1, (300, dim))
    k[5] = 0                                                  # all zero: scale 0
    k[6] = 0x8000                                             # negative zeros
    rng = np.random.default_rng(seed)
    k[7] = orc.f64_to_bf16(rng.normal(0, 1e-6, dim))
    k[7, 3] = orc.f64_to_bf16(1e4)[0]                         # one huge value: the rest subnormal or zero
    k[8] = orc.f64_to_bf16(rng.normal(0, 1, dim) * 2.0 ** -9)  # tiny but normal scale
    k[9] = orc.f64_to_bf16(np.full(dim, -3.0))                # every value at -448 * scale
    k[10] = orc.f64_to_bf16(rng.uniform(-1, 1, dim) * np.array([1.0, 1e-5] * (dim // 2)))
    return k


@pytest.mark.parametrize("dim", [128, 64])
def test_quantize_keys_bit_exact(pkg, dim):
    _print_case("quantize_keys", dim=dim)
    keys_np = np.stack([_special_keys(dim, 61), qc.bits(62, 2, (300, dim))])
    keys = qc.to_dev(keys_np)
    out = pkg.fp8_keys_empty(2, 300, dim)
    pkg.qsa_quantize_keys(keys, out)
    torch.cuda.synchronize()
    buf = out.cpu().numpy()
    for s in range(2):
        codes, scales = qc.unpack_fp8_pages(buf[s], 300, dim)
        want_c, want_s = orc.fp8_keys(keys_np[s])
        assert np.array_equal(scales.view(np.uint32), want_s.view(np.uint32)), f"sequence {s}: scales"
        bad = np.argwhere(codes != want_c)
        assert bad.size == 0, f"sequence {s}: codes differ at {bad[:8].tolist()}"
    # a sub-range writes exactly its own keys
    part = pkg.fp8_keys_empty(2, 300, dim)
    pkg.qsa_quantize_keys(keys, part, key_begin=70, key_end=251)
    torch.cuda.synchronize()
    pb = part.cpu().numpy()
    for s in range(2):
        codes, scales = qc.unpack_fp8_pages(pb[s], 300, dim)
        full_c, full_s = qc.unpack_fp8_pages(buf[s], 300, dim)
        assert np.array_equal(codes[70:251], full_c[70:251]) and np.array_equal(scales[70:251], full_s[70:251])
        assert not codes[:70].any() and not codes[251:].any()
        assert not scales[:70].any() and not scales[251:].any()


def test_append_fp8_pooled_keys(pkg):
    cap, n_seq = 64, 2
    seed = qi.config_seed(1) + 91
    k = torch.zeros(n_seq, cap, 2, 256, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    raw_np = qc.bits(seed, 3, (n_seq, cap, 128))
    raw_np[1, 8:12] = 0  # a block whose pooled key is zero
    raw = qc.to_dev(raw_np)
    pooled = pkg.fp8_keys_empty(n_seq, cap // 4, 128)
    kv = pkg.make_kv(k, v)
    start = [9, 5]
    raw_cur = raw_np.copy()
    for step in range(14):
        pos = [p + step for p in start]
        _print_case("append_fp8", step=step, pos=pos)
        new_np = qc.bits(seed + 1, 10 + step, (n_seq, 128))
        if step in (1, 2, 3, 4):
            new_np[1] = 0
        rows = qc.to_dev(np.zeros((n_seq, 2, 256), dtype=np.uint16))
        pkg.qsa_kv_append(pkg.SEL_A_FP8, pkg.ATTN_A, qc.i32(pos), rows, kv, v_new=rows, raw_new=qc.to_dev(new_np),
                          raw_keys=raw, pooled=pooled)
        torch.cuda.synchronize()
        for s in range(n_seq):
            raw_cur[s, pos[s]] = new_np[s]
        buf = pooled.cpu().numpy()
        for s in range(n_seq):
            nb = (pos[s] + 1) // 4
            done = [b for b in range(nb) if 4 * b + 3 >= start[s]]  # blocks completed by an append
            if not done:
                continue
            codes, scales = qc.unpack_fp8_pages(buf[s], nb, 128)
            want_c, want_s = orc.fp8_keys(orc.pool_keys(raw_cur[s, :4 * nb], 4))
            assert np.array_equal(codes[done], want_c[done]), f"seq {s} step {step}: codes"
            assert np.array_equal(scales[done].view(np.uint32), want_s[done].view(np.uint32)), f"seq {s}: scales"


def _fp8_keys_dev(pkg, keys):
    """FP8 pages of bf16 device keys [n_seq, n, 128] (the quantizer is pinned
    bit-exact above)."""
    out = pkg.fp8_keys_empty(keys.shape[0], keys.shape[1], 128)
    pkg.qsa_quantize_keys(keys, out)
    return out


def _fp8_tolerance(q_bits, codes, scales, n):
    q = orc.bf16_to_f64(q_bits)
    k = orc.dequantize_e4m3(codes[:n], scales[:n, None], 128)
    return 130 * 2.0 ** -24 * (np.abs(k) @ np.abs(q)) + 1e-30


def test_fp8_scores_decode_and_prefill(pkg):
    n_blk = 20000
    keys_np = np.stack([qc.bits(63, s, (n_blk, 128)) for s in range(2)])
    keys = qc.to_dev(keys_np)
    f8 = _fp8_keys_dev(pkg, keys)
    ref_keys = [orc.fp8_keys(keys_np[s]) for s in range(2)]
    # decode path: queries on their own sequences
    ctxs = [4 * n_blk, 33, 4 * n_blk - 3, 2052, 0, 257]
    q_seq = [0, 1, 0, 1, 0, 1]
    q_np = qc.bits(64, 1, (len(ctxs), 1, 128))
    _print_case("fp8_scores_decode", ctxs=ctxs)
    max_ctx = 4 * n_blk
    sc = torch.full((len(ctxs), n_blk + 3), float("nan"), device="cuda")
    pkg.qsa_index_scores(pkg.SEL_A_FP8, qc.i32(ctxs), max_ctx, qc.to_dev(q_np), f8, sc, q_seq=qc.i32(q_seq))
    torch.cuda.synchronize()
    got = sc.cpu().numpy()
    for i, ctx in enumerate(ctxs):
        n = ctx // 4
        c, s = ref_keys[q_seq[i]]
        ref = orc.index_scores_fp8(q_np[i, 0], c, s, n)
        assert np.all(np.abs(got[i, :n] - ref) <= _fp8_tolerance(q_np[i, 0], c, s, n)), f"query {i}"
        assert np.all(np.isnan(got[i, n:])), f"query {i}: wrote past the candidates"
    # prefill path: a chunk of queries of sequence 0 (MFMA tiles)
    rng = np.random.default_rng(65)
    ctxs = [int(x) for x in rng.integers(0, 4 * n_blk + 1, 37)] + [4 * n_blk, 0, 5]
    q_np = qc.bits(66, 1, (len(ctxs), 1, 128))
    _print_case("fp8_scores_prefill", nq=len(ctxs))
    sc = torch.full((len(ctxs), n_blk), float("nan"), device="cuda")
    pkg.qsa_index_scores(pkg.SEL_A_FP8, qc.i32(ctxs), max_ctx, qc.to_dev(q_np), f8[0:1], sc)
    torch.cuda.synchronize()
    got = sc.cpu().numpy()
    c, s = ref_keys[0]
    for i, ctx in enumerate(ctxs):
        n = ctx // 4
        ref = orc.index_scores_fp8(q_np[i, 0], c, s, n)
        assert np.all(np.abs(got[i, :n] - ref) <= _fp8_tolerance(q_np[i, 0], c, s, n)), f"query {i}"
        assert np.all(np.isnan(got[i, n:]))


def test_fp8_select_and_decode_layer_full_size(pkg):
    """The 1,048,320-token batch-4 decode shape with FP8 pooled keys: the
    fused scan + top-k, the lists-only scan and the decode layer agree with
    qsa_index_scores + qsa_topk_blocks bit for bit; against the oracle, end
    to end: the oracle regenerates the bf16 keys on the host and quantizes
    them itself (the GPU's pages must equal its codes and scales), scores
    them, and the GPU selection must be the oracle's selection on the
    oracle's scores (boundary rule), the GPU scores within the accumulation
    bound, and the attention output the oracle's on the selected tokens
    (K/V rows regenerated by index). Mixed contexts in a second call take
    the other selection paths."""
    from indexer_selected_sparse_pooled_amd import pipeline
    from qsa_inputs.gpu import fill_normal_bf16
    L, B = 1048320, 4
    nb = L // 4
    seed = qi.config_seed(3) + 17
    S = lambda s, kind: qi.stream_id(0, s, kind)
    _print_case("fp8_decode_full", ctx=L, batch=B)
    keys = torch.empty(B, nb, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.empty(B, L, 2, 256, dtype=torch.bfloat16, device="cuda")
    v = torch.empty(B, L, 2, 256, dtype=torch.bfloat16, device="cuda")
    q = torch.empty(B, 16, 256, dtype=torch.bfloat16, device="cuda")
    q_idx = torch.empty(B, 1, 128, dtype=torch.bfloat16, device="cuda")
    for s in range(B):
        for t, kind in ((keys, "misc"), (k, "k"), (v, "v"), (q, "q"), (q_idx, "q_idx")):
            fill_normal_bf16(t[s], seed, S(s, kind))
    f8 = _fp8_keys_dev(pkg, keys)
    del keys
    kv = pkg.make_kv(k, v)
    cfg, acfg = pkg.SEL_A_FP8, pkg.ATTN_A
    # the oracle's own inputs: regenerated on the host, quantized by the oracle
    ref_keys = [orc.fp8_keys(qc.bits(seed, S(s, "misc"), (nb, 128))) for s in range(B)]
    q_idx_np = [qc.bits(seed, S(s, "q_idx"), (128,)) for s in range(B)]
    q_np = [qc.bits(seed, S(s, "q"), (16, 256)) for s in range(B)]
    f8h = f8.cpu().numpy()
    for s in range(B):
        c, scl = qc.unpack_fp8_pages(f8h[s], nb, 128)
        assert np.array_equal(c, ref_keys[s][0]), f"seq {s}: FP8 codes differ from the oracle's"
        assert np.array_equal(scl.view(np.uint32), ref_keys[s][1].view(np.uint32)), f"seq {s}: scales"
    del f8h
    for ctxs in ([L] * B, [L - 4001, 2052, 600004, 9001]):
        _print_case("fp8_decode_full_ctxs", ctxs=ctxs)
        q_ctx, q_seq = qc.i32(ctxs), qc.i32(range(B))
        bufs = pipeline.decode_buffers(cfg, acfg, B, L)
        bufs.scores.fill_(float("nan"))
        pipeline.decode_layer(cfg, acfg, q_ctx, L, q_idx, f8, q, kv, bufs, q_seq=q_seq, fused=True)
        sc = torch.full_like(bufs.scores, float("nan"))
        pkg.qsa_index_scores(cfg, q_ctx, L, q_idx, f8, sc, q_seq=q_seq)
        sel = torch.full((B, 512), -7, dtype=torch.int32, device="cuda")
        n_sel = torch.zeros(B, dtype=torch.int32, device="cuda")
        pkg.qsa_topk_blocks(cfg, q_ctx, L, sc, sel, n_sel, pkg.topk_workspace(cfg, B, L))
        sc2 = torch.full_like(sc, float("nan"))
        sel2 = torch.full_like(sel, -7)
        n_sel2 = torch.zeros_like(n_sel)
        pkg.qsa_index_topk(cfg, q_ctx, L, q_idx, f8, sc2, sel2, n_sel2, pkg.index_topk_workspace(cfg, B, L),
                           q_seq=q_seq)
        sc3 = torch.full_like(sc, float("nan"))
        pkg.qsa_index_lists(cfg, q_ctx, L, q_idx, f8, sc3, pkg.index_topk_workspace(cfg, B, L), q_seq=q_seq)
        torch.cuda.synchronize()
        pkg.check_decode_layer_error(bufs.layer_ws)
        for name, t in (("decode_layer", bufs.scores), ("index_topk", sc2), ("index_lists", sc3)):
            assert torch.equal(t.nan_to_num(7.0), sc.nan_to_num(7.0)), f"{name}: scores differ"
        for name, (a, b) in (("decode_layer", (bufs.sel, bufs.n_sel)), ("index_topk", (sel2, n_sel2))):
            assert torch.equal(a, sel) and torch.equal(b, n_sel), f"{name}: selection differs"
        got_sc, got_sel, got_n = sc.cpu().numpy(), sel.cpu().numpy(), n_sel.cpu().numpy()
        o, lse, ob = bufs.o.cpu().numpy(), bufs.lse.cpu().numpy(), qc.from_dev_bits(bufs.o_bf16)
        for s, ctx in enumerate(ctxs):
            n = ctx // 4
            c, scl = ref_keys[s]
            ref = orc.index_scores_fp8(q_idx_np[s], c, scl, n)
            assert np.all(np.abs(got_sc[s, :n] - ref) <= _fp8_tolerance(q_idx_np[s], c, scl, n)), f"seq {s}: scores"

            def attend_ref(toks, s=s):
                kr = _rows(seed, S(s, "k"), toks, 512).reshape(-1, 2, 256)
                vr = _rows(seed, S(s, "v"), toks, 512).reshape(-1, 2, 256)
                return orc.attend(q_np[s], kr, vr, np.arange(toks.size), 1.0 / 16)

            qc.check_row_with(got_sel[s], got_n[s], o[s], lse[s], ob[s], ref, ctx, 4, 512, attend_ref)
        assert torch.count_nonzero(bufs.layer_ws[:64]).item() == 0, "control words not reset"


def _rows(seed, stream, toks, width):
    """Rows `toks` of a [tokens][width] bf16 tensor filled by the generator."""
    idx = (np.asarray(toks, dtype=np.int64)[:, None] * width + np.arange(width)[None, :]).reshape(-1)
    return qi.normal_bf16(seed, stream, 0, index=idx.astype(np.uint64)).reshape(len(toks), width)
