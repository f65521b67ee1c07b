"""GPU parity of the FP8 sparse-MLA rows (656 bytes per token: 512 E4M3
codes in 4 groups of 128 with one fp32 scale each, then the 64 rotary values
in bf16) through the C ABI, against the oracle.

* qsa_quantize_latent and qsa_kv_append write the oracle's rows (fp8_latent)
  bit for bit, and nothing outside their rows.
* Attention over FP8 rows (decode splits merged, and a tiled prefill chunk
  whose result must not depend on the tile size) matches the oracle's
  attention over the dequantized rows within the attention tolerances.
"""
import numpy as np
import pytest
import torch

import qsa_inputs as qi
from oracle import qsa_oracle as orc
from tests import qsa_cases as qc

pytestmark = pytest.mark.gpu

SCALE = 1.0 / 24.0


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


def _unpack_rows(rows):
    """(codes [.., 512], scales [.., 4], rope bits [.., 64]) of uint8 rows [.., 656]."""
    rows = np.ascontiguousarray(rows)
    codes = rows[..., :512]
    scales = np.ascontiguousarray(rows[..., 512:528]).view(np.float32)
    rope = np.ascontiguousarray(rows[..., 528:656]).view(np.uint16)
    return codes, scales, rope


def _latent(seed, n_seq, cap):
    lat = np.stack([qc.bits(seed, qi.stream_id(0, s, "latent"), (cap, 1, 576)) for s in range(n_seq)])
    lat[0, 3, 0, 128:256] = 0                  # one all-zero group
    lat[0, 4, 0, :512] = 0x8000                # negative zeros
    lat[0, 5, 0, 7] = orc.f64_to_bf16(3e3)[0]  # one dominant value: the group's rest subnormal / zero
    return lat


def _fp8_rows(pkg, lat_dev):
    n_seq, cap = lat_dev.shape[:2]
    out = torch.zeros(n_seq, cap, 656, dtype=torch.uint8, device="cuda")
    pkg.qsa_quantize_latent(lat_dev, out)
    return out


def test_quantize_latent_bit_exact(Q):
    pkg, _ = Q
    _print_case("quantize_latent")
    lat = _latent(71, 2, 200)
    out = _fp8_rows(pkg, qc.to_dev(lat))
    torch.cuda.synchronize()
    codes, scales, rope = _unpack_rows(out.cpu().numpy())
    for s in range(2):
        c, sc, rp = orc.fp8_latent(lat[s, :, 0, :])
        assert np.array_equal(codes[s], c), f"sequence {s}: codes"
        assert np.array_equal(scales[s].view(np.uint32), sc.view(np.uint32)), f"sequence {s}: scales"
        assert np.array_equal(rope[s], rp), f"sequence {s}: rotary values"
    part = torch.zeros_like(out)
    pkg.qsa_quantize_latent(qc.to_dev(lat), part, tok_begin=17, tok_end=150)
    torch.cuda.synchronize()
    p, full = part.cpu().numpy(), out.cpu().numpy()
    assert np.array_equal(p[:, 17:150], full[:, 17:150])
    assert not p[:, :17].any() and not p[:, 150:].any()


def test_append_fp8_latent_rows(Q):
    pkg, _ = Q
    cap, n_seq = 40, 2
    rows = torch.zeros(n_seq, cap, 656, dtype=torch.uint8, device="cuda")
    kv = pkg.make_kv(rows)
    keys = torch.zeros(n_seq, cap, 64, dtype=torch.bfloat16, device="cuda")
    for step, pos in enumerate(([3, 39], [4, 0])):
        _print_case("append_fp8_latent", step=step, pos=pos)
        new = qc.bits(72, step, (n_seq, 1, 576))
        knew = qc.bits(73, step, (n_seq, 64))
        before = rows.cpu().numpy()
        pkg.qsa_kv_append(pkg.SEL_B, pkg.ATTN_B, qc.i32(pos), qc.to_dev(new), kv, raw_new=qc.to_dev(knew),
                          raw_keys=keys)
        torch.cuda.synchronize()
        after = rows.cpu().numpy()
        for s, p in enumerate(pos):
            c, sc, rp = orc.fp8_latent(new[s])
            codes, scales, rope = _unpack_rows(after[s, p])
            assert np.array_equal(codes, c[0]) and np.array_equal(scales.view(np.uint32), sc[0].view(np.uint32))
            assert np.array_equal(rope, rp[0])
            assert np.array_equal(qc.from_dev_bits(keys[s, p]), knew[s])
        mask = np.ones(after.shape[:2], dtype=bool)
        for s, p in enumerate(pos):
            mask[s, p] = False
        assert np.array_equal(after[mask], before[mask]), "rows outside the appended positions changed"


def _oracle_values(lat_bits):
    """The float64 values the oracle's own FP8 rows of bf16 latent rows
    [n][576] stand for (the GPU rows are pinned to these codes bit for bit
    in test_quantize_latent_bit_exact)."""
    return orc.fp8_latent_values(*orc.fp8_latent(lat_bits))  # [n, 576] float64


@pytest.mark.parametrize("n_split", [1, 5, 16])
def test_fp8_mla_attention_on_given_selection(Q, n_split):
    pkg, _ = Q
    ctxs = [5000, 2048, 2049, 1, 0, 3001]
    nq, cap = len(ctxs), 5000
    _print_case("fp8_mla_attend", n_split=n_split)
    lat = _latent(74, nq, cap)
    rows = _fp8_rows(pkg, qc.to_dev(lat))
    vals = [_oracle_values(lat[s, :, 0, :]) for s in range(nq)]
    q = np.stack([qc.bits(75, s, (64, 576)) for s in range(nq)])
    rng = np.random.default_rng(76)
    sel = torch.full((nq, 2048), -1, dtype=torch.int32, device="cuda")
    n_sel = torch.zeros(nq, dtype=torch.int32, device="cuda")
    chosen = []
    for i, ctx in enumerate(ctxs):
        s_i = np.arange(ctx) if ctx <= 2048 else np.sort(rng.choice(ctx, 2048, replace=False))
        chosen.append(s_i)
        sel[i, :s_i.size] = torch.tensor(s_i.astype(np.int32))
        n_sel[i] = int(s_i.size)
    kv = pkg.make_kv(rows)
    o_part = torch.empty(n_split, nq, 64, 512, device="cuda")
    lse_part = torch.empty(n_split, nq, 64, device="cuda")
    pkg.qsa_sparse_decode(pkg.SEL_B, pkg.ATTN_B, qc.i32(ctxs), cap, qc.to_dev(q), kv, sel, n_sel, n_split,
                          o_part, lse_part, q_seq=qc.i32(range(nq)))
    o = torch.empty(nq, 64, 512, device="cuda")
    ob = torch.empty(nq, 64, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(nq, 64, device="cuda")
    pkg.qsa_lse_merge(o_part, lse_part, o_out=o, o_out_bf16=ob, lse_out=lse)
    torch.cuda.synchronize()
    o, lse, ob = o.cpu().numpy(), lse.cpu().numpy(), qc.from_dev_bits(ob)
    for i in range(nq):
        v = vals[i][:, None, :]
        o_ref, lse_ref = orc.attend_values(q[i], v, v, chosen[i], SCALE, dv=512)
        qc.check_attention(o[i], lse[i], o_ref, lse_ref, ob[i])


@pytest.mark.parametrize("tile", [16384, 777])
def test_fp8_mla_prefill_chunk_tiled(Q, tile):
    """32 queries at positions 9000..9031 select among their earlier tokens
    (bf16 indexer keys); attention over FP8 rows tile by tile, merged; each
    row equals the oracle's attention over the dequantized rows whatever the
    tile size."""
    pkg, pipeline = Q
    hist, nq = 9000, 32
    ctx_max = hist + nq
    _print_case("fp8_mla_prefill", tile=tile)
    seed = 77
    lat = qc.bits(seed, 1, (1, ctx_max, 1, 576))
    keys = qc.bits(seed, 2, (ctx_max, 64))
    q = qc.bits(seed, 3, (nq, 64, 576))
    q_idx = qc.bits(seed, 4, (nq, 4, 64))
    w = np.stack([qi.uniform_f32(seed, 100 + i, 4) for i in range(nq)])
    ctxs = [hist + i + 1 for i in range(nq)]
    rows = _fp8_rows(pkg, qc.to_dev(lat))
    vals = _oracle_values(lat[0, :, 0, :])
    kv = pkg.make_kv(rows)
    bufs = pipeline.prefill_buffers(pkg.SEL_B, pkg.ATTN_B, nq, ctx_max, tile)
    pipeline.prefill_chunk(pkg.SEL_B, pkg.ATTN_B, qc.i32(ctxs), ctx_max, qc.to_dev(q_idx), qc.to_dev(keys[None]),
                           qc.to_dev(q), kv, bufs, w_idx=torch.tensor(w, device="cuda"))
    torch.cuda.synchronize()
    sel, n_sel = bufs.sel.cpu().numpy(), bufs.n_sel.cpu().numpy()
    o, lse, ob = bufs.o.cpu().numpy(), bufs.lse.cpu().numpy(), qc.from_dev_bits(bufs.o_bf16)
    v = vals[:, None, :]
    for i in range(nq):
        sc = orc.index_scores_relu(q_idx[i], w[i], keys, ctxs[i])
        qc.check_row_with(sel[i], n_sel[i], o[i], lse[i], ob[i], sc, ctxs[i], 1, 2048,
                          lambda toks, i=i: orc.attend_values(q[i], v, v, toks, SCALE, dv=512))


def _relu_tolerance(q_bits, w, codes, scales, n):
    q = orc.bf16_to_f64(q_bits)
    k = orc.dequantize_e4m3(codes[:n], scales[:n, None], 64)
    return 70 * 2.0 ** -24 * (np.abs(k) @ np.abs(q).T) @ np.abs(np.asarray(w, dtype=np.float64)) + 1e-30


def test_fp8_token_key_scores(Q):
    """The 4-head ReLU-weighted indexer over FP8 token keys (64 codes + a
    scale per token): decode stream and prefill MFMA paths against the
    oracle on the dequantized keys."""
    pkg, _ = Q
    n = 20000
    keys_np = np.stack([qc.bits(81, s, (n, 64)) for s in range(2)])
    keys8 = pkg.fp8_keys_empty(2, n, 64)
    pkg.qsa_quantize_keys(qc.to_dev(keys_np), keys8)
    ref = [orc.fp8_keys(keys_np[s]) for s in range(2)]
    for chunk in (False, True):
        rng = np.random.default_rng(82)
        nq = 40 if chunk else 6
        ctxs = [int(x) for x in rng.integers(0, n + 1, nq)]
        ctxs[0], ctxs[-1] = n, 1
        q_seq = None if chunk else [i % 2 for i in range(nq)]
        _print_case("fp8_token_key_scores", chunk=chunk)
        q_np = qc.bits(83, int(chunk), (nq, 4, 64))
        w_np = np.stack([qi.uniform_f32(84, i, 4) for i in range(nq)])
        sc = torch.full((nq, n + 5), float("nan"), device="cuda")
        pkg.qsa_index_scores(pkg.SEL_B_FP8, qc.i32(ctxs), n, qc.to_dev(q_np), keys8[0:1] if chunk else keys8, sc,
                             q_seq=None if chunk else qc.i32(q_seq), w_idx=torch.tensor(w_np, device="cuda"))
        torch.cuda.synchronize()
        got = sc.cpu().numpy()
        for i, ctx in enumerate(ctxs):
            c, s = ref[0 if chunk else q_seq[i]]
            want = orc.index_scores_relu_fp8(q_np[i], w_np[i], c, s, ctx)
            assert np.all(np.abs(got[i, :ctx] - want) <= _relu_tolerance(q_np[i], w_np[i], c, s, ctx)), f"query {i}"
            assert np.all(np.isnan(got[i, ctx:]))


def test_fp8_mla_decode_keys_and_rows(Q):
    """Decode over FP8 token keys and FP8 rows (the GLM cache: 68 + 656
    bytes per token), end to end against the oracle, which quantizes the
    bf16 keys and rows itself: scores within the accumulation bound, the
    selection the oracle's on its own scores (boundary rule), attention the
    oracle's over its dequantized rows."""
    pkg, pipeline = Q
    ctxs = [20000, 2048, 2049, 7, 12345]
    nq, cap = len(ctxs), 20000
    _print_case("fp8_mla_decode_keys_rows", ctxs=ctxs)
    lat = _latent(85, nq, cap)
    keys_np = np.stack([qc.bits(86, s, (cap, 64)) for s in range(nq)])
    q = np.stack([qc.bits(87, s, (64, 576)) for s in range(nq)])
    q_idx = np.stack([qc.bits(88, s, (4, 64)) for s in range(nq)])
    w = np.stack([qi.uniform_f32(89, s, 4) for s in range(nq)])
    rows = _fp8_rows(pkg, qc.to_dev(lat))
    keys8 = pkg.fp8_keys_empty(nq, cap, 64)
    pkg.qsa_quantize_keys(qc.to_dev(keys_np), keys8)
    kv = pkg.make_kv(rows)
    bufs = pipeline.decode_buffers(pkg.SEL_B_FP8, pkg.ATTN_B, nq, cap)
    bufs.scores.fill_(float("nan"))
    pipeline.decode_layer(pkg.SEL_B_FP8, pkg.ATTN_B, qc.i32(ctxs), cap, qc.to_dev(q_idx), keys8, qc.to_dev(q), kv,
                          bufs, q_seq=qc.i32(range(nq)), w_idx=torch.tensor(w, device="cuda"))
    torch.cuda.synchronize()
    sc, sel, n_sel = bufs.scores.cpu().numpy(), bufs.sel.cpu().numpy(), bufs.n_sel.cpu().numpy()
    o, lse, ob = bufs.o.cpu().numpy(), bufs.lse.cpu().numpy(), qc.from_dev_bits(bufs.o_bf16)
    for i, ctx in enumerate(ctxs):
        # the oracle quantizes the bf16 keys and rows itself
        c, s = orc.fp8_keys(keys_np[i])
        want = orc.index_scores_relu_fp8(q_idx[i], w[i], c, s, ctx)
        assert np.all(np.abs(sc[i, :ctx] - want) <= _relu_tolerance(q_idx[i], w[i], c, s, ctx)), f"query {i}: scores"
        v = _oracle_values(lat[i, :, 0, :])[:, None, :]
        qc.check_row_with(sel[i], n_sel[i], o[i], lse[i], ob[i], want, ctx, 1, 2048,
                          lambda toks, i=i, v=v: orc.attend_values(q[i], v, v, toks, SCALE, dv=512))


def test_append_fp8_token_keys(Q):
    pkg, _ = Q
    cap, n_seq = 130, 2
    rows = torch.zeros(n_seq, cap, 656, dtype=torch.uint8, device="cuda")
    kv = pkg.make_kv(rows)
    keys8 = pkg.fp8_keys_empty(n_seq, cap, 64)
    for step, pos in enumerate(([0, 129], [64, 63], [65, 1])):
        _print_case("append_fp8_token_keys", pos=pos)
        new = qc.bits(90, step, (n_seq, 1, 576))
        knew = qc.bits(91, step, (n_seq, 64))
        knew[1, :5] = 0x8000
        before = keys8.cpu().numpy()
        pkg.qsa_kv_append(pkg.SEL_B_FP8, pkg.ATTN_B, qc.i32(pos), qc.to_dev(new), kv, raw_new=qc.to_dev(knew),
                          raw_keys=keys8)
        torch.cuda.synchronize()
        after = keys8.cpu().numpy()
        for s, p in enumerate(pos):
            codes, scales = qc.unpack_fp8_pages(after[s], cap, 64)
            wc, ws = orc.fp8_keys(knew[s:s + 1])
            assert np.array_equal(codes[p], wc[0]) and scales[p].view(np.uint32) == ws[0].view(np.uint32)
            oc, os_ = qc.unpack_fp8_pages(before[s], cap, 64)
            others = np.arange(cap) != p
            assert np.array_equal(codes[others], oc[others]) and np.array_equal(scales[others], os_[others])
