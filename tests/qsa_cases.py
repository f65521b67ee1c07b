"""Seeded cases and comparison rules shared by the GPU parity tests.

Inputs come from qsa_inputs only; expected values come from the oracle
only. Tolerances (from the method's stated bar and the arithmetic):
  * pooled keys, selections, counts: bit-exact;
  * a selection may differ from the oracle's only in blocks whose oracle
    score lies within 1e-5 relative of the topk-th largest oracle score
    (same count);
  * scores: fp32 accumulation of 128 exact bf16 products, any order:
    |gpu - fp64| <= 128 * 2**-24 * sum |q_d k_d|  (plus fp32 underflow slack);
  * attention, fp32 output: max |gpu - ref| <= 1e-3 * max |ref| per
    (query, head) row; bf16 output: max-abs <= 2e-2; lse: |delta| <= 1e-4
    (absolute; lse values are O(10)).
"""
from __future__ import annotations

import numpy as np
import torch

import qsa_inputs as qi
from oracle import qsa_oracle as orc

ATTN_TOL_REL = 1e-3
BF16_TOL_ABS = 2e-2
LSE_TOL_ABS = 1e-4
SEL_TOL_REL = 1e-5


def bits(seed, stream, shape, start=0):
    n = int(np.prod(shape))
    return qi.normal_bf16(seed, stream, start, n).reshape(shape)


def to_dev(bits_arr, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(bits_arr).view(np.int16)).to(device).view(torch.bfloat16)


def from_dev_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def i32(x, device="cuda"):
    return torch.tensor(np.asarray(x, dtype=np.int32), device=device)


class DecodeCase:
    """nq sequences (one decode query each) of one layer, variant A."""

    def __init__(self, seed, ctxs, cap=None, hq=16, hkv=2, d=256, idx_dim=128):
        self.seed, self.ctxs = seed, list(ctxs)
        self.nq = len(ctxs)
        self.cap = cap or max(max(ctxs), 4)
        self.cap = (self.cap + 7) // 8 * 8
        self.hq, self.hkv, self.d, self.idx_dim = hq, hkv, d, idx_dim
        S = lambda s, kind: qi.stream_id(0, s, kind)
        self.raw = np.stack([bits(seed, S(s, "raw_key"), (self.cap, idx_dim)) for s in range(self.nq)])
        self.k = np.stack([bits(seed, S(s, "k"), (self.cap, hkv, d)) for s in range(self.nq)])
        self.v = np.stack([bits(seed, S(s, "v"), (self.cap, hkv, d)) for s in range(self.nq)])
        self.q = np.stack([bits(seed, S(s, "q"), (hq, d)) for s in range(self.nq)])
        self.q_idx = np.stack([bits(seed, S(s, "q_idx"), (idx_dim,)) for s in range(self.nq)])

    def oracle(self, block=4, topk=512, scale=1.0 / 16):
        out = []
        for s, ctx in enumerate(self.ctxs):
            pooled = orc.pool_keys(self.raw[s, :ctx], block)
            r = orc.decode_query(self.q[s], self.q_idx[s], pooled, self.k[s], self.v[s], ctx,
                                 block=block, topk=topk, scale=scale)
            r["pooled"] = pooled
            out.append(r)
        return out


def score_tolerance(q_idx_bits, keys_bits, n):
    q = orc.bf16_to_f64(q_idx_bits)
    k = orc.bf16_to_f64(keys_bits[:n])
    return 128 * 2.0**-24 * (np.abs(k) @ np.abs(q)) + 1e-30


def check_selection(gpu_sel, gpu_n, oracle_scores, ctx, block, topk):
    """Raise AssertionError unless the GPU selection matches the oracle's
    within the boundary rule. Returns True if bit-identical."""
    want = orc.select_blocks(oracle_scores, ctx, block, topk)
    assert gpu_n == want.size, (gpu_n, want.size)
    got = np.asarray(gpu_sel[:gpu_n], dtype=np.int64)
    assert np.all(np.diff(got) > 0), "selection not strictly ascending"
    assert np.all(np.asarray(gpu_sel[gpu_n:]) == -1), "padding not -1"
    if np.array_equal(got, want):
        return True
    n = orc.n_candidates(ctx, block)
    s = np.asarray(oracle_scores[:n], dtype=np.float64)
    tau = np.sort(s)[::-1][topk - 1]
    diff = np.setxor1d(got, want)
    assert np.all(np.abs(s[diff] - tau) <= SEL_TOL_REL * abs(tau)), \
        f"selection differs beyond the boundary rule at blocks {diff[:10]}"
    return False


def check_attention(o_gpu, lse_gpu, o_ref, lse_ref, o_bf16=None):
    """o_*: [hq, dv]; lse_*: [hq]. Empty rows (lse = -inf) must be exactly 0."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    for h in range(o_ref.shape[0]):
        if np.isneginf(lse_ref[h]):
            assert np.isneginf(lse_gpu[h]) and np.all(o_gpu[h] == 0), f"head {h}: empty row"
            continue
        scale = np.max(np.abs(o_ref[h]))
        err = np.max(np.abs(o_gpu[h] - o_ref[h]))
        assert err <= ATTN_TOL_REL * scale, f"head {h}: max err {err:.3e} > {ATTN_TOL_REL} * {scale:.3e}"
        assert abs(lse_gpu[h] - lse_ref[h]) <= LSE_TOL_ABS, f"head {h}: lse {lse_gpu[h]} vs {lse_ref[h]}"
    if o_bf16 is not None:
        ob = orc.bf16_to_f64(o_bf16)
        live = ~np.isneginf(lse_ref)
        assert np.max(np.abs(ob[live] - o_ref[live]), initial=0.0) <= BF16_TOL_ABS


def check_row(gpu_sel, gpu_n, o, lse, ob, ref, ctx, block, topk, q_bits, k_bits, v_bits, scale, dv=None):
    """One query's selection and attention against the oracle result ref
    (decode_query). Where the boundary rule tolerated a swap, the attention
    is checked against the oracle run on the GPU's own selection. Returns
    True if the selection was bit-identical."""
    same = check_selection(gpu_sel, gpu_n, ref["scores"], ctx, block, topk)
    if same:
        o_ref, lse_ref = ref["o"], ref["lse"]
    else:
        toks = orc.selected_tokens(np.asarray(gpu_sel[:gpu_n]), ctx, block)
        o_ref, lse_ref = orc.attend(q_bits, k_bits, v_bits, toks, scale, dv)
    check_attention(o, lse, o_ref, lse_ref, ob)
    return same


def check_row_with(gpu_sel, gpu_n, o, lse, ob, oracle_scores, ctx, block, topk, attend_ref):
    """check_row with the oracle's attention given as a function:
    attend_ref(tokens) -> (o_ref, lse_ref) over the listed token positions
    (e.g. rows the oracle dequantized itself, or rows regenerated by index).
    The selection is checked against the oracle's scores first; the
    attention is then compared with the oracle on the GPU's selection, which
    is the oracle's own unless a boundary swap was tolerated. Returns True if
    the selection was bit-identical."""
    same = check_selection(gpu_sel, gpu_n, oracle_scores, ctx, block, topk)
    toks = orc.selected_tokens(np.asarray(gpu_sel[:gpu_n]), ctx, block)
    o_ref, lse_ref = attend_ref(toks)
    check_attention(o, lse, o_ref, lse_ref, ob)
    return same


# ---- FP8 key pages (layout only: 64 keys per page, codes then fp32 scales)

def unpack_fp8_pages(buf, n, dim):
    """(codes uint8 [n][dim], scales float32 [n]) of keys 0..n-1 in one
    sequence's page buffer (uint8 array)."""
    buf = np.asarray(buf, dtype=np.uint8)
    page = 64 * (dim + 4)
    npg = -(-n // 64)
    p = buf[:npg * page].reshape(npg, page)
    codes = p[:, :64 * dim].reshape(npg * 64, dim)[:n]
    scales = np.ascontiguousarray(p[:, 64 * dim:]).view(np.float32).reshape(-1)[:n]
    return codes, scales


def pack_fp8_pages(codes, scales):
    """The page buffer of keys given as codes [n][dim] and scales [n]."""
    n, dim = codes.shape
    npg = -(-n // 64)
    c = np.zeros((npg * 64, dim), dtype=np.uint8)
    c[:n] = codes
    s = np.zeros(npg * 64, dtype=np.float32)
    s[:n] = scales
    pages = np.concatenate([c.reshape(npg, 64 * dim), s.view(np.uint8).reshape(npg, 256)], axis=1)
    return pages.reshape(-1)
