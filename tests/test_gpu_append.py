"""GPU tests of qsa_kv_append, the decode step's write of new tokens into the
cache (K/V rows, raw indexer keys, and the pooled key of each block a token
completes).

The copies must be the inputs bit for bit; every pooled key must equal
qsa_pool_keys over the same raw keys and the oracle's pool_keys (the exact
mean rounded once to bf16), bit for bit, after every step; a position outside
the cache writes nothing; the shared-latent layout writes one row (V is its
first columns); and a captured graph of append + decode layer replayed with
advancing positions matches the same calls made eagerly.
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


def _fill(shape, seed, stream):
    from qsa_inputs.gpu import fill_normal_bf16
    t = torch.empty(*shape, dtype=torch.bfloat16, device="cuda")
    fill_normal_bf16(t, seed, stream)
    return t


def _bits(t):
    return qc.from_dev_bits(t)


def test_append_rows_and_pooled_keys(pkg):
    cap, n_seq, nq = 64, 3, 3
    seed = qi.config_seed(1) + 77
    k = _fill((n_seq, cap, 2, 256), seed, qi.stream_id(0, 0, "k"))
    v = _fill((n_seq, cap, 2, 256), seed, qi.stream_id(0, 0, "v"))
    raw = _fill((n_seq, cap, 128), seed, qi.stream_id(0, 0, "raw_key"))
    pooled = torch.zeros(n_seq, cap // 4, 128, dtype=torch.bfloat16, device="cuda")
    kv = pkg.make_kv(k, v)
    q_seq = [2, 0, 1]
    start = [13, 17, 22]  # the tokens before these are already in the cache
    for s in range(n_seq):
        b0 = start[q_seq.index(s)] // 4
        pkg.qsa_pool_keys(raw[s:s + 1], pooled[s:s + 1], tok_begin=0, tok_end=4 * b0, block=4)
    for step in range(11):
        pos = [p + step for p in start]
        print(f"[case] append step {step} pos {pos}", flush=True)
        k_new = _fill((nq, 2, 256), seed + 1, qi.stream_id(step, 0, "k"))
        v_new = _fill((nq, 2, 256), seed + 1, qi.stream_id(step, 0, "v"))
        raw_new = _fill((nq, 128), seed + 1, qi.stream_id(step, 0, "raw_key"))
        pkg.qsa_kv_append(pkg.SEL_A, pkg.ATTN_A, qc.i32(pos), k_new, kv, v_new=v_new, raw_new=raw_new,
                          raw_keys=raw, pooled=pooled, q_seq=qc.i32(q_seq))
        torch.cuda.synchronize()
        for i, (s, p) in enumerate(zip(q_seq, pos)):
            assert np.array_equal(_bits(k[s, p]), _bits(k_new[i]))
            assert np.array_equal(_bits(v[s, p]), _bits(v_new[i]))
            assert np.array_equal(_bits(raw[s, p]), _bits(raw_new[i]))
            nb = (p + 1) // 4  # complete blocks of this sequence so far
            ref = torch.zeros(1, nb, 128, dtype=torch.bfloat16, device="cuda")
            pkg.qsa_pool_keys(raw[s:s + 1, :4 * nb], ref, block=4)
            torch.cuda.synchronize()
            assert np.array_equal(_bits(pooled[s, :nb]), _bits(ref[0])), f"seq {s} step {step}"
            assert np.array_equal(_bits(pooled[s, :nb]), orc.pool_keys(_bits(raw[s, :4 * nb]), 4))
            # blocks not yet complete are untouched
            assert not np.any(_bits(pooled[s, nb:]))


def test_append_outside_the_cache_writes_nothing(pkg):
    cap = 16
    k = torch.zeros(2, cap, 2, 256, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    raw = torch.zeros(2, cap, 128, dtype=torch.bfloat16, device="cuda")
    pooled = torch.zeros(2, cap // 4, 128, dtype=torch.bfloat16, device="cuda")
    kv = pkg.make_kv(k, v)
    ones = torch.ones(2, 2, 256, dtype=torch.bfloat16, device="cuda")
    pkg.qsa_kv_append(pkg.SEL_A, pkg.ATTN_A, qc.i32([cap, -1]), ones, kv, v_new=ones,
                      raw_new=torch.ones(2, 128, dtype=torch.bfloat16, device="cuda"), raw_keys=raw, pooled=pooled)
    torch.cuda.synchronize()
    for t in (k, v, raw, pooled):
        assert not torch.any(t != 0)


def test_append_shared_latent_rows(pkg):
    """Shared latent (V = first 512 columns of the 576-wide row): one row per
    token; token-level indexer keys (block 1) are copied, nothing is pooled."""
    cap, n_seq = 40, 2
    seed = qi.config_seed(5) + 3
    lat = _fill((n_seq, cap, 1, 576), seed, qi.stream_id(0, 0, "latent"))
    keys = _fill((n_seq, cap, 64), seed, qi.stream_id(0, 0, "raw_key"))
    kv = pkg.make_kv(lat)
    before = _bits(lat).copy()
    new = _fill((n_seq, 1, 576), seed + 1, qi.stream_id(0, 0, "latent"))
    knew = _fill((n_seq, 64), seed + 1, qi.stream_id(0, 0, "raw_key"))
    pos = [7, 39]
    pkg.qsa_kv_append(pkg.SEL_B, pkg.ATTN_B, qc.i32(pos), new, kv, raw_new=knew, raw_keys=keys)
    torch.cuda.synchronize()
    after = _bits(lat)
    for s, p in enumerate(pos):
        assert np.array_equal(after[s, p], _bits(new[s]))
        assert np.array_equal(_bits(keys[s, p]), _bits(knew[s]))
    mask = np.ones(after.shape[:2], dtype=bool)
    for s, p in enumerate(pos):
        mask[s, p] = False
    assert np.array_equal(after[mask], before[mask])


def test_append_and_decode_layer_in_a_graph(pkg):
    """Append + qsa_decode_layer captured once; replays with advancing
    positions (device-side) give the eager results, step by step."""
    from indexer_selected_sparse_pooled_amd import pipeline
    cap, nq = 12000, 2
    seed = qi.config_seed(2) + 5
    k = _fill((nq, cap, 2, 256), seed, qi.stream_id(0, 0, "k"))
    v = _fill((nq, cap, 2, 256), seed, qi.stream_id(0, 0, "v"))
    raw = _fill((nq, cap, 128), seed, qi.stream_id(0, 0, "raw_key"))
    pooled = torch.zeros(nq, cap // 4, 128, dtype=torch.bfloat16, device="cuda")
    start = 10001
    pkg.qsa_pool_keys(raw, pooled, tok_begin=0, tok_end=start - start % 4, block=4)
    kv = pkg.make_kv(k, v)
    k_new = _fill((nq, 2, 256), seed + 1, qi.stream_id(1, 0, "k"))
    v_new = _fill((nq, 2, 256), seed + 1, qi.stream_id(1, 0, "v"))
    raw_new = _fill((nq, 128), seed + 1, qi.stream_id(1, 0, "raw_key"))
    q = _fill((nq, 16, 256), seed + 2, qi.stream_id(1, 0, "q"))
    q_idx = _fill((nq, 1, 128), seed + 2, qi.stream_id(1, 0, "q_idx"))
    q_pos = qc.i32([start, start + 3])
    q_ctx = q_pos + 1
    q_seq = qc.i32(range(nq))
    bufs = pipeline.decode_buffers(pkg.SEL_A, pkg.ATTN_A, nq, cap)

    def step():
        pkg.qsa_kv_append(pkg.SEL_A, pkg.ATTN_A, q_pos, k_new, kv, v_new=v_new, raw_new=raw_new, raw_keys=raw,
                          pooled=pooled, q_seq=q_seq)
        pipeline.decode_layer(pkg.SEL_A, pkg.ATTN_A, q_ctx, cap, q_idx, pooled, q, kv, bufs, q_seq=q_seq, fused=True)

    snap = [t.clone() for t in (k, v, raw, pooled)]
    eager = []
    for j in range(3):
        step()
        torch.cuda.synchronize()
        eager.append((bufs.o.clone(), bufs.sel.clone(), pooled.clone()))
        q_pos += 1
        q_ctx += 1
    # back to the starting state, then the same steps as graph replays
    for t, s in zip((k, v, raw, pooled), snap):
        t.copy_(s)
    q_pos -= 3
    q_ctx -= 3
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g):
            step()
    torch.cuda.synchronize()
    for t, s in zip((k, v, raw, pooled), snap):  # capture may have run nothing, but be sure
        t.copy_(s)
    torch.cuda.synchronize()
    for j in range(3):
        print(f"[case] graph replay {j}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        o, sel, pl = eager[j]
        assert torch.equal(bufs.sel, sel)
        assert torch.equal(bufs.o, o)
        assert torch.equal(pooled, pl)
        q_pos += 1
        q_ctx += 1
