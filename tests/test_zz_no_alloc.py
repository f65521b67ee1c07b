"""qsa_decode_layer_noalloc (the decode layer on the library's static device
scratch, for callers that cannot allocate) through the C ABI: two calls in a
row, the second with a smaller input, each bit-identical to qsa_decode_layer
with a caller workspace on the same inputs (scores, selection, outputs);
and a call whose scratch need exceeds the static array is refused on the
host."""
import numpy as np
import pytest
import torch

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


def _inputs(pkg, seed, ctxs):
    case = qc.DecodeCase(seed, ctxs)
    nq = case.nq
    pooled = torch.zeros(nq, max(1, case.cap // 4), 128, dtype=torch.bfloat16, device="cuda")
    pkg.qsa_pool_keys(qc.to_dev(case.raw), pooled, block=4)
    kv = pkg.make_kv(qc.to_dev(case.k), qc.to_dev(case.v))
    return case, pooled, kv, qc.to_dev(case.q_idx[:, None, :]), qc.to_dev(case.q)


def _outputs(nq, max_ctx):
    f32 = dict(dtype=torch.float32, device="cuda")
    return dict(scores=torch.full((nq, max_ctx // 4), float("nan"), **f32),
                sel=torch.full((nq, 512), -7, dtype=torch.int32, device="cuda"),
                n_sel=torch.full((nq,), -7, dtype=torch.int32, device="cuda"),
                o=torch.full((nq, 16, 256), float("nan"), **f32),
                ob=torch.zeros(nq, 16, 256, dtype=torch.bfloat16, device="cuda"),
                lse=torch.full((nq, 16), float("nan"), **f32))


@pytest.mark.parametrize("n_split", [16, 5])
def test_noalloc_matches_workspace_call_twice(Q, n_split):
    pkg, _ = Q
    for call, ctxs in enumerate(([40000, 9001, 2052, 300, 20001], [8195, 2051])):
        print(f"[case] decode_layer_noalloc call {call} ctxs {ctxs} n_split {n_split}", flush=True)
        case, pooled, kv, q_idx, q = _inputs(pkg, 61 + call, ctxs)
        nq, max_ctx = case.nq, max(ctxs)
        q_ctx, q_seq = qc.i32(ctxs), qc.i32(range(nq))
        ref, got = _outputs(nq, max_ctx), _outputs(nq, max_ctx)
        ws = pkg.decode_layer_workspace(pkg.SEL_A, pkg.ATTN_A, nq, max_ctx, n_split)
        pkg.qsa_decode_layer(pkg.SEL_A, pkg.ATTN_A, q_ctx, max_ctx, q_idx, pooled, q, kv, ref["scores"], ref["sel"],
                             ref["n_sel"], n_split, ws, o_out=ref["o"], o_out_bf16=ref["ob"], lse_out=ref["lse"],
                             q_seq=q_seq)
        pkg.qsa_decode_layer_noalloc(pkg.SEL_A, pkg.ATTN_A, q_ctx, max_ctx, q_idx, pooled, q, kv, got["scores"],
                                     got["sel"], got["n_sel"], n_split, o_out=got["o"], o_out_bf16=got["ob"],
                                     lse_out=got["lse"], q_seq=q_seq)
        torch.cuda.synchronize()
        pkg.check_decode_layer_error(ws)
        for k in ref:
            a, b = ref[k], got[k]
            if a.dtype == torch.float32:
                a, b = a.nan_to_num(7.0), b.nan_to_num(7.0)
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), f"call {call}: {k} differs"
        # and the selections are the oracle's (boundary rule)
        refs = case.oracle()
        sel = got["sel"].cpu().numpy()
        n_sel = got["n_sel"].cpu().numpy()
        for i, r in enumerate(refs):
            qc.check_selection(sel[i], n_sel[i], r["scores"], ctxs[i], 4, 512)
        assert np.all(n_sel == [min(c // 4, 512) for c in ctxs])


def test_noalloc_refuses_calls_beyond_the_scratch(Q):
    pkg, _ = Q
    nq, max_ctx, n_split = 8, 4096, 256  # 256 splits x 8 queries x 16 KiB of partials: more than 16 MiB
    assert pkg.qsa_decode_layer_workspace_bytes(pkg.SEL_A, pkg.ATTN_A, nq, max_ctx, n_split) > 16 << 20
    pooled = torch.zeros(nq, max_ctx // 4, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(nq, max_ctx, 2, 256, dtype=torch.bfloat16, device="cuda")
    kv = pkg.make_kv(k, k)
    o = _outputs(nq, max_ctx)
    q_idx = torch.zeros(nq, 1, 128, dtype=torch.bfloat16, device="cuda")
    q = torch.zeros(nq, 16, 256, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pkg.QsaError) as e:
        pkg.qsa_decode_layer_noalloc(pkg.SEL_A, pkg.ATTN_A, qc.i32([max_ctx] * nq), max_ctx, q_idx, pooled, q, kv,
                                     o["scores"], o["sel"], o["n_sel"], n_split, o_out=o["o"],
                                     q_seq=qc.i32(range(nq)))
    assert e.value.status == 2 and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(o["n_sel"] == -7), "a refused call launched work"
