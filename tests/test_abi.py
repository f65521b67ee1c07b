"""The C ABI library loads on a CPU-only host and exports every entry point
that include/qsa.h declares; argument checks that need no device work."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from indexer_selected_sparse_pooled_amd import qsa
    if not os.path.exists(qsa.LIB_PATH):
        pytest.fail("libqsa.so is not built (run __graft_entry__.build())")
    return qsa.lib()


def test_header_declares_the_five_operations():
    names = _declared()
    for n in ("qsa_index_scores", "qsa_topk_blocks", "qsa_sparse_decode", "qsa_sparse_prefill", "qsa_lse_merge"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from indexer_selected_sparse_pooled_amd import qsa
    for name in _declared():
        assert hasattr(lib, name), name
        assert name in qsa.EXPORTS, f"binding has no signature for {name}"


def test_status_strings_and_version(lib):
    assert lib.qsa_version() == 100
    assert lib.qsa_status_string(0) == b"ok"
    assert lib.qsa_status_string(3) == b"workspace too small"


def test_validation_happens_before_any_device_call(lib):
    from indexer_selected_sparse_pooled_amd import qsa
    # unsupported block: rejected on the host, no GPU needed
    st = lib.qsa_pool_keys(None, 0, None, 0, 1, 0, 8, 128, 3, None)
    assert st == 2 and b"block" in lib.qsa_last_error()
    # unsupported top-k
    cfg = qsa.SelCfg(4, 4096, 128, 1)
    st = lib.qsa_topk_blocks(ctypes.byref(cfg), 1, None, 100, None, 100, None, None, None, 0, None)
    assert st == 2
    # empty work is a no-op that succeeds without touching the device
    st = lib.qsa_index_scores(ctypes.byref(qsa.SEL_A), 0, None, None, 0, None, None, None, 0, None, 0, None)
    assert st == 0
    st = lib.qsa_lse_merge(1, 0, 256, None, 0, None, 0, None, None, None, None)
    assert st == 0
    # negative sizes
    st = lib.qsa_lse_merge(0, 4, 256, None, 0, None, 0, None, None, None, None)
    assert st == 1
    # attention shape not compiled
    bad = qsa.AttnCfg(8, 2, 128, 128, 0.1)
    kv = qsa.KV()
    st = lib.qsa_sparse_decode(ctypes.byref(qsa.SEL_A), ctypes.byref(bad), 1, None, None, 10, None,
                               ctypes.byref(kv), None, None, 1, None, None, None)
    assert st == 2


def test_topk_workspace_query(lib):
    from indexer_selected_sparse_pooled_amd import qsa
    # small contexts need no workspace; 1M-token contexts need the chunk lists
    assert qsa.qsa_topk_workspace_bytes(qsa.SEL_A, 4, 8192) == 0
    big = qsa.qsa_topk_workspace_bytes(qsa.SEL_A, 4, 1048320)
    assert big > 0 and big % 16 == 0


def test_fp8_key_layout_sizes(lib):
    """Pages of 64 keys, each key idx_dim codes + a 4-byte scale (132 bytes
    for the 128-d pooled key)."""
    assert lib.qsa_fp8_keys_bytes(64, 128) == 64 * 132
    assert lib.qsa_fp8_keys_bytes(65, 128) == 2 * 64 * 132
    assert lib.qsa_fp8_keys_bytes(0, 128) == 0
    assert lib.qsa_fp8_keys_bytes(262080, 128) == 262080 * 132  # 4095 whole pages
    assert lib.qsa_fp8_keys_bytes(1, 64) == 64 * 68


def test_fp8_validation_on_the_host(lib):
    from indexer_selected_sparse_pooled_amd import qsa
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation
    # unknown key format
    cfg = qsa.SelCfg(4, 512, 128, 1, 7)
    st = lib.qsa_index_scores(ctypes.byref(cfg), 1, None, fake, 4096, fake, None, fake, 0, fake, 1024, None)
    assert st == 2 and b"key_format" in lib.qsa_last_error()
    # FP8 rows only for the shared-latent attention shape
    kv = qsa.KV(fake, fake, 0, 656, 0, 4096, qsa.KV_FP8_MLA)
    st = lib.qsa_sparse_decode(ctypes.byref(qsa.SEL_A), ctypes.byref(qsa.ATTN_A), 1, None, fake, 4096, fake,
                               ctypes.byref(kv), fake, fake, 1, fake, fake, None)
    assert st == 2 and b"FP8 rows" in lib.qsa_last_error()
    # FP8 sequence stride must be a multiple of 16 bytes and hold the pages
    st = lib.qsa_index_scores(ctypes.byref(qsa.SEL_A_FP8), 1, fake, fake, 4096, fake, None, fake, 8, fake, 1024,
                              None)
    assert st == 1
    st = lib.qsa_index_scores(ctypes.byref(qsa.SEL_A_FP8), 1, fake, fake, 4096, fake, None, fake, 16 * 100,
                              fake, 1024, None)
    assert st == 1 and b"pages" in lib.qsa_last_error()
    # quantize: only 64- and 128-d keys
    st = lib.qsa_quantize_keys(fake, 0, fake, 0, 1, 0, 10, 96, None)
    assert st == 2


def test_row_cache_sizes_and_host_validation(lib):
    """Row cache buffer: a 256-byte header (the epoch), then per slot a tag
    (8 B), a hit mark (4 B), a claim (8 B) and the row (K and V of both kv
    heads, 2 KiB), each array 256-byte aligned. Misuse fails on the host."""
    from indexer_selected_sparse_pooled_amd import qsa
    up = lambda x: (x + 255) // 256 * 256
    n = 1000
    want = up(up(up(256 + 8 * n) + 4 * n) + 8 * n) + n * 2048
    assert qsa.qsa_row_cache_bytes(qsa.ATTN_A, n) == want
    assert qsa.qsa_row_cache_bytes(qsa.ATTN_B, n) == 0
    assert qsa.qsa_row_cache_bytes(qsa.ATTN_A, 0) == 0
    assert qsa.qsa_decode_cached_plan_bytes(qsa.SEL_A, 4) == 4 * 2051 * 4
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation
    kv = qsa.KV(fake, fake, 4096 * 1024, 1024, 256, 4096, qsa.KV_BF16)

    def decode(attn, kvd, cache_bytes, n_slots, plan_bytes):
        return lib.qsa_sparse_decode_cached(ctypes.byref(qsa.SEL_A), ctypes.byref(attn), 1, None, fake, 4096, fake,
                                            ctypes.byref(kvd), fake, fake, 1, fake, fake, fake, cache_bytes, n_slots,
                                            fake, plan_bytes, None)
    assert decode(qsa.ATTN_A, kv, want - 1, n, 2051 * 4) == 3
    assert decode(qsa.ATTN_A, kv, want, n, 2051 * 4 - 1) == 3
    assert decode(qsa.ATTN_A, kv, want, 0, 2051 * 4) == 1
    kv8 = qsa.KV(fake, fake, 0, 656, 0, 4096, qsa.KV_FP8_MLA)
    st = decode(qsa.ATTN_A, kv8, want, n, 2051 * 4)
    assert st == 2
    st = lib.qsa_row_cache_step(ctypes.byref(qsa.ATTN_B), fake, want, n, 0, None, None, ctypes.byref(kv), None)
    assert st == 2 and b"row cache" in lib.qsa_last_error()
    st = lib.qsa_row_cache_step(ctypes.byref(qsa.ATTN_A), fake, want, n, -1, None, None, ctypes.byref(kv), None)
    assert st == 1


def test_prefill_select_workspace_and_host_validation(lib):
    """qsa_index_topk_prefill: workspace = sample scores (nq x ceil(keys / s),
    s = ceil(keys / 4096)), thresholds, one 128-byte counter line and a flag
    per query and lists of 8192 entries per query, each 256-byte aligned;
    unsupported shapes and short workspaces
    fail on the host."""
    from indexer_selected_sparse_pooled_amd import qsa
    up = lambda x: (x + 255) // 256 * 256
    nq, ctx = 2048, 131072
    n_samp = 4096
    want = up(up(up(up(nq * n_samp * 4) + nq * 8) + nq * 128) + nq * 4) + nq * 8192 * 8
    assert qsa.qsa_index_topk_prefill_workspace_bytes(qsa.SEL_B, nq, ctx) == want
    assert qsa.qsa_index_topk_prefill_workspace_bytes(qsa.SEL_B, 16, 262145) == 0  # past the bitmap
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation

    def call(cfg, n, ws_bytes):
        return lib.qsa_index_topk_prefill(ctypes.byref(cfg), n, fake, ctx, fake, fake, fake, fake, ctx, fake, fake,
                                          fake, ws_bytes, None)
    assert call(qsa.SEL_A, 64, want) == 2  # the pooled-block indexer
    assert call(qsa.SEL_B, 8, want) == 2   # fewer than 16 queries
    ws64 = qsa.qsa_index_topk_prefill_workspace_bytes(qsa.SEL_B, 64, ctx)
    assert call(qsa.SEL_B, 64, ws64 - 1) == 3
    assert call(qsa.SEL_B, 0, 0) == 0      # no work


def test_noalloc_decode_layer_refuses_beyond_its_scratch_on_the_host(lib):
    """qsa_decode_layer_noalloc needs no workspace argument, and a call whose
    workspace need exceeds the library's 16 MiB static scratch is refused on
    the host (nothing launched, no device needed); so is a malformed one."""
    from indexer_selected_sparse_pooled_amd import qsa
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation
    kv = qsa.KV(fake, fake, 1 << 30, 512, 256, 1 << 20, 0)

    def call(nq, max_ctx, n_split, cfg=qsa.SEL_A):
        return lib.qsa_decode_layer_noalloc(ctypes.byref(cfg), ctypes.byref(qsa.ATTN_A), nq, fake, fake, max_ctx,
                                            fake, fake, 1 << 24, fake, ctypes.byref(kv), fake, max_ctx // 4, fake,
                                            fake, n_split, fake, None, None, None)
    assert qsa.qsa_decode_layer_workspace_bytes(qsa.SEL_A, qsa.ATTN_A, 8, 4096, 256) > 16 << 20
    assert call(8, 4096, 256) == 2 and b"static scratch" in lib.qsa_last_error()
    assert call(1, 4096, 300) == 1                  # n_split out of range
    assert call(1, 4096, 16, qsa.SEL_B) == 2        # the token-level indexer
    assert call(0, 4096, 16) == 0                   # no work
