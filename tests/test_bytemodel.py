"""The byte model reproduces the figures printed on the QSA offload page
(tests/golden/byte_model.txt) and the budget rule."""
import os

from indexer_selected_sparse_pooled_amd import bytemodel as bm

GOLD = os.path.join(os.path.dirname(__file__), "golden", "byte_model.txt")


def _golden():
    out = {}
    for line in open(GOLD):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split()
            out[k] = float(v)
    return out


def test_page_figures():
    g = _golden()
    assert bm.kv_bytes(2048) == g["kv_bytes_per_layer_seq"]
    assert 12 * bm.kv_bytes(2048) / 2**20 == g["kv_mib_per_step_12_layers"]
    # 250,000 blocks x 128 x 2 B per layer -> 732 MiB per token over 12 layers
    scan = bm.scan_bytes(4 * int(g["scan_blocks"]))
    assert round(12 * scan / 2**20) == g["scan_mib_per_token_12_layers"]
    t = bm.per_token_bytes()
    assert t["pooled"] / 1024 == g["pooled_kib_per_token_12_layers"]
    assert t["kv_and_raw_keys"] / 1024 == g["host_kib_per_token_12_layers"]


def test_decode_unit_at_1m():
    # 262,080 blocks x 256 B scanned + 2048 rows x 2 KiB gathered + q_idx, Q, O
    b = bm.decode_unit_bytes(1048320)
    assert b == 262080 * 256 + 256 + 4194304 + 8192 + 8192
    assert bm.attended_tokens(2051) == 2051 and bm.attended_tokens(2052) == 2048
    assert bm.attended_tokens(1048323) == 2051


def test_fp8_scan_bytes():
    """FP8 keys: 128 codes + a 4-byte scale = 132 bytes per pooled block
    ("GLM-5.3 ...", footnote 3), against 256 for bf16."""
    assert bm.scan_bytes_fp8(1048320) == 262080 * 132
    assert bm.decode_unit_bytes(1048320) - bm.decode_unit_bytes_fp8(1048320) == 262080 * (256 - 132)
