"""Python binding of libqsa (argument marshalling only).

Every function here has the name of the C entry point it calls (declared in
include/qsa.h), takes torch tensors that already live on the GPU, reads
their pointers and strides, and calls the library on the given (or current)
torch stream. No arithmetic of the method happens here; if libqsa.so is
missing the first call raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqsa.so")

QSA_OK = 0
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape", 3: "workspace too small",
          4: "launch failed", 5: "no usable gfx950 device"}


class QsaError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {msg}")
        self.status = status


KEYS_BF16, KEYS_FP8 = 0, 1  # qsa_key_format


class SelCfg(ctypes.Structure):
    _fields_ = [("block", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("idx_dim", ctypes.c_int32), ("idx_heads", ctypes.c_int32),
                ("key_format", ctypes.c_int32)]


class AttnCfg(ctypes.Structure):
    _fields_ = [("hq", ctypes.c_int32), ("hkv", ctypes.c_int32), ("dk", ctypes.c_int32),
                ("dv", ctypes.c_int32), ("scale", ctypes.c_float)]


KV_BF16, KV_FP8_MLA = 0, 1  # qsa_kv_format
FP8_MLA_ROW = 656          # bytes of an FP8 sparse-MLA row


class KV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("seq_stride", ctypes.c_int64),
                ("tok_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64),
                ("capacity", ctypes.c_int64), ("format", ctypes.c_int32)]


# The two parameter sets of the pages (variant A: pooled 4-token blocks,
# variant B: token-level indexer with an MLA-like shared latent).
SEL_A = SelCfg(4, 512, 128, 1, KEYS_BF16)
# variant A with FP8 pooled keys (128 E4M3 codes + an fp32 scale per block)
SEL_A_FP8 = SelCfg(4, 512, 128, 1, KEYS_FP8)
ATTN_A = AttnCfg(16, 2, 256, 256, 1.0 / 16.0)
SEL_B = SelCfg(1, 2048, 64, 4, KEYS_BF16)
# variant B with FP8 token keys (64 E4M3 codes + an fp32 scale per token)
SEL_B_FP8 = SelCfg(1, 2048, 64, 4, KEYS_FP8)
ATTN_B = AttnCfg(64, 1, 576, 512, 1.0 / 24.0)

_lib = None

_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_SIGS = {
    "qsa_pool_keys": [_vp, _i64, _vp, _i64, _i32, _i64, _i64, _i32, _i32, _vp],
    "qsa_quantize_keys": [_vp, _i64, _vp, _i64, _i32, _i64, _i64, _i32, _vp],
    "qsa_fp8_keys_bytes": [_i64, _i32],
    "qsa_quantize_latent": [_vp, _i64, _i64, _vp, _i64, _i64, _i32, _i64, _i64, _vp],
    "qsa_kv_append": [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64, _vp],
    "qsa_index_scores": [_vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _i64, _vp, _i64, _vp],
    "qsa_topk_blocks": [_vp, _i32, _vp, _i32, _vp, _i64, _vp, _vp, _vp, _sz, _vp],
    "qsa_topk_workspace_bytes": [_vp, _i32, _i32],
    "qsa_index_topk": [_vp, _i32, _vp, _vp, _i32, _vp, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _sz, _vp],
    "qsa_index_topk_workspace_bytes": [_vp, _i32, _i32],
    "qsa_index_topk_prefill": [_vp, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp],
    "qsa_index_topk_prefill_workspace_bytes": [_vp, _i32, _i32],
    "qsa_index_lists": [_vp, _i32, _vp, _vp, _i32, _vp, _vp, _i64, _vp, _i64, _vp, _sz, _vp],
    "qsa_decode_layer": [_vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _i64, _vp, _vp, _vp, _i64, _vp, _vp, _i32,
                         _vp, _vp, _vp, _vp, _sz, _vp],
    "qsa_decode_layer_workspace_bytes": [_vp, _vp, _i32, _i32, _i32],
    "qsa_decode_layer_latent": [_vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _i64, _vp, _vp,
                                _i32, _vp, _vp, _vp, _vp, _sz, _vp],
    "qsa_decode_layer_latent_workspace_bytes": [_vp, _vp, _i32, _i32, _i32],
    "qsa_decode_layer_noalloc": [_vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _i64, _vp, _vp, _vp, _i64, _vp, _vp,
                                 _i32, _vp, _vp, _vp, _vp],
    "qsa_sparse_decode": [_vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp],
    "qsa_row_cache_bytes": [_vp, _i64],
    "qsa_decode_cached_plan_bytes": [_vp, _i32],
    "qsa_row_cache_step": [_vp, _vp, _sz, _i64, _i32, _vp, _vp, _vp, _vp],
    "qsa_sparse_decode_cached": [_vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _sz,
                                 _i64, _vp, _sz, _vp],
    "qsa_sparse_prefill": [_vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp],
    "qsa_sparse_prefill_merge": [_vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _vp,
                                 _vp, _vp, _vp],
    "qsa_lse_merge": [_i32, _i64, _i32, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp],
    "qsa_status_string": [_i32],
    "qsa_last_error": [],
    "qsa_version": [],
}
_RES = {"qsa_topk_workspace_bytes": _sz, "qsa_index_topk_workspace_bytes": _sz, "qsa_index_topk_prefill_workspace_bytes": _sz, "qsa_fp8_keys_bytes": _i64,
        "qsa_decode_layer_workspace_bytes": _sz, "qsa_decode_layer_latent_workspace_bytes": _sz,
        "qsa_row_cache_bytes": _sz, "qsa_decode_cached_plan_bytes": _sz, "qsa_status_string": ctypes.c_char_p,
        "qsa_last_error": ctypes.c_char_p, "qsa_version": _i32}
EXPORTS = tuple(_SIGS)


def lib():
    """The loaded libqsa (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with indexer_selected_sparse_pooled_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = _RES.get(name, ctypes.c_int)
        _lib = L
    return _lib


def _check(fn, status):
    if status != QSA_OK:
        raise QsaError(fn, status, lib().qsa_last_error().decode())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, dtypes, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return ctypes.c_void_p(t.data_ptr())


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_U8 = (torch.uint8,)
_F32 = (torch.float32,)
_I32 = (torch.int32,)


def _rowmajor_tail(t, name, n):
    """Require the last n dims of t to be densely packed (row-major)."""
    expect = 1
    for d in range(t.dim() - 1, t.dim() - 1 - n, -1):
        if t.size(d) > 1 and t.stride(d) != expect:
            raise ValueError(f"{name}: the last {n} dims must be contiguous")
        expect *= t.size(d)


def qsa_version() -> int:
    return lib().qsa_version()


def qsa_pool_keys(raw, pooled, tok_begin=0, tok_end=None, block=4, stream=None):
    """raw: [n_seq, n_tok, dim] bf16; pooled: [n_seq, n_blk, dim] bf16."""
    n_seq, n_tok, dim = raw.shape
    _rowmajor_tail(raw, "raw", 2)
    _rowmajor_tail(pooled, "pooled", 2)
    if tok_end is None:
        tok_end = n_tok
    if tok_end > n_tok or (tok_end // block) > pooled.shape[1] or pooled.shape[0] != n_seq or pooled.shape[2] != dim:
        raise ValueError("qsa_pool_keys: shapes do not cover the token range")
    _check("qsa_pool_keys", lib().qsa_pool_keys(
        _dev(raw, _BF16, "raw"), raw.stride(0), _dev(pooled, _BF16, "pooled"), pooled.stride(0),
        n_seq, tok_begin, tok_end, dim, block, _stream(stream)))


def qsa_quantize_latent(latent, out, tok_begin=0, tok_end=None, stream=None):
    """latent: [n_seq, capacity, 1, 576] (or [n_seq, capacity, 576]) bf16;
    out: uint8 [n_seq, capacity, 656] FP8 sparse-MLA rows."""
    n_seq, cap = latent.shape[:2]
    if latent.shape[-1] != 576 or latent.stride(-1) != 1:
        raise ValueError("qsa_quantize_latent: latent rows must be 576 contiguous bf16 values")
    if out.dtype != torch.uint8 or out.dim() != 3 or out.shape[2] != FP8_MLA_ROW or out.shape[:2] != (n_seq, cap) \
            or out.stride(2) != 1:
        raise ValueError("qsa_quantize_latent: out must be uint8 [n_seq, capacity, 656]")
    if tok_end is None:
        tok_end = cap
    _check("qsa_quantize_latent", lib().qsa_quantize_latent(
        _dev(latent, _BF16, "latent"), latent.stride(0), latent.stride(1), _dev(out, _U8, "out"), out.stride(0),
        out.stride(1), n_seq, tok_begin, tok_end, _stream(stream)))


def qsa_fp8_keys_bytes(n_keys, dim) -> int:
    return int(lib().qsa_fp8_keys_bytes(n_keys, dim))


def fp8_keys_empty(n_seq, n_keys, dim, device="cuda"):
    """A zero-filled uint8 [n_seq, bytes] tensor that holds n_keys FP8 keys
    per sequence in the library's page layout."""
    return torch.zeros(n_seq, qsa_fp8_keys_bytes(n_keys, dim), dtype=torch.uint8, device=device)


def qsa_quantize_keys(keys, out, key_begin=0, key_end=None, stream=None):
    """keys: [n_seq, n_keys, dim] bf16; out: fp8_keys_empty(n_seq, >= key_end, dim)."""
    n_seq, n_keys, dim = keys.shape
    _rowmajor_tail(keys, "keys", 2)
    if key_end is None:
        key_end = n_keys
    if key_end > n_keys or out.dim() != 2 or out.shape[0] != n_seq or out.stride(1) != 1 or \
            out.shape[1] < qsa_fp8_keys_bytes(key_end, dim):
        raise ValueError("qsa_quantize_keys: shapes do not cover the key range")
    _check("qsa_quantize_keys", lib().qsa_quantize_keys(
        _dev(keys, _BF16, "keys"), keys.stride(0), _dev(out, _U8, "out"), out.stride(0), n_seq, key_begin, key_end,
        dim, _stream(stream)))


def _keys_arg(cfg, keys, max_ctx, fn):
    """(pointer, sequence stride) of indexer keys: bf16 [n_seq, n_keys, dim]
    (stride in elements) or, for FP8 configurations, the uint8 [n_seq, bytes]
    page buffer (stride in bytes)."""
    n = max_ctx // cfg.block
    if cfg.key_format == KEYS_FP8:
        if keys.dim() != 2 or keys.stride(1) != 1 or keys.shape[1] < qsa_fp8_keys_bytes(n, cfg.idx_dim):
            raise ValueError(f"{fn}: FP8 keys must be a uint8 [n_seq, bytes] buffer holding max_ctx / block keys")
        return _dev(keys, _U8, "keys"), keys.stride(0)
    _rowmajor_tail(keys, "keys", 2)
    if n > keys.shape[1]:
        raise ValueError(f"{fn}: keys hold fewer than max_ctx / block rows")
    return _dev(keys, _BF16, "keys"), keys.stride(0)


def qsa_index_scores(cfg, q_ctx, max_ctx, q_idx, keys, scores, q_seq=None, w_idx=None, stream=None):
    """q_ctx: [nq] int32; q_idx: [nq, heads, dim] bf16; keys: [n_seq, n_keys, dim] bf16, or
    for cfg.key_format KEYS_FP8 a uint8 [n_seq, bytes] page buffer (fp8_keys_empty);
    scores: [nq, ld] fp32; q_seq: [nq] int32 or None; w_idx: [nq, heads] fp32 or None."""
    nq = q_ctx.shape[0]
    _rowmajor_tail(q_idx, "q_idx", 3)
    _rowmajor_tail(scores, "scores", 1)
    kp, kss = _keys_arg(cfg, keys, max_ctx, "qsa_index_scores")
    _check("qsa_index_scores", lib().qsa_index_scores(
        ctypes.byref(cfg), nq, _dev(q_seq, _I32, "q_seq"), _dev(q_ctx, _I32, "q_ctx"), max_ctx,
        _dev(q_idx, _BF16, "q_idx"), _dev(w_idx, _F32, "w_idx"), kp, kss, _dev(scores, _F32, "scores"),
        scores.stride(0), _stream(stream)))


def qsa_index_topk_prefill_workspace_bytes(cfg, nq, max_ctx) -> int:
    return int(lib().qsa_index_topk_prefill_workspace_bytes(ctypes.byref(cfg), nq, max_ctx))


def index_topk_prefill_workspace(cfg, nq, max_ctx, device="cuda"):
    """A workspace tensor for qsa_index_topk_prefill, or None where that call
    does not apply."""
    n = qsa_index_topk_prefill_workspace_bytes(cfg, nq, max_ctx)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def qsa_index_topk_prefill(cfg, q_ctx, max_ctx, q_idx, w_idx, keys, scores, sel, n_sel, ws, stream=None):
    """The selections of qsa_index_scores + qsa_topk_blocks for a prefill
    chunk of one sequence (token-level 4-head indexer), without writing every
    score. keys: [1, n_keys, 64] bf16 or an FP8 page buffer; ws:
    index_topk_prefill_workspace(...)."""
    nq = q_ctx.shape[0]
    _rowmajor_tail(q_idx, "q_idx", 3)
    _rowmajor_tail(scores, "scores", 1)
    kp, _ = _keys_arg(cfg, keys, max_ctx, "qsa_index_topk_prefill")
    _check("qsa_index_topk_prefill", lib().qsa_index_topk_prefill(
        ctypes.byref(cfg), nq, _dev(q_ctx, _I32, "q_ctx"), max_ctx, _dev(q_idx, _BF16, "q_idx"),
        _dev(w_idx, _F32, "w_idx"), kp, _dev(scores, _F32, "scores"), scores.stride(0),
        _dev(sel, _I32, "sel"), _dev(n_sel, _I32, "n_sel"), _dev(ws, _U8, "ws"), ws.numel(), _stream(stream)))


def qsa_topk_workspace_bytes(cfg, nq, max_ctx) -> int:
    return int(lib().qsa_topk_workspace_bytes(ctypes.byref(cfg), nq, max_ctx))


def topk_workspace(cfg, nq, max_ctx, device="cuda"):
    """A workspace tensor of the size qsa_topk_blocks needs (or None)."""
    n = qsa_topk_workspace_bytes(cfg, nq, max_ctx)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device) if n else None


def qsa_topk_blocks(cfg, q_ctx, max_ctx, scores, sel, n_sel, ws=None, stream=None):
    """scores: [nq, ld] fp32; sel: [nq, topk] int32; n_sel: [nq] int32; ws: uint8 tensor."""
    nq = q_ctx.shape[0]
    _rowmajor_tail(scores, "scores", 1)
    if sel.shape != (nq, cfg.topk) or not sel.is_contiguous():
        raise ValueError("qsa_topk_blocks: sel must be a contiguous [nq, topk] tensor")
    ws_ptr = None if ws is None else ctypes.c_void_p(ws.data_ptr())
    ws_n = 0 if ws is None else ws.numel() * ws.element_size()
    _check("qsa_topk_blocks", lib().qsa_topk_blocks(
        ctypes.byref(cfg), nq, _dev(q_ctx, _I32, "q_ctx"), max_ctx, _dev(scores, _F32, "scores"),
        scores.stride(0), _dev(sel, _I32, "sel"), _dev(n_sel, _I32, "n_sel"), ws_ptr, ws_n,
        _stream(stream)))


def qsa_index_topk_workspace_bytes(cfg, nq, max_ctx) -> int:
    return int(lib().qsa_index_topk_workspace_bytes(ctypes.byref(cfg), nq, max_ctx))


def index_topk_workspace(cfg, nq, max_ctx, device="cuda"):
    """A zero-filled workspace tensor for qsa_index_topk (its counters must
    start at zero; every call leaves them zero)."""
    n = qsa_index_topk_workspace_bytes(cfg, nq, max_ctx)
    return torch.zeros(max(n, 16), dtype=torch.uint8, device=device)


def qsa_index_topk(cfg, q_ctx, max_ctx, q_idx, keys, scores, sel, n_sel, ws, q_seq=None, stream=None):
    """qsa_index_scores + qsa_topk_blocks in one launch. Shapes as those two;
    ws: index_topk_workspace(...)."""
    nq = q_ctx.shape[0]
    _rowmajor_tail(q_idx, "q_idx", 3)
    _rowmajor_tail(scores, "scores", 1)
    kp, kss = _keys_arg(cfg, keys, max_ctx, "qsa_index_topk")
    if sel.shape != (nq, cfg.topk) or not sel.is_contiguous():
        raise ValueError("qsa_index_topk: sel must be a contiguous [nq, topk] tensor")
    _check("qsa_index_topk", lib().qsa_index_topk(
        ctypes.byref(cfg), nq, _dev(q_seq, _I32, "q_seq"), _dev(q_ctx, _I32, "q_ctx"), max_ctx,
        _dev(q_idx, _BF16, "q_idx"), kp, kss,
        _dev(scores, _F32, "scores"), scores.stride(0), _dev(sel, _I32, "sel"), _dev(n_sel, _I32, "n_sel"),
        ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(), _stream(stream)))


def qsa_index_lists(cfg, q_ctx, max_ctx, q_idx, keys, scores, ws, q_seq=None, stream=None):
    """The scan qsa_decode_layer issues first, on its own: scores (unless
    scores is None) and the chunk candidate lists (in ws:
    index_topk_workspace(...)); no selection."""
    nq = q_ctx.shape[0]
    _rowmajor_tail(q_idx, "q_idx", 3)
    if scores is not None:
        _rowmajor_tail(scores, "scores", 1)
    kp, kss = _keys_arg(cfg, keys, max_ctx, "qsa_index_lists")
    _check("qsa_index_lists", lib().qsa_index_lists(
        ctypes.byref(cfg), nq, _dev(q_seq, _I32, "q_seq"), _dev(q_ctx, _I32, "q_ctx"), max_ctx,
        _dev(q_idx, _BF16, "q_idx"), kp, kss,
        _dev(scores, _F32, "scores"), scores.stride(0) if scores is not None else 0, ctypes.c_void_p(ws.data_ptr()),
        ws.numel() * ws.element_size(), _stream(stream)))


def qsa_decode_layer_workspace_bytes(sel_cfg, attn_cfg, nq, max_ctx, n_split) -> int:
    return int(lib().qsa_decode_layer_workspace_bytes(ctypes.byref(sel_cfg), ctypes.byref(attn_cfg), nq, max_ctx,
                                                      n_split))


def decode_layer_workspace(sel_cfg, attn_cfg, nq, max_ctx, n_split, device="cuda"):
    """A zero-filled workspace tensor for qsa_decode_layer (its counters must
    start at zero; every call leaves them zero)."""
    n = qsa_decode_layer_workspace_bytes(sel_cfg, attn_cfg, nq, max_ctx, n_split)
    return torch.zeros(max(n, 16), dtype=torch.uint8, device=device)


def decode_layer_error(ws) -> int:
    """The sticky error word of a qsa_decode_layer workspace (its first 4
    bytes, uint32): 0 when every bounded wait of the calls made on it since
    it was zero-filled ended in time. Reading it synchronises with the
    device."""
    return int(ws[:4].view(torch.int32).item()) & 0xFFFFFFFF


def check_decode_layer_error(ws) -> None:
    """Raise QsaError if the workspace's error word is set (the outputs of
    the calls that set it are unspecified)."""
    e = decode_layer_error(ws)
    if e:
        raise QsaError("qsa_decode_layer", 4, f"error word {e:#x}: a bounded wait in the layer ran out")


def _decode_layer_args(fn, sel_cfg, attn_cfg, q_ctx, max_ctx, q_idx, keys, q, kv, scores, sel, n_sel, n_split,
                       o_out, o_out_bf16, lse_out, q_seq):
    nq = q_ctx.shape[0]
    _rowmajor_tail(q_idx, "q_idx", 3)
    if scores is not None:
        _rowmajor_tail(scores, "scores", 1)
    kp, kss = _keys_arg(sel_cfg, keys, max_ctx, fn)
    if sel.shape != (nq, sel_cfg.topk) or not sel.is_contiguous():
        raise ValueError(f"{fn}: sel must be a contiguous [nq, topk] tensor")
    if not q.is_contiguous():
        raise ValueError(f"{fn}: q must be contiguous")
    for t, shp, name in ((o_out, (nq, attn_cfg.hq, attn_cfg.dv), "o_out"),
                         (o_out_bf16, (nq, attn_cfg.hq, attn_cfg.dv), "o_out_bf16"),
                         (lse_out, (nq, attn_cfg.hq), "lse_out")):
        if t is not None and (tuple(t.shape) != shp or not t.is_contiguous()):
            raise ValueError(f"{fn}: {name} must be a contiguous {list(shp)} tensor")
    return [ctypes.byref(sel_cfg), ctypes.byref(attn_cfg), nq, _dev(q_seq, _I32, "q_seq"), _dev(q_ctx, _I32, "q_ctx"),
            max_ctx, _dev(q_idx, _BF16, "q_idx"), kp, kss, _dev(q, _BF16, "q"),
            ctypes.byref(kv), _dev(scores, _F32, "scores"), scores.stride(0) if scores is not None else 0,
            _dev(sel, _I32, "sel"),
            _dev(n_sel, _I32, "n_sel"), n_split, _dev(o_out, _F32, "o_out"), _dev(o_out_bf16, _BF16, "o_out_bf16"),
            _dev(lse_out, _F32, "lse_out")]


def qsa_decode_layer(sel_cfg, attn_cfg, q_ctx, max_ctx, q_idx, keys, q, kv, scores, sel, n_sel, n_split, ws,
                     o_out=None, o_out_bf16=None, lse_out=None, q_seq=None, stream=None):
    """One decode layer (two launches): qsa_index_topk, then qsa_sparse_decode
    and qsa_lse_merge. q_idx: [nq, 1, 128] bf16; keys: [n_seq, n_blocks, 128]
    bf16 (or FP8 pages, see qsa_index_scores); q: [nq, hq, dk] bf16; scores/sel/n_sel as qsa_index_topk
    (scores may be None: no scores are written, see include/qsa.h);
    o_out: [nq, hq, dv] fp32, o_out_bf16: [nq, hq, dv] bf16, lse_out: [nq, hq]
    fp32 (each optional); ws: decode_layer_workspace(...)."""
    args = _decode_layer_args("qsa_decode_layer", sel_cfg, attn_cfg, q_ctx, max_ctx, q_idx, keys, q, kv, scores, sel,
                              n_sel, n_split, o_out, o_out_bf16, lse_out, q_seq)
    _check("qsa_decode_layer", lib().qsa_decode_layer(
        *args, ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(), _stream(stream)))


def qsa_decode_layer_noalloc(sel_cfg, attn_cfg, q_ctx, max_ctx, q_idx, keys, q, kv, scores, sel, n_sel, n_split,
                             o_out=None, o_out_bf16=None, lse_out=None, q_seq=None, stream=None):
    """qsa_decode_layer without a workspace argument: the library's static
    device scratch (16 MiB per device) serves as the workspace. Calls on one
    device must not overlap."""
    args = _decode_layer_args("qsa_decode_layer_noalloc", sel_cfg, attn_cfg, q_ctx, max_ctx, q_idx, keys, q, kv,
                              scores, sel, n_sel, n_split, o_out, o_out_bf16, lse_out, q_seq)
    _check("qsa_decode_layer_noalloc", lib().qsa_decode_layer_noalloc(*args, _stream(stream)))


def qsa_decode_layer_latent_workspace_bytes(sel_cfg, attn_cfg, nq, max_ctx, n_split) -> int:
    return int(lib().qsa_decode_layer_latent_workspace_bytes(ctypes.byref(sel_cfg), ctypes.byref(attn_cfg), nq,
                                                             max_ctx, n_split))


def decode_layer_latent_workspace(sel_cfg, attn_cfg, nq, max_ctx, n_split, device="cuda"):
    """A workspace tensor for qsa_decode_layer_latent (no state is kept in it
    between calls)."""
    n = qsa_decode_layer_latent_workspace_bytes(sel_cfg, attn_cfg, nq, max_ctx, n_split)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def qsa_decode_layer_latent(sel_cfg, attn_cfg, q_ctx, max_ctx, q_idx, w_idx, keys, q, kv, scores, sel, n_sel,
                            n_split, ws, o_out=None, o_out_bf16=None, lse_out=None, q_seq=None, stream=None):
    """One decode layer of the shared-latent variant (three launches):
    qsa_index_scores, qsa_topk_blocks, qsa_sparse_decode and qsa_lse_merge.
    q_idx: [nq, 4, 64] bf16; w_idx: [nq, 4] fp32; keys: [n_seq, n_keys, 64]
    bf16 (or FP8 pages); q: [nq, 64, 576] bf16; kv: bf16 latent rows;
    scores/sel/n_sel as qsa_index_scores / qsa_topk_blocks write them;
    outputs as qsa_decode_layer; ws: decode_layer_latent_workspace(...)."""
    fn = "qsa_decode_layer_latent"
    args = _decode_layer_args(fn, sel_cfg, attn_cfg, q_ctx, max_ctx, q_idx, keys, q, kv, scores, sel, n_sel,
                              n_split, o_out, o_out_bf16, lse_out, q_seq)
    if w_idx is None or tuple(w_idx.shape) != (q_ctx.shape[0], 4) or not w_idx.is_contiguous():
        raise ValueError(f"{fn}: w_idx must be a contiguous [nq, 4] tensor")
    args.insert(7, _dev(w_idx, _F32, "w_idx"))
    _check(fn, lib().qsa_decode_layer_latent(
        *args, ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(), _stream(stream)))


def qsa_kv_append(sel_cfg, attn_cfg, q_pos, k_new, kv, v_new=None, raw_new=None, raw_keys=None, pooled=None,
                  q_seq=None, stream=None):
    """Write one new token per query into the cache at q_pos (device int32
    [nq]): k_new [nq, hkv, dk] (and v_new [nq, hkv, dv] unless the cache's v
    is its k), raw_new [nq, idx_dim] into raw_keys [n_seq, capacity, idx_dim],
    and the pooled key [n_seq, n_blocks, idx_dim] of each block a token
    completes (for an FP8 sel_cfg: quantized into the uint8 [n_seq, bytes]
    page buffer). kv: make_kv(...) of the cache."""
    nq = q_pos.shape[0]
    for t, name in ((k_new, "k_new"), (v_new, "v_new"), (raw_new, "raw_new")):
        if t is not None and (t.shape[0] != nq or not t.is_contiguous()):
            raise ValueError(f"qsa_kv_append: {name} must be contiguous with {nq} rows")
    fp8 = sel_cfg.key_format == KEYS_FP8
    raw_fp8 = fp8 and sel_cfg.block == 1  # the token key is the indexer key: FP8 pages
    if raw_keys is not None:
        if raw_fp8 and (raw_keys.dim() != 2 or raw_keys.stride(1) != 1):
            raise ValueError("qsa_kv_append: FP8 token keys must be a uint8 [n_seq, bytes] page buffer")
        if not raw_fp8:
            _rowmajor_tail(raw_keys, "raw_keys", 2)
    if pooled is not None:
        if fp8 and (pooled.dim() != 2 or pooled.stride(1) != 1):
            raise ValueError("qsa_kv_append: FP8 pooled keys must be a uint8 [n_seq, bytes] page buffer")
        if not fp8:
            _rowmajor_tail(pooled, "pooled", 2)
    _check("qsa_kv_append", lib().qsa_kv_append(
        ctypes.byref(sel_cfg), ctypes.byref(attn_cfg), nq, _dev(q_seq, _I32, "q_seq"), _dev(q_pos, _I32, "q_pos"),
        _dev(k_new, _BF16, "k_new"), _dev(v_new, _BF16, "v_new"), _dev(raw_new, _BF16, "raw_new"), ctypes.byref(kv),
        _dev(raw_keys, _U8 if raw_fp8 else _BF16, "raw_keys"), 0 if raw_keys is None else raw_keys.stride(0),
        _dev(pooled, _U8 if fp8 else _BF16, "pooled"), 0 if pooled is None else pooled.stride(0), _stream(stream)))


_hip = None


def _kv_address(t, name):
    """Device address of a K/V tensor: device memory as is; pinned host memory
    (torch.empty(..., pin_memory=True)) through the address HIP maps it to,
    so kernels read it over the host link. Anything else is refused."""
    global _hip
    if t.dtype not in _BF16 + _U8:
        raise TypeError(f"{name} has dtype {t.dtype}, expected bf16 (or uint8 FP8 rows)")
    if t.is_cuda:
        return t.data_ptr()
    if not t.is_pinned():
        raise ValueError(f"{name} must be a CUDA tensor or pinned host memory")
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_uint]
    dptr = ctypes.c_void_p()
    err = _hip.hipHostGetDevicePointer(ctypes.byref(dptr), ctypes.c_void_p(t.data_ptr()), 0)
    if err != 0 or not dptr.value:
        raise ValueError(f"{name}: pinned host memory is not mapped for the device (hip error {err})")
    return dptr.value


def make_kv(k, v=None):
    """KV descriptor of k, v: [n_seq, capacity, hkv, d] bf16 (v defaults to k),
    in device memory or in pinned host memory (read zero-copy); or of FP8
    sparse-MLA rows: k a uint8 [n_seq, capacity, 656] tensor (v None)."""
    if k.dtype == torch.uint8:
        if v is not None or k.dim() != 3 or k.shape[2] != FP8_MLA_ROW or k.stride(2) != 1:
            raise ValueError("FP8 rows: k must be a uint8 [n_seq, capacity, 656] tensor, v None")
        addr = ctypes.c_void_p(_kv_address(k, "k"))
        kv = KV(addr, addr, k.stride(0), k.stride(1), 0, k.shape[1], KV_FP8_MLA)
        kv._keep = (k,)
        return kv
    if v is None:
        v = k
    for t, name in ((k, "k"), (v, "v")):
        if t.dim() != 4 or t.stride(3) != 1:
            raise ValueError(f"{name} must be [n_seq, capacity, hkv, d] with unit last stride")
    if k.stride()[:3] != v.stride()[:3] or k.shape[:2] != v.shape[:2]:
        raise ValueError("k and v must share their sequence, token and head strides")
    kv = KV(ctypes.c_void_p(_kv_address(k, "k")), ctypes.c_void_p(_kv_address(v, "v")), k.stride(0), k.stride(1),
            k.stride(2), k.shape[1], KV_BF16)
    kv._keep = (k, v)
    return kv


def qsa_sparse_decode(sel_cfg, attn_cfg, q_ctx, max_ctx, q, kv, sel, n_sel, n_split, o_part, lse_part,
                      q_seq=None, stream=None):
    """q: [nq, hq, dk] bf16; kv: make_kv(...); o_part: [n_split, nq, hq, dv] fp32;
    lse_part: [n_split, nq, hq] fp32."""
    nq = q_ctx.shape[0]
    if not q.is_contiguous() or not o_part.is_contiguous() or not lse_part.is_contiguous():
        raise ValueError("q, o_part and lse_part must be contiguous")
    if tuple(o_part.shape) != (n_split, nq, attn_cfg.hq, attn_cfg.dv):
        raise ValueError("o_part must be [n_split, nq, hq, dv]")
    if tuple(lse_part.shape) != (n_split, nq, attn_cfg.hq):
        raise ValueError("lse_part must be [n_split, nq, hq]")
    _check("qsa_sparse_decode", lib().qsa_sparse_decode(
        ctypes.byref(sel_cfg), ctypes.byref(attn_cfg), nq, _dev(q_seq, _I32, "q_seq"),
        _dev(q_ctx, _I32, "q_ctx"), max_ctx, _dev(q, _BF16, "q"), ctypes.byref(kv),
        _dev(sel, _I32, "sel"), _dev(n_sel, _I32, "n_sel"), n_split, _dev(o_part, _F32, "o_part"),
        _dev(lse_part, _F32, "lse_part"), _stream(stream)))


def qsa_row_cache_bytes(attn_cfg, n_slots):
    """Bytes of an HBM row cache of n_slots rows (0: shape not supported)."""
    return lib().qsa_row_cache_bytes(ctypes.byref(attn_cfg), n_slots)


def qsa_decode_cached_plan_bytes(sel_cfg, nq):
    return lib().qsa_decode_cached_plan_bytes(ctypes.byref(sel_cfg), nq)


def row_cache_empty(attn_cfg, n_slots, device="cuda"):
    """A zero-filled row cache (uint8 device tensor) of n_slots rows."""
    n = qsa_row_cache_bytes(attn_cfg, n_slots)
    if n == 0:
        raise ValueError("row cache: unsupported attention shape or slot count")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def qsa_row_cache_step(attn_cfg, cache, n_slots, row_pos, kv, row_seq=None, stream=None):
    """Advance the cache's epoch and drop the rows at (row_seq[j], row_pos[j])
    (int32 device tensors; row_seq None: sequence j)."""
    n_rows = 0 if row_pos is None else row_pos.shape[0]
    _check("qsa_row_cache_step", lib().qsa_row_cache_step(
        ctypes.byref(attn_cfg), _dev(cache, _U8, "cache"), cache.numel(), n_slots, n_rows,
        _dev(row_seq, _I32, "row_seq"), _dev(row_pos, _I32, "row_pos"), ctypes.byref(kv), _stream(stream)))


def qsa_sparse_decode_cached(sel_cfg, attn_cfg, q_ctx, max_ctx, q, kv, sel, n_sel, n_split, o_part, lse_part,
                             cache, n_slots, plan_ws, q_seq=None, stream=None):
    """qsa_sparse_decode reading rows through the HBM row cache `cache`
    (row_cache_empty); plan_ws: device tensor of at least
    qsa_decode_cached_plan_bytes(sel_cfg, nq) bytes."""
    nq = q_ctx.shape[0]
    if not q.is_contiguous() or not o_part.is_contiguous() or not lse_part.is_contiguous():
        raise ValueError("q, o_part and lse_part must be contiguous")
    if tuple(o_part.shape) != (n_split, nq, attn_cfg.hq, attn_cfg.dv):
        raise ValueError("o_part must be [n_split, nq, hq, dv]")
    if tuple(lse_part.shape) != (n_split, nq, attn_cfg.hq):
        raise ValueError("lse_part must be [n_split, nq, hq]")
    if not plan_ws.is_contiguous():
        raise ValueError("plan_ws must be contiguous")
    _check("qsa_sparse_decode_cached", lib().qsa_sparse_decode_cached(
        ctypes.byref(sel_cfg), ctypes.byref(attn_cfg), nq, _dev(q_seq, _I32, "q_seq"),
        _dev(q_ctx, _I32, "q_ctx"), max_ctx, _dev(q, _BF16, "q"), ctypes.byref(kv),
        _dev(sel, _I32, "sel"), _dev(n_sel, _I32, "n_sel"), n_split, _dev(o_part, _F32, "o_part"),
        _dev(lse_part, _F32, "lse_part"), _dev(cache, _U8, "cache"), cache.numel(), n_slots,
        _dev(plan_ws, _U8 + _I32, "plan_ws"), plan_ws.numel() * plan_ws.element_size(), _stream(stream)))


def qsa_sparse_prefill(sel_cfg, attn_cfg, q_ctx, max_ctx, q, kv, sel, n_sel, tile_begin, tile_end,
                       o_part, lse_part, q_seq=None, stream=None):
    """q: [nq, hq, dk] bf16; o_part: [nq, hq, dv] fp32; lse_part: [nq, hq] fp32."""
    nq = q_ctx.shape[0]
    if not q.is_contiguous() or not o_part.is_contiguous() or not lse_part.is_contiguous():
        raise ValueError("q, o_part and lse_part must be contiguous")
    if tuple(o_part.shape[-3:]) != (nq, attn_cfg.hq, attn_cfg.dv) or tuple(lse_part.shape[-2:]) != (nq, attn_cfg.hq):
        raise ValueError("o_part must end in [nq, hq, dv] and lse_part in [nq, hq]")
    _check("qsa_sparse_prefill", lib().qsa_sparse_prefill(
        ctypes.byref(sel_cfg), ctypes.byref(attn_cfg), nq, _dev(q_seq, _I32, "q_seq"),
        _dev(q_ctx, _I32, "q_ctx"), max_ctx, _dev(q, _BF16, "q"), ctypes.byref(kv),
        _dev(sel, _I32, "sel"), _dev(n_sel, _I32, "n_sel"), tile_begin, tile_end,
        _dev(o_part, _F32, "o_part"), _dev(lse_part, _F32, "lse_part"), _stream(stream)))


def qsa_sparse_prefill_merge(sel_cfg, attn_cfg, q_ctx, max_ctx, q, kv, sel, n_sel, tile_begin, tile_end, first,
                             last, o_run, lse_run, o_out_bf16=None, q_seq=None, stream=None):
    """One history tile merged into the running result: o_run [nq, hq, dv] fp32, lse_run [nq, hq] fp32 (read
    unless first, written); with last, the merged output also goes to o_out_bf16 [nq, hq, dv] bf16 if given."""
    nq = q_ctx.shape[0]
    if not q.is_contiguous() or not o_run.is_contiguous() or not lse_run.is_contiguous():
        raise ValueError("q, o_run and lse_run must be contiguous")
    if tuple(o_run.shape) != (nq, attn_cfg.hq, attn_cfg.dv) or tuple(lse_run.shape) != (nq, attn_cfg.hq):
        raise ValueError("o_run must be [nq, hq, dv] and lse_run [nq, hq]")
    if o_out_bf16 is not None and (tuple(o_out_bf16.shape) != tuple(o_run.shape) or not o_out_bf16.is_contiguous()):
        raise ValueError("o_out_bf16 must be a contiguous [nq, hq, dv] tensor")
    _check("qsa_sparse_prefill_merge", lib().qsa_sparse_prefill_merge(
        ctypes.byref(sel_cfg), ctypes.byref(attn_cfg), nq, _dev(q_seq, _I32, "q_seq"),
        _dev(q_ctx, _I32, "q_ctx"), max_ctx, _dev(q, _BF16, "q"), ctypes.byref(kv),
        _dev(sel, _I32, "sel"), _dev(n_sel, _I32, "n_sel"), tile_begin, tile_end, int(bool(first)),
        int(bool(last)), _dev(o_run, _F32, "o_run"), _dev(lse_run, _F32, "lse_run"),
        _dev(o_out_bf16, _BF16, "o_out_bf16"), _stream(stream)))


def qsa_lse_merge(o_parts, lse_parts, o_out=None, o_out_bf16=None, lse_out=None, stream=None):
    """o_parts: [P, rows..., dv] fp32 (contiguous rows); lse_parts: [P, rows...] fp32."""
    n_part = o_parts.shape[0]
    dv = o_parts.shape[-1]
    rows = lse_parts[0].numel()
    if o_parts[0].numel() != rows * dv:
        raise ValueError("o_parts and lse_parts disagree on the number of rows")
    _rowmajor_tail(o_parts, "o_parts", o_parts.dim() - 1)
    _rowmajor_tail(lse_parts, "lse_parts", lse_parts.dim() - 1)
    _check("qsa_lse_merge", lib().qsa_lse_merge(
        n_part, rows, dv, _dev(o_parts, _F32, "o_parts"), o_parts.stride(0),
        _dev(lse_parts, _F32, "lse_parts"), lse_parts.stride(0), _dev(o_out, _F32, "o_out"),
        _dev(o_out_bf16, _BF16, "o_out_bf16"), _dev(lse_out, _F32, "lse_out"), _stream(stream)))
