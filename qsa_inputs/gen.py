"""Host (numpy) implementation of the counter-based input generator.

See the package docstring for the definition. Nothing here knows about
attention, pooling or selection.
"""
from __future__ import annotations

import statistics

import numpy as np

G = 0x9E3779B97F4A7C15  # SplitMix64 increment (golden-ratio constant)
H = 0xD1B54A32D192ED03  # odd multiplier used only to spread stream ids
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK = (1 << 64) - 1

# Tensor kinds, used to derive independent streams per (layer, sequence).
KIND = {
    "q": 1, "q_idx": 2, "k": 3, "v": 4, "raw_key": 5, "w_idx": 6,
    "latent": 7, "scores": 8, "misc": 9,
}


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function on a uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def _mix64_int(z: int) -> int:
    z &= _MASK
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
    return z ^ (z >> 31)


def stream_key(seed: int, stream: int) -> int:
    return _mix64_int(((seed * G) & _MASK) ^ ((stream * H) & _MASK))


def config_seed(config_id: int) -> int:
    """Fixed seed per workload: 0x51A5EED0 + workload number."""
    return 0x51A5EED0 + int(config_id)


def stream_id(layer: int, seq: int, kind: str, salt: int = 0) -> int:
    """Stream number of one tensor of one (layer, sequence) unit."""
    return ((((int(salt) * 256 + int(layer)) * 65536 + int(seq)) * 16) + KIND[kind]) & _MASK


def _mix64_inplace(z: np.ndarray, t: np.ndarray) -> None:
    """mix64 applied in place to z (t: scratch of the same shape)."""
    np.right_shift(z, np.uint64(30), out=t)
    np.bitwise_xor(z, t, out=z)
    np.multiply(z, _M1, out=z)
    np.right_shift(z, np.uint64(27), out=t)
    np.bitwise_xor(z, t, out=z)
    np.multiply(z, _M2, out=z)
    np.right_shift(z, np.uint64(31), out=t)
    np.bitwise_xor(z, t, out=z)


def words(seed: int, stream: int, word_index: np.ndarray) -> np.ndarray:
    """The SplitMix64 outputs with the given indices (0-based) of one stream."""
    key = np.uint64(stream_key(seed, stream))
    wi = np.asarray(word_index, dtype=np.uint64).reshape(-1)
    out = np.empty(wi.size, dtype=np.uint64)
    chunk = 1 << 20
    t = np.empty(min(chunk, max(1, wi.size)), dtype=np.uint64)
    for a in range(0, wi.size, chunk):
        z = out[a:a + chunk]
        tt = t[: z.size]
        np.add(wi[a:a + chunk], np.uint64(1), out=z)
        np.multiply(z, np.uint64(G), out=z)
        np.add(z, key, out=z)
        _mix64_inplace(z, tt)
    return out.reshape(np.shape(word_index))


def codes(seed: int, stream: int, index: np.ndarray) -> np.ndarray:
    """16-bit codes of the given element indices of one stream."""
    idx = np.asarray(index, dtype=np.uint64)
    u = words(seed, stream, idx >> np.uint64(2))
    shift = np.uint64(48) - np.uint64(16) * (idx & np.uint64(3))
    return ((u >> shift) & np.uint64(0xFFFF)).astype(np.uint16)


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


_TABLE = None


def normal_table() -> np.ndarray:
    """65536 bf16 bit patterns: N(0,1) quantiles at (c + 0.5) / 65536."""
    global _TABLE
    if _TABLE is None:
        nd = statistics.NormalDist()
        q = np.array([nd.inv_cdf((c + 0.5) / 65536.0) for c in range(65536)], dtype=np.float64)
        _TABLE = _f32_to_bf16_bits(q.astype(np.float32))
        _TABLE.setflags(write=False)
    return _TABLE


def _codes_range(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """16-bit codes of elements [start, start + count): each word hashed once."""
    w0, w1 = start >> 2, (start + count + 3) >> 2
    u = words(seed, stream, np.arange(w0, w1, dtype=np.uint64))
    # little-endian uint16 view of a word holds lanes 3, 2, 1, 0 (lane 0 = most significant)
    c = u.view(np.uint16).reshape(-1, 4)[:, ::-1].reshape(-1)
    off = start - 4 * w0
    return c[off: off + count]


def normal_bf16(seed: int, stream: int, start: int, count: int = None, index=None) -> np.ndarray:
    """bf16 bit patterns of elements [start, start+count) (or the given indices)."""
    if index is None:
        return normal_table()[_codes_range(seed, stream, start, count)]
    return normal_table()[codes(seed, stream, index)]


def ar1_normal_bf16(seed: int, stream: int, n_rows: int, dim: int, rho: float) -> np.ndarray:
    """bf16 bit patterns [n_rows][dim] of a first-order autoregressive
    sequence of standard-normal vectors: x_0 = z_0 and
    x_r = rho * x_{r-1} + sqrt(1 - rho**2) * z_r, computed in float64 from
    z = normal_bf16 elements of (seed, stream) (row-major), then rounded to
    fp32 and to bf16 (nearest, ties to even). Neighbouring rows have
    correlation rho; each row is N(0, 1) per element."""
    z = bf16_bits_to_f32(normal_bf16(seed, stream, 0, n_rows * dim)).astype(np.float64).reshape(n_rows, dim)
    x = np.empty_like(z)
    c = float(np.sqrt(1.0 - rho * rho))
    x[0] = z[0]
    for r in range(1, n_rows):
        x[r] = rho * x[r - 1] + c * z[r]
    return _f32_to_bf16_bits(x.astype(np.float32))


def uniform_f32(seed: int, stream: int, count: int, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    """fp32 values on a 2**-24 grid of [lo, hi) (exactly representable)."""
    u = words(seed, stream, np.arange(count, dtype=np.uint64))
    frac = (u >> np.uint64(40)).astype(np.float64) / float(1 << 24)
    return (lo + (hi - lo) * frac).astype(np.float32)


def tie_heavy_f32(seed: int, stream: int, count: int, levels: int = 64) -> np.ndarray:
    """fp32 values drawn from a few levels (many exact ties, includes -0.0 and +0.0)."""
    u = words(seed, stream, np.arange(count, dtype=np.uint64))
    lev = (u >> np.uint64(40)).astype(np.int64) % levels - levels // 2
    out = (lev.astype(np.float32) * np.float32(0.25))
    neg0 = ((u >> np.uint64(8)) & np.uint64(7)) == 0
    out[(lev == 0) & neg0] = np.float32(-0.0)
    return out
