"""Seeded synthetic inputs for indexer-selected sparse attention.

This module is the only code that both the CPU oracle side (tests, the CPU
baseline) and the GPU side use. It holds none of the attention method's
arithmetic: it only turns (seed, stream, element index) into numbers.

Definition (identical on the host here and in the GPU fill kernel
``qsa_inputs/fill.hip``):

* ``key(seed, stream) = mix64(seed * G ^ stream * H)`` (all arithmetic mod 2**64)
* element ``i`` of a stream takes the 64-bit word
  ``u = mix64(key + (i // 4 + 1) * G)``, i.e. the ``(i // 4)``-th output of a
  SplitMix64 generator started at ``key`` (Steele, Lea and Flood, "Fast
  splittable pseudorandom number generators", OOPSLA 2014), and uses its
  16-bit lane ``c = (u >> (48 - 16 * (i % 4))) & 0xFFFF``;
* a bf16 "N(0,1)" element is ``NORMAL_TABLE[c]``: the standard-normal
  quantile at ``(c + 0.5) / 65536`` rounded to bf16 (inverse-CDF sampling
  at 16-bit resolution, so values lie within about +-4.3).

Because every element is addressable by index, the oracle side can
regenerate exactly the rows it needs of a tensor the GPU filled whole.
"""
from .gen import (  # noqa: F401
    G, H, mix64, stream_key, words, codes, normal_table, normal_bf16,
    uniform_f32, tie_heavy_f32, ar1_normal_bf16, stream_id, config_seed, KIND,
    bf16_bits_to_f32,
)
