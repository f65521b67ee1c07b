"""Tunes the correlated-selection workload of the 1M-token decode and records
it in correlated_overlap_decode.txt.

"125B MoE を 3090 3 枚で運用する vLLM 最適化編", section 5 (decode, third part): the indexer's
selections at consecutive decode steps overlap by 60-85%, 0.72 on average
with the previous step and 0.86 with the union of the previous four. The
decode workload here is one layer of the batch-4 step at 1,048,320 tokens
(262,080 candidate blocks, top-512): its pooled keys are those of the
benchmark's layer 0, and the indexer queries of consecutive steps follow an
AR(1) sequence (qsa_inputs.ar1_normal_bf16, the stream the benchmark uses)
with the correlation rho chosen here so that consecutive selections overlap
by 0.72 on average. A selection among 262,080 blocks moves more per step
than one among the 15,000 of the prefill workload, so the rho is higher
than that workload's. Everything below the input generation is the
oracle's: pooling, scores and selection.
Run: python tests/golden/correlated_overlap_decode.py (a few minutes).
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import qsa_inputs as qi  # noqa: E402
from oracle import qsa_oracle as orc  # noqa: E402

CTX, BATCH, CONFIG, TOPK, BLOCK = 1048320, 4, 3, 512, 4
STEPS = 48  # the benchmark's warm-up + timed steps
TARGET = 0.72


def pooled_keys(s):
    seed = qi.config_seed(CONFIG)
    raw = qi.normal_bf16(seed, qi.stream_id(0, s, "raw_key"), 0, CTX * 128).reshape(CTX, 128)
    return orc.pool_keys(raw, BLOCK)


def queries(s, rho, n):
    seed = qi.config_seed(CONFIG)
    return qi.ar1_normal_bf16(seed, qi.stream_id(0, s, "q_idx", salt=2), n, 128, rho)


def selections(pooled, q_idx):
    return [set(orc.select_blocks(orc.index_scores(q_idx[t], pooled, CTX // BLOCK), CTX, BLOCK, TOPK).tolist())
            for t in range(q_idx.shape[0])]


def overlaps(sels):
    prev = [len(sels[t] & sels[t - 1]) / TOPK for t in range(1, len(sels))]
    union4 = [len(sels[t] & set().union(*sels[t - 4:t])) / TOPK for t in range(4, len(sels))]
    return prev, union4


def main():
    p0 = pooled_keys(0)
    lo, hi = 0.9, 0.99999
    for _ in range(10):
        mid = 0.5 * (lo + hi)
        ov = float(np.mean(overlaps(selections(p0, queries(0, mid, 24)))[0]))
        print(f"rho {mid:.6f}: mean overlap {ov:.4f} (sequence 0, 24 steps)", flush=True)
        if ov < TARGET:
            lo = mid
        else:
            hi = mid
    rho = round(0.5 * (lo + hi), 5)
    prev, union4 = [], []
    for s in range(BATCH):
        p = p0 if s == 0 else pooled_keys(s)
        a, b = overlaps(selections(p, queries(s, rho, STEPS)))
        prev += a
        union4 += b
        print(f"sequence {s}: overlap {np.mean(a):.4f}", flush=True)
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "correlated_overlap_decode.txt")
    with open(out, "w") as f:
        f.write("# correlated-selection workload of the decode (written by correlated_overlap_decode.py; oracle\n")
        f.write("# selection): one layer of the batch-4 step at 1,048,320 tokens, top-512 of the 4-token blocks,\n")
        f.write(f"# {STEPS} consecutive steps per sequence; indexer queries AR(1) over steps with correlation rho\n")
        f.write(f"rho {rho}\n")
        f.write(f"mean_overlap_previous {np.mean(prev):.4f}\n")
        f.write(f"mean_overlap_union4 {np.mean(union4):.4f}\n")
        f.write(f"min_overlap_previous {np.min(prev):.4f}\n")
        f.write(f"max_overlap_previous {np.max(prev):.4f}\n")
    print(open(out).read())


if __name__ == "__main__":
    main()
