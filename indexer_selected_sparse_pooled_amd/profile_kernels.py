"""Small, fixed workload for hardware-counter runs (rocprofv3 --pmc).

Runs, each `--reps` times, on seeded synthetic inputs already in HBM:
  * a plain device copy of 256 MiB (torch copy_): the reference that scales
    the memory counters (it reads and writes exactly 268,435,456 bytes);
  * one layer of the 1,048,320-token batch-4 decode step: qsa_index_topk
    (pooled-key scan + exact top-512), qsa_sparse_decode, qsa_lse_merge,
    and the same layer as one qsa_decode_layer call with no score buffer
    (two launches), with bf16 and with FP8 pooled keys;
  * one history tile of the 4096-query prefill chunk (qsa_sparse_prefill);
  * the shared-latent prefill attention of 2048 queries at context 131,072
    (one qsa_sparse_prefill over the whole history);
  * the shared-latent decode step at batch 8, context 131,072, as one
    qsa_decode_layer_latent call.
`--parts` picks a subset (copy, decode, prefill, mla, mladecode).
`--useful-out FILE` writes, per MFMA kernel of these workloads, the useful
FLOPs of one dispatch (the contraction the method needs: selected tokens
only, causal keys only), computed on the host from the run's own
selections; `--counters ... --useful FILE` then reports executed bf16 MFMA
work (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) over it.

Usage (one counter group per run):
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT -o run -- \
      python <repo>/indexer_selected_sparse_pooled_amd/profile_kernels.py

Summaries of rocprofv3 CSV output (host only, no GPU):
  python profile_kernels.py --trace OUT/run_kernel_trace.csv
  python profile_kernels.py --pmc FETCH/run_counter_collection.csv WRITE/run_counter_collection.csv
  python profile_kernels.py --counters A/run_counter_collection.csv [B/...] [--useful FILE]   (MFMA, LDS, waits)
The counter summary scales each memory counter by what it reads for the
256 MiB copy, so its figures are bytes moved to and from memory.
"""
from __future__ import annotations

import argparse
import collections
import csv
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

COPY_BYTES = 256 << 20
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def kernel_name(raw: str) -> str:
    n = raw.replace("(anonymous namespace)::", "").replace("qsa::", "")
    n = re.sub(r"\(.*", "", n).replace("void ", "")
    return n.strip()[:40]


def summarize_trace(path: str) -> str:
    """Per (kernel, grid): launches and average / min / max duration (us)."""
    g = collections.OrderedDict()
    for r in csv.DictReader(open(path)):
        wg = int(r["Workgroup_Size_X"])
        key = (kernel_name(r["Kernel_Name"]), f'{int(r["Grid_Size_X"]) // wg}x{r["Grid_Size_Y"]}', wg,
               r["VGPR_Count"], r["Accum_VGPR_Count"], r["LDS_Block_Size"])
        g.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    out = [f"{'kernel':40s} {'grid(wg)':>10s} {'wg':>5s} {'vgpr':>4s} {'agpr':>4s} {'lds':>6s} {'calls':>6s} "
           f"{'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    for (n, grid, wg, v, a, lds), ds in sorted(g.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"{n:40s} {grid:>10s} {wg:5d} {v:>4s} {a:>4s} {lds:>6s} {len(ds):6d} {sum(ds) / len(ds):9.2f} "
                   f"{min(ds):9.2f} {max(ds):9.2f}")
    return "\n".join(out)


def _counter(path: str, name: str):
    g = collections.OrderedDict()
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != name:
            continue
        wg = int(r["Workgroup_Size"])
        key = (kernel_name(r["Kernel_Name"]), f'{int(r["Grid_Size"]) // wg}', wg)
        g.setdefault(key, []).append(float(r["Counter_Value"]))
    return g


def source_digest() -> str:
    """sha256 over the library's kernel sources (csrc/*.hip, *.hpp), so a
    counter summary can tell whether the kernels changed since."""
    import hashlib
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".hpp")):
            h.update(name.encode())
            h.update(open(os.path.join(d, name), "rb").read())
    return h.hexdigest()


def summarize_pmc(fetch_csv: str, write_csv: str) -> str:
    """Per (kernel, grid): FETCH_SIZE and WRITE_SIZE per dispatch (KiB as
    read), and bytes after scaling by the copy reference."""
    f, w = _counter(fetch_csv, "FETCH_SIZE"), _counter(write_csv, "WRITE_SIZE")
    copy_f = [v for k, v in f.items() if k[0] == COPY_KERNEL]
    copy_w = [v for k, v in w.items() if k[0] == COPY_KERNEL]
    if not copy_f or not copy_w:
        raise SystemExit("no copy reference in the counter files")
    sf = COPY_BYTES / (1024.0 * sum(copy_f[0]) / len(copy_f[0]))
    sw = COPY_BYTES / (1024.0 * sum(copy_w[0]) / len(copy_w[0]))
    out = [f"source digest: {source_digest()}",
           f"scale: FETCH_SIZE x {sf:.4f}, WRITE_SIZE x {sw:.4f} (the {COPY_BYTES}-byte copy reads and writes "
           f"{COPY_BYTES} bytes)",
           f"{'kernel':40s} {'wgs':>8s} {'n':>3s} {'FETCH_KiB':>12s} {'WRITE_KiB':>12s} {'read_B':>14s} "
           f"{'written_B':>14s}"]
    for k, fv in f.items():
        wv = w.get(k, [0.0])
        fa, wa = sum(fv) / len(fv), sum(wv) / len(wv)
        out.append(f"{k[0]:40s} {k[1]:>8s} {len(fv):3d} {fa:12.1f} {wa:12.1f} {fa * 1024 * sf:14.0f} "
                   f"{wa * 1024 * sw:14.0f}")
    return "\n".join(out)


def summarize_counters(paths, useful=None) -> str:
    """Per (kernel, grid): the per-dispatch average of every counter found in
    the given counter_collection.csv files (one per rocprofv3 --pmc pass),
    and, where present: MFMA busy % (AMD's MfmaUtil: MFMA-busy cycles of all
    SIMDs over active cycles x SIMDs), executed bf16 MFMA work
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 FLOP), the LDS bank-conflict share of
    LDS-active cycles, and the share of wave cycles spent waiting."""
    g = collections.OrderedDict()
    names = []
    for path in paths:
        for r in csv.DictReader(open(path)):
            wg = int(r["Workgroup_Size"])
            key = (kernel_name(r["Kernel_Name"]), f'{int(r["Grid_Size"]) // wg}')
            c = r["Counter_Name"]
            if c not in names:
                names.append(c)
            g.setdefault(key, {}).setdefault(c, []).append(float(r["Counter_Value"]))
    out = [f"source digest: {source_digest()}", "counters: " + " ".join(names)]
    for (kern, grid), cs in g.items():
        avg = {c: sum(v) / len(v) for c, v in cs.items()}
        n = max(len(v) for v in cs.values())
        parts = [f"{kern} [{grid} wgs, {n} dispatches]"]
        parts += [f"  {c} {avg[c]:.6g}" for c in names if c in avg]
        if "MfmaUtil" in avg:
            parts.append(f"  => MFMA busy {avg['MfmaUtil']:.2f} %")
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in avg:
            ex = avg['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512
            parts.append(f"  => executed bf16 MFMA {ex / 1e9:.3f} GFLOP per dispatch")
            u = (useful or {}).get(kern)
            if u:
                parts.append(f"  => useful {u / 1e9:.3f} GFLOP per dispatch: executed / useful = {ex / u:.2f}")
        if "SQ_LDS_BANK_CONFLICT" in avg and avg.get("SQ_LDS_IDX_ACTIVE"):
            parts.append(f"  => LDS bank conflicts {100 * avg['SQ_LDS_BANK_CONFLICT'] / avg['SQ_LDS_IDX_ACTIVE']:.1f} % "
                         f"of LDS-active cycles")
        if "SQ_WAIT_INST_ANY" in avg and avg.get("SQ_WAVE_CYCLES"):
            parts.append(f"  => waiting on any instruction {100 * avg['SQ_WAIT_INST_ANY'] / avg['SQ_WAVE_CYCLES']:.1f} % "
                         f"of wave cycles" + (f", on LDS {100 * avg['SQ_WAIT_INST_LDS'] / avg['SQ_WAVE_CYCLES']:.1f} %"
                                              if "SQ_WAIT_INST_LDS" in avg else ""))
        out.append("\n".join(parts))
    return "\n".join(out)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--parts", default="copy,decode,prefill,mla")
    ap.add_argument("--trace", help="summarize a rocprofv3 kernel_trace.csv and exit")
    ap.add_argument("--pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarize two rocprofv3 counter_collection.csv files and exit")
    ap.add_argument("--counters", nargs="+", metavar="CSV",
                    help="summarize any rocprofv3 counter_collection.csv files (MFMA, LDS, waits) and exit")
    ap.add_argument("--useful", help="with --counters: the useful-FLOP file a run wrote (--useful-out)")
    ap.add_argument("--useful-out", help="write the useful FLOPs per dispatch of the MFMA kernels run here")
    args = ap.parse_args()
    if args.trace:
        print(summarize_trace(args.trace))
        return 0
    if args.counters:
        import json
        useful = json.load(open(args.useful)) if args.useful else None
        print(summarize_counters(args.counters, useful))
        return 0
    if args.pmc:
        print(summarize_pmc(*args.pmc))
        return 0
    import torch

    import indexer_selected_sparse_pooled_amd as pkg
    import qsa_inputs as qi
    from indexer_selected_sparse_pooled_amd import pipeline
    from qsa_inputs.gpu import fill_normal_bf16

    pkg.qsa.lib()
    parts = set(args.parts.split(","))
    useful = {}
    if "copy" in parts:
        copy_reference(torch, fill_normal_bf16, args.reps)
    if "decode" in parts:
        decode_layer(torch, pkg, qi, pipeline, fill_normal_bf16, args.reps)
    if "prefill" in parts:
        useful.update(prefill_tile(torch, pkg, qi, pipeline, fill_normal_bf16, args.reps))
    if "mla" in parts:
        useful.update(mla_prefill(torch, pkg, qi, pipeline, fill_normal_bf16, args.reps))
    if "mladecode" in parts:
        mla_decode(torch, pkg, qi, pipeline, fill_normal_bf16, args.reps)
    torch.cuda.synchronize()
    if args.useful_out:
        import json
        json.dump(useful, open(args.useful_out, "w"), indent=1)
    print("profile_kernels: done", flush=True)
    return 0


def copy_reference(torch, fill_normal_bf16, reps):
    dev = "cuda"
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    fill_normal_bf16(src, 1, 1)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()


def decode_layer(torch, pkg, qi, pipeline, fill_normal_bf16, reps):
    """One decode layer, 1,048,320-token context, batch 4."""
    dev = "cuda"
    L, B = 1048320, 4
    seed = qi.config_seed(3)
    keys = torch.empty(B, L // 4, 128, dtype=torch.bfloat16, device=dev)
    k = torch.empty(B, L, 2, 256, dtype=torch.bfloat16, device=dev)
    v = torch.empty(B, L, 2, 256, dtype=torch.bfloat16, device=dev)
    q = torch.empty(B, 16, 256, dtype=torch.bfloat16, device=dev)
    q_idx = torch.empty(B, 1, 128, dtype=torch.bfloat16, device=dev)
    for s in range(B):
        for t, kind in ((keys, "misc"), (k, "k"), (v, "v"), (q, "q"), (q_idx, "q_idx")):
            fill_normal_bf16(t[s], seed, qi.stream_id(0, s, kind))
    kv = pkg.make_kv(k, v)
    q_ctx = torch.full((B,), L, dtype=torch.int32, device=dev)
    q_seq = torch.arange(B, dtype=torch.int32, device=dev)
    bufs = pipeline.decode_buffers(pkg.SEL_A, pkg.ATTN_A, B, L)
    for _ in range(reps):
        pipeline.decode_layer(pkg.SEL_A, pkg.ATTN_A, q_ctx, L, q_idx, keys, q, kv, bufs, q_seq=q_seq)
    # the one-call layer as the headline runs it: no score buffer
    bufs_ns = pipeline.decode_buffers(pkg.SEL_A, pkg.ATTN_A, B, L, keep_scores=False)
    for _ in range(reps):
        pipeline.decode_layer(pkg.SEL_A, pkg.ATTN_A, q_ctx, L, q_idx, keys, q, kv, bufs_ns, q_seq=q_seq, fused=True)
    # the same layer over FP8 pooled keys (132 B per block)
    keys8 = pkg.fp8_keys_empty(B, L // 4, 128)
    pkg.qsa_quantize_keys(keys, keys8)
    for _ in range(reps):
        pipeline.decode_layer(pkg.SEL_A_FP8, pkg.ATTN_A, q_ctx, L, q_idx, keys8, q, kv, bufs_ns, q_seq=q_seq,
                              fused=True)
    torch.cuda.synchronize()
    del keys, keys8, k, v, kv, bufs, bufs_ns
    torch.cuda.empty_cache()


def prefill_tile(torch, pkg, qi, pipeline, fill_normal_bf16, reps):
    """One history tile of the prefill chunk: 4096 queries after 60,000 tokens."""
    dev = "cuda"
    H, C = 60000, 4096
    ctx_max = H + C
    seed = qi.config_seed(4)
    pooled = torch.empty(1, ctx_max // 4, 128, dtype=torch.bfloat16, device=dev)
    k = torch.empty(1, ctx_max, 2, 256, dtype=torch.bfloat16, device=dev)
    v = torch.empty(1, ctx_max, 2, 256, dtype=torch.bfloat16, device=dev)
    q = torch.empty(C, 16, 256, dtype=torch.bfloat16, device=dev)
    q_idx = torch.empty(C, 1, 128, dtype=torch.bfloat16, device=dev)
    for t, kind in ((pooled, "misc"), (k, "k"), (v, "v"), (q, "q"), (q_idx, "q_idx")):
        fill_normal_bf16(t, seed, qi.stream_id(0, 0, kind))
    kv = pkg.make_kv(k, v)
    q_ctx = torch.arange(H + 1, H + C + 1, dtype=torch.int32, device=dev)
    pb = pipeline.prefill_buffers(pkg.SEL_A, pkg.ATTN_A, C, ctx_max, 8192)
    for _ in range(reps):  # the indexer GEMM of the chunk (scores_gemm_a)
        pkg.qsa_index_scores(pkg.SEL_A, q_ctx, ctx_max, q_idx, pooled, pb.scores)
    pkg.qsa_topk_blocks(pkg.SEL_A, q_ctx, ctx_max, pb.scores, pb.sel, pb.n_sel, pb.ws)
    a0, a1 = pb.tiles[3]
    for _ in range(reps):
        pkg.qsa_sparse_prefill(pkg.SEL_A, pkg.ATTN_A, q_ctx, ctx_max, q, kv, pb.sel, pb.n_sel, a0, a1,
                               pb.o_tiles[3], pb.lse_tiles[3])
    torch.cuda.synchronize()
    # useful work: the indexer dot of every complete block before each query;
    # QK and PV (16 heads, 256 + 256 dims) over the query's selected tokens
    # inside the tile: its selected blocks' 4 tokens and its trailing tokens
    import numpy as np
    ctx = q_ctx.cpu().numpy().astype(np.int64)
    sel, ns = pb.sel.cpu().numpy(), pb.n_sel.cpu().numpy()
    att = 0
    for i in range(C):
        blk = sel[i, :ns[i]].astype(np.int64)
        att += int((np.clip(4 * blk + 4, a0, a1) - np.clip(4 * blk, a0, a1)).sum())
        tr0, tr1 = 4 * (ctx[i] // 4), ctx[i]  # the trailing tokens
        att += max(0, min(tr1, a1) - max(tr0, a0))
    useful = {"scores_gemm_a": float((ctx // 4).sum() * 128 * 2),
              "attend_a": float(att * 16 * (256 + 256) * 2)}
    del pb, k, v, kv
    torch.cuda.empty_cache()
    return useful


def mla_prefill(torch, pkg, qi, pipeline, fill_normal_bf16, reps):
    """Shared-latent prefill attention: 2048 queries at positions
    129,024..131,071, each over its top-2048 tokens, one history tile."""
    import numpy as np
    dev = "cuda"
    L, C = 131072, 2048
    seed = qi.config_seed(5)
    lat = torch.empty(1, L, 1, 576, dtype=torch.bfloat16, device=dev)
    keys = torch.empty(1, L, 64, dtype=torch.bfloat16, device=dev)
    q = torch.empty(C, 64, 576, dtype=torch.bfloat16, device=dev)
    q_idx = torch.empty(C, 4, 64, dtype=torch.bfloat16, device=dev)
    for t, kind in ((lat, "latent"), (keys, "raw_key"), (q, "q"), (q_idx, "q_idx")):
        fill_normal_bf16(t, seed, qi.stream_id(1, 0, kind))
    w = torch.tensor(qi.uniform_f32(seed, qi.stream_id(1, 0, "w_idx"), C * 4).reshape(C, 4), device=dev)
    kv = pkg.make_kv(lat, lat)
    q_ctx = torch.tensor(np.arange(L - C + 1, L + 1, dtype=np.int32), device=dev)
    pb = pipeline.prefill_buffers(pkg.SEL_B, pkg.ATTN_B, C, L, L)
    for _ in range(reps):  # the indexer GEMM of the chunk (scores_gemm_b)
        pkg.qsa_index_scores(pkg.SEL_B, q_ctx, L, q_idx, keys, pb.scores, w_idx=w)
    pkg.qsa_topk_blocks(pkg.SEL_B, q_ctx, L, pb.scores, pb.sel, pb.n_sel, pb.ws)
    for _ in range(reps):  # the one-call selection (list-mode score GEMM, list select)
        pkg.qsa_index_topk_prefill(pkg.SEL_B, q_ctx, L, q_idx, w, keys, pb.scores, pb.sel, pb.n_sel, pb.sel_ws)
    for _ in range(reps):
        pkg.qsa_sparse_prefill(pkg.SEL_B, pkg.ATTN_B, q_ctx, L, q, kv, pb.sel, pb.n_sel, 0, L, pb.o_tiles[0],
                               pb.lse_tiles[0])
    # the same attention over FP8 sparse-MLA rows (656 B per token)
    rows = torch.empty(1, L, 656, dtype=torch.uint8, device=dev)
    pkg.qsa_quantize_latent(lat, rows)
    kv8 = pkg.make_kv(rows)
    for _ in range(reps):
        pkg.qsa_sparse_prefill(pkg.SEL_B, pkg.ATTN_B, q_ctx, L, q, kv8, pb.sel, pb.n_sel, 0, L, pb.o_tiles[0],
                               pb.lse_tiles[0])
    torch.cuda.synchronize()
    # useful work: the 4-head indexer over every earlier token; QK (576
    # dims) and PV (512) of 64 heads over each query's selected tokens
    ctx = q_ctx.cpu().numpy().astype(np.int64)
    ns = pb.n_sel.cpu().numpy().astype(np.int64)
    att = float(ns.sum() * 64 * (576 + 512) * 2)
    # (scores_gemm_b<false, true>: the list-mode GEMM of qsa_index_topk_prefill, one dispatch per call)
    useful = {"scores_gemm_b<false, true>": float(ctx.sum() * 4 * 64 * 2), "attend_b_t": att, "attend_b_fp8": att}
    del pb, lat, keys, kv, rows, kv8
    torch.cuda.empty_cache()
    return useful


def mla_decode(torch, pkg, qi, pipeline, fill_normal_bf16, reps):
    """The shared-latent decode step: batch 8 at context 131,072, one
    qsa_decode_layer_latent call (scan with chunk lists, then select and
    attend)."""
    import numpy as np
    dev = "cuda"
    L, B = 131072, 8
    seed = qi.config_seed(5)
    lat = torch.empty(B, L, 1, 576, dtype=torch.bfloat16, device=dev)
    keys = torch.empty(B, L, 64, dtype=torch.bfloat16, device=dev)
    q = torch.empty(B, 64, 576, dtype=torch.bfloat16, device=dev)
    q_idx = torch.empty(B, 4, 64, dtype=torch.bfloat16, device=dev)
    for s in range(B):
        for t, kind in ((lat, "latent"), (keys, "raw_key"), (q, "q"), (q_idx, "q_idx")):
            fill_normal_bf16(t[s], seed, qi.stream_id(0, s, kind))
    w = torch.tensor(np.stack([qi.uniform_f32(seed, qi.stream_id(0, s, "w_idx"), 4) for s in range(B)]), device=dev)
    kv = pkg.make_kv(lat, lat)
    q_ctx = torch.full((B,), L, dtype=torch.int32, device=dev)
    q_seq = torch.arange(B, dtype=torch.int32, device=dev)
    bufs = pipeline.decode_buffers(pkg.SEL_B, pkg.ATTN_B, B, L)
    for _ in range(reps):
        pipeline.decode_layer(pkg.SEL_B, pkg.ATTN_B, q_ctx, L, q_idx, keys, q, kv, bufs, q_seq=q_seq, w_idx=w,
                              fused=True)
    torch.cuda.synchronize()


if __name__ == "__main__":
    sys.exit(main())
