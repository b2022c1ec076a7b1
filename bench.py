"""Benchmark of the tree-verification pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c5]

One step = the whole pass over one batch of synthetic inputs already resident
in HBM: tree_mask_build -> tree_attn_verify -> tree_accept_commit (the
acceptance walk and the compaction of the accepted path in one launch; with
--separate-commit, tree_accept_greedy -> kv_compact_path as two launches),
each through the C ABI.  The default (headline) workload is c5, the largest
configuration that one GPU holds: eight concurrent requests in the Qwen3-8B
head layout (32 query / 8 KV heads, head_dim 128) with ragged prefixes of
2048-8192 tokens and trees of 32-128 nodes in one varlen launch.  The same
run then measures the two other Qwen3-8B-shaped layers, c3 (prefix 4096,
128-node best-first tree) and c4 (prefix 8192, 256-node width-first tree), the
same way and reports them under "per_config"; --secondary none skips them and
--workload picks another headline.  --dtype f32 runs the same workloads with
fp32 inputs (the vector kernel; roofline against the fp32 vector peak when the
call is compute-bound there).

Timing:
  * cold cache: inputs rotate over R copies with R x footprint >= 512 MiB, so
    the 256 MiB Infinity Cache cannot hold them between uses;
  * a spin kernel queued ahead of the timed region keeps the GPU busy while
    the host enqueues every timed step, so the steps (and the HIP events
    around each tree_attn_verify call, on the launching stream) measure GPU
    time rather than Python launch gaps;
  * value = verified tree tokens (tree nodes) per second over the K steps.

The printed JSON line carries the roofline of tree_attn_verify (algorithmic
bytes and flops per call over its measured average duration, against the
MI355X peaks) and the CPU oracle's rate on a bounded sample ('cpu_baseline').

Measured HBM traffic (roofline.traffic) comes from two rocprofv3 counter
passes over this same script (FETCH_SIZE, then WRITE_SIZE), each run with
--calib-copy-mib so that a device-to-device copy of known size is in the
same trace:

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/fetch -o p -- \
        python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline --calib-copy-mib 256
    (the same with WRITE_SIZE into OUT/write)
    python3 bench.py --workload c3 --ingest-traffic OUT/fetch OUT/write

The last step writes profiles/tree_attn_verify_<workload>_traffic.md with
the per-call bytes and the copy's scale factor; later runs report it only
while the attention source it was taken on is unchanged (SHA-256).
"""
from __future__ import annotations

import argparse
import ctypes
import csv
import glob
import hashlib
import re
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from tree_attention_verification_bitmask_amd import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
FP32_VECTOR_PEAK_TFLOPS = 157.3
METRIC = "verified tree-tokens/sec per GPU; % of HBM-BW / bf16-MFMA roofline"
COLD_BYTES = 512 << 20
ATTN_SOURCES = ("tree_attention_verification_bitmask_amd/csrc/attn_mfma.hip",)
# the main kernel of a call (one of them runs per call), then the others a
# call may run: the merge and the batch planners
ATTN_MAIN_KERNELS = ("attn_fwd_kernel", "attn_fwd_bal_kernel")
ATTN_KERNELS = ATTN_MAIN_KERNELS + ("attn_combine_kernel", "attn_plan_kernel", "attn_bal_plan_kernel")


def attn_source_hash() -> str:
    """SHA-256 of the attention source's code: line comments and blank space
    are dropped first, so an edit to comments alone keeps the stored counter
    figures valid while any change to the code voids them."""
    h = hashlib.sha256()
    for rel in ATTN_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].split()
                if code:
                    h.update(" ".join(code).encode() + b"\n")
    return h.hexdigest()


def traffic_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"tree_attn_verify_{workload}_traffic.md")


def _counter_rows(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no rocprofv3 counter_collection.csv under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def ingest_traffic(workload: str, fetch_dir: str, write_dir: str, calib_mib: int) -> str:
    """Per-call FETCH_SIZE / WRITE_SIZE of tree_attn_verify (its two kernels,
    summed per call) from two rocprofv3 --pmc runs, scaled by what the same
    counters read for the calibration copy of calib_mib MiB."""
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _counter_rows(d) if r["Counter_Name"] == counter]
        # (names matched as whole identifiers: attn_fwd_kernel is not a part of
        # attn_fwd_bal_kernel, nor attn_plan_kernel of attn_bal_plan_kernel)
        per_kernel = {k: [float(r["Counter_Value"]) for r in rows if re.search(r"\b" + k + r"\b", r["Kernel_Name"])]
                      for k in ATTN_KERNELS}
        calls = sum(len(per_kernel[k]) for k in ATTN_MAIN_KERNELS)
        if calls == 0:
            raise RuntimeError(f"{counter}: no {' / '.join(ATTN_MAIN_KERNELS)} dispatches in {d}")
        # average KiB per call: the main kernel every call, the combine when it ran
        kib = sum(sum(v) for v in per_kernel.values()) / calls
        # the calibration copy is by far the largest copy in the trace; the
        # counter need not read its true size (that is what the scale is for)
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        target = calib_mib * 1024.0
        best = max(copies) if copies else None
        if best is None or not (0.25 * target <= best <= 4.0 * target):
            raise RuntimeError(f"{counter}: no calibration copy of ~{calib_mib} MiB in {d}")
        scale = target / best
        out[counter] = (kib, best, scale, calls)
    fk, fcopy, fscale, calls = out["FETCH_SIZE"]
    wk, wcopy, wscale, _ = out["WRITE_SIZE"]
    fetch_b = fk * 1024.0 * fscale
    write_b = wk * 1024.0 * wscale
    text = (
        f"# HBM traffic of tree_attn_verify: {workload}\n\n"
        "Counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch), from two separate\n"
        "`rocprofv3 --pmc <counter>` runs of bench.py with `--calib-copy-mib "
        f"{calib_mib}`; run from /tmp on the GPU box:\n\n"
        "```\n"
        "rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/fetch -o p -- python3 $REPO/bench.py "
        f"--workload {workload} --secondary none --steps 5 --warmup 2 --no-cpu-baseline --calib-copy-mib {calib_mib}\n"
        "rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/write -o p -- python3 $REPO/bench.py "
        f"--workload {workload} --secondary none --steps 5 --warmup 2 --no-cpu-baseline --calib-copy-mib {calib_mib}\n"
        f"python3 $REPO/bench.py --workload {workload} --ingest-traffic OUT/fetch OUT/write\n"
        "```\n\n"
        "A call of tree_attn_verify is attn_fwd_kernel plus attn_combine_kernel, or for\n"
        "batches attn_bal_plan_kernel, attn_fwd_bal_kernel and attn_combine_kernel (the\n"
        "longest-first order: attn_plan_kernel first); the figures are their per-call\n"
        "sums averaged over the calls in the trace.  Each\n"
        f"counter is scaled by {calib_mib} MiB over what it read for the calibration copy.\n\n"
        "| counter | KiB per call (raw) | calibration copy (KiB raw) | scale | bytes per call |\n"
        "|---|---|---|---|---|\n"
        f"| FETCH_SIZE | {fk:.1f} | {fcopy:.1f} | {fscale:.4f} | {fetch_b:.0f} |\n"
        f"| WRITE_SIZE | {wk:.1f} | {wcopy:.1f} | {wscale:.4f} | {write_b:.0f} |\n\n"
        f"calls: {calls}\n\n"
        f"traffic_bytes_per_call: {fetch_b + write_b:.0f}\n"
        f"fetch_bytes_per_call: {fetch_b:.0f}\n"
        f"write_bytes_per_call: {write_b:.0f}\n"
        f"attn_source_sha256: {attn_source_hash()}\n"
    )
    path = traffic_path(workload)
    with open(path, "w") as f:
        f.write(text)
    return path


def load_traffic(workload: str):
    """(bytes per call, detail) from the committed traffic summary, or
    (None, reason) when there is none or the attention source changed since."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None, "no counter summary"
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(("#", "|", "`")):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("attn_source_sha256") != attn_source_hash():
        return None, "kernel changed since the counters were taken"
    return float(vals["traffic_bytes_per_call"]), {
        "fetch_bytes": float(vals["fetch_bytes_per_call"]), "write_bytes": float(vals["write_bytes_per_call"]),
        "source": os.path.relpath(path, ROOT)}


def algorithmic_work(wl):
    """Bytes and flops the method itself must move / compute per call of
    tree_attn_verify: K+V of every key row read once, Q read and O written
    once; 2 flops per multiply-add for Q.K and P.V over each node's own key
    set (prefix plus ancestors-or-self)."""
    es = 2 if wl.dtype == "bf16" else 4
    byts = 0
    flops = 0
    for b in range(wl.batch):
        n = int(wl.cu_nodes[b + 1] - wl.cu_nodes[b])
        P = int(wl.prefix_len[b])
        levels = int(W._depths(wl.parent[wl.nodes_of(b)]).sum()) if n else 0
        byts += (P + n) * wl.hkv * wl.d * 2 * es + 2 * n * wl.hq * wl.d * es
        flops += 4 * wl.hq * wl.d * (n * P + levels)
    return byts, flops


def blas_threads() -> int:
    """Threads numpy's BLAS may use (the oracle's matrix routines)."""
    try:
        import threadpoolctl
        blas = [p for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
        return int(max([p["num_threads"] for p in blas] or [1]))
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(wl, budget_s: float = 15.0):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    mask, acceptance and compaction for the whole batch, and attention for as
    many whole nodes (all heads) as fit in about budget_s seconds."""
    from oracle import tree_verify_oracle as O
    threads = blas_threads()
    t0 = time.perf_counter()
    O.mask_build(wl.parent, wl.cu_nodes, wl.prefix_len, wl.max_nodes, wl.max_depth)
    alen, aidx, _ = O.accept_greedy(wl.parent, wl.draft, wl.target, wl.root_target, wl.cu_nodes, wl.max_depth)
    O.kv_compact(wl.k, wl.v, wl.kv_start, wl.prefix_len, alen, aidx)
    t_rest = time.perf_counter() - t0
    done = 0
    t1 = time.perf_counter()
    while done < wl.total_nodes and time.perf_counter() - t1 < budget_s:
        O.tree_attention(wl.q, wl.k, wl.v, wl.parent, wl.cu_nodes, wl.kv_start, wl.prefix_len, wl.scale,
                         rows=[(done, h) for h in range(wl.hq)])
        done += 1
    t_attn = time.perf_counter() - t1
    per_node = t_attn / done + t_rest / wl.total_nodes
    return {"value": 1.0 / per_node, "unit": "tree-tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"{wl.name} seed {wl.seed}: float64 oracle attention for nodes 0..{done - 1} of "
                       f"{wl.total_nodes} (all {wl.hq} heads, {t_attn:.1f} s) plus mask, acceptance and "
                       f"compaction of the whole batch ({t_rest:.2f} s, charged per node)"),
            "os_cpu_count": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c5", choices=sorted(W.CONFIGS),
                    help="headline workload (default c5, the largest single-GPU configuration)")
    ap.add_argument("--secondary", default="",
                    help="comma-separated workloads measured after the headline and reported under "
                         "per_config (default c3,c4; 'none' for none)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--dtype", default="config", choices=("config", "f32"),
                    help="element type of the attention inputs: the workload's own (config), or fp32 "
                         "(the vector kernel, roofline against the fp32 vector peak)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--waves", type=int, default=0,
                    help="tuning: plan override for tree_attn_verify, waves per workgroup (4 or 8; 0 = library)")
    ap.add_argument("--paged", action="store_true",
                    help="attention variant: K/V through a token table over a permuted pool of cache rows")
    ap.add_argument("--rope-base", type=float, default=0.0,
                    help="attention variant: RoPE inside the call at this base (0 = off)")
    ap.add_argument("--splits", type=int, default=0,
                    help="tuning: plan override for tree_attn_verify, key-axis slices (0 = library)")
    ap.add_argument("--order", choices=("auto", "static", "planned", "balanced"), default="auto",
                    help="tuning: plan override for tree_attn_verify, batch task order (auto = library)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB first (counter calibration)")
    ap.add_argument("--ingest-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic summary from two rocprofv3 --pmc output folders and exit")
    ap.add_argument("--separate-commit", action="store_true",
                    help="run the walk and the compaction as two launches")
    ap.add_argument("--warm", action="store_true",
                    help="reuse one input set every step (warm Infinity Cache); the default rotates "
                         "over enough copies to keep it cold, and roofline claims use the cold runs")
    ap.add_argument("--select", action="store_true",
                    help="time tree_select_topb (draft tree from a frontier ledger) instead of the pass")
    ap.add_argument("--select-batch", type=int, default=32)
    ap.add_argument("--select-budget", type=int, default=64)
    ap.add_argument("--select-depth", type=int, default=16)
    ap.add_argument("--select-k", type=int, default=4)
    ap.add_argument("--argmax", action="store_true",
                    help="time tree_target_argmax (the target's choice per node) instead of the pass")
    ap.add_argument("--argmax-rows", type=int, default=129)
    ap.add_argument("--argmax-vocab", type=int, default=151936)
    ap.add_argument("--argmax-dtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--sample", action="store_true",
                    help="time tree_target_sample (the target's sampled choice per node, T > 0) on the "
                         "--argmax-rows x --argmax-vocab logits instead of the pass")
    ap.add_argument("--sample-temperature", type=float, default=1.0)
    ap.add_argument("--stochastic", action="store_true",
                    help="time tree_accept_stochastic instead (c3's tree, the Qwen3 vocabulary, fp32 logits)")
    ap.add_argument("--rope", action="store_true",
                    help="time tree_rope_apply and kv_rollback_token_table on the workload instead of the pass")
    ap.add_argument("--gdn", action="store_true",
                    help="time one Gated-DeltaNet layer's tree verification (conv, verify, commit) on the "
                         "workload's trees instead of the pass")
    args = ap.parse_args(argv)
    if args.ingest_traffic:
        print(ingest_traffic(args.workload, args.ingest_traffic[0], args.ingest_traffic[1],
                             args.calib_copy_mib or 256))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this pass is built and timed on a single MI355X); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        return 2

    import torch
    from tree_attention_verification_bitmask_amd import binding as BND

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    L = BND.lib()  # raises if the HIP library is missing
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    if args.select:
        return bench_select(args, torch, BND, L, dev)
    if args.argmax:
        return bench_argmax(args, torch, BND, L, dev)
    if args.sample:
        return bench_sample(args, torch, BND, L, dev)
    if args.stochastic:
        return bench_stochastic(args, torch, BND, L, dev)
    if args.rope:
        return bench_rope(args, torch, BND, L, dev)
    if args.gdn:
        return bench_gdn(args, torch, BND, L, dev)

    if args.calib_copy_mib > 0:
        n_el = args.calib_copy_mib << 18  # float32 elements
        src_c = torch.ones(n_el, dtype=torch.float32, device=dev)
        dst_c = torch.empty_like(src_c)
        torch.cuda.synchronize()
        dst_c.copy_(src_c)
        torch.cuda.synchronize()
        del src_c, dst_c

    names = [args.workload]
    if args.secondary != "none":
        names += [n for n in (args.secondary.split(",") if args.secondary else ("c3", "c4")) if n != args.workload]
    lines = {}
    for name in names:
        seed = args.seed if name == args.workload else 0
        wl = W.make_workload(name, seed=seed, force_path=True, **dtype_override(args))
        lines[name] = time_pass(args, torch, BND, L, dev, wl, args.steps, args.warmup)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    line = lines.pop(args.workload)
    # Secondary denominator: the HBM rate a plain device-to-device copy reaches
    # on this GPU (read + write bytes over time), measured after the timed
    # regions.  (Skipped in counter runs: the traffic calibration takes the
    # largest copy in the trace as its reference.)
    # And the matrix rate a plain bf16 GEMM reaches on it (the library's,
    # under the same clock and power limits as the attention kernel).
    copy_gbs = hbm_copy_probe(torch, dev) if args.calib_copy_mib == 0 else None
    gemm_tflops = mfma_gemm_probe(torch, dev) if args.calib_copy_mib == 0 else None
    for ln in [line, *lines.values()]:
        roof = ln["roofline"]
        roof["hbm_copy_probe_gbs"] = copy_gbs
        roof["frac_of_copy_probe"] = roof["achieved_gbs"] / copy_gbs if copy_gbs else None
        roof["gemm_probe_tflops"] = gemm_tflops
        roof["frac_of_gemm_probe"] = roof["achieved_tflops"] / gemm_tflops if gemm_tflops else None
    if lines:
        line["per_config"] = {
            name: {"workload": ln["config"]["workload"], "value": ln["value"], "unit": ln["unit"],
                   "ms_per_step": ln["ms_per_step"], "steps": ln["steps"], "config": ln["config"],
                   "roofline": ln["roofline"]}
            for name, ln in lines.items()}
    if not args.no_cpu_baseline:
        wl = W.make_workload(args.workload, seed=args.seed, force_path=True, **dtype_override(args))
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    print(json.dumps(line), flush=True)
    return 0


def dtype_override(args) -> dict:
    return {} if args.dtype == "config" else {"dtype": args.dtype}


def time_pass(args, torch, BND, L, dev, wl, steps: int, warmup: int) -> dict:
    """Times `steps` steps of the pass on workload wl (after `warmup` untimed
    ones) and returns the JSON line's fields for it (without cpu_baseline)."""
    fdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    code = BND.TV_BF16 if wl.dtype == "bf16" else BND.TV_F32
    es = 2 if wl.dtype == "bf16" else 4
    T, B = wl.total_nodes, wl.batch

    def i32(x):
        return torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(dev)

    parent, cu, P, ks = i32(wl.parent), i32(wl.cu_nodes), i32(wl.prefix_len), i32(wl.kv_start)
    draft, target, root = i32(wl.draft), i32(wl.target), i32(wl.root_target)
    q0 = torch.from_numpy(wl.q).to(dev).to(fdt).contiguous()
    k0 = torch.from_numpy(wl.k).to(dev).to(fdt).contiguous()
    v0 = torch.from_numpy(wl.v).to(dev).to(fdt).contiguous()
    footprint = (q0.numel() + k0.numel() + v0.numel() + q0.numel()) * es
    R = 1 if args.warm else max(1, math.ceil(COLD_BYTES / footprint))
    sets = [(q0.clone(), k0.clone(), v0.clone()) for _ in range(R)]
    del q0, k0, v0
    words = (wl.max_nodes + 63) // 64
    anc = torch.empty((T, words), dtype=torch.int64, device=dev)
    level = torch.empty(T, dtype=torch.int32, device=dev)
    pos = torch.empty(T, dtype=torch.int32, device=dev)
    outs = [torch.empty((T, wl.hq, wl.d), dtype=fdt, device=dev) for _ in range(R)]
    alen = torch.empty(B, dtype=torch.int32, device=dev)
    aidx = torch.empty((B, wl.max_depth), dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    newlen = torch.empty(B, dtype=torch.int32, device=dev)
    err = torch.zeros(4, dtype=torch.int32, device=dev)
    order = {"auto": BND.TV_ORDER_AUTO, "static": BND.TV_ORDER_STATIC, "planned": BND.TV_ORDER_PLANNED,
             "balanced": BND.TV_ORDER_BALANCED}[args.order]
    ov = BND._override(args.splits, order, args.waves)
    # variants of the attention call: K/V through a token table over a
    # permuted pool (1.5x the rows), and RoPE inside the call
    pools, tables = [], []
    if args.paged:
        rng = np.random.default_rng(1234)
        rows = sets[0][1].shape[0]
        pool = rows * 3 // 2
        lens = (wl.prefix_len.astype(np.int64) + np.diff(wl.cu_nodes)).astype(np.int64)
        stride = int(lens.max())
        for (q, k, v) in sets:
            slot_of_row = rng.permutation(pool)[:rows]
            idx = torch.from_numpy(slot_of_row).to(dev)
            kp = torch.zeros((pool,) + tuple(k.shape[1:]), dtype=k.dtype, device=dev)
            vp = torch.zeros_like(kp)
            kp[idx] = k
            vp[idx] = v
            tab = np.zeros((B, stride), np.int32)
            for b in range(B):
                k0s = int(wl.kv_start[b])
                tab[b, :lens[b]] = slot_of_row[k0s:k0s + lens[b]]
            pools.append((kp, vp))
            tables.append(i32(tab))
    inputs = [BND._inputs(None, 0.0, None)] * R
    if args.paged or args.rope_base > 0:
        inputs = [BND.AttnInputs(int(pos.data_ptr()) if args.rope_base > 0 else None,
                                 int(tables[r].data_ptr()) if args.paged else None,
                                 int(tables[r].shape[1]) if args.paged else 0, float(args.rope_base))
                  for r in range(R)]
    ws_bytes = BND.tree_attn_verify_workspace_size(B, T, wl.max_nodes, wl.max_prefix, wl.hq, wl.hkv, wl.d, code,
                                                   args.splits, order, args.waves, inputs[0])
    plan = BND.tree_attn_verify_plan(B, T, wl.max_nodes, wl.max_prefix, wl.hq, wl.hkv, wl.d, code,
                                     args.splits, order, args.waves)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sp = C_void(stream.cuda_stream)

    # raw C calls with pre-marshalled arguments (the binding's checks are
    # done once here, by the shapes above)
    P_ = lambda t: C_void(t.data_ptr())  # noqa: E731
    mask_args = (P_(parent), P_(cu), P_(P), B, T, wl.max_nodes, wl.max_depth, P_(anc), P_(level), P_(pos),
                 C_void(err.data_ptr()), sp)
    attn_args = []
    for r, ((q, k, v), o) in enumerate(zip(sets, outs)):
        ka, va = pools[r] if args.paged else (k, v)
        attn_args.append((P_(q), P_(ka), P_(va), P_(cu), P_(ks), P_(P), P_(anc), B, T, wl.max_nodes, wl.max_prefix,
                          ka.shape[0], wl.hq, wl.hkv, wl.d, float(wl.scale), code, P_(o), P_(ws), ws.numel(),
                          C_void(err.data_ptr() + 4), sp))
    acc_args = (P_(parent), P_(draft), P_(target), P_(root), P_(cu), B, T, wl.max_depth, P_(alen), P_(aidx),
                P_(nxt), C_void(err.data_ptr() + 8), sp)
    cmp_args = [(P_(k), P_(v), P_(cu), P_(ks), P_(P), P_(alen), P_(aidx), B, T, wl.max_depth, k.shape[0], wl.hkv,
                 wl.d, code, P_(newlen), C_void(err.data_ptr() + 12), sp) for (q, k, v) in sets]
    com_args = [(P_(parent), P_(draft), P_(target), P_(root), P_(cu), P_(ks), P_(P), B, T, wl.max_depth,
                 k.shape[0], wl.hkv, wl.d, code, P_(k), P_(v), P_(alen), P_(aidx), P_(nxt), P_(newlen),
                 C_void(err.data_ptr() + 8), sp) for (q, k, v) in sets]

    def step(i, ev=None):
        r = i % R
        st = L.tree_mask_build(*mask_args)
        if ev is not None:
            ev[0].record(stream)
        if ov is None and inputs[r] is None:
            st |= L.tree_attn_verify(*attn_args[r])
        else:
            a = attn_args[r]   # (..., scale, dtype, out, workspace, bytes, err, stream)
            st |= L.tree_attn_verify_ex(*a[:17], ctypes.byref(inputs[r]) if inputs[r] is not None else None,
                                        *a[17:-1], ctypes.byref(ov) if ov is not None else None, a[-1])
        if ev is not None:
            ev[1].record(stream)
        if args.separate_commit:
            st |= L.tree_accept_greedy(*acc_args)
            st |= L.kv_compact_path(*cmp_args[r])
        else:
            st |= L.tree_accept_commit(*com_args[r])
        return st

    for i in range(warmup):
        if step(i):
            raise RuntimeError("a call was rejected during warmup")
    torch.cuda.synchronize()
    if int(err.abs().sum().item()) != 0:
        raise RuntimeError(f"device error words {err.tolist()}")

    K = steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # calibrate the spin kernel, then queue enough spin to cover the host's
    # enqueue time of the timed steps (measured during warmup, with margin)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    torch.cuda._sleep(1 << 22)
    c1.record(stream)
    torch.cuda.synchronize()
    cycles_per_ms = (1 << 22) / max(c0.elapsed_time(c1), 1e-3)
    t0 = time.perf_counter()
    for i in range(8):
        step(i)
    torch.cuda.synchronize()
    host_ms_per_step = (time.perf_counter() - t0) * 1e3 / 8
    spin_ms = min(5000.0, max(20.0, 3.0 * K * host_ms_per_step))
    torch.cuda.synchronize()
    torch.cuda._sleep(int(cycles_per_ms * spin_ms))
    start.record(stream)
    t_host0 = time.perf_counter()
    status = 0
    for i in range(K):
        status |= step(warmup + i, evs[i])
    end.record(stream)
    t_host_enq = time.perf_counter() - t_host0
    torch.cuda.synchronize()
    if status:
        raise RuntimeError("a call was rejected in the timed region")
    if int(err.abs().sum().item()) != 0:
        raise RuntimeError(f"device error words {err.tolist()}")
    total_ms = start.elapsed_time(end)
    attn_ms = np.array([a.elapsed_time(b) for a, b in evs])
    ms_step = total_ms / K
    attn_us = float(attn_ms.mean() * 1e3)

    byts, flops = algorithmic_work(wl)
    ai = flops / byts
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    # fp32 runs on the vector units: 256 CUs x 4 SIMDs x 16 lanes x 2 flops
    # per fused multiply-add x 2.4 GHz = 157.3 TFLOP/s
    valu_ridge = FP32_VECTOR_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if wl.dtype == "bf16" and ai >= ridge:
        roof = {"bound": "mfma", "achieved": flops / (attn_us * 1e-6) / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    elif wl.dtype == "f32" and ai >= valu_ridge:
        roof = {"bound": "alu", "achieved": flops / (attn_us * 1e-6) / 1e12, "peak": FP32_VECTOR_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": byts / (attn_us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # (the committed counter summaries are of the bf16 kernel)
    traffic, tdetail = load_traffic(wl.name) if wl.dtype == "bf16" else (None, "no counter summary for fp32")
    roof["traffic"] = traffic
    roof["traffic_detail"] = tdetail
    roof.update({"kernel": "tree_attn_verify", "avg_us": attn_us,
                 "p10_us": float(np.percentile(attn_ms, 10) * 1e3),
                 "p50_us": float(np.percentile(attn_ms, 50) * 1e3),
                 "p90_us": float(np.percentile(attn_ms, 90) * 1e3),
                 "alg_bytes": byts, "alg_flops": flops, "arith_intensity": ai,
                 "achieved_gbs": byts / (attn_us * 1e-6) / 1e9,
                 "achieved_tflops": flops / (attn_us * 1e-6) / 1e12})
    # Secondary denominator: the HBM rate a plain device-to-device copy reaches
    # on this GPU (read + write bytes over time), measured after the timed region.
    # (Skipped in counter runs: the traffic calibration takes the largest copy
    # in the trace as its reference.)

    line = {
        "metric": METRIC,
        "value": T / (ms_step * 1e-3),
        "unit": "tree-tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {W.CONFIGS[wl.name]['desc']}", "seed": wl.seed, "batch": B,
                   "tree_nodes": T, "max_prefix": wl.max_prefix, "hq": wl.hq, "hkv": wl.hkv,
                   "head_dim": wl.d, "max_depth": wl.max_depth, "cold_cache_sets": R,
                   "cache": "warm" if args.warm else "cold",
                   "commit": "two launches" if args.separate_commit else "one launch",
                   "workspace_bytes": ws_bytes, "plan": plan, "host_enqueue_ms": t_host_enq * 1e3,
                   "spin_ahead_ms": spin_ms,
                   "attention_inputs": {"token_table": bool(args.paged), "rope_base": float(args.rope_base)}},
        "roofline": roof,
    }
    return line


def bench_select(args, torch, BND, L, dev):
    """One step = one tree_select_topb call over a batch of frontier-shaped
    ledgers ([batch, depth, budget * k] slots: W = B lanes of k children per
    depth, as [DT] section 3.3 sets them), rotated over enough copies to keep
    the Infinity Cache cold.  value = draft trees selected per second."""
    Bt, Bn, D, k = args.select_batch, args.select_budget, args.select_depth, args.select_k
    L_ = Bn * k
    rng = np.random.default_rng(args.seed)
    score, parent, token = W.frontier_shaped_ledger(rng, Bt, D, Bn, k)
    set_bytes = score.nbytes + parent.nbytes + token.nbytes
    R = max(1, math.ceil(COLD_BYTES / set_bytes))
    sc0 = torch.from_numpy(score).to(dev)
    pa0 = torch.from_numpy(parent).to(dev)
    tk0 = torch.from_numpy(token).to(dev)
    sets = [(sc0.clone(), pa0.clone(), tk0.clone()) for _ in range(R)]
    tp = torch.empty((Bt, Bn), dtype=torch.int32, device=dev)
    tt = torch.empty((Bt, Bn), dtype=torch.int32, device=dev)
    nr = torch.empty(Bt, dtype=torch.int32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    sp = C_void(stream.cuda_stream)
    P_ = lambda t: C_void(t.data_ptr())  # noqa: E731
    call_args = [(P_(a), P_(b), P_(c), Bt, D, L_, Bn, 0.0, P_(tp), P_(tt), P_(nr), P_(err), sp)
                 for (a, b, c) in sets]
    for i in range(args.warmup):
        if L.tree_select_topb(*call_args[i % R]):
            raise RuntimeError("tree_select_topb rejected its arguments")
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        raise RuntimeError(f"device error word {int(err.item()):#x}")
    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1 << 24)
    start.record(stream)
    for i in range(K):
        evs[i][0].record(stream)
        L.tree_select_topb(*call_args[(args.warmup + i) % R])
        evs[i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    call_ms = np.array([a.elapsed_time(b) for a, b in evs])
    ms_step = start.elapsed_time(end) / K
    us = float(call_ms.mean() * 1e3)
    byts = Bt * D * L_ * 12 + Bt * Bn * 8 + Bt * 4   # ledger read once, tree and counts written
    roof = {"bound": "hbm", "achieved": byts / (us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "traffic": None, "traffic_detail": "not measured for this kernel",
            "kernel": "tree_select_topb", "avg_us": us,
            "p10_us": float(np.percentile(call_ms, 10) * 1e3), "p90_us": float(np.percentile(call_ms, 90) * 1e3),
            "alg_bytes": byts}
    roof["frac"] = roof["achieved"] / roof["peak"]
    line = {
        "metric": "draft trees selected per second (tree_select_topb)",
        "value": Bt / (us * 1e-6),
        "unit": "trees/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64 keys, int32",
        "data": "synthetic",
        "config": {"workload": f"frontier ledgers: batch {Bt}, depth {D}, W = B = {Bn} lanes x k = {k}",
                   "seed": args.seed, "ledger_slots_per_request": D * L_, "cold_cache_sets": R},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        from oracle import tree_select_oracle as S
        t0 = time.perf_counter()
        n = 0
        while n < Bt and time.perf_counter() - t0 < args.cpu_budget:
            S.select_one(score[n], parent[n], token[n], Bn, 0.0)
            n += 1
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": n / dt, "unit": "trees/s", "cores": 1, "kind": "oracle",
                                "sample": f"select_one on requests 0..{n - 1} of the same ledgers ({dt:.2f} s)"}
    print(json.dumps(line), flush=True)
    return 0


def bench_argmax(args, torch, BND, L, dev):
    """One step = one tree_target_argmax call over [rows, vocab] logits (the
    default 129 x 151936 fp32 is c3's 128 tree nodes plus the root row at the
    Qwen3 vocabulary, 78 MB), rotated over enough copies to keep the
    Infinity Cache cold.  value = node choices per second."""
    rows, V = args.argmax_rows, args.argmax_vocab
    bf = args.argmax_dtype == "bf16"
    es = 2 if bf else 4
    rng = np.random.default_rng(args.seed)
    x = torch.from_numpy(rng.normal(0, 3, (rows, V)).astype(np.float32)).to(dev)
    if bf:
        x = x.to(torch.bfloat16)
    set_bytes = rows * V * es
    R = max(2, math.ceil(COLD_BYTES / set_bytes))
    sets = [x.clone() for _ in range(R)]
    del x
    tok = torch.empty(rows, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    sp = C_void(stream.cuda_stream)
    code = BND.TV_BF16 if bf else BND.TV_F32
    call_args = [(C_void(t.data_ptr()), rows, V, code, C_void(tok.data_ptr()), sp) for t in sets]
    for i in range(args.warmup):
        if L.tree_target_argmax(*call_args[i % R]):
            raise RuntimeError("tree_target_argmax rejected its arguments")
    torch.cuda.synchronize()
    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1 << 24)
    start.record(stream)
    for i in range(K):
        evs[i][0].record(stream)
        L.tree_target_argmax(*call_args[(args.warmup + i) % R])
        evs[i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    call_ms = np.array([a.elapsed_time(b) for a, b in evs])
    us = float(call_ms.mean() * 1e3)
    byts = rows * V * es + rows * 4
    roof = {"bound": "hbm", "achieved": byts / (us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "traffic": None, "traffic_detail": "not measured for this kernel",
            "kernel": "tree_target_argmax", "avg_us": us,
            "p10_us": float(np.percentile(call_ms, 10) * 1e3), "p90_us": float(np.percentile(call_ms, 90) * 1e3),
            "alg_bytes": byts}
    roof["frac"] = roof["achieved"] / roof["peak"]
    line = {
        "metric": "node target choices per second (tree_target_argmax)",
        "value": rows / (us * 1e-6),
        "unit": "nodes/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": start.elapsed_time(end) / K,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": args.argmax_dtype,
        "data": "synthetic",
        "config": {"workload": f"logits {rows} x {V} {args.argmax_dtype}", "seed": args.seed,
                   "cold_cache_sets": R},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        from oracle import tree_verify_oracle as O
        xs = sets[0].float().cpu().numpy()
        t0 = time.perf_counter()
        n = 0
        while n < rows and time.perf_counter() - t0 < args.cpu_budget:
            O.target_argmax(xs[n:n + 16])
            n = min(rows, n + 16)
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": n / dt, "unit": "nodes/s", "cores": 1, "kind": "oracle",
                                "sample": f"target_argmax on rows 0..{n - 1} of the same logits ({dt:.2f} s)"}
    print(json.dumps(line), flush=True)
    return 0


def hbm_copy_probe(torch, dev, mib: int = 512, reps: int = 10) -> float:
    """GB/s of a device-to-device copy of `mib` MiB (bytes read + written),
    averaged over `reps` copies timed with HIP events."""
    n = mib << 18  # float32 elements
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return 2 * n * 4 / (ms * 1e-3) / 1e9


def mfma_gemm_probe(torch, dev, n: int = 8192, reps: int = 10) -> float:
    """TFLOP/s of an n x n x n bf16 matrix product (torch.matmul on contiguous
    2-D operands, fp32 accumulation in the library), averaged over `reps`
    products timed with HIP events: the matrix rate this GPU sustains."""
    a = torch.randn((n, n), dtype=torch.float32, device=dev).to(torch.bfloat16).contiguous()
    b = torch.randn((n, n), dtype=torch.float32, device=dev).to(torch.bfloat16).contiguous()
    for _ in range(3):
        c = torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    return 2.0 * n ** 3 / (ms * 1e-3) / 1e12


def bench_sample(args, torch, BND, L, dev):
    """One step = one tree_target_sample call (chunk pass + pick pass) over
    [rows, vocab] logits with one float64 uniform per row, rotated over enough
    copies to keep the Infinity Cache cold.  value = node choices per second.
    The roofline counts the logits read once plus the uniforms and tokens."""
    rows, V = args.argmax_rows, args.argmax_vocab
    bf = args.argmax_dtype == "bf16"
    es = 2 if bf else 4
    rng = np.random.default_rng(args.seed)
    x = torch.from_numpy(rng.normal(0, 3, (rows, V)).astype(np.float32)).to(dev)
    if bf:
        x = x.to(torch.bfloat16)
    set_bytes = rows * V * es
    R = max(2, math.ceil(COLD_BYTES / set_bytes))
    sets = [x.clone() for _ in range(R)]
    del x
    u = torch.from_numpy(rng.random(rows)).to(dev)
    tok = torch.empty(rows, dtype=torch.int32, device=dev)
    ws_bytes = int(L.tree_target_sample_workspace_size(rows, V))
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sp = C_void(stream.cuda_stream)
    code = BND.TV_BF16 if bf else BND.TV_F32
    temp = float(np.float32(args.sample_temperature))
    call_args = [(C_void(t.data_ptr()), rows, V, code, temp, C_void(u.data_ptr()), C_void(tok.data_ptr()),
                  C_void(ws.data_ptr()), ws_bytes, sp) for t in sets]
    for i in range(args.warmup):
        if L.tree_target_sample(*call_args[i % R]):
            raise RuntimeError("tree_target_sample rejected its arguments")
    torch.cuda.synchronize()
    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1 << 24)
    start.record(stream)
    for i in range(K):
        evs[i][0].record(stream)
        L.tree_target_sample(*call_args[(args.warmup + i) % R])
        evs[i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    call_ms = np.array([a.elapsed_time(b) for a, b in evs])
    us = float(call_ms.mean() * 1e3)
    byts = rows * V * es + rows * (8 + 4)
    roof = {"bound": "hbm", "achieved": byts / (us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "traffic": None, "traffic_detail": "not measured for this kernel",
            "kernel": "tree_target_sample", "avg_us": us,
            "p10_us": float(np.percentile(call_ms, 10) * 1e3), "p90_us": float(np.percentile(call_ms, 90) * 1e3),
            "alg_bytes": byts, "fp64_exp_per_s": rows * V / (us * 1e-6)}
    roof["frac"] = roof["achieved"] / roof["peak"]
    line = {
        "metric": "node sampled target choices per second (tree_target_sample)",
        "value": rows / (us * 1e-6),
        "unit": "nodes/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": start.elapsed_time(end) / K,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": args.argmax_dtype + "->f64",
        "data": "synthetic",
        "config": {"workload": f"logits {rows} x {V} {args.argmax_dtype}, T {temp}", "seed": args.seed,
                   "cold_cache_sets": R},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        from oracle import tree_verify_oracle as O
        xs = sets[0].float().cpu().numpy()
        uh = u.cpu().numpy()
        t0 = time.perf_counter()
        n = 0
        while n < rows and time.perf_counter() - t0 < args.cpu_budget:
            O.target_sample(xs[n:n + 16], temp, uh[n:n + 16])
            n = min(rows, n + 16)
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": n / dt, "unit": "nodes/s", "cores": 1, "kind": "oracle",
                                "sample": f"target_sample on rows 0..{n - 1} of the same logits ({dt:.2f} s)"}
    print(json.dumps(line), flush=True)
    return 0


def bench_stochastic(args, torch, BND, L, dev):
    """One step = one tree_accept_stochastic call on c3's tree (one request,
    128 nodes) over the Qwen3 vocabulary (151936): target logits fp32
    [1 + 128, V], draft probabilities fp32 [1 + 128, V] (the target's logits
    plus noise, so candidates are often but not always accepted), each child's
    token drawn from its parent's q, seeded uniforms; rotated copies keep the
    Infinity Cache cold.  value = verification steps (requests) per second.
    The roofline counts the logits read once (the statistics pass); the
    rejection passes re-read the logits and draft probabilities of every row
    whose test was rejected (each node's tests are decided whether or not
    the walk reaches it), and the draw re-reads one chunk; these depend on
    the data and come on top."""
    wl = W.make_workload("c3", seed=args.seed)
    V = args.argmax_vocab
    T = wl.total_nodes
    rng = np.random.default_rng(args.seed)
    rl = rng.normal(0, 3, (1, V)).astype(np.float32)
    nl = rng.normal(0, 3, (T, V)).astype(np.float32)

    def qd(x):
        z = x.astype(np.float64) + rng.normal(0, 1.0, x.shape)
        z = np.exp(z - z.max(axis=1, keepdims=True))
        return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    rq, nq = qd(rl), qd(nl)
    draft = np.empty(T, np.int32)
    for i in range(T):
        pa = int(wl.parent[i])
        q = (rq[0] if pa < 0 else nq[pa]).astype(np.float64)
        draft[i] = int(rng.choice(V, p=q / q.sum()))
    ua, uf = rng.random(T), rng.random(1)
    set_bytes = 2 * (1 + T) * V * 4
    R = max(2, math.ceil(COLD_BYTES / set_bytes))
    t32 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    sets = [(t32(rl), t32(nl), t32(rq), t32(nq)) for _ in range(R)]
    parent, dr, cu = t32(wl.parent.astype(np.int32)), t32(draft), t32(wl.cu_nodes.astype(np.int32))
    u_a, u_f = t32(ua), t32(uf)
    D = wl.max_depth
    alen = torch.empty(1, dtype=torch.int32, device=dev)
    aidx = torch.empty((1, D), dtype=torch.int32, device=dev)
    nxt = torch.empty(1, dtype=torch.int32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ws_bytes = int(L.tree_accept_stochastic_workspace_size(1, T, V))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sp = C_void(stream.cuda_stream)
    P_ = lambda t: C_void(t.data_ptr())
    temp = 1.0
    call_args = [(P_(parent), P_(dr), P_(cu), 1, T, D, P_(a), P_(b), BND.TV_F32, temp, P_(c), P_(d), V, P_(u_a),
                  P_(u_f), P_(alen), P_(aidx), P_(nxt), P_(ws), ws_bytes, P_(err), sp) for (a, b, c, d) in sets]
    for i in range(args.warmup):
        if L.tree_accept_stochastic(*call_args[i % R]):
            raise RuntimeError("tree_accept_stochastic rejected its arguments")
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        raise RuntimeError(f"device error {int(err.item()):#x}")
    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1 << 24)
    start.record(stream)
    for i in range(K):
        evs[i][0].record(stream)
        L.tree_accept_stochastic(*call_args[(args.warmup + i) % R])
        evs[i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    call_ms = np.array([a.elapsed_time(b) for a, b in evs])
    us = float(call_ms.mean() * 1e3)
    byts = (1 + T) * V * 4
    roof = {"bound": "hbm", "achieved": byts / (us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "traffic": None, "traffic_detail": "not measured for this kernel",
            "kernel": "tree_accept_stochastic", "avg_us": us,
            "p10_us": float(np.percentile(call_ms, 10) * 1e3), "p90_us": float(np.percentile(call_ms, 90) * 1e3),
            "alg_bytes": byts, "accept_len": int(alen.item())}
    roof["frac"] = roof["achieved"] / roof["peak"]
    line = {
        "metric": "stochastic verification steps per second (tree_accept_stochastic)",
        "value": 1.0 / (us * 1e-6),
        "unit": "requests/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": start.elapsed_time(end) / K,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32->f64",
        "data": "synthetic",
        "config": {"workload": f"c3 tree ({T} nodes), vocab {V}, fp32 logits and draft probabilities, T {temp}",
                   "seed": args.seed, "cold_cache_sets": R},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        from oracle import tree_verify_oracle as O
        t0 = time.perf_counter()
        n = 0
        while n < 3 and time.perf_counter() - t0 < args.cpu_budget:
            O.accept_stochastic(wl.parent, draft, wl.cu_nodes, rl.astype(np.float64), nl.astype(np.float64), temp,
                                rq.astype(np.float64), nq.astype(np.float64), ua, uf, D)
            n += 1
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": n / dt, "unit": "requests/s", "cores": 1, "kind": "oracle",
                                "sample": f"{n} oracle walks of the same request ({dt:.2f} s)"}
    print(json.dumps(line), flush=True)
    return 0


def bench_rope(args, torch, BND, L, dev):
    """tree_rope_apply (Q and the tree's K rows of the workload, rotated at the
    tree position ids) and kv_rollback_token_table (accepted path of the
    workload, one token per page), each timed with HIP events per call.  The
    rotation is applied repeatedly to the same buffers (timing only)."""
    wl = W.make_workload(args.workload, seed=args.seed, force_path=True)
    fdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    code = BND.TV_BF16 if wl.dtype == "bf16" else BND.TV_F32
    es = 2 if wl.dtype == "bf16" else 4
    T, B = wl.total_nodes, wl.batch
    i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(dev)  # noqa: E731
    parent, cu, P, ks = i32(wl.parent), i32(wl.cu_nodes), i32(wl.prefix_len), i32(wl.kv_start)
    q = torch.from_numpy(wl.q).to(dev).to(fdt).contiguous()
    k = torch.from_numpy(wl.k).to(dev).to(fdt).contiguous()
    anc, lev, pos, err = BND.tree_mask_build(parent, cu, P, wl.max_nodes, wl.max_depth)
    alen, aidx, _, _ = BND.tree_accept_greedy(parent, i32(wl.draft), i32(wl.target), i32(wl.root_target), cu,
                                              wl.max_depth)
    stride = int((wl.prefix_len + np.diff(wl.cu_nodes)).max())
    table = torch.zeros((B, stride), dtype=torch.int32, device=dev)
    slots = torch.arange(T, dtype=torch.int32, device=dev)
    nl = torch.empty(B, dtype=torch.int32, device=dev)
    fr = torch.empty(max(T, 1), dtype=torch.int32, device=dev)
    nf = torch.empty(B, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    sp = C_void(stream.cuda_stream)
    P_ = lambda t: C_void(t.data_ptr())  # noqa: E731
    rope_args = (P_(q), P_(k), P_(pos), P_(cu), P_(ks), P_(P), B, T, k.shape[0], wl.hq, wl.hkv, wl.d, 1.0e6, code,
                 P_(err), sp)
    rb_args = (P_(table), stride, P_(slots), P_(cu), P_(P), P_(alen), P_(aidx), B, T, wl.max_depth, P_(nl), P_(fr),
               P_(nf), P_(err), sp)
    out = {}
    for name, fn, a in (("tree_rope_apply", L.tree_rope_apply, rope_args),
                        ("kv_rollback_token_table", L.kv_rollback_token_table, rb_args)):
        for _ in range(args.warmup):
            if fn(*a):
                raise RuntimeError(f"{name} rejected its arguments")
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda._sleep(1 << 22)
        for e0, e1 in evs:
            e0.record(stream)
            fn(*a)
            e1.record(stream)
        torch.cuda.synchronize()
        ms = np.array([a_.elapsed_time(b_) for a_, b_ in evs])
        out[name] = float(ms.mean() * 1e3)
    if int(err.item()) != 0:
        raise RuntimeError(f"device error word {int(err.item()):#x}")
    rope_bytes = 2 * T * (wl.hq + wl.hkv) * wl.d * es + T * 4
    us = out["tree_rope_apply"]
    roof = {"bound": "hbm", "achieved": rope_bytes / (us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "traffic": None, "traffic_detail": "not measured for this kernel", "kernel": "tree_rope_apply",
            "avg_us": us, "alg_bytes": rope_bytes, "rollback_avg_us": out["kv_rollback_token_table"]}
    roof["frac"] = roof["achieved"] / roof["peak"]
    line = {
        "metric": "tree nodes rotated per second (tree_rope_apply)",
        "value": T / (us * 1e-6), "unit": "nodes/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": us * 1e-3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": f"{wl.name}: {W.CONFIGS[wl.name]['desc']}", "seed": wl.seed},
        "roofline": roof,
    }
    print(json.dumps(line), flush=True)
    return 0


def gdn_alg_bytes(T, B, hk, hv, d, C, K, D, n_acc):
    """Algorithmic HBM bytes of the three calls: every input read once, every
    output written once (bf16 activations, fp32 g/beta/state/outputs)."""
    conv = T * C * 2 + B * (K - 1) * C * 2 + C * K * 2 + T * C * 2 + T * 4
    verify = T * (2 * hk + hv) * d * 2 + 2 * T * hv * 4 + B * hv * d * d * 4 + T * hv * d * 4 + T * 4
    commit = 2 * B * hv * d * d * 4 + n_acc * (hk + hv) * d * 2 + 2 * n_acc * hv * 4 \
        + B * (K - 1) * C * 2 * 2 + n_acc * C * 2 + B * (1 + D) * 4
    return conv, verify, commit


def bench_gdn(args, torch, BND, L, dev):
    """One step = one Gated-DeltaNet layer verifying the workload's draft
    trees: tree_gdn_conv, tree_gdn_verify and tree_gdn_commit of the greedy
    accepted path, for a 16 q/k-head, 32 v-head, 128-channel layer with a
    width-4 convolution (8192 mixed channels).  Each call is timed with HIP
    events.  The commit advances the state in place on every step (timing
    only; its cost does not depend on the values)."""
    import ctypes
    from tree_attention_verification_bitmask_amd import workloads as Wm
    wl = W.make_workload(args.workload, seed=args.seed, force_path=True)
    lay = Wm.GDN_LAYER
    hk, hv, d, K = lay["hk"], lay["hv"], lay["dk"], lay["conv_k"]
    parents = [wl.parent[wl.cu_nodes[b]:wl.cu_nodes[b + 1]] for b in range(wl.batch)]
    gi = Wm.gdn_inputs(np.random.default_rng(args.seed), parents, hk=hk, hv=hv, dk=d, dv=d, conv_k=K)
    T, B, C = wl.total_nodes, wl.batch, gi.x.shape[1]
    D = wl.max_depth
    i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(dev)  # noqa: E731
    f32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)  # noqa: E731
    bf = lambda x: f32(x).to(torch.bfloat16).contiguous()  # noqa: E731
    parent, cu = i32(wl.parent), i32(wl.cu_nodes)
    x, cs, w = bf(gi.x), bf(gi.conv_state), bf(gi.conv_w)
    g, beta, state = f32(gi.g), f32(gi.beta), f32(gi.state)
    y = torch.empty_like(x)
    out = torch.empty((T, hv, d), dtype=torch.float32, device=dev)
    alen, aidx, _, err = BND.tree_accept_greedy(parent, i32(wl.draft), i32(wl.target), i32(wl.root_target), cu, D)
    torch.cuda.synchronize()
    n_acc = int(alen.sum().item())
    stream = torch.cuda.current_stream()
    sp = C_void(stream.cuda_stream)
    P_ = lambda t: C_void(t.data_ptr())  # noqa: E731
    qv, kv, vv = BND.gdn_split(y, hk, hv)
    rs = y.stride(0)
    scale = d ** -0.5
    conv_args = (P_(x), P_(cs), P_(w), P_(parent), P_(cu), B, T, C, K, P_(y), P_(err), sp)
    ver_args = (P_(qv), P_(kv), P_(vv), rs, P_(g), P_(beta), P_(state), P_(parent), P_(cu), B, T, D, hk, hv, d,
                ctypes.c_float(scale), 1, P_(out), P_(err), sp)
    com_args = (P_(state), P_(cs), P_(x), P_(kv), P_(vv), rs, P_(g), P_(beta), P_(cu), P_(alen), P_(aidx), B, T, D,
                hk, hv, d, C, K, 1, P_(err), sp)
    calls = (("tree_gdn_conv", L.tree_gdn_conv, conv_args), ("tree_gdn_verify", L.tree_gdn_verify, ver_args),
             ("tree_gdn_commit", L.tree_gdn_commit, com_args))
    for _ in range(args.warmup):
        for name, fn, a in calls:
            if fn(*a):
                raise RuntimeError(f"{name} rejected its arguments")
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        raise RuntimeError(f"device error word {int(err.item()):#x}")
    K_ = args.steps
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    evs = [[ev() for _ in range(4)] for _ in range(K_)]
    start, end = ev(), ev()
    torch.cuda._sleep(1 << 22)
    start.record(stream)
    for i in range(K_):
        evs[i][0].record(stream)
        for j, (_, fn, a) in enumerate(calls):
            fn(*a)
            evs[i][j + 1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    per = {name: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(K_)]) * 1e3)
           for j, (name, _, _) in enumerate(calls)}
    step_us = float(np.mean([evs[i][0].elapsed_time(evs[i][3]) for i in range(K_)]) * 1e3)
    conv_b, ver_b, com_b = gdn_alg_bytes(T, B, hk, hv, d, C, K, D, n_acc)
    us = per["tree_gdn_verify"]
    roof = {"bound": "hbm", "achieved": ver_b / (us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "traffic": None, "traffic_detail": "not measured for this kernel", "kernel": "tree_gdn_verify",
            "avg_us": us, "alg_bytes": ver_b,
            "others": {n: {"avg_us": per[n], "alg_bytes": b_, "frac": b_ / (per[n] * 1e-6) / 1e9 / HBM_PEAK_GBS}
                       for n, b_ in (("tree_gdn_conv", conv_b), ("tree_gdn_commit", com_b))}}
    roof["frac"] = roof["achieved"] / roof["peak"]
    line = {
        "metric": "tree nodes verified per second through one Gated-DeltaNet layer (conv + verify + commit)",
        "value": T / (step_us * 1e-6), "unit": "nodes/s", "n_gpus": 1, "steps": K_, "warmup": args.warmup,
        "ms_per_step": start.elapsed_time(end) / K_, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{wl.name} trees ({W.CONFIGS[wl.name]['desc']}); Gated-DeltaNet layer "
                               f"{hk} q/k heads, {hv} v heads, d {d}, conv {K}, {C} channels", "seed": wl.seed,
                   "accepted_tokens": n_acc},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        from oracle import tree_gdn_oracle as G
        # the first n nodes of request 0 (a prefix of a tree is a tree)
        n = int(wl.cu_nodes[1])
        sub = np.array([0, n])
        t0 = time.perf_counter()
        yo = G.gdn_conv_tree(gi.x[:n], gi.conv_state[:1], gi.conv_w, wl.parent[:n], sub)
        G.gdn_tree_verify(gi.q[:n], gi.k[:n], gi.v[:n], gi.g[:n], gi.beta[:n], gi.state[:1], wl.parent[:n], sub,
                          scale, True)
        dt = time.perf_counter() - t0
        del yo
        line["cpu_baseline"] = {"value": n / dt, "unit": "nodes/s", "cores": blas_threads(),
                                "kind": "oracle",
                                "sample": f"conv + verify of the first {n} nodes of request 0, all {hv} heads "
                                          f"({dt:.2f} s)"}
    print(json.dumps(line), flush=True)
    return 0


def C_void(x):
    import ctypes
    return ctypes.c_void_p(x)


if __name__ == "__main__":
    sys.exit(main())
