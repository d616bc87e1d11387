"""Benchmark: one verification step of tree attention on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
the ancestor mask, the attention and the greedy verifier.  By default the mask
is built inside the forward kernel (tree_attn_mask_and_forward ->
tree_verify_greedy); --separate-mask runs tree_attn_build_mask ->
tree_attn_forward -> tree_verify_greedy instead.  The default
workload is the Llama-3-8B-shaped layer (B=1, Hq=32, Hkv=8, D=128, prefix
L=4096, a 64-node draft tree of depth <= 6 and branching <= 4, bf16), with
greedy verification over a 64 x 128256 bf16 logits block (draft token equal to
the target argmax with probability 0.6).

Inputs are resident in HBM before timing starts.  To keep the 256 MB Infinity
Cache from serving repeated reads, the step rotates over --sets copies of every
input (16 x ~35 MB by default), so each step reads cold data.  Each step is
captured once per copy into a HIP graph and replayed (--eager launches every
call from Python instead); the graphs are checked bit for bit against eager
steps before timing.

Prints ONE JSON line: tree-tokens/s of the whole step (value), plus per-call
device times from HIP events on the launch stream, the roofline of the
dominant kernel, and the fp64 CPU oracle timed on a bounded sample of the same
workload (cpu_baseline).

    python bench.py [--steps K] [--warmup W] [--config llama3_8b] [--sets 16]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="llama3_8b")
    p.add_argument("--sets", type=int, default=32)
    p.add_argument("--separate-mask", action="store_true",
                   help="build the mask with its own call (tree_attn_build_mask) instead of "
                        "inside the forward (tree_attn_mask_and_forward)")
    p.add_argument("--eager", action="store_true",
                   help="launch every call from Python instead of replaying captured HIP graphs")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra-calls", action="store_true",
                   help="time only the step's calls (no standalone commit or next-token "
                        "verifier), so that profiler averages per kernel name cover the step")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--hbm-ceiling", action="store_true",
                   help="time plain device copies and a read-only reduction at several sizes "
                        "(the practical HBM ceiling) and print one JSON line")
    p.add_argument("--summarize-ceiling", metavar="FILE",
                   help="write profiles/hbm_ceiling.md from the --hbm-ceiling output in FILE")
    p.add_argument("--calib-copy", action="store_true",
                   help="only run a plain 256 MiB device-to-device copy (counter calibration)")
    p.add_argument("--summarize-mfma", metavar="DIR",
                   help="write profiles/tree_attn_forward_mfma.md from the MfmaUtil runs under DIR "
                        "(see MFMA_CMD)")
    p.add_argument("--summarize-configs", metavar="DIR",
                   help="write profiles/tree_attn_forward_configs.md from the per-workload runs "
                        "under DIR (see CONFIG_CMDS)")
    p.add_argument("--summarize-profiles", metavar="DIR",
                   help="write profiles/ summaries from rocprofv3 CSV output under DIR")
    return p.parse_args()


def src_hash(*names):
    """Hash of the named kernel sources and of the build script (which holds
    their compile flags): a change to either means a different kernel."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "tree_masked_attention_forward_amd")
    for path in [os.path.join(pkg, "csrc", n) for n in names] + [os.path.join(pkg, "build.py")]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key, current_hash):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, or None
    when absent or taken on a different kernel source."""
    path = os.path.join(PROFILES, "pmc_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != current_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


CALIB_BYTES = 256 * 2**20


def calib_copy():
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings scale
    the counters of the library's kernels to bytes."""
    import torch
    src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": CALIB_BYTES}))


HBM_CEILING_CMD = "python -u bench.py --hbm-ceiling > gpurun_out/hbm_ceiling.json"
CEILING_SIZES_MB = (16, 32, 64, 256, 1024)


def hbm_ceiling():
    """The practical HBM rate on this GPU: torch's device-to-device copy (bytes
    read + written) over buffers of each size, rotated over enough copies to
    exceed twice the 256 MB Infinity Cache so every pass reads cold data; HIP
    events around 50 passes."""
    import torch
    dev = torch.device("cuda:0")
    out = []
    for mb in CEILING_SIZES_MB:
        n = mb << 20
        sets = max(2, -(-1024 // mb))   # >= 1 GiB in rotation
        src = [torch.empty(n, dtype=torch.uint8, device=dev).fill_(1) for _ in range(sets)]
        dst = [torch.empty_like(src[0]) for _ in range(sets)]
        torch.cuda.synchronize()
        for i in range(2 * sets):   # warm-up: touch every page
            dst[i % sets].copy_(src[i % sets])
        reps = 50
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            dst[i % sets].copy_(src[i % sets])
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        res = {"MB": mb, "us": round(us, 2), "GBps": round(2 * n / (us * 1e-6) / 1e9, 1)}
        out.append(res)
        print(f"[ceiling] {res}", file=sys.stderr, flush=True)
        del src, dst
        torch.cuda.empty_cache()
    print(json.dumps({"hbm_ceiling": out, "peak_GBps": HBM_PEAK_GBS}))


def summarize_ceiling(path):
    with open(path) as f:
        rec = json.loads(f.read().strip().splitlines()[-1])
    lines = ["# Practical HBM ceiling on the MI355X box", "",
             "Command (repository root, MI355X box):", "", "    " + HBM_CEILING_CMD, "",
             "torch device-to-device copy of a buffer of each size (GB/s counts the bytes read "
             "plus the bytes written), 50 passes timed with HIP events, buffers rotated over "
             ">= 1 GiB so every pass reads cold data (the Infinity Cache is 256 MB). The "
             "published peak is 8 TB/s. For scale: one 8B-shaped forward call moves 18.1 "
             "algorithmic MB (35.9 MB counted by FETCH_SIZE + WRITE_SIZE).", "",
             "| buffer | us per copy | GB/s (read + write) |", "|---|---|---|"]
    for r in rec["hbm_ceiling"]:
        lines.append(f"| {r['MB']} MB | {r['us']} | {r['GBps']} |")
    with open(os.path.join(PROFILES, "hbm_ceiling.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def _read_csvs(root, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(root, "**", "*" + suffix), recursive=True)):
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _pmc_means(root, counter):
    """Mean counter value per kernel name over all dispatches (KiB for
    FETCH_SIZE / WRITE_SIZE)."""
    acc = {}
    for r in _read_csvs(root, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def summarize_profiles(root):
    """Turn rocprofv3 CSV output (runs made by the commands in PROFILE_CMDS,
    written under root/<name>) into profiles/*.md and profiles/pmc_traffic.json."""
    os.makedirs(PROFILES, exist_ok=True)
    # kernel trace summary
    stats = _read_csvs(os.path.join(root, "prof_trace"), "kernel_stats.csv")
    lines = ["# Kernel trace: one verification step, Llama-3-8B-shaped layer (N=64, L=4096)", "",
             "Command (run from the repository root on the MI355X box):", "",
             "    " + PROFILE_CMDS["prof_trace"], "",
             "| kernel | calls | avg us | min us | max us | % |", "|---|---|---|---|---|---|"]
    other_calls, other_ns = 0, 0.0
    for r in stats:
        name = r["Name"]
        if "ta::" not in name:
            # torch kernels of input setup and of the graph-vs-eager checks, outside the
            # timed region
            other_calls += int(r["Calls"])
            other_ns += float(r["TotalDurationNs"])
            continue
        short = name.replace("ta::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs'])/1e3:.3f} | "
                     f"{float(r['MinNs'])/1e3:.3f} | {float(r['MaxNs'])/1e3:.3f} | "
                     f"{float(r['Percentage']):.1f} |")
    if other_calls:
        lines += ["", f"Other kernels (input setup and the graph-vs-eager checks, outside the timed "
                      f"region): {other_calls} calls, {other_ns / 1e3:.1f} us in total."]
    with open(os.path.join(PROFILES, "tree_attn_step_llama3_8b_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    # HBM traffic from FETCH_SIZE / WRITE_SIZE, scaled by the copy calibration
    fetch = _pmc_means(os.path.join(root, "prof_fetch"), "FETCH_SIZE")
    write = _pmc_means(os.path.join(root, "prof_write"), "WRITE_SIZE")
    cf = _pmc_means(os.path.join(root, "prof_calib_fetch"), "FETCH_SIZE")
    cw = _pmc_means(os.path.join(root, "prof_calib_write"), "WRITE_SIZE")
    copy_f = max((v for k, v in cf.items() if "copy" in k.lower() or "elementwise" in k.lower()),
                 default=None)
    copy_w = max((v for k, v in cw.items() if "copy" in k.lower() or "elementwise" in k.lower()),
                 default=None)
    sf = (CALIB_BYTES / 1024) / copy_f if copy_f else 1.0
    sw = (CALIB_BYTES / 1024) / copy_w if copy_w else 1.0
    # The profiled runs take the default step, whose forward call is
    # tree_attn_mask_and_forward (the mask is built inside the forward kernel).
    groups = {"tree_attn_mask_and_forward": ("fwd_bf16_kernel", "merge_bf16_kernel"),
              "tree_verify_greedy": ("argmax_partial_kernel", "path_select_kernel"),
              "tree_attn_build_mask": ("build_mask_kernel",)}
    hashes = {"tree_attn_mask_and_forward": src_hash("attn_fwd.hip"),
              "tree_verify_greedy": src_hash("verify.hip"),
              "tree_attn_build_mask": src_hash("mask_build.hip")}
    rec = {"calibration": {"copy_bytes": CALIB_BYTES, "fetch_kib": copy_f, "write_kib": copy_w,
                           "fetch_scale": sf, "write_scale": sw}}
    md = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
          "Workload: one verification step of the Llama-3-8B-shaped layer (N=64, L=4096, bf16).",
          "Counters are KiB per dispatch; each is scaled by what the same counter reads for a",
          f"plain {CALIB_BYTES >> 20} MiB device copy (fetch x{sf:.3f}, write x{sw:.3f}).", "",
          "Commands (repository root, MI355X box):", ""]
    md += ["    " + PROFILE_CMDS[k] for k in ("prof_fetch", "prof_write", "prof_calib_fetch",
                                             "prof_calib_write")]
    md += ["", "| call | kernel | fetch KiB | write KiB | HBM bytes (scaled) |", "|---|---|---|---|---|"]
    for call, kernels in groups.items():
        total = 0.0
        for kn in kernels:
            fk = next((v for k, v in fetch.items() if kn in k), None)
            wk = next((v for k, v in write.items() if kn in k), None)
            if fk is None or wk is None:
                continue
            b = fk * 1024 * sf + wk * 1024 * sw
            total += b
            md.append(f"| {call} | `{kn}` | {fk:.1f} | {wk:.1f} | {b / 1e6:.3f} MB |")
        rec[call] = {"source_hash": hashes[call], "hbm_bytes_per_launch": round(total)}
    with open(os.path.join(PROFILES, "tree_attn_step_llama3_8b_hbm_traffic.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    with open(os.path.join(PROFILES, "pmc_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


PROFILE_CMDS = {
    "prof_trace": "rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof_trace -o run -- "
                  "python -u bench.py --steps 50 --warmup 5 --no-cpu-baseline --no-extra-calls",
    "prof_fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/prof_fetch -o run -- "
                  "python -u bench.py --steps 10 --warmup 2 --no-cpu-baseline --no-extra-calls",
    "prof_write": "rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/prof_write -o run -- "
                  "python -u bench.py --steps 10 --warmup 2 --no-cpu-baseline --no-extra-calls",
    "prof_calib_fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/prof_calib_fetch -o run -- "
                        "python -u bench.py --calib-copy",
    "prof_calib_write": "rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/prof_calib_write -o run -- "
                        "python -u bench.py --calib-copy",
}


# Per-workload runs: the bench line (per-call HIP-event times) and a kernel trace.
CONFIG_NAMES = ("llama3_8b", "batched", "llama3_70b", "forest")
CONFIG_CMDS = {
    "bench": "python -u bench.py --config {name} --steps 30 --warmup 5 --no-cpu-baseline "
             "> gpurun_out/cfg_{name}.json",
    "trace": "rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/cfg_trace_{name} -o run -- "
             "python -u bench.py --config {name} --steps 10 --warmup 2 --no-cpu-baseline "
             "--no-extra-calls",
}


def summarize_configs(root):
    """One table over the workloads: the forward call's device time (HIP events, p50
    over graph replays, and the kernel-trace average of its kernels), its algorithmic
    rate against the roof that bounds it, and the verifier's time."""
    rows = []
    for name in CONFIG_NAMES:
        try:
            with open(os.path.join(root, f"cfg_{name}.json")) as f:
                line = json.loads(f.read().strip().splitlines()[-1])
        except (OSError, ValueError, IndexError):
            continue
        d = line["detail"]
        fwd_call = line["roofline"]["kernel"] if line["roofline"]["kernel"] != "tree_verify_greedy" \
            else line["detail"]["roofline_other"]["kernel"]
        fw = d["forward"]
        r = line["roofline"] if line["roofline"]["kernel"] == fwd_call else d["roofline_other"]
        stats = _read_csvs(os.path.join(root, f"cfg_trace_{name}"), "kernel_stats.csv")
        fwd_ns = sum(float(x["AverageNs"]) for x in stats
                     if "fwd_bf16_kernel" in x["Name"] or "merge_bf16_kernel" in x["Name"])
        rows.append(f"| {name} | {line['config']['workload'].split(';')[0]} | "
                    f"{d['us_per_call_spread'][fwd_call]['p50']:.1f} | {fwd_ns / 1e3:.1f} | "
                    f"{r['achieved']} {r['unit']} | {r['bound']} | {r['frac']:.3f} | "
                    f"{fw['t_roof_us']:.1f} | {d['us_per_call']['tree_verify_greedy']:.1f} |")
    md = ["# Forward call on every workload (MI355X, one GPU)", "",
          "Commands (repository root, MI355X box), for each workload name:", "",
          "    " + CONFIG_CMDS["bench"], "    " + CONFIG_CMDS["trace"], "",
          "Times in microseconds per call. `events p50`: median over graph replays of the call on",
          "resident inputs (HIP events on the launch stream); `trace`: kernel-trace average of",
          "the forward's kernels (split kernel + merge kernel where there is one). The rate and",
          "fraction are the algorithmic bytes or flops per call over the events mean, against",
          "8 TB/s HBM or 2.5 PFLOP/s dense bf16 MFMA, whichever bounds the workload.", "",
          "| workload | shape | events p50 | trace | achieved | bound | roofline frac | roof | verify |",
          "|---|---|---|---|---|---|---|---|---|"] + rows
    with open(os.path.join(PROFILES, "tree_attn_forward_configs.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md))


MFMA_CMD = ("rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16 -f csv -d gpurun_out/mfma_{name} "
            "-o run -- python -u bench.py --config {name} --steps 10 --warmup 2 --no-cpu-baseline "
            "--no-extra-calls")


def summarize_mfma(root):
    """MFMA evidence for the forward kernel: the share of cycles the matrix units are
    busy (rocprofv3's MfmaUtil: SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs) and
    the MFMA work executed (SQ_INSTS_VALU_MFMA_MOPS_BF16, 512 flops per unit) against the
    algorithmic flops (taken from the per-workload bench line in the same directory)."""
    lines = ["# MFMA use of the forward kernel (rocprofv3 counters)", "",
             "Command (repository root, MI355X box), per workload name:", "",
             "    " + MFMA_CMD, "",
             "`MfmaUtil`: mean over the dispatches of the split kernel of the cycles its matrix",
             "units are busy, as a share of the cycles the GPU is active times the SIMD count.",
             "`executed`: MFMA flops the kernel issued (MOPS x 512); `algorithmic`: the dense",
             "prefix and visible tree pairs only; the excess is padding keys and masked tree keys.", "",
             "| workload | kernel | dispatches | MfmaUtil % | executed GFLOP | algorithmic GFLOP |",
             "|---|---|---|---|---|---|"]
    for name in CONFIG_NAMES:
        acc = {}
        for r in _read_csvs(os.path.join(root, f"mfma_{name}"), "counter_collection.csv"):
            if "fwd_bf16_kernel" not in r["Kernel_Name"]:
                continue
            short = r["Kernel_Name"].replace("ta::(anonymous namespace)::", "").replace(
                "void ", "").split("(")[0]
            acc.setdefault((short, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
        if not acc:
            continue
        alg = None
        try:
            with open(os.path.join(root, f"cfg_{name}.json")) as f:
                alg = json.loads(f.read().strip().splitlines()[-1])["detail"]["forward"]["alg_flops"]
        except (OSError, ValueError, IndexError, KeyError):
            pass
        for kname in sorted({k for k, _ in acc}):
            util = acc.get((kname, "MfmaUtil"), [])
            mops = acc.get((kname, "SQ_INSTS_VALU_MFMA_MOPS_BF16"), [])
            u = sum(util) / len(util) if util else float("nan")
            ex = sum(mops) / len(mops) * 512 / 1e9 if mops else float("nan")
            lines.append(f"| {name} | `{kname}` | {len(util)} | {u:.1f} | {ex:.2f} | "
                         f"{'' if alg is None else f'{alg / 1e9:.2f}'} |")
    with open(os.path.join(PROFILES, "tree_attn_forward_mfma.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    args = parse()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.summarize_configs:
        summarize_configs(args.summarize_configs)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma)
        return
    if args.calib_copy:
        calib_copy()
        return
    if args.hbm_ceiling:
        hbm_ceiling()
        return
    if args.summarize_ceiling:
        summarize_ceiling(args.summarize_ceiling)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path: sequences, KV heads or prefix chunks would shard across GPUs "
              "with an LSE merge, which is not built.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synthetic
    import tree_masked_attention_forward_amd as ta

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    case = synthetic.make_config_case(args.config, with_logits=True)
    B, Hq, Hkv, D = case.B, case.Hq, case.Hkv, case.D
    sum_n, sum_l = case.total_nodes, case.total_prefix
    max_nodes, max_prefix = case.max_nodes, case.max_prefix
    V = case.vocab
    W = ta.mask_words(max_nodes)

    # --- resident inputs, rotated over `sets` copies --------------------------------------
    base = {
        "parents": torch.from_numpy(case.parents).to(dev),
        "noffs": torch.from_numpy(case.node_offsets).to(dev),
        "poffs": torch.from_numpy(case.prefix_offsets).to(dev),
        "q": case.q.to(dev), "kt": case.k_tree.to(dev), "vt": case.v_tree.to(dev),
        "kp": case.k_prefix.to(dev), "vp": case.v_prefix.to(dev),
        "logits": case.logits.to(dev), "draft": torch.from_numpy(case.draft).to(dev),
    }
    # Enough distinct copies to cycle through 2x the 256 MB Infinity Cache.
    set_bytes = sum(v.numel() * v.element_size() for v in base.values())
    n_sets = max(1, min(args.sets, -(-2 * 256 * 2**20 // set_bytes)))
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(n_sets - 1)]
    mask = torch.empty((sum_n, W), dtype=torch.uint64, device=dev)
    depth = torch.empty(sum_n, dtype=torch.int32, device=dev)
    status = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty_like(base["q"])
    fws = torch.zeros(max(ta.forward_workspace_size(case.dtype, B, sum_n, max_nodes, Hq, Hkv, D,
                                                    sum_l, max_prefix), 16),
                      dtype=torch.uint8, device=dev)
    vws = torch.empty(max(ta.verify_workspace_size(sum_n, max_nodes, V), 16), dtype=torch.uint8,
                      device=dev)
    pred = torch.empty(sum_n, dtype=torch.int32, device=dev)
    alen = torch.empty(B, dtype=torch.int32, device=dev)
    anodes = torch.empty((B, max_nodes), dtype=torch.int32, device=dev)
    atok = torch.empty((B, max_nodes), dtype=torch.int32, device=dev)

    def do_mask(s):
        ta.build_mask(s["parents"], s["noffs"], max_nodes, mask=mask, depth=depth, status=status)

    def do_forward(s):
        ta.forward(s["q"], s["kt"], s["vt"], s["kp"], s["vp"], s["poffs"], s["noffs"], mask,
                   max_nodes, max_prefix, case.scale, out=out, workspace=fws)

    def do_mask_forward(s):
        ta.mask_and_forward(s["parents"], s["q"], s["kt"], s["vt"], s["kp"], s["vp"], s["poffs"],
                            s["noffs"], max_nodes, max_prefix, case.scale, out=out, mask=mask,
                            depth=depth, status=status, workspace=fws)

    def do_verify(s):
        ta.verify_greedy(s["logits"], s["draft"], mask, s["noffs"], max_nodes, workspace=vws,
                         target_argmax=pred, accept_len=alen, accept_nodes=anodes,
                         accept_tokens=atok)

    # A step: the ancestor mask (a1), the attention (a2-a4) and the greedy verifier (a5-a6).
    # By default the mask is built inside the forward kernel (one launch fewer).
    if args.separate_mask:
        calls = [("tree_attn_build_mask", do_mask), ("tree_attn_forward", do_forward),
                 ("tree_verify_greedy", do_verify)]
    else:
        calls = [("tree_attn_mask_and_forward", do_mask_forward),
                 ("tree_verify_greedy", do_verify)]
    fwd_call, fwd_fn = calls[-2]

    def one_step(s):
        for _, fn in calls:
            fn(s)

    def step(i):
        one_step(sets[i % len(sets)])

    # --- HIP graphs ------------------------------------------------------------------------
    # The Python binding costs tens of microseconds of host time per call, about as
    # much as the whole step on the GPU, so by default each step is captured once per
    # rotation set into a HIP graph (torch.cuda.CUDAGraph) and replayed: every replay
    # runs all the kernels of the step on that set's inputs.  The warmup runs eagerly
    # first (it also sets the kernels' LDS limits, which capture must not do).
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    def outputs():
        return [t.clone() for t in (mask, depth, status, out, pred, alen, anodes, atok)]

    def capture(fn, idx):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in idx:
                fn(sets[i])
        return g

    use_graphs = not args.eager
    n_rot = len(sets)
    if use_graphs:
        # A graph launch itself costs host time comparable to a step, so one graph holds
        # the steps of all rotation sets in order; single-step graphs cover the rest.
        step_graphs = [capture(one_step, [i]) for i in range(n_rot)]
        round_graph = capture(one_step, range(n_rot))
        # Every graph must reproduce the eager step bit for bit, replayed twice with eager
        # work on other inputs in between.
        for k, g in ((0, step_graphs[0]), (n_rot - 1, step_graphs[n_rot - 1]),
                     (n_rot - 1, round_graph)):
            step(k)
            torch.cuda.synchronize()
            ref = outputs()
            for rep in range(2):
                step(k + 1)
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                for a, b in zip(outputs(), ref):
                    if not torch.equal(a, b):
                        raise SystemExit(f"graph replay {rep} (last set {k}) differs from the "
                                         "eager step")

        def run_steps(k):
            for _ in range(k // n_rot):
                round_graph.replay()
            for i in range(k % n_rot):
                step_graphs[i].replay()
    else:
        def run_steps(k):
            for i in range(k):
                step(i)

    # --- whole-step timing ----------------------------------------------------------------
    run_steps(n_rot)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(args.steps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = sum_n * args.steps / elapsed
    print(f"[bench] {args.steps} steps in {elapsed:.4f} s ({'graphs' if use_graphs else 'eager'})",
          file=sys.stderr, flush=True)

    # --- per-call device time with HIP events on the launch stream ------------------------
    # One graph holds one call per rotation set; events bracket whole replays.
    stream = torch.cuda.current_stream(dev)

    def event_time(fn, n):
        """Mean device time per call (us) over about n calls, and the p10 / p50 /
        p90 over replays of the per-call time of one replay (one call per
        rotation set with graphs, one call without)."""
        if use_graphs:
            g = capture(fn, range(len(sets)))
            per = len(sets)
            reps = max(20, -(-n // per))
            run = lambda i: g.replay()
        else:
            per, reps = 1, max(20, n)
            run = lambda i: fn(sets[i % len(sets)])
        for i in range(2):
            run(i)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for i in range(reps):
            run(i)
            ev[i + 1].record(stream)
        ev[-1].synchronize()
        each = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 / per for i in range(reps))
        pct = lambda q: each[min(reps - 1, int(round(q * (reps - 1))))]
        mean = ev[0].elapsed_time(ev[-1]) * 1e3 / (reps * per)
        return mean, {"p10": round(pct(0.1), 3), "p50": round(pct(0.5), 3),
                      "p90": round(pct(0.9), 3), "replays": reps, "calls_per_replay": per}

    # The commit of the accepted path (the step after verification): the accepted rows
    # of each set's tree are appended to one cache slot per sequence, sized so that
    # every timed call finds room.
    one_step(sets[0])
    torch.cuda.synchronize()
    calls_max = 4 * max(20 * len(sets), args.steps) + 64   # above what event_time makes
    room = max(1, int(alen.max())) * calls_max
    L_b = torch.diff(base["poffs"])
    cache_offs = torch.zeros(B + 1, dtype=torch.int64, device=dev)
    cache_offs[1:] = torch.cumsum(L_b + room, 0)
    k_cache = torch.empty((int(cache_offs[-1]), Hkv, D), dtype=base["kt"].dtype, device=dev)
    v_cache = torch.empty_like(k_cache)
    cache_lens = L_b.clone()
    commit_status = torch.empty(B, dtype=torch.int32, device=dev)
    acc_len, acc_nodes = alen.clone(), anodes.clone()

    # The verifier on next-token rows: the same logits read as the token after each
    # node, plus one prefix row per sequence, and the bonus token.
    root_rows = torch.randn((B, V), generator=torch.Generator().manual_seed(99)).to(
        base["logits"].dtype).to(dev)
    vws_next = torch.empty(max(ta.verify_workspace_size(sum_n + B, max_nodes, V), 16),
                           dtype=torch.uint8, device=dev)
    nx = [torch.empty_like(t) for t in (pred, alen, anodes, atok)] + [
        torch.empty(B, dtype=torch.int32, device=dev)]

    def do_verify_next(s):
        ta.verify_greedy_next(s["logits"], root_rows, s["draft"], mask, s["noffs"], max_nodes,
                              workspace=vws_next, target_argmax=nx[0], accept_len=nx[1],
                              accept_nodes=nx[2], accept_tokens=nx[3], bonus_token=nx[4])

    def do_commit(s):
        ta.kv_commit(s["kt"], s["vt"], s["noffs"], acc_len, acc_nodes, k_cache, v_cache,
                     cache_offs, cache_lens, status=commit_status)

    do_mask(sets[0])
    t_mask, d_mask = event_time(do_mask, args.steps)
    t_fwd, d_fwd = event_time(fwd_fn, args.steps)
    t_ver, d_ver = event_time(do_verify, args.steps)
    t_commit = t_vnext = d_commit = d_vnext = None
    if not args.no_extra_calls:
        t_commit, d_commit = event_time(do_commit, args.steps)
        t_vnext, d_vnext = event_time(do_verify_next, args.steps)
    if t_commit is not None and not bool((commit_status == 0).all()):
        raise SystemExit("tree_kv_commit reported a failure in the timing loop")
    print(f"[bench] per call us: mask {t_mask:.2f} forward {t_fwd:.2f} verify {t_ver:.2f}",
          file=sys.stderr, flush=True)

    # --- algorithmic bytes / flops --------------------------------------------------------
    depth_h = depth.cpu().numpy().astype(np.int64)
    kv_bytes = 2 * sum_l * Hkv * D * 2 + 2 * sum_n * Hkv * D * 2
    fwd_bytes = kv_bytes + 2 * sum_n * Hq * D * 2 + sum_n * W * 8
    if not args.separate_mask:
        fwd_bytes += sum_n * 4 + sum_n * 4 + B * 4   # parents in; depth and status out
    lens = np.diff(case.prefix_offsets).astype(np.int64)
    nn = np.diff(case.node_offsets).astype(np.int64)
    fwd_flops = 4 * Hq * D * (int((nn * lens).sum()) + int((depth_h + 1).sum()))
    ver_bytes = sum_n * V * 2 + sum_n * 4 + sum_n * W * 8 + sum_n * 4 + B * (1 + 2 * max_nodes) * 4
    fwd_hash = src_hash("attn_fwd.hip")
    ver_hash = src_hash("verify.hip")

    fwd_gbs = fwd_bytes / (t_fwd * 1e-6) / 1e9
    fwd_tfs = fwd_flops / (t_fwd * 1e-6) / 1e12
    t_roof_fwd = max(fwd_bytes / (HBM_PEAK_GBS * 1e9), fwd_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12))
    ver_gbs = ver_bytes / (t_ver * 1e-6) / 1e9
    fwd_bound = "hbm" if fwd_bytes / (HBM_PEAK_GBS * 1e9) >= fwd_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) else "mfma"

    def roof(kind):
        if kind == "forward":
            if fwd_bound == "hbm":
                r = {"bound": "hbm", "achieved": round(fwd_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(fwd_gbs / HBM_PEAK_GBS, 4)}
            else:
                r = {"bound": "mfma", "achieved": round(fwd_tfs, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fwd_tfs / MFMA_BF16_PEAK_TFLOPS, 4)}
            r["traffic"] = load_traffic(fwd_call, fwd_hash)
            r["kernel"] = fwd_call
            return r
        r = {"bound": "hbm", "achieved": round(ver_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(ver_gbs / HBM_PEAK_GBS, 4),
             "traffic": load_traffic("tree_verify_greedy", ver_hash), "kernel": "tree_verify_greedy"}
        return r

    dominant = "forward" if t_fwd >= t_ver else "verify"
    other = "verify" if dominant == "forward" else "forward"

    # --- CPU baseline: the fp64 oracle on a bounded sample ----------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, args.cpu_seconds)

    line = {
        "metric": "tree-tokens/s and achieved KV GB/s (% roofline), Llama-3-8B shape, N=64, L=4096",
        "value": round(value, 1),
        "unit": "tree-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.config}: B={B} Hq={Hq} Hkv={Hkv} D={D} L={max_prefix} N={max_nodes} "
                        f"(sum_L={sum_l}, sum_N={sum_n}); greedy verify over V={V} bf16 logits",
            "step": " + ".join(n for n, _ in calls) + ", inputs rotated over "
                    f"{len(sets)} resident copies of {set_bytes / 2**20:.1f} MiB, "
                    + ("replayed from captured HIP graphs (one per round over the copies)"
                       if use_graphs else "launched eagerly from Python"),
            "global_batch": B, "seq_len": max_prefix, "tree_nodes": sum_n,
        },
        "roofline": roof(dominant),
        "cpu_baseline": cpu,
        "detail": {
            "us_per_call": {fwd_call: round(t_fwd, 3), "tree_verify_greedy": round(t_ver, 3),
                            "tree_attn_build_mask (standalone)": round(t_mask, 3),
                            "tree_kv_commit (standalone)": t_commit and round(t_commit, 3),
                            "tree_verify_greedy_next (standalone)": t_vnext and round(t_vnext, 3)},
            "us_per_call_spread": {fwd_call: d_fwd, "tree_verify_greedy": d_ver,
                                   "tree_attn_build_mask (standalone)": d_mask,
                                   "tree_kv_commit (standalone)": d_commit,
                                   "tree_verify_greedy_next (standalone)": d_vnext},
            "commit": {"accepted_rows": int(acc_len.sum()),
                       "alg_bytes": int(acc_len.sum()) * Hkv * D * base["kt"].element_size() * 4},
            "forward": {"tree_tokens_per_s": round(sum_n / (t_fwd * 1e-6), 1),
                        "kv_GBps": round(kv_bytes / (t_fwd * 1e-6) / 1e9, 1),
                        "alg_GBps": round(fwd_gbs, 1), "alg_TFLOPs": round(fwd_tfs, 2),
                        "alg_bytes": fwd_bytes, "alg_flops": fwd_flops,
                        "t_roof_us": round(t_roof_fwd * 1e6, 3),
                        "roofline_frac": round(t_roof_fwd / (t_fwd * 1e-6), 4)},
            "verify": {"alg_bytes": ver_bytes, "alg_GBps": round(ver_gbs, 1)},
            "roofline_other": roof(other),
            "source_hash": {"attn_fwd.hip": fwd_hash, "verify.hip": ver_hash},
        },
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(case, seconds):
    """The fp64 oracle as it stands, on whole steps of the same workload
    (mask + attention of every node + greedy verification), repeated until
    about `seconds` of CPU work; tree-tokens per second."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_info = threadpool_limits = None
    share = min(len(os.sched_getaffinity(0)), 16)
    limiter = threadpool_limits(limits=share) if threadpool_limits else None
    reps, t0 = 0, time.perf_counter()
    try:
        while True:
            oracle.build_mask(case.parents, case.node_offsets, case.max_nodes)
            oracle.tree_attention(case.q, case.k_tree, case.v_tree, case.k_prefix, case.v_prefix,
                                  case.parents, case.node_offsets, case.prefix_offsets, case.scale)
            oracle.verify_greedy(case.logits, case.draft, case.parents, case.node_offsets,
                                 case.max_nodes)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds or reps >= 20:
                break
        threads = share
        if threadpool_info:
            infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
            if infos:
                threads = max(i["num_threads"] for i in infos)
    finally:
        if limiter is not None:
            limiter.restore_original_limits()
    return {"value": round(case.total_nodes * reps / el, 2), "unit": "tree-tokens/s",
            "cores": int(threads), "kind": "oracle",
            "sample": f"{reps} whole step(s) of {case.name} (all {case.total_nodes} nodes, mask + "
                      f"fp64 attention + greedy verify over V={case.vocab}) in {el:.1f} s"}


if __name__ == "__main__":
    main()
