"""Benchmark: the tree attention forward of one layer, and the verification
step around it, on one MI355X.

The headline is the forward call's throughput in tree tokens per second: the
tree_attn_mask_and_forward call (the ancestor mask built inside the forward
kernel; --separate-mask: tree_attn_forward on a mask from its own
tree_attn_build_mask call) timed with HIP events over exactly --steps calls.
The default workload is the Llama-3-8B-shaped layer (B=1, Hq=32, Hkv=8, D=128,
prefix L=4096, a 64-node draft tree of depth <= 6 and branching <= 4, bf16).
The whole step (mask, forward and the greedy verifier over a 64 x 128256 bf16
logits block, draft token equal to the target argmax with probability 0.6) is
timed over the same number of steps and reported in `detail`, with every call's
own device time, the cost of one candidate against 64 at the same prefix (a
one-node tree, `detail.M3`), the roofline of the forward, and the fp64 CPU
oracle timed on a bounded sample of the same workload (cpu_baseline).

Inputs are resident in HBM before timing starts.  To keep the 256 MB Infinity
Cache from serving repeated reads, calls rotate over copies of every input (at
least 512 MB in rotation); the number of copies divides --steps, so the timed
region is a whole number of rotation rounds.  Each round is captured once into
a HIP graph and replayed (--eager launches every call from Python instead); the
graphs are checked bit for bit against eager calls before timing.

    python bench.py [--steps K] [--warmup W] [--config llama3_8b]
    python bench.py --hbm-ceiling      # copy, streaming-read and launch floors
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
    p.add_argument("--sets", type=int, default=16,
                   help="most input copies in rotation needed to pass 512 MB (the count is then "
                        "rounded up to a divisor of --steps)")
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
                   help="time plain device copies and a streaming read at several sizes (the "
                        "practical HBM ceilings) and empty kernels (the launch floor); print one "
                        "JSON line")
    p.add_argument("--summarize-ceiling", metavar="FILE",
                   help="write profiles/hbm_ceiling.md and profiles/launch_floor.md from the "
                        "--hbm-ceiling output in FILE")
    p.add_argument("--compute-ceiling", action="store_true",
                   help="time the MFMA and VALU rate probes and print one JSON line")
    p.add_argument("--summarize-compute", metavar="FILE",
                   help="write profiles/compute_ceiling.md from the --compute-ceiling output in FILE")
    p.add_argument("--timeline", metavar="WORKLOAD",
                   help="per-workgroup timeline of one forward call on WORKLOAD from the timeline "
                        "build (build.py --timeline); print one JSON line")
    p.add_argument("--summarize-timeline", metavar="DIR",
                   help="write profiles/tree_attn_forward_timeline.md from the --timeline outputs "
                        "(timeline_*.json) in DIR")
    p.add_argument("--no-m3", action="store_true",
                   help="skip the one-node-tree variant of the workload")
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


def load_traffic(config, kernel_key, current_hash):
    """HBM bytes per call from committed rocprofv3 --pmc summaries of this
    workload, or None when absent or taken on a different kernel source."""
    path = os.path.join(PROFILES, "pmc_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(config, {}).get(kernel_key)
    except (OSError, ValueError, AttributeError):
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
LAUNCH_TRACE_CMD = ("rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof_ceiling -o run -- "
                    "python -u bench.py --hbm-ceiling")
CEILING_SIZES_MB = (16, 32, 64, 256, 1024)
READ_GRIDS = (1024, 2048, 4096, 8192)
EMPTY_GRIDS = (1, 256, 2048, 16384)


def _probes():
    """The measurement probes (libtaprobes.so, built next to the library)."""
    import ctypes
    path = os.path.join(ROOT, "tree_masked_attention_forward_amd", "libtaprobes.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing: run tree_masked_attention_forward_amd/build.py")
    lib = ctypes.CDLL(path)
    lib.ta_probe_read.restype = ctypes.c_int
    lib.ta_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_void_p]
    lib.ta_probe_empty.restype = ctypes.c_int
    lib.ta_probe_empty.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.ta_probe_mfma.restype = ctypes.c_int
    lib.ta_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.ta_probe_valu.restype = ctypes.c_int
    lib.ta_probe_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_void_p]
    lib.ta_probe_lds.restype = ctypes.c_int
    lib.ta_probe_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.c_void_p]
    return lib


COMPUTE_CEILING_CMD = "python -u bench.py --compute-ceiling > gpurun_out/compute_ceiling.json"
SIMDS, CLOCK_HZ = 256 * 4, 2.4e9   # MI355X: 256 CUs of 4 SIMDs, 2.4 GHz


def compute_ceiling():
    """Sustained matrix and vector rates: 512 workgroups of 8 waves (two per
    SIMD) running independent v_mfma_f32_32x32x16_bf16 chains, fp32 FMA chains
    and exp2 chains; HIP events around one launch each (after a warm-up)."""
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    probes = _probes()
    stream = torch.cuda.current_stream(dev)
    grid = 512
    sink = torch.zeros(grid, dtype=torch.float32, device=dev)

    def timed(fn):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3

    def check(rc, what):
        if rc:
            raise SystemExit(f"{what} failed ({rc})")

    out = {}
    iters = 4096
    t = timed(lambda: check(probes.ta_probe_mfma(grid, iters, sink.data_ptr(), stream.cuda_stream),
                            "ta_probe_mfma"))
    flops = grid * 8 * 4 * iters * 32768
    out["mfma_bf16_32x32x16"] = {"s": t, "TFLOPs": round(flops / t / 1e12, 1),
                                 "frac_of_2500": round(flops / t / 2.5e15, 3),
                                 "cycles_per_mfma_per_simd": round(SIMDS * CLOCK_HZ * t /
                                                                   (grid * 8 * 4 * iters), 2)}
    for op, name in ((0, "fma_f32"), (1, "exp2_f32")):
        iters = 16384
        t = timed(lambda: check(probes.ta_probe_valu(grid, iters, op, sink.data_ptr(),
                                                     stream.cuda_stream), "ta_probe_valu"))
        instr = grid * 8 * 8 * iters   # wave64 instructions
        out[name] = {"s": t, "wave_instr_per_s": instr / t,
                     "cycles_per_wave_instr_per_simd": round(SIMDS * CLOCK_HZ * t / instr, 2)}
    # LDS: 16-byte reads alone, then each feeding an MFMA (the score step's pattern).
    iters = 4096
    for op, name in ((0, "lds_read_b128"), (1, "mfma_from_lds")):
        t = timed(lambda: check(probes.ta_probe_lds(grid, iters, op, sink.data_ptr(),
                                                    stream.cuda_stream), "ta_probe_lds"))
        reads = grid * 8 * 8 * iters   # wave64 16-byte reads, 1 KB each
        rec = {"s": t, "bytes_per_clk_per_cu": round(reads * 1024 / t / 256 / CLOCK_HZ, 1)}
        if op == 1:
            flops = reads * 32768
            rec.update({"TFLOPs": round(flops / t / 1e12, 1),
                        "frac_of_2500": round(flops / t / 2.5e15, 3)})
        out[name] = rec
    print(json.dumps({"compute_ceiling": out}))


def summarize_compute(path):
    with open(path) as f:
        rec = json.loads(f.read().strip().splitlines()[-1])["compute_ceiling"]
    m, fma, ex = rec["mfma_bf16_32x32x16"], rec["fma_f32"], rec["exp2_f32"]
    lines = ["# Matrix and vector rates on the MI355X box", "",
             "Command (repository root, MI355X box):", "", "    " + COMPUTE_CEILING_CMD, "",
             "Probes in `csrc/probes.hip` (`libtaprobes.so`): 512 workgroups of 8 waves (two per "
             "SIMD), each wave running independent dependency chains; one launch timed with HIP "
             "events after a warm-up; cycles per instruction per SIMD at 2.4 GHz over 1024 SIMDs.",
             "", "| probe | rate | cycles per wave instruction per SIMD |", "|---|---|---|",
             f"| `v_mfma_f32_32x32x16_bf16`, 4 chains per wave | {m['TFLOPs']} TFLOP/s "
             f"({m['frac_of_2500']} of 2.5 PFLOP/s) | {m['cycles_per_mfma_per_simd']} |",
             f"| fp32 FMA, 8 chains per thread | {fma['wave_instr_per_s'] / 1e12:.2f} T wave "
             f"instr/s | {fma['cycles_per_wave_instr_per_simd']} |",
             f"| `v_exp_f32` (exp2), 8 chains per thread | {ex['wave_instr_per_s'] / 1e12:.2f} T wave "
             f"instr/s | {ex['cycles_per_wave_instr_per_simd']} |"]
    if "lds_read_b128" in rec:
        lr, ml = rec["lds_read_b128"], rec["mfma_from_lds"]
        lines += ["", "LDS (`ta_probe_lds`, same grid): 16-byte reads with no bank conflicts, eight "
                  "in flight per wave; then the same reads each feeding one "
                  "`v_mfma_f32_32x32x16_bf16` as its A operand (two accumulator chains per wave, "
                  "B in registers), the attention's score-step pattern.", "",
                  "| probe | rate | LDS bytes per clock per CU (2.4 GHz) |", "|---|---|---|",
                  f"| LDS reads alone | {lr['bytes_per_clk_per_cu'] * 256 * CLOCK_HZ / 1e12:.1f} TB/s "
                  f"| {lr['bytes_per_clk_per_cu']} |",
                  f"| MFMA fed from LDS | {ml['TFLOPs']} TFLOP/s ({ml['frac_of_2500']} of 2.5 "
                  f"PFLOP/s) | {ml['bytes_per_clk_per_cu']} |"]
    with open(os.path.join(PROFILES, "compute_ceiling.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


TIMELINE_CMD = "python -u bench.py --timeline {name} > gpurun_out/timeline_{name}.json"
TIMELINE_WORKLOADS = ["llama3_8b", "batched", "llama3_70b", "tree_4096"]


def timeline(name):
    """Per-workgroup timeline of one tree_attn_mask_and_forward call on a
    workload, from the timeline build of the library (csrc/attn_fwd.hip with
    TA_TIMELINE: thread 0 of every forward workgroup stamps a 100 MHz counter
    at fixed points, see the slot list there).  Twelve input copies rotate in
    a captured graph, as the benchmark replays them; the stamps are those of
    the graph's last call."""
    import ctypes
    import numpy as np
    import torch
    import synthetic
    import tree_masked_attention_forward_amd  # noqa: F401  (loads the library first)
    import tree_masked_attention_forward_amd._binding as tb
    path = os.path.join(ROOT, "tree_masked_attention_forward_amd", "libtreeattn_timeline.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing: run tree_masked_attention_forward_amd/build.py "
                         "--timeline")
    lib = tb.load_library(path)
    tb._lib = lib   # the binding's calls now go to the timeline build
    lib.ta_timeline_set.restype = ctypes.c_int
    lib.ta_timeline_set.argtypes = [ctypes.c_void_p, ctypes.c_longlong]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    case = synthetic.make_config_case(name, with_logits=False)
    cap = 1 << 16
    buf = torch.zeros(cap * 16, dtype=torch.int64, device=dev)
    sets = []
    for _ in range(12):
        sets.append((torch.from_numpy(case.parents).to(dev), case.q.to(dev), case.k_tree.to(dev),
                     case.v_tree.to(dev), case.k_prefix.to(dev), case.v_prefix.to(dev),
                     torch.from_numpy(case.prefix_offsets).to(dev),
                     torch.from_numpy(case.node_offsets).to(dev)))
    n = tb.forward_workspace_size(torch.bfloat16, case.B, case.total_nodes, case.max_nodes,
                                  case.Hq, case.Hkv, case.D, case.total_prefix, case.max_prefix)
    ws = torch.zeros(max(n, 16), dtype=torch.uint8, device=dev)
    out = torch.empty_like(sets[0][1])

    def call(i):
        tb.mask_and_forward(*sets[i % len(sets)], case.max_nodes, case.max_prefix, case.scale,
                            out=out, workspace=ws)
    for i in range(30):
        call(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(len(sets)):
            call(i)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    if lib.ta_timeline_set(buf.data_ptr(), cap) != 0:
        raise SystemExit("ta_timeline_set failed")
    buf.zero_()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    lib.ta_timeline_set(None, 0)
    t = buf.view(cap, 16).cpu().numpy().astype(np.int64)
    t = t[t[:, 0] != 0]
    print(json.dumps({"timeline": {"workload": name, **timeline_summary(t)}}))


def timeline_summary(t):
    """Percentiles (us from the call's first workgroup start) of each stamp,
    and the per-CU picture (CU from HW_REG_HW_ID bits: CU 8-11, SH 12, SE 13-15)."""
    import numpy as np
    kind = t[:, 6] & 255
    sp, mg = kind == 1, kind == 2
    t0 = t[:, 0].min()

    def us(c):
        return (t[:, c] - t0) / 100.0

    def pct(x):
        x = np.asarray(x, dtype=float)
        if x.size == 0:
            return None
        return {q: round(float(np.percentile(x, p)), 2)
                for q, p in (("p0", 0), ("p10", 10), ("p50", 50), ("p90", 90), ("p100", 100))}
    tiles = t[:, 14] & 0xffff
    end_split = us(5)[sp]
    res = {"workgroups": int(len(t)), "splits": int(sp.sum()), "merge_workgroups": int(mg.sum()),
           "span_us": round(float(us(5).max()), 2),
           "split": {"start": pct(us(0)[sp]), "offsets_decoded": pct(us(1)[sp]),
                     "first_stage": pct(us(2)[sp]), "loop_done": pct(us(3)[sp]),
                     "end": pct(end_split),
                     "loop_us_per_tile": pct((us(3) - us(2))[sp] / np.maximum(tiles[sp], 1)),
                     "before_loop_us": pct((us(2) - us(0))[sp]),
                     "after_loop_us": pct((us(5) - us(3))[sp])}}
    if mg.any():
        res["merge"] = {"start": pct(us(0)[mg]), "group_seen_complete": pct(us(4)[mg]),
                        "end": pct(us(5)[mg])}
    hw = t[:, 15]
    xcc = (t[:, 6] >> 8) & 255
    cu = xcc * 1000 + ((hw >> 13) & 7) * 100 + ((hw >> 12) & 1) * 16 + ((hw >> 8) & 15)
    ends, ntiles, nwg = {}, {}, {}
    for i in np.flatnonzero(sp):
        k = int(cu[i])
        ends[k] = max(ends.get(k, 0.0), float(us(5)[i]))
        ntiles[k] = ntiles.get(k, 0) + int(tiles[i])
        nwg[k] = nwg.get(k, 0) + 1
    res["cus"] = {"used": len(ends), "split_workgroups_per_cu": pct(list(nwg.values())),
                  "tiles_per_cu": pct(list(ntiles.values())),
                  "last_split_end_per_cu": pct(list(ends.values()))}
    return res


def summarize_timeline(root):
    recs = []
    for name in TIMELINE_WORKLOADS:
        path = os.path.join(root, f"timeline_{name}.json")
        if os.path.exists(path):
            with open(path) as f:
                recs.append(json.loads(f.read().strip().splitlines()[-1])["timeline"])

    def p(d, key="p50"):
        return "" if d is None else f"{d[key]:.1f}"
    lines = ["# Per-workgroup timeline of one forward call", "",
             "Build and commands (repository root; the timeline build is "
             "`csrc/attn_fwd.hip` compiled with `TA_TIMELINE`, whose workgroups stamp a 100 MHz "
             "counter at fixed points; the product library has no trace code):", "",
             "    python tree_masked_attention_forward_amd/build.py --timeline",
             *["    " + TIMELINE_CMD.format(name=n) for n in TIMELINE_WORKLOADS], "",
             "Times in microseconds from the call's first workgroup start, p50 over the split "
             "workgroups (p10 / p90 where given); the last call of a replayed graph of twelve.", "",
             "| workload | split wgs | offsets decoded | first stage in LDS | loop done | split end "
             "(p50 / p100) | us per 32-key tile | before loop | merge wgs: group complete / end "
             "(p50 / p100) | CUs: tiles per CU (p0 / p50 / p100) | call span |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in recs:
        s = r["split"]
        m = r.get("merge")
        mtxt = (f"{p(m['group_seen_complete'])} / {p(m['end'])} / {p(m['end'], 'p100')}"
                if m else "separate kernel")
        c = r["cus"]["tiles_per_cu"]
        lines.append(f"| {r['workload']} | {r['splits']} | {p(s['offsets_decoded'])} | "
                     f"{p(s['first_stage'])} | {p(s['loop_done'])} | {p(s['end'])} / "
                     f"{p(s['end'], 'p100')} | {s['loop_us_per_tile']['p50']:.3f} | "
                     f"{p(s['before_loop_us'])} | {mtxt} | {c['p0']:.0f} / {c['p50']:.0f} / "
                     f"{c['p100']:.0f} | {r['span_us']:.1f} |")
    with open(os.path.join(PROFILES, "tree_attn_forward_timeline.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def hbm_ceiling():
    """Practical ceilings on this GPU, each timed with HIP events:
    * copy: torch's device-to-device copy (bytes read + written) per size;
    * read: a plain streaming read (16-byte nontemporal loads, libtaprobes.so)
      per size, best over a few grid sizes -- the rate a read-bound kernel can
      reach at that size;
    * launch: back-to-back empty kernels per grid size, launched eagerly and
      replayed from a captured graph -- the floor under a one-launch call.
    Buffers rotate over >= 1 GiB so every pass reads cold data (the Infinity
    Cache is 256 MB)."""
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    probes = _probes()
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    sink = torch.zeros(1 << 20, dtype=torch.int32, device=dev)

    def timed(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    def read(buf, grid):
        rc = probes.ta_probe_read(buf.data_ptr(), buf.numel(), sink.data_ptr(), grid, sh)
        if rc:
            raise SystemExit(f"ta_probe_read failed ({rc})")

    copy, reads = [], []
    for mb in CEILING_SIZES_MB:
        n = mb << 20
        sets = max(2, -(-1024 // mb))   # >= 1 GiB in rotation
        src = [torch.empty(n, dtype=torch.uint8, device=dev).fill_(1) for _ in range(sets)]
        dst = [torch.empty_like(src[0]) for _ in range(sets)]
        torch.cuda.synchronize()
        for i in range(2 * sets):   # touch every page
            dst[i % sets].copy_(src[i % sets])
        us = timed(lambda i: dst[i % sets].copy_(src[i % sets]), 50)
        copy.append({"MB": mb, "us": round(us, 2), "GBps": round(2 * n / (us * 1e-6) / 1e9, 1)})
        del dst
        best = None
        per_grid = {}
        for grid in READ_GRIDS:
            for i in range(sets):
                read(src[i], grid)
            us = timed(lambda i: read(src[i % sets], grid), 50)
            per_grid[grid] = round(n / (us * 1e-6) / 1e9, 1)
            if best is None or us < best[0]:
                best = (us, grid)
        reads.append({"MB": mb, "us": round(best[0], 2), "grid": best[1],
                      "GBps": round(n / (best[0] * 1e-6) / 1e9, 1), "GBps_per_grid": per_grid})
        print(f"[ceiling] {mb} MB copy {copy[-1]['GBps']} GB/s read {reads[-1]['GBps']} GB/s",
              file=sys.stderr, flush=True)
        del src
        torch.cuda.empty_cache()

    launch = []
    reps = 200
    for grid in EMPTY_GRIDS:
        def empty(i, grid=grid):
            # the current stream: torch's capture stream while a graph is captured
            rc = probes.ta_probe_empty(grid, 256, torch.cuda.current_stream(dev).cuda_stream)
            if rc:
                raise SystemExit(f"ta_probe_empty failed ({rc})")
        for i in range(20):
            empty(i)
        eager = timed(empty, reps)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                empty(i)
        g.replay()
        torch.cuda.synchronize()
        graph = timed(lambda i: g.replay(), 5) / reps
        launch.append({"grid": grid, "block": 256, "eager_us": round(eager, 3),
                       "graph_us": round(graph, 3)})
        print(f"[launch] grid {grid}: eager {eager:.2f} us, graph {graph:.2f} us per launch",
              file=sys.stderr, flush=True)
    print(json.dumps({"hbm_copy": copy, "hbm_read": reads, "launch_floor": launch,
                      "peak_GBps": HBM_PEAK_GBS}))


def summarize_ceiling(path, trace_root=None):
    with open(path) as f:
        rec = json.loads(f.read().strip().splitlines()[-1])
    lines = ["# Practical HBM ceilings on the MI355X box", "",
             "Command (repository root, MI355X box):", "", "    " + HBM_CEILING_CMD, "",
             "Buffers rotate over >= 1 GiB so every pass reads cold data (the Infinity Cache is "
             "256 MB); HIP events around 50 passes. The published peak is 8 TB/s.", "",
             "* **read**: a plain streaming read (`ta_probe_read` in `csrc/probes.hip`: 16-byte "
             "nontemporal loads, eight in flight per thread, folded so they stay live), best over "
             f"grids of {', '.join(map(str, READ_GRIDS))} workgroups of 256 threads. This is the "
             "rate a read-bound kernel can reach at that size: the ceiling for the forward, "
             "whose traffic is K/V reads.",
             "* **copy**: torch's device-to-device copy; GB/s counts bytes read plus bytes "
             "written.", "",
             "| buffer | read us | read GB/s | best grid | copy us | copy GB/s (read + write) |",
             "|---|---|---|---|---|---|"]
    for r, c in zip(rec["hbm_read"], rec["hbm_copy"]):
        lines.append(f"| {r['MB']} MB | {r['us']} | {r['GBps']} | {r['grid']} | {c['us']} | "
                     f"{c['GBps']} |")
    lines += ["", "Read GB/s per grid size:", "",
              "| buffer | " + " | ".join(f"{g} WG" for g in READ_GRIDS) + " |",
              "|---|" + "---|" * len(READ_GRIDS)]
    for r in rec["hbm_read"]:
        lines.append(f"| {r['MB']} MB | " + " | ".join(
            str(r["GBps_per_grid"].get(str(g), r["GBps_per_grid"].get(g, ""))) for g in READ_GRIDS)
            + " |")
    with open(os.path.join(PROFILES, "hbm_ceiling.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    lines = ["# Launch floor on the MI355X box", "",
             "Command (repository root, MI355X box):", "", "    " + HBM_CEILING_CMD, "",
             "An empty kernel (`ta_probe_empty` in `csrc/probes.hip`) of the given grid of "
             "256-thread workgroups, 200 launches back to back on one stream, timed with HIP "
             "events: eagerly from Python, and replayed from one captured HIP graph holding all "
             "200. Microseconds per launch, launch to launch: the least any call of one launch "
             "costs in a stream of calls.", "",
             "| grid | eager us per launch | graph us per launch |", "|---|---|---|"]
    for r in rec["launch_floor"]:
        lines.append(f"| {r['grid']} | {r['eager_us']} | {r['graph_us']} |")
    if trace_root:
        stats = _read_csvs(trace_root, "kernel_stats.csv")
        rows = [r for r in stats if "empty_kernel" in r["Name"] or "read_kernel" in r["Name"]]
        if rows:
            lines += ["", "Kernel trace of the same run (every grid size together):", "",
                      "    " + LAUNCH_TRACE_CMD, "",
                      "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
            for r in rows:
                short = r["Name"].replace("(anonymous namespace)::", "").split("(")[0]
                lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                             f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} |")
    with open(os.path.join(PROFILES, "launch_floor.md"), "w") as f:
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


def _short(name):
    return name.replace("ta::(anonymous namespace)::", "").replace("void ", "").split("(")[0]


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
        lines.append(f"| `{_short(name)}` | {r['Calls']} | {float(r['AverageNs'])/1e3:.3f} | "
                     f"{float(r['MinNs'])/1e3:.3f} | {float(r['MaxNs'])/1e3:.3f} | "
                     f"{float(r['Percentage']):.1f} |")
    if other_calls:
        lines += ["", f"Other kernels (input setup and the graph-vs-eager checks, outside the timed "
                      f"region): {other_calls} calls, {other_ns / 1e3:.1f} us in total."]
    if stats:
        with open(os.path.join(PROFILES, "tree_attn_step_llama3_8b_kernel_trace.md"), "w") as f:
            f.write("\n".join(lines) + "\n")
    # the calls outside the step (commit, next-token and stochastic verifiers)
    extra = _read_csvs(os.path.join(root, "prof_trace_extra"), "kernel_stats.csv")
    if extra:
        lines = ["# Kernel trace: the standalone calls, Llama-3-8B-shaped step (N=64, V=128256)", "",
                 "The same step as the main trace plus the calls timed beside it: the commit of",
                 "the accepted path (`kv_commit_kernel`), the next-token verifier (the argmax over",
                 "node and prefix rows, `path_select_kernel<true>`) and stochastic verification",
                 "(`softmax_stats_kernel` over the 65 rows, then `spec_sample_kernel`).", "",
                 "Command (run from the repository root on the MI355X box):", "",
                 "    " + PROFILE_CMDS["prof_trace_extra"], "",
                 "| kernel | calls | avg us | min us | max us | % |", "|---|---|---|---|---|---|"]
        for r in extra:
            if "ta::" not in r["Name"]:
                continue
            lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | "
                         f"{float(r['AverageNs'])/1e3:.3f} | {float(r['MinNs'])/1e3:.3f} | "
                         f"{float(r['MaxNs'])/1e3:.3f} | {float(r['Percentage']):.1f} |")
        with open(os.path.join(PROFILES, "tree_attn_extra_calls_llama3_8b_kernel_trace.md"),
                  "w") as f:
            f.write("\n".join(lines) + "\n")
    # HBM traffic from FETCH_SIZE / WRITE_SIZE, scaled by the copy calibration
    cf = _pmc_means(os.path.join(root, "prof_calib_fetch"), "FETCH_SIZE")
    cw = _pmc_means(os.path.join(root, "prof_calib_write"), "WRITE_SIZE")
    copy_f = max((v for k, v in cf.items() if "copy" in k.lower() or "elementwise" in k.lower()),
                 default=None)
    copy_w = max((v for k, v in cw.items() if "copy" in k.lower() or "elementwise" in k.lower()),
                 default=None)
    sf = (CALIB_BYTES / 1024) / copy_f if copy_f else 1.0
    sw = (CALIB_BYTES / 1024) / copy_w if copy_w else 1.0
    # The profiled runs take the default step, whose forward call is
    # tree_attn_mask_and_forward (the mask is built inside the forward kernel,
    # or by build_mask_kernel within the call for trees above 128 nodes).
    groups = {"tree_attn_mask_and_forward": ("fwd_bf16_kernel", "merge_bf16_kernel",
                                             "build_mask_kernel", "build_mask_large_kernel"),
              "tree_verify_greedy": ("argmax_partial_kernel", "path_select", "large_rows_kernel",
                                     "large_accept_kernel", "large_place_kernel")}
    hashes = {"tree_attn_mask_and_forward": src_hash("attn_fwd.hip"),
              "tree_verify_greedy": src_hash("verify.hip")}
    rec = {"calibration": {"copy_bytes": CALIB_BYTES, "fetch_kib": copy_f, "write_kib": copy_w,
                           "fetch_scale": sf, "write_scale": sw}}
    md = ["# HBM traffic per call (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
          "Counters are KiB per dispatch, averaged over the run's dispatches of each kernel;",
          "each is scaled by what the same counter reads for a plain",
          f"{CALIB_BYTES >> 20} MiB device copy (fetch x{sf:.3f}, write x{sw:.3f}). `alg` is",
          "the call's algorithmic bytes (K/V, Q, mask words, outputs) from the workload's bench",
          "line; `ratio` = counted / algorithmic.", "",
          "Commands (repository root, MI355X box), per workload name:", "",
          "    " + PROFILE_CMDS["prof_fetch"], "    " + PROFILE_CMDS["prof_write"],
          "    " + PROFILE_CMDS["prof_calib_fetch"], "    " + PROFILE_CMDS["prof_calib_write"], "",
          "| workload | call | kernel | fetch KiB | write KiB | HBM bytes (scaled) | alg | ratio |",
          "|---|---|---|---|---|---|---|---|"]
    for name in CONFIG_NAMES:
        fetch = _pmc_means(os.path.join(root, f"prof_fetch_{name}"), "FETCH_SIZE")
        write = _pmc_means(os.path.join(root, f"prof_write_{name}"), "WRITE_SIZE")
        if not fetch or not write:
            continue
        alg = {}
        try:
            with open(os.path.join(root, f"cfg_{name}.json")) as f:
                d = json.loads(f.read().strip().splitlines()[-1])["detail"]
            alg = {"tree_attn_mask_and_forward": d["forward"]["alg_bytes"],
                   "tree_verify_greedy": d["verify"]["alg_bytes"]}
        except (OSError, ValueError, IndexError, KeyError):
            pass
        rec[name] = {}
        for call, kernels in groups.items():
            total, parts = 0.0, []
            for kn in kernels:
                fk = next((v for k, v in fetch.items() if kn in k), None)
                wk = next((v for k, v in write.items() if kn in k), None)
                if fk is None or wk is None:
                    continue
                b = fk * 1024 * sf + wk * 1024 * sw
                total += b
                parts.append((kn, fk, wk, b))
            if not parts:
                continue
            a = alg.get(call)
            for kn, fk, wk, b in parts:
                md.append(f"| {name} | {call} | `{kn}` | {fk:.1f} | {wk:.1f} | {b / 1e6:.3f} MB | | |")
            md.append(f"| {name} | {call} | **all** | | | **{total / 1e6:.3f} MB** | "
                      f"{'' if a is None else f'{a / 1e6:.3f} MB'} | "
                      f"{'' if a is None else f'{total / a:.2f}'} |")
            rec[name][call] = {"source_hash": hashes[call], "hbm_bytes_per_launch": round(total),
                               "alg_bytes": a}
    with open(os.path.join(PROFILES, "tree_attn_hbm_traffic.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    with open(os.path.join(PROFILES, "pmc_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


PROFILE_CMDS = {
    "prof_trace": "rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof_trace -o run -- "
                  "python -u bench.py --steps 50 --warmup 5 --no-cpu-baseline --no-extra-calls "
                  "--no-m3",
    "prof_trace_extra": "rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof_trace_extra "
                        "-o run -- python -u bench.py --steps 20 --warmup 2 --no-cpu-baseline "
                        "--no-m3",
    "prof_fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/prof_fetch_{name} -o run -- "
                  "python -u bench.py --config {name} --steps 10 --warmup 2 --no-cpu-baseline "
                  "--no-extra-calls --no-m3",
    "prof_write": "rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/prof_write_{name} -o run -- "
                  "python -u bench.py --config {name} --steps 10 --warmup 2 --no-cpu-baseline "
                  "--no-extra-calls --no-m3",
    "prof_calib_fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/prof_calib_fetch -o run -- "
                        "python -u bench.py --calib-copy",
    "prof_calib_write": "rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/prof_calib_write -o run -- "
                        "python -u bench.py --calib-copy",
}


# Per-workload runs: the bench line (per-call HIP-event times) and a kernel trace.
CONFIG_NAMES = ("llama3_8b", "llama3_8b_n1", "batched", "llama3_70b", "forest", "tree_4096")
CONFIG_CMDS = {
    "bench": "python -u bench.py --config {name} --steps 30 --warmup 5 --no-cpu-baseline "
             "> gpurun_out/cfg_{name}.json",
    "trace": "rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/cfg_trace_{name} -o run -- "
             "python -u bench.py --config {name} --steps 10 --warmup 2 --no-cpu-baseline "
             "--no-extra-calls --no-m3",
}


def summarize_m3(root):
    """profiles/tree_attn_forward_m3.md: the 8B layer's forward with 64 nodes
    against one node, from the two workloads' bench lines and kernel traces."""
    rows = []
    for name in ("llama3_8b", "llama3_8b_n1"):
        try:
            with open(os.path.join(root, f"cfg_{name}.json")) as f:
                line = json.loads(f.read().strip().splitlines()[-1])
        except (OSError, ValueError, IndexError):
            return
        stats = _read_csvs(os.path.join(root, f"cfg_trace_{name}"), "kernel_stats.csv")
        ks = [(_short(x["Name"]), float(x["AverageNs"]) / 1e3) for x in stats
              if "fwd_bf16_kernel" in x["Name"] or "merge_bf16_kernel" in x["Name"]
              or "build_mask_kernel" in x["Name"]]
        rows.append((name, line, ks))
    (_, l64, k64), (_, l1, k1) = rows
    m3 = l64["detail"].get("M3") or {}
    t64, t1 = l64["ms_per_step"] * 1e3, l1["ms_per_step"] * 1e3
    md = ["# One candidate against 64 at the same prefix (Llama-3-8B layer, L=4096)", "",
          "Commands (repository root, MI355X box), for llama3_8b and llama3_8b_n1:", "",
          "    " + CONFIG_CMDS["bench"], "    " + CONFIG_CMDS["trace"], "",
          "The forward call (tree_attn_mask_and_forward) of the 8B-shaped layer with its 64-node",
          "draft tree, and with a one-node tree over the same prefix length, each timed over 30",
          "calls on cold rotated inputs (HIP events; graph replays). The pages hold that checking",
          "many candidates costs about what checking one does, both reading the same prefix K/V.",
          "", "| tree | us per call (events) | kernels (trace avg us) |", "|---|---|---|",
          f"| 64 nodes | {t64:.3f} | " + ", ".join(f"`{k}` {v:.3f}" for k, v in k64) + " |",
          f"| 1 node | {t1:.3f} | " + ", ".join(f"`{k}` {v:.3f}" for k, v in k1) + " |", "",
          f"Ratio 64 / 1 across the two runs: **{t64 / t1:.3f}**."]
    if m3:
        md.append(f"Ratio measured inside the 64-node run (`detail.M3`, same process): "
                  f"{m3['t_N_us']:.3f} / {m3['t_N1_us']:.3f} us = **{m3['ratio']:.3f}**.")
    with open(os.path.join(PROFILES, "tree_attn_forward_m3.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md))


def summarize_configs(root):
    """One table over the workloads: the forward call's device time (HIP events over
    the timed calls, p50 over per-round graph replays, and the kernel-trace average of
    its kernels), its algorithmic rate against the roof that bounds it, and the
    verifier's time; then the one-node comparison (summarize_m3)."""
    rows = []
    for name in CONFIG_NAMES:
        try:
            with open(os.path.join(root, f"cfg_{name}.json")) as f:
                line = json.loads(f.read().strip().splitlines()[-1])
        except (OSError, ValueError, IndexError):
            continue
        d = line["detail"]
        r = line["roofline"]
        fwd_call = r["kernel"]
        fw = d["forward"]
        stats = _read_csvs(os.path.join(root, f"cfg_trace_{name}"), "kernel_stats.csv")
        fwd_ns = sum(float(x["AverageNs"]) for x in stats
                     if "fwd_bf16_kernel" in x["Name"] or "merge_bf16_kernel" in x["Name"]
                     or "build_mask_kernel" in x["Name"])
        rows.append(f"| {name} | {line['config']['workload'].split(';')[0]} | "
                    f"{line['ms_per_step'] * 1e3:.1f} | "
                    f"{d['us_per_call_spread'][fwd_call]['p50']:.1f} | {fwd_ns / 1e3:.1f} | "
                    f"{r['achieved']} {r['unit']} | {r['bound']} | {r['frac']:.3f} | "
                    f"{fw['t_roof_us']:.1f} | {d['us_per_call']['tree_verify_greedy']:.1f} |")
    md = ["# Forward call on every workload (MI355X, one GPU)", "",
          "Commands (repository root, MI355X box), for each workload name:", "",
          "    " + CONFIG_CMDS["bench"], "    " + CONFIG_CMDS["trace"], "",
          "Times in microseconds per call. `events`: the bench line's headline timing (HIP",
          "events around the 30 timed calls on cold rotated inputs, graph replays); `p50`: median",
          "per-call time over replays of one graph round; `trace`: kernel-trace average of the",
          "forward's kernels (split kernel + merge kernel where there is one, mask kernel above",
          "128 nodes). The rate and fraction are the algorithmic bytes or flops per call over",
          "the events time, against 8 TB/s HBM or 2.5 PFLOP/s dense bf16 MFMA, whichever bounds",
          "the workload; `roof` is that bound's time.", "",
          "| workload | shape | events | p50 | trace | achieved | bound | roofline frac | roof | verify |",
          "|---|---|---|---|---|---|---|---|---|---|"] + rows
    with open(os.path.join(PROFILES, "tree_attn_forward_configs.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md))
    summarize_m3(root)


MFMA_CMD = ("rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16 -f csv -d gpurun_out/mfma_{name} "
            "-o run -- python -u bench.py --config {name} --steps 10 --warmup 2 --no-cpu-baseline "
            "--no-extra-calls --no-m3")


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


def rotation_sets(steps, need, set_bytes):
    """Copies of the inputs to rotate over: the smallest divisor of `steps` that
    is at least `need` (all of them when steps < need), so that `steps` calls
    are a whole number of rounds over the copies."""
    if steps <= need:
        return max(1, steps)
    d = next(d for d in range(need, steps + 1) if steps % d == 0)
    if d * set_bytes > 32 * 2**30:
        raise SystemExit(f"--steps {steps} needs {d} input copies to be whole rotation rounds "
                         f"({d * set_bytes / 2**30:.1f} GiB); pick a --steps with a divisor "
                         f"near {need}")
    return d


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
    if args.compute_ceiling:
        compute_ceiling()
        return
    if args.summarize_compute:
        summarize_compute(args.summarize_compute)
        return
    if args.timeline:
        timeline(args.timeline)
        return
    if args.summarize_timeline:
        summarize_timeline(args.summarize_timeline)
        return
    if args.summarize_ceiling:
        summarize_ceiling(args.summarize_ceiling, os.path.join(
            os.path.dirname(os.path.abspath(args.summarize_ceiling)), "prof_ceiling"))
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
    # Enough distinct copies to cycle through 2x the 256 MB Infinity Cache, their
    # count a divisor of --steps so that the timed region is whole rounds.
    set_bytes = sum(v.numel() * v.element_size() for v in base.values())
    n_sets = rotation_sets(args.steps, min(args.sets, -(-2 * 256 * 2**20 // set_bytes)), set_bytes)
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
        # the steps of all rotation sets in order.
        round_graph = capture(one_step, range(n_rot))
        # The graph must reproduce the eager step bit for bit, replayed twice with eager
        # work on other inputs in between.
        step(n_rot - 1)
        torch.cuda.synchronize()
        ref = outputs()
        for rep in range(2):
            step(n_rot)
            torch.cuda.synchronize()
            round_graph.replay()
            torch.cuda.synchronize()
            for a, b in zip(outputs(), ref):
                if not torch.equal(a, b):
                    raise SystemExit(f"graph replay {rep} differs from the eager step")

    stream = torch.cuda.current_stream(dev)

    def timed_steps(fn_round):
        """Device time (HIP events on the launch stream) and host time of exactly
        args.steps calls: args.steps / n_rot rounds over the input copies."""
        rounds = args.steps // n_rot
        fn_round()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(rounds):
            fn_round()
        e1.record(stream)
        torch.cuda.synchronize()
        host = time.perf_counter() - t0
        return e0.elapsed_time(e1) * 1e-3, host

    # --- headline: exactly --steps forward calls ------------------------------------------
    if use_graphs:
        fwd_round_graph = capture(fwd_fn, range(n_rot))
        fwd_round = fwd_round_graph.replay
        # The forward graph must give the eager call's bits as well.
        fwd_fn(sets[n_rot - 1])
        torch.cuda.synchronize()
        ref = outputs()
        fwd_fn(sets[0])
        fwd_round()
        torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(outputs()[:4], ref[:4])):
            raise SystemExit("the forward graph's replay differs from the eager call")
    else:
        def fwd_round():
            for i in range(n_rot):
                fwd_fn(sets[i])
    fwd_dev, fwd_host = timed_steps(fwd_round)
    t_fwd = fwd_dev * 1e6 / args.steps
    value = sum_n * args.steps / fwd_dev
    print(f"[bench] {args.steps} forward calls: {fwd_dev * 1e3:.4f} ms device, "
          f"{fwd_host * 1e3:.4f} ms host ({'graphs' if use_graphs else 'eager'})",
          file=sys.stderr, flush=True)

    # --- the whole step over as many steps --------------------------------------------------
    if use_graphs:
        step_round = round_graph.replay
    else:
        def step_round():
            for i in range(n_rot):
                one_step(sets[i])
    step_dev, step_host = timed_steps(step_round)
    ms_step = step_dev * 1e3 / args.steps
    print(f"[bench] {args.steps} whole steps: {step_dev * 1e3:.4f} ms device, "
          f"{step_host * 1e3:.4f} ms host", file=sys.stderr, flush=True)

    # --- per-call device time with HIP events on the launch stream ------------------------
    # One graph holds one call per rotation set; events bracket whole replays.

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

    # Stochastic verification (rejection sampling down the tree) on the same trees and
    # vocabulary: synthetic target logits and draft distributions close to them, each
    # node's token drawn from its parent's draft row, fixed uniforms.  Set up only where
    # the fp32 draft rows stay small (sum_N * V <= 2^26).
    samp = None
    if not args.no_extra_calls and sum_n * V <= (1 << 26):
        trees = [case.parents[int(case.node_offsets[b]):int(case.node_offsets[b + 1])].tolist()
                 for b in range(B)]
        sc = synthetic.make_sampling_case(trees, V, dtype=base["logits"].dtype, seed=7,
                                          temperature=1.0, noise=0.5, max_nodes=max_nodes)
        sd = {k: (v.to(dev) if isinstance(v, torch.Tensor) else torch.from_numpy(v).to(dev))
              for k, v in (("lg", sc.logits), ("rl", sc.root_logits), ("q", sc.draft_probs),
                           ("rq", sc.root_draft_probs), ("d", sc.draft), ("p", sc.parents),
                           ("o", sc.node_offsets), ("ua", sc.u_accept), ("uf", sc.u_final))}
        sws = torch.empty(max(ta.verify_sample_workspace_size(B, sum_n, V), 16), dtype=torch.uint8,
                          device=dev)
        so = [torch.empty(B, dtype=torch.int32, device=dev),
              torch.empty((B, max_nodes), dtype=torch.int32, device=dev),
              torch.empty((B, max_nodes), dtype=torch.int32, device=dev),
              torch.empty(B, dtype=torch.int32, device=dev)]

        def do_sample(s):
            ta.verify_sample(sd["lg"], sd["rl"], sd["q"], sd["rq"], sd["d"], sd["p"], sd["o"],
                             max_nodes, sc.temperature, sd["ua"], sd["uf"], workspace=sws,
                             accept_len=so[0], accept_nodes=so[1], accept_tokens=so[2],
                             bonus_token=so[3])
        samp = do_sample

    do_mask(sets[0])
    t_mask, d_mask = event_time(do_mask, args.steps)
    t_fwd_ev, d_fwd = event_time(fwd_fn, args.steps)
    t_ver, d_ver = event_time(do_verify, args.steps)
    t_commit = t_vnext = d_commit = d_vnext = None
    if not args.no_extra_calls:
        t_commit, d_commit = event_time(do_commit, args.steps)
        t_vnext, d_vnext = event_time(do_verify_next, args.steps)
    t_samp = d_samp = None
    if samp is not None:
        t_samp, d_samp = event_time(samp, args.steps)
        samp_len = so[0].float().mean().item()
    if t_commit is not None and not bool((commit_status == 0).all()):
        raise SystemExit("tree_kv_commit reported a failure in the timing loop")
    print(f"[bench] per call us: mask {t_mask:.2f} forward {t_fwd:.2f} ({t_fwd_ev:.2f} in the "
          f"per-call graphs) verify {t_ver:.2f}", file=sys.stderr, flush=True)

    # --- one candidate against N at the same prefix (the N=1 variant) ---------------------
    m3 = None
    if not args.no_m3 and max_nodes > 1:
        m3 = one_node_ratio(case, ta, dev, args.steps, t_fwd, args.separate_mask)

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
            r["traffic"] = load_traffic(args.config, fwd_call, fwd_hash)
            r["kernel"] = fwd_call
            return r
        r = {"bound": "hbm", "achieved": round(ver_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(ver_gbs / HBM_PEAK_GBS, 4),
             "traffic": load_traffic(args.config, "tree_verify_greedy", ver_hash),
             "kernel": "tree_verify_greedy"}
        return r


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
        "ms_per_step": round(t_fwd * 1e-3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.config}: B={B} Hq={Hq} Hkv={Hkv} D={D} L={max_prefix} N={max_nodes} "
                        f"(sum_L={sum_l}, sum_N={sum_n}); greedy verify over V={V} bf16 logits",
            "timed": f"{args.steps} {fwd_call} calls ({args.steps // n_rot} rounds over "
                     f"{n_rot} resident input copies of {set_bytes / 2**20:.1f} MiB), "
                     + ("replayed from a captured HIP graph per round" if use_graphs
                        else "launched eagerly from Python")
                     + "; HIP events on the launch stream",
            "global_batch": B, "seq_len": max_prefix, "tree_nodes": sum_n,
        },
        "roofline": roof("forward"),
        "cpu_baseline": cpu,
        "detail": {
            "step": {"calls": " + ".join(n for n, _ in calls), "steps": args.steps,
                     "ms_per_step": round(ms_step, 6),
                     "tree_tokens_per_s": round(sum_n * args.steps / step_dev, 1),
                     "host_ms_per_step": round(step_host * 1e3 / args.steps, 6)},
            "forward_host_ms_per_call": round(fwd_host * 1e3 / args.steps, 6),
            "M3": m3,
            "us_per_call": {fwd_call: round(t_fwd_ev, 3), "tree_verify_greedy": round(t_ver, 3),
                            "tree_attn_build_mask (standalone)": round(t_mask, 3),
                            "tree_kv_commit (standalone)": t_commit and round(t_commit, 3),
                            "tree_verify_greedy_next (standalone)": t_vnext and round(t_vnext, 3),
                            "tree_verify_sample (standalone)": t_samp and round(t_samp, 3)},
            "us_per_call_spread": {fwd_call: d_fwd, "tree_verify_greedy": d_ver,
                                   "tree_attn_build_mask (standalone)": d_mask,
                                   "tree_kv_commit (standalone)": d_commit,
                                   "tree_verify_greedy_next (standalone)": d_vnext,
                                   "tree_verify_sample (standalone)": d_samp},
            "sample": t_samp and {"accept_len_mean": round(samp_len, 3),
                                  "inputs": "target logits 2*randn, draft = softmax(logits + "
                                            "0.5*randn), T=1, tokens drawn from the draft"},
            "commit": {"accepted_rows": int(acc_len.sum()),
                       "alg_bytes": int(acc_len.sum()) * Hkv * D * base["kt"].element_size() * 4},
            "forward": {"tree_tokens_per_s": round(value, 1),
                        "kv_GBps": round(kv_bytes / (t_fwd * 1e-6) / 1e9, 1),
                        "alg_GBps": round(fwd_gbs, 1), "alg_TFLOPs": round(fwd_tfs, 2),
                        "alg_bytes": fwd_bytes, "alg_flops": fwd_flops,
                        "t_roof_us": round(t_roof_fwd * 1e6, 3),
                        "roofline_frac": round(t_roof_fwd / (t_fwd * 1e-6), 4)},
            "verify": {"alg_bytes": ver_bytes, "alg_GBps": round(ver_gbs, 1),
                       "roofline": roof("verify")},
            "source_hash": {"attn_fwd.hip": fwd_hash, "verify.hip": ver_hash},
        },
    }
    print(json.dumps(line), flush=True)


def one_node_ratio(case, ta, dev, steps, t_fwd_us, separate_mask):
    """The forward of the same workload with every sequence's tree cut to its
    first root (same prefix lengths, fresh inputs): device time per call over
    exactly `steps` calls, rotated over cold copies and replayed from a graph,
    and the ratio of the N-node call to it ("Speculative Tree Attention: How
    Multi-Candidate Draft Models and Parallel Verification Deliver 4x LLM
    Speedups", news.premlal.in, The Speculative Paradigm: checking many
    candidates at once costs about what checking one does, both being bound by
    reading the prefix's K/V)."""
    import numpy as np
    import torch

    import synthetic
    lens = [int(x) for x in np.diff(case.prefix_offsets)]
    c1 = synthetic.make_case(case.name + "_n1", prefix_lens=lens, trees=[[-1]] * case.B,
                             Hq=case.Hq, Hkv=case.Hkv, D=case.D, dtype=case.dtype,
                             seed=case.seed + 1000)
    base = {"parents": torch.from_numpy(c1.parents).to(dev),
            "noffs": torch.from_numpy(c1.node_offsets).to(dev),
            "poffs": torch.from_numpy(c1.prefix_offsets).to(dev),
            "q": c1.q.to(dev), "kt": c1.k_tree.to(dev), "vt": c1.v_tree.to(dev),
            "kp": c1.k_prefix.to(dev), "vp": c1.v_prefix.to(dev)}
    set_bytes = sum(v.numel() * v.element_size() for v in base.values())
    n = rotation_sets(steps, -(-2 * 256 * 2**20 // set_bytes), set_bytes)
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(n - 1)]
    B, max_prefix = c1.B, c1.max_prefix
    mask = torch.empty((c1.total_nodes, 1), dtype=torch.uint64, device=dev)
    depth = torch.empty(c1.total_nodes, dtype=torch.int32, device=dev)
    status = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty_like(base["q"])
    ws = torch.zeros(max(ta.forward_workspace_size(c1.dtype, B, c1.total_nodes, 1, c1.Hq, c1.Hkv,
                                                   c1.D, c1.total_prefix, max_prefix), 16),
                     dtype=torch.uint8, device=dev)

    def call(s):
        if separate_mask:
            ta.forward(s["q"], s["kt"], s["vt"], s["kp"], s["vp"], s["poffs"], s["noffs"], mask, 1,
                       max_prefix, c1.scale, out=out, workspace=ws)
        else:
            ta.mask_and_forward(s["parents"], s["q"], s["kt"], s["vt"], s["kp"], s["vp"],
                                s["poffs"], s["noffs"], 1, max_prefix, c1.scale, out=out,
                                mask=mask, depth=depth, status=status, workspace=ws)

    ta.build_mask(base["parents"], base["noffs"], 1, mask=mask, depth=depth, status=status)
    for s in sets:
        call(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in sets:
            call(s)
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps // n):
        g.replay()
    e1.record(stream)
    e1.synchronize()
    t1 = e0.elapsed_time(e1) * 1e3 / steps
    return {"what": f"forward with {case.max_nodes}-node trees over the time with one-node trees, "
                    "same prefixes", "t_N_us": round(t_fwd_us, 3), "t_N1_us": round(t1, 3),
            "N": case.max_nodes, "ratio": round(t_fwd_us / t1, 4)}


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
