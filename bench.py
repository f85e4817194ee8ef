"""Benchmark: one rank's share of tensor-parallel DiT linear layers, every rank in turn, on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:

  full block (hidden 6144, 48 heads x 128, FFN 18432, 4608 tokens), for each
  tp degree P in {2, 4, 8}:
    * shard every weight for every rank: head-aligned fused-QKV split,
      out-proj rowwise, FFN-up colwise, FFN-down rowwise (index kernels);
    * every rank: colwise QKV, rowwise out-proj (fp32 partial), colwise
      FFN-up + GELU-tanh, rowwise FFN-down (fp32 partial);
    * layer-boundary combines: SUM of the out-proj partials (fp32) and of the
      FFN-down partials (bf16 out), CONCAT of the QKV outputs (packed [1,1,1])
      and of the FFN-up outputs;
  FLUX.2-style fused FFN gate/up projection (6144 -> 2 x 18432, packed with
  blocks [1, 1], P=4): packed slices for the 4 ranks, then each rank's GEMM
  with the fused SwiGLU epilogue (bf16 [4608, 4608] out);
  adaLN modulation (6144 -> 36864, P=4, 4 conditioning rows), twice:
    * colwise: shard the weight for the 4 ranks, then each rank's skinny
      weight-streaming GEMV;
    * rowwise_split_input: shard the weight's input features for the 4 ranks,
      each rank's skinny GEMV on its slice of the replicated input (fp32
      partial), then the SUM of the 4 partials with the bias (bf16 out).

Inputs are seeded synthetic bf16 tensors already resident in HBM when the timed
region starts.  `value` is the step's sharded-linear TFLOP/s (all GEMM and GEMV
flops / wall time per step).  Per-kernel durations come from HIP events around
every launch of the timed steps, on the stream the library launches on.
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

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic.json")
GEMM_SRC = os.path.join(ROOT, "tensor_sharded_linear_amd", "csrc", "gemm_bf16.hip")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--tp", type=str, default="2,4,8", help="tp degrees of the full block")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--detail", action="store_true", help="time every launch with its own event pair (adds the events' overhead to the step) "
                         "and print a per-shape table to stderr")
    ap.add_argument("--streams", type=int, default=1, choices=(1, 2),
                    help="2: slicing and combines on a second stream beside the GEMMs (measured slower)")
    ap.add_argument("--probe", metavar="OUT_JSON",
                    help="untimed: two steps, then a calibration copy of known size, for rocprofv3 --pmc runs; "
                         "writes the second step's launch list (family, shape, flops, algorithmic bytes) to "
                         "OUT_JSON")
    ap.add_argument("--cold-md", metavar="OUT_MD",
                    help="also write the cold per-call table of the HBM-bound calls to OUT_MD")
    ap.add_argument("--counters", nargs="+", metavar="PATH",
                    help="no GPU: PROBE_JSON RUN_DIR [RUN_DIR ...]: join rocprofv3 --pmc runs of --probe with its "
                         "launch list; writes profiles/dit_block_step_counters.md and, from FETCH_SIZE and "
                         "WRITE_SIZE runs, " + os.path.relpath(TRAFFIC_FILE, ROOT))
    ap.add_argument("--load", action="store_true",
                    help="checkpoint-load benchmark instead of the step: the full block's weights in a synthetic "
                         "safetensors file, every rank of --load-tp loaded by tp_load_shard (shard as read) and "
                         "by reading whole tensors then slicing on the device; time and peak host memory")
    ap.add_argument("--load-tp", type=int, default=4)
    ap.add_argument("--load-dir", default=None, help="directory for the synthetic checkpoint (default: a temp dir)")
    ap.add_argument("--load-child", nargs=4, metavar=("METHOD", "TP", "PATH", "OUT_JSON"), help=argparse.SUPPRESS)
    ap.add_argument("--configs", metavar="OUT_MD",
                    help="per-call table instead of the step: every call of the tiny MLP (tp 2), the attention "
                         "projections (hidden 3072, tp 4), the large MLP (tp 4) and the adaLN GEMV (tp 4, 1-4 "
                         "rows) for rank 0, cold (a 512 MiB read before each call) and warm, median of --steps "
                         "calls, each against its roofline; the oracle timed beside each workload; writes a "
                         "markdown table to OUT_MD and one JSON line to stdout")
    ap.add_argument("--cold-trace", nargs=2, metavar=("TRACE_CSV", "COLD_MD"),
                    help="no GPU: from the rocprofv3 kernel trace of a --cold-md run and the table that run "
                         "wrote, print the table with each call's kernel duration from the trace (median of "
                         "its cold dispatches) beside the event-timed one")
    ap.add_argument("--vendor", metavar="OUT_MD",
                    help="instead of the step: every GEMM shape of the step through this library and through "
                         "torch.matmul / torch.mm (hipBLASLt), plain products without epilogue, back to back on "
                         "three rotating operand sets; writes a markdown table to OUT_MD")
    ap.add_argument("--vendor-square", metavar="OUT_MD",
                    help="instead of the step: large products whose 256 x 256 tiles fill the CUs in whole "
                         "rounds (8192 and 16384 rows and columns) through this library and through "
                         "torch.matmul (hipBLASLt), measured like --vendor; writes a markdown table to OUT_MD")
    ap.add_argument("--configs-trace", metavar="TRACE_CSV",
                    help="no GPU: from the rocprofv3 kernel trace of a --configs run, print per-kernel medians "
                         "of the dispatches right after the cache-flush read (cold) and of the others (warm)")
    ap.add_argument("--pmc-summary", nargs="+", metavar="RUN_DIR",
                    help="no GPU: average every counter of rocprofv3 --pmc runs per kernel of this library "
                         "and per hipBLASLt GEMM kernel (name and grid) and print a markdown table")
    return ap.parse_args()


# ---------------------------------------------------------------------------------------------
# checkpoint-load benchmark ("Load a sharded model" / "Loading performance" of the TP page)
# ---------------------------------------------------------------------------------------------

# The full block's weights and the plan each is loaded with: (name, style, blocks).
LOAD_PLAN = [("attn.to_qkv.weight", "colwise", [1, 1, 1]), ("attn.to_out.weight", "rowwise", None),
             ("ff.w1.weight", "colwise", None), ("ff.w2.weight", "rowwise", None)]
LOAD_SRC = {"attn.to_qkv.weight": "w_qkv", "attn.to_out.weight": "w_o", "ff.w1.weight": "w1", "ff.w2.weight": "w2"}


def _evict(path):
    """Drop the file's clean pages from the page cache (posix_fadvise, no privileges
    needed), so the next read comes from the storage device."""
    fd = os.open(path, os.O_RDONLY)
    try:
        os.fsync(fd)
        os.posix_fadvise(fd, 0, 0, os.POSIX_FADV_DONTNEED)
    finally:
        os.close(fd)


def _fs_type(path):
    best, fs = "", "?"
    with open("/proc/mounts") as f:
        for line in f:
            parts = line.split()
            if len(parts) >= 3 and os.path.realpath(path).startswith(parts[1]) and len(parts[1]) > len(best):
                best, fs = parts[1], parts[2]
    return fs


def _rss_now_bytes():
    with open("/proc/self/statm") as f:
        return int(f.read().split()[1]) * os.sysconf("SC_PAGE_SIZE")


class _RssPeak:
    """Highest resident set size seen while active (sampled every millisecond)."""

    def __init__(self):
        import threading
        self.peak = _rss_now_bytes()
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self._stop.is_set():
            self.peak = max(self.peak, _rss_now_bytes())
            self._stop.wait(0.001)

    def __enter__(self):
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join()
        self.peak = max(self.peak, _rss_now_bytes())


def load_child(method, tp, path, out_json):
    """One process per method: every rank in turn, the file's pages evicted before each.
    Host memory is the peak resident set during a rank's load above the process's resident
    set before its first load (so the pinned staging buffers count, even where the runtime
    keeps them between calls)."""
    import torch
    import tensor_sharded_linear_amd as tsl
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    torch.empty(1, device=dev)
    torch.cuda.synchronize()
    ranks = []
    peak_above = 0
    base_rss = _rss_now_bytes()   # host memory in use before any load (torch and the HIP runtime)
    for i, r in enumerate([0] + list(range(tp))):
        warm = i == 0   # an untimed first pass (rank 0) warms up the HIP runtime
        _evict(path)
        mon = _RssPeak().__enter__()
        t0 = time.perf_counter()
        shard_bytes = 0
        held = []
        per = {}
        if method == "shard":
            for name, style, blocks in LOAD_PLAN:
                t1 = time.perf_counter()
                t = tsl.tp_load_shard(path, name, style, tp, r, blocks=blocks)
                per[name] = round(time.perf_counter() - t1, 4)
                shard_bytes += t.numel() * t.element_size()
                held.append(t)
        else:
            from safetensors.torch import load_file
            full = load_file(path)            # the whole checkpoint in host memory
            for name, style, blocks in LOAD_PLAN:
                w = full[name].to(dev)
                ws, _ = tsl.tp_plan_shard_slice(w, None, style, tp, r, blocks=blocks)
                shard_bytes += ws.numel() * ws.element_size()
                held.append(ws)
                del w
            del full
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        mon.__exit__()
        if warm:
            del held
            continue
        ranks.append(dict(rank=r, seconds=round(dt, 4), shard_bytes=shard_bytes,
                          gbs=round(shard_bytes / dt / 1e9, 3), peak_host_bytes=mon.peak - base_rss))
        if per:
            ranks[-1]["seconds_per_tensor"] = per
        peak_above = max(peak_above, mon.peak - base_rss)
        del held
        torch.cuda.empty_cache()
    with open(out_json, "w") as f:
        json.dump(dict(method=method, ranks=ranks, peak_host_bytes_above_start=peak_above), f)


def load_bench(args):
    """Parent process: writes the checkpoint (CPU only, never touches the GPU), then runs one
    child process per method and prints one JSON line."""
    import subprocess
    import tempfile

    import numpy as np
    import torch
    from safetensors.torch import save_file

    import synth_inputs as si

    d = args.load_dir or tempfile.mkdtemp(prefix="tp_load_", dir="/tmp")
    path = os.path.join(d, "dit_block_h6144.safetensors")
    t0 = time.perf_counter()
    fb = si.workload("full_block").arrays
    tensors = {n: torch.from_numpy(fb[src].view(np.int16)).view(torch.bfloat16) for n, src in LOAD_SRC.items()}
    save_file(tensors, path)
    file_bytes = os.path.getsize(path)
    del tensors, fb
    print(f"# checkpoint {path}: {file_bytes / 1e6:.1f} MB written in {time.perf_counter() - t0:.1f}s "
          f"({_fs_type(path)})", file=sys.stderr, flush=True)
    def seq_read_gbs():
        t = time.perf_counter()
        with open(path, "rb", buffering=0) as f:
            while f.read(32 << 20):
                pass
        return round(file_bytes / (time.perf_counter() - t) / 1e9, 2)
    _evict(path)
    cold = seq_read_gbs()
    warm = seq_read_gbs()
    print(f"# sequential read of the file: {cold} GB/s after eviction, {warm} GB/s again", file=sys.stderr,
          flush=True)
    res = {}
    for method in ("shard", "full"):
        out = os.path.join(d, f"{method}.json")
        cmd = [sys.executable, os.path.abspath(__file__), "--load-child", method, str(args.load_tp), path, out]
        subprocess.run(cmd, check=True)
        with open(out) as f:
            res[method] = json.load(f)
        print(f"# {method}: {res[method]}", file=sys.stderr, flush=True)
    if not args.load_dir:
        os.remove(path)
    tp = args.load_tp

    def summary(m):
        rs = res[m]["ranks"]
        return dict(seconds_per_rank_max=max(r["seconds"] for r in rs),
                    seconds_per_rank_mean=round(sum(r["seconds"] for r in rs) / len(rs), 4),
                    shard_gbs_mean=round(sum(r["gbs"] for r in rs) / len(rs), 3),
                    peak_host_bytes=res[m]["peak_host_bytes_above_start"], ranks=rs)
    print(json.dumps({
        "metric": "sharded checkpoint load time per rank (s)", "value": summary("shard")["seconds_per_rank_max"],
        "unit": "s", "higher_is_better": False, "n_gpus": 1, "data": "synthetic",
        "config": {"workload": f"DiT block weights (hidden 6144, FFN 18432; W_qkv, W_o, W1, W2 bf16) in one "
                               f"safetensors file, every rank of tp {tp} loaded in turn on one GPU",
                   "file_bytes": file_bytes, "tp_degree": tp, "filesystem": _fs_type(path),
                   "page_cache": "file pages dropped with posix_fadvise(DONTNEED) before each rank",
                   "sequential_read_gbs": {"after_eviction": cold, "cached": warm}},
        "shard_as_read": summary("shard"), "full_then_slice": summary("full"),
    }), flush=True)


CAL_ROWS, CAL_COLS = 8192, 8192   # calibration copy: a 128 MiB bf16 weight, copied whole (colwise, P = 1)


ATTR_LDS = "SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE"
ATTR_WAIT = ("SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU "
             "SQ_ACTIVE_INST_LDS GRBM_GUI_ACTIVE TA_TA_BUSY TD_TD_BUSY")
# issue back-pressure: loads refused by full TA FIFOs, LDS FIFOs full, LDS issue waits, and the
# cycles spent sending load addresses
ATTR_ISSUE = ("SQ_VMEM_TA_ADDR_FIFO_FULL SQ_VMEM_TA_CMD_FIFO_FULL SQ_LDS_CMD_FIFO_FULL "
              "SQ_LDS_DATA_FIFO_FULL SQ_WAIT_INST_LDS SQ_INST_CYCLES_VMEM_RD GRBM_GUI_ACTIVE")
# "bf16_nt_kernel" matches both tiled GEMM kernels: gemm4_bf16_nt_kernel (four waves, 192- to
# 256-row tiles: every GEMM of the step) and gemm_bf16_nt_kernel (eight waves, 64 and 128 rows).
KERNEL_OF = {"gemm": "bf16_nt_kernel", "gemv": "gemv_bf16_kernel", "sum": "combine_sum_kernel",
             "slice": "copy_segments_kernel", "concat": "copy_segments_kernel"}
N_XCC = 8          # GRBM_GUI_ACTIVE is counted per XCD; the CSV value is their sum
SIMDS = 1024       # 256 CUs x 4 SIMDs


def _dispatches(d):
    """{dispatch id: [kernel name, {counter: value}, duration ns or None]} of one rocprofv3 run
    directory (--pmc CSV output, with or without a kernel trace)."""
    import csv
    import glob
    out = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                e = out.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], {}, None])
                name = r["Counter_Name"]
                e[1][name] = e[1].get(name, 0.0) + float(r["Counter_Value"])
                if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                    e[2] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    for path in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                k = int(r["Dispatch_Id"])
                if k in out:
                    out[k][2] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    if not out:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return out


def reduce_counters(probe_json, dirs):
    """Joins rocprofv3 --pmc runs of `bench.py --probe` with the probe's launch list.

    Each run's last len(launches) + 1 dispatches of this library's kernels are the probe's
    second step and the calibration copy (a copy of known size: CAL bytes read and the same
    written).  FETCH_SIZE and WRITE_SIZE are scaled by what they read for that copy; MfmaUtil
    (rocprofv3's derived metric: MFMA-busy cycles over GUI-active cycles x SIMDs), MfmaFlopsBF16
    and GRBM_GUI_ACTIVE are taken as they are.  Writes profiles/gemm_traffic.json (the GEMM
    family's HBM bytes per launch, read by the bench line) when both byte counters are there, and
    profiles/dit_block_step_counters.md with the per-family and per-GEMM-shape tables."""
    with open(probe_json) as f:
        probe = json.load(f)
    launches = probe["launches"]
    n = len(launches)
    per = [dict() for _ in range(n)]       # counter -> value, per launch
    dur = [[] for _ in range(n)]           # durations (ns) seen for the launch across runs
    scale = {}
    runs = []
    for d in dirs:
        disp = _dispatches(d)
        ours = [(k, v) for k, v in sorted(disp.items()) if any(kn in v[0] for kn in set(KERNEL_OF.values()))]
        if len(ours) < n + 1:
            raise SystemExit(f"{d}: {len(ours)} library dispatches, fewer than the probe's {n} + 1")
        step, cal = ours[-(n + 1):-1], ours[-1][1]
        if "copy_segments_kernel" not in cal[0]:
            raise SystemExit(f"{d}: the last dispatch is {cal[0]}, not the calibration copy")
        for i, ((_, (name, cnt, ns)), (cat, key, _, _)) in enumerate(zip(step, launches)):
            if KERNEL_OF[cat] not in name:
                raise SystemExit(f"{d}: dispatch {i} is {name}, the probe says {cat} {key}")
            for c, v in cnt.items():
                per[i][c] = v
            if ns:
                dur[i].append(ns)
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            if c in cal[1]:
                scale[c] = probe["cal_bytes"] / (cal[1][c] * 1024.0)
                scale[c + "_cal_kib"] = cal[1][c]
        runs.append(f"{os.path.basename(os.path.normpath(d))}: {', '.join(sorted(step[0][1][1]))}")

    def mean(xs):
        return sum(xs) / len(xs) if xs else float("nan")

    # per family: counter bytes against algorithmic bytes
    fam = {}
    for i, (cat, key, flops, nbytes) in enumerate(launches):
        e = fam.setdefault(cat, dict(n=0, alg=0.0, fetch=0.0, write=0.0))
        e["n"] += 1
        e["alg"] += nbytes
        e["fetch"] += per[i].get("FETCH_SIZE", float("nan")) * 1024.0 * scale.get("FETCH_SIZE", float("nan"))
        e["write"] += per[i].get("WRITE_SIZE", float("nan")) * 1024.0 * scale.get("WRITE_SIZE", float("nan"))
    # per shape: everything averaged over the shape's launches
    shp = {}
    for i, (cat, key, flops, nbytes) in enumerate(launches):
        e = shp.setdefault((cat, key), dict(n=0, flops=flops, alg=nbytes, rows=[]))
        e["n"] += 1
        e["rows"].append(i)
    md = ["# Hardware counters of one bench step, per kernel family and per GEMM shape", "",
          "Commands (run from the repository root on one MI355X; one counter set per run):", "", "```"]
    for c in ("FETCH_SIZE", "WRITE_SIZE", "MfmaUtil MfmaFlopsBF16 GRBM_GUI_ACTIVE", ATTR_LDS, ATTR_WAIT,
              ATTR_ISSUE):
        tag = c.split()[0].lower()
        md.append(f"rocprofv3 --pmc {c} --kernel-trace --output-format csv -d out/pmc_{tag} -o run -- "
                  f"python3 bench.py --probe out/probe_{tag}.json")
    md += ["python3 bench.py --counters out/probe_fetch_size.json out/pmc_fetch_size "
           "out/pmc_write_size out/pmc_mfmautil out/pmc_sq_lds_idx_active "
           "out/pmc_sq_wave_cycles out/pmc_sq_vmem_ta_addr_fifo_full", "```", "",
           f"`--probe` runs two bench steps untimed, then one copy of a {CAL_ROWS} x {CAL_COLS} bf16 weight "
           f"({probe['cal_bytes']} bytes read, the same written) whose counters calibrate the byte counts.  "
           f"The tables cover the {n} launches of the second step.  Under counter collection every dispatch "
           "runs alone, so durations here are longer than in the timed bench, and the caches hold what the "
           "step's previous kernel left, as in the bench.", "",
           "Runs: " + "; ".join(runs), ""]
    if "FETCH_SIZE" in scale and "WRITE_SIZE" in scale:
        md += [f"Calibration: FETCH_SIZE read {scale['FETCH_SIZE_cal_kib']:.0f} KiB and WRITE_SIZE "
               f"{scale['WRITE_SIZE_cal_kib']:.0f} KiB for {probe['cal_bytes'] / 1024:.0f} KiB moved each way: "
               f"factors {scale['FETCH_SIZE']:.4f} and {scale['WRITE_SIZE']:.4f}.", "",
               "## HBM traffic per family (counter bytes against algorithmic bytes)", "",
               "| family | launches | algorithmic MB / launch | fetched MB / launch | written MB / launch | "
               "traffic / algorithmic |", "|---|---|---|---|---|---|"]
        for cat, e in sorted(fam.items()):
            md.append(f"| {cat} | {e['n']} | {e['alg'] / e['n'] / 1e6:.1f} | {e['fetch'] / e['n'] / 1e6:.1f} | "
                      f"{e['write'] / e['n'] / 1e6:.1f} | {(e['fetch'] + e['write']) / e['alg']:.3f} |")
        md += ["", "Per shape:", "", "| family: shape | launches | algorithmic MB | fetched MB | written MB | ratio |",
               "|---|---|---|---|---|---|"]
        for (cat, key), e in sorted(shp.items()):
            fe = mean([per[i].get("FETCH_SIZE", float("nan")) for i in e["rows"]]) * 1024 * scale["FETCH_SIZE"]
            wr = mean([per[i].get("WRITE_SIZE", float("nan")) for i in e["rows"]]) * 1024 * scale["WRITE_SIZE"]
            md.append(f"| {cat}: {key} | {e['n']} | {e['alg'] / 1e6:.1f} | {fe / 1e6:.1f} | {wr / 1e6:.1f} | "
                      f"{(fe + wr) / e['alg']:.3f} |")
        g = fam["gemm"]
        out = {
            "kernel": "gemm4_bf16_nt_kernel", "source_sha": file_sha(GEMM_SRC),
            "bytes_per_launch": round((g["fetch"] + g["write"]) / g["n"]),
            "algorithmic_bytes_per_launch": round(g["alg"] / g["n"]),
            "ratio_to_algorithmic": round((g["fetch"] + g["write"]) / g["alg"], 4),
            "fetch_bytes_per_launch": round(g["fetch"] / g["n"]), "write_bytes_per_launch": round(g["write"] / g["n"]),
            "factors": {"FETCH_SIZE": scale["FETCH_SIZE"], "WRITE_SIZE": scale["WRITE_SIZE"]},
            "launches_averaged": g["n"],
        }
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(out, f, indent=1)
        print(json.dumps(out))
    if any("MfmaUtil" in p for p in per):
        md += ["", "## MFMA utilisation per GEMM shape", "",
               "MfmaUtil is rocprofv3's derived metric: MFMA-busy cycles summed over the SIMDs, over "
               "GUI-active cycles x 1024 SIMDs.  MFMA flops are MfmaFlopsBF16 (512 x the bf16 MFMA "
               "math-op count); against the algorithmic 2MNK they show the work of the tiles' padding rows.  "
               "The clock is GUI-active cycles (per XCD) over the dispatch's duration.", "",
               "| shape | launches | µs (alone) | TFLOP/s (alone) | MfmaUtil % | MFMA flops / 2MNK | clock GHz | "
               "MFMA flops per GUI cycle, % of 1024 x 1024 |", "|---|---|---|---|---|---|---|---|"]
        tot = dict(busy=0.0, n=0)
        for (cat, key), e in sorted(shp.items()):
            if cat != "gemm":
                continue
            util = mean([per[i].get("MfmaUtil", float("nan")) for i in e["rows"]])
            mf = mean([per[i].get("MfmaFlopsBF16", float("nan")) for i in e["rows"]])
            gui = mean([per[i].get("GRBM_GUI_ACTIVE", float("nan")) for i in e["rows"]]) / N_XCC
            us = mean([x for i in e["rows"] for x in dur[i]]) / 1e3
            md.append(f"| {key} | {e['n']} | {us:.1f} | {e['flops'] / us / 1e6:.0f} | {util:.1f} | "
                      f"{mf / e['flops']:.4f} | {gui / us / 1e3:.2f} | {100 * mf / gui / (SIMDS * 1024):.1f} |")
            tot["busy"] += util * e["n"]
            tot["n"] += e["n"]
        md += ["", f"Launch-weighted MfmaUtil over the step's {tot['n']} GEMM launches: "
                   f"{tot['busy'] / tot['n']:.1f}%."]
    # Attribution counters, where a run collected them: per CU cycle (LDS, TA, TD activity) or
    # per wave cycle (wait and issue states; SQ_WAVE_CYCLES counts in units of 4 cycles, like
    # the wait and active counters it divides).
    per_cu = ["SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "TA_TA_BUSY", "TD_TD_BUSY",
              "SQ_VMEM_TA_ADDR_FIFO_FULL", "SQ_VMEM_TA_CMD_FIFO_FULL", "SQ_LDS_CMD_FIFO_FULL",
              "SQ_LDS_DATA_FIFO_FULL"]
    per_wave = ["SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS", "SQ_INST_CYCLES_VMEM_RD"]
    have = [c for c in per_cu + per_wave if any(c in p for p in per)]
    if have:
        md += ["", "## Where the GEMM's cycles go (attribution counters)", "",
               "Per CU cycle: the counter summed over the chip / (GUI-active cycles per XCD x 256 CUs).  "
               "Per wave cycle: the counter / SQ_WAVE_CYCLES (both in units of 4 cycles).  A ratio's "
               "counter and divisor can come from different runs of the same step (GRBM_GUI_ACTIVE from "
               "the last run that has it).  FIFO_FULL: cycles a load was held back by a full TA "
               "address or command FIFO, or the LDS command or data FIFO was full; WAIT_INST_LDS: "
               "waiting to issue an LDS instruction; INST_CYCLES_VMEM_RD: cycles sending the "
               "addresses of loads.", "",
               "| family: shape | " + " | ".join(c.replace("SQ_", "") for c in have) + " |",
               "|---|" + "---|" * len(have)]
        for (cat, key), e in sorted(shp.items()):
            if cat != "gemm" and cat not in ("sum", "slice", "concat", "gemv"):
                continue
            rowsel = e["rows"]
            vals = []
            for c in have:
                num = sum(per[i].get(c, float("nan")) for i in rowsel)
                if c in per_cu:
                    den = sum(per[i].get("GRBM_GUI_ACTIVE", float("nan")) for i in rowsel) / N_XCC * 256
                else:
                    den = sum(per[i].get("SQ_WAVE_CYCLES", float("nan")) for i in rowsel)
                vals.append(f"{num / den:.3f}" if den == den and den > 0 else "-")
            md.append(f"| {cat}: {key} | " + " | ".join(vals) + " |")
    with open(os.path.join(ROOT, "profiles", "dit_block_step_counters.md"), "w") as f:
        f.write("\n".join(md) + "\n")


class TimingEvent:
    """A HIP event used only to time GPU work, created with hipEventDisableSystemFence.

    A default event record ends with a system-scope release: the L2 is written back and
    invalidated.  Between two kernels that costs about 5 us of idle GPU per record, and the next
    kernel restarts from cold caches.  Timing needs neither: the timestamps are read only after
    a device synchronize.  The event lives in the HIP runtime that torch loaded, so torch's
    stream handles are valid for it.
    """

    _hip = None
    FLAGS = 0x20000000  # hipEventDisableSystemFence

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes
            lib = ctypes.CDLL("libamdhip64.so.7")  # the copy torch already loaded (same soname)
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            for fn in (lib.hipEventCreateWithFlags, lib.hipEventRecord, lib.hipEventElapsedTime, lib.hipEventDestroy):
                fn.restype = ctypes.c_int
            cls._hip = lib
        return cls._hip

    def __init__(self):
        import ctypes
        self._ct = ctypes
        self.h = ctypes.c_void_p()
        self._check(self._lib().hipEventCreateWithFlags(ctypes.byref(self.h), self.FLAGS), "hipEventCreateWithFlags")

    @staticmethod
    def _check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def record(self, stream):
        self._check(self._lib().hipEventRecord(self.h, self._ct.c_void_p(stream.cuda_stream)), "hipEventRecord")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end`; call after a device synchronize."""
        ms = self._ct.c_float()
        self._check(self._lib().hipEventElapsedTime(self._ct.byref(ms), self.h, end.h), "hipEventElapsedTime")
        return ms.value

    def destroy(self):
        if self.h:
            self._check(self._lib().hipEventDestroy(self.h), "hipEventDestroy")
            self.h = self._ct.c_void_p()


class Timer:
    """HIP events over the timed launches, on the stream each launch runs on.

    By default consecutive launches of one kernel family on one stream share
    one event pair, so the events add no gaps between them; a family's
    average launch time is the summed group time over its launch count.  The
    event that closes one group opens the next one on the same stream.
    With per_launch=True every launch gets its own pair (per-shape detail).
    """

    def __init__(self, torch, per_launch=False):
        self.torch = torch
        self.on = False
        self.per_launch = per_launch
        self.rec = []    # (category, [(key, flops, bytes), ...], ev0, ev1)
        self.open = {}   # stream -> [category, items, ev0]

    def _close(self, s):
        """Ends the open group on stream s; returns the event that ended it (or None)."""
        g = self.open.pop(s, None)
        if g is None:
            return None
        e1 = TimingEvent()
        e1.record(s)
        self.rec.append((g[0], g[1], g[2], e1))
        return e1

    def run(self, cat, key, flops, nbytes, fn, stream=None):
        """Launch fn on `stream` (torch's current stream if None), timed by events on it."""
        s = stream if stream is not None else self.torch.cuda.current_stream()
        with self.torch.cuda.stream(s):
            if not self.on:
                return fn()
            g = self.open.get(s)
            if self.per_launch or g is None or g[0] != cat:
                # Where one group follows another on the stream, the event that ends the first
                # also starts the second: one record per change of family.
                e0 = self._close(s)
                if e0 is None or self.per_launch:
                    e0 = TimingEvent()
                    e0.record(s)
                g = self.open[s] = [cat, [], e0]
            out = fn()
            g[1].append((key, flops, nbytes))
            if self.per_launch:
                self._close(s)
        return out

    def flush(self):
        """Close the open groups (end of a step)."""
        for s in list(self.open):
            with self.torch.cuda.stream(s):
                self._close(s)

    def summary(self):
        """Per-family and per-shape totals; call once, after a device synchronize."""
        cats = {}
        shapes = {}
        for cat, items, e0, e1 in self.rec:
            ms = e0.elapsed_time(e1)
            c = cats.setdefault(cat, dict(ms=0.0, flops=0.0, bytes=0.0, launches=0))
            c["ms"] += ms
            c["launches"] += len(items)
            for key, flops, nbytes in items:
                c["flops"] += flops
                c["bytes"] += nbytes
            if len(items) == 1:
                key, flops, nbytes = items[0]
                sh = shapes.setdefault(f"{cat}: {key}", dict(ms=0.0, flops=0.0, bytes=0.0, launches=0))
                sh["ms"] += ms
                sh["flops"] += flops
                sh["bytes"] += nbytes
                sh["launches"] += 1
        # The timestamps are read; the events are released (the records stay for their keys).
        done = set()
        for r in self.rec:
            for e in (r[2], r[3]):
                if id(e) not in done:
                    done.add(id(e))
                    e.destroy()
        return cats, shapes


def file_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def main():
    args = parse()
    if args.counters:
        if len(args.counters) < 2:
            raise SystemExit("--counters needs PROBE_JSON and at least one run directory")
        reduce_counters(args.counters[0], args.counters[1:])
        return
    if args.load_child:
        m, tp, path, out = args.load_child
        load_child(m, int(tp), path, out)
        return
    if args.load:
        load_bench(args)
        return
    if args.configs_trace:
        configs_trace(args.configs_trace)
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary)
        return
    if args.cold_trace:
        cold_trace(*args.cold_trace)
        return
    if args.configs:
        configs_bench(args)
        return
    if args.vendor:
        vendor_bench(args)
        return
    if args.vendor_square:
        vendor_bench(args, square=True)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU's share on one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) "
              "is not supported: the multi-GPU path (RCCL collectives) is not built.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth_inputs as si
    import tensor_sharded_linear_amd as tsl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tsl.load_library()

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    t_gen = time.time()
    fb = si.workload("full_block")
    ada = si.workload("adaln")
    m = fb.meta
    M, hidden, ffn, H, hd = m["M"], m["hidden"], m["ffn"], m["heads"], m["head_dim"]
    x, A = up(fb.arrays["x"]), up(fb.arrays["a"])
    wqkv, wo = up(fb.arrays["w_qkv"]), up(fb.arrays["w_o"])
    w1, w2 = up(fb.arrays["w1"]), up(fb.arrays["w2"])
    c_ada, w_ada = up(ada.arrays["c"]), up(ada.arrays["w_ada"])
    gu = si.workload("swiglu_ffn")
    x_gu, w_gu, b_gu = up(gu.arrays["x"]), up(gu.arrays["w_gu"]), up(gu.arrays["b_gu"])
    del fb, ada, gu
    si.workload.cache_clear()
    print(f"# inputs generated and uploaded in {time.time() - t_gen:.1f}s", file=sys.stderr, flush=True)

    tps = [int(p) for p in args.tp.split(",")]
    B_ADA, P_ADA = 4, 4
    n_ada = w_ada.shape[0] // P_ADA

    # Preallocated shards and outputs (per tp degree, per rank).
    bufs = {}
    for P in tps:
        b = dict(
            wq=[torch.empty(3 * H // P * hd, hidden, dtype=torch.bfloat16, device=dev) for _ in range(P)],
            wo=[torch.empty(hidden, hidden // P, dtype=torch.bfloat16, device=dev) for _ in range(P)],
            w1=[torch.empty(ffn // P, hidden, dtype=torch.bfloat16, device=dev) for _ in range(P)],
            w2=[torch.empty(hidden, ffn // P, dtype=torch.bfloat16, device=dev) for _ in range(P)],
            q=[torch.empty(M, 3 * H // P * hd, dtype=torch.bfloat16, device=dev) for _ in range(P)],
            h=[torch.empty(M, ffn // P, dtype=torch.bfloat16, device=dev) for _ in range(P)],
            po=[torch.empty(M, hidden, dtype=torch.float32, device=dev) for _ in range(P)],
            pd=[torch.empty(M, hidden, dtype=torch.float32, device=dev) for _ in range(P)],
            out_sum=torch.empty(M, hidden, dtype=torch.float32, device=dev),
            down_sum=torch.empty(M, hidden, dtype=torch.bfloat16, device=dev),
            q_cat=torch.empty(M, 3 * H * hd, dtype=torch.bfloat16, device=dev),
            h_cat=torch.empty(M, ffn, dtype=torch.bfloat16, device=dev),
        )
        bufs[P] = b
    ada_w = [torch.empty(n_ada, hidden, dtype=torch.bfloat16, device=dev) for _ in range(P_ADA)]
    ada_y = [torch.empty(B_ADA, n_ada, dtype=torch.bfloat16, device=dev) for _ in range(P_ADA)]
    # the same adaLN projection sharded rowwise_split_input: column blocks of W, fp32 partials, SUM
    n_full_ada, k_ada = w_ada.shape[0], hidden // P_ADA
    ada_ws = [torch.empty(n_full_ada, k_ada, dtype=torch.bfloat16, device=dev) for _ in range(P_ADA)]
    ada_p = [torch.empty(B_ADA, n_full_ada, dtype=torch.float32, device=dev) for _ in range(P_ADA)]
    ada_sum = torch.empty(B_ADA, n_full_ada, dtype=torch.bfloat16, device=dev)
    # FLUX.2-style fused gate/up projection, blocks [1, 1], SwiGLU epilogue, tp 4
    P_GU = 4
    n_gu = ffn // P_GU
    gu_w = [torch.empty(2 * n_gu, hidden, dtype=torch.bfloat16, device=dev) for _ in range(P_GU)]
    gu_b = [torch.empty(2 * n_gu, dtype=torch.bfloat16, device=dev) for _ in range(P_GU)]
    gu_y = [torch.empty(M, n_gu, dtype=torch.bfloat16, device=dev) for _ in range(P_GU)]
    gen = torch.Generator(device="cpu").manual_seed(5)
    b_ada = torch.randn(n_full_ada, generator=gen).to(torch.bfloat16).to(dev)

    T = Timer(torch, per_launch=args.detail)
    gemm_flops_step = 0.0

    def gemm_cost(m_, n_, k_, out_es):
        return 2.0 * m_ * n_ * k_, 2.0 * (m_ * k_ + n_ * k_) + out_es * m_ * n_

    # Two streams: the index and combine kernels (HBM-bound) run on `cs` and overlap
    # the GEMMs (MFMA-bound) on `ms`; events carry every producer -> consumer and
    # reader -> next writer dependency between them, across steps too.
    ms = torch.cuda.current_stream()
    cs = torch.cuda.Stream(device=dev) if args.streams > 1 else ms
    two = cs is not ms
    ev = {}

    def wait(stream, key):
        if two and key in ev:
            stream.wait_event(ev[key])

    def mark(stream, key):
        if two:
            e = torch.cuda.Event()
            e.record(stream)
            ev[key] = e

    def slice_rank(P, r):
        """Shard every weight for rank r (index kernels)."""
        b = bufs[P]
        kq = 3 * H // P * hd
        wait(cs, ("w read", P, r))
        T.run("slice", f"qkv P{P}", 0, 2 * 2 * kq * hidden,
              lambda: tsl.tp_fused_qkv_split(wqkv, None, H, hd, P, r, w_out=b["wq"][r]), cs)
        T.run("slice", f"wo P{P}", 0, 2 * 2 * hidden * hidden // P,
              lambda: tsl.tp_plan_shard_slice(wo, None, "rowwise", P, r, w_out=b["wo"][r]), cs)
        T.run("slice", f"w1 P{P}", 0, 2 * 2 * ffn // P * hidden,
              lambda: tsl.tp_plan_shard_slice(w1, None, "colwise", P, r, w_out=b["w1"][r]), cs)
        T.run("slice", f"w2 P{P}", 0, 2 * 2 * hidden * ffn // P,
              lambda: tsl.tp_plan_shard_slice(w2, None, "rowwise", P, r, w_out=b["w2"][r]), cs)
        mark(cs, ("w ready", P, r))

    def gemm_rank(P, r):
        """Rank r's four projections."""
        b = bufs[P]
        kq = 3 * H // P * hd
        k_loc = hidden // P
        wait(ms, ("w ready", P, r))
        f, by = gemm_cost(M, kq, hidden, 2)
        T.run("gemm", f"colwise {M}x{kq}x{hidden}", f, by,
              lambda: tsl.tp_linear_colwise(x, b["wq"][r], out=b["q"][r]), ms)
        f, by = gemm_cost(M, hidden, k_loc, 4)
        T.run("gemm", f"rowwise {M}x{hidden}x{k_loc}", f, by,
              lambda: tsl.tp_linear_rowwise(A[:, r * k_loc:(r + 1) * k_loc], b["wo"][r],
                                            out=b["po"][r]), ms)
        f, by = gemm_cost(M, ffn // P, hidden, 2)
        T.run("gemm", f"colwise+gelu {M}x{ffn // P}x{hidden}", f, by,
              lambda: tsl.tp_linear_colwise(x, b["w1"][r], act="gelu_tanh", out=b["h"][r]), ms)
        f, by = gemm_cost(M, hidden, ffn // P, 4)
        T.run("gemm", f"rowwise {M}x{hidden}x{ffn // P}", f, by,
              lambda: tsl.tp_linear_rowwise(b["h"][r], b["w2"][r], out=b["pd"][r]), ms)
        mark(ms, ("w read", P, r))

    def step():
        for P in tps:
            b = bufs[P]
            for r in range(P):
                slice_rank(P, r)
            wait(ms, ("out read", P))
            for r in range(P):
                gemm_rank(P, r)
            mark(ms, ("out ready", P))
            # layer-boundary combines
            wait(cs, ("out ready", P))
            T.run("sum", f"P{P} f32", 0, (P + 1) * 4.0 * M * hidden,
                  lambda: tsl.tp_partial_combine(b["po"], "sum", out=b["out_sum"]), cs)
            T.run("sum", f"P{P} bf16", 0, (P * 4.0 + 2.0) * M * hidden,
                  lambda: tsl.tp_partial_combine(b["pd"], "sum", out=b["down_sum"]), cs)
            T.run("concat", f"qkv P{P}", 0, 2 * 2.0 * M * 3 * H * hd,
                  lambda: tsl.tp_partial_combine(b["q"], "concat", blocks=[1, 1, 1], out=b["q_cat"]), cs)
            T.run("concat", f"up P{P}", 0, 2 * 2.0 * M * ffn,
                  lambda: tsl.tp_partial_combine(b["h"], "concat", out=b["h_cat"]), cs)
            mark(cs, ("out read", P))
        # fused gate/up projection with SwiGLU: packed [1, 1] slices, then each rank's GEMM
        for r in range(P_GU):
            wait(cs, ("gu read", r))
            T.run("slice", "w_gu [1,1]", 0, 2 * 2 * 2 * n_gu * hidden,
                  lambda: tsl.tp_plan_shard_slice(w_gu, b_gu, "colwise", P_GU, r, blocks=[1, 1],
                                                  w_out=gu_w[r], b_out=gu_b[r]), cs)
            mark(cs, ("gu ready", r))
        for r in range(P_GU):
            wait(ms, ("gu ready", r))
            f, by = gemm_cost(M, 2 * n_gu, hidden, 0)
            T.run("gemm", f"colwise+swiglu {M}x{2 * n_gu}x{hidden}", f, by + 2.0 * M * n_gu,
                  lambda: tsl.tp_linear_colwise(x_gu, gu_w[r], gu_b[r], act="swiglu", out=gu_y[r]), ms)
            mark(ms, ("gu read", r))
        # adaLN modulation: shard for 4 ranks, then each rank's skinny GEMV
        for r in range(P_ADA):
            wait(cs, ("ada read", r))
            T.run("slice", "w_ada", 0, 2 * 2 * n_ada * hidden,
                  lambda: tsl.tp_plan_shard_slice(w_ada, None, "colwise", P_ADA, r, w_out=ada_w[r]), cs)
            mark(cs, ("ada ready", r))
        for r in range(P_ADA):
            wait(ms, ("ada ready", r))
            T.run("gemv", f"adaLN B{B_ADA} {n_ada}x{hidden}", 2.0 * B_ADA * n_ada * hidden,
                  2.0 * n_ada * hidden + 2.0 * B_ADA * (hidden + n_ada),
                  lambda: tsl.tp_linear_colwise(c_ada, ada_w[r], out=ada_y[r]), ms)
            mark(ms, ("ada read", r))
        # adaLN modulation, rowwise_split_input: shard, each rank's partial from its input slice, SUM
        for r in range(P_ADA):
            wait(cs, ("adas read", r))
            T.run("slice", "w_ada split", 0, 2 * 2 * n_full_ada * k_ada,
                  lambda: tsl.tp_plan_shard_slice(w_ada, None, "rowwise_split_input", P_ADA, r,
                                                  w_out=ada_ws[r]), cs)
            mark(cs, ("adas ready", r))
        for r in range(P_ADA):
            wait(ms, ("adas ready", r))
            T.run("gemv", f"adaLN split-input B{B_ADA} {n_full_ada}x{k_ada}", 2.0 * B_ADA * n_full_ada * k_ada,
                  2.0 * n_full_ada * k_ada + 2.0 * B_ADA * k_ada + 4.0 * B_ADA * n_full_ada,
                  lambda: tsl.tp_linear_rowwise_split_input(c_ada, ada_ws[r], P_ADA, r, out=ada_p[r]), ms)
            mark(ms, ("adas read", r))
        T.run("sum", f"adaLN P{P_ADA} bf16", 0, (P_ADA * 4.0 + 2.0) * B_ADA * n_full_ada + 2.0 * n_full_ada,
              lambda: tsl.tp_partial_combine(ada_p, "sum", bias=b_ada, out=ada_sum), ms)
        T.flush()

    for P in tps:
        gemm_flops_step += P * 2.0 * M * hidden * (3 * H // P * hd + ffn // P) + \
            P * 2.0 * M * hidden * (hidden // P + ffn // P)
    gemm_flops_step += P_GU * 2.0 * M * 2 * n_gu * hidden
    lin_flops_step = gemm_flops_step + P_ADA * 2.0 * B_ADA * n_ada * hidden \
        + P_ADA * 2.0 * B_ADA * n_full_ada * k_ada

    if args.probe:
        step()
        torch.cuda.synchronize()
        T.on = True
        step()
        torch.cuda.synchronize()
        T.on = False
        launches = [[r[0], key, flops, nbytes] for r in T.rec for key, flops, nbytes in r[1]]
        g = [it for it in launches if it[0] == "gemm"]
        cal = torch.empty(CAL_ROWS, CAL_COLS, dtype=torch.bfloat16, device=dev)
        tsl.tp_plan_shard_slice(cal, None, "colwise", 1, 0)
        torch.cuda.synchronize()
        with open(args.probe, "w") as f:
            json.dump(dict(launches=launches, gemm_launches_per_step=len(g),
                           alg_bytes_per_launch=sum(it[3] for it in g) / len(g),
                           cal_bytes=2 * CAL_ROWS * CAL_COLS), f)
        print(f"probe: {len(launches)} launches per step, {len(g)} of them GEMMs", flush=True)
        return

    import gc
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    T.on = True
    # No collector pauses on the host while the GPU timeline is timed: a pause long enough to
    # drain the launch queue would show up inside an event pair.
    gc.collect()
    gc.disable()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gc.enable()
    T.on = False
    ms_per_step = (t1 - t0) * 1e3 / max(args.steps, 1)
    cats, shapes = T.summary()

    # Outside the step: the colwise adaLN GEMV for each number of conditioning rows the
    # workload allows (1 to 4), every rank's shard in turn, timed like the step's kernels.
    gemv_rows = {}
    for nb in [n for n in range(1, B_ADA + 1)] * 2:   # the first pass over the row counts is a warm-up
        Tb = Timer(torch)
        Tb.on = True
        ys = [torch.empty(nb, n_ada, dtype=torch.bfloat16, device=dev) for _ in range(P_ADA)]
        for _ in range(3):
            for r in range(P_ADA):
                Tb.run("gemv", f"B{nb}", 2.0 * nb * n_ada * hidden, 2.0 * n_ada * hidden + 2.0 * nb * (hidden + n_ada),
                       lambda: tsl.tp_linear_colwise(c_ada[:nb], ada_w[r], out=ys[r]), ms)
            Tb.flush()
        torch.cuda.synchronize()
        c = Tb.summary()[0]["gemv"]
        gemv_rows[str(nb)] = dict(avg_us=round(c["ms"] * 1e3 / c["launches"], 2),
                                  gbs=round(c["bytes"] / (c["ms"] * 1e-3) / 1e9, 1),
                                  pct_hbm_peak=round(100 * c["bytes"] / (c["ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 1))

    # Outside the step: every HBM-bound call of the step once per shape (rank 0), cold: a
    # 512 MiB read evicts the 256 MB Infinity Cache before each call, and the call is timed
    # alone by an event pair on its stream (median of 5).  Family figures weight each call by
    # how often the step makes it.
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    def cold_us(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        evs = []
        for _ in range(reps):
            flush.sum()
            e0, e1 = TimingEvent(), TimingEvent()
            e0.record(ms)
            fn()
            e1.record(ms)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        for a, b in evs:
            a.destroy()
            b.destroy()
        return ts[len(ts) // 2]

    cold_calls = []   # (family, key, bytes, times per step, fn)
    for P in tps:
        b = bufs[P]
        kq = 3 * H // P * hd
        cold_calls += [
            ("slice", f"qkv P{P}", 2 * 2 * kq * hidden, P,
             lambda b=b, P=P: tsl.tp_fused_qkv_split(wqkv, None, H, hd, P, 0, w_out=b["wq"][0])),
            ("slice", f"wo P{P}", 2 * 2 * hidden * hidden // P, P,
             lambda b=b, P=P: tsl.tp_plan_shard_slice(wo, None, "rowwise", P, 0, w_out=b["wo"][0])),
            ("slice", f"w1 P{P}", 2 * 2 * ffn // P * hidden, P,
             lambda b=b, P=P: tsl.tp_plan_shard_slice(w1, None, "colwise", P, 0, w_out=b["w1"][0])),
            ("slice", f"w2 P{P}", 2 * 2 * hidden * ffn // P, P,
             lambda b=b, P=P: tsl.tp_plan_shard_slice(w2, None, "rowwise", P, 0, w_out=b["w2"][0])),
            ("sum", f"P{P} f32", (P + 1) * 4.0 * M * hidden, 1,
             lambda b=b: tsl.tp_partial_combine(b["po"], "sum", out=b["out_sum"])),
            ("sum", f"P{P} bf16", (P * 4.0 + 2.0) * M * hidden, 1,
             lambda b=b: tsl.tp_partial_combine(b["pd"], "sum", out=b["down_sum"])),
            ("concat", f"qkv P{P}", 2 * 2.0 * M * 3 * H * hd, 1,
             lambda b=b: tsl.tp_partial_combine(b["q"], "concat", blocks=[1, 1, 1], out=b["q_cat"])),
            ("concat", f"up P{P}", 2 * 2.0 * M * ffn, 1,
             lambda b=b: tsl.tp_partial_combine(b["h"], "concat", out=b["h_cat"])),
        ]
    cold_calls += [
        ("slice", "w_gu [1,1]", 2 * 2 * 2 * n_gu * hidden, P_GU,
         lambda: tsl.tp_plan_shard_slice(w_gu, b_gu, "colwise", P_GU, 0, blocks=[1, 1], w_out=gu_w[0],
                                         b_out=gu_b[0])),
        ("slice", "w_ada", 2 * 2 * n_ada * hidden, P_ADA,
         lambda: tsl.tp_plan_shard_slice(w_ada, None, "colwise", P_ADA, 0, w_out=ada_w[0])),
        ("slice", "w_ada split", 2 * 2 * n_full_ada * k_ada, P_ADA,
         lambda: tsl.tp_plan_shard_slice(w_ada, None, "rowwise_split_input", P_ADA, 0, w_out=ada_ws[0])),
        ("gemv", f"adaLN split-input B{B_ADA}", 2.0 * n_full_ada * k_ada + 2.0 * B_ADA * k_ada
         + 4.0 * B_ADA * n_full_ada, P_ADA,
         lambda: tsl.tp_linear_rowwise_split_input(c_ada, ada_ws[0], P_ADA, 0, out=ada_p[0])),
    ]
    for nb in range(1, B_ADA + 1):
        yb = torch.empty(nb, n_ada, dtype=torch.bfloat16, device=dev)
        cold_calls.append(("gemv", f"adaLN B{nb}", 2.0 * n_ada * hidden + 2.0 * nb * (hidden + n_ada),
                           P_ADA if nb == B_ADA else 0,
                           lambda nb=nb, yb=yb: tsl.tp_linear_colwise(c_ada[:nb], ada_w[0], out=yb)))
    cold_rows = []
    for fam, key, nbytes, mult, fn in cold_calls:
        us = cold_us(fn)
        cold_rows.append((fam, key, nbytes, mult, us))
    del flush
    cold_fam = {}
    for fam, key, nbytes, mult, us in cold_rows:
        if mult:
            e = cold_fam.setdefault(fam, [0.0, 0.0])
            e[0] += mult * nbytes
            e[1] += mult * us * 1e-6
    cold = {fam: dict(gbs=round(bb / t / 1e9, 1), pct_hbm_peak=round(100 * bb / t / 1e9 / PEAK_HBM_GBS, 1))
            for fam, (bb, t) in sorted(cold_fam.items())}
    cold["gemv_by_rows"] = {key.split("B")[-1]: round(100 * nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 1)
                            for fam, key, nbytes, mult, us in cold_rows if key.startswith("adaLN B")}
    if args.cold_md:
        md = ["# Cold per-call times of the step's HBM-bound calls", "",
              "Command (run from the repository root on one MI355X):", "", "```",
              "python3 bench.py " + " ".join(sys.argv[1:]), "```", "",
              "After the timed steps, each call below runs once per shape (rank 0) right after a 512 MiB read "
              "that evicts the 256 MB Infinity Cache, timed alone by an event pair on its stream; the figure "
              "is the median of 5.  GB/s is algorithmic bytes (read + write of a copy; every part plus the "
              "output for a SUM; the weight plus activations and outputs for a GEMV) over that time.  The "
              "family lines weight each call by how often one step makes it.", "",
              "| family | call | MB | per step | µs | GB/s | % of 8 TB/s |", "|---|---|---|---|---|---|---|"]
        for fam, key, nbytes, mult, us in cold_rows:
            g_ = nbytes / (us * 1e-6) / 1e9
            md.append(f"| {fam} | {key} | {nbytes / 1e6:.1f} | {mult} | {us:.1f} | {g_:.0f} | "
                      f"{100 * g_ / PEAK_HBM_GBS:.1f} |")
        md += ["", "| family (weighted) | GB/s | % of 8 TB/s |", "|---|---|---|"]
        for fam, v in cold.items():
            if fam != "gemv_by_rows":
                md.append(f"| {fam} | {v['gbs']:.0f} | {v['pct_hbm_peak']:.1f} |")
        with open(args.cold_md, "w") as f:
            f.write("\n".join(md) + "\n")

    def gbs(c):
        return c["bytes"] / (c["ms"] * 1e-3) / 1e9 if c["ms"] > 0 else 0.0

    g = cats["gemm"]
    gemm_tflops = g["flops"] / (g["ms"] * 1e-3) / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_sha") == file_sha(GEMM_SRC):
            traffic = tr.get("bytes_per_launch")
    kernels = {}
    for name, c in cats.items():
        ent = dict(launches=c["launches"], avg_us=round(c["ms"] * 1e3 / c["launches"], 2))
        if c["flops"]:
            tf = c["flops"] / (c["ms"] * 1e-3) / 1e12
            ent.update(tflops=round(tf, 1), pct_mfma_peak=round(100 * tf / PEAK_BF16_TFLOPS, 1))
        ent.update(gbs=round(gbs(c), 1), pct_hbm_peak=round(100 * gbs(c) / PEAK_HBM_GBS, 1))
        kernels[name] = ent
    result = {
        "metric": "sharded bf16 linear TFLOP/s (% MFMA peak); combine GB/s (% HBM peak)",
        "value": round(lin_flops_step / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "DiT block linear set, every rank of tp 2/4/8 in turn (hidden 6144, 48 heads x 128, "
                        "FFN 18432, 4608 tokens) + FLUX.2-style fused gate/up 6144->2x18432 with SwiGLU at tp 4 "
                        "+ adaLN 6144->36864 at tp 4, 4 rows, colwise and rowwise_split_input",
            "tokens": M, "hidden": hidden, "ffn": ffn, "heads": H, "head_dim": hd,
            "tp_degrees": tps, "adaln_rows": B_ADA, "adaln_tp": P_ADA,
            "parallelism": "tp shares computed sequentially on 1 GPU" + (
                "; slicing and combines on a second HIP stream, overlapping the GEMMs" if args.streams > 1 else ""),
        },
        "roofline": {
            "kernel": "gemm4_bf16_nt_kernel",
            "bound": "mfma",
            "achieved": round(gemm_tflops, 1),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
        "kernels": kernels,
        "pct_mfma_peak_whole_step": round(100 * lin_flops_step / (ms_per_step * 1e-3) / 1e12
                                          / PEAK_BF16_TFLOPS, 1),
        "adaln_gemv_by_rows": gemv_rows,
        "cold": cold,
    }
    if args.detail:
        for k, s in sorted(shapes.items()):
            sec = s["ms"] * 1e-3
            # roofline fraction: max(flops / MFMA peak, bytes / HBM peak) over the measured time
            roof = max(s["flops"] / (PEAK_BF16_TFLOPS * 1e12), s["bytes"] / (PEAK_HBM_GBS * 1e9)) / sec
            print(f"# {k:48s} launches={s['launches']:4d} avg_us={s['ms'] * 1e3 / s['launches']:9.1f} "
                  f"TFLOP/s={s['flops'] / sec / 1e12:8.1f} GB/s={s['bytes'] / sec / 1e9:8.1f} "
                  f"roofline_frac={roof:.3f}", file=sys.stderr)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds, lin_flops_step)
    print(json.dumps(result), flush=True)


# ---------------------------------------------------------------------------------------------
# per-call table of the named workloads (rank 0 of each), cold and warm
# ---------------------------------------------------------------------------------------------

FLUSH_BYTES = 512 << 20  # twice the 256 MB Infinity Cache: reading it evicts every operand


def configs_bench(args):
    """Time every call of the tiny MLP, attention, large-MLP and adaLN workloads (rank 0).

    Cold: a 512 MiB read runs before each call, so operands come from HBM; the figure is the
    median of --steps calls, each timed by its own HIP event pair.  Warm: --steps calls back to
    back under one event pair, averaged.  MFMA calls report TFLOP/s and the roofline fraction
    max(flops / 2.5 PF, bytes / 8 TB/s) / time; HBM calls report GB/s of algorithmic bytes."""
    import numpy as np
    import torch

    import synth_inputs as si
    import tensor_sharded_linear_amd as tsl

    if not torch.cuda.is_available():
        print("bench.py --configs needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tsl.load_library()
    reps, warm = max(args.steps, 20), max(args.warmup, 5)
    # A read-only flush: a fill would leave dirty lines that the timed call then writes back.
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def cold_us(fn):
        """Median over reps of one call after the cache flush; the flush keeps the GPU busy while
        the host enqueues the events and the call, so no launch gap is timed (the event pair
        itself adds 2-3 us)."""
        for _ in range(warm):
            fn()
        evs = []
        for _ in range(reps):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) * 1e3 for a, b in evs]))

    def warm_us(fn):
        """Average of reps back-to-back calls under one event pair; a spin kernel first keeps the
        GPU busy while the host enqueues them all."""
        for _ in range(warm):
            fn()
        torch.cuda._sleep(40000 * reps)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    rows = []

    def call(cfg, name, fn, flops, nbytes):
        c, w = cold_us(fn), warm_us(fn)
        if flops:
            t_roof = max(flops / (PEAK_BF16_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9)) * 1e6
            bound = "mfma" if flops / (PEAK_BF16_TFLOPS * 1e12) >= nbytes / (PEAK_HBM_GBS * 1e9) else "hbm"
            r = dict(config=cfg, call=name, bound=bound, flops=flops, bytes=nbytes, cold_us=round(c, 2),
                     warm_us=round(w, 2), tflops=round(flops / c / 1e6, 1),
                     pct_mfma_peak=round(100 * flops / c / 1e6 / PEAK_BF16_TFLOPS, 1),
                     roofline_frac=round(t_roof / c, 3))
        else:
            r = dict(config=cfg, call=name, bound="hbm", flops=0, bytes=nbytes, cold_us=round(c, 2),
                     warm_us=round(w, 2), gbs=round(nbytes / c / 1e3, 1),
                     pct_hbm_peak=round(100 * nbytes / c / 1e3 / PEAK_HBM_GBS, 1), roofline_frac=None)
            r["roofline_frac"] = round(r["pct_hbm_peak"] / 100, 3)
        rows.append(r)
        print(f"# {cfg:10s} {name:44s} cold {c:8.1f} us  warm {w:8.1f} us", file=sys.stderr, flush=True)

    def gemm_bytes(m_, n_, k_, out_es, bias=False):
        return 2 * (m_ * k_ + n_ * k_) + out_es * m_ * n_ + (2 * n_ if bias else 0)

    oracle_rows = []
    # tiny MLP, tp 2: both ranks' slices and GEMMs, then the SUM with the bias
    wl = si.workload("tiny_mlp")
    a = {k: up(v) for k, v in wl.arrays.items()}
    P, M, D, F = 2, wl.meta["M"], wl.meta["hidden"], wl.meta["ffn"]
    f = F // P
    w1s = [tsl.tp_plan_shard_slice(a["w1"], a["b1"], "colwise", P, r) for r in range(P)]
    w2s = [tsl.tp_plan_shard_slice(a["w2"], None, "rowwise", P, r)[0] for r in range(P)]
    hs = [tsl.tp_linear_colwise(a["x"], w, b, act="gelu_tanh") for w, b in w1s]
    parts = [tsl.tp_linear_rowwise(h, w) for h, w in zip(hs, w2s)]
    call("tiny_mlp", f"slice W1 colwise + b1 [{f},{D}]", lambda: tsl.tp_plan_shard_slice(
        a["w1"], a["b1"], "colwise", P, 0, w_out=w1s[0][0], b_out=w1s[0][1]), 0, 2 * 2 * (f * D + f))
    call("tiny_mlp", f"slice W2 rowwise [{D},{f}]", lambda: tsl.tp_plan_shard_slice(
        a["w2"], None, "rowwise", P, 0, w_out=w2s[0]), 0, 2 * 2 * D * f)
    call("tiny_mlp", f"colwise+b1+GELU {M}x{f}x{D}", lambda: tsl.tp_linear_colwise(
        a["x"], w1s[0][0], w1s[0][1], act="gelu_tanh", out=hs[0]), 2 * M * f * D, gemm_bytes(M, f, D, 2, True))
    call("tiny_mlp", f"rowwise {M}x{D}x{f} -> f32", lambda: tsl.tp_linear_rowwise(hs[0], w2s[0], out=parts[0]),
         2 * M * D * f, gemm_bytes(M, D, f, 4))
    y = torch.empty(M, D, dtype=torch.float32, device=dev)
    call("tiny_mlp", f"SUM of {P} x [{M},{D}] f32 + b2", lambda: tsl.tp_partial_combine(
        parts, "sum", bias=a["b2"], out=y), 0, P * 4 * M * D + 4 * M * D + 2 * D)

    # The whole forward (both ranks' GEMMs and the SUM, 2 P + 1 launches) is launch-bound:
    # launched call by call against one replay of a HIP graph captured from the same calls.
    def forward():
        for r in range(P):
            tsl.tp_linear_colwise(a["x"], w1s[r][0], w1s[r][1], act="gelu_tanh", out=hs[r])
            tsl.tp_linear_rowwise(hs[r], w2s[r], out=parts[r])
        tsl.tp_partial_combine(parts, "sum", bias=a["b2"], out=y)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        forward()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        forward()
    forward()
    torch.cuda.synchronize()
    y_eager = y.clone()
    graph.replay()
    torch.cuda.synchronize()
    if not torch.equal(y.view(torch.int32), y_eager.view(torch.int32)):
        raise SystemExit("tiny MLP: the graph replay differs from the eager forward")
    def paced_us(fn):
        """Average of reps calls issued from Python with no spin kernel ahead of them, so the
        host's launch overhead is timed too (a caller's view of a launch-bound sequence)."""
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    graph_rows = [dict(config="tiny_mlp", call=f"forward, {2 * P + 1} launches (both ranks' GEMMs, SUM)",
                       eager_us=round(warm_us(forward), 2), graph_us=round(warm_us(graph.replay), 2),
                       eager_paced_us=round(paced_us(forward), 2), graph_paced_us=round(paced_us(graph.replay), 2))]
    print(f"# tiny_mlp forward: queued ahead eager {graph_rows[0]['eager_us']} us, graph {graph_rows[0]['graph_us']} us;"
          f" issued from Python eager {graph_rows[0]['eager_paced_us']} us, graph {graph_rows[0]['graph_paced_us']} us",
          file=sys.stderr, flush=True)
    del graph
    oracle_rows.append(_oracle_config("tiny_mlp", wl))
    del a, w1s, w2s, hs, parts

    # attention projections, tp 4, rank 0: QKV split, colwise QKV, rowwise out-proj on A's column slice
    wl = si.workload("attention_proj")
    a = {k: up(v) for k, v in wl.arrays.items()}
    P, M, D, H, hd = 4, wl.meta["M"], wl.meta["hidden"], wl.meta["heads"], wl.meta["head_dim"]
    kq, kl = 3 * H // P * hd, D // P
    wq, _ = tsl.tp_fused_qkv_split(a["w_qkv"], None, H, hd, P, 0)
    wo, _ = tsl.tp_plan_shard_slice(a["w_o"], None, "rowwise", P, 0)
    q = torch.empty(M, kq, dtype=torch.bfloat16, device=dev)
    po = torch.empty(M, D, dtype=torch.float32, device=dev)
    call("attention", f"QKV split (head-aligned) [{kq},{D}]", lambda: tsl.tp_fused_qkv_split(
        a["w_qkv"], None, H, hd, P, 0, w_out=wq), 0, 2 * 2 * kq * D)
    call("attention", f"slice W_o rowwise [{D},{kl}]", lambda: tsl.tp_plan_shard_slice(
        a["w_o"], None, "rowwise", P, 0, w_out=wo), 0, 2 * 2 * D * kl)
    call("attention", f"colwise QKV {M}x{kq}x{D}", lambda: tsl.tp_linear_colwise(a["x"], wq, out=q),
         2 * M * kq * D, gemm_bytes(M, kq, D, 2))
    call("attention", f"rowwise out-proj {M}x{D}x{kl} -> f32", lambda: tsl.tp_linear_rowwise(
        a["a"][:, :kl], wo, out=po), 2 * M * D * kl, gemm_bytes(M, D, kl, 4))
    oracle_rows.append(_oracle_config("attention", wl))
    del a, wq, wo, q, po

    # large MLP, tp 4, rank 0
    wl = si.workload("mlp_large")
    a = {k: up(v) for k, v in wl.arrays.items()}
    P, M, D, F = 4, wl.meta["M"], wl.meta["hidden"], wl.meta["ffn"]
    f = F // P
    w1, _ = tsl.tp_plan_shard_slice(a["w1"], None, "colwise", P, 0)
    w2, _ = tsl.tp_plan_shard_slice(a["w2"], None, "rowwise", P, 0)
    h = tsl.tp_linear_colwise(a["x"], w1, act="gelu_tanh")
    pd = torch.empty(M, D, dtype=torch.float32, device=dev)
    call("mlp", f"slice W1 colwise [{f},{D}]", lambda: tsl.tp_plan_shard_slice(
        a["w1"], None, "colwise", P, 0, w_out=w1), 0, 2 * 2 * f * D)
    call("mlp", f"slice W2 rowwise [{D},{f}]", lambda: tsl.tp_plan_shard_slice(
        a["w2"], None, "rowwise", P, 0, w_out=w2), 0, 2 * 2 * D * f)
    call("mlp", f"colwise+GELU {M}x{f}x{D}", lambda: tsl.tp_linear_colwise(
        a["x"], w1, act="gelu_tanh", out=h), 2 * M * f * D, gemm_bytes(M, f, D, 2))
    call("mlp", f"rowwise {M}x{D}x{f} -> f32", lambda: tsl.tp_linear_rowwise(h, w2, out=pd),
         2 * M * D * f, gemm_bytes(M, D, f, 4))
    oracle_rows.append(_oracle_config("mlp", wl))
    del a, w1, w2, h, pd

    # adaLN, tp 4, rank 0: the colwise slice, then the GEMV for 1..4 conditioning rows
    wl = si.workload("adaln")
    a = {k: up(v) for k, v in wl.arrays.items()}
    P, D = 4, wl.meta["hidden"]
    n = wl.meta["out"] // P
    wa, _ = tsl.tp_plan_shard_slice(a["w_ada"], None, "colwise", P, 0)
    call("adaln", f"slice W_ada colwise [{n},{D}]", lambda: tsl.tp_plan_shard_slice(
        a["w_ada"], None, "colwise", P, 0, w_out=wa), 0, 2 * 2 * n * D)
    for B in range(1, 5):
        yb = torch.empty(B, n, dtype=torch.bfloat16, device=dev)
        c = a["c"][:B]
        call("adaln", f"colwise GEMV {B} row{'s' if B > 1 else ''} x [{n},{D}]", lambda c=c, yb=yb:
             tsl.tp_linear_colwise(c, wa, out=yb), 2 * B * n * D, 2 * n * D)
    oracle_rows.append(_oracle_config("adaln", wl))
    del a, wa

    out = {"configs": rows, "graph": graph_rows, "cpu_baseline": oracle_rows, "reps": reps, "warmup": warm,
           "cold": f"{FLUSH_BYTES >> 20} MiB read before each call"}
    md = ["| workload | call | bound | cold µs | warm µs | cold rate | % of peak | roofline frac |",
          "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        rate = f"{r['tflops']} TFLOP/s" if r["flops"] else f"{r['gbs']} GB/s"
        pct = r.get("pct_mfma_peak", r.get("pct_hbm_peak"))
        md.append(f"| {r['config']} | {r['call']} | {r['bound']} | {r['cold_us']} | {r['warm_us']} | {rate} | "
                  f"{pct} | {r['roofline_frac']} |")
    md += ["", "Short sequences replayed from a HIP graph (warm, per forward; the graph is captured from "
           "the same library calls and its output checked against them bit for bit).  'Queued ahead': a "
           "spin kernel first lets the host enqueue every call before the GPU reaches them, so only GPU "
           "time counts; 'issued from Python': the calls are timed as a Python caller issues them, host "
           "overhead included.", "",
           "| workload | sequence | call by call, queued ahead, µs | graph, queued ahead, µs | "
           "call by call, issued from Python, µs | graph, issued from Python, µs |", "|---|---|---|---|---|---|"]
    for g in graph_rows:
        md.append(f"| {g['config']} | {g['call']} | {g['eager_us']} | {g['graph_us']} | {g['eager_paced_us']} | "
                  f"{g['graph_paced_us']} |")
    md += ["", "| workload | oracle sample | oracle seconds | oracle GFLOP/s | threads |", "|---|---|---|---|---|"]
    for o in oracle_rows:
        md.append(f"| {o['config']} | {o['sample']} | {o['seconds']} | {o['gflops']} | {o['cores']} |")
    with open(args.configs, "w") as fh:
        fh.write("\n".join(md) + "\n")
    print(json.dumps(out), flush=True)


COLD_REPS = 5     # cold dispatches per call in the cold table (each after its own flush read)
FAMILY_KERNEL = {"slice": "copy_segments_kernel", "concat": "copy_segments_kernel", "sum": "combine_sum_kernel",
                 "gemv": "gemv_bf16_kernel"}


VENDOR_SHAPES = [("colwise", 4608, 2304, 6144), ("colwise", 4608, 4608, 6144), ("colwise", 4608, 9216, 6144),
                 ("rowwise", 4608, 6144, 768), ("rowwise", 4608, 6144, 1536), ("rowwise", 4608, 6144, 2304),
                 ("rowwise", 4608, 6144, 3072), ("rowwise", 4608, 6144, 4608), ("rowwise", 4608, 6144, 9216)]
# Large products whose 256 x 256 tiles fill the CUs in whole rounds (4 and 16 rounds), and the
# step's largest product for comparison.
SQUARE_SHAPES = [("colwise", 8192, 8192, 4096), ("colwise", 8192, 8192, 8192), ("colwise", 16384, 16384, 8192),
                 ("colwise", 4608, 9216, 6144)]
# Few token rows: the adaLN shard's weight (9216 x 6144) and the tp 4 rowwise_split_input
# shard (36864 x 1536) at 1-64 rows, the tiny MLP's two GEMMs, and 128-512 rows (tiled kernel).
FEW_ROW_SHAPES = ([("colwise", m, 9216, 6144) for m in (1, 4, 6, 16, 32, 64, 128, 256, 512)]
                  + [("colwise", 64, 18432, 6144), ("rowwise", 8, 36864, 1536), ("rowwise", 64, 6144, 1536),
                     ("colwise", 64, 512, 256), ("rowwise", 64, 256, 512)])


def vendor_bench(args, square=False):
    """The step's GEMM shapes (no bias or activation) through this library and through the
    vendor BLAS that torch calls (hipBLASLt): colwise with bf16 output (torch.matmul), rowwise
    with fp32 output (torch.mm with out_dtype).  Each measurement is 3 warm-up calls, then 20
    calls back to back on three rotating operand sets under one event pair (dispatch gaps
    included, as in the step); the two implementations alternate twice per shape and the
    faster of each pair of measurements is kept.  With square=True the shapes are the large
    products of SQUARE_SHAPES instead (10 calls per measurement)."""
    import torch
    import tensor_sharded_linear_amd as tsl
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tsl.load_library()
    reps, warm = (10, 2) if square else (20, 3)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for i in range(warm):
            fn(i % 3)
        torch.cuda.synchronize()
        # A 1 ms spin first: the host enqueues all reps calls before the GPU reaches them, so
        # the pair times the GPU work back to back, not the host's launch rate (which bounds
        # the few-microsecond products otherwise).
        torch.cuda._sleep(2_000_000)
        e0, e1 = TimingEvent(), TimingEvent()
        e0.record(stream)
        for i in range(reps):
            fn(i % 3)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        e0.destroy()
        e1.destroy()
        return us

    rows = []
    if square:
        shapes = [(s, "square") for s in SQUARE_SHAPES]
    else:
        shapes = [(s, "step") for s in VENDOR_SHAPES] + [(s, "few") for s in FEW_ROW_SHAPES]
    for (kind, M, N, K), group in shapes:
        g = torch.Generator(device=dev)
        g.manual_seed(M * 7 + N * 3 + K)
        xs = [torch.randn(M, K, device=dev, generator=g).to(torch.bfloat16) for _ in range(3)]
        ws = [(torch.randn(N, K, device=dev, generator=g) / K ** 0.5).to(torch.bfloat16) for _ in range(3)]
        if kind == "colwise":
            ours = lambda i: tsl.tp_linear_colwise(xs[i], ws[i])
            vend = lambda i: torch.matmul(xs[i], ws[i].t())
            vend_note = "torch.matmul, bf16 out"
        else:
            ours = lambda i: tsl.tp_linear_rowwise(xs[i], ws[i])
            try:
                torch.mm(xs[0], ws[0].t(), out_dtype=torch.float32)
                vend = lambda i: torch.mm(xs[i], ws[i].t(), out_dtype=torch.float32)
                vend_note = "torch.mm, fp32 out"
            except (RuntimeError, TypeError):
                vend = lambda i: torch.matmul(xs[i], ws[i].t())
                vend_note = "torch.matmul, bf16 out (no fp32-output product available)"
        t_ours, t_vend = [], []
        for _ in range(2):
            t_ours.append(timed(ours))
            t_vend.append(timed(vend))
        a, b = min(t_ours), min(t_vend)
        fl = 2.0 * M * N * K
        rows.append(dict(group=group, kind=kind, shape=f"{M}x{N}x{K}", ours_us=round(a, 1),
                         ours_tflops=round(fl / a / 1e6, 1), ours_gbs=round(2.0 * N * K / a / 1e3),
                         vendor_us=round(b, 1), vendor_tflops=round(fl / b / 1e6, 1), vendor_gbs=round(2.0 * N * K / b / 1e3),
                         vendor=vend_note,
                         tile=tsl.tp_linear_tile_shape(M, N, K)))
        print(f"# {kind} {M}x{N}x{K}: ours {a:.1f} us, vendor {b:.1f} us", file=sys.stderr, flush=True)
        del xs, ws
    if square:
        vendor_square_md(args.vendor_square, rows)
        return
    md = ["# GEMM shapes: this library against the vendor BLAS (hipBLASLt)", "",
          "Command (run from the repository root on one MI355X):", "", "```",
          "python3 bench.py " + " ".join(sys.argv[1:]), "```", "",
          "Plain products without bias or activation, the shapes of the step's GEMMs (M x N x K: tokens x "
          "output features x input features).  Each figure: 3 warm-up calls, then a 1 ms spin kernel and "
          "20 calls back to back on three rotating operand sets (random normal bf16) under one event pair "
          "(the spin lets the host queue every call first, so dispatch gaps are included as in the step "
          "but host launch time is not); the two implementations alternate twice per shape, and the faster "
          "measurement of each is kept.  Percent of the 2.5 PFLOP/s bf16 dense peak.", "",
          "| product | M x N x K | this library (tile) | µs | TFLOP/s | % | vendor | µs | TFLOP/s | % | vendor / library time |",
          "|---|---|---|---|---|---|---|---|---|---|---|"]
    def kernel_of(r):
        t0, t1 = r["tile"]
        if (t0, t1) == (0, 0):
            return "weight-streaming"
        return f"split-K, {t1} columns" if t1 <= 48 else f"tiled {t0}x{t1}"

    for r in rows:
        if r["group"] != "step":
            continue
        md.append(f"| {r['kind']} | {r['shape']} | {r['tile'][0]}x{r['tile'][1]} | {r['ours_us']} | "
                  f"{r['ours_tflops']:.0f} | {100 * r['ours_tflops'] / PEAK_BF16_TFLOPS:.1f} | {r['vendor']} | "
                  f"{r['vendor_us']} | {r['vendor_tflops']:.0f} | {100 * r['vendor_tflops'] / PEAK_BF16_TFLOPS:.1f} | "
                  f"{r['vendor_us'] / r['ours_us']:.3f} |")
    md += ["", "## Few token rows", "",
           "The same measurement for products with 1 to 512 rows: the weight (2 N K bytes) dominates "
           "the traffic, so the rate is given as weight GB/s against the 8 TB/s HBM peak.  Three "
           "rotating operand sets take 340 MB and more for the 9216 x 6144 weight, beyond the "
           "256 MB Infinity Cache.", "",
           "| product | M x N x K | this library (kernel) | µs | weight GB/s | % of 8 TB/s | vendor µs | "
           "weight GB/s | vendor / library time |", "|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        if r["group"] != "few":
            continue
        md.append(f"| {r['kind']} | {r['shape']} | {kernel_of(r)} | {r['ours_us']} | {r['ours_gbs']} | "
                  f"{r['ours_gbs'] / 80:.1f} | {r['vendor_us']} | {r['vendor_gbs']} | "
                  f"{r['vendor_us'] / r['ours_us']:.3f} |")
    with open(args.vendor, "w") as f:
        f.write("\n".join(md) + "\n")
    print(json.dumps({"vendor_comparison": rows}), flush=True)


def vendor_square_md(path, rows):
    """The --vendor-square table."""
    md = ["# Large products: this library against the vendor BLAS (hipBLASLt)", "",
          "Command (run from the repository root on one MI355X):", "", "```",
          "python3 bench.py " + " ".join(sys.argv[1:]), "```", "",
          "Plain colwise products (bf16 output, no bias or activation) of random normal bf16 operands "
          "whose 256 x 256 output tiles cover the 256 CUs in whole rounds, beside the step's largest "
          "product.  Measured as in `gemm_vs_vendor_blas.md` (three rotating operand sets, a spin kernel, "
          "then 10 calls back to back under one event pair; the two implementations alternate twice and "
          "the faster measurement of each is kept).  Percent of the 2.5 PFLOP/s bf16 dense peak.", "",
          "| M x N x K | tiles of this library | rounds over 256 CUs | this library µs | TFLOP/s | % | "
          "hipBLASLt µs | TFLOP/s | % | vendor / library time |",
          "|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        m, n, _ = (int(v) for v in r["shape"].split("x"))
        t0, t1 = r["tile"]
        tiles = -(-m // t0) * -(-n // t1)
        md.append(f"| {r['shape']} | {t0}x{t1} ({tiles}) | {tiles / 256:.2f} | {r['ours_us']} | "
                  f"{r['ours_tflops']:.0f} | {100 * r['ours_tflops'] / PEAK_BF16_TFLOPS:.1f} | {r['vendor_us']} | "
                  f"{r['vendor_tflops']:.0f} | {100 * r['vendor_tflops'] / PEAK_BF16_TFLOPS:.1f} | "
                  f"{r['vendor_us'] / r['ours_us']:.3f} |")
    with open(path, "w") as f:
        f.write("\n".join(md) + "\n")
    print(json.dumps({"vendor_square": rows}), flush=True)


def cold_trace(trace_csv, cold_md):
    """The cold table of a --cold-md run with kernel durations from the same run's rocprofv3 trace.

    The cold section is the last part of the run that reads the flush buffer: its dispatches that
    directly follow torch's reduction kernel are, in order, COLD_REPS per row of the table.  Each
    row's kernel family is checked against the dispatch names.  Trace durations carry no event
    overhead (an event pair adds 1-3 us to a short call)."""
    import csv
    import statistics

    recs = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    cold, prev = [], ""
    for r in recs:
        name = r["Kernel_Name"]
        if "reduce_kernel" in prev and any(k in name for k in FAMILY_KERNEL.values()):
            cold.append((name, (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
        prev = name
    lines = open(cold_md).read().rstrip("\n").split("\n")
    head = lines.index("| family | call | MB | per step | µs | GB/s | % of 8 TB/s |")
    rows = []
    for ln in lines[head + 2:]:
        if not ln.startswith("| "):
            break
        rows.append([c.strip() for c in ln.strip("|").split("|")])
    need = COLD_REPS * len(rows)
    if len(cold) < need:
        raise SystemExit(f"{trace_csv}: {len(cold)} cold dispatches, the table needs {need}")
    cold = cold[-need:]
    out = lines[:head] + ["| family | call | MB | per step | µs (events) | % of 8 TB/s (events) | µs (trace) | "
                          "GB/s (trace) | % of 8 TB/s (trace) |", "|---|---|---|---|---|---|---|---|---|"]
    fam_tot = {}
    for i, (fam, key, mb, mult, us, _gbs, pct) in enumerate(rows):
        names = {n for n, _ in cold[i * COLD_REPS:(i + 1) * COLD_REPS]}
        if any(FAMILY_KERNEL[fam] not in n for n in names):
            raise SystemExit(f"row {fam} {key}: trace dispatches are {sorted(names)}")
        t = statistics.median(u for _, u in cold[i * COLD_REPS:(i + 1) * COLD_REPS])
        g = float(mb) * 1e6 / (t * 1e-6) / 1e9
        out.append(f"| {fam} | {key} | {mb} | {mult} | {us} | {pct} | {t:.1f} | {g:.0f} | "
                   f"{100 * g / PEAK_HBM_GBS:.1f} |")
        if int(mult):
            e = fam_tot.setdefault(fam, [0.0, 0.0])
            e[0] += int(mult) * float(mb) * 1e6
            e[1] += int(mult) * t * 1e-6
    out += lines[head + 2 + len(rows):]
    out += ["", "The trace durations, weighted in the same way:", "",
            "| family (weighted, trace) | GB/s | % of 8 TB/s |", "|---|---|---|"]
    for fam, (bb, t) in sorted(fam_tot.items()):
        out.append(f"| {fam} | {bb / t / 1e9:.0f} | {100 * bb / t / 1e9 / PEAK_HBM_GBS:.1f} |")
    print("\n".join(out))


def _short_kernel(name):
    """A short label for a kernel of this library or a hipBLASLt GEMM kernel; None for others."""
    short = name.replace("void ", "").replace("tpl::(anonymous namespace)::", "").split("(")[0]
    if short.startswith(("gemm_", "gemm4_", "gemv_", "copy_", "combine_")):
        return short
    if "Cijk" in name:
        mt = next((t for t in name.split("_") if t.startswith("MT")), "MT?")
        return f"hipBLASLt {mt}" + (" stream-K" if "_SK" in name else "")
    return None


def pmc_summary(dirs):
    """Per kernel of this library, and per hipBLASLt GEMM kernel (short name and grid size), the
    mean of every counter over its dispatches, across one or more rocprofv3 --pmc run directories
    (one counter set each), with the mean dispatch time under counter collection.  Where a run
    collected GRBM_GUI_ACTIVE (summed over the 8 XCDs), the clock (GUI-active cycles per XCD over
    the dispatch time) is added, and the busy fractions MfmaUtil (as rocprofv3 derives it),
    TD_TD_BUSY and TA_TA_BUSY per CU cycle, where collected."""
    import csv
    import glob

    paths = [p for d in dirs for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)]
    # Runs of one program dispatch the same kernels in the same order, so a run that counted
    # MfmaFlopsBF16 labels every run's dispatch of a GEMM with its flops (its shape).
    gflop = {}
    for path in paths:
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == "MfmaFlopsBF16" and _short_kernel(r["Kernel_Name"]):
                    gflop[int(r["Dispatch_Id"])] = round(float(r["Counter_Value"]) / 1e9, 1)
    acc = {}   # (kernel, grid, GFLOP) -> counter -> [values]
    for path in paths:
        per = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                short = _short_kernel(r["Kernel_Name"])
                if short is None:
                    continue
                key = (short, int(r["Grid_Size"]), int(r["Dispatch_Id"]))
                e = per.setdefault(key, {})
                e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                e["us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        for (k, grid, disp), cnt in per.items():
            e = acc.setdefault((k, grid, gflop.get(disp, "-")), {})
            if "GRBM_GUI_ACTIVE" in cnt:
                gui = cnt["GRBM_GUI_ACTIVE"] / N_XCC
                e.setdefault("clock GHz", []).append(gui / cnt["us"] / 1e3)
                for c in ("TD_TD_BUSY", "TA_TA_BUSY"):
                    if c in cnt:
                        e.setdefault(c + " / CU cycle", []).append(cnt[c] / (gui * 256))
            for c, v in cnt.items():
                e.setdefault(c, []).append(v)
    if not acc:
        raise SystemExit("no counter_collection.csv with these kernels under " + " ".join(dirs))
    names = sorted({c for e in acc.values() for c in e})

    def fmt(v):
        return f"{v:.0f}" if abs(v) >= 100 else f"{v:.3g}"
    print("| kernel | grid (threads) | GFLOP | dispatches | " + " | ".join(names) + " |")
    print("|---|---|---|---|" + "---|" * len(names))
    for (k, grid, gf), e in sorted(acc.items(), key=lambda kv: (kv[0][0], kv[0][1], str(kv[0][2]))):
        n = min(len(v) for v in e.values())  # a counter of one run: the dispatches per run
        vals = [fmt(sum(e[c]) / len(e[c])) if c in e else "-" for c in names]
        print(f"| `{k}` | {grid} | {gf} | {n} | " + " | ".join(vals) + " |")


def configs_trace(path):
    """Cold and warm medians per kernel (name and grid) from a --configs run's kernel trace.

    A dispatch is cold when the dispatch before it is the flush read (torch's reduction
    kernel).  Unlike the call table's event pairs, these durations carry no event overhead."""
    import csv
    import statistics

    recs = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
    groups, prev = {}, ""
    for r in recs:
        name = r["Kernel_Name"]
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        short = name.replace("void ", "").replace("tpl::(anonymous namespace)::", "").split("(")[0]
        if short.startswith(("gemm_", "gemm4_", "gemv_", "copy_", "combine_")):
            g = groups.setdefault((short, int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"])), ([], []))
            g[0 if "reduce" in prev else 1].append(us)
        prev = name
    print("| kernel | grid (threads) | workgroup | cold dispatches | cold median µs | warm dispatches | warm median µs |")
    print("|---|---|---|---|---|---|---|")
    for (k, grid, wg), (c, w) in groups.items():
        med = lambda v: f"{statistics.median(v):.1f}" if v else "-"
        print(f"| `{k}` | {grid} | {wg} | {len(c)} | {med(c)} | {len(w)} | {med(w)} |")


def _oracle_config(cfg, wl):
    """The oracle (as it stands) on the same workload's rank-0 GEMM work: whole for the tiny MLP
    and the adaLN GEMV, a 192-row sample of the 4608 tokens for the attention and MLP workloads."""
    import numpy as np

    import oracle

    a, meta = wl.arrays, wl.meta
    threads = oracle.default_threads()
    t = time.perf_counter()
    if cfg == "tiny_mlp":
        P, D, F = 2, meta["hidden"], meta["ffn"]
        parts = []
        for r in range(P):
            w1, b1 = oracle.shard_colwise(a["w1"], a["b1"], P, r)
            h = oracle.bf16_round(oracle.colwise(a["x"], w1, b1, act=oracle.ACT_GELU_TANH, threads=threads))
            parts.append(oracle.linear(h, oracle.shard_rowwise(a["w2"], P, r), threads=threads))
        oracle.combine_sum(parts, a["b2"])
        flops, sample = 2.0 * meta["M"] * 2 * F * D, "whole workload (both ranks, SUM)"
    elif cfg == "attention":
        P, D, H, hd = 4, meta["hidden"], meta["heads"], meta["head_dim"]
        rows = np.arange(0, meta["M"], meta["M"] // 192)
        wq, _ = oracle.qkv_split(a["w_qkv"], None, H, hd, P, 0)
        oracle.colwise(a["x"], wq, rows=rows, threads=threads)
        oracle.rowwise(a["a"], 0, P, oracle.shard_rowwise(a["w_o"], P, 0), rows=rows, threads=threads)
        flops = 2.0 * len(rows) * (wq.shape[0] * D + D * D // P)
        sample = f"{len(rows)} of {meta['M']} token rows, rank 0 (QKV colwise, out-proj rowwise)"
    elif cfg == "mlp":
        P, D, F = 4, meta["hidden"], meta["ffn"]
        rows = np.arange(0, meta["M"], meta["M"] // 192)
        w1, _ = oracle.shard_colwise(a["w1"], None, P, 0)
        h = oracle.bf16_round(oracle.colwise(a["x"], w1, act=oracle.ACT_GELU_TANH, rows=rows, threads=threads))
        oracle.linear(h, oracle.shard_rowwise(a["w2"], P, 0), threads=threads)
        flops = 2.0 * len(rows) * 2 * (F // P) * D
        sample = f"{len(rows)} of {meta['M']} token rows, rank 0 (FFN-up colwise+GELU, FFN-down rowwise)"
    else:
        P, D = 4, meta["hidden"]
        w, _ = oracle.shard_colwise(a["w_ada"], None, P, 0)
        for B in range(1, 5):
            oracle.colwise(a["c"][:B], w, threads=threads)
        flops = 2.0 * (1 + 2 + 3 + 4) * w.shape[0] * D
        sample = "whole workload (rank 0, 1 to 4 rows)"
    dt = time.perf_counter() - t
    return {"config": cfg, "kind": "oracle", "sample": sample, "seconds": round(dt, 3),
            "gflops": round(flops / dt / 1e9, 2), "cores": threads}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(target_s: float, step_flops: float = 0.0):
    """The CPU oracle (as it stands) on a bounded row sample of the same step's GEMM work.

    The oracle splits rows over threads, so its time is linear in the number of rows: the
    sample's time scaled by M / rows is the full-shape time (labelled "extrapolated")."""
    import numpy as np

    import oracle
    import synth_inputs as si

    fb = si.workload("full_block")
    a, m = fb.arrays, fb.meta
    M, hidden, ffn, H, hd = m["M"], m["hidden"], m["ffn"], m["heads"], m["head_dim"]
    threads = oracle.default_threads()
    P = 4
    r = 0
    wq, _ = oracle.qkv_split(a["w_qkv"], None, H, hd, P, r)
    wo_s = oracle.shard_rowwise(a["w_o"], P, r)
    w1_s, _ = oracle.shard_colwise(a["w1"], None, P, r)
    w2_s = oracle.shard_rowwise(a["w2"], P, r)
    k_loc = hidden // P

    def run(rows):
        oracle.colwise(a["x"], wq, rows=rows, threads=threads)
        oracle.rowwise(a["a"], r, P, wo_s, rows=rows, threads=threads)
        h = oracle.bf16_round(oracle.colwise(a["x"], w1_s, act=oracle.ACT_GELU_TANH, rows=rows,
                                             threads=threads))
        oracle.linear(h, w2_s, threads=threads)
        return len(rows) * 2.0 * (wq.shape[0] * hidden + hidden * k_loc + w1_s.shape[0] * hidden
                                  + hidden * w2_s.shape[1])

    rng = np.random.default_rng(0)
    probe = np.sort(rng.choice(M, size=threads, replace=False))
    t = time.perf_counter()
    run(probe)
    dt = time.perf_counter() - t
    n = int(max(threads, min(M, threads * max(1, round(target_s / max(dt, 1e-3))))))
    rows = np.sort(rng.choice(M, size=n, replace=False))
    t = time.perf_counter()
    flops = run(rows)
    dt = time.perf_counter() - t
    rate = flops / dt
    out = {
        "value": round(rate / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "seconds": round(dt, 2),
        "sample": f"{n} of {M} token rows through rank 0 of tp 4 of the full block (QKV colwise, out-proj "
                  f"rowwise, FFN-up colwise+GELU, FFN-down rowwise); fp64-accumulating C oracle",
        "cpu_model": _cpu_model(),
        "nproc": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count(),
        "cpu_count": os.cpu_count(),
        "extrapolated_full_shape_s": round(dt * M / n, 2),
        "extrapolated_note": f"extrapolated (linear in M): the same four GEMMs for all {M} rows of rank 0 of tp 4",
    }
    if step_flops:
        out["extrapolated_step_s"] = round(step_flops / rate, 1)
    return out


if __name__ == "__main__":
    main()
