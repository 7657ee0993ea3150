"""Benchmark of the Fathom decode-step hot path on one MI355X.

One step = the work of one decode step over a resident bit-plane store:
encode the newest 64-token block of every KV head into its slot, plan the
read depths for a fresh query group (importance, 30-step bisection), scan
every key at those depths, and select the top-k of every query head.

Workload (default): one Qwen3-8B-shaped layer, 8 KV heads x 4 query heads,
d = 128, n = 1,048,576 keys per head, budget 92 code bits, k = 4096; keys,
queries and variances from fathom_inputs (synthetic, seeded).  The store is
held in several copies that the steps rotate through, so the index a step
reads is not left in the 256 MB last-level cache by the previous step.

Passes over the same inputs, each K steps after W warm-up steps:
  * the headline pass: plain calls, timed as a whole (value, ms_per_step);
  * a scan pass: every scan through fathom_scan_timed, whose events take the
    scan kernels' own start and end timestamps (scan median, p10, p90; the
    roofline figures);
  * a stage pass: events between the stages (per-stage and per-step
    medians, p10, p90);
  * the fused call fathom_scan_topk.
Then, unless switched off: the other workloads and budgets (scan and top-k
times, roofline fractions), the fixed-depth plans the pages compare against
read through the same scan (scan time and recall against exact top-k), the
host-resident gather against run size, and the CPU oracle's rate on a
bounded sample (one thread and all host threads).

Prints one JSON line.  HBM traffic of the scan comes from rocprofv3 counter
runs of this command (read requests by size, TCC_EA0_RDREQ_32B/64B/128B, and
write requests, TCC_EA0_WRREQ and TCC_EA0_WRREQ_64B), each scaled by the
factor that makes the counters read the known bytes of a plain copy
(torch.neg over 256 MiB, run here before the timed steps).  The figures are
kept in profiles/scan_q1m_b92_traffic.txt with the sha256 of the scan source
they were taken on; a different source reports traffic null.
`python bench.py --summarize DIR [DIR ...]` turns rocprofv3 csv output into
the text kept under profiles/.
"""
from __future__ import annotations

import argparse
import ctypes
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0                    # MI355X HBM3E
CUS, CLOCK_GHZ = 256, 2.4
# VALU issue per CU per clock, in lanes: fp32 FMA 128 (157.3 TFLOP/s = 78.6 T
# FMA/s); 32-bit integer ops, and every op that reads a scalar register such
# as the plane word, 64 (39.3 T/s).
FMA_PEAK_TOPS = CUS * 128 * CLOCK_GHZ / 1e3      # 78.64 T lane-FMA/s
INT_PEAK_TOPS = CUS * 64 * CLOCK_GHZ / 1e3       # 39.32 T lane-ops/s
CALIB_BYTES = 256 << 20                   # plain copy used to scale the HBM byte counters
SCAN_SRC = os.path.join(ROOT, "sparse_top_kv_fathom_amd", "csrc", "scan.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_q1m_b92_traffic.txt")
INSTR_FILE = os.path.join(ROOT, "profiles", "scan_q1m_b92_instructions.txt")
METRIC = "keys scanned/sec (and HBM GB/s, % roofline) at 1M keys, 92-bit budget"

HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class TimingEvent:
    """A HIP timing event recorded on torch's current stream (the stream the
    library launches on), created with hipEventDisableSystemFence.

    Recording a default event ends with a system-scope release: a cache
    writeback and invalidation that leaves the GPU idle for several
    microseconds around every record and slows the work after it.  These
    events only take timestamps; they are read after a device synchronize.
    Same interface as torch.cuda.Event: record(), elapsed_time(other) in ms.
    """
    _lib = None

    @classmethod
    def _hip(cls):
        if cls._lib is None:
            # The HIP runtime torch has loaded (one runtime per process).
            path = next(line.split()[-1] for line in open("/proc/self/maps")
                        if "libamdhip64" in line)
            lib = ctypes.CDLL(path)
            P = ctypes.c_void_p
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(P), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [P, P]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
            lib.hipEventDestroy.argtypes = [P]
            cls._lib = lib
        return cls._lib

    def __init__(self):
        self.h = ctypes.c_void_p()
        rc = self._hip().hipEventCreateWithFlags(ctypes.byref(self.h),
                                                 HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed: %d" % rc)

    def record(self):
        import torch
        rc = self._hip().hipEventRecord(self.h, ctypes.c_void_p(
            torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def elapsed_time(self, other) -> float:
        ms = ctypes.c_float()
        rc = self._hip().hipEventElapsedTime(ctypes.byref(ms), self.h, other.h)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return ms.value

    def __del__(self):
        if self.h and TimingEvent._lib is not None:
            TimingEvent._lib.hipEventDestroy(self.h)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="q1m")
    ap.add_argument("--budget", type=int, default=92)
    ap.add_argument("--copies", type=int, default=4, help="store copies the steps rotate through")
    ap.add_argument("--step-mode", choices=("fused", "separate"), default="fused",
                    help="the headline step's scan and selection: fathom_scan_topk without a "
                         "score buffer (fused), or fathom_scan then fathom_topk (separate)")
    ap.add_argument("--queries", type=int, default=8, help="distinct query groups drawn")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--store", choices=("raw", "klt"), default="raw",
                    help="raw channel planes, or planes of the KLT-rotated keys")
    ap.add_argument("--no-klt", action="store_true",
                    help="skip timing the KLT fit and rotations (raw store only)")
    ap.add_argument("--no-gather", action="store_true",
                    help="skip timing fathom_gather from a pinned host store")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads and budgets")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the fixed-depth plans read through the same scan")
    ap.add_argument("--sweep", action="store_true",
                    help="budget sweep over layers of the 1M-key shape with planted needles: "
                         "recall against exact scores and scan rate per budget (one JSON object)")
    ap.add_argument("--layers", default="0,17,35",
                    help="sweep layers: comma-separated indices or 'all' (36)")
    ap.add_argument("--summarize", nargs="+", metavar="DIR",
                    help="print rocprofv3 csv output under DIR as text and exit (no GPU use)")
    return ap.parse_args()


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def recorded_counter(path, key):
    """A per-launch scan figure from a committed counter summary, or None when
    it is missing or was taken on another scan source."""
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return None
    kv = dict(l.split(":", 1) for l in lines if ":" in l and not l.startswith((" ", "#")))
    try:
        if kv["scan_source_sha256"].strip() != source_sha(SCAN_SRC):
            return None
        return float(kv[key])
    except (KeyError, ValueError):
        return None


def short_name(name):
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    return name.split("(")[0][:60]


def summarize(dirs):
    """rocprofv3 csv (kernel stats, counter collection) as plain text."""
    means = {}
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
            print("## kernel stats: %s" % os.path.relpath(f, d))
            print("%-60s %6s %12s %12s %7s" % ("kernel", "calls", "avg_us", "total_us", "pct"))
            for r in csv.DictReader(open(f)):
                print("%-60s %6s %12.2f %12.1f %7.2f" % (
                    short_name(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
                    float(r["TotalDurationNs"]) / 1e3, float(r["Percentage"])))
        for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
            # The scan and selection kernels per launch shape (grid threads),
            # so that one workload's launches can be read apart from the
            # others a run makes.
            per = {}
            for r in csv.DictReader(open(f)):
                name = short_name(r["Kernel_Name"])
                if not name.startswith(("fathom::scan", "fathom::fused", "fathom::topk")):
                    continue
                grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
                dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                per.setdefault((name, grid), []).append(dur)
            print("## per launch shape: %s" % os.path.relpath(f, d))
            print("%-44s %12s %6s %10s %10s" % ("kernel", "grid", "calls", "avg_us", "median_us"))
            for (name, grid), v in sorted(per.items()):
                print("%-44s %12d %6d %10.2f %10.2f" % (name[:44], grid, len(v), sum(v) / len(v),
                                                       float(np.median(v))))
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"),
                                  recursive=True)):
            print("## counters: %s" % os.path.relpath(f, d))
            agg = {}
            for r in csv.DictReader(open(f)):
                key = (short_name(r["Kernel_Name"]), r["Counter_Name"])
                agg.setdefault(key, []).append(float(r["Counter_Value"]))
            print("%-60s %-24s %6s %14s" % ("kernel", "counter", "n", "mean"))
            for (kname, cname), v in sorted(agg.items()):
                print("%-60s %-24s %6d %14.1f" % (kname, cname, len(v), sum(v) / len(v)))
                means[(kname, cname)] = sum(v) / len(v)

    def scan_key(k):   # the full scan: scan_main<G, 0> (any rounds per workgroup)
        return re.fullmatch(r"fathom::scan_main<\d+, 0(, \d+)?>", k[0]) is not None
    valu = [v for k, v in means.items() if scan_key(k) and k[1] == "SQ_INSTS_VALU"]
    if valu:
        print("scan_valu_instructions_per_launch: %.0f" % valu[0])
        print("scan_source_sha256: %s" % source_sha(SCAN_SRC))
    # HBM traffic: read requests by size and write requests, in bytes per
    # dispatch, scaled by the factor that makes them read the plain copy's
    # known bytes (reads 256 MiB, writes 256 MiB).
    def get(kfilter, cname):
        v = [val for k, val in means.items() if kfilter(k) and k[1].startswith(cname)
             and (k[1] == cname or k[1] == cname + "_sum")]
        return v[0] if v else None
    is_copy = lambda k: "neg" in k[0]
    rd = ("TCC_EA0_RDREQ_32B", "TCC_EA0_RDREQ_64B", "TCC_EA0_RDREQ_128B")
    if all(get(scan_key, c) is not None for c in rd) and all(get(is_copy, c) is not None for c in rd):
        def rbytes(f):
            return 32 * get(f, rd[0]) + 64 * get(f, rd[1]) + 128 * get(f, rd[2])
        rfac = CALIB_BYTES / rbytes(is_copy)
        scan_r = rbytes(scan_key) * rfac
        print("## scan traffic (request counts by size, scaled by the plain-copy factor)")
        print("    reads: copy of %d bytes counts %.0f -> factor %.4f; scan %.0f bytes"
              % (CALIB_BYTES, rbytes(is_copy), rfac, scan_r))
        total = scan_r
        wr, wr64 = "TCC_EA0_WRREQ", "TCC_EA0_WRREQ_64B"
        if all(get(f, c) is not None for f in (scan_key, is_copy) for c in (wr, wr64)):
            def wbytes(f):
                return 32 * (get(f, wr) - get(f, wr64)) + 64 * get(f, wr64)
            wfac = CALIB_BYTES / wbytes(is_copy)
            scan_w = wbytes(scan_key) * wfac
            print("    writes: copy of %d bytes counts %.0f -> factor %.4f; scan %.0f bytes"
                  % (CALIB_BYTES, wbytes(is_copy), wfac, scan_w))
            total += scan_w
            print("scan_hbm_read_bytes_per_launch: %.0f" % scan_r)
            print("scan_hbm_write_bytes_per_launch: %.0f" % scan_w)
            print("scan_hbm_bytes_per_launch: %.0f" % total)
            print("scan_source_sha256: %s" % source_sha(SCAN_SRC))
    # The same from FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled
    # by the plain copy's factor; FETCH_SIZE weighs a request by the copy's
    # request size, so it over- or under-states other request mixes.
    fw = [get(f, c) for f in (scan_key, is_copy) for c in ("FETCH_SIZE", "WRITE_SIZE")]
    if all(x is not None for x in fw):
        ffac, wfac = CALIB_BYTES / (fw[2] * 1024), CALIB_BYTES / (fw[3] * 1024)
        fb, wb = fw[0] * 1024 * ffac, fw[1] * 1024 * wfac
        print("## scan traffic (FETCH_SIZE / WRITE_SIZE, scaled by the plain-copy factors "
              "%.4f / %.4f)" % (ffac, wfac))
        print("scan_fetch_bytes_per_launch: %.0f" % fb)
        print("scan_write_bytes_per_launch: %.0f" % wb)
        print("scan_fetch_write_bytes_per_launch: %.0f" % (fb + wb))
        print("scan_source_sha256: %s" % source_sha(SCAN_SRC))


def plan_stats(depths: np.ndarray):
    """Per group: code bits T = sum t_j and active channels A = #{t_j > 0}."""
    d = depths.astype(np.int64)
    return d.sum(axis=1), (d > 0).sum(axis=1)


def stats(xs):
    """median, p10, p90, mean of a list of times (ms), rounded."""
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "mean": round(float(a.mean()), 4),
            "n": int(a.size)}


def exact_topk(s: np.ndarray, k: int) -> np.ndarray:
    """The k largest of s, ties to the lower index (the selection's order),
    as sorted indices."""
    part = np.argpartition(-s, k - 1)[:k]
    kth = s[part].min()
    above = np.flatnonzero(s > kth)
    eq = np.flatnonzero(s == kth)
    return np.sort(np.concatenate([above, eq[:k - len(above)]]))


def exact_topk_rows(k16: np.ndarray, q: np.ndarray, k: int):
    """Top-k of the exact fp64 scores q . k over the fp16 keys, per query
    head: k16 [groups][n][d] fp16, q [groups][G][d] -> list of index arrays
    (row r = group * G + head)."""
    groups, n, _ = k16.shape
    out = []
    step = 1 << 17
    for g in range(groups):
        qg = q[g].astype(np.float64)
        s = np.empty((qg.shape[0], n))
        for a in range(0, n, step):
            s[:, a:a + step] = qg @ k16[g, a:a + step].astype(np.float64).T
        out.extend(exact_topk(s[h], k) for h in range(qg.shape[0]))
    return out


def roofline_of(T, A, G, n, scan_ms):
    """Algorithmic bytes and ALU work of one scan launch over the plans' code
    bits T and active channels A (arrays over groups), against its time."""
    nb = n // 64
    bytes_per_launch = float((T * nb * 8 + A * nb * 2).sum()) + T.size * G * n * 4
    # one integer op per plane bit and token, one fp32 multiply-add per
    # active channel, token and query head
    int_ops = float(T.sum()) * nb * 64
    fma_ops = float((G * A).sum()) * nb * 64
    s = scan_ms / 1e3
    t_hbm = bytes_per_launch / (HBM_PEAK_GBPS * 1e9)
    t_alu = int_ops / (INT_PEAK_TOPS * 1e12) + fma_ops / (FMA_PEAK_TOPS * 1e12)
    return {
        "bytes": bytes_per_launch, "int_ops": int_ops, "fma_ops": fma_ops,
        "t_hbm_ms": t_hbm * 1e3, "t_alu_ms": t_alu * 1e3,
        "alu_peak": (int_ops + fma_ops) / t_alu / 1e12,
        "alu_tops": (int_ops + fma_ops) / s / 1e12,
        "alu_frac": t_alu / s, "hbm_gbps": bytes_per_launch / s / 1e9,
        "hbm_frac": t_hbm / s, "bound": "alu" if t_alu >= t_hbm else "hbm",
    }


def host_info():
    """What the host offers the CPU baseline: logical CPUs, the ones this
    process may run on, model name and sockets (from /proc/cpuinfo)."""
    info = {"logical_cpus": os.cpu_count()}
    try:
        info["affinity_cpus"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        info["affinity_cpus"] = os.cpu_count()
    model, sockets, cores = None, set(), {}
    try:
        phys = None
        for line in open("/proc/cpuinfo"):
            if ":" not in line:
                continue
            key, val = (x.strip() for x in line.split(":", 1))
            if key == "model name" and model is None:
                model = val
            elif key == "physical id":
                phys = val
                sockets.add(val)
            elif key == "cpu cores" and phys is not None:
                cores[phys] = int(val)
    except OSError:
        pass
    info["cpu_model"] = model
    info["sockets"] = len(sockets) or None
    info["physical_cores"] = sum(cores.values()) or None
    return info


def run_sweep(args):
    """Budgets 32..256 over layers of the 1M-key shape with needles: per
    budget, recall of the top-k against the top-k of exact fp64 scores over
    the fp16 keys, needle recall, plan sizes and the scan's event time."""
    import torch

    import fathom_inputs
    import sparse_top_kv_fathom_amd as fk

    layers = (list(range(fathom_inputs.SWEEP_LAYERS)) if args.layers == "all"
              else [int(x) for x in args.layers.split(",")])
    budgets = fathom_inputs.SWEEP_BUDGETS
    w = fathom_inputs.WORKLOADS["q1m"]
    H, G, n, d, k = w.groups, w.G, w.n, w.d, fathom_inputs.SWEEP_K
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ws = fk.topk_workspace(H * G, n, k, dev)
    scores = torch.empty((H, G, n), dtype=torch.float32, device=dev)
    idx = torch.empty((H * G, k), dtype=torch.int32, device=dev)
    depths = torch.empty((H, d), dtype=torch.uint8, device=dev)
    acc = {B: {"recall": [], "needle_own": [], "needle_all": [], "scan_ms": [], "topk_ms": [],
               "T": [], "A": []} for B in budgets}
    for L in layers:
        t0 = time.perf_counter()
        ins = fathom_inputs.sweep_inputs(L)
        pos = ins.extra["needles"]
        kd = torch.from_numpy(ins.k).to(dev)
        planes, scales = fk.encode(kd)
        del kd
        q_d, var_d = torch.from_numpy(ins.q).to(dev), torch.from_numpy(ins.var).to(dev)
        exact = exact_topk_rows(ins.k, ins.q, k)
        for B in budgets:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            for rep in range(3):   # the last repetition is timed
                fk.plan(q_d, var_d, B, depths=depths)
                ev[0].record()
                fk.scan(planes, scales, depths, q_d, n, scores=scores)
                ev[1].record()
                fk.topk(scores, k, indices=idx, workspace=ws)
                ev[2].record()
            torch.cuda.synchronize()
            got = idx.cpu().numpy()
            T, A = plan_stats(depths.cpu().numpy())
            a = acc[B]
            a["scan_ms"].append(ev[0].elapsed_time(ev[1]))
            a["topk_ms"].append(ev[1].elapsed_time(ev[2]))
            a["T"].extend(T.tolist())
            a["A"].extend(A.tolist())
            for r in range(H * G):
                g, h = divmod(r, G)
                sel = got[r]
                a["recall"].append(np.intersect1d(sel, exact[r], assume_unique=True).size / k)
                own = pos[g][h::G]
                a["needle_own"].append(np.isin(own, sel).mean())
                a["needle_all"].append(np.isin(pos[g], sel).mean())
        del planes, scales
        print("[sweep] layer %d done in %.1f s" % (L, time.perf_counter() - t0), file=sys.stderr,
              flush=True)
    rows = []
    for B in budgets:
        a = acc[B]
        scan_ms = float(np.mean(a["scan_ms"]))
        rows.append({
            "budget_bits": B,
            "code_bits_mean": float(np.mean(a["T"])),
            "total_bits_mean": float(np.mean(np.array(a["T"]) + np.array(a["A"]) / 4.0)),
            "active_channels_mean": float(np.mean(a["A"])),
            "recall_mean": float(np.mean(a["recall"])),
            "recall_min": float(np.min(a["recall"])),
            "needle_recall_own_head": float(np.mean(a["needle_own"])),
            "needle_recall_all": float(np.mean(a["needle_all"])),
            "scan_ms": round(scan_ms, 4),
            "topk_ms": round(float(np.mean(a["topk_ms"])), 4),
            "keys_per_s": H * n / (scan_ms / 1e3),
        })
    print(json.dumps({
        "sweep": "budget sweep, 1M keys x 8 KV heads per layer, G=%d, k=%d, %d needles per KV "
                 "head (cosine %.1f); recall against the top-k of exact fp64 scores over the "
                 "fp16 keys" % (G, k, fathom_inputs.SWEEP_NEEDLES, fathom_inputs.SWEEP_COSINE),
        "layers": layers, "data": "synthetic", "rows": rows}))


def timed_scans(fk, stores, depths_of, q_of, n, reps, scores):
    """Scan event times (ms) over `reps` launches rotating through the store
    copies, each through fathom_scan_timed (the kernels' own timestamps)."""
    import torch
    evs = [[TimingEvent() for _ in range(2)] for _ in range(reps)]
    torch.cuda.synchronize()
    for i in range(reps):
        p, s = stores[i % len(stores)]
        fk.scan(p, s, depths_of(i), q_of(i), n, scores=scores, events=(evs[i][0].h, evs[i][1].h))
    torch.cuda.synchronize()
    return [e[0].elapsed_time(e[1]) for e in evs]


def run_configs(fk, args, main_ctx):
    """The other workloads and budgets: scan (event-timed) and top-k medians,
    roofline fractions and keys/s, per (workload, budget)."""
    import torch

    import fathom_inputs
    out = []
    reps = max(10, min(args.steps, 30))
    dev = torch.device("cuda:0")
    todo = [("q256k", (68, 92, 136)), ("q1m", (68, 136)), ("s16", (92,))]
    for name, budgets in todo:
        w = fathom_inputs.WORKLOADS[name]
        H, G, n, d, k = w.groups, w.G, w.n, w.d, w.k
        t0 = time.perf_counter()
        if name == args.workload and main_ctx is not None:
            stores, qs_d, var_d = main_ctx["stores"], main_ctx["q_d"], main_ctx["var_d"]
        else:
            ins = fathom_inputs.make_inputs(H, G, n, w.seed)
            qs = np.stack([fathom_inputs.make_queries(H, G, 1000 + i, d) for i in range(4)])
            kd = torch.from_numpy(ins.k).to(dev)
            del ins.k
            ncop = max(1, min(4, int(2.2e9 // (H * n * 68)) + 1))
            stores = [fk.encode(kd) for _ in range(ncop)]
            del kd
            qs_d = torch.from_numpy(qs).to(dev)
            var_d = torch.from_numpy(ins.var).to(dev)
        nq = qs_d.shape[0]
        scores = torch.empty((H, G, n), dtype=torch.float32, device=dev)
        idx = torch.empty((H * G, k), dtype=torch.int32, device=dev)
        ws = fk.topk_workspace(H * G, n, k, dev)
        for B in budgets:
            deps = [fk.plan(qs_d[i], var_d, B) for i in range(nq)]
            timed_scans(fk, stores, lambda i: deps[i % nq], lambda i: qs_d[i % nq], n, 3, scores)
            sc = timed_scans(fk, stores, lambda i: deps[i % nq], lambda i: qs_d[i % nq], n, reps,
                             scores)
            tev = [[TimingEvent() for _ in range(2)] for _ in range(reps)]
            for i in range(reps):
                tev[i][0].record()
                fk.topk(scores, k, indices=idx, workspace=ws)
                tev[i][1].record()
            torch.cuda.synchronize()
            tk = [e[0].elapsed_time(e[1]) for e in tev]
            TA = [plan_stats(x.cpu().numpy()) for x in deps]
            T = np.mean([x[0] for x in TA], axis=0)
            A = np.mean([x[1] for x in TA], axis=0)
            med = float(np.median(sc))
            rf = roofline_of(T, A, G, n, med)
            out.append({
                "workload": name, "budget_bits": B, "kv_heads": H, "G": G, "n": n, "k": k,
                "scan_ms": stats(sc), "topk_ms": stats(tk),
                "scan_keys_per_s": H * n / (med / 1e3),
                "code_bits_mean": float(T.mean()), "active_channels_mean": float(A.mean()),
                "roofline_bound": rf["bound"], "alu_frac": round(rf["alu_frac"], 4),
                "hbm_frac": round(rf["hbm_frac"], 4), "hbm_GBps": round(rf["hbm_gbps"], 1),
            })
        del stores, scores, ws
        torch.cuda.empty_cache()
        print("[bench] configs %s done in %.1f s" % (name, time.perf_counter() - t0),
              file=sys.stderr, flush=True)
    return out


def run_layouts(fk, args, ctx, ins):
    """Store layouts and row lengths off the main kernel's 16-byte path: the
    scan on a copy of the store with capacity n/64 + 3 blocks (scale rows not
    16-byte aligned) beside the store itself, fathom_scan_topk on a ragged
    row length (whole rounds plus a tail) beside scan then top-k, and
    fathom_scan_topk on a store whose top keys crowd into one round beside
    the plain store.  Event medians in ms."""
    import torch
    stores, q_d, var_d, n, k, B = (ctx["stores"], ctx["q_d"], ctx["var_d"], ctx["n"], ctx["k"],
                                   ctx["B"])
    dev = q_d.device
    reps = max(10, min(args.steps, 30))
    H, G = q_d.shape[1], q_d.shape[2]
    nb = n // 64
    p0, s0 = stores[0]
    p3, s3 = fk.empty_store(H, nb + 3, dev)
    p3[..., :nb].copy_(p0)
    s3[..., :nb].copy_(s0)
    depths = fk.plan(q_d[0], var_d, B)
    scores = torch.empty((H, G, n), dtype=torch.float32, device=dev)
    out = {}
    odd = {}
    for tag, (pp, ss) in (("aligned", (p0, s0)), ("odd", (p3, s3))):
        timed_scans(fk, [(pp, ss)], lambda i: depths, lambda i: q_d[0], n, 3, scores)
        odd[tag] = stats(timed_scans(fk, [(pp, ss)], lambda i: depths, lambda i: q_d[0], n, reps,
                                     scores))
    out["odd_capacity"] = {"nb_store": nb + 3, "scan_ms": odd["odd"],
                           "scan_ms_nb_store_n_over_64": odd["aligned"]}
    nr = n - 64 * 37
    idx = torch.empty((H * G, k), dtype=torch.int32, device=dev)
    fws = fk.scan_topk_workspace(H, G, nr, k, dev)
    tws = fk.topk_workspace(H * G, nr, k, dev)
    sr = torch.empty((H, G, nr), dtype=torch.float32, device=dev)

    def timed(fn):
        for _ in range(3):
            fn()
        evs = [[TimingEvent() for _ in range(2)] for _ in range(reps)]
        for i in range(reps):
            evs[i][0].record()
            fn()
            evs[i][1].record()
        torch.cuda.synchronize()
        return stats([e[0].elapsed_time(e[1]) for e in evs])

    out["ragged_n"] = {
        "n": nr,
        "fused_scan_topk_ms": timed(lambda: fk.scan_topk(p0, s0, depths, q_d[0], nr, k,
                                                         indices=idx, workspace=fws,
                                                         write_scores=False)),
        "separate_scan_topk_ms": timed(lambda: (fk.scan(p0, s0, depths, q_d[0], nr, scores=sr),
                                                fk.topk(sr, k, indices=idx, workspace=tws))),
    }
    del p3, s3, fws, tws, sr
    # Top keys crowded into one stretch of each row: 420 keys aligned with
    # the group's queries inside the last 2048-key round (the sample reads
    # none of it), the round re-encoded into a copy of the store.
    width, r0 = 420, n - 2048
    kr = ins.k[:, r0:, :].copy()
    q0 = ctx["qs"][0]
    rng = np.random.default_rng(7)
    for g in range(H):
        qn = q0[g].astype(np.float64).sum(axis=0)
        qn /= np.abs(qn).max()
        top = 4.0 * float(np.abs(ins.k[g]).max())
        mag = top * rng.uniform(0.5, 1.0, width)
        kr[g, 512:512 + width] = (mag[:, None] * qn[None, :]).astype(np.float16)
    pc, sc = p0.clone(), s0.clone()
    fk.encode(torch.from_numpy(kr).to(dev), planes=pc, scales=sc, block_offset=r0 // 64)
    fws = fk.scan_topk_workspace(H, G, n, k, dev)
    tws = fk.topk_workspace(H * G, n, k, dev)
    idx2 = torch.empty((H * G, k), dtype=torch.int32, device=dev)
    fused_c = timed(lambda: fk.scan_topk(pc, sc, depths, q_d[0], n, k, indices=idx,
                                         workspace=fws, write_scores=False))
    fused_p = timed(lambda: fk.scan_topk(p0, s0, depths, q_d[0], n, k, indices=idx2,
                                         workspace=fws, write_scores=False))
    fk.scan(pc, sc, depths, q_d[0], n, scores=scores)
    fk.topk(scores, k, indices=idx2, workspace=tws)
    fk.scan_topk(pc, sc, depths, q_d[0], n, k, indices=idx, workspace=fws, write_scores=False)
    torch.cuda.synchronize()
    out["clustered"] = {"window_keys": width, "round_first_key": r0,
                        "fused_scan_topk_ms": fused_c, "fused_scan_topk_ms_plain_store": fused_p,
                        "indices_equal_scan_then_topk": bool(torch.equal(idx, idx2))}
    del pc, sc, fws, tws, scores, idx2
    torch.cuda.empty_cache()
    return out


def run_compare(fk, args, ctx, ins):
    """The pages' comparison reads through the same store, scan and top-k at
    the main workload: Fathom at several budgets, SparQ's top-r channels at
    r = 16 and 32 (68 and 136 bits with scales), the 2-bit thumbnail and the
    full 4-bit read; scan time and recall against the exact top-k."""
    import torch
    stores, q_d, var_d, n, k = ctx["stores"], ctx["q_d"], ctx["var_d"], ctx["n"], ctx["k"]
    H, G = q_d.shape[1], q_d.shape[2]
    nq = q_d.shape[0]
    reps = max(10, min(args.steps, 30))
    dev = q_d.device
    scores = torch.empty((H, G, n), dtype=torch.float32, device=dev)
    idx = torch.empty((H * G, k), dtype=torch.int32, device=dev)
    ws = fk.topk_workspace(H * G, n, k, dev)
    exact = exact_topk_rows(ins.k, ctx["qs"][0], k)
    plans = [("fathom", B, lambda i, B=B: fk.plan(q_d[i], var_d, B)) for B in (48, 68, 92, 136)]
    plans += [("sparq", r, lambda i, r=r: fk.plan_fixed("sparq", r, q=q_d[i])) for r in (16, 32)]
    plans += [("thumbnail_2bit", 2, lambda i: fk.plan_fixed("uniform", 2, groups=H, G=G)),
              ("full_4bit", 4, lambda i: fk.plan_fixed("uniform", 4, groups=H, G=G))]
    rows = []
    for name, param, mk in plans:
        deps = [mk(i) for i in range(nq)]
        timed_scans(fk, stores, lambda i: deps[i % nq], lambda i: q_d[i % nq], n, 3, scores)
        sc = timed_scans(fk, stores, lambda i: deps[i % nq], lambda i: q_d[i % nq], n, reps, scores)
        p, s = stores[0]
        fk.scan(p, s, deps[0], q_d[0], n, scores=scores)
        fk.topk(scores, k, indices=idx, workspace=ws)
        got = idx.cpu().numpy()
        rec = [np.intersect1d(got[r], exact[r], assume_unique=True).size / k for r in range(H * G)]
        TA = [plan_stats(x.cpu().numpy()) for x in deps]
        T = np.mean([x[0] for x in TA], axis=0)
        A = np.mean([x[1] for x in TA], axis=0)
        med = float(np.median(sc))
        rows.append({"plan": name, "param": param, "scan_ms": stats(sc),
                     "scan_keys_per_s": H * n / (med / 1e3),
                     "code_bits_mean": float(T.mean()),
                     "total_bits_mean": float((T + A / 4.0).mean()),
                     "recall_mean": round(float(np.mean(rec)), 4),
                     "recall_min": round(float(np.min(rec)), 4),
                     "alu_frac": round(roofline_of(T, A, G, n, med)["alu_frac"], 4)})
    return {"workload": ctx["name"], "k": k,
            "recall": "|top-k of the plan's scores & top-k of exact fp64 scores over the fp16 "
                      "keys| / k per query head, query group 0",
            "rows": rows}


def run_gather(fk, args, ctx):
    """fathom_gather from pinned host memory: the runs of the step's plans
    (B as benchmarked) at the main workload, and GB/s against contiguous run
    size (every channel at depth 4, so a channel's run is 4 * n / 8 bytes:
    4 KB at n = 8192 ... 512 KB at n = 2^20), each beside a contiguous pinned
    copy of the same byte count."""
    import torch
    stores, q_d, var_d, n, B = ctx["stores"], ctx["q_d"], ctx["var_d"], ctx["n"], ctx["B"]
    H = q_d.shape[1]
    nb = n // 64
    reps = 10
    dev = q_d.device

    def copy_rate(nbytes, hsrc, ddst):
        """GB/s of one contiguous pinned-to-device copy of nbytes (at most the
        size of the two buffers)."""
        m = min(nbytes // 8, hsrc.numel() * hsrc.element_size() // 8,
                ddst.numel() * ddst.element_size() // 8)
        nbytes = m * 8
        src = hsrc.view(torch.int64).view(-1)[:m]
        dst = ddst.view(torch.int64).view(-1)[:m]
        dst.copy_(src, non_blocking=True)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            dst.copy_(src, non_blocking=True)
        ev[1].record()
        torch.cuda.synchronize()
        return nbytes / (ev[0].elapsed_time(ev[1]) / reps / 1e3) / 1e9

    def gather_ms(hp, hs, dep, nn, gp, gs):
        fk.gather(hp, hs, dep, nn, gp, gs)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            fk.gather(hp, hs, dep, nn, gp, gs)
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    hp = stores[0][0].view(torch.int64).cpu().pin_memory().view(torch.uint64)
    hs = stores[0][1].view(torch.int16).cpu().pin_memory().view(torch.uint16)
    gp, gs = fk.empty_store(H, nb, dev)
    deps = [fk.plan(q_d[i % q_d.shape[0]], var_d, B) for i in range(4)]
    g_ms = float(np.mean([gather_ms(hp, hs, dp, n, gp, gs) for dp in deps]))
    g_bytes = float(np.mean([(lambda T, A: (T * nb * 8 + A * nb * 2).sum())(
        *plan_stats(x.cpu().numpy())) for x in deps]))
    step = {"ms": round(g_ms, 4), "bytes_per_call": int(g_bytes),
            "host_GBps": round(g_bytes / (g_ms / 1e3) / 1e9, 2),
            "contiguous_copy_GBps": round(copy_rate(int(g_bytes) // 8 * 8, hp, gp), 2),
            "source": "pinned host store, all %d groups, the step's plans at B=%d" % (H, B)}
    curve = []
    full = fk.plan_fixed("uniform", 4, groups=H, G=q_d.shape[2])
    for nn in [8192 << i for i in range(8)]:
        if nn > n:
            break
        nbs = nn // 64
        # a store of exactly nn keys per channel: a channel's 4 planes are one run
        shp = (H, 128, 4, nbs)
        hpp = torch.empty(shp, dtype=torch.int64, pin_memory=True)
        hpp.copy_(stores[0][0].view(torch.int64)[..., :nbs])
        hss = torch.empty((H, 128, nbs), dtype=torch.int16, pin_memory=True)
        hss.copy_(stores[0][1].view(torch.int16)[..., :nbs])
        dpp, dss = fk.empty_store(H, nbs, dev)
        ms = gather_ms(hpp.view(torch.uint64), hss.view(torch.uint16), full, nn, dpp, dss)
        nbytes = H * 128 * (4 * nbs * 8 + nbs * 2)
        curve.append({"run_bytes": 4 * nbs * 8, "n": nn, "bytes": nbytes,
                      "gather_GBps": round(nbytes / (ms / 1e3) / 1e9, 2),
                      "contiguous_copy_GBps": round(copy_rate(nbytes // 8 * 8, hpp, dpp), 2)})
        del hpp, hss, dpp, dss
    del hp, hs, gp, gs
    return {"step": step, "by_run_size": curve}


def cpu_baseline(args, ins, qs, H, G, n, k, B):
    """The CPU oracle as it stands, timed on this host: one full decode step
    of the workload on all threads, and the same step for one KV head on one
    thread (the step's work per key is the same for every head)."""
    import oracle
    info = host_info()
    nthreads = info["affinity_cpus"] or 1
    nb = n // 64
    res = {}
    for label, groups, th in (("all_threads", H, nthreads), ("one_thread", 1, 1)):
        kk = np.ascontiguousarray(ins.k[:groups])
        var = np.ascontiguousarray(ins.var[:groups])
        op, os_, _ = oracle.encode(kk, nthreads=nthreads)            # resident store (setup)
        kb = np.ascontiguousarray(kk[:, n - 64:, :])
        steps, spent = 0, 0.0
        while steps < 3 and (steps == 0 or spent < 10.0):
            qh = np.ascontiguousarray(qs[steps % len(qs)][:groups])
            t0 = time.perf_counter()
            oracle.encode(kb, nb_store=nb, block_offset=nb - 1, planes=op, scales=os_, nthreads=th)
            od, _, _ = oracle.plan(qh, var, B, nthreads=th)
            sc = oracle.scan_ref32(op, os_, od, qh, n, nthreads=th)
            oracle.topk(sc.reshape(-1, n), k, nthreads=th)
            spent += time.perf_counter() - t0
            steps += 1
        res[label] = {"value": steps * groups * n / spent, "threads": th,
                      "sample": "%d decode step(s) of %d KV head(s) x %d keys (1-block encode, "
                                "plan, fp32 scan, full-sort top-k), %.1f s"
                                % (steps, groups, n, spent)}
        print("[bench] cpu baseline %s: %.3g keys/s" % (label, res[label]["value"]),
              file=sys.stderr, flush=True)
    a = res["all_threads"]
    return {"value": a["value"], "unit": "keys/s", "cores": a["threads"], "kind": "oracle",
            "sample": a["sample"], "threads": a["threads"],
            "host_logical_cpus": info["logical_cpus"], "host_physical_cores": info["physical_cores"],
            "cpu_model": info["cpu_model"], "sockets": info["sockets"],
            "one_thread": res["one_thread"]}


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        run_sweep(args)
        return

    import torch

    import fathom_inputs
    import sparse_top_kv_fathom_amd as fk

    w = fathom_inputs.WORKLOADS[args.workload]
    H, G, n, d, k, B = w.groups, w.G, w.n, w.d, w.k, args.budget
    nb = n // 64
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("[bench] generating %s: H=%d G=%d n=%d B=%d k=%d" % (w.name, H, G, n, B, k),
          file=sys.stderr, flush=True)
    ins = fathom_inputs.make_inputs(H, G, n, w.seed)
    qs = np.stack([fathom_inputs.make_queries(H, G, 1000 + i, d) for i in range(args.queries)])

    k_d = torch.from_numpy(ins.k).to(dev)
    q_d = torch.from_numpy(qs).to(dev)
    var_d = torch.from_numpy(ins.var).to(dev)

    # KLT-rotated store: the fit on the keys themselves, the key rotation and
    # one query rotation, each timed with events (one-time costs, outside
    # the step).
    klt, basis_k, src = None, None, k_d
    if args.store == "klt" or not args.no_klt:
        kws = fk.klt_fit_workspace(H, n, dev)
        mu_k, basis_k, lam_k = fk.klt_fit(k_d, kws)
        kr = fk.klt_rotate_keys(k_d, mu_k, basis_k)
        qr = fk.klt_rotate_queries(q_d[0], basis_k)
        ts = {}
        for name, fn, reps in (("fit_ms", lambda: fk.klt_fit(k_d, kws), 3),
                               ("rotate_keys_ms", lambda: fk.klt_rotate_keys(k_d, mu_k, basis_k,
                                                                             out=kr), 3),
                               ("rotate_queries_ms", lambda: fk.klt_rotate_queries(
                                   q_d[0], basis_k, out=qr), 10)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ts[name] = round(e0.elapsed_time(e1) / reps, 4)
        klt = dict(ts, keys=H * n, groups=H)
        if args.store == "klt":
            src, var_d = kr, lam_k
        else:
            del kr, basis_k
            basis_k = None
        del kws

    # Resident store copies, encoded on the GPU; the full-store encode timed.
    stores = [fk.encode(src)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.copies - 1):
        stores.append(fk.encode(src))
    e1.record()
    torch.cuda.synchronize()
    encode_full_ms = e0.elapsed_time(e1) / max(1, args.copies - 1)
    newest = src[:, n - 64:, :].contiguous()            # the block each step re-encodes
    del k_d, src
    qrot = torch.empty((H, G, d), dtype=torch.float32, device=dev)

    def query(i):
        """Query group i as the plan and scan take it (rotated for the KLT store)."""
        q = q_d[i % args.queries]
        return q if basis_k is None else fk.klt_rotate_queries(q, basis_k, out=qrot)
    depths = torch.empty((H, d), dtype=torch.uint8, device=dev)
    scores = torch.empty((H, G, n), dtype=torch.float32, device=dev)
    idx = torch.empty((H * G, k), dtype=torch.int32, device=dev)
    ws = fk.topk_workspace(H * G, n, k, dev)
    fws = fk.scan_topk_workspace(H, G, n, k, dev)
    torch.cuda.synchronize()

    def step(s, ev=None, scan_ev=None, mode="separate"):
        """One decode step: append the newest block and plan (fathom_append_plan;
        fathom_encode and fathom_plan in the stage pass), scan, select.
        mode "fused": the scan and the selection as fathom_scan_topk without a
        score buffer; "separate": fathom_scan then fathom_topk.
        ev: five events between the stages (separate mode); scan_ev: two
        events that fathom_scan_timed records from the scan kernels' own
        timestamps."""
        planes, scales = stores[s % len(stores)]
        q = query(s)
        if ev is None:   # the append and the plan as one call (one launch)
            fk.append_plan(newest, planes, scales, nb - 1, q, var_d, B, depths=depths)
        else:            # the stage pass times them apart
            ev[0].record()
            fk.encode(newest, planes, scales, block_offset=nb - 1)
            ev[1].record()
            fk.plan(q, var_d, B, depths=depths)
            ev[2].record()
        if mode == "fused":
            fk.scan_topk(planes, scales, depths, q, n, k, indices=idx, workspace=fws,
                         write_scores=False)
            return
        if scan_ev is not None:   # the scan kernels' own start and end timestamps
            fk.scan(planes, scales, depths, q, n, scores=scores,
                    events=(scan_ev[0].h, scan_ev[1].h))
        else:
            fk.scan(planes, scales, depths, q, n, scores=scores)
        if ev is not None:
            ev[3].record()
        fk.topk(scores, k, indices=idx, workspace=ws)
        if ev is not None:
            ev[4].record()

    def fused(s, ev, write_scores):
        """The scan and selection as the one call fathom_scan_topk."""
        planes, scales = stores[s % len(stores)]
        q = query(s)
        fk.plan(q, var_d, B, depths=depths)
        ev[0].record()
        fk.scan_topk(planes, scales, depths, q, n, k, scores=scores, indices=idx, workspace=fws,
                     write_scores=write_scores)
        ev[1].record()

    # Plain copy of known size, for scaling HBM byte counters (untimed).
    calib_src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    calib_dst = torch.empty_like(calib_src)
    for _ in range(3):
        torch.neg(calib_src, out=calib_dst)
    del calib_src, calib_dst

    def plain_pass(mode):
        """W warm-up steps, then K steps between two events, nothing between
        the calls: (ms per step, host wall seconds)."""
        for s in range(args.warmup):
            step(s, mode=mode)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        start.record()
        for s in range(args.steps):
            step(args.warmup + s, mode=mode)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps, time.perf_counter() - wall0

    # The headline pass in the chosen step mode, then the other mode.
    other = "separate" if args.step_mode == "fused" else "fused"
    ms_per_step, wall = plain_pass(args.step_mode)
    ms_other, _ = plain_pass(other)
    print("[bench] %s steps %.4f ms, %s steps %.4f ms" % (args.step_mode, ms_per_step, other,
                                                       ms_other), file=sys.stderr, flush=True)

    # The scan pass: the same steps with every scan through fathom_scan_timed.
    sevs = [[TimingEvent() for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        step(args.warmup + s, scan_ev=sevs[s])
    torch.cuda.synchronize()
    scan_list = [e[0].elapsed_time(e[1]) for e in sevs]
    scan_st = stats(scan_list)

    # The stage pass: events between all stages.
    evs = [[TimingEvent() for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        step(args.warmup + s, evs[s])
    torch.cuda.synchronize()
    stage = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in evs])
    step_list = [e[0].elapsed_time(e[4]) for e in evs]

    # The fused call on the same inputs, with and without a score buffer.
    fused_st = {}
    for ws_flag in (True, False):
        for s in range(args.warmup):
            fused(s, [TimingEvent() for _ in range(2)], ws_flag)
        fev = [[TimingEvent() for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for s in range(args.steps):
            fused(args.warmup + s, fev[s], ws_flag)
        torch.cuda.synchronize()
        fused_st["scores_written" if ws_flag else "no_scores"] = stats(
            [e[0].elapsed_time(e[1]) for e in fev])
    print("[bench] passes done: %.4f ms/step, scan median %.4f ms"
          % (ms_per_step, scan_st["median"]), file=sys.stderr, flush=True)

    # Algorithmic work of each timed step's scan (plans recomputed after timing).
    Ts, As = [], []
    for s in range(args.steps):
        dep = fk.plan(query(args.warmup + s), var_d, B)
        T, A = plan_stats(dep.cpu().numpy())
        Ts.append(T)
        As.append(A)
    Ts, As = np.array(Ts), np.array(As)
    rf = roofline_of(Ts.mean(axis=0), As.mean(axis=0), G, n, scan_st["median"])
    traffic = recorded_counter(TRAFFIC_FILE, "scan_hbm_bytes_per_launch")
    if rf["bound"] == "alu":
        roof = {"bound": "alu", "achieved": round(rf["alu_tops"], 3),
                "peak": round(rf["alu_peak"], 2), "unit": "Tlane-op/s",
                "frac": round(rf["alu_frac"], 4), "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": round(rf["hbm_gbps"], 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(rf["hbm_frac"], 4), "traffic": traffic}
    valu = recorded_counter(INSTR_FILE, "scan_valu_instructions_per_launch")
    scan_s = scan_st["median"] / 1e3
    roof.update({
        "kernel": "scan_main",
        "traffic_unit": "HBM bytes per launch (read requests by size + write requests)",
        "traffic_read_bytes": recorded_counter(TRAFFIC_FILE, "scan_hbm_read_bytes_per_launch"),
        "traffic_fetch_write_size": recorded_counter(TRAFFIC_FILE,
                                                     "scan_fetch_write_bytes_per_launch"),
        "traffic_over_algorithmic": (None if traffic is None else
                                     round(traffic / rf["bytes"], 4)),
        "launch_ms": scan_st["median"],
        "launch_time": "median of the scan pass's event-timed launches",
        "alg_bytes_per_launch": int(rf["bytes"]),
        "alg_int_ops_per_launch": int(rf["int_ops"]),
        "alg_fma_ops_per_launch": int(rf["fma_ops"]),
        "alu_bound_ms": round(rf["t_alu_ms"], 4),
        "hbm_bound_ms": round(rf["t_hbm_ms"], 4),
        "hbm_GBps": round(rf["hbm_gbps"], 1), "hbm_frac": round(rf["hbm_frac"], 4),
        "alu_frac_target": 0.70,
        "valu_instructions_per_launch": valu,
        "valu_issue_frac": (None if valu is None else
                            round(valu / (scan_s * CUS * CLOCK_GHZ * 1e9), 4)),
    })

    keys = H * n
    value = keys / (ms_per_step / 1e3)
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "%s: %s, G=%d, d=%d, B=%d code bits, k=%d%s" % (
                w.name, w.note, G, d, B, k,
                ", KLT-rotated store" if args.store == "klt" else ""),
            "store": args.store,
            "kv_heads": H, "G": G, "n": n, "budget_bits": B, "k": k,
            "store_copies": args.copies, "parallelism": "single GPU",
        },
        "step_mode": args.step_mode,
        "step_mode_note": ("fused: the scan and the selection as fathom_scan_topk without a "
                           "score buffer; separate: fathom_scan then fathom_topk"),
        "ms_per_step_%s" % other: ms_other,
        "scan_keys_per_s": keys / scan_s,
        "scan_ms": scan_st,
        "step_ms": stats(step_list),
        "stages_ms": {"encode_block": stats(stage[:, 0]), "plan": stats(stage[:, 1]),
                      "scan": stats(stage[:, 2]), "topk": stats(stage[:, 3]),
                      "note": "a pass of the steps with events between the stages"},
        "fused_scan_topk_ms": fused_st,
        "separate_scan_topk_ms": stats(stage[:, 2] + stage[:, 3]),
        "encode_full_store_ms": round(encode_full_ms, 4),
        "klt_store": klt,
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "plan": {"code_bits_mean": float(Ts.mean()), "active_channels_mean": float(As.mean()),
                 "total_bits_per_key_mean": float((Ts + As / 4.0).mean())},
        "roofline": roof,
    }

    ctx = {"name": w.name, "stores": stores, "q_d": q_d, "qs": qs, "var_d": var_d, "n": n,
           "k": k, "B": B}
    if not args.no_compare and args.store == "raw":
        out["layouts"] = run_layouts(fk, args, ctx, ins)
        print("[bench] layouts done", file=sys.stderr, flush=True)
        out["compare_plans"] = run_compare(fk, args, ctx, ins)
        print("[bench] fixed-plan comparison done", file=sys.stderr, flush=True)
    if not args.no_gather and args.store == "raw":
        out["gather_from_host"] = run_gather(fk, args, ctx)
        print("[bench] gather done", file=sys.stderr, flush=True)
    if not args.no_configs and args.store == "raw":
        del scores, ws, fws
        out["configs"] = run_configs(fk, args, ctx if w.name == "q1m" else None)
    del stores, ctx
    torch.cuda.empty_cache()

    if not args.no_cpu_baseline and args.store == "raw":
        out["cpu_baseline"] = cpu_baseline(args, ins, qs, H, G, n, k, B)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
