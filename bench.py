"""Benchmark of the Fathom decode-step hot path on one MI355X.

One step = the work of one decode step over a resident bit-plane store:
encode the newest 64-token block of every KV head into its slot, plan the
read depths for a fresh query group (importance, 30-step bisection), scan
every key at those depths, and select the top-k of every query head.  The
fused call fathom_scan_topk (the scan takes the top-k candidates itself) is
timed on the same inputs after the steps and reported beside them.

Workload (default): one Qwen3-8B-shaped layer, 8 KV heads x 4 query heads,
d = 128, n = 1,048,576 keys per head, budget 92 code bits, k = 4096; keys,
queries and variances from fathom_inputs (synthetic, seeded).  The store is
held in several copies that the steps rotate through, so the index a step
reads is not left in the 256 MB last-level cache by the previous step.

Prints one JSON line: keys scanned per second for the whole step (value),
plus the scan kernel's roofline figures (algorithmic bytes and VALU work per
launch, over its event-timed average duration) and the CPU oracle's rate on
a bounded sample.

HBM traffic of the scan comes from rocprofv3 counter runs of this same
command (FETCH_SIZE, then WRITE_SIZE), each scaled by the factor that makes
the counter agree with the known bytes of a plain copy (torch.neg over
256 MiB, run here before the timed steps).  The figures are kept in
profiles/scan_q1m_b92_traffic.txt together with the sha256 of the scan
source they were taken on; a different source reports traffic null.
`python bench.py --summarize DIR [DIR ...]` turns rocprofv3 csv output
(kernel stats, counter collections) into the text kept under profiles/.
"""
from __future__ import annotations

import argparse
import ctypes
import csv
import glob
import hashlib
import json
import os
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
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="q1m")
    ap.add_argument("--budget", type=int, default=92)
    ap.add_argument("--copies", type=int, default=4, help="store copies the steps rotate through")
    ap.add_argument("--queries", type=int, default=8, help="distinct query groups drawn")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--store", choices=("raw", "klt"), default="raw",
                    help="raw channel planes, or planes of the KLT-rotated keys")
    ap.add_argument("--no-klt", action="store_true",
                    help="skip timing the KLT fit and rotations (raw store only)")
    ap.add_argument("--no-gather", action="store_true",
                    help="skip timing fathom_gather from a pinned host store")
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


def recorded_traffic():
    """Scan HBM bytes per launch (scaled FETCH_SIZE + WRITE_SIZE)."""
    return recorded_counter(TRAFFIC_FILE, "scan_hbm_bytes_per_launch")


def recorded_valu():
    """Scan VALU instructions (wave64) per launch (SQ_INSTS_VALU)."""
    return recorded_counter(INSTR_FILE, "scan_valu_instructions_per_launch")


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
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"),
                                  recursive=True)):
            print("## counters: %s" % os.path.relpath(f, d))
            agg = {}
            for r in csv.DictReader(open(f)):
                key = (short_name(r["Kernel_Name"]), r["Counter_Name"])
                agg.setdefault(key, []).append(float(r["Counter_Value"]))
            print("%-60s %-14s %6s %14s" % ("kernel", "counter", "n", "mean"))
            for (kname, cname), v in sorted(agg.items()):
                print("%-60s %-14s %6d %14.1f" % (kname, cname, len(v), sum(v) / len(v)))
                means[(kname, cname)] = sum(v) / len(v)
    valu = [v for (kname, cname), v in means.items()
            if kname.startswith("fathom::scan_main<") and kname.endswith(", 0>") and cname == "SQ_INSTS_VALU"]
    if valu:
        print("scan_valu_instructions_per_launch: %.0f" % valu[0])
        print("scan_source_sha256: %s" % source_sha(SCAN_SRC))
    # HBM traffic of the scan: each byte counter (KiB per dispatch) scaled by
    # the factor that makes it read the known bytes of the plain copy.
    calib = [k for k in means if "neg" in k[0]]
    scan = [k for k in means if "scan_main" in k[0]]
    if calib and scan:
        total = 0.0
        print("## scan traffic (counters scaled by the plain-copy factor)")
        for cname, known_kib in (("FETCH_SIZE", CALIB_BYTES / 1024), ("WRITE_SIZE", CALIB_BYTES / 1024)):
            c = [means[k] for k in calib if k[1] == cname]
            sc = [means[k] for k in scan if k[1] == cname]
            if not c or not sc:
                return
            factor = known_kib / c[0]
            print("    %s: copy of %d KiB reads %.1f KiB -> factor %.4f; scan %.1f KiB -> %.0f bytes"
                  % (cname, known_kib, c[0], factor, sc[0], sc[0] * factor * 1024))
            total += sc[0] * factor * 1024
        print("scan_hbm_bytes_per_launch: %.0f" % total)
        print("scan_source_sha256: %s" % source_sha(SCAN_SRC))


def plan_stats(depths: np.ndarray):
    """Per group: code bits T = sum t_j and active channels A = #{t_j > 0}."""
    d = depths.astype(np.int64)
    return d.sum(axis=1), (d > 0).sum(axis=1)


def exact_topk(s: np.ndarray, k: int) -> np.ndarray:
    """The k largest of s, ties to the lower index (the selection's order),
    as sorted indices."""
    part = np.argpartition(-s, k - 1)[:k]
    kth = s[part].min()
    above = np.flatnonzero(s > kth)
    eq = np.flatnonzero(s == kth)
    return np.sort(np.concatenate([above, eq[:k - len(above)]]))


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
        exact = []
        for g in range(H):
            s = ins.q[g].astype(np.float64) @ ins.k[g].astype(np.float64).T
            exact.extend(exact_topk(s[h], k) for h in range(G))
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


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.sweep:
        if args.gpus != 1:
            print("bench.py runs on one GPU only (--gpus %d requested)" % args.gpus,
                  file=sys.stderr)
            sys.exit(2)
        run_sweep(args)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

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

    # Resident store copies, encoded on the GPU.
    stores = []
    for _ in range(args.copies):
        stores.append(fk.encode(src))
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
    torch.cuda.synchronize()

    fws = fk.scan_topk_workspace(H, G, n, k, dev)

    def step(s, ev=None, scan_ev=None):
        """One decode step: append the newest block, plan, scan, select.
        ev: five events between the stages; scan_ev: two events that
        fathom_scan_timed records from the scan kernels' own timestamps."""
        planes, scales = stores[s % len(stores)]
        if ev is not None:
            ev[0].record()
        fk.encode(newest, planes, scales, block_offset=nb - 1)
        if ev is not None:
            ev[1].record()
        q = query(s)
        fk.plan(q, var_d, B, depths=depths)
        if ev is not None:
            ev[2].record()
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

    def fused(s, ev):
        """The scan and selection as the one call fathom_scan_topk."""
        planes, scales = stores[s % len(stores)]
        q = query(s)
        fk.plan(q, var_d, B, depths=depths)
        ev[0].record()
        fk.scan_topk(planes, scales, depths, q, n, k, scores=scores, indices=idx, workspace=fws)
        ev[1].record()

    # Plain copy of known size, for scaling HBM byte counters (untimed).
    calib_src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    calib_dst = torch.empty_like(calib_src)
    for _ in range(3):
        torch.neg(calib_src, out=calib_dst)
    del calib_src, calib_dst

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    print("[bench] warmup done; timing %d steps" % args.steps, file=sys.stderr, flush=True)

    # The timed steps: the scan's launch time for the roofline comes from
    # events the scan kernels record themselves (fathom_scan_timed), so no
    # marker packet sits between the calls.
    sevs = [[TimingEvent() for _ in range(2)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for s in range(args.steps):
        step(args.warmup + s, scan_ev=sevs[s])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    scan_ms_timed = float(np.mean([e[0].elapsed_time(e[1]) for e in sevs]))

    # The same steps again with events between all stages, for the breakdown.
    evs = [[TimingEvent() for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        step(args.warmup + s, evs[s])
    torch.cuda.synchronize()
    stage = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in evs])
    stage_ms = stage.mean(axis=0)

    # The fused call on the same inputs, timed after the steps.
    for s in range(args.warmup):
        fused(s, [TimingEvent() for _ in range(2)])
    fev = [[TimingEvent() for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        fused(args.warmup + s, fev[s])
    torch.cuda.synchronize()
    fused_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in fev]))

    # fathom_gather: the runs each step's plan reads, copied from a pinned host
    # copy of the store into a device store (outside the step: the store the
    # step scans is resident).
    gather = None
    if not args.no_gather:
        hp = stores[0][0].view(torch.int64).cpu().pin_memory().view(torch.uint64)
        hs = stores[0][1].view(torch.int16).cpu().pin_memory().view(torch.uint16)
        gp, gs = fk.empty_store(H, nb, dev)
        gdep = [fk.plan(query(i), var_d, B) for i in range(args.steps)]
        for i in range(2):
            fk.gather(hp, hs, gdep[i], n, gp, gs)
        gev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            gev[i][0].record()
            fk.gather(hp, hs, gdep[i], n, gp, gs)
            gev[i][1].record()
        torch.cuda.synchronize()
        g_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in gev]))
        g_bytes = float(np.mean([(lambda T, A: (T * nb * 8 + A * nb * 2).sum())(
            *plan_stats(x.cpu().numpy())) for x in gdep]))
        # The host link's own rate: one contiguous pinned-to-device copy of
        # the same byte count.
        nbytes = int(g_bytes) // 8 * 8
        src = hp.view(torch.int64).view(-1)[: nbytes // 8]
        dst = gp.view(torch.int64).view(-1)[: nbytes // 8]
        dst.copy_(src, non_blocking=True)
        cev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        cev[0].record()
        for _ in range(args.steps):
            dst.copy_(src, non_blocking=True)
        cev[1].record()
        torch.cuda.synchronize()
        c_ms = cev[0].elapsed_time(cev[1]) / args.steps
        gather = {"ms": round(g_ms, 4), "bytes_per_call": int(g_bytes),
                  "host_GBps": round(g_bytes / (g_ms / 1e3) / 1e9, 2),
                  "contiguous_copy_GBps": round(nbytes / (c_ms / 1e3) / 1e9, 2),
                  "source": "pinned host store, all %d groups" % H}
        del src, dst
        del hp, hs, gp, gs

    # Algorithmic work of each timed step's scan (plans recomputed after timing).
    Ts, As = [], []
    for s in range(args.steps):
        dep = fk.plan(query(args.warmup + s), var_d, B)
        T, A = plan_stats(dep.cpu().numpy())
        Ts.append(T)
        As.append(A)
    Ts, As = np.array(Ts), np.array(As)
    bytes_per_launch = float(np.mean((Ts * nb * 8 + As * nb * 2).sum(axis=1))) + H * G * n * 4
    # Algorithmic ALU work: one integer op per plane bit and token, one fp32
    # multiply-add per active channel, token and query head.
    int_ops = float(np.mean(Ts.sum(axis=1))) * nb * 64
    fma_ops = float(np.mean((G * As).sum(axis=1))) * nb * 64
    ops_per_launch = int_ops + fma_ops
    scan_s = scan_ms_timed / 1e3
    hbm_gbps = bytes_per_launch / scan_s / 1e9
    t_hbm = bytes_per_launch / (HBM_PEAK_GBPS * 1e9)
    t_alu = int_ops / (INT_PEAK_TOPS * 1e12) + fma_ops / (FMA_PEAK_TOPS * 1e12)
    alu_peak = ops_per_launch / t_alu / 1e12         # the op mix's own peak rate
    alu_tops = ops_per_launch / scan_s / 1e12
    bound = "alu" if t_alu >= t_hbm else "hbm"
    traffic = recorded_traffic()
    if bound == "alu":
        roof = {"bound": "alu", "achieved": round(alu_tops, 3), "peak": round(alu_peak, 2),
                "unit": "Tlane-op/s", "frac": round(alu_tops / alu_peak, 4), "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": round(hbm_gbps, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(hbm_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic}
    roof.update({
        "kernel": "scan_main",
        "traffic_unit": "HBM bytes per launch (scaled FETCH_SIZE + WRITE_SIZE)",
        "launch_ms": round(scan_ms_timed, 4),
        "alg_bytes_per_launch": int(bytes_per_launch),
        "alg_int_ops_per_launch": int(int_ops),
        "alg_fma_ops_per_launch": int(fma_ops),
        "alu_bound_ms": round(t_alu * 1e3, 4),
        "hbm_bound_ms": round(t_hbm * 1e3, 4),
        "hbm_GBps": round(hbm_gbps, 1), "hbm_frac": round(hbm_gbps / HBM_PEAK_GBPS, 4),
    })
    # VALU issue: wave64 VALU instructions per launch (SQ_INSTS_VALU, from the
    # committed counter summary) over one issue per CU per clock.
    valu = recorded_valu()
    roof.update({
        "valu_instructions_per_launch": valu,
        "valu_issue_frac": (None if valu is None else
                            round(valu / (scan_s * CUS * CLOCK_GHZ * 1e9), 4)),
    })

    keys = H * n
    value = keys / (ms_per_step / 1e3)
    out = {
        "metric": "keys scanned/sec (and HBM GB/s, % roofline) at 1M keys, 92-bit budget",
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
        "stages_ms": {"encode_block": round(stage_ms[0], 4), "plan": round(stage_ms[1], 4),
                      "scan": round(stage_ms[2], 4), "topk": round(stage_ms[3], 4),
                      "note": "a second pass of the steps with events between the stages"},
        "fused_scan_topk_ms": round(fused_ms, 4),
        "gather_from_host": gather,
        "klt_store": klt,
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "plan": {"code_bits_mean": float(Ts.mean()), "active_channels_mean": float(As.mean()),
                 "total_bits_per_key_mean": float((Ts + As / 4.0).mean())},
        "roofline": roof,
    }

    if not args.no_cpu_baseline and args.store == "raw":
        import oracle
        nthreads = args.cpu_threads or min(H, os.cpu_count() or 1)
        print("[bench] cpu baseline: oracle step on %d threads" % nthreads, file=sys.stderr,
              flush=True)
        op, os_, _ = oracle.encode(ins.k, nthreads=nthreads)           # resident store (setup)
        kb = np.ascontiguousarray(ins.k[:, n - 64:, :])
        cpu_steps = 3
        t0 = time.perf_counter()
        for s in range(cpu_steps):
            qh = qs[(args.warmup + s) % args.queries]
            oracle.encode(kb, nb_store=nb, block_offset=nb - 1, planes=op, scales=os_,
                          nthreads=nthreads)
            od, _, _ = oracle.plan(qh, ins.var, B, nthreads=nthreads)
            sc = oracle.scan_ref32(op, os_, od, qh, n, nthreads=nthreads)
            oracle.topk(sc.reshape(-1, n), k, nthreads=nthreads)
        cpu_s = time.perf_counter() - t0
        out["cpu_baseline"] = {
            "value": cpu_steps * keys / cpu_s, "unit": "keys/s", "cores": nthreads,
            "kind": "oracle",
            "sample": "%d full decode steps of the same workload (1-block encode, plan, fp32 "
                      "scan of all %d keys, full-sort top-k), %.1f s" % (cpu_steps, keys, cpu_s),
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
