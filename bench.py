"""Benchmark of the ROSA retrieval hot path on one MI355X.

One step = the whole path over one batch: bf16 hidden states -> sign bits ->
4-bit route symbols (512 streams) -> longest-recurring-suffix match for all
65,536 positions of every stream (E and next symbol) -> gather of the matched
value slices from V.  Inputs are resident in HBM before timing starts.

Prints one JSON line: throughput in matched positions/s, the roofline of the
dominant kernel (the retrieval kernel, timed with HIP events on its own
stream), and the CPU oracle timed on the host as a reported baseline.  Every
output of the timed run is compared with the oracle before the line is
printed.

    python bench.py [--steps K] [--warmup W]
                    [--workload long|batched|repeat|decode] [--no-cpu]

The decode workload builds one automaton per stream over the long
workload's 65,536-position prefix, then appends 1024 positions with one
rosa_step each (extend + match + gather of the value row); it reports the
per-step latency (HIP events around every step) and positions/s over the
appended positions.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "matched positions/sec (streams×T) at T=64K, 512 streams"
HBM_PEAK = 8.0e12     # MI355X HBM3E, bytes/s
# Algorithmic bytes per stream-position of the retrieval kernel (streams of
# up to 65536 positions): the symbol read (1 B) and one 4-byte result record
# (position, E+1) written; a separate kernel puts the records in time order.
KERNEL_BYTES_PER_POS = 1 + 4
PMC_FILE = os.path.join(ROOT, "profiles", "stream_kernel_long_pmc.txt")


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("rosa_match.hip", "rosa_internal.h"):
        with open(os.path.join(ROOT, "online_suffix_automaton_amd", "csrc",
                               name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the retrieval kernel from the committed
    rocprofv3 counter summary, if it was taken on the current source."""
    try:
        txt = open(PMC_FILE).read()
    except OSError:
        return None
    m = re.search(r"^source_sha\s*=\s*(\w+)", txt, re.M)
    b = re.search(r"^traffic_bytes_per_launch\s*=\s*([0-9.eE+]+)", txt, re.M)
    if not m or not b or m.group(1) != kernel_source_hash():
        return None
    return float(b.group(1))


# ------------------------------------------------------------- workloads

def make_workload(name):
    from online_suffix_automaton_amd import synth
    if name == "long":
        w = synth.long()
        return dict(kind="bf16", H=w["H"], V=w["V"], M=4, S=512, T=65536,
                    metric=METRIC,
                    desc="long: hidden [1,65536,2048] bf16 N(0,1), M=4 -> 512 "
                         "streams x 65536 positions, K=16; match + gather of "
                         "V [65536,2048] bf16 slices")
    if name == "batched":
        w = synth.batched()
        return dict(kind="bf16", H=w["H"], V=None, M=4, S=512, T=4096,
                    metric="matched positions/sec (streams×T), 512 streams x 4096",
                    desc="batched: hidden [8,4096,256] bf16 N(0,1), M=4 -> 512 "
                         "streams x 4096, K=16; match")
    if name == "repeat":
        w = synth.repeat()
        return dict(kind="symbols", sym=w["sym"], K=16, S=1024, T=32768,
                    metric="matched positions/sec (streams×T), 1024 streams x 32768",
                    desc="repeat: 1024 streams x 32768, K=16, planted copies "
                         "(U{32..512}) over ~30% of positions; match")
    raise ValueError(name)


# ------------------------------------------------------------ CPU oracle

def oracle_run(w, threads):
    """The oracle over the whole workload, streams split across threads
    (each thread runs the unchanged single-threaded oracle).  Returns
    (wall seconds, E, SYM, gathered or None)."""
    import oracle
    S, T = w["S"], w["T"]
    chunks = np.array_split(np.arange(S), threads)
    jobs = []
    for c in chunks:
        if len(c) == 0:
            continue
        s0, s1 = int(c[0]), int(c[-1]) + 1
        if w["kind"] == "bf16":
            H = w["H"]
            B, _, D = H.shape
            R = D // w["M"]
            # streams of one batch row, as contiguous channel slices
            b0, b1 = s0 // R, (s1 - 1) // R
            assert b0 == b1, "thread chunk crosses a batch row"
            M = w["M"]
            h = np.ascontiguousarray(H[b0:b0 + 1, :, (s0 % R) * M:((s1 - 1) % R + 1) * M])
            v = None
            if w["V"] is not None:
                v = np.ascontiguousarray(w["V"][b0:b0 + 1, :, (s0 % R) * M:((s1 - 1) % R + 1) * M])
            jobs.append((s0, s1, h, v))
        else:
            jobs.append((s0, s1, np.ascontiguousarray(w["sym"][s0:s1]), None))

    def work(job):
        s0, s1, a, v = job
        if w["kind"] == "bf16":
            sym = oracle.discretize_bf16(a, w["M"])
            E, SYM, _ = oracle.match(sym, 1 << w["M"])
            g = oracle.gather(v, E, w["M"]) if v is not None else None
        else:
            E, SYM, _ = oracle.match(a, w["K"])
            g = None
        return s0, s1, E, SYM, g

    oracle._load()
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        res = list(ex.map(work, jobs))
    wall = time.perf_counter() - t0
    E = np.empty((S, T), np.int32)
    SYM = np.empty((S, T), np.int16)
    G = None
    if w["kind"] == "bf16" and w["V"] is not None:
        G = np.empty_like(w["V"])
    for (s0, s1, e, sy, g) in res:
        E[s0:s1], SYM[s0:s1] = e, sy
        if g is not None:
            R = w["H"].shape[2] // w["M"]
            b = s0 // R
            M = w["M"]
            G[b, :, (s0 % R) * M:((s1 - 1) % R + 1) * M] = g[0]
    return wall, E, SYM, G


# ------------------------------------------------------------------ decode

DECODE_METRIC = ("decode positions/sec (512 streams, 65,536-position prefix, "
                 "1024 appended positions, one rosa_step each)")
# Compulsory bytes of one step for all 512 streams: the new hidden row
# (2048 bf16), E and SYM out (6 B per stream), the gathered value slices
# (8 B per stream read, 8 B written).
DECODE_BYTES_PER_STEP = 2048 * 2 + 512 * (4 + 2) + 512 * (8 + 8)


def run_decode(args):
    import torch
    from online_suffix_automaton_amd import rosa, synth
    dev = torch.device("cuda:0")
    _log("workload decode: generating")
    pre = synth.long()
    n = 1024
    tail = synth.decode_tail(n)
    H = np.concatenate([pre["H"], tail["H"]], axis=1)
    V = np.concatenate([pre["V"], tail["V"]], axis=1)
    T0 = pre["H"].shape[1]
    Tc = T0 + n
    S, M = 512, 4
    Hd = torch.from_numpy(H.view(np.int16)).to(dev)
    Vd = torch.from_numpy(V.view(np.int16)).to(dev)
    buf = torch.empty(rosa.rosa_state_bytes(S, 1 << M, Tc), dtype=torch.uint8,
                      device=dev)
    # warm-up on a separate short automaton (same kernels, other buffer)
    wbuf = torch.empty(rosa.rosa_state_bytes(S, 1 << M, 64), dtype=torch.uint8,
                       device=dev)
    we = torch.empty(S, dtype=torch.int32, device=dev)
    wst = rosa.rosa_build(rosa.bf16_input(Hd[:, :32], M), 64, wbuf)
    for i in range(min(args.warmup, 32)):
        rosa.rosa_step(wst, rosa.bf16_input(Hd[:, 32 + i:33 + i], M), Vd, we)
    torch.cuda.synchronize()
    del wst, wbuf
    _log("build over the prefix")
    b0 = torch.cuda.Event(enable_timing=True)
    b1 = torch.cuda.Event(enable_timing=True)
    b0.record()
    st = rosa.rosa_build(rosa.bf16_input(Hd[:, :T0], M), Tc, buf)
    b1.record()
    torch.cuda.synchronize()
    build_ms = b0.elapsed_time(b1)
    ends = torch.empty((n, S), dtype=torch.int32, device=dev)
    syms = torch.empty((n, S), dtype=torch.int16, device=dev)
    orows = torch.empty((n, 2048), dtype=torch.int16, device=dev)
    rows = [rosa.bf16_input(Hd[:, T0 + i:T0 + i + 1], M) for i in range(n)]
    outs = [(ends[i], syms[i], orows[i:i + 1]) for i in range(n)]
    # throughput: the n steps back to back, events only around the loop
    _log(f"timing {n} steps")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record()
    for i in range(n):
        rosa.rosa_step(st, rows[i], Vd, *outs[i])
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = ev0.elapsed_time(ev1)
    if rosa.rosa_state_status(st) != rosa.ROSA_OK:
        raise SystemExit("symbol range flag raised")
    # latency: the same steps on a second automaton over the same prefix,
    # an event after every step (the events add host time per step)
    _log("per-step latency pass")
    del st
    st = rosa.rosa_build(rosa.bf16_input(Hd[:, :T0], M), Tc, buf)
    ends2, syms2, orows2 = (torch.empty_like(ends), torch.empty_like(syms),
                            torch.empty_like(orows))
    outs2 = [(ends2[i], syms2[i], orows2[i:i + 1]) for i in range(n)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(n):
        rosa.rosa_step(st, rows[i], Vd, *outs2[i])
        ev[i + 1].record()
    torch.cuda.synchronize()
    step_ms = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(n)])
    if not torch.equal(ends, ends2):
        raise SystemExit("decode: the two passes disagree")
    med = float(np.median(step_ms))
    achieved = DECODE_BYTES_PER_STEP / (total_ms / n / 1e3)
    roof = {"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9,
            "unit": "GB/s", "frac": achieved / HBM_PEAK, "traffic": None}
    cpu = None
    if not args.no_cpu:
        import oracle
        _log("oracle over prefix + appended positions (parity + baseline)")
        oracle._load()
        threads = max(1, min(args.cpu_threads, os.cpu_count() or 1))
        chunks = [c for c in np.array_split(np.arange(S), threads) if len(c)]

        def work(c):
            s0, s1 = int(c[0]), int(c[-1]) + 1
            h = np.ascontiguousarray(H[:, :, s0 * M:s1 * M])
            sym = oracle.discretize_bf16(h, M)
            E, SYM, _ = oracle.match(sym, 1 << M)
            return s0, s1, E, SYM
        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            res = list(ex.map(work, chunks))
        cwall = time.perf_counter() - t0
        Eo = np.empty((S, Tc), np.int32)
        So = np.empty((S, Tc), np.int16)
        for s0, s1, e, sy in res:
            Eo[s0:s1], So[s0:s1] = e, sy
        if not np.array_equal(ends.cpu().numpy(), Eo[:, T0:].T):
            raise SystemExit("parity failure: decode E differs from the oracle")
        if not np.array_equal(syms.cpu().numpy(), So[:, T0:].T):
            raise SystemExit("parity failure: decode SYM differs from the oracle")
        go = oracle.gather(V, Eo, M)[0, T0:]
        if not np.array_equal(orows.cpu().numpy().view(np.uint16), go):
            raise SystemExit("parity failure: decode gather differs")
        _log(f"parity ok; oracle {cwall:.3f} s")
        cpu = {"value": S * Tc / cwall, "unit": "positions/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{S} streams x {Tc} positions (prefix + appended), "
                         f"discretize + automaton match, streams split over "
                         f"{threads} threads"}
    return {
        "metric": DECODE_METRIC, "value": S * n / (total_ms / 1e3),
        "unit": "positions/s", "n_gpus": 1, "steps": n, "warmup": args.warmup,
        "ms_per_step": total_ms / n, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": "decode: 512 streams (hidden [1,T,2048] bf16, "
                               "M=4, K=16), prefix 65536, 1024 appended "
                               "positions, step = extend + match + gather",
                   "streams": S, "T": Tc, "K": 1 << M,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "step_latency_us": {"median": med * 1e3,
                            "p99": float(np.percentile(step_ms, 99)) * 1e3,
                            "host_wall_per_step": wall / n * 1e6,
                            "note": "median/p99: intervals between events "
                                    "recorded after every step (second pass); "
                                    "host_wall_per_step: the timed pass"},
        "build_ms": build_ms,
        "cpu_baseline": cpu,
    }


# ---------------------------------------------------------------------- qk

def run_qk(args):
    """Query/key retrieval on the batched shape: separate query and key
    hidden states [8, 4096, 256] bf16, M = 4 (512 streams, K = 16)."""
    import torch
    from online_suffix_automaton_amd import rosa, synth
    dev = torch.device("cuda:0")
    B, T, D, M = 8, 4096, 256, 4
    S, K = B * (D // M), 1 << M
    _log("workload qk: generating")
    Hq = synth.bf16_normal((B, T, D), 31)
    Hk = synth.bf16_normal((B, T, D), 32)
    dq = torch.from_numpy(Hq.view(np.int16)).to(dev)
    dk = torch.from_numpy(Hk.view(np.int16)).to(dev)
    qi, ki = rosa.bf16_input(dq, M), rosa.bf16_input(dk, M)
    res = {n: torch.empty((S, T), dtype=torch.int32, device=dev)
           for n in ("tau", "end", "len", "run_of", "run_start", "ridx")}
    if args.cf:
        res["cf_tau"] = torch.empty((S, T, M, 2), dtype=torch.int32, device=dev)
        res["cf_ridx"] = torch.empty((S, T, M, 2), dtype=torch.int32, device=dev)
    out = rosa.make_qk_out(res["tau"], **{n: v for n, v in res.items()
                                          if n != "tau"})
    ws = torch.empty(rosa.rosa_match_qk_workspace_bytes(S, T, K),
                     dtype=torch.uint8, device=dev)
    flags = rosa.ROSA_QK_RLE if args.rle else 0
    for _ in range(args.warmup):
        rosa.rosa_match_qk(qi, ki, flags, out, ws)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    steps = max(1, min(args.steps, 5))
    _log(f"timing {steps} steps")
    e0.record()
    for _ in range(steps):
        rosa.rosa_match_qk(qi, ki, flags, out, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # compulsory bytes per stream-position: query and key rows (4 bf16
    # each), the six int32 outputs, and 2M int32 x 2 tables with --cf
    bpp = 8 + 8 + 6 * 4 + (2 * M * 2 * 4 if args.cf else 0)
    achieved = bpp * S * T / (ms / 1e3)
    cpu = None
    if not args.no_cpu:
        import oracle
        oracle._load()
        _log("oracle (parity + baseline)")
        q = oracle.discretize_bf16(Hq, M)
        k = oracle.discretize_bf16(Hk, M)
        threads = max(1, min(args.cpu_threads, os.cpu_count() or 1))
        chunks = [c for c in np.array_split(np.arange(S), threads) if len(c)]

        def work(c):
            return int(c[0]), oracle.match_qk(q[c[0]:c[-1] + 1],
                                               k[c[0]:c[-1] + 1], K, M,
                                               args.rle, cf=args.cf)
        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            parts = list(ex.map(work, chunks))
        wall = time.perf_counter() - t0
        for name, g in res.items():
            want = np.concatenate([pt[name] for _, pt in sorted(parts, key=lambda z: z[0])])
            if not np.array_equal(g.cpu().numpy(), want):
                raise SystemExit(f"parity failure: qk {name} differs")
        _log(f"parity ok; oracle {wall:.3f} s")
        cpu = {"value": S * T / wall, "unit": "positions/s", "cores": threads,
               "kind": "oracle",
               "sample": f"whole workload ({S} streams x {T}), query/key "
                         f"match{' with folding' if args.rle else ''}"
                         f"{' and counterfactual tables' if args.cf else ''}, "
                         f"streams split over {threads} threads"}
    return {
        "metric": "query/key matched positions/sec (512 streams x 4096)",
        "value": S * T / (ms / 1e3), "unit": "positions/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u8", "data": "synthetic",
        "config": {"workload": "qk: query and key hidden states [8,4096,256] "
                               "bf16 N(0,1) (seeds 31, 32), M=4 -> 512 streams, "
                               "K=16" + (", key runs folded" if args.rle else "")
                               + (", counterfactual tables" if args.cf else ""),
                   "streams": S, "T": T, "K": K, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved / 1e9,
                     "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK, "traffic": None},
        "cpu_baseline": cpu,
    }


# ----------------------------------------------------------------- scatter

def run_scatter(args):
    """Destination-scatter gradient on the long workload: destinations from
    rosa_match on the long workload's hidden states, upstream gradient theta
    [1, 65536, 2048] float32 N(0,1) (seed 45)."""
    import torch
    from online_suffix_automaton_amd import rosa, synth
    dev = torch.device("cuda:0")
    B, T, D, M = 1, 65536, 2048, 4
    S = B * D // M
    _log("workload scatter: generating")
    w = synth.long(with_v=False)
    Hd = torch.from_numpy(w["H"].view(np.int16)).to(dev)
    E, _, _, _ = rosa.match(Hd, M=M, want_len=False)
    del Hd
    theta = np.random.default_rng(45).standard_normal((B, T, D), dtype=np.float32)
    # theta's rows at a pitch of D + theta_pad floats (any pitch is taken; one
    # that is not a multiple of 2 KiB keeps the rows' L2 sets apart)
    thbuf = torch.zeros((B, T, D + args.theta_pad), dtype=torch.float32, device=dev)
    thbuf[:, :, :D] = torch.from_numpy(theta).to(dev)
    th = thbuf[:, :, :D]
    G = torch.empty((B, T, D), dtype=torch.float32, device=dev)
    ws = torch.empty(rosa.rosa_scatter_grad_workspace_bytes(S, T),
                     dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        rosa.rosa_scatter_grad(th, M, E, G, ws)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    _log(f"timing {args.steps} steps")
    e0.record()
    for _ in range(args.steps):
        rosa.rosa_scatter_grad(th, M, E, G, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # compulsory bytes per stream-position: E in (4), theta's M floats in
    # (16), G's M floats out (16)
    bpp = 4 + 4 * M + 4 * M
    achieved = bpp * S * T / (ms / 1e3)
    cpu = None
    if not args.no_cpu:
        import oracle
        oracle._load()
        _log("oracle (parity + baseline)")
        Eh = E.cpu().numpy()
        t0 = time.perf_counter()
        want = oracle.scatter_grad(theta, Eh, M)
        wall = time.perf_counter() - t0
        if not np.array_equal(G.cpu().numpy().view(np.uint32), want.view(np.uint32)):
            raise SystemExit("parity failure: scatter gradient differs")
        _log(f"parity ok; oracle {wall:.3f} s")
        cpu = {"value": S * T / wall, "unit": "positions/s", "cores": 1,
               "kind": "oracle",
               "sample": f"whole workload ({S} streams x {T}), single thread "
                         "(the oracle sums every stream into one array)"}
    return {
        "metric": "scatter-gradient positions/sec (512 streams x 65536)",
        "value": S * T / (ms / 1e3), "unit": "positions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f64 accumulate, f32 in/out", "data": "synthetic",
        "config": {"workload": "scatter: destinations of the long workload "
                               "(512 streams x 65536, K=16), theta "
                               "[1,65536,2048] f32 N(0,1)",
                   "streams": S, "T": T, "K": 16, "parallelism": "single GPU",
                   "theta_row_pitch": int(th.stride(1))},
        "roofline": {"bound": "hbm", "achieved": achieved / 1e9,
                     "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK, "traffic": None},
        "cpu_baseline": cpu,
    }


# -------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long",
                    choices=["long", "batched", "repeat", "decode", "qk",
                             "scatter"])
    ap.add_argument("--rle", action="store_true",
                    help="qk workload: fold the key stream into runs")
    ap.add_argument("--cf", action="store_true",
                    help="qk workload: also the per-bit counterfactual tables")
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the oracle baseline and parity check")
    ap.add_argument("--cpu-threads", type=int, default=16)
    ap.add_argument("--theta-pad", type=int, default=32, metavar="ELEMS",
                    help="scatter workload: theta rows stored at a pitch of D + "
                         "ELEMS floats (0: dense rows)")
    ap.add_argument("--v-pad", type=int, default=64, metavar="ELEMS",
                    help="long workload: V rows stored at a pitch of D + ELEMS "
                         "bf16 (0: dense rows)")
    ap.add_argument("--copy-reference", type=int, default=0, metavar="BYTES",
                    help="after timing, run one plain device-to-device copy of "
                         "BYTES (the reference for scaling HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the retrieval path has no "
              "cross-GPU step and this build runs on a single MI355X; "
              "use --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.workload == "decode":
        print(json.dumps(run_decode(args)), flush=True)
        return
    if args.workload == "qk":
        print(json.dumps(run_qk(args)), flush=True)
        return
    if args.workload == "scatter":
        print(json.dumps(run_scatter(args)), flush=True)
        return

    import torch
    from online_suffix_automaton_amd import rosa

    dev = torch.device("cuda:0")
    _log(f"workload {args.workload}: generating")
    w = make_workload(args.workload)
    S, T = w["S"], w["T"]

    if w["kind"] == "bf16":
        Hd = torch.from_numpy(w["H"].view(np.int16)).to(dev)
        Vd = None
        if w["V"] is not None:
            # V's rows at a pitch of D + v_pad elements (the gather takes any
            # pitch; one that is not a multiple of 2 KiB keeps its L2 sets apart)
            Bv, Tv, Dv = w["V"].shape
            Vbuf = torch.zeros((Bv, Tv, Dv + args.v_pad), dtype=torch.int16, device=dev)
            Vbuf[:, :, :Dv] = torch.from_numpy(w["V"].view(np.int16)).to(dev)
            Vd = Vbuf[:, :, :Dv]
        inp = rosa.bf16_input(Hd, w["M"])
        K = 1 << w["M"]
    else:
        Xd = torch.from_numpy(w["sym"]).to(dev)
        inp = rosa.symbols_input(Xd, w["K"])
        Vd = None
        K = w["K"]
    E = torch.empty((S, T), dtype=torch.int32, device=dev)
    SYM = torch.empty((S, T), dtype=torch.int16, device=dev)
    out = (torch.empty(tuple(Vd.shape), dtype=torch.int16, device=dev)
           if Vd is not None else None)
    ws = torch.empty(rosa.rosa_match_workspace_bytes(S, T, K), dtype=torch.uint8,
                     device=dev)
    outs = rosa.make_out(E, SYM)
    stream = torch.cuda.current_stream()

    n_ev = args.steps
    kb = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ke = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]

    def step(i=None):
        if i is None:
            rosa.rosa_match(inp, outs, ws, stream)
        else:
            rosa.rosa_match_timed(inp, outs, ws, kb[i], ke[i], stream)
        if Vd is not None:
            rosa.rosa_gather(Vd, w["M"], E, out, stream)

    _log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    _log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    k_ms = [kb[i].elapsed_time(ke[i]) for i in range(n_ev)]
    k_avg = float(np.mean(k_ms))
    if rosa.rosa_match_status(ws) != rosa.ROSA_OK:
        raise SystemExit("symbol range flag raised")
    if args.copy_reference > 0:
        # two plain copies of known size for scaling HBM byte counters: the
        # runtime's buffer copy, and an elementwise kernel (int32 x + 1) that
        # reads and writes with ordinary vector loads and stores
        src = torch.zeros(args.copy_reference // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.add(src, 1, out=dst)
        torch.cuda.synchronize()
        del src, dst
    value = S * T / (ms_step / 1e3)
    _log(f"ms/step {ms_step:.4f}  retrieval kernel {k_avg:.4f} ms")

    kbytes = KERNEL_BYTES_PER_POS * S * T
    achieved = kbytes / (k_avg / 1e3)
    roof = {"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9,
            "unit": "GB/s", "frac": achieved / HBM_PEAK,
            "traffic": measured_traffic() if args.workload == "long" else None}

    cpu = None
    if not args.no_cpu:
        threads = max(1, min(args.cpu_threads, os.cpu_count() or 1))
        _log(f"oracle on {threads} threads (parity check + baseline)")
        walls = []
        for _ in range(3):
            wall, Eo, SYMo, Go = oracle_run(w, threads)
            walls.append(wall)
        wall = float(np.median(walls))
        if not np.array_equal(E.cpu().numpy(), Eo):
            raise SystemExit("parity failure: E differs from the oracle")
        if not np.array_equal(SYM.cpu().numpy(), SYMo):
            raise SystemExit("parity failure: SYM differs from the oracle")
        if Go is not None and not np.array_equal(
                out.cpu().numpy().view(np.uint16), Go):
            raise SystemExit("parity failure: gathered values differ")
        _log(f"parity ok; oracle {wall:.3f} s")
        cpu = {"value": S * T / wall, "unit": "positions/s", "cores": threads,
               "kind": "oracle",
               "sample": f"whole workload ({S} streams x {T}), "
                         + ("discretize + match + gather" if w["kind"] == "bf16"
                            and w["V"] is not None else "match")
                         + f", streams split over {threads} threads, median of 3"}

    line = {
        "metric": w["metric"], "value": value, "unit": "positions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u8", "data": "synthetic",
        "config": {"workload": w["desc"], "streams": S, "T": T, "K": K,
                   "parallelism": "single GPU",
                   **({"v_row_pitch": int(Vd.stride(1))} if Vd is not None else {})},
        "roofline": roof,
        "kernel_ms": k_avg,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
