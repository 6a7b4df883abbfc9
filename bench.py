"""Benchmark of the ROSA retrieval hot path on one MI355X.

One step = the whole path over one batch: bf16 hidden states -> sign bits ->
4-bit route symbols (512 streams) -> longest-recurring-suffix match for all
65,536 positions of every stream (E and next symbol) -> gather of the matched
value slices from V.  Inputs are resident in HBM before timing starts.

Prints one JSON line: throughput in matched positions/s; the roofline of the
dominant kernel (the retrieval kernel, timed with HIP events recorded on the
stream it is launched on: its VALU issue rate against the vector issue peak
when a counter summary of the current source is committed, with its bytes
against HBM peak beside it) and of the whole step (30 B per stream-position
against HBM peak); the same steps with V's rows at the dense pitch; and the
CPU oracle timed on the host on 16 threads and on one thread, as a reported
baseline.  Every output of the timed run is compared with the oracle before
the line is printed.

    python bench.py [--steps K] [--warmup W] [--no-cpu] [--no-dense]
                    [--workload long|batched|repeat|decode|qk|scatter]

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
# Algorithmic bytes per stream-position of the retrieval kernel on these
# workloads (streams of up to 65536 positions over 16 symbols, where the
# kernel also runs the time-ordered pass and writes E and SYM itself): the
# symbol read (1 B; the batched workload reads its 4 bf16 channels, 8 B,
# straight from the hidden rows) and E and SYM written (4 + 2 B).  The
# result records the kernel writes and reads back are an intermediate.
KERNEL_BYTES_PER_POS = {"batched": 8 + 6}
KERNEL_BYTES_DEFAULT = 1 + 6
# Compulsory bytes per stream-position of the whole step on the long
# workload: 4 bf16 channels in (8 B), E and SYM out (4 + 2 B), the gathered
# 4 bf16 values read (8 B) and written (8 B).
STEP_BYTES_PER_POS = 8 + 6 + 16
# Vector issue peak: 256 CUs x 4 SIMDs x 2.4 GHz, one wave64 VALU instruction
# per SIMD every 4 cycles (16 lanes per cycle), in wave instructions/s.
VALU_PEAK = 256 * 4 * 2.4e9 / 4
PMC_FILE = os.path.join(ROOT, "profiles", "stream_kernel_long_pmc.txt")
ISSUE_FILE = os.path.join(ROOT, "profiles", "stream_kernel_long_issue.txt")


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


def measured_valu():
    """VALU wave instructions per launch of the retrieval kernel from the
    committed instruction-issue counter summary, if it was taken on the
    current source."""
    try:
        txt = open(ISSUE_FILE).read()
    except OSError:
        return None
    m = re.search(r"^source_sha\s*=\s*(\w+)", txt, re.M)
    v = re.search(r"^stream_kernel_valu_per_launch\s*=\s*([0-9.eE+]+)", txt, re.M)
    if not m or not v or m.group(1) != kernel_source_hash():
        return None
    return float(v.group(1))


def kernel_roofline(npos, k_ms, workload):
    """Roofline of the retrieval kernel.  It is bound by vector instruction
    issue: `achieved` is its VALU wave instructions per launch (counters of
    the committed summary, same source) over the live event-timed duration,
    against VALU_PEAK.  Its bytes (7 B per stream-position, symbol in and
    E and SYM out; 14 B when it reads bf16 rows) against HBM peak are
    reported beside it; without a current counter summary the bytes are the
    reported bound."""
    kbytes = KERNEL_BYTES_PER_POS.get(workload, KERNEL_BYTES_DEFAULT) * npos
    hbm = kbytes / (k_ms / 1e3)
    traffic = measured_traffic() if workload == "long" else None
    valu = measured_valu() if workload == "long" else None
    if valu is None:
        return {"bound": "hbm", "achieved": hbm / 1e9, "peak": HBM_PEAK / 1e9,
                "unit": "GB/s", "frac": hbm / HBM_PEAK, "traffic": traffic}
    rate = valu / (k_ms / 1e3)
    return {"bound": "alu", "achieved": rate / 1e9, "peak": VALU_PEAK / 1e9,
            "unit": "G VALU wave instructions/s", "frac": rate / VALU_PEAK,
            "traffic": traffic, "valu_per_position": valu / npos,
            "hbm_achieved": hbm / 1e9, "hbm_peak": HBM_PEAK / 1e9,
            "hbm_frac": hbm / HBM_PEAK}


def host_cpu_info(threads):
    """The host the oracle ran on: CPU model, SMT state, logical CPUs and the
    CPUs this process may use."""
    info = {"threads_used": threads, "nproc": os.cpu_count()}
    try:
        info["affinity"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    try:
        import subprocess
        txt = subprocess.run(["lscpu"], capture_output=True, text=True,
                             timeout=10).stdout
        for key, name in (("Model name", "model"), ("Thread(s) per core",
                                                     "threads_per_core"),
                          ("Socket(s)", "sockets")):
            m = re.search(rf"^{re.escape(key)}:\s*(.+)$", txt, re.M)
            if m:
                info[name] = m.group(1).strip()
    except Exception:
        pass
    try:
        with open("/sys/devices/system/cpu/smt/active") as f:
            info["smt_active"] = f.read().strip() == "1"
    except OSError:
        pass
    return info


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
    if name == "lowent":
        w = synth.long()
        H = w["H"].copy()
        R, M = 512, 4
        mag = H & np.uint16(0x7FFF)
        for r in range(R):
            c = slice(r * M, (r + 1) * M)
            if r < 128:
                # dead channel group: every channel <= 0, the symbol is 0
                H[:, :, c] = mag[:, :, c] | np.uint16(0x8000)
            elif r < 256:
                # period 2 .. 9 over distinct symbols: channel j carries
                # bit j of the symbol as its sign
                per = 2 + (r % 8)
                sym = (np.arange(65536) % per).astype(np.uint16)
                for j in range(M):
                    neg = ((sym >> j) & 1) == 0
                    H[0, :, r * M + j] = np.where(neg, mag[0, :, r * M + j] | np.uint16(0x8000),
                                                  mag[0, :, r * M + j])
        return dict(kind="bf16", H=H, V=w["V"], M=M, S=512, T=65536,
                    metric="matched positions/sec (streams×T), 512 low-entropy "
                           "streams x 65536",
                    desc="lowent: hidden [1,65536,2048] bf16 N(0,1) with routes "
                         "0-127 dead (every channel <= 0: constant streams) and "
                         "routes 128-255 periodic (periods 2-9), M=4 -> 512 "
                         "streams x 65536, K=16; match + gather of V",
                    closed_form=256)
    raise ValueError(name)


def closed_form_streams(Sym, n):
    """E of the first n streams of the low-entropy workload from their
    closed forms (constant: E = t-1; period p over p distinct symbols: -1
    before p, then t-p), identified from the packed symbols."""
    T = Sym.shape[1]
    t = np.arange(T)
    E = np.empty((n, T), np.int32)
    for s in range(n):
        x = Sym[s]
        p = 1
        while p < 16 and x[p] != x[0]:
            p += 1
        assert np.array_equal(x, np.resize(x[:p], T)) and len(set(x[:p])) == p
        E[s] = np.where(t < p, -1, t - p)
    return E


# ------------------------------------------------------------ CPU oracle

def oracle_run(w, threads):
    """The oracle over the whole workload, streams split across threads
    (each thread runs the unchanged single-threaded oracle).  Returns
    (wall seconds, E, SYM, gathered or None)."""
    import oracle
    S, T = w["S"], w["T"]
    chunks = np.array_split(np.arange(S), threads)
    if w["kind"] == "bf16":
        # a job never crosses a batch row (its streams are a contiguous
        # channel slice of one row)
        R = w["H"].shape[2] // w["M"]
        chunks = [part for c in chunks if len(c)
                  for part in np.split(c, np.nonzero(np.diff(c // R))[0] + 1)]
    jobs = []
    for c in chunks:
        if len(c) == 0:
            continue
        s0, s1 = int(c[0]), int(c[-1]) + 1
        if w["kind"] == "bf16":
            H = w["H"]
            B, _, D = H.shape
            R = D // w["M"]
            b0, b1 = s0 // R, (s1 - 1) // R
            assert b0 == b1, "job crosses a batch row"
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


# -------------------------------------------------------------- qk decode

QKD_METRIC = ("query/key decode positions/sec (512 streams, 65,536-step "
              "prefix, 1024 steps, one rosa_step_qk each)")


def run_qk_decode(args):
    """Query/key decode: query and key hidden states [1, 65536 + 1024, 2048]
    bf16 (N(0,1), independent), M = 4: 512 streams.  rosa_build_qk over the
    prefix, then 1024 rosa_step_qk calls (one time step of every stream
    each), with --rle and --cf as for the qk workload."""
    import torch
    from online_suffix_automaton_amd import rosa, synth
    dev = torch.device("cuda:0")
    T0, n, D, M = 65536, 1024, 2048, 4
    Tc = T0 + n
    S, K = D // M, 1 << M
    _log("workload qk_decode: generating")
    Hq = synth.bf16_normal((1, Tc, D), 71)
    Hk = synth.bf16_normal((1, Tc, D), 72)
    hq = torch.from_numpy(Hq.view(np.int16)).to(dev)
    hk = torch.from_numpy(Hk.view(np.int16)).to(dev)
    flags = rosa.ROSA_QK_RLE if args.rle else 0
    cfw = M if args.cf else 0
    buf = torch.empty(rosa.rosa_qk_state_bytes(S, K, Tc), dtype=torch.uint8,
                      device=dev)

    def outs(rows):
        o = {f: torch.empty((rows, S), dtype=torch.int32, device=dev)
             for f in ("tau", "end", "len", "run_of", "ridx")}
        if cfw:
            for f in ("cf_tau", "cf_ridx"):
                o[f] = torch.empty((rows, S, M, 2), dtype=torch.int32, device=dev)
        return o

    def step_out(o, i):
        return rosa.make_qk_out(o["tau"][i], **{f: v[i] for f, v in o.items()
                                                if f != "tau"})
    # warm-up on a separate short state (same kernel, other buffer)
    wbuf = torch.empty(rosa.rosa_qk_state_bytes(S, K, 64), dtype=torch.uint8,
                       device=dev)
    wo = outs(1)
    wst = rosa.rosa_build_qk(rosa.bf16_input(hq[:, :32], M),
                             rosa.bf16_input(hk[:, :32], M), flags, 64, wbuf)
    for i in range(min(args.warmup, 32)):
        rosa.rosa_step_qk(wst, rosa.bf16_input(hq[:, 32 + i:33 + i], M),
                          rosa.bf16_input(hk[:, 32 + i:33 + i], M), step_out(wo, 0))
    torch.cuda.synchronize()
    del wst, wbuf
    _log("build over the prefix")
    qpre, kpre = rosa.bf16_input(hq[:, :T0], M), rosa.bf16_input(hk[:, :T0], M)
    b0 = torch.cuda.Event(enable_timing=True)
    b1 = torch.cuda.Event(enable_timing=True)
    b0.record()
    st = rosa.rosa_build_qk(qpre, kpre, flags, Tc, buf)
    b1.record()
    torch.cuda.synchronize()
    build_ms = b0.elapsed_time(b1)
    qrows = [rosa.bf16_input(hq[:, T0 + i:T0 + i + 1], M) for i in range(n)]
    krows = [rosa.bf16_input(hk[:, T0 + i:T0 + i + 1], M) for i in range(n)]
    o1 = outs(n)
    so1 = [step_out(o1, i) for i in range(n)]
    _log(f"timing {n} steps")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record()
    for i in range(n):
        rosa.rosa_step_qk(st, qrows[i], krows[i], so1[i])
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = ev0.elapsed_time(ev1)
    if rosa.rosa_state_status(st) != rosa.ROSA_OK:
        raise SystemExit("symbol range flag raised")
    _log("per-step latency pass")
    del st
    st = rosa.rosa_build_qk(qpre, kpre, flags, Tc, buf)
    o2 = outs(n)
    so2 = [step_out(o2, i) for i in range(n)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(n):
        rosa.rosa_step_qk(st, qrows[i], krows[i], so2[i])
        ev[i + 1].record()
    torch.cuda.synchronize()
    step_ms = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(n)])
    for f in o1:
        if not torch.equal(o1[f], o2[f]):
            raise SystemExit("qk decode: the two passes disagree")
    # compulsory bytes of one step for all streams: the query and key rows
    # (2 x 2048 bf16) and the outputs (5 int32 per stream, 16 more with the
    # tables at M = 4)
    step_bytes = 2 * D * 2 + S * 4 * (5 + (4 * cfw if cfw else 0))
    achieved = step_bytes / (total_ms / n / 1e3)
    roof = {"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9,
            "unit": "GB/s", "frac": achieved / HBM_PEAK, "traffic": None}
    cpu = None
    if not args.no_cpu:
        import oracle
        _log("oracle over prefix + steps (parity + baseline)")
        oracle._load()
        threads = max(1, min(args.cpu_threads, os.cpu_count() or 1))
        chunks = [c for c in np.array_split(np.arange(S), threads) if len(c)]

        def work(c):
            s0, s1 = int(c[0]), int(c[-1]) + 1
            q = oracle.discretize_bf16(np.ascontiguousarray(Hq[:, :, s0 * M:s1 * M]), M)
            k = oracle.discretize_bf16(np.ascontiguousarray(Hk[:, :, s0 * M:s1 * M]), M)
            return s0, s1, oracle.match_qk(q, k, K, M, bool(args.rle), cf=bool(cfw))
        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            res = list(ex.map(work, chunks))
        cwall = time.perf_counter() - t0
        for f in o1:
            got = o1[f].cpu().numpy()
            for s0, s1, w in res:
                want = np.moveaxis(w[f][:, T0:], 0, 1)
                if not np.array_equal(got[:, s0:s1], want):
                    raise SystemExit(f"parity failure: qk decode {f} differs")
        _log(f"parity ok; oracle {cwall:.3f} s")
        cpu = {"value": S * Tc / cwall, "unit": "positions/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{S} streams x {Tc} time steps (prefix + steps), "
                         f"discretize + query/key automaton match"
                         f"{' with run folding' if args.rle else ''}"
                         f"{' and tables' if cfw else ''}, streams split over "
                         f"{threads} threads"}
    return {
        "metric": QKD_METRIC, "value": S * n / (total_ms / 1e3),
        "unit": "positions/s", "n_gpus": 1, "steps": n, "warmup": args.warmup,
        "ms_per_step": total_ms / n, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": "qk_decode: query and key hidden [1,T,2048] bf16, "
                               "M=4 -> 512 streams, prefix 65536, 1024 steps"
                               f"{', run folding' if args.rle else ''}"
                               f"{', counterfactual tables' if cfw else ''}",
                   "streams": S, "T": Tc, "K": K, "rle": bool(args.rle),
                   "cf": bool(cfw), "parallelism": "single GPU"},
        "roofline": roof,
        "step_latency_us": {"median": float(np.median(step_ms)) * 1e3,
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
    """Query/key retrieval: separate query and key hidden states
    [B, T, 256] bf16, M = 4 (K = 16), B = 8 at the batched shape T = 4096
    (512 streams) and B = 32768 / T past it (64 streams of 65536 at
    T = 65536)."""
    import torch
    from online_suffix_automaton_amd import rosa, synth
    dev = torch.device("cuda:0")
    T, D, M = args.T, 256, 4
    B = 8 if T <= 4096 else max(1, 32768 // T)
    S, K = B * (D // M), 1 << M
    _log("workload qk: generating")
    Hq = synth.bf16_normal((B, T, D), 31)
    Hk = synth.bf16_normal((B, T, D), 32)
    if args.qk_data == "lowent":
        # routes 0-15: dead (every channel <= 0, constant symbol 0) in both
        # streams; routes 16-31: the same period 2..9 in query and key
        # (matches as long as the stream); routes 32-63 independent N(0,1)
        mag = Hk & np.uint16(0x7FFF)
        for r in range(32):
            c = slice(r * M, (r + 1) * M)
            if r < 16:
                Hk[:, :, c] = mag[:, :, c] | np.uint16(0x8000)
            else:
                per = 2 + (r % 8)
                sym = (np.arange(T) % per).astype(np.uint16)
                for j in range(M):
                    neg = ((sym >> j) & 1) == 0
                    Hk[:, :, r * M + j] = np.where(neg[None], mag[:, :, r * M + j] | np.uint16(0x8000),
                                                   mag[:, :, r * M + j])
            Hq[:, :, c] = Hk[:, :, c]
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
    steps = max(1, min(args.steps, 20))
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
        "metric": f"query/key matched positions/sec ({S} streams x {T})",
        "value": S * T / (ms / 1e3), "unit": "positions/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u8", "data": "synthetic",
        "config": {"workload": f"qk: query and key hidden states [{B},{T},256] "
                               f"bf16 N(0,1) (seeds 31, 32), M=4 -> {S} streams, "
                               "K=16" + (", key runs folded" if args.rle else "")
                               + (", routes 0-15 dead and 16-31 periodic (2-9) "
                                  "with equal query and key"
                                  if args.qk_data == "lowent" else "")
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
                    choices=["long", "batched", "repeat", "lowent", "decode",
                             "qk", "qk_decode", "scatter"])
    ap.add_argument("--rle", action="store_true",
                    help="qk and qk_decode workloads: fold the key stream into runs")
    ap.add_argument("--cf", action="store_true",
                    help="qk and qk_decode workloads: also the per-bit "
                         "counterfactual tables")
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the oracle baseline and parity check")
    ap.add_argument("--cpu-threads", type=int, default=16)
    ap.add_argument("--qk-data", default="iid", choices=["iid", "lowent"],
                    help="qk workload: independent N(0,1) states, or half the "
                         "routes dead / periodic with equal query and key")
    ap.add_argument("--T", type=int, default=4096,
                    help="qk workload: steps per stream (B = 8 at 4096, "
                         "32768 / T streams of 256 channels past it)")
    ap.add_argument("--theta-pad", type=int, default=32, metavar="ELEMS",
                    help="scatter workload: theta rows stored at a pitch of D + "
                         "ELEMS floats (0: dense rows)")
    ap.add_argument("--v-pad", type=int, default=64, metavar="ELEMS",
                    help="long workload: V rows stored at a pitch of D + ELEMS "
                         "bf16 (0: dense rows)")
    ap.add_argument("--no-split", action="store_true",
                    help="workloads with a gather: time unsplit steps one after "
                         "another on one stream instead of the two pipelined "
                         "stream halves")
    ap.add_argument("--no-dense", action="store_true",
                    help="long workload: skip the second timed pass with V's "
                         "rows at the dense pitch")
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
    if args.workload == "qk_decode":
        print(json.dumps(run_qk_decode(args)), flush=True)
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

    Vd = Vdense = None
    if w["kind"] == "bf16":
        Hd = torch.from_numpy(w["H"].view(np.int16)).to(dev)
        if w["V"] is not None:
            # V's rows at a pitch of D + v_pad elements (the gather takes any
            # pitch; one that is not a multiple of 2 KiB keeps its L2 sets
            # apart), and a dense copy for the second timed pass
            Bv, Tv, Dv = w["V"].shape
            Vdense = torch.from_numpy(w["V"].view(np.int16)).to(dev)
            Vbuf = torch.zeros((Bv, Tv, Dv + args.v_pad), dtype=torch.int16, device=dev)
            Vbuf[:, :, :Dv] = Vdense
            Vd = Vbuf[:, :, :Dv]
        inp = rosa.bf16_input(Hd, w["M"])
        K = 1 << w["M"]
    else:
        Xd = torch.from_numpy(w["sym"]).to(dev)
        inp = rosa.symbols_input(Xd, w["K"])
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
    gb = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ge = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]

    def step(V, i=None):
        if i is None:
            rosa.rosa_match(inp, outs, ws, stream)
        else:
            rosa.rosa_match_timed(inp, outs, ws, kb[i], ke[i], stream)
        if V is not None:
            if i is not None:
                gb[i].record(stream)
            rosa.rosa_gather(V, w["M"], E, out, stream)
            if i is not None:
                ge[i].record(stream)

    # Pipelined steps (with a gather): the streams in two halves by channel
    # (routes 0..R/2-1 and R/2..R-1 of H and V), each with its own workspace
    # and HIP stream (default priority).  A retrieval kernel holds one
    # workgroup per CU with nearly all of its LDS and is bound by VALU issue;
    # the gather and the discretisation use no LDS and are bound by memory,
    # so each runs beside the other half's retrieval kernel:
    #  - the first half's gather waits for the event rosa_match_timed records
    #    just before the second half's retrieval kernel, and the second
    #    half's gather for the first half's (one gather at a time);
    #  - each half's symbols are made by rosa_discretize one step ahead
    #    (software pipelining: every timed step still discretises, matches
    #    and gathers all streams once), after that half's gather, so they are
    #    made beside the other half's retrieval; rosa_match then reads them
    #    as 16-byte aligned symbol rows;
    #  - one half's match does not wait for the other's: the halves share
    #    no buffer, each half's own order (symbols, match, gather, next
    #    symbols) is that of its stream, and a retrieval kernel's workgroups
    #    take the CUs that the other half's slowest workgroups leave idle
    #    (measured: 0.69 ms per step when each match waited for the
    #    other, 0.63 ms without).
    split = (Vd is not None and w["kind"] == "bf16" and not args.no_split
             and S % 2 == 0 and (w["H"].shape[2] // 2) % w["M"] == 0)
    if split:
        h, Dh = S // 2, w["H"].shape[2] // 2
        inA = rosa.bf16_input(Hd[:, :, :Dh], w["M"])
        inB = rosa.bf16_input(Hd[:, :, Dh:], w["M"])
        symA = torch.empty((h, T), dtype=torch.uint8, device=dev)
        symB = torch.empty_like(symA)
        sinA, sinB = rosa.symbols_input(symA, K), rosa.symbols_input(symB, K)
        wsA = torch.empty(rosa.rosa_match_workspace_bytes(h, T, K), dtype=torch.uint8,
                          device=dev)
        wsB = torch.empty_like(wsA)
        oA, oB = rosa.make_out(E[:h], SYM[:h]), rosa.make_out(E[h:], SYM[h:])
        s2 = torch.cuda.Stream(device=dev)
        evB0, evB1, evJ, evGA, evGB = (torch.cuda.Event() for _ in range(5))

    def prologue():
        """The first step's symbols of both halves."""
        rosa.rosa_discretize(inA, symA, stream)
        rosa.rosa_discretize(inB, symB, s2)

    def step_piped(V):
        rosa.rosa_match(sinA, oA, wsA, stream)
        rosa.rosa_match_timed(sinB, oB, wsB, evB0, evB1, s2)
        stream.wait_event(evB0)
        stream.wait_event(evGB)    # the previous step's second-half gather
        rosa.rosa_gather(V[:, :, :Dh], w["M"], E[:h], out[:, :, :Dh], stream)
        evGA.record(stream)
        rosa.rosa_discretize(inA, symA, stream)   # next step's, beside this step's second retrieval
        s2.wait_event(evGA)
        rosa.rosa_gather(V[:, :, Dh:], w["M"], E[h:], out[:, :, Dh:], s2)
        evGB.record(s2)
        rosa.rosa_discretize(inB, symB, s2)       # next step's, beside the next first retrieval

    def join():
        evJ.record(s2)
        stream.wait_event(evJ)

    def loop_ms(V, piped):
        """Warm-up, then `steps` steps between two events on the stream."""
        run = step_piped if piped else step
        if piped:
            prologue()
        for _ in range(args.warmup):
            run(V)
        if piped:
            join()
        torch.cuda.synchronize()
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        t_start.record(stream)
        if piped:
            s2.wait_event(t_start)
        for _ in range(args.steps):
            run(V)
        if piped:
            join()
        t_end.record(stream)
        torch.cuda.synchronize()
        return t_start.elapsed_time(t_end) / args.steps

    def piped_for(V):
        """Pipeline the steps unless V's row pitch is a multiple of 2 KiB: there
        the gather keeps a route group's lines in a few L2 sets, and a
        retrieval kernel running beside it evicts them (measured on the long
        workload at the dense pitch: 1.48 ms pipelined, 0.99 ms serial)."""
        return split and (V.stride(1) * 2) % 2048 != 0

    def timed(V):
        """The steps serial and unsplit with events around the retrieval and
        gather kernels (their mean durations; the events are kept out of the
        timed loop, where they would add to short steps), then ms per step
        (pipelined when split and the pitch allows) over the timed loop.  The
        kernel-timed steps (after warm-up steps of their own) run first, so
        the timed loop does not start on a GPU that is still raising its
        clocks."""
        piped = piped_for(V)
        for _ in range(args.warmup):
            step(V)
        for i in range(args.steps):
            step(V, i)
        torch.cuda.synchronize()
        serial_out = (E.clone(), SYM.clone(), out.clone()) if piped else None
        ms = loop_ms(V, piped)
        if serial_out is not None and not (torch.equal(serial_out[0], E) and
                                           torch.equal(serial_out[1], SYM) and
                                           torch.equal(serial_out[2], out)):
            raise SystemExit("pipelined steps differ from serial steps")
        k = float(np.mean([kb[i].elapsed_time(ke[i]) for i in range(n_ev)]))
        g = (float(np.mean([gb[i].elapsed_time(ge[i]) for i in range(n_ev)]))
             if V is not None else None)
        return ms, k, g

    piped = Vd is not None and piped_for(Vd)
    _log(f"warmup {args.warmup}, timing {args.steps} steps"
         + (" (two stream halves, pipelined)" if piped else ""))
    ms_step, k_avg, g_avg = timed(Vd)
    if rosa.rosa_match_status(ws) != rosa.ROSA_OK or (
            split and (rosa.rosa_match_status(wsA) != rosa.ROSA_OK or
                       rosa.rosa_match_status(wsB) != rosa.ROSA_OK)):
        raise SystemExit("symbol range flag raised")
    # the same steps one after another on one stream, unsplit (reported beside
    # the pipelined figure)
    ms_serial = loop_ms(Vd, False) if piped else None
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
    _log(f"ms/step {ms_step:.4f}  retrieval kernel {k_avg:.4f} ms"
         + (f"  gather {g_avg:.4f} ms" if g_avg is not None else "")
         + (f"  serial unsplit steps {ms_serial:.4f} ms" if piped else ""))
    dense = None
    if Vd is not None and args.v_pad != 0 and not args.no_dense:
        # the same steps with V's rows at the dense pitch (D elements); the
        # outputs are compared with the padded run's
        out_pad = out.clone()
        ms_d, k_d, g_d = timed(Vdense)
        if not torch.equal(out, out_pad):
            raise SystemExit("dense-pitch gather differs from the padded one")
        dense = {"ms_per_step": ms_d, "retrieval_ms": k_d, "gather_ms": g_d,
                 "v_row_pitch": int(Vdense.stride(1)),
                 "schedule": "pipelined" if piped_for(Vdense) else "serial"}
        if split and not piped_for(Vdense):
            dense["ms_per_step_pipelined"] = loop_ms(Vdense, True)
        _log(f"dense V rows: ms/step {ms_d:.4f}  gather {g_d:.4f} ms")

    roof = kernel_roofline(S * T, k_avg, args.workload)
    if w["kind"] == "bf16" and Vd is not None:
        sb = STEP_BYTES_PER_POS * S * T
        roof["step_bytes_per_position"] = STEP_BYTES_PER_POS
        roof["step_achieved"] = sb / (ms_step / 1e3) / 1e9
        roof["step_frac"] = sb / (ms_step / 1e3) / HBM_PEAK

    cpu = None
    if not args.no_cpu and w.get("closed_form"):
        # the constant and periodic streams against their closed forms (the
        # oracle's automaton walks every state of a constant stream's suffix
        # path, O(T^2)); the other streams, the symbols and the gather against
        # the oracle; no CPU baseline
        import oracle
        n = w["closed_form"]
        Hs = w["H"]
        Sym = oracle.discretize_bf16(Hs, w["M"])
        Ec = closed_form_streams(Sym, n)
        Eg = E.cpu().numpy()
        if not np.array_equal(Eg[:n], Ec):
            raise SystemExit("parity failure: low-entropy E differs from the closed form")
        Eo, SYMo, _ = oracle.match(Sym[n:], 1 << w["M"])
        if not np.array_equal(Eg[n:], Eo):
            raise SystemExit("parity failure: E differs from the oracle")
        Eall = np.concatenate([Ec, Eo])
        SYMw = np.where(Eall >= 0, np.take_along_axis(Sym, np.maximum(Eall + 1, 0),
                                                      1).astype(np.int16), -1)
        if not np.array_equal(SYM.cpu().numpy(), SYMw):
            raise SystemExit("parity failure: SYM differs")
        if not np.array_equal(out.cpu().numpy().view(np.uint16),
                              oracle.gather(w["V"], Eall, w["M"])):
            raise SystemExit("parity failure: gathered values differ")
        _log("parity ok (closed forms and oracle)")
    elif not args.no_cpu:
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
        _log(f"parity ok; oracle {wall:.3f} s on {threads} threads")
        what = ("discretize + match + gather" if w["kind"] == "bf16"
                and w["V"] is not None else "match")
        cpu = {"value": S * T / wall, "unit": "positions/s", "cores": threads,
               "kind": "oracle",
               "sample": f"whole workload ({S} streams x {T}), {what}, streams "
                         f"split over {threads} threads, median of 3"}
        if threads > 1:
            _log("oracle on 1 thread")
            wall1, _, _, _ = oracle_run(w, 1)
            cpu["one_thread"] = {"value": S * T / wall1, "cores": 1,
                                 "sample": f"whole workload, {what}, one "
                                           "thread, one run"}
        cpu["host"] = host_cpu_info(threads)

    line = {
        "metric": w["metric"], "value": value, "unit": "positions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u8", "data": "synthetic",
        "config": {"workload": w["desc"], "streams": S, "T": T, "K": K,
                   "parallelism": "single GPU",
                   **({"v_row_pitch": int(Vd.stride(1))} if Vd is not None else {}),
                   **({"pipeline": "streams in two halves by channel on two HIP "
                                   "streams: each half's gather and its next "
                                   "step's discretisation beside the other half's "
                                   "retrieval kernel, consecutive steps "
                                   "overlapping (each timed step discretises, "
                                   "matches and gathers all streams once)"}
                      if piped else {})},
        **({"ms_per_step_serial": ms_serial} if piped else {}),
        "roofline": roof,
        "kernel_ms": {"retrieval": k_avg,
                      **({"gather": g_avg} if g_avg is not None else {})},
        **({"dense_v_rows": dense} if dense is not None else {}),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
