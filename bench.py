#!/usr/bin/env python3
"""Benchmark one GPU's share of an Echo all-reduce call.

A step is one rank's share of one call, i.e. the whole hot path on one GPU:
  entry pass (feedback-add + quantize the P-1 non-owned segments + state),
  owner pass (dequantize P-1 incoming payloads + fp32 sum + requantize +
  state), dequantize pass (P gathered payloads -> 16-bit output).
The other P-1 ranks are simulated on the same device: their payloads are
produced by the same library before timing.  Inputs are resident in HBM.

value = effective all-reduce bandwidth = 2 bytes * n / step time (16-bit
input bytes per second), the metric the method is quoted on; hbm_frac is
the algorithmic bytes per step over MI355X's 8 TB/s.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--site S]
                       [--state f32|bf16] [--group G] [--graph] [--rotate K]
       python bench.py --n N [--ranks P] [--bits 4|8] ...   (any message size)
       python bench.py --copy-calibration BYTES     (plain copy for PMC scaling)
       python bench.py --summarize-profiles DIR     (rocprofv3 CSVs -> profiles/)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, AMD's published peak
METRIC = "effective all-reduce GB/s per GPU (16-bit input bytes/s) and % of HBM peak"
KERNELS = ("k_quant_feedback", "k_owner_reduce_requant", "k_dequant_gather")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def payload_bytes_per_elem(bits: int, group: int = 128) -> float:
    return bits / 8 + 4 / group


def algorithmic_bytes(P: int, n: int, bits: int, state_bytes: int, in_bytes=2, out_bytes=2,
                      group: int = 128):
    """Bytes each kernel must move per launch (one rank's share):
    entry: (P-1)/P of x, S and L read, S and L written, P-1 payloads written;
    owner: 1/P of x, S, L read and S, L written, P-1 payloads read, one written;
    gather: P payloads read, n outputs written."""
    seg = n // P
    pb = payload_bytes_per_elem(bits, group)
    st = 4 * state_bytes   # S and L, read and written
    k1 = (P - 1) * seg * (in_bytes + st + pb)
    k2 = seg * (in_bytes + st + (P - 1) * pb + pb)
    k3 = n * (pb + out_bytes)
    return {"k_quant_feedback": k1, "k_owner_reduce_requant": k2, "k_dequant_gather": k3}


def kernel_source_digest() -> str:
    """Digest of what determines the kernels' code: their source, the header
    they include and the compiler flags (not the argument-checking layer).
    Paths in the flags are taken relative to the repository, so the digest
    does not depend on where the repository sits."""
    from error_compensated_bit_amd import build as eb
    h = hashlib.sha256()
    for f in (os.path.join(eb.CSRC, "echo_kernels.hip"), os.path.join(eb.CSRC, "echo_internal.h")):
        h.update(open(f, "rb").read())
    flags = [os.path.relpath(f, HERE) if os.path.isabs(f) else f for f in eb.hipcc_flags()]
    h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


def input_digests(xs):
    """SHA-256 (first 16 hex digits) of every rank's input bytes: the bytes,
    not the seeds, define a run's input."""
    import torch
    out = []
    for x in xs:
        h = hashlib.sha256()
        flat = x.reshape(-1)
        for i in range(0, flat.numel(), 1 << 27):
            h.update(flat[i:i + (1 << 27)].view(torch.int16).cpu().numpy().tobytes())
        out.append(h.hexdigest()[:16])
    return out


# bench.py's default launch configuration (what a plain `python bench.py` runs).
DEFAULT_CONFIG = {"state": "f32", "group": 128, "site": 0, "rank": 0}


def profile_key(workload: str, config: dict) -> str:
    """Name of a workload + launch configuration in profiles/: the workload,
    then every setting that differs from the default."""
    extra = [f"{k}-{config[k]}" for k in DEFAULT_CONFIG if config.get(k, DEFAULT_CONFIG[k]) != DEFAULT_CONFIG[k]]
    return "_".join([workload] + extra)


def bench_args(workload: str, config: dict) -> str:
    c = {**DEFAULT_CONFIG, **config}
    return (f"--workload {workload} --site {c['site']} --rank {c['rank']} --state {c['state']} "
            f"--group {c['group']}")


def profile_commands(workload: str, config: dict) -> dict:
    """rocprofv3 runs whose CSVs --summarize-profiles reduces (DIR = their
    output folder; run from the repository root after `cd /tmp && export
    TMPDIR=/tmp`)."""
    a = bench_args(workload, config)
    return {
        "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d DIR/prof_trace -o bench -- "
                 f"python3 bench.py {a} --steps 10 --warmup 2 --no-cpu-baseline",
        "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/pmc_FETCH_SIZE -o bench -- "
                 f"python3 bench.py {a} --steps 2 --warmup 0 --no-cpu-baseline",
        "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/pmc_WRITE_SIZE -o bench -- "
                 f"python3 bench.py {a} --steps 2 --warmup 0 --no-cpu-baseline",
        "copy_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/pmc_copy_FETCH_SIZE -o copy -- "
                      "python3 bench.py --copy-calibration 1073741824",
        "copy_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/pmc_copy_WRITE_SIZE -o copy -- "
                      "python3 bench.py --copy-calibration 1073741824",
    }


def traffic_from_profile(workload: str, kernel: str, config: dict):
    """HBM bytes per launch measured by rocprofv3 FETCH_SIZE / WRITE_SIZE,
    scaled by the same counters on a plain copy of known size; None when no
    summary in profiles/ covers this workload and launch configuration for
    the current kernel source."""
    import glob
    config = {**DEFAULT_CONFIG, **config}
    digest = kernel_source_digest()
    for path in sorted(glob.glob(os.path.join(HERE, "profiles", "pmc_*.json"))):
        d = json.load(open(path))
        if d.get("workload") != workload or d.get("kernel_source_digest") != digest:
            continue
        if {**DEFAULT_CONFIG, **d.get("config", {})} != config:
            continue
        k = d["kernels"].get(kernel)
        c = d["copy_calibration"]
        if not k or not c:
            return None
        fr = c["bytes_read"] / (c["fetch_kib"] * 1024.0)
        fw = c["bytes_written"] / (c["write_kib"] * 1024.0)
        return k["fetch_kib"] * 1024.0 * fr + k["write_kib"] * 1024.0 * fw
    return None


def _kernel_key(name: str) -> str:
    base = name.split("(")[0].split("<")[0]
    return base.replace("void ", "").split("::")[-1]


def summarize_profiles(d: str, workload: str, config: dict, copy_bytes: int = 1 << 30):
    """Reduce the rocprofv3 CSVs of profile_commands(workload, config) (run on
    the machine with the GPU, DIR = their output folder) to
    profiles/pmc_<key>.json and profiles/kernels_<key>.md."""
    import csv
    from collections import defaultdict
    from error_compensated_bit_amd.inputs import WORKLOADS

    config = {**DEFAULT_CONFIG, **config}
    key = profile_key(workload, config)

    def counters(path):
        acc = defaultdict(list)
        for r in csv.DictReader(open(path)):
            acc[_kernel_key(r["Kernel_Name"])].append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}

    fetch, nf = counters(os.path.join(d, "pmc_FETCH_SIZE", "bench_counter_collection.csv"))
    write, _ = counters(os.path.join(d, "pmc_WRITE_SIZE", "bench_counter_collection.csv"))
    cfetch, _ = counters(os.path.join(d, "pmc_copy_FETCH_SIZE", "copy_counter_collection.csv"))
    cwrite, _ = counters(os.path.join(d, "pmc_copy_WRITE_SIZE", "copy_counter_collection.csv"))
    copy_key = next(k for k in cfetch if "copy" in k.lower())   # the copy, not the fill before it
    trace = {}
    for r in csv.DictReader(open(os.path.join(d, "prof_trace", "bench_kernel_stats.csv"))):
        trace[_kernel_key(r["Name"])] = {"calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                                         "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3}
    w = WORKLOADS[workload]
    bits = w.bits(config["site"])
    sbytes = 4 if config["state"] == "f32" else 2
    alg = algorithmic_bytes(w.P, w.n, bits, sbytes, group=config["group"])
    cmds = profile_commands(workload, config)
    out = {
        "workload": workload,
        "config": config,
        "bits": bits,
        "kernel_source_digest": kernel_source_digest(),
        "commands": cmds,
        "copy_calibration": {"kernel": copy_key, "bytes_read": copy_bytes, "bytes_written": copy_bytes,
                             "fetch_kib": cfetch[copy_key], "write_kib": cwrite[copy_key]},
        "kernels": {k: {"fetch_kib": fetch[k], "write_kib": write[k], "dispatches": nf[k]}
                    for k in KERNELS if k in fetch},
        "trace": {k: trace[k] for k in KERNELS if k in trace},
    }
    os.makedirs(os.path.join(HERE, "profiles"), exist_ok=True)
    json.dump(out, open(os.path.join(HERE, "profiles", f"pmc_{key}.json"), "w"), indent=1)
    fr = copy_bytes / (cfetch[copy_key] * 1024)
    fw = copy_bytes / (cwrite[copy_key] * 1024)
    lines = [f"# Kernel profile: one rank's share, {w.description}",
             "",
             f"Launch configuration: site {config['site']} ({bits}-bit codes), rank {config['rank']}, "
             f"{config['state']} error state, group {config['group']}, bf16 input and output.",
             "",
             f"Kernel source digest `{out['kernel_source_digest']}` (sources + hipcc flags, "
             "`bench.py kernel_source_digest()`). Commands, run from the repository root with "
             "`cd /tmp && export TMPDIR=/tmp` first (DIR = output folder):",
             ""]
    lines += [f"- {k}: `{v}`" for k, v in cmds.items()]
    lines += ["", f"Reduced with `python bench.py --summarize-profiles DIR {bench_args(workload, config)}`. "
              f"Copy calibration (`{copy_key}`, {copy_bytes} B read and written): FETCH_SIZE reads "
              f"{cfetch[copy_key]:.0f} KiB (read factor {fr:.4f}), WRITE_SIZE "
              f"{cwrite[copy_key]:.0f} KiB (write factor {fw:.4f}).", "",
              "| kernel | trace avg µs (calls) | algorithmic GB | HBM read GB | HBM write GB | "
              "HBM total / algorithmic | algorithmic GB/s at trace avg | % of 8 TB/s |",
              "|---|---|---|---|---|---|---|---|"]
    for k in KERNELS:
        if k not in fetch or k not in trace:
            continue
        rd = fetch[k] * 1024 * fr
        wr = write[k] * 1024 * fw
        t = trace[k]["avg_us"]
        lines.append(f"| `{k}` | {t:.1f} ({trace[k]['calls']}) | {alg[k] / 1e9:.4f} | {rd / 1e9:.4f} | "
                     f"{wr / 1e9:.4f} | {(rd + wr) / alg[k]:.4f} | {alg[k] / t / 1e3:.1f} | "
                     f"{alg[k] / t / 1e3 / HBM_PEAK_GBS:.1%} |")
    lines += ["", "Counter values are means over all dispatches of a kernel (the set-up call over "
              "all ranks and the timed steps have the same sizes). FETCH_SIZE and WRITE_SIZE count "
              "the L2's traffic to the memory fabric, which includes what the memory-side "
              "Infinity Cache serves."]
    open(os.path.join(HERE, "profiles", f"kernels_{key}.md"), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def copy_calibration(nbytes: int):
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {nbytes} bytes read and written per launch, 3 launches")


def host_cpu() -> str:
    """The host's CPU model and logical CPU count, for the baseline's record."""
    model = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return f"{model}, {os.cpu_count()} logical CPUs ({usable} usable by this process)"


def usable_cpus() -> int:
    """Logical CPUs this process may run on, at most 16 (the host share that
    goes with one GPU on the measuring machines)."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return max(1, min(avail, 16))


def cpu_baseline(cfg, w, xs_dev, frac_den: int):
    """The CPU oracle on a bounded sample: the first 1/frac_den of every
    segment of every rank, one call from an empty state, all P ranks.

    Timed twice on the same sample.  Single-threaded: one rank's share = mean
    entry pass + mean owner pass + one gather (the median of several runs
    when one run is short).  Parallel, on every usable CPU: every group of a
    call is independent of the others, so the sample is cut into slices of
    whole groups (the same groups of every segment) and each slice -- a
    smaller message of all P ranks -- goes through the oracle's three passes
    for every rank on a thread pool (the oracle's C calls release the
    interpreter lock).  The host's throughput is P shares of input over the
    wall time.  The slices' outputs, put back together, must equal the
    single-threaded output bit for bit.  `value` is the parallel figure."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import oracle as O
    from error_compensated_bit_amd.inputs import bits16_numpy
    P, n = w.P, w.n
    G = cfg.group
    seg = n // P
    sseg = max(G, (seg // frac_den) // G * G)
    ns = sseg * P
    xs = []
    for x in xs_dev:
        xs.append(np.concatenate([bits16_numpy(x[o * seg:o * seg + sseg]) for o in range(P)]))
    ocfg = O.Config(bits=cfg.bits, group=cfg.group, eta=cfg.eta, beta_short=cfg.beta_short,
                    beta_long=cfg.beta_long, mix_long=cfg.mix_long, in_dtype=cfg.in_dtype,
                    out_dtype=cfg.out_dtype, state_dtype=cfg.state_dtype)

    def fresh(m):
        Ss = [np.zeros(m, O.state_np_dtype(ocfg)) for _ in range(P)]
        Ls = [np.zeros(m, O.state_np_dtype(ocfg)) for _ in range(P)]
        return Ss, Ls

    def entry(xm, p, Ss, Ls, sent):
        O.quantize_feedback(ocfg, P, p, xm[p], Ss[p], Ls[p],
                            [None if o == p else sent[p][o][0] for o in range(P)],
                            [None if o == p else sent[p][o][1] for o in range(P)])

    def owner(xm, o, Ss, Ls, sent, owned):
        O.owner_reduce_requant(ocfg, P, o, xm[o], Ss[o], Ls[o],
                               [None if p == o else sent[p][o][0] for p in range(P)],
                               [None if p == o else sent[p][o][1] for p in range(P)],
                               owned[o][0], owned[o][1])

    def gather(m, owned):
        return O.dequant_gather(ocfg, P, m, [c for c, _ in owned], [q for _, q in owned])

    def single_run():
        Ss, Ls = fresh(ns)
        sent = [[None if o == p else O.new_payload(ocfg, sseg) for o in range(P)] for p in range(P)]
        owned = [O.new_payload(ocfg, sseg) for _ in range(P)]
        t0 = time.perf_counter()
        for p in range(P):
            entry(xs, p, Ss, Ls, sent)
        t1 = time.perf_counter()
        for o in range(P):
            owner(xs, o, Ss, Ls, sent, owned)
        t2 = time.perf_counter()
        out = gather(ns, owned)
        t3 = time.perf_counter()
        return (t1 - t0) / P, (t2 - t1) / P, t3 - t2, out

    runs = [single_run()]
    while sum(r[0] + r[1] + r[2] for r in runs) < 1.0 and len(runs) < 20:
        runs.append(single_run())
    shares = sorted(runs, key=lambda r: r[0] + r[1] + r[2])
    t_entry, t_owner, t_gather, out1 = shares[len(shares) // 2]
    t_share = t_entry + t_owner + t_gather
    single = 2.0 * ns / t_share / 1e9

    # parallel: slices of whole groups, the same groups of every segment
    T = usable_cpus()
    gps = sseg // G
    nsl = max(1, min(4 * T, gps // 16))     # at least 16 groups per slice
    bounds = [(gps * i // nsl, gps * (i + 1) // nsl) for i in range(nsl)]
    slice_x = []
    for lo, hi in bounds:
        slice_x.append([np.concatenate([x[o * sseg + lo * G:o * sseg + hi * G] for o in range(P)])
                        for x in xs])

    def run_slice(i):
        lo, hi = bounds[i]
        m = (hi - lo) * G * P
        xm = slice_x[i]
        Ss, Ls = fresh(m)
        sent = [[None if o == p else O.new_payload(ocfg, m // P) for o in range(P)] for p in range(P)]
        owned = [O.new_payload(ocfg, m // P) for _ in range(P)]
        for p in range(P):
            entry(xm, p, Ss, Ls, sent)
        for o in range(P):
            owner(xm, o, Ss, Ls, sent, owned)
        return gather(m, owned)

    par_times = []
    with ThreadPoolExecutor(max_workers=T) as pool:
        while not par_times or (sum(par_times) < 1.0 and len(par_times) < 20):
            t0 = time.perf_counter()
            outs = list(pool.map(run_slice, range(nsl)))
            par_times.append(time.perf_counter() - t0)
    t_par = sorted(par_times)[len(par_times) // 2]
    joined = np.empty_like(out1)
    for (lo, hi), o_sl in zip(bounds, outs):
        k = (hi - lo) * G
        for o in range(P):
            joined[o * sseg + lo * G:o * sseg + hi * G] = o_sl[o * k:(o + 1) * k]
    if not np.array_equal(joined.view(np.uint8), out1.view(np.uint8)):
        raise RuntimeError("parallel oracle run disagrees with the single-threaded one")
    par = P * 2.0 * ns / t_par / 1e9
    return {"value": round(par, 4), "unit": "GB/s", "cores": T, "kind": "oracle",
            "single_core_value": round(single, 4),
            "sample": f"first {sseg} elements of every segment ({ns} of {n} elements per rank), "
                      f"all {P} ranks, one call from an empty state. Parallel: {nsl} slices of "
                      f"whole groups, each a message of all {P} ranks through the entry, owner and "
                      f"gather passes, on {T} threads: {t_par:.3f} s wall for {P} shares "
                      f"(median of {len(par_times)} run(s)). "
                      f"Single-threaded (median of {len(runs)} run(s)): one share {t_share:.3f} s "
                      f"(entry {t_entry:.3f} + owner {t_owner:.3f} + gather {t_gather:.3f}) "
                      f"= {single:.4f} GB/s. Scalar C oracle. Host: {host_cpu()}."}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="msg1gib_p8")
    ap.add_argument("--n", type=int, default=0,
                    help="instead of a named workload: a message of N bf16 elements per rank, "
                         "iid N(0,1), one call (N a multiple of ranks * group)")
    ap.add_argument("--ranks", type=int, default=8, help="simulated ranks P with --n")
    ap.add_argument("--bits", type=int, choices=(4, 8), default=4, help="code width with --n")
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--site", type=int, default=0,
                    help="call of a chained workload whose inputs and width are used")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph (launch-bound messages)")
    ap.add_argument("--rotate", type=int, default=1, metavar="K",
                    help="time steps over K independent copies of every buffer in turn (no cache "
                         "reuse between consecutive steps of a mid-size message)")
    ap.add_argument("--state", choices=("f32", "bf16"), default="f32")
    ap.add_argument("--group", type=int, choices=(32, 64, 128), default=128)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-den", type=int, default=0,
                    help="oracle sample = 1/DEN of every segment (default: about 10 s of CPU work)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--summarize-profiles", metavar="DIR")
    args = ap.parse_args()

    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.workload,
                           {"state": args.state, "group": args.group, "site": args.site,
                            "rank": args.rank})
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the all-reduce (the other ranks are "
              "simulated on the same device); only --gpus 1 is supported.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    from error_compensated_bit_amd import binding as B
    from error_compensated_bit_amd import sim
    from error_compensated_bit_amd.inputs import WORKLOADS, Workload, make_x

    B.load_library()
    if args.n:
        if args.n % (args.ranks * args.group) or not 1 <= args.ranks <= B.ECHO_MAX_RANKS:
            sys.exit(f"--n must be a positive multiple of ranks * group ({args.ranks} * {args.group})")
        w = Workload(f"custom_p{args.ranks}_n{args.n}", 90, args.ranks, (args.n,), "normal", 1,
                     (1, args.bits, args.bits),
                     description=f"{args.n} bf16 elements per rank, P={args.ranks}, iid N(0,1)")
    else:
        w = WORKLOADS[args.workload]
    P, n = w.P, w.n
    bits = w.bits(args.site)
    sdt = B.ECHO_STATE_F32 if args.state == "f32" else B.ECHO_STATE_BF16
    cfg = B.make_config(bits=bits, state_dtype=sdt, group=args.group)
    dev = "cuda:0"
    log(f"workload {w.name}: {w.description}; site {args.site}, rank {args.rank} of {P}, n={n}, "
        f"bits={bits}, state={args.state}")

    t_setup = time.perf_counter()
    xs = [make_x(w, args.site, p, device=dev) for p in range(P)]
    # --rotate K: K independent copies of every buffer, used in turn, so that a
    # step finds nothing of the previous steps in the caches
    sets = []
    for i in range(args.rotate):
        xs_i = xs if i == 0 else [x.clone() for x in xs]
        r_i = sim.alloc_ranks(cfg, P, n, dev)
        sim.allreduce(cfg, r_i, xs_i)          # every rank's payloads exist before timing
        sets.append((xs_i, r_i))
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t_setup:.1f} s ({args.rotate} buffer set(s))")

    rank = args.rank
    stream = torch.cuda.current_stream()
    alg = algorithmic_bytes(P, n, bits, 4 if sdt == B.ECHO_STATE_F32 else 2, group=args.group)
    alg_total = sum(alg.values())
    dom = max(KERNELS, key=lambda k: alg[k])     # the kernel that moves the most bytes
    jdom = KERNELS.index(dom)

    def prepare(i, st):
        """The three calls of one buffer set's step, marshalled once."""
        xs_i, r = sets[i]
        x = xs_i[rank]
        inp = [None if p == rank else r.sent[p][rank] for p in range(P)]
        return (B.prepare_quantize_feedback(cfg, P, rank, n, x, r.state[rank], r.sent[rank], st),
                B.prepare_owner_reduce_requant(cfg, P, rank, n, x, r.state[rank], inp, r.owned[rank], st),
                B.prepare_dequant_gather(cfg, P, n, r.owned, r.out, st))

    calls = [prepare(i, stream) for i in range(len(sets))]

    def step(i, ev=None):
        """One rank's share.  ev: two events bracketing the dominant kernel, or
        four events around the three kernels."""
        ks = calls[i % len(calls)]
        for j, k in enumerate(ks):
            if ev is not None and (len(ev) == 4 or j == jdom):
                ev[0 if len(ev) == 2 else j].record(stream)
            k()
            if ev is not None and len(ev) == 4 and j == 2:
                ev[3].record(stream)
            elif ev is not None and len(ev) == 2 and j == jdom:
                ev[1].record(stream)

    for i in range(args.warmup):
        step(i)
    # timed region: the K steps.  Two events bracket the dominant kernel on
    # every `stride`-th step (about 20 samples): an event between two short
    # kernels costs the stream a few microseconds, so a mid-size or small
    # message is not bracketed on every step.
    stride = max(1, args.steps // 20)
    events = {i: [torch.cuda.Event(enable_timing=True) for _ in range(2)]
              for i in range(0, args.steps, stride)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_ms = sum(ev[0].elapsed_time(ev[1]) for ev in events.values()) / len(events)
    ms_per_step = wall * 1e3 / args.steps
    ms_eager = ms_per_step
    # per-kernel split, untimed: the same steps with events around every kernel
    events4 = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, events4[i])
    torch.cuda.synchronize()
    k_ms = {k: sum(ev[j].elapsed_time(ev[j + 1]) for ev in events4) / args.steps
            for j, k in enumerate(KERNELS)}
    ev_steps = sorted(ev[0].elapsed_time(ev[3]) for ev in events4)
    ms_graph = None
    if args.graph:
        # one step per buffer set captured once and replayed (no memset nodes)
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            cap = torch.cuda.current_stream()
            for i in range(len(sets)):
                for k in prepare(i, cap):
                    k()
        replays = max(1, -(-args.steps // len(sets)))
        for _ in range(max(1, args.warmup // len(sets))):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(replays):
            g.replay()
        torch.cuda.synchronize()
        ms_graph = (time.perf_counter() - t0) * 1e3 / (replays * len(sets))
        log(f"  step {ms_graph:.4f} ms wall as a graph replay (eager {ms_eager:.4f} ms)")
    for k in KERNELS:
        log(f"  {k:24s} {k_ms[k]:8.4f} ms  {alg[k] / k_ms[k] / 1e6:8.1f} GB/s algorithmic "
            f"({alg[k] / k_ms[k] / 1e6 / HBM_PEAK_GBS:.1%} of HBM peak)")
    log(f"  step {ms_per_step:.4f} ms wall, {sum(k_ms.values()):.4f} ms in kernels")

    achieved = alg[dom] / dom_ms / 1e6
    traffic = traffic_from_profile(w.name, dom, {"state": args.state, "group": args.group,
                                                 "site": args.site, "rank": args.rank})
    value = 2.0 * n / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "hbm_frac": round(alg_total / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "config": {"workload": w.name, "site": args.site, "P": P, "n_per_rank": n, "rank": rank,
                   "buffer_sets": args.rotate,
                   "bits": bits,
                   "group": args.group, "state": args.state, "input": "bf16", "output": "bf16",
                   "eta": cfg.eta, "beta_short": cfg.beta_short, "beta_long": cfg.beta_long,
                   "mix_long": round(cfg.mix_long, 6),
                   "algorithmic_bytes_per_step": int(alg_total),
                   "input_sha256": input_digests(xs),
                   "kernel_source_digest": kernel_source_digest()},
        "kernel_ms": {k: round(v, 5) for k, v in k_ms.items()},
        "ms_per_step_eager": round(ms_eager, 5),
        "ms_step_events": {"median": round(statistics.median(ev_steps), 5),
                           "min": round(ev_steps[0], 5)},
        "ms_dominant_kernel_events": round(dom_ms, 5),
        "dominant_kernel_samples": len(events),
        "ms_per_step_graph": None if ms_graph is None else round(ms_graph, 5),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "algorithmic_bytes": int(alg[dom])},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on a sample ...")
        den = args.cpu_sample_den or max(1, round(n * P / 5.4e8))
        line["cpu_baseline"] = cpu_baseline(cfg, w, xs, den)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
