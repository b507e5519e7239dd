"""Throughput of the Newton-Schulz hot path on one MI355X.

One step = the whole path over one batch: select / cost / LPT homes (ns_plan,
host), pack the row shards into their homes (one HIP launch; the route plan is
built once and reused, as the pages' cached `plan` dict is), batched 5-step
quintic Newton-Schulz on the home buffers (input staging + 15 product
launches), and unpack the results into result shards (one HIP launch). Inputs
are resident in HBM before the timed region. With --routing fused the step is
one ns_orthogonalize_routed call instead, which reads the shard buffers and
writes the result shards itself (no home buffers, no pack / unpack launches);
the mode not selected is timed as well and reported under `other_routing`.

Default workload: the dense-transformer set (32 layers x q, k, v, o 4096-wide
projections, gate, up and down 14336 x 4096 FFN weights: 224 bf16 matrices,
N(0, 0.02)), stored as 4 even row shards. Other workloads: --workload
routed-square (16 bf16 1024x1024 in 4 uneven row shards, one home empty) or
many-small (3000 random + 192 MoE matrices).

Prints ONE JSON line. `value` is matrices per second for the whole step.
`roofline` covers the dominant kernel, the one with the largest share of the
step's kernel time: its algorithmic flops (or bytes) per launch over its
average launch time, from HIP event pairs that the dispatches record
(hipExtLaunchKernelGGL: kernel execution only, as rocprofv3 reports it) in a
pass of the same steps right after the timed region, with every launch timed
as rocprofv3 times every dispatch; the timed region itself carries no events.
`cpu_baseline` times the CPU oracle (plan, pack, fp64 Newton-Schulz, unpack)
on a bounded sample of the same workload: one matrix per frequent shape plus a
seeded sample of the rest, extrapolated to the whole set by count.
"""

from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "NS matrices/sec + achieved TFLOP/s (% bf16 MFMA peak), 5-step quintic NS"
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk/CU
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
KERNEL_SRC = os.path.join(ROOT, "newton_schulz_quintic_amd", "csrc", "ns_kernels.hip")
ROUTE_SRC = os.path.join(ROOT, "newton_schulz_quintic_amd", "csrc", "route.hip")
PROFILES = os.path.join(ROOT, "profiles")
TIMING_KINDS = {0: "bx", 1: "route", 2: "norm", 3: "bx_final", 4: "syrk_x", 5: "syrk_a", 6: "small"}
# What each timing kind is, and the parts of its rocprofv3 kernel names that
# pick it (rocprofv3 gives some names mangled, some demangled). The bf16
# 256-tiles run on ns_pinned_kernel<mode, last>, the 128-tiles on
# ns_product_kernel.
PHASES = {
    "syrk_x": ("ns_pinned_kernel / ns_product_kernel<bf16, A = X X^T, upper tiles>",
               ("ELi0ELb0E", "ns_pinned_kernel<0, false>", "ns_pinned_kernelILi0ELb0E"), "mfma"),
    "syrk_a": ("ns_pinned_kernel / ns_product_kernel<bf16, B' = a I + b A + c A A, upper tiles>",
               ("ELi1ELb0E", "ns_pinned_kernel<1, false>", "ns_pinned_kernelILi1ELb0E"), "mfma"),
    "bx": ("ns_pinned_kernel / ns_product_kernel<bf16, X' = B' X>",
           ("ELi2ELb0E", "ns_pinned_kernel<2, false>", "ns_pinned_kernelILi2ELb0E"), "mfma"),
    "bx_final": ("ns_pinned_kernel / ns_product_kernel<bf16, X' = B' X, last step writes the output>",
                 ("ELi2ELb1E", "ns_pinned_kernel<2, true>", "ns_pinned_kernelILi2ELb1E"), "mfma"),
    "small": ("ns_small_kernel (every step of the matrices with m <= 128)", ("ns_small_kernel",), "mfma"),
    "norm": ("ns_prepare_kernel (input staging + norm partials)", ("ns_prepare_kernel",), "hbm"),
    "tables": ("ns_table_copy_kernel (large per-call tables to device memory)", ("ns_table_copy_kernel",), "hbm"),
    "route": ("route_copy_kernel (pack / unpack)", ("route_copy_kernel",), "hbm"),
}
WORKLOADS = ["dense-transformer", "routed-square", "many-small"]


def _code_sha256(path: str) -> str:
    """sha256 of a C/C++/HIP source with its comments and whitespace removed,
    so that only a change to the code itself marks a measurement as stale."""
    import hashlib
    import re
    with open(path, encoding="utf-8") as f:
        text = f.read()
    # string and character literals are kept whole; comments are dropped
    token = re.compile(r'"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'|//[^\n]*|/\*.*?\*/', re.S)
    code = token.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", text)
    return hashlib.sha256("".join(code.split()).encode()).hexdigest()


def counters_file(workload: str) -> str:
    return os.path.join(PROFILES, f"counters_{workload}.json")


def stored_traffic(workload: str, phase: str):
    """HBM bytes per launch of `phase` on `workload` from the committed counter
    summary, or None if it is missing or the kernel's source changed since."""
    try:
        with open(counters_file(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    src = ROUTE_SRC if phase == "route" else KERNEL_SRC
    if t.get("source_code_sha256", {}).get(os.path.basename(src)) != _code_sha256(src):
        return None
    return t.get("phases", {}).get(phase, {}).get("traffic_bytes_per_launch")


def _phase_of(kernel_name: str):
    for phase, (_, keys, _) in PHASES.items():
        if any(k in kernel_name for k in keys):
            return phase
    return None


def summarize_counters(dirs, workload: str) -> dict:
    """Per-phase counters from rocprofv3 --pmc runs (one directory per pass) of
    one bench step of `workload`: per-dispatch averages of every counter, and

      * mfma_busy = rocprofv3's MfmaUtil (the MFMA busy cycles of every SIMD
        over the GPU's active cycles times the SIMD count): the fraction of
        SIMD cycles the matrix cores were busy (clock independent);
      * mfma_flops = 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16 (rocprof's convention),
        beside the algorithmic flops of the same launch (the ratio is the
        padding and diagonal-tile work the algorithmic count leaves out);
      * traffic = FETCH_SIZE and WRITE_SIZE (KiB), each scaled by what the same
        counter reads for the pack copy kernel of the run, which reads and
        writes a known number of bytes per launch.
    """
    import csv
    import glob
    import statistics
    ms = build_workload(workload)
    vals = {}          # phase -> counter -> dispatch -> value
    names = {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    phase = _phase_of(r["Kernel_Name"])
                    if phase is None:
                        continue
                    names.setdefault(phase, r["Kernel_Name"].split("(")[0][:160])
                    c = vals.setdefault(phase, {}).setdefault(r["Counter_Name"], {})
                    c[r["Dispatch_Id"]] = c.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    avg = {p: {k: statistics.mean(v.values()) for k, v in cs.items()} for p, cs in vals.items()}
    copy_bytes = sum(_numel(s) for s in ms.shapes) * 2
    route = avg.get("route", {})
    ff = copy_bytes / 1024.0 / route["FETCH_SIZE"] if route.get("FETCH_SIZE") else None
    fw = copy_bytes / 1024.0 / route["WRITE_SIZE"] if route.get("WRITE_SIZE") else None
    flops = alg_phase_flops(ms)
    num_xcd, cus = 8, 256
    out = {"workload": ms.name, "source_code_sha256": {os.path.basename(KERNEL_SRC): _code_sha256(KERNEL_SRC),
                                                       os.path.basename(ROUTE_SRC): _code_sha256(ROUTE_SRC)},
           "copy_kernel_bytes_each_way": copy_bytes, "factor_fetch": ff, "factor_write": fw, "phases": {}}
    for phase, c in sorted(avg.items()):
        e = {"kernel": PHASES[phase][0], "symbol": names.get(phase), "dispatches": len(next(iter(vals[phase].values()))),
             "counters_per_dispatch": {k: round(v, 1) for k, v in sorted(c.items())}}
        if "MfmaUtil" in c:      # rocprofv3's own: sum of MFMA busy cycles / (max GRBM_GUI_ACTIVE x SIMDs)
            e["mfma_busy"] = round(c["MfmaUtil"] / 100.0, 4)
        elif "SQ_VALU_MFMA_BUSY_CYCLES" in c and c.get("GRBM_GUI_ACTIVE"):
            e["mfma_busy"] = round(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (4 * cus * c["GRBM_GUI_ACTIVE"] / num_xcd), 4)
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c:
            e["mfma_flops"] = 512.0 * c["SQ_INSTS_VALU_MFMA_MOPS_BF16"]
            if flops.get(phase):
                e["alg_flops"] = flops[phase]
                e["mfma_over_alg"] = round(e["mfma_flops"] / flops[phase], 4)
        if ff and fw and "FETCH_SIZE" in c and "WRITE_SIZE" in c:
            e["traffic_bytes_per_launch"] = (c["FETCH_SIZE"] * ff + c["WRITE_SIZE"] * fw) * 1024.0
        out["phases"][phase] = e
    return out


def summarize_trace(trace_dir: str, workload: str, steps: int) -> str:
    """Markdown table of a rocprofv3 --kernel-trace --stats run of bench.py:
    per phase the launches, average / min / max duration and time share, and
    for the product phases the algorithmic TFLOP/s of an average launch."""
    import csv
    import glob
    ms = build_workload(workload)
    flops = alg_phase_flops(ms)
    rows = {}
    path = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)[0]
    with open(path) as f:
        for r in csv.DictReader(f):
            phase = _phase_of(r["Name"]) or r["Name"].split("(")[0][:60]
            e = rows.setdefault(phase, [0, 0.0, float("inf"), 0.0])
            n = int(r["Calls"])
            e[0] += n
            e[1] += float(r["TotalDurationNs"])
            e[2] = min(e[2], float(r["MinNs"]))
            e[3] = max(e[3], float(r["MaxNs"]))
    total = sum(e[1] for e in rows.values())
    lines = ["| Kernel | Calls | Average (us) | Min (us) | Max (us) | Share | Algorithmic TFLOP/s (% of 2516.6) |",
             "|---|---|---|---|---|---|---|"]
    for phase, (n, tot, lo, hi) in sorted(rows.items(), key=lambda kv: -kv[1][1]):
        avg_ns = tot / n
        rate = ""
        if phase in flops and PHASES[phase][2] == "mfma":
            tf = flops[phase] / (avg_ns * 1e-9) / 1e12
            rate = f"{tf:.1f} ({100 * tf / PEAK_BF16_TFLOPS:.1f} %)"
        name = PHASES[phase][0] if phase in PHASES else phase
        lines.append(f"| {name} | {n} | {avg_ns / 1e3:.2f} | {lo / 1e3:.2f} | {hi / 1e3:.2f} | "
                     f"{100 * tot / total:.1f} % | {rate} |")
    return "\n".join(lines)


def _numel(shape) -> int:
    n = 1
    for d in shape:
        n *= int(d)
    return n


def alg_phase_flops(ms) -> dict:
    """Algorithmic flops of one launch of each product phase over the whole set."""
    c_nonzero = ms.coeffs[2] != 0.0
    fx = fa = fb = 0.0
    for s in ms.shapes:
        m, n = oriented(s)
        if m == 0:
            continue
        fx += m * (m + 1) * n
        fa += m * m * (m + 1) if c_nonzero else 0
        fb += 2 * m * m * n
    return {"syrk_x": fx, "syrk_a": fa, "bx": fb, "bx_final": fb}


def tiling_traffic(ms, phase: str):
    """HBM bytes per launch of the B'X product if every group of 4 x 8 tiles of
    256 reads each of its operand panels (256 rows x K, K rounded up to a
    64-element stage) once and writes its tiles (bf16 B'X reads X K-major and
    keeps no X'^T; the last launch writes the output itself). The measured
    FETCH_SIZE + WRITE_SIZE of these launches equal it to 0.1 %: the excess
    over the algorithmic bytes is panels shared by several groups, not
    re-reads within one. None outside that configuration (other phases, the
    small size class, too few tiles for the 256-tile configuration)."""
    if phase not in ("bx", "bx_final"):
        return None
    tile, gr, gc, es = 256, 4, 8, 2
    reads = writes = tiles = 0
    for s in ms.shapes:
        m, n = oriented(s)
        if m == 0:
            continue
        if m <= 128:
            return None
        mp, np_ = -(-m // tile) * tile, -(-n // tile) * tile
        tm, tn = mp // tile, np_ // tile
        k = -(-m // 64) * 64
        tiles += tm * tn
        for bi in range(0, tm, gr):
            for bj in range(0, tn, gc):
                reads += (min(gr, tm - bi) + min(gc, tn - bj)) * tile * k * es
        if phase == "bx":
            writes += tm * tn * tile * tile * es
        else:
            writes += m * n * es
    if tiles < 256:
        return None
    return reads + writes


def alg_flops(m: int, n: int, steps: int, c_nonzero: bool = True) -> float:
    """Algorithmic flops of one matrix: per step SYRK(X) m(m+1)n, SYRK(A) m^2(m+1)
    (skipped when c == 0), GEMM(B X) 2 m^2 n; symmetric products counted once."""
    per = m * (m + 1) * n + (m * m * (m + 1) if c_nonzero else 0) + 2 * m * m * n
    return float(steps) * per


def oriented(shape):
    rows, cols = shape[0], 1
    for d in shape[1:]:
        cols *= d
    return min(rows, cols), max(rows, cols)


def build_workload(name: str):
    from workloads import dense_transformer, even_split_rows, many_small, routed_square_batch
    if name == "routed-square":
        ms = routed_square_batch(uneven=True)
    elif name == "dense-transformer":
        ms = dense_transformer()
        ms.split_rows = [even_split_rows(s[0], 4) for s in ms.shapes]
        ms.num_shards = 4
    elif name == "many-small":
        ms = many_small()
        ms.split_rows = [even_split_rows(s[0], 4) for s in ms.shapes]
        ms.num_shards = 4
    else:
        raise SystemExit(f"unknown workload {name}")
    return ms


def make_shards(ms, device_gen: bool, shard_dim: int = 0):
    """Shard buffers (device) holding every matrix's slices along shard_dim
    (row pieces for 0), end to end."""
    import numpy as np
    import torch
    from workloads import device_matrix, host_matrix
    S = ms.num_shards
    parts = [[] for _ in range(S)]
    for i, shape in enumerate(ms.shapes):
        if device_gen:
            full = device_matrix(ms.seed, i, shape, std=ms.std)
        else:
            bits = host_matrix(ms.seed, i, shape, std=ms.std)
            full = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
        full = full.reshape(shape)
        r0 = 0
        for s in range(S):
            r = ms.split_rows[i][s]
            parts[s].append(full.narrow(shard_dim, r0, r).reshape(-1))
            r0 += r
    shards = []
    for s in range(S):
        shards.append(torch.cat(parts[s]) if parts[s] and sum(p.numel() for p in parts[s]) else None)
    torch.cuda.synchronize()
    return shards


def cpu_baseline(ms, budget_s: float):
    """The oracle on a bounded sample of the workload, extrapolated to the set.

    The sample: one matrix of every shape that makes up at least 1 % of the
    set (every shape of a set with at most 8 distinct ones), plus a seeded
    sample of up to 64 of the remaining matrices. Each sampled matrix goes
    through the oracle's plan, pack, fp64 Newton-Schulz and unpack on its own,
    repeated until about budget_s / (number of samples) of work (at least
    once); its mean time stands for every matrix it represents. The set's
    time is the sum over the sample of (time x matrices represented) plus the
    oracle planner run once on the whole set."""
    import collections
    import random

    import numpy as np
    import threadpoolctl

    from oracle import ns as ons
    from oracle import planner, route
    from workloads import host_matrix

    a, b, c = (float(np.float32(x)) for x in ms.coeffs)
    np.ones((64, 64)) @ np.ones((64, 64))      # load the BLAS so threadpoolctl sees it
    threads = sum(p.get("num_threads", 0) for p in threadpoolctl.threadpool_info()
                  if p.get("user_api") == "blas") or 1
    S = ms.num_shards
    counts = collections.Counter(tuple(s) for s in ms.shapes)
    first = {}
    for i, s in enumerate(ms.shapes):
        first.setdefault(tuple(s), i)
    frequent = {s for s, k in counts.items() if len(counts) <= 8 or k >= max(2, 0.01 * ms.n)}
    sample = [(first[s], counts[s]) for s in sorted(frequent, key=lambda s: first[s])]
    rest = [i for i, s in enumerate(ms.shapes) if tuple(s) not in frequent]
    if rest:
        picked = sorted(random.Random(0).sample(rest, min(64, len(rest))))
        sample += [(i, len(rest) / len(picked)) for i in picked]
    per_sample = budget_s / len(sample)
    t_wall = time.perf_counter()
    set_seconds, work, reps_total = 0.0, 0.0, 0
    for i, weight in sample:
        shape, split = ms.shapes[i], ms.split_rows[i]
        full = host_matrix(ms.seed, i, shape, std=ms.std)
        shards = [x.ravel() for x in np.split(full, np.cumsum(split)[:-1], axis=0)]
        spent, reps = 0.0, 0
        while reps == 0 or spent < per_sample:
            t0 = time.perf_counter()
            p = planner.plan([shape], ms.steps, S, [split])
            homes = route.pack(shards, [shape], [split], p["home"], S)
            x = ons.bf16_bits_to_f64(homes[p["home"][0]]).reshape(shape)
            y = ons.newton_schulz(x, ms.steps, a, b, c, 1e-7)
            res = [np.zeros(0)] * S
            res[p["home"][0]] = y.ravel()
            route.unpack(res, [shape], [split], p["home"], S)
            spent += time.perf_counter() - t0
            reps += 1
        set_seconds += weight * spent / reps
        work += spent
        reps_total += reps
    t0 = time.perf_counter()
    planner.plan(ms.shapes, ms.steps, S, ms.split_rows)
    t_plan = time.perf_counter() - t0
    set_seconds += t_plan
    kind = "the whole set" if len(sample) == ms.n and all(w == 1 for _, w in sample) else "extrapolated"
    return {"value": ms.n / set_seconds, "unit": "matrices/s", "cores": int(threads), "kind": "oracle",
            "extrapolated": kind == "extrapolated", "set_seconds": round(set_seconds, 3),
            "sample": (f"{len(sample)} matrices ({len(frequent)} frequent shapes, one each"
                       + (f", + {len(sample) - len(frequent)} seeded picks from the other {len(rest)}" if rest else "")
                       + f"), {reps_total} oracle runs of plan + pack + fp64 NS ({ms.steps} steps) + unpack, "
                       f"{work:.1f} s of work ({time.perf_counter() - t_wall:.1f} s wall), {kind} to the "
                       f"{ms.n}-matrix set by count, + the oracle planner on the whole set ({t_plan * 1e3:.1f} ms)")}


def wave_bench(ms, slots: int, tokens: int, reps: int) -> dict:
    """Wave dispatch against one NS call after the whole backward, on one GPU.

    The backward pass is simulated per tensor, in reverse index order (the
    order gradients become ready): two bf16 products of `tokens` rows with the
    tensor's shape (standing in for its weight- and input-gradient GEMMs),
    then the momentum update M = 0.95 M + G. Sequential: backward, then one
    ns_orthogonalize_batched call, on one stream. Waves: the backward on one
    stream records an event when each wave's last momentum is complete, and
    ns_orthogonalize_waves on a second stream starts each wave on its event.
    `tail` is the time from the end of the backward to the end of the NS work.
    """
    import torch
    import newton_schulz_quintic_amd as nsq
    from workloads import device_matrix
    dev = torch.device("cuda:0")
    mats = [device_matrix(ms.seed, i, s, std=ms.std) for i, s in enumerate(ms.shapes)]
    grads = [device_matrix(ms.seed + 1, i, s, std=ms.std) for i, s in enumerate(ms.shapes)]
    acts = {}
    for s in ms.shapes:
        acts.setdefault(s[0], torch.randn(tokens, s[0], device=dev).to(torch.bfloat16) * 0.02)
    outs = [torch.empty_like(m) for m in mats]
    wave_of, num = nsq.ns_wave_plan(ms.shapes, slots)
    order = list(range(ms.n - 1, -1, -1))
    last_of_wave = {}
    for i in order:
        last_of_wave[wave_of[i]] = i
    need, _ = nsq.ns_workspace_bytes(ms.shapes, nsq.NS_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    bwd, nss = torch.cuda.Stream(), torch.cuda.Stream()

    def backward(stream, events):
        with torch.cuda.stream(stream):
            for i in order:
                x = acts[ms.shapes[i][0]]
                w2 = mats[i].reshape(ms.shapes[i][0], -1)
                y = x @ w2                      # input-gradient stand-in
                _ = x.t().contiguous() @ y      # weight-gradient stand-in
                mats[i].mul_(0.95).add_(grads[i])
                if events is not None and last_of_wave.get(wave_of[i]) == i:
                    events[wave_of[i]].record(stream)

    def timed(fn):
        start, mid, end = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        torch.cuda.synchronize()
        start.record(torch.cuda.current_stream())
        fn(mid)
        end_ev = end
        torch.cuda.current_stream().wait_stream(bwd)
        torch.cuda.current_stream().wait_stream(nss)
        end_ev.record(torch.cuda.current_stream())
        torch.cuda.synchronize()
        return start.elapsed_time(end_ev), start.elapsed_time(mid)

    def sequential(mid):
        bwd.wait_stream(torch.cuda.current_stream())
        backward(bwd, None)
        mid.record(bwd)
        nsq.ns_orthogonalize_batched(mats, outs, steps=ms.steps, coeffs=ms.coeffs, workspace=ws, stream=bwd)

    def waves(mid):
        bwd.wait_stream(torch.cuda.current_stream())
        nss.wait_stream(torch.cuda.current_stream())
        events = [torch.cuda.Event() for _ in range(num)]
        backward(bwd, events)
        mid.record(bwd)
        nsq.ns_orthogonalize_waves(mats, outs, wave_of, num, ready_events=events, steps=ms.steps,
                                   coeffs=ms.coeffs, workspace=ws, stream=nss)

    def backward_only(mid):
        bwd.wait_stream(torch.cuda.current_stream())
        backward(bwd, None)
        mid.record(bwd)

    res = {}
    for name, fn in (("backward_only", backward_only), ("sequential", sequential), ("waves", waves)):
        fn_times = [timed(fn) for _ in range(reps + 1)][1:]    # first run warms up
        tot = sorted(t[0] for t in fn_times)[len(fn_times) // 2]
        bw = sorted(t[1] for t in fn_times)[len(fn_times) // 2]
        res[name] = {"total_ms": round(tot, 3), "backward_end_ms": round(bw, 3),
                     "tail_ms": round(tot - bw, 3)}
    return {"metric": "NS tail after the last gradient (wave dispatch vs one call after backward)",
            "unit": "ms", "config": {"workload": ms.name, "matrices": ms.n, "slots": slots,
                                     "num_waves": num, "tokens": tokens, "reps": reps},
            "backward_only_ms": res["backward_only"]["total_ms"], "sequential": res["sequential"],
            "waves": res["waves"], "data": "synthetic"}


PEAK_F32_TFLOPS = 157.3      # MI355X dense fp32 MFMA, published


def gram_flops(m: int, n: int, steps: int, c_nonzero: bool = True) -> float:
    """Algorithmic flops of Gram-space NS on one matrix: the Gram m(m+1)n
    (symmetric, counted once); step 0 (Q0 = I) one product G G; every later
    step four full m x m products (Q G, (Q G) Q, A A, B' Q), 2 m^3 each (A A
    skipped when c == 0); the output Q X0, 2 m^2 n."""
    full = 2 * m * m * m
    per_step = (4 if c_nonzero else 3) * full
    return float(m * (m + 1) * n + (full if c_nonzero else 0) + max(0, steps - 1) * per_step + 2 * m * m * n)


def gram_bench(ms, ridge: float, reps: int) -> dict:
    """Gram-space NS (fp32) and the standard bf16 NS on the same matrices, one
    call each over the whole set, inputs resident in HBM."""
    import torch
    import newton_schulz_quintic_amd as nsq
    from workloads import device_matrix
    mats = [device_matrix(ms.seed, i, s, std=ms.std) for i, s in enumerate(ms.shapes)]
    outs = [torch.empty_like(m) for m in mats]
    ws = torch.empty(max(nsq.ns_gram_workspace_bytes(ms.shapes, nsq.NS_BF16)[0],
                         nsq.ns_workspace_bytes(ms.shapes, nsq.NS_BF16)[0]), dtype=torch.uint8, device="cuda")

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            torch.cuda.synchronize()
            times.append(s.elapsed_time(e))
        return sorted(times)[len(times) // 2]

    t_gram = timed(lambda: nsq.ns_orthogonalize_gram(mats, outs, steps=ms.steps, coeffs=ms.coeffs, ridge=ridge,
                                                     workspace=ws))
    t_std = timed(lambda: nsq.ns_orthogonalize_batched(mats, outs, steps=ms.steps, coeffs=ms.coeffs, workspace=ws))
    flops = sum(gram_flops(*oriented(s), ms.steps, ms.coeffs[2] != 0.0) for s in ms.shapes)
    tf = flops / (t_gram * 1e-3) / 1e12
    return {"metric": "Gram-space NS matrices/s (fp32 products), beside the bf16 NS on the same set",
            "value": round(ms.n / (t_gram * 1e-3), 3), "unit": "matrices/s", "ms_per_call": round(t_gram, 3),
            "dtype": "f32", "data": "synthetic",
            "config": {"workload": ms.name, "matrices": ms.n, "ns_steps": ms.steps, "ridge": ridge, "reps": reps},
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_F32_TFLOPS, 4), "traffic": None,
                         "note": "whole call: algorithmic flops / call time"},
            "alg_flops_per_call": flops,
            "standard_bf16_ns": {"ms_per_call": round(t_std, 3), "value": round(ms.n / (t_std * 1e-3), 3)}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dense-transformer", choices=WORKLOADS)
    ap.add_argument("--routing", default="pack", choices=["pack", "fused"],
                    help="pack: pack -> batched NS on the home buffers -> unpack (three calls); fused: "
                         "ns_orthogonalize_routed reads and writes the shard buffers directly. The other "
                         "mode is timed too and reported under `other_routing`")
    ap.add_argument("--waves", type=int, metavar="SLOTS",
                    help="measure wave dispatch (tensors per wave = SLOTS) against one NS call after a "
                         "simulated backward; prints its own JSON line and exits")
    ap.add_argument("--gram", type=float, metavar="RIDGE",
                    help="time Gram-space NS (fp32, this trace ridge) beside the bf16 NS on the workload's "
                         "matrices; prints its own JSON line and exits")
    ap.add_argument("--tokens", type=int, default=4096, help="tokens of the simulated backward (--waves)")
    ap.add_argument("--shard-dim", type=int, default=0,
                    help="cut every tensor's shards along this dimension (0 = rows; 1 = the TP stage's "
                         "column shards, evenly over the workload's shard count); pack / unpack routing only")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work (at least one run "
                    "of each sampled matrix)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="skip the HIP-event timing of every launch")
    ap.add_argument("--no-other-routing", action="store_true", help="do not time the other routing mode")
    ap.add_argument("--counters", nargs="+", metavar="PMC_DIR",
                    help="summarise rocprofv3 --pmc runs (one directory per pass) of one step of --workload "
                         "into the per-phase counter JSON (printed) and exit")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR",
                    help="print the per-phase table of a rocprofv3 --kernel-trace --stats run of --workload and exit")
    args = ap.parse_args()
    if args.counters:
        print(json.dumps(summarize_counters(args.counters, args.workload), indent=1))
        return
    if args.trace_summary:
        print(summarize_trace(args.trace_summary, args.workload, args.steps))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the path has no cross-GPU "
              "part; how it would shard is described in the design notes.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import newton_schulz_quintic_amd as nsq

    if not os.path.exists(nsq.LIB_PATH):
        from newton_schulz_quintic_amd.build import build
        build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ms = build_workload(args.workload)
    if args.shard_dim:
        from workloads import even_split_rows
        if args.routing == "fused":
            raise SystemExit("fused routing reads row shards only; use --routing pack with --shard-dim")
        ms.split_rows = [even_split_rows(shape[args.shard_dim], ms.num_shards) for shape in ms.shapes]
        ms.name += f"-shard-dim{args.shard_dim}"
    if args.waves:
        print(json.dumps(wave_bench(ms, args.waves, args.tokens, max(1, args.steps))), flush=True)
        return
    if args.gram is not None:
        print(json.dumps(gram_bench(ms, args.gram, max(1, args.steps))), flush=True)
        return
    S = ms.num_shards
    big = args.workload != "routed-square"
    shards_in = make_shards(ms, device_gen=big, shard_dim=args.shard_dim)

    # route plan: built once, reused every step
    # homes: LPT over the row holders (ns_plan's candidates are row shards)
    p = nsq.ns_plan(ms.shapes, ms.steps, S, None if args.shard_dim else ms.split_rows)
    plan = nsq.ns_route_plan_create_axis(ms.shapes, S, ms.split_rows, [args.shard_dim] * ms.n, p["home"], 2)
    q = nsq.ns_route_plan_query(plan)
    nsq.ns_route_plan_upload(plan)
    homes = [torch.empty(n, dtype=torch.bfloat16, device=dev) if n else None for n in q["home_elems"]]
    shards_out = [torch.empty(n, dtype=torch.bfloat16, device=dev) if n else None
                  for n in q["shard_elems"]]
    views = []
    for i, shape in enumerate(ms.shapes):
        h, off = p["home"][i], q["home_offset"][i]
        numel = 1
        for d in shape:
            numel *= d
        views.append(homes[h][off:off + numel].view(shape))
    need = nsq.ns_workspace_bytes(ms.shapes, nsq.NS_BF16)[0]
    if not args.shard_dim:
        need = max(need, nsq.ns_routed_workspace_bytes(plan, nsq.NS_BF16)[0])
    workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream

    plan_split = None if args.shard_dim else ms.split_rows

    def step_pack():
        pl = nsq.ns_plan(ms.shapes, ms.steps, S, plan_split)
        nsq.ns_pack_shards(plan, shards_in, homes, stream)
        nsq.ns_orthogonalize_batched(views, views, steps=ms.steps, coeffs=ms.coeffs, order=pl["order"],
                                     workspace=workspace, stream=stream)
        nsq.ns_unpack_shards(plan, homes, shards_out, stream)

    def step_fused():
        pl = nsq.ns_plan(ms.shapes, ms.steps, S, plan_split)
        nsq.ns_orthogonalize_routed(plan, shards_in, shards_out, nsq.NS_BF16, steps=ms.steps,
                                    coeffs=ms.coeffs, order=pl["order"], workspace=workspace, stream=stream)

    step, other = (step_pack, step_fused) if args.routing == "pack" else (step_fused, step_pack)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    for k in TIMING_KINDS:
        nsq.ns_timing_read(k)           # drop anything recorded before the timed region
    # The timed region carries no instrumentation. Kernel durations come from a
    # second pass of the same steps with every launch event-timed, as
    # rocprofv3's kernel trace times every dispatch: timing one kernel alone
    # shifts work between it and its untimed neighbours (its own launches then
    # measured up to 12 % longer than rocprofv3 reports).
    # The timed loops run with Python's collector paused (after a collection):
    # a full collection landing inside a loop stalls the host for tens of ms.
    gc.collect()
    gc.disable()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    # Kernel pass: the same steps with HIP events on every launch.
    breakdown = {}
    if not args.no_kernel_timing:
        nsq.ns_timing_enable(True)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        nsq.ns_timing_enable(False)
        breakdown = {name: nsq.ns_timing_read(k) for k, name in TIMING_KINDS.items()}
    # The other routing mode, same inputs and step count, no instrumentation.
    ms_other = None
    if not args.shard_dim and not args.no_other_routing:
        for _ in range(args.warmup):
            other()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for _ in range(args.steps):
            other()
        torch.cuda.synchronize()
        ms_other = (time.perf_counter() - t2) * 1e3 / args.steps
    gc.enable()

    flops = sum(alg_flops(*oriented(s), ms.steps, ms.coeffs[2] != 0.0) for s in ms.shapes)
    dense = sum(ms.steps * (4 * m * m * n + 2 * m ** 3) for m, n in (oriented(s) for s in ms.shapes))
    tflops = flops / (ms_step * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(ms.n / (ms_step * 1e-3), 3),
        "unit": "matrices/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": ms.name, "matrices": ms.n, "distinct_shapes": len(set(ms.shapes)),
                   "shards": S, "ns_steps": ms.steps, "coeffs": list(ms.coeffs),
                   "homes_used": len(set(p["home"])), "routing": args.routing,
                   "shard_dim": args.shard_dim},
        "tflops": round(tflops, 2),
        "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "alg_flops_per_step": flops,
        "dense_equiv_flops_per_step": float(dense),
        "other_routing": None if ms_other is None else {
            "routing": "fused" if args.routing == "pack" else "pack", "ms_per_step": round(ms_other, 4),
            "value": round(ms.n / (ms_other * 1e-3), 3)},
    }
    if not args.no_kernel_timing:
        t = breakdown
        total_ms = sum(v[0] for v in t.values())
        # the dominant kernel: the largest share of the step's kernel time
        dom = max((k for k in t if t[k][1]), key=lambda k: t[k][0])
        kms, kn, kwork = t[dom]
        name, _, bound = PHASES[dom]
        avg_s = kms / kn * 1e-3
        if bound == "mfma":
            achieved, peak, unit = (kwork / kn) / avg_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
        else:
            achieved, peak, unit = (kwork / kn) / avg_s / 1e9, PEAK_HBM_GBS, "GB/s"
        out["roofline"] = {"kernel": name, "phase": dom, "bound": bound, "achieved": round(achieved, 2),
                           "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                           "traffic": stored_traffic(args.workload, dom) if not args.shard_dim else None,
                           "traffic_model": tiling_traffic(ms, dom) if bound == "mfma" else None,
                           "time_share": round(kms / total_ms, 4), "avg_launch_us": round(kms / kn * 1e3, 2),
                           ("alg_flops_per_launch" if bound == "mfma" else "alg_bytes_per_launch"): kwork / kn,
                           "launches": kn}
        phases = {}
        for name in ("syrk_x", "syrk_a", "bx", "bx_final", "small"):
            pms, pn, pwork = t[name]
            if pn:
                tf = (pwork / pn) / (pms / pn * 1e-3) / 1e12
                phases[name] = {"avg_us": round(pms / pn * 1e3, 2), "tflops": round(tf, 1),
                                "frac": round(tf / PEAK_BF16_TFLOPS, 4), "time_share": round(pms / total_ms, 4),
                                "launches": pn}
        out["product_phases"] = phases
        if phases:
            low = min(phases, key=lambda k: phases[k]["tflops"])
            out["lowest_utilisation_phase"] = low
        out["breakdown_note"] = ("roofline, product_phases, route_kernel and norm_kernels come from a second "
                                 "pass of the same steps with HIP events on every launch (kernel execution "
                                 "only); the timed region itself carries no events")
        rms, rn, rwork = t["route"]
        if rn:
            gbs = (rwork / rn) / (rms / rn * 1e-3) / 1e9
            out["route_kernel"] = {"kernel": "route_copy_kernel", "bound": "hbm",
                                   "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": round(gbs / PEAK_HBM_GBS, 4),
                                   "avg_launch_us": round(rms / rn * 1e3, 2),
                                   "bytes_per_launch": rwork / rn,
                                   "note": "working set fits the 256 MB MALL" if rwork / rn < 256e6
                                   else "working set exceeds the MALL"}
        nms, nn, nwork = t["norm"]
        if nn:
            ngbs = nwork / (nms * 1e-3) / 1e9
            out["norm_kernels"] = {"kernel": "ns_prepare_kernel (input staging + norm partials; with large tables "
                                             "a table copy launch before it)", "bound": "hbm",
                                   "us_per_step": round(nms / args.steps * 1e3, 2),
                                   "bytes_per_step": nwork / args.steps, "launches_per_step": nn / args.steps,
                                   "achieved": round(ngbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": round(ngbs / PEAK_HBM_GBS, 4)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(ms, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
