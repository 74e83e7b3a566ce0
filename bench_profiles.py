"""Summaries of rocprofv3 runs of bench.py, written to profiles/.

For one workload, four profiler runs of the same bench command (one
workload's rounds only, no extras, no host baseline) are summarised:

  stats  rocprofv3 --kernel-trace --stats            -> kernel_stats_<config>.md
  fetch  rocprofv3 --pmc FETCH_SIZE                  \\
  write  rocprofv3 --pmc WRITE_SIZE                   > traffic_<config>.txt
  mfma   rocprofv3 --pmc MfmaUtil MfmaFlopsBF16       -> mfma_<config>.txt
                 SQ_INSTS_MFMA

each with ``--output-format csv -d <dir>/<run> -o run``.  Usage:

  python bench_profiles.py <config> <dir>

Only the dispatches of the timed drafting rounds count: from the first
attention launch on (the untimed context fill, which runs inject_kv over
large slices, comes before it).  Each call's kernels are the library's
kernels of that call (inject_kv: ik_*, draft_block_attn: attn_*,
verify_block: vb_*) launched at least half as often as the call's most
launched kernel; each kernel's figure is its average over the dispatches
at its most frequent grid, and a call's figure is the sum over its kernels
(each runs once per call).

HBM bytes: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by what
the same counters read for a plain 256 MiB device copy that bench.py runs
after the rounds (``--copy-calibration``): the copy reads and writes
exactly 256 MiB.

MFMA use: the tool's derived MfmaUtil (MFMA busy cycles over the GPU-active
cycles of the dispatch times the SIMD count) and MfmaFlopsBF16 (bf16 matrix
flops executed); bench.py divides the latter by the call's time.
"""
import csv
import os
import statistics
import sys
from collections import Counter, defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
from bench import KERNEL_SOURCES, source_sha  # noqa: E402

# call -> the name prefixes of its kernels in the round (the weight-streaming
# GEMM runs the projection of up to 256 rows; nothing else in a round uses it)
CALLS = {
    "inject_kv": ("bd::ik_", "bd::fg_gemm"),
    "draft_block_attn": ("bd::attn_",),
    "verify_block": ("bd::vb_",),
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_KIB = 262144.0  # the calibration copy: 256 MiB read and 256 MiB written


def short(name):
    """Kernel name without the return type and the argument list."""
    name = name.strip()
    if name.startswith("void "):
        name = name[5:]
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def call_of(name):
    for call, prefixes in CALLS.items():
        if name.startswith(prefixes):
            return call
    return None


def read_csv(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def round_window(rows, name_key="Kernel_Name"):
    """Rows from the first attention dispatch on."""
    t0 = min(int(r["Start_Timestamp"]) for r in rows if short(r[name_key]).startswith("bd::attn_partial"))
    return [r for r in rows if int(r["Start_Timestamp"]) >= t0]


def call_kernels(launches):
    """launches: {(kernel, grid): count} in the window -> {call: [(kernel, grid, count)]}:
    per kernel its most frequent grid, and per call the kernels launched at
    least half as often as the call's most launched one."""
    best = {}
    for (k, g), n in launches.items():
        if k not in best or n > best[k][1]:
            best[k] = (g, n)
    out = defaultdict(list)
    for k, (g, n) in best.items():
        c = call_of(k)
        if c is not None:
            out[c].append((k, g, n))
    for c in out:
        top = max(n for _, _, n in out[c])
        out[c] = sorted([x for x in out[c] if 2 * x[2] >= top])
    return out


def counter_table(path):
    """{(kernel, grid, counter): [values per dispatch]}, launches {(kernel, grid): count},
    and the copy calibration's values {counter: KiB}."""
    rows = read_csv(path)
    copy = defaultdict(list)
    for r in rows:
        if short(r["Kernel_Name"]) == COPY_KERNEL:
            copy[r["Counter_Name"]].append((int(r["Grid_Size"]), float(r["Counter_Value"])))
    win = round_window(rows)
    vals = defaultdict(list)
    disp = defaultdict(set)
    for r in win:
        k, g = short(r["Kernel_Name"]), int(r["Grid_Size"])
        vals[(k, g, r["Counter_Name"])].append(float(r["Counter_Value"]))
        disp[(k, g)].add(r["Dispatch_Id"])
    launches = {kg: len(d) for kg, d in disp.items()}
    # the calibration copy is the largest copy dispatch of the run
    cal = {}
    for c, v in copy.items():
        cal[c] = max(v)[1]
    return vals, launches, cal


def traffic(config, d):
    fv, fl, fc = counter_table(os.path.join(d, "fetch", "run_counter_collection.csv"))
    wv, wl, wc = counter_table(os.path.join(d, "write", "run_counter_collection.csv"))
    cf = COPY_KIB / fc["FETCH_SIZE"]
    cw = COPY_KIB / wc["WRITE_SIZE"]
    kf, kw = call_kernels(fl), call_kernels(wl)
    cmd = ("python3 <repo>/bench.py --config {c} --no-other-configs --no-extras --no-cpu-baseline --no-graph "
           "--steps 3 --warmup 1 --copy-calibration").format(c=config)
    lines = [f"# HBM traffic per call, {config} round, from rocprofv3 counters (MI355X)",
             f"# pass 1: cd /tmp && TMPDIR=/tmp rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/fetch -o run -- {cmd}",
             f"# pass 2: cd /tmp && TMPDIR=/tmp rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/write -o run -- {cmd}",
             f"# summary: python3 bench_profiles.py {config} <dir>",
             f"# copy calibration (256 MiB device copy, {COPY_KERNEL}): FETCH_SIZE {fc['FETCH_SIZE']:.1f} KiB -> factor "
             f"{cf:.4f}; WRITE_SIZE {wc['WRITE_SIZE']:.1f} KiB -> factor {cw:.4f}",
             "# dispatches from the first attention launch on; bytes_per_call = sum over the call's kernels of "
             "(FETCH_SIZE * fetch factor + WRITE_SIZE * write factor) * 1024, each kernel averaged over its "
             "dispatches at its most frequent grid; source_sha = sha256[:16] of the kernel sources measured"]
    for call in CALLS:
        src = KERNEL_SOURCES[call]
        if call not in kf or call not in kw:
            continue
        tot, parts = 0.0, []
        for (k, g, _), (k2, g2, _) in zip(kf[call], kw[call]):
            assert (k, g) == (k2, g2), (k, g, k2, g2)
            f = statistics.fmean(fv[(k, g, "FETCH_SIZE")]) * cf * 1024
            w = statistics.fmean(wv[(k, g, "WRITE_SIZE")]) * cw * 1024
            tot += f + w
            parts.append(f"{k.replace(' ', '')}[grid={g}]:read={f / 1e6:.1f}MB,write={w / 1e6:.1f}MB")
        lines.append(f"{call} source_sha={source_sha(src)} bytes_per_call={tot:.0f} kernels={';'.join(parts)}")
    return lines


def mfma(config, d):
    v, l, _ = counter_table(os.path.join(d, "mfma", "run_counter_collection.csv"))
    kk = call_kernels(l)
    cmd = ("python3 <repo>/bench.py --config {c} --no-other-configs --no-extras --no-cpu-baseline --no-graph "
           "--steps 3 --warmup 1").format(c=config)
    lines = [f"# MFMA use per call, {config} round, from rocprofv3 counters (MI355X)",
             "# command: cd /tmp && TMPDIR=/tmp rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 SQ_INSTS_MFMA "
             f"--output-format csv -d <dir>/mfma -o run -- {cmd}",
             f"# summary: python3 bench_profiles.py {config} <dir>",
             "# util = the tool's MfmaUtil / 100 (MFMA busy cycles summed over SIMDs over the dispatch's GPU-active "
             "cycles x SIMDs) of the call's matrix kernels, weighted by their MFMA instructions; exec_flops = bf16 "
             "matrix flops executed per call (MfmaFlopsBF16, 512 per counted operation), summed over the call's "
             "kernels"]
    for call in CALLS:
        src = KERNEL_SOURCES[call]
        flops = util_w = n_w = 0.0
        parts = []
        for k, g, _ in kk.get(call, []):
            n = statistics.fmean(v[(k, g, "SQ_INSTS_MFMA")])
            if n <= 0:
                continue
            u = statistics.fmean(v[(k, g, "MfmaUtil")]) / 100
            f = statistics.fmean(v[(k, g, "MfmaFlopsBF16")])
            flops += f
            util_w += u * n
            n_w += n
            parts.append(f"{k.replace(' ', '')}:util={u:.3f},exec_flops={f:.4g},mfma_insts={n:.4g}")
        if n_w > 0:
            lines.append(f"{call} source_sha={source_sha(src)} util={util_w / n_w:.4f} exec_flops={flops:.6g} "
                         f"kernels={';'.join(parts)}")
    return lines


def stats(config, d):
    st = read_csv(os.path.join(d, "stats", "run_kernel_stats.csv"))
    tr = read_csv(os.path.join(d, "stats", "run_kernel_trace.csv"))
    cmd = ("python3 <repo>/bench.py --config {c} --no-other-configs --no-extras --no-cpu-baseline "
           "--no-graph --steps 20 --warmup 5").format(c=config)
    out = [f"# Kernel time summary, {config} round: rocprofv3 --kernel-trace --stats (MI355X)", "",
           f"Command: `cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/stats "
           f"-o run -- {cmd}`; summary: `python3 bench_profiles.py {config} <dir>`.", "",
           "The whole-run table also covers the untimed context fill (inject_kv over 8192-row slices) and "
           "torch's RNG kernels; the per-call table below counts only the drafting rounds.", "",
           "| kernel | calls | average us | total ms | % |", "|---|---|---|---|---|"]
    for r in st[:16]:
        out.append(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['TotalDurationNs']) / 1e6:.2f} | {float(r['Percentage']):.2f} |")
    win = round_window(tr)
    durs = defaultdict(list)
    for r in win:
        g = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        durs[(short(r["Kernel_Name"]), g)].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    kk = call_kernels(Counter({kg: len(v) for kg, v in durs.items()}))
    out += ["", "## Kernels of the drafting rounds", "",
            "From the first attention launch on; per kernel the grid (threads) launched most often.", "",
            "| call | kernel | grid | launches | average us |", "|---|---|---|---|---|"]
    per_call = {}
    for call in CALLS:
        s = 0.0
        for k, g, n in kk.get(call, []):
            a = statistics.fmean(durs[(k, g)]) / 1e3
            s += a
            out.append(f"| {call} | {k} | {g} | {n} | {a:.2f} |")
        per_call[call] = s
    out += ["", "## Per call (sum of the call's kernels; compare with the per-call HIP-event times bench.py "
            "reports)", "", "| call | average us |", "|---|---|"]
    for call, s in per_call.items():
        out.append(f"| {call} | {s:.2f} |")
    return out


def main():
    if len(sys.argv) != 3:
        sys.exit("usage: python bench_profiles.py <config> <dir>")
    config, d = sys.argv[1], sys.argv[2]
    prof = os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    done = []
    if os.path.isdir(os.path.join(d, "stats")):
        with open(os.path.join(prof, f"kernel_stats_{config}.md"), "w") as f:
            f.write("\n".join(stats(config, d)) + "\n")
        done.append("stats")
    if os.path.isdir(os.path.join(d, "fetch")) and os.path.isdir(os.path.join(d, "write")):
        with open(os.path.join(prof, f"traffic_{config}.txt"), "w") as f:
            f.write("\n".join(traffic(config, d)) + "\n")
        done.append("traffic")
    if os.path.isdir(os.path.join(d, "mfma")):
        with open(os.path.join(prof, f"mfma_{config}.txt"), "w") as f:
            f.write("\n".join(mfma(config, d)) + "\n")
        done.append("mfma")
    print(f"{config}: wrote {', '.join(done) or 'nothing'}")


if __name__ == "__main__":
    main()
