"""Measured ceilings of one MI355X that the kernels' rooflines are read against.

Builds ``bench_ceilings.hip`` with hipcc (into ``_build/``) and runs it on the
current GPU: plain streaming reads (non-temporal and ordinary), LDS-direct tile
rings in the attention kernel's access patterns (contiguous 8 KB tiles, one
head's 256 B of each 2 KB cache row, heads interleaved), and back-to-back bf16
32x32x16 MFMAs.

Usage: python3 bench_ceilings.py [--build-only] [--out FILE]
With --out the output is also written to FILE under a header naming this
command.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(ROOT, "bench_ceilings.hip")
EXE = os.path.join(ROOT, "_build", "bench_ceilings")


def build() -> str:
    sys.path.insert(0, ROOT)
    from block_drafting_amd.build import hipcc
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", ROOT, SRC, "-o", EXE]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise SystemExit(f"hipcc failed:\n{r.stderr}")
    return EXE


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--build-only", action="store_true")
    ap.add_argument("--no-build", action="store_true", help="run the executable built before")
    ap.add_argument("--out", default=None)
    a = ap.parse_args()
    if not a.no_build or not os.path.exists(EXE):
        build()
    if a.build_only:
        return 0
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=300)
    sys.stdout.write(r.stdout)
    sys.stderr.write(r.stderr)
    if r.returncode == 0 and a.out:
        with open(a.out, "w") as f:
            f.write("# Ceilings of one MI355X (gfx950): stand-alone probes, no arithmetic on the data\n")
            f.write("# command: python3 bench_ceilings.py --out <file>   (source: bench_ceilings.hip)\n")
            f.write("# each line: test, bytes (or flops) per launch, microseconds per launch (HIP events,\n")
            f.write("# 10 launches after 3 warm-up), rate\n")
            f.write(r.stdout)
    return r.returncode


if __name__ == "__main__":
    sys.exit(main())
