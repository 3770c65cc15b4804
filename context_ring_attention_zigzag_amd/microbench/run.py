"""Build and run the gfx950 micro-benchmarks behind the cycle and LDS figures of the kernel designs.

    python context_ring_attention_zigzag_amd/microbench/run.py --build   # compile (no GPU needed)
    python context_ring_attention_zigzag_amd/microbench/run.py           # run the built programs

cycles.hip: the bf16 32x32x16 MFMA stream, vector instruction costs, MFMA and vector co-execution.
lds.hip: LDS read/write throughput, direct-to-LDS load issue cost, a read issued after such a load.
The programs are standalone HIP (no torch); they write only their own buffers.
"""

import argparse
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
BUILD = os.path.join(HERE, "_build")
PROGRAMS = ("cycles", "lds")
FLAGS = ["-O3", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build():
    os.makedirs(BUILD, exist_ok=True)
    for p in PROGRAMS:
        cmd = ["/opt/rocm/bin/hipcc", *FLAGS, os.path.join(HERE, p + ".hip"), "-o", os.path.join(BUILD, p)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.exit(f"hipcc failed for {p}.hip:\n{res.stderr}")
        print(f"built {p}", flush=True)


def run(timeout_s):
    rc = 0
    for p in PROGRAMS:
        exe = os.path.join(BUILD, p)
        if not os.path.exists(exe):
            sys.exit(f"{exe} is missing: run with --build first")
        print(f"== {p}", flush=True)
        res = subprocess.run([exe], timeout=timeout_s)
        rc = rc or res.returncode
    return rc


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--build", action="store_true", help="compile the programs into microbench/_build")
    ap.add_argument("--timeout", type=float, default=120.0, help="seconds per program")
    args = ap.parse_args()
    if args.build:
        build()
    else:
        sys.exit(run(args.timeout))
