"""Build the HIP libraries in-tree with hipcc for gfx950.

  libengram.so       the Engram forward library (hashed_gram_engram_amd/csrc, include/engram.h)
  libsynth_fill.so   device-side fill of seeded synthetic inputs (synth/fill.hip)
  liboracle.so       the CPU oracle (oracle/engram_oracle.cc, plain C++ built with g++; test
                     infrastructure, never linked into libengram.so)
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# packed fp32 vector ops stay off (every kernel is built with the feature disabled)
COMMON = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-flush-denormals-to-zero", "-Wno-unused-command-line-argument"]

ENGRAM_SRC = ["engram_api.hip", "gather_gate.hip", "hash.hip", "stream.hip", "tiled.hip"]
LIB_ENGRAM = os.path.join(HERE, "libengram.so")
LIB_SYNTH = os.path.join(ROOT, "synth", "libsynth_fill.so")
LIB_ORACLE = os.path.join(ROOT, "oracle", "liboracle.so")
CXX = os.environ.get("CXX", "g++")
# IEEE double throughout: no fused multiply-add, no reassociation, no fast-math
ORACLE_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-ffp-contract=off"]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False) -> None:
    obj_dir = os.path.join(ROOT, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    csrc = os.path.join(HERE, "csrc")
    jobs = []
    for s in ENGRAM_SRC:
        o = os.path.join(obj_dir, s.replace(".hip", ".o"))
        jobs.append((o, [HIPCC] + COMMON + ["-I", os.path.join(ROOT, "include"), "-c",
                                            os.path.join(csrc, s), "-o", o]))
    synth_o = os.path.join(obj_dir, "synth_fill.o")
    jobs.append((synth_o, [HIPCC] + COMMON + ["-ffp-contract=off", "-c",
                                              os.path.join(ROOT, "synth", "fill.hip"), "-o", synth_o]))
    oracle_tmp = LIB_ORACLE + ".tmp"
    jobs_all = jobs + [(oracle_tmp, [CXX] + ORACLE_FLAGS + [
        os.path.join(ROOT, "oracle", "engram_oracle.cc"), "-o", oracle_tmp])]
    with ThreadPoolExecutor(max_workers=min(8, len(jobs_all))) as ex:
        outs = list(ex.map(lambda j: _run(j[1]), jobs_all))
    os.replace(oracle_tmp, LIB_ORACLE)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB_ENGRAM + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + [j[0] for j in jobs[:-1]])
    os.replace(tmp, LIB_ENGRAM)
    tmp = LIB_SYNTH + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, synth_o])
    os.replace(tmp, LIB_SYNTH)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print("built", LIB_ENGRAM, LIB_SYNTH, LIB_ORACLE)
