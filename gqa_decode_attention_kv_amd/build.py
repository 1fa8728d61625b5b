"""Build ``libuaii_decode.so`` (HIP for gfx950) in-tree with hipcc, and the
measurement probe ``libuaii_probe.so`` (a plain streaming read, used only by
the benchmark to find the practical HBM read rate).

Each translation unit compiles in its own process, then one link step.
Flags: -O3, gfx950 only, and packed-FP32 instructions disabled
(``-target-feature -packed-fp32-ops``) for every device compile.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libuaii_decode.so")
PROBE_LIBRARY = os.path.join(HERE, "libuaii_probe.so")
PROBE_SOURCES = ["stream_probe.hip"]
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "kv_produce.hip", "decode_partial.hip", "decode_partial_paged.hip",
           "decode_combine.hip", "decode_step.hip", "decode_step_paged.hip", "prefill_attn.hip",
           "prefill_attn_vq8.hip", "prefill_attn_q8.hip", "prefill_attn_f32.hip",
           "decode_step_noalloc.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-command-line-argument",
          "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    # The host pass does not know the packed-fp32 target feature and says so;
    # that warning is expected and dropped.
    err = "\n".join(l for l in res.stderr.splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l
                    and l.strip())
    return err


def build(verbose: bool = False) -> str:
    """Compile every translation unit, then link both libraries; returns the
    path of the decode library."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cmds = []
    objs = {}
    for lib, sources in ((LIBRARY, SOURCES), (PROBE_LIBRARY, PROBE_SOURCES)):
        objs[lib] = []
        for src in sources:
            obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmds.append([HIPCC, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
            objs[lib].append(obj)
    with ThreadPoolExecutor(len(cmds)) as ex:
        for err in ex.map(_run, cmds):
            if err and verbose:
                sys.stderr.write(err + "\n")
    for lib, lib_objs in objs.items():
        tmp = lib + ".tmp"
        err = _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *lib_objs, "-o", tmp])
        if err and verbose:
            sys.stderr.write(err + "\n")
        os.replace(tmp, lib)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
