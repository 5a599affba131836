"""Compile the HIP sources into libmtp_hip.so for gfx950 (in-tree, next to this file).

    python -m speculative_decoding_mtp_amd.build
"""
import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmtp_hip.so")
BUILD = os.path.join(os.path.dirname(HERE), "_build")
SOURCES = ["draft_bf16.hip", "draft_f32.hip", "draft.hip", "attn.hip", "verify.hip", "state.hip", "capi.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
         # packed fp32 VALU forms are kept out of the device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    t0 = time.time()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines() if "unknown target feature" not in l and "packed-fp32-ops" not in l
                        and l.strip() and "warning generated" not in l and "warnings generated" not in l)
        if p.returncode != 0:
            failed.append(src)
            print(out, file=sys.stderr)
        elif out and verbose:
            print(out, file=sys.stderr)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        print(r.stdout, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f} s", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
