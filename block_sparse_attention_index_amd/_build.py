"""Build ``libmsa.so`` (the HIP library behind include/msa.h) for gfx950.

hipcc compiles every ``csrc/*.hip`` file and links one shared library in the
package directory.  Packed FP32 instructions are switched off for device code
(they are not needed: the FP32 work of these kernels is scalar), FP32
division stays IEEE-correct (the insert kernel's quantiser depends on it) and
nothing is compiled with fast-math.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["msa_api.hip", "msa_insert.hip", "msa_index.hip", "msa_prefix.hip", "msa_topk.hip", "msa_attn.hip",
           "msa_qkv.hip", "msa_stream.hip", "msa_prefill_attn.hip"]
# Per-file flags (none at present: every file keeps IEEE NaN semantics, so the
# indexers' max-pools skip NaN scores as the definition does).
EXTRA_FLAGS = {}


def build(verbose: bool = False, jobs: int = 5) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = [
        HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall",
    ]
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = common + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len([p for p in procs if p[1].poll() is None]) >= jobs:
            procs[0][1].wait()
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append(src)
            print(text, file=sys.stderr)
        elif verbose and text.strip():
            print(text)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
