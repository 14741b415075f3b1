"""Builds libmk.so (the C-ABI library) in place with hipcc for gfx950."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmk.so")
SOURCES = ["mk_api.cpp", "mk_layer.hip", "mk_layer_kv8.hip", "mk_layer_lr.hip", "mk_layer_lr_spec.hip", "mk_layer_sparse.hip",
           "mk_layer_sparse_kv8.hip", "mk_pack.hip",
           "mk_stack.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-munsafe-fp-atomics", "-Wno-unused-result",
         # atomics here are issued by one lane; the wave-level rewrite would
         # wait for the result (and every load in flight) right after issue
         "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]


def build(verbose: bool = False, extra=()) -> str:
    # the units compile in parallel (the two layer-kernel units take the longest)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(CSRC, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = ["/opt/rocm/bin/hipcc", *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    failed = []
    for src, pr in procs:
        _, err = pr.communicate()
        if pr.returncode != 0:
            failed.append("hipcc failed for %s:\n%s" % (src, err))
        elif verbose and err.strip():
            print(err, file=sys.stderr)
    if failed:
        raise RuntimeError("\n".join(failed))
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
