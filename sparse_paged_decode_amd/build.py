"""Build libmono_decode.so for gfx950 with hipcc, in-tree.

``build()`` always recompiles; ``ensure_built()`` builds only when the
library is missing.  Objects go to ``_build/`` next to this file.
"""

import concurrent.futures
import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libmono_decode.so")
# The same library with the kernels' phase stamps compiled in (MONO_TRACE):
# only step.hip differs; include/mono_trace.h declares its two extra calls.
TRACE_LIB_PATH = os.path.join(PKG_DIR, "libmono_decode_trace.so")
TRACE_SOURCE = "step.hip"
SOURCES = ["plan.cpp", "pages.hip", "step.hip", "merge.hip", "bench_read.hip", "bench_scan.hip", "abi.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Wno-unused-command-line-argument",
    # Atomics keep their results where the source uses them: the atomic
    # optimizer would broadcast each result at once (a wait for the atomic
    # right after it is issued), even when the result is needed only later.
    "-mllvm",
    "-amdgpu-atomic-optimizer-strategy=None",
    # No packed-fp32 instructions in generated code.
    "-Xclang",
    "-target-feature",
    "-Xclang",
    "-packed-fp32-ops",
    "-I",
    os.path.join(ROOT, "include"),
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: cannot build libmono_decode.so")


def _run(cmd):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{proc.stdout}\n{proc.stderr}")
    return proc


def build(jobs=4):
    """Compile every HIP source for gfx950 and link libmono_decode.so; returns its path."""
    hipcc = _hipcc()
    obj_dir = os.path.join(PKG_DIR, "_build")
    os.makedirs(obj_dir, exist_ok=True)

    def compile_one(job):
        src, extra, suffix = job
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + suffix + ".o")
        _run([hipcc, *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    jobs_list = [(src, [], "") for src in SOURCES] + [(TRACE_SOURCE, ["-DMONO_TRACE"], "_trace")]
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, jobs_list))
    trace_obj = objs.pop()
    for path, lib_objs in ((LIB_PATH, objs),
                           (TRACE_LIB_PATH, [trace_obj if o.endswith(os.sep + "step.o") else o for o in objs])):
        tmp = path + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *lib_objs])
        os.replace(tmp, path)
    return LIB_PATH


def ensure_built():
    if not os.path.exists(LIB_PATH):
        build()
    return LIB_PATH


if __name__ == "__main__":
    print(build())
