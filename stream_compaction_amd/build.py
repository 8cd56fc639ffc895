"""Build libscan_amd.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m stream_compaction_amd.build

Each source compiles to an object under ``_build/`` in parallel, then hipcc
links the shared library next to this file.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libscan_amd.so")
SOURCES = ["scan_rows.hip", "scan_device.hip", "select.hip", "reduce.hip", "reduce_by_key.hip",
           "radix_sort.hip", "api.cpp"]
# measurement aid for the benchmark (16-byte copy kernel), kept out of the scan library
COPY_LIB_PATH = os.path.join(HERE, "libscan_copy.so")
COPY_SOURCES = ["copy_ceiling.hip"]
# test-only build of the scan library whose look-back never waits: any
# predecessor descriptor not yet published is recomputed from the input at
# once, so the tests exercise that recovery path on every call
FALLBACK_LIB_PATH = os.path.join(HERE, "libscan_amd_lbtest.so")
FALLBACK_DEFINES = ["-DSCA_LOOKBACK_TIMEOUT_TICKS=0ull"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def compile_cmd(src, obj, defines=()):
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    return [HIPCC, *CFLAGS, *defines, *lang, "-c", os.path.join(CSRC, src), "-o", obj]


def build(verbose=False):
    os.makedirs(OBJ_DIR, exist_ok=True)
    procs = []
    libs = {LIB_PATH: [], COPY_LIB_PATH: [], FALLBACK_LIB_PATH: []}
    jobs = [(LIB_PATH, s, ()) for s in SOURCES] + [(COPY_LIB_PATH, s, ()) for s in COPY_SOURCES] + \
        [(FALLBACK_LIB_PATH, s, FALLBACK_DEFINES) for s in SOURCES]
    for lib, src, defines in jobs:
        tag = "_lbtest" if defines else ""
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + tag + ".o")
        libs[lib].append(obj)
        cmd = compile_cmd(src, obj, defines)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the device-only feature flag: drop that note
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if lines and (verbose or p.returncode != 0):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    for path, lib_objs in libs.items():
        tmp = path + ".tmp"
        subprocess.check_call([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *lib_objs,
                               "-o", tmp])
        os.replace(tmp, path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
