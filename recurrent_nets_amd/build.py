"""Build the HIP library in-tree: every csrc/*.hip compiled for gfx950 and linked into one
shared object, recurrent_nets_amd/lib/libslstm_mi355x.so.

    python -m recurrent_nets_amd.build [--verbose]
"""
from __future__ import annotations

import argparse
import concurrent.futures
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIBNAME = "libslstm_mi355x.so"
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 instructions stay off for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def lib_path() -> str:
    return os.path.join(LIBDIR, LIBNAME)


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="slstm_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [cc, *HIPCC_FLAGS, "-c", src, "-o", obj]
            if resource_usage:
                cmd += ["-Rpass-analysis=kernel-resource-usage"]
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            # the host pass warns that it does not know the device-only feature; drop that line
            err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
            return src, obj, res.returncode, err

        # one hipcc process per source, a few at a time (the machine's CPU share is 16)
        workers = max(1, min(8, os.cpu_count() or 1, len(sources())))
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as pool:
            results = list(pool.map(compile_one, sources()))
        objs = []
        for src, obj, rc, err in results:
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{err}")
            if err.strip() and (verbose or resource_usage):
                print(err, file=sys.stderr)
            objs.append(obj)
        tmp_lib = os.path.join(tmp, LIBNAME)
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stderr}")
        os.replace(tmp_lib, lib_path())
    return lib_path()


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true",
                    help="print per-kernel VGPR/SGPR/LDS/spill figures")
    a = ap.parse_args(argv)
    print(build(a.verbose, a.resource_usage))


if __name__ == "__main__":
    main()
