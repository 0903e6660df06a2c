"""Build libsga.so (the SGA HIP library for gfx950) in-tree with hipcc.

    python -m sparse_top_latent_amd.build

Compiles every csrc/*.hip file for gfx950 and links them into
sparse_top_latent_amd/libsga.so. Always recompiles (the build check relies on it).
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libsga.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


# extra flags per source file
PER_FILE = {
    # the indexer's ReLU runs on MFMA accumulators that are never NaN for finite
    # inputs; without this every max is preceded by a NaN-quieting max
    "index_scores.hip": ["-fno-honor-nans", "-Wno-nan-infinity-disabled"],
    "index_prefill.hip": ["-fno-honor-nans", "-Wno-nan-infinity-disabled"],
}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "unused-command-line-argument" not in l
                    and l.strip() != "1 warning generated." and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    if verbose and out:
        print(out)
    return r


def build(verbose: bool = False, jobs: int = 4, out: str = LIB, defines=()) -> str:
    """Compile and link the library to `out`; `defines` are extra -D options
    (build variants for side-by-side measurements)."""
    cc = hipcc()
    objdir = os.path.join(HERE, "_build") if out == LIB else out + ".objs"
    os.makedirs(objdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(objdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_run, [cc, "-c", *COMMON, *[f"-D{d}" for d in defines],
                                 *PER_FILE.get(os.path.basename(s), []), "-o", o, s],
                          verbose) for s, o in zip(srcs, objs)]
        for f in futs:
            f.result()
    tmp = out + ".tmp"
    _run([cc, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
