"""Builds librouter.so (the HIP kernels and the C ABI of include/router.h)
for gfx950 with hipcc, in-tree next to this file.

Each kernel translation unit compiles in its own hipcc process, in
parallel; objects go to _build/ and are linked into one shared library.
"""
import json
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "librouter.so")
# what the library was built from and with (written next to it by build())
BUILD_INFO = os.path.join(HERE, "librouter.build.json")
ARCH = os.environ.get("ROUTER_OFFLOAD_ARCH", "gfx950")

SOURCES = ["router_api.cpp", "router_lpt16.hip", "router_lpt32.hip",
           "router_lpt64a.hip", "router_lpt64b.hip", "router_lpt64c.hip",
           "router_scalar.hip", "router_scalar2.hip", "router_loss.hip", "router_route.hip",
           "router_gate.hip", "router_stream.hip", ("router_grouped.hip", 16),
           ("router_grouped.hip", 32)]

FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # packed fp32 VALU forms (v_pk_*_f32) stay off: hipcc otherwise
         # forms them by itself from scalar and float2 code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src):
    # a source is a file name, or (file name, lanes) for the grouped kernels,
    # compiled once per lane width
    lpt = None
    if isinstance(src, tuple):
        src, lpt = src
    stem = os.path.splitext(src)[0] + ("" if lpt is None else f"_lpt{lpt}")
    out = os.path.join(OBJ, stem + ".o")
    defs = [] if lpt is None else [f"-DROUTER_GROUPED_LPT={lpt}"]
    cmd = ["hipcc", *FLAGS, *defs, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    return out, msg


def build(jobs=None):
    """Compiles every source and links librouter.so; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    for _, msg in results:
        if msg.strip():
            print(msg, file=sys.stderr)
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    subprocess.run(["hipcc", "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs,
                    "-o", tmp], check=True)
    os.replace(tmp, LIB)
    _write_build_info()
    return LIB


def _run(cmd):
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, cwd=ROOT, timeout=60)
        return r.stdout.strip() if r.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        return None


def _write_build_info():
    ver = _run(["hipcc", "--version"])
    info = {"flags": FLAGS, "sources": SOURCES,
            "hipcc": ver.splitlines()[0] if ver else None,
            # the commit the tree was checked out at, "-dirty" with local changes
            "git": _run(["git", "describe", "--always", "--dirty", "--abbrev=12"])}
    with open(BUILD_INFO, "w") as f:
        json.dump(info, f, indent=1)


if __name__ == "__main__":
    print(build())
