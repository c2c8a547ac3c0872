"""Build the HIP library libkascade_mi355x.so for gfx950 with hipcc.

Run as a module (python -m sparse_attention_long_anchor_amd.build) or call
build(). The library is written next to this file.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libkascade_mi355x.so")
SOURCES = ["kascade_api.hip", "decode_kernels.hip", "prefill_kernels.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
         # packed fp32 VALU forms are kept out of the generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Wno-unused-result"]


def _compile(src: str, build_dir: str) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build() -> str:
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir), SOURCES))
    tmp = OUT + ".tmp"
    # -z defs: an undefined symbol (say, a kernel whose launch stub the host
    # pass did not emit) fails the link instead of the first dlopen
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-Wl,-z,defs", "-o", tmp, *objs]
    subprocess.check_call(cmd)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
