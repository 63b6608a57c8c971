"""Build libselattn.so for gfx950 in-tree with hipcc (no JIT, no torch extension).

    python -m split_flash_attention_amd.build        # or build() from Python
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libselattn.so")
SOURCES = ["api.hip", "valu_attn.hip", "mfma_attn.hip", "mfma_decode.hip", "mfma_prefill.hip", "noalloc.hip",
           "wide_decode.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def _compile(src):
    obj = os.path.join(CSRC, "_build", src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


PROBE_DIR = os.path.join(os.path.dirname(HERE), "tests", "probe")
PROBE_SRC = os.path.join(PROBE_DIR, "mfma_probe.hip")
PROBE_OUT = os.path.join(PROBE_DIR, "libmfma_probe.so")
GATHER_SRC = os.path.join(PROBE_DIR, "gather_probe.hip")
GATHER_OUT = os.path.join(PROBE_DIR, "libgather_probe.so")


def build_probe():
    """The one-wave MFMA layout probe used by the GPU tests, and the gather-bandwidth
    probe the benchmark measures its selected-key roof with."""
    for src, out in ((PROBE_SRC, PROBE_OUT), (GATHER_SRC, GATHER_OUT)):
        if not os.path.exists(src):
            continue
        cmd = [HIPCC, *FLAGS, "-shared", src, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"probe build failed for {src}:\n" + r.stderr)
    return PROBE_OUT


def build(verbose=False):
    os.makedirs(os.path.join(CSRC, "_build"), exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    if os.path.exists(PROBE_SRC):
        build_probe()
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
