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


# Test-only builds with one planted mistake each: the GPU tests run named parity
# tests through them and require each to fail.  name -> (translation unit, define).
PLANTS = {
    "combine_nan_to_zero": ("valu_attn.hip", "SELATTN_PLANT_COMBINE_NAN_TO_ZERO"),
    "alibi_before_softcap": ("mfma_prefill.hip", "SELATTN_PLANT_ALIBI_BEFORE_SOFTCAP"),
    "keep_repeats": ("mfma_prefill.hip", "SELATTN_PLANT_KEEP_REPEATS"),
}
PLANT_DIR = os.path.join(os.path.dirname(HERE), "tests", "planted")


def plant_path(name):
    return os.path.join(PLANT_DIR, f"libselattn_{name}.so")


def _compile(src, define=None, tag=None):
    obj = os.path.join(CSRC, "_build", src.replace(".hip", f".{tag}.o" if tag else ".o"))
    cmd = [HIPCC, *FLAGS, *([f"-D{define}"] if define else []), "-c", os.path.join(CSRC, src), "-o", obj]
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


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, out)


def build(verbose=False):
    os.makedirs(os.path.join(CSRC, "_build"), exist_ok=True)
    os.makedirs(PLANT_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        jobs = [ex.submit(_compile, src) for src in SOURCES]
        pjobs = {name: ex.submit(_compile, src, define, name) for name, (src, define) in PLANTS.items()}
        objs = [j.result() for j in jobs]
        pobjs = {name: j.result() for name, j in pjobs.items()}
    _link(objs, OUT)
    for name, (src, _) in PLANTS.items():
        _link([pobjs[name] if s == src else o for s, o in zip(SOURCES, objs)], plant_path(name))
    if os.path.exists(PROBE_SRC):
        build_probe()
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
