"""Build libattn.so (the gfx950 HIP kernels and their C ABI) in-tree, and
its checked twin libattn_checked.so (the same sources with ATTN_CHECKED=1:
device-side index checks with an error word).

    python -m attention_tiled_fmha_amd.build

Each source is compiled with hipcc for gfx950 only, in parallel, then linked
into attention_tiled_fmha_amd/libattn.so (and libattn_checked.so).
Packed-fp32 instruction selection is switched off for device code.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn.so")
LIB_CHECKED = os.path.join(PKG, "libattn_checked.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Per-file extras: the prefill and shared-prefix softmax never see NaN
# (scores are finite or -inf, and the cache tail past the prefix reads as
# zeros), so fmax needs no NaN canonicalisation there.  The prefill selects
# the VGPR form of the MFMA instructions, so that the softmax reads the
# score accumulators without copying them out of AGPRs.
FILE_FLAGS = {"prefill_bf16.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
              "prefix_mfma.hip": ["-fno-honor-nans"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(src, extra, objdir):
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def _build_one(extra, out, objdir, verbose):
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra), objdir), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def build(extra=(), verbose=False, checked=True):
    """Build libattn.so and, with checked, libattn_checked.so."""
    _build_one(list(extra), LIB, BUILD, verbose)
    if checked:
        _build_one(list(extra) + ["-DATTN_CHECKED=1"], LIB_CHECKED,
                   os.path.join(BUILD, "checked"), verbose)
    return LIB


if __name__ == "__main__":
    build(extra=sys.argv[1:], verbose=True)
