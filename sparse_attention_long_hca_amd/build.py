"""Build libsparse_attn_hca.so for gfx950 in-tree.

    python -m sparse_attention_long_hca_amd.build [--jobs N]

Every HIP source and the C-ABI host layer are compiled with hipcc for
gfx950 (in parallel), then linked into sparse_attention_long_hca_amd/lib/.
Packed-FP32 instruction selection is disabled for all device code.
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIBNAME = "libsparse_attn_hca.so"
ARCH = "gfx950"

SOURCES = [
    "api.cpp",
    "hca_compress.hip",
    "hca_prefill.hip",
    "hca_decode.hip",
    "hca_quant.hip",
    "dsa_indexer.hip",
    "dsa_topk.hip",
    "dsa_fused.hip",
    "dsa_sparse_attn.hip",
    "dsa_sparse_bwd.hip",
    "hca_bwd.hip",
]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]

# Keep MFMA accumulators in ordinary VGPRs: the attention loops rescale and
# read them with VALU ops, and splitting them across the two register files
# makes the compiler copy every accumulator at each loop iteration.  The
# backward passes' gradient accumulators are only ever MFMA operands (no
# rescaling) and need more than 256 registers per wave with everything else,
# so those files let the compiler place them in the accumulation registers.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
NO_VGPR_FORM = {"hca_bwd.hip", "dsa_sparse_bwd.hip"}


def hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


# Per-source flags.  The indexer's scores are finite for finite inputs; without
# NaN semantics its ReLU (max(x, 0)) is one instruction instead of a quieting
# max followed by the max.
SOURCE_FLAGS = {
    "dsa_indexer.hip": ["-fno-honor-nans"],
}


def _compile(src, extra):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    form = [] if src in NO_VGPR_FORM else VGPR_FORM
    cmd = [hipcc()] + lang + COMMON_FLAGS + form + SOURCE_FLAGS.get(src, []) + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that note is harmless.
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{out}")
    return obj, out


def build(jobs=None, extra=None, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    extra = list(extra or [])
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 8)
    objs = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = {ex.submit(_compile, s, extra): s for s in SOURCES}
        for f in cf.as_completed(futs):
            obj, out = f.result()
            if verbose and out.strip():
                print(out)
            objs.append(obj)
    lib = os.path.join(LIBDIR, LIBNAME)
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + sorted(objs)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}")
    os.replace(tmp, lib)
    return lib


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    lib = build(args.jobs, verbose=args.verbose)
    print(lib)


if __name__ == "__main__":
    sys.exit(main())
