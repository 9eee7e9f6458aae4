"""Build liblsd_attn.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

Usage: python -m long_sequence_dense_amd.build   (or build() from Python).
Every call recompiles.  Output: long_sequence_dense_amd/liblsd_attn.so and the
standalone ceiling probes long_sequence_dense_amd/mfma_ceiling_probe (matrix
cores) and long_sequence_dense_amd/hbm_ceiling_probe (HBM streaming rates).
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblsd_attn.so")
PROBES = ("mfma_ceiling_probe", "hbm_ceiling_probe")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# Per-source extra flags.  The prep kernel must evaluate every float
# operation exactly as written (no contraction into fma).
SOURCES = {
    "abi.hip": [],
    "attn_fwd.hip": ["-fno-honor-nans"],
    "attn_bwd.hip": ["-fno-honor-nans"],
    "qk_prep.hip": ["-ffp-contract=off"],
    "nvfp4_gemm.hip": [],
}


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed (%d): %s\n%s" % (r.returncode, " ".join(cmd), out))
    return out


def build(verbose=False):
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src, extra in SOURCES.items():
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        out = _run([cc] + COMMON + extra + ["-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs)
    os.replace(tmp, LIB)
    # the ceiling probes (standalone executables, not part of the library)
    for name in PROBES:
        exe = os.path.join(HERE, name)
        _run([cc] + COMMON + ["-o", exe + ".tmp", os.path.join(CSRC, name + ".hip")])
        os.replace(exe + ".tmp", exe)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
