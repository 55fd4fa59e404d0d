"""Build the HIP library in place: ``python -m causal_depthwise_conv1d_width_amd.build``.

Compiles the gfx950 kernels and the C-ABI entry points (``csrc/``) with hipcc into
``libcausal_conv1d.so`` inside the package directory.  Packed FP32 instructions are disabled
(``-packed-fp32-ops``); FMAs appear only where the sources write them (``-ffp-contract=off``).
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libcausal_conv1d.so")
SOURCES = ["conv1d_fwd.hip", "conv1d_bwd.hip", "conv1d_cf.hip", "conv1d_api.cpp"]
ARCH = "gfx950"


def hipcc_flags():
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-ffp-contract=off",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]


CEILING_SRC = "ceiling.hip"  # copy kernels for the benchmark's bandwidth ceilings (not the ABI)
CEILING_LIB = os.path.join(PKG, "libconv1d_ceiling.so")


def build_ceiling(out=CEILING_LIB):
    """The benchmark's copy kernels (csrc/ceiling.hip) as their own small library."""
    tmp = out + ".tmp"
    subprocess.run(["hipcc", *hipcc_flags(), "-shared", "-x", "hip", os.path.join(CSRC, CEILING_SRC), "-o", tmp],
                   check=True, stderr=subprocess.DEVNULL)
    os.replace(tmp, out)
    return out


def build(out=LIB, jobs=4, verbose=False, defines=()):
    objdir = os.path.join(PKG, "_build", os.path.basename(out))
    os.makedirs(objdir, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = ["hipcc", *hipcc_flags(), *[f"-D{d}" for d in defines], *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd))
        procs.append(subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True))
        objs.append(obj)
    errs = []
    for p in procs:
        _, err = p.communicate()
        lines = [l for l in err.splitlines() if "packed-fp32-ops" not in l]
        if p.returncode != 0:
            errs.append("\n".join(lines))
        elif lines and verbose:
            print("\n".join(lines))
    if errs:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    tmp = out + ".tmp"
    subprocess.run(["hipcc", "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs], check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_ceiling())
