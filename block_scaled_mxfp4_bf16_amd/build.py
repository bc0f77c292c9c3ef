"""Build libmxfp4.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmxfp4.so")
# Measurement probes for bench.py --floors (a library of their own: nothing
# in libmxfp4.so uses them).  probe_phases.hip and probe_wide.hip
# instantiate the library's kernels and take the flags of the library
# sources that do; probes.hip has its own.
PROBES_SOURCES = ["probes.hip", "probe_phases.hip", "probe_wide.hip"]
PROBES_LIB = os.path.join(PKG, "libmxfp4_probes.so")
SOURCES = ["mxfp4_api.hip", "quant_kernels.hip", "gemm_kernels.hip", "gemm_wide.hip"] + [
    "gemm_table_%d.hip" % i for i in range(8)]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep packed-f32 arithmetic instructions out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
    "-I" + os.path.join(ROOT, "include"),
]


# Per-source extra flags.  The scaled matrix instruction has no form whose
# result is tied to its accumulator input when the accumulator lives in
# AGPRs, so long accumulation loops get copies between every pair of
# instructions; keeping accumulators in VGPRs lets them update in place.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
EXTRA_FLAGS = {"gemm_wide.hip": VGPR_FORM, "probes.hip": VGPR_FORM, "probe_wide.hip": VGPR_FORM}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source to an object in parallel, then link the shared library."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [hipcc(), *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature name; that warning is expected
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write(text)
        elif verbose and lines:
            sys.stderr.write("\n".join(lines) + "\n")
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    probe_objs = [os.path.join(objdir, "probe_" + src.replace(".hip", ".o")) for src in PROBES_SOURCES]
    pprocs = [(src, subprocess.Popen([hipcc(), *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
                                      "-o", obj], stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
              for src, obj in zip(PROBES_SOURCES, probe_objs)]
    for src, p in pprocs:
        out, _ = p.communicate()
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write(out.decode(errors="replace"))
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    ptmp = PROBES_LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", ptmp, *probe_objs])
    os.replace(ptmp, PROBES_LIB)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
