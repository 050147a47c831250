"""Build libfa.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m tiled_attention_forward_fwd_amd.build [--resource-usage]

The library lands next to this file; the Python binding loads it from there.
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_api.hip", "fa_fwd_kernel.hip", "fa_bwd_kernel.hip"]
ARCH = "gfx950"


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(resource_usage=False, out=LIB):
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           # packed fp32 VALU forms are kept out of the generated code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-Wl,-rpath," + os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")]
    if resource_usage:
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    cmd += ["-o", out + ".tmp"]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    log = "\n".join(line for line in (proc.stdout + proc.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + log)
    os.replace(out + ".tmp", out)
    return log


if __name__ == "__main__":
    print(build(resource_usage="--resource-usage" in sys.argv))
