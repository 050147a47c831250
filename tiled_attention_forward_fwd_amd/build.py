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
SOURCES = ["fa_api.hip", "fa_fwd_kernel.hip", "fa_fwd_masked.hip", "fa_fwd_hdim.hip",
           "fa_fwd_hdim_masked.hip", "fa_fwd_ks.hip", "fa_fwd_f32.hip", "fa_bwd_kernel.hip",
           "fa_bwd_hdim.hip"]
ARCH = "gfx950"


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _filtered(text):
    return "\n".join(line for line in text.splitlines() if "packed-fp32-ops" not in line)


def build(resource_usage=False, out=LIB):
    """Compiles every source to an object in parallel, then links libfa.so."""
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             # packed fp32 VALU forms are kept out of the generated code
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    if resource_usage:
        flags.append("-Rpass-analysis=kernel-resource-usage")
    objs, procs = [], []
    for src in SOURCES:
        obj = f"{out}.{src}.o"
        objs.append(obj)
        procs.append(subprocess.Popen([hipcc()] + flags + ["-c", os.path.join(CSRC, src), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    logs, failed = [], False
    for src, proc in zip(SOURCES, procs):
        text = proc.communicate()[0]
        logs.append(_filtered(text))
        failed = failed or proc.returncode != 0
    try:
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(logs))
        link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC",
                "-Wl,-rpath," + os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")]
        proc = subprocess.run(link + objs + ["-o", out + ".tmp"], capture_output=True, text=True)
        if proc.returncode != 0:
            raise RuntimeError("link failed:\n" + _filtered(proc.stdout + proc.stderr))
        os.replace(out + ".tmp", out)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    return "\n".join(logs)


if __name__ == "__main__":
    print(build(resource_usage="--resource-usage" in sys.argv))
