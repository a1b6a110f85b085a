"""Build libbfp8.so for gfx950 with hipcc, and read the compiler's per-kernel
resource report.

The library is built in-tree (``blockwise_scaled_fp8_amd/libbfp8.so``) so
that it travels with the source tree.  ``kernel_resources()`` parses the
AMDGPU backend's kernel-resource-usage remarks of a fresh compile: VGPRs,
AGPRs, scratch bytes, spills and occupancy per kernel.  A hot loop that
spills shows up there as nonzero scratch ([ADA] "Reading the kernel name":
a register-capped kernel with a 600-byte stack frame was spilling in its
main loop; [ADA] "What I learned": check registers on a machine without a
GPU before tuning).
"""

import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbfp8.so")

SOURCES = ["api.hip", "quant.hip", "gemm_w8a8.hip", "gemm_w8a8_tile.hip", "gemm_w8a16.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 VALU forms are kept out of the generated code on purpose.
# MFMA results go to ArchVGPRs (not AGPRs) so the fp32 FMAs that apply the
# per-block scales read them directly, without v_accvgpr_read copies.
COMMON_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I" + INCLUDE, "-I" + CSRC,
    "-Wall", "-Wno-unused-parameter", "-Wno-unused-command-line-argument",
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    if p.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + p.stdout + p.stderr)
    return p


# The benchmark's streaming-read probe: a separate library, not part of the
# GEMM library's C ABI.
PROBE_SOURCES = ["read_probe.hip"]
PROBE_LIB = os.path.join(PKG, "libbfp8_probe.so")


def _link(sources, out, verbose):
    tmp = out + ".tmp"
    p = _run([HIPCC] + COMMON_FLAGS + ["-shared", "-o", tmp] + [os.path.join(CSRC, s) for s in sources])
    os.replace(tmp, out)
    if verbose:
        sys.stderr.write(p.stderr)


def build(verbose=False):
    """Compile every HIP source for gfx950 into libbfp8.so, and the read
    probe into libbfp8_probe.so (always recompiles)."""
    _link(SOURCES, LIB, verbose)
    _link(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


# Host code under AddressSanitizer and UndefinedBehaviorSanitizer, device
# code as for libbfp8.so: each -fsanitize= applies to the host compile only.
SANITIZE_HOST_FLAGS = [f for opt in ("-fsanitize=address", "-fsanitize=undefined",
                                      "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer")
                       for f in ("-Xarch_host", opt)]


def build_host_sanitized(out):
    """libbfp8.so's sources built into `out` with the host code instrumented
    by AddressSanitizer and UndefinedBehaviorSanitizer, for CPU tests of the
    host-side argument checks, planners and the block-32 packer.  The
    sanitizer runtime is not linked in: a process that loads the library
    preloads it (LD_PRELOAD)."""
    _link_to(SOURCES, out, SANITIZE_HOST_FLAGS)
    return out


def _link_to(sources, out, extra):
    tmp = out + ".tmp"
    _run([HIPCC] + COMMON_FLAGS + extra + ["-shared", "-o", tmp] + [os.path.join(CSRC, s) for s in sources])
    os.replace(tmp, out)


def kernel_resources(sources=None):
    """Per-kernel resource usage from a device-only compile of the sources.

    Returns {kernel_name: {"VGPRs": .., "AGPRs": .., "ScratchSize [bytes/lane]": .., ...}}.
    """
    out = {}
    for s in (sources or SOURCES):
        cmd = [HIPCC] + COMMON_FLAGS + ["--cuda-device-only", "-c", "-o", os.devnull,
                                        "-Rpass-analysis=kernel-resource-usage", os.path.join(CSRC, s)]
        p = _run(cmd)
        cur = None
        for line in p.stderr.splitlines():
            m = re.search(r"remark: Function Name: (\S+)", line)
            if m:
                cur = m.group(1)
                out[cur] = {}
                continue
            m = re.search(r"remark:\s+(.+?): (\S+) \[-Rpass-analysis", line)
            if m and cur is not None:
                val = m.group(2)
                out[cur][m.group(1).strip()] = int(val) if re.fullmatch(r"-?\d+", val) else val
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    for k, v in kernel_resources().items():
        print(k, v)
