"""Builds libgconv.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python grouped_convolution_conv_amd/build.py

Each source under csrc/ is compiled to an object in parallel, then linked
into grouped_convolution_conv_amd/libgconv.so.  Packed FP32 instructions are
disabled (-packed-fp32-ops); nothing is built with fast-math or
flush-to-zero, so FP32 arithmetic rounds to nearest even with denormals.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgconv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer (the device code
# is built as always): every -fsanitize flag goes to the host compilation only.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-g"]
LIB_SANITIZED = os.path.join(PKG, "libgconv_san.so")


def build(verbose: bool = False, extra_flags=None, sanitize: bool = False) -> str:
    """Compile every source and link libgconv.so; returns its path.  With
    sanitize, the host code is instrumented with AddressSanitizer and
    UndefinedBehaviorSanitizer and the result is libgconv_san.so."""
    extra = list(extra_flags or []) + (SANITIZE_HOST if sanitize else [])
    lib_out = LIB_SANITIZED if sanitize else LIB
    with tempfile.TemporaryDirectory(prefix="gconv_build_") as tmp:
        procs = []
        objs = []
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [HIPCC, "-x", "hip", "-c", src, "-o", obj] + COMMON + extra
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
        failed = []
        for src, pr in procs:
            out, _ = pr.communicate()
            text = out.decode(errors="replace")
            if pr.returncode != 0:
                failed.append((src, text))
            elif verbose and text.strip():
                print(text)
        if failed:
            msg = "\n".join("%s:\n%s" % (s, t) for s, t in failed)
            raise RuntimeError("hipcc failed:\n" + msg)
        tmp_lib = lib_out + ".tmp%d" % os.getpid()
        # every symbol resolved at link time: a kernel whose host launch stub
        # is missing fails the build, not the first load (the sanitized build
        # leaves the sanitizer runtime's symbols to the preloaded runtime)
        link = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp_lib] + objs
        link += (["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-shared-libsan"] if sanitize
                 else ["-Wl,--no-undefined"])
        subprocess.run(link, check=True)
        os.replace(tmp_lib, lib_out)
    return lib_out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
