"""Runs the CPU test suite (-m "not gpu") against builds whose host code carries
AddressSanitizer and UndefinedBehaviorSanitizer: the oracle (oracle.c, clang)
and the library's host side (descriptor validation, dispatch, workspace sizing,
the allocation-free entry point's checks and the timing helpers; device code is
built as always).  Not collected by pytest; run it by hand:

    python tests/sanitize_host.py [extra pytest arguments]

It builds oracle/liboracle_san.so and grouped_convolution_conv_amd/libgconv_san.so,
then runs pytest in a child process with clang's ASan runtime preloaded
(appended to any LD_PRELOAD the environment already has) and GCONV_SANITIZED=1,
which makes both loaders pick the sanitized builds.  Leak detection is off (the
Python interpreter itself is not instrumented and keeps its allocations until
exit); any address or undefined-behaviour error aborts the run.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def main():
    import importlib.util
    spec = importlib.util.spec_from_file_location("_gconv_build", os.path.join(ROOT, "grouped_convolution_conv_amd",
                                                                                "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    print("building", b.build(sanitize=True), flush=True)
    import oracle
    print("building", oracle.build(force=True, sanitize=True), flush=True)
    rt = subprocess.run([oracle.CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], check=True,
                        capture_output=True, text=True).stdout.strip()
    env = dict(os.environ)
    env["LD_PRELOAD"] = ":".join(p for p in (env.get("LD_PRELOAD", ""), rt) if p)
    env["GCONV_SANITIZED"] = "1"
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    # the child must have mapped the sanitizer runtime and both sanitized builds
    probe = ("import sys; sys.path.insert(0, %r); import oracle, grouped_convolution_conv_amd; oracle._load(); "
             "m = open('/proc/self/maps').read(); "
             "need = ('libclang_rt.asan', 'liboracle_san.so', 'libgconv_san.so'); "
             "missing = [n for n in need if n not in m]; print('mapped:', need, 'missing:', missing); "
             "sys.exit(1 if missing else 0)" % ROOT)
    rc = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT).returncode
    if rc != 0:
        return rc
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu", "-p", "no:cacheprovider"]
    cmd += sys.argv[1:]
    print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main())
