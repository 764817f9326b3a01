"""Host AddressSanitizer + UndefinedBehaviorSanitizer run of the CPU tests (no GPU needed).

    python -m tests.sanitize_host

Builds, under _build/sanitize/: the library with its host code sanitized (the C ABI, the
planning and argument checks, the launchers; device code is built as usual) and the oracle with
clang and both sanitizers. Then runs `pytest -m "not gpu"` on them with clang's ASan runtime
preloaded into the interpreter (leak detection off: the interpreter itself keeps memory until
exit). Any sanitizer report fails the run.
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
LIB = os.path.join(OUT, "libpdecode.so")
ORACLE_LIB = os.path.join(OUT, "liboracle.so")
HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def asan_runtime() -> str:
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("clang's ASan runtime was not found under /opt/rocm/llvm")
    return found[-1]


def build() -> None:
    sys.path.insert(0, ROOT)
    from paged_kv_decode_08_amd import build as lib_build
    os.makedirs(OUT, exist_ok=True)
    lib_build.build(extra=HOST_FLAGS, out=LIB, build_dir=os.path.join(OUT, "obj"))
    # the oracle: plain host C++, with clang so that one sanitizer runtime serves both libraries
    subprocess.run(["/opt/rocm/llvm/bin/clang++", "-O1", "-g", "-std=c++17", "-shared", "-fPIC",
                    "-pthread", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                    "-fno-sanitize-recover=all", os.path.join(ROOT, "oracle", "oracle.cpp"),
                    "-o", ORACLE_LIB], check=True)


def main() -> int:
    build()
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["PDECODE_SANITIZED_LIB"] = LIB
    env["PDECODE_SANITIZED_ORACLE"] = ORACLE_LIB
    cmd = [sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests")]
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main())
