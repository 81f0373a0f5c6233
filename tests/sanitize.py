"""Host AddressSanitizer + UndefinedBehaviorSanitizer run of the CPU test suite.

Builds, with ROCm's clang so that one sanitizer runtime serves both:
  oracle/liboracle_sanitized.so   oracle.c with -fsanitize=address,undefined
  eagle_tree_verification_draft_amd/libeagle_sanitized.so
                                   the HIP sources with the same sanitizers on
                                   the host side only (device code is built as
                                   usual for gfx950)
then runs `pytest tests -m "not gpu"` with those libraries (ORACLE_LIB,
EAGLE_LIB) and the sanitizer runtime preloaded; any report fails the run.

    python tests/sanitize.py [extra pytest args]

CPU only: the GPU tests are not run under it.
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = "/opt/rocm/llvm"
ORACLE_SAN = os.path.join(ROOT, "oracle", "liboracle_sanitized.so")
EAGLE_SAN = os.path.join(ROOT, "eagle_tree_verification_draft_amd", "libeagle_sanitized.so")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def runtime() -> str:
    hits = sorted(glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise SystemExit("no clang address-sanitizer runtime under " + LLVM)
    return hits[-1]


def build():
    subprocess.check_call([os.path.join(LLVM, "bin", "clang"), "-O1", "-g", "-std=c11", "-fopenmp",
                           "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", *SAN, "-shared-libsan",
                           "-o", ORACLE_SAN, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    sys.path.insert(0, ROOT)
    from eagle_tree_verification_draft_amd import build as eb
    host_san = []
    for f in SAN:
        host_san += ["-Xarch_host", f]
    flags = [f for f in eb.FLAGS if f != "-O3"] + ["-O1", "-g", "-shared-libsan"] + host_san
    subprocess.check_call([eb.HIPCC, *flags, "-o", EAGLE_SAN, *eb.sources()])


def main():
    build()
    env = dict(os.environ)
    env.update(ORACLE_LIB=ORACLE_SAN, EAGLE_LIB=EAGLE_SAN, LD_PRELOAD=runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", *sys.argv[1:]], env=env, cwd=ROOT)
    sys.exit(r.returncode)


if __name__ == "__main__":
    main()
