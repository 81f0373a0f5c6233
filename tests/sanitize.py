"""Host AddressSanitizer + UndefinedBehaviorSanitizer run of the CPU test suite.

Builds, with ROCm's clang so that one sanitizer runtime serves both, into a
temporary directory removed afterwards:
  liboracle_sanitized.so   oracle.c with -fsanitize=address,undefined
  libeagle_sanitized.so    the HIP sources with the same sanitizers on the
                           host side only (device code is built as usual for
                           gfx950)
then runs `pytest tests -m "not gpu"` with those libraries (ORACLE_LIB,
EAGLE_LIB) and the sanitizer runtime preloaded; any report fails the run.

    python tests/sanitize.py [extra pytest args]

CPU only: the GPU tests are not run under it.
"""
import glob
import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = "/opt/rocm/llvm"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def runtime() -> str:
    hits = sorted(glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise SystemExit("no clang address-sanitizer runtime under " + LLVM)
    return hits[-1]


def build(out_dir):
    oracle_san = os.path.join(out_dir, "liboracle_sanitized.so")
    eagle_san = os.path.join(out_dir, "libeagle_sanitized.so")
    subprocess.check_call([os.path.join(LLVM, "bin", "clang"), "-O1", "-g", "-std=c11", "-fopenmp",
                           "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", *SAN, "-shared-libsan",
                           "-o", oracle_san, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    sys.path.insert(0, ROOT)
    from eagle_tree_verification_draft_amd import build as eb
    host_san = []
    for f in SAN:
        host_san += ["-Xarch_host", f]
    flags = [f for f in eb.FLAGS if f != "-O3"] + ["-O1", "-g", "-shared-libsan"] + host_san
    subprocess.check_call([eb.HIPCC, *flags, "-o", eagle_san, *eb.sources()])
    return oracle_san, eagle_san


def main():
    out_dir = tempfile.mkdtemp(prefix="eagle_sanitize_")
    try:
        return run(*build(out_dir))
    finally:
        shutil.rmtree(out_dir, ignore_errors=True)


def run(oracle_san, eagle_san):
    env = dict(os.environ)
    env.update(ORACLE_LIB=oracle_san, EAGLE_LIB=eagle_san, LD_PRELOAD=runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", *sys.argv[1:]], env=env, cwd=ROOT)
    sys.exit(r.returncode)


if __name__ == "__main__":
    main()
