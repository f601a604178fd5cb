"""CPU sanitizer run of the host-side code: AddressSanitizer and
UndefinedBehaviorSanitizer over the oracle (oracle.c) and the host code of
libpagedattn (argument checks, size arithmetic, split heuristic, launch
wrappers), exercised by the CPU test suite (pytest -m "not gpu").

Both are rebuilt with LLVM's sanitizer runtime in a scratch directory (the
in-tree builds are not touched): oracle.c with ROCm's clang, every HIP unit
with hipcc where the sanitizer flags apply to the host pass only (device code
is built as usual and never runs here). The test suite then runs with that
runtime preloaded and PAGEDATTN_LIB / PA_ORACLE_LIB pointing at the sanitized
builds; any report fails the run.

    python tests/sanitize_host.py      (from the repository root, no GPU needed)
"""
import glob
import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = "/opt/rocm/llvm"
HIPCC = "/opt/rocm/bin/hipcc"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g"]


def host_only(flags):
    """Each flag for the host pass only (-Xarch_host before every one)."""
    out = []
    for f in flags:
        out += ["-Xarch_host", f]
    return out


def build(out_dir):
    sys.path.insert(0, os.path.join(ROOT, "paged_kv_cache_52_amd"))
    import build as hip_build  # the library's own flags and source list
    objs = []
    for src in hip_build.sources():
        obj = os.path.join(out_dir, os.path.basename(src)[:-4] + ".o")
        subprocess.run([HIPCC, *hip_build.FLAGS, *host_only(SAN), "-c", src, "-o", obj],
                       check=True, capture_output=True)
        objs.append(obj)
    lib = os.path.join(out_dir, "libpagedattn.so")
    subprocess.run([HIPCC, f"--offload-arch={hip_build.ARCH}", "-shared", "-fPIC",
                    *host_only(["-fsanitize=address", "-fsanitize=undefined", "-shared-libasan"]),
                    "-o", lib, *objs], check=True, capture_output=True)
    orc = os.path.join(out_dir, "liboracle.so")
    subprocess.run([f"{LLVM}/bin/clang", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    "-ffp-contract=off", *SAN, "-shared-libasan",
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", orc, "-lm",
                    f"-Wl,-rpath,{LLVM}/lib"], check=True, capture_output=True)
    return lib, orc


def main():
    runtime = glob.glob(f"{LLVM}/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not runtime:
        sys.exit("no LLVM AddressSanitizer runtime under /opt/rocm/llvm")
    out_dir = tempfile.mkdtemp(prefix="pa_sanitize_")
    try:
        lib, orc = build(out_dir)
        env = dict(os.environ, LD_PRELOAD=runtime[0], PAGEDATTN_LIB=lib, PA_ORACLE_LIB=orc,
                   LD_LIBRARY_PATH=f"{LLVM}/lib:" + os.environ.get("LD_LIBRARY_PATH", ""),
                   ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([sys.executable, "-m", "pytest", "tests", "-m", "not gpu", "-x", "-q",
                            "-p", "no:cacheprovider"], cwd=ROOT, env=env)
        sys.exit(r.returncode)
    finally:
        shutil.rmtree(out_dir, ignore_errors=True)


if __name__ == "__main__":
    main()
