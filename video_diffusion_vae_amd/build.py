"""Build libvae_mi355x.so (gfx950) in-tree: ``python video_diffusion_vae_amd/build.py``.

Each HIP source under csrc/ is compiled to an object under _build/ in parallel, then all objects
are linked into video_diffusion_vae_amd/libvae_mi355x.so. The build always recompiles.

``python video_diffusion_vae_amd/build.py --sanitize`` builds the library with its host code
under AddressSanitizer and UndefinedBehaviorSanitizer (the device code as usual, unsanitized)
into _build_san/libvae_mi355x.so, for the host-only tests (argument checks, tiling maths,
workspace queries). Run them with that library and the sanitizer runtime preloaded:
``python video_diffusion_vae_amd/build.py --sanitize --run-host-tests``.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libvae_mi355x.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-fvisibility=hidden", "-I", os.path.join(ROOT, "include"),
    # keep packed-fp32 instructions out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, sources()))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stderr}")
    shutil.move(tmp, LIB)
    return LIB


SAN_BUILD = os.path.join(ROOT, "_build_san")
SAN_LIB = os.path.join(SAN_BUILD, "libvae_mi355x.so")
# each sanitizer flag applies to the host compilation only
SAN_FLAGS = FLAGS + ["-Xarch_host", "-g",
                     "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                     "-Xarch_host", "-fno-sanitize-recover=undefined",
                     "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile_san(src):
    obj = os.path.join(SAN_BUILD, os.path.basename(src)[:-4] + ".o")
    r = subprocess.run([HIPCC, *SAN_FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stderr}")
    return obj


def sanitizer_runtime() -> str:
    """The shared AddressSanitizer runtime of the ROCm clang (preloaded into Python)."""
    r = subprocess.run([os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm",
                                     "bin", "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("AddressSanitizer runtime not found")
    return path


def build_sanitized(jobs: int = 8) -> str:
    os.makedirs(SAN_BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile_san, sources()))
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan",
                        "-fsanitize=address,undefined", *objs, "-o", SAN_LIB],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stderr}")
    return SAN_LIB


def run_host_tests_sanitized() -> int:
    """tests/test_abi_host.py against the sanitized library (VAE_MI355X_LIB)."""
    env = dict(os.environ, VAE_MI355X_LIB=SAN_LIB, LD_PRELOAD=sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_abi_host.py")], env=env).returncode


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized())
        if "--run-host-tests" in sys.argv:
            sys.exit(run_host_tests_sanitized())
    else:
        print(build())
