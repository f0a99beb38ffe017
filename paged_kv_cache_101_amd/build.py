"""Build libpkv.so in-tree with hipcc for gfx950.

Each .hip source compiles to an object under _build/ (in parallel), then one
shared library is linked next to this file. Packed fp32 instructions are
switched off for every device compilation.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpkv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["pkv_api.hip", "kv_append.hip", "paged_decode.hip",
           "paged_prefill.hip", "stream_read.hip"]
HOST_SOURCES = ["block_manager.cpp"]  # plain host C++ (g++)
CXX = os.environ.get("CXX", "g++")
HOST_CFLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", f"-I{INCLUDE}"]
# PKV_SANITIZE=1: the host C++ (the block manager) is built with gcc's
# AddressSanitizer and UndefinedBehaviorSanitizer, and the library links their
# runtimes; the device code is unchanged. Load it in a process that preloads
# the runtimes (see sanitizer_env()); rebuild without the variable before any
# GPU run.
SANITIZE = os.environ.get("PKV_SANITIZE", "") == "1"
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"]


def sanitizer_runtimes():
    """gcc's ASan and UBSan runtime libraries (paths)."""
    return [subprocess.run([CXX, f"-print-file-name={n}"], capture_output=True, text=True,
                           check=True).stdout.strip() for n in ("libasan.so", "libubsan.so")]


def sanitizer_env() -> dict:
    """Environment for a Python process that loads sanitized builds."""
    env = dict(os.environ)
    env["LD_PRELOAD"] = ":".join(sanitizer_runtimes())
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning
    # is expected and dropped here.
    msgs = [l for l in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in l]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs))
    return obj


def _compile_host(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [CXX, *HOST_CFLAGS, *(SAN_FLAGS if SANITIZE else []), "-c", os.path.join(CSRC, src),
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{CXX} failed for {src}:\n" + r.stdout + r.stderr)
    if (r.stdout + r.stderr).strip() and verbose:
        print(r.stdout + r.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES) + len(HOST_SOURCES)) as ex:
        jobs = [ex.submit(_compile, s, verbose) for s in SOURCES]
        jobs += [ex.submit(_compile_host, s, verbose) for s in HOST_SOURCES]
        objs = [j.result() for j in jobs]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if SANITIZE:
        cmd += sanitizer_runtimes()  # the instrumented host objects need them
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def sanitized_cpu_tests() -> int:
    """Build libpkv.so and the oracle with the sanitizers, run the CPU test
    suite (pytest -m "not gpu") in a process that preloads their runtimes,
    then rebuild both without them. Returns pytest's exit status."""
    env = dict(os.environ, PKV_SANITIZE="1")
    for mod in ("paged_kv_cache_101_amd.build", "oracle.build"):
        subprocess.run([sys.executable, "-c", f"import {mod} as b; b.build()"], cwd=ROOT, env=env,
                       check=True)
    rc = subprocess.run([sys.executable, "-m", "pytest", "tests", "-m", "not gpu", "-q",
                         "-p", "no:cacheprovider"], cwd=ROOT, env=sanitizer_env()).returncode
    for mod in ("paged_kv_cache_101_amd.build", "oracle.build"):
        subprocess.run([sys.executable, "-c", f"import {mod} as b; b.build()"], cwd=ROOT,
                       env={k: v for k, v in os.environ.items() if k != "PKV_SANITIZE"},
                       check=True)
    return rc


if __name__ == "__main__":
    if "--sanitized-cpu-tests" in sys.argv:
        sys.exit(sanitized_cpu_tests())
    print(build(verbose="-v" in sys.argv))
