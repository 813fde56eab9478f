"""Host AddressSanitizer + UndefinedBehaviorSanitizer run of the C-ABI
validation layer (argument, shape, alignment and size checks; codebook and
size queries), on the CPU.

Builds a copy of the library whose host code is instrumented (every
-fsanitize flag goes to the host compilation only: GPU code is never
sanitized) into _build/sanitize/, then runs tests/test_abi.py against it
with the ASan runtime preloaded into the Python process. Those tests make
no GPU compute call, so the run needs no GPU.

    python bit_nf4_quantized_amd/sanitize.py
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
from bit_nf4_quantized_amd import build as B  # noqa: E402

OUT = os.path.join(B.ROOT, "_build", "sanitize")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def compile_one(src: str) -> str:
    obj = os.path.join(OUT, src + ".o")
    cmd = [B.hipcc()] + B.common_flags() + B.EXTRA_FLAGS.get(src, []) + HOST_SAN + \
        ["-c", os.path.join(B.CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise SystemExit(f"compile {src} failed:\n{r.stderr}")
    return obj


def asan_runtime() -> str:
    clang = os.path.join(os.path.dirname(B.hipcc()), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    return subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                          text=True, check=True).stdout.strip()


def main() -> int:
    os.makedirs(OUT, exist_ok=True)
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, B.SOURCES))
    lib = os.path.join(OUT, B.LIB_NAME)
    link = [B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-o", lib] + objs + \
        ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan"]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode:
        raise SystemExit(f"link failed:\n{r.stderr}")
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["QLORA_NF4_LIB"] = lib
    test = os.path.join(B.ROOT, "tests", "test_abi.py")
    return subprocess.call([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", test], env=env,
                           cwd=B.ROOT)


if __name__ == "__main__":
    sys.exit(main())
