"""Builds the host-side sanitizer driver (driver.cpp) with AddressSanitizer
and UndefinedBehaviorSanitizer: the driver, the C ABI's host code
(csrc/abi.cpp, its device code unsanitized), the host leg and residency
policy, the oracle and the input generator are instrumented; the other HIP
objects of the library build are linked as they are.  Output:
_build/sanitize/driver.  CPU only; run by tests/test_sanitizers.py."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
OUT = os.path.join(ROOT, "_build", "sanitize")
EXE = os.path.join(OUT, "driver")
LLVM = "/opt/rocm/llvm/bin"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
# hipcc: each sanitizer flag for the host side only, right after -Xarch_host
SAN_HOST_ONLY = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
                 "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd: list) -> None:
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd[:3])} ... failed:\n{r.stderr[-4000:]}")


def build() -> str:
    from quantized_routed_expert_moe_amd import build as B

    os.makedirs(OUT, exist_ok=True)
    csrc = os.path.join(ROOT, "quantized_routed_expert_moe_amd", "csrc")
    host = os.path.join(ROOT, "quantized_routed_expert_moe_amd", "host")
    inc = ["-I" + os.path.join(ROOT, "include")]
    objs = []
    # the C ABI's host code, instrumented (device code as in the library)
    abi = os.path.join(OUT, "abi.o")
    _run([B.HIPCC, *[f for f in B.FLAGS if f not in ("-O3",)], *SAN_HOST_ONLY, "-x", "hip", "-c",
          os.path.join(csrc, "abi.cpp"), "-o", abi])
    objs.append(abi)
    for src, lang in ((os.path.join(ROOT, "oracle", "oracle.c"), "c"), (os.path.join(ROOT, "fixtures", "fixtures.c"), "c"),
                      (os.path.join(host, "host_leg.cpp"), "c++"), (os.path.join(host, "residency.cpp"), "c++"),
                      (os.path.join(HERE, "driver.cpp"), "c++")):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        cc = os.path.join(LLVM, "clang" if lang == "c" else "clang++")
        std = "-std=c11" if lang == "c" else "-std=c++17"
        _run([cc, std, *SAN, "-fopenmp", "-fPIC", *inc, "-c", src, "-o", obj])
        objs.append(obj)
    # the library's other objects, as built by the package build
    for src in B.SOURCES:
        if src == "abi.cpp":
            continue
        obj = os.path.join(B.BUILD, os.path.splitext(src)[0] + ".o")
        if not os.path.exists(obj):
            B.build()
        objs.append(obj)
    objs += [os.path.join(B.BUILD, f"ffn_prefill_{t}.o") for t in B.PREFILL_TYPES]
    _run([os.path.join(LLVM, "clang++"), *SAN, "-fopenmp", *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/llvm/lib", "-o", EXE])
    return EXE


if __name__ == "__main__":
    print(build())
