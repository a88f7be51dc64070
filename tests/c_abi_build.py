"""Build tests/c_abi_main (a plain C99 caller of the library, see c_abi_main.c)
with the host C compiler: include/int8lin.h compiled as C, linked against
libint8lin.so and the HIP runtime, found at run time through the rpath."""
from __future__ import annotations

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi_main.c")
OUT = os.path.join(ROOT, "tests", "c_abi_main")
PKG = os.path.join(ROOT, "int8_quantized_linear_rowwise_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CC = os.environ.get("CC", "gcc")


def command(out: str = OUT) -> list:
    return [CC, "-std=c99", "-O3", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
            f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}", SRC, f"-L{PKG}", "-lint8lin",
            f"-L{ROCM}/lib", "-lamdhip64",
            "-Wl,-rpath,$ORIGIN/../int8_quantized_linear_rowwise_amd", f"-Wl,-rpath,{ROCM}/lib", "-o", out]


def build(out: str = OUT) -> str:
    r = subprocess.run(command(out), capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C caller build failed:\n{' '.join(command(out))}\n{r.stdout}\n{r.stderr}")
    return out


if __name__ == "__main__":
    print(build())
