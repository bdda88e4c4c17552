"""Builds tests/c_host/fa_host_check (a plain C program linked against
libfa.so through include/fa.h) into tests/c_host/_build/. Called by
__graft_entry__.build() after the library itself; test infrastructure."""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "exact_tiled_attention_38_amd")
OUT_DIR = os.path.join(HERE, "_build")
EXE = os.path.join(OUT_DIR, "fa_host_check")


def build():
    os.makedirs(OUT_DIR, exist_ok=True)
    # a plain C compile: the HIP runtime headers only need to be told the
    # platform (hipcc would add that, and compile as HIP)
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           f"-I{os.path.join(ROOT, 'include')}", os.path.join(HERE, "fa_host_check.c"),
           f"-L{PKG}", "-L/opt/rocm/lib", "-lfa", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../../exact_tiled_attention_38_amd:/opt/rocm/lib", "-o", EXE]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host program build failed:\n{' '.join(cmd)}\n{r.stderr}")
    return EXE


if __name__ == "__main__":
    print(build())
