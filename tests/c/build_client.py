"""Compile the plain C client of libdita (tests/c/dita_c_client) with gcc.

It links the in-tree libdita.so and the HIP runtime; run after the library is
built.  Usage: ``python tests/c/build_client.py`` or ``build()``.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "partial_state_reuse_amd")
OUT = os.path.join(HERE, "dita_c_client")


def build() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           f"-I{rocm}/include", os.path.join(HERE, "dita_c_client.c"), "-o", OUT,
           f"-L{PKG}", "-ldita", f"-L{rocm}/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../partial_state_reuse_amd", f"-Wl,-rpath,{rocm}/lib"]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode:
        raise RuntimeError("C client build failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return OUT


if __name__ == "__main__":
    print(build())
    sys.exit(0)
