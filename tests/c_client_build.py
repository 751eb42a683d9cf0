"""Compile tests/c_abi_client.c (a plain C99 program that calls libsage_mi355x.so
through its public header) with gcc against the HIP runtime's C API."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_client.c")
EXE = os.path.join(HERE, "c_abi_client")
LIBDIR = os.path.join(ROOT, "quantized_softmax_attention_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    tmp = EXE + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), SRC, "-o", tmp,
           "-L", LIBDIR, "-lsage_mi355x", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../quantized_softmax_attention_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("gcc failed for c_abi_client.c:\n" + r.stdout + r.stderr)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print("built", build())
