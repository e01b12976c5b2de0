"""Build the C consumer of the ABI (tests/c_abi/uly_c_smoke) with the host C compiler."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "uly_c_smoke")


def build() -> str:
    rpath = "$ORIGIN/../../sequence_attention_ulysses_amd:$ORIGIN/../../oracle:/opt/rocm/lib"
    cmd = ["gcc", "-O2", "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", os.path.join(HERE, "uly_c_smoke.c"), "-o", EXE + ".tmp",
           "-L", os.path.join(ROOT, "sequence_attention_ulysses_amd"), "-luly",
           "-L", os.path.join(ROOT, "oracle"), "-loracle", "-L", "/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath," + rpath]
    subprocess.check_call(cmd)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build())
