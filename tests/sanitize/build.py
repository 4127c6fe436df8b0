"""Host-only builds with AddressSanitizer and UndefinedBehaviorSanitizer
(test infrastructure): the CPU oracle (oracle/mx_oracle.c) and the C-ABI
validation layer (mx_api.cpp) linked against stub launchers.  Plain gcc/g++,
no device code.  Outputs go to _build/sanitize/."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(ROOT, "_build", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ORACLE_LIB = os.path.join(OUT, "libmxoracle_san.so")
API_LIB = os.path.join(OUT, "libmxfp8_api_san.so")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(" ".join(cmd) + "\n" + r.stdout + r.stderr)


def build():
    os.makedirs(OUT, exist_ok=True)
    _run(["gcc", "-std=c11", "-shared", "-fPIC", *SAN, os.path.join(ROOT, "oracle", "mx_oracle.c"),
          "-o", ORACLE_LIB, "-lm"])
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    _run(["g++", "-std=c++17", "-shared", "-fPIC", *SAN, "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
          os.path.join(ROOT, "mxfp8_block_scaled_08_amd", "csrc", "mx_api.cpp"),
          os.path.join(HERE, "stub_launchers.cpp"), "-o", API_LIB,
          "-L", os.path.join(rocm, "lib"), "-Wl,-rpath," + os.path.join(rocm, "lib"), "-lamdhip64"])
    return ORACLE_LIB, API_LIB


def runtime_preload() -> str:
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
