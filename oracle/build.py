"""Build the CPU oracle shared library (test infrastructure).

Compiles oracle/moe_oracle.c with gcc into oracle/libmoe_oracle.so. Plain
-O2 (no -march=native: the library built here also runs on other hosts).

build(sanitize=True) makes oracle/libmoe_oracle_san.so instead: the same
source under AddressSanitizer and UndefinedBehaviorSanitizer (plus the
float -> int conversion check, which -fsanitize=undefined leaves out), with
every UB report fatal. A process loads it with the ASan runtime preloaded
(asan_runtime()) and MOE_ORACLE_LIB pointing at it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmoe_oracle.so")
SAN_LIB = os.path.join(HERE, "libmoe_oracle_san.so")

_SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer",
              "-fsanitize=address,undefined,float-cast-overflow",
              "-fno-sanitize-recover=all"]


def asan_runtime() -> str:
    """Path of gcc's ASan runtime (to preload into an unsanitized Python)."""
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def build(verbose: bool = False, sanitize: bool = False) -> str:
    src = os.path.join(HERE, "moe_oracle.c")
    out = SAN_LIB if sanitize else LIB
    tmp = out + ".tmp"
    opt = _SAN_FLAGS if sanitize else ["-O2"]
    cmd = ["gcc", *opt, "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import sys
    print(build(verbose=True, sanitize="--sanitize" in sys.argv))
