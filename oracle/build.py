"""Builds the CPU oracle library (test infrastructure only).

``build()`` compiles ``gdn_oracle.c`` with gcc into ``liboracle.so`` next to
this file; ``build(mutant=n)`` builds the variant with planted mistake ``n``
into ``_mutants/liboracle_m{n}.so`` (used only by the pin-sensitivity test).
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
         "-Wall", "-Wextra"]


def lib_path(mutant: int = 0) -> str:
    if mutant == 0:
        return os.path.join(HERE, "liboracle.so")
    return os.path.join(HERE, "_mutants", f"liboracle_m{mutant}.so")


def build(mutant: int = 0) -> str:
    out = lib_path(mutant)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", *FLAGS, *(["-Werror"] if mutant == 0 else ["-Wno-unused"]), f"-DORACLE_MUTANT={mutant}",
           os.path.join(HERE, "gdn_oracle.c"), "-o", tmp, "-lpthread", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
