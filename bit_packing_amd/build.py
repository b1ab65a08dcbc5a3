"""Build libibp.so for gfx950 in-tree with hipcc (no JIT cache, so the library
travels with the source tree).  Each source compiles in its own hipcc process
(in parallel), then one link."""
from __future__ import annotations

import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("ibp_meta.hip", "ibp_encode.hip", "ibp_decode.hip", "ibp_decode_pos.hip", "ibp_slots.hip", "ibp_zip.hip", "ibp_api.hip")]
LIB = os.path.join(HERE, "libibp.so")
LIB_SANITIZED = os.path.join(HERE, "libibp_san.so")
# host code only: each -fsanitize= after -Xarch_host, so no GPU code is instrumented
HOST_SAN_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                  "-Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer").split()

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed-FP32 instructions stay off in every HIP build of this project
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
]
_NOISE = "is not a recognized feature for this target"


def _run(procs):
    errs = []
    for cmd, p in procs:
        out, _ = p.communicate()
        msg = "\n".join(l for l in out.splitlines() if _NOISE not in l)
        if p.returncode != 0:
            errs.append(f"{' '.join(cmd)}\n{msg}")
    if errs:
        raise RuntimeError("hipcc failed:\n" + "\n\n".join(errs))


def build_library(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile csrc/*.hip into bit_packing_amd/libibp.so (always recompiles).  sanitize:
    libibp_san.so, whose host code (argument checks, launch set-up) is instrumented
    with AddressSanitizer and UndefinedBehaviorSanitizer."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out_lib = LIB_SANITIZED if sanitize else LIB
    extra = HOST_SAN_FLAGS if sanitize else []
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    with tempfile.TemporaryDirectory(prefix="ibp_build_") as tmpd:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmpd, os.path.basename(src) + ".o")
            cmd = [hipcc, *HIPCC_FLAGS, *extra, *inc, "-c", src, "-o", obj]
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        _run(procs)
        tmp = out_lib + ".tmp"
        cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *extra, *objs, "-o", tmp]
        _run([(cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))])
    os.replace(tmp, out_lib)
    return out_lib


if __name__ == "__main__":
    print(build_library(verbose=True))
