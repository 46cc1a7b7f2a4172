"""Build the HIP library (libmla_decode.so) in-tree for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
SRC = PKG / "csrc" / "mla_decode.hip"
INCLUDE = ROOT / "include"
LIB = PKG / "libmla_decode.so"
# the streaming-read probe the benchmark measures attainable HBM reads with
PROBE_SRC = PKG / "csrc" / "hbm_probe.hip"
PROBE_LIB = PKG / "libhbm_probe.so"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build_library(out: Path | str = LIB, extra_flags=(), src: Path | str = SRC) -> Path:
    """Compile csrc/mla_decode.hip (or another source) for gfx950 into a
    shared library."""
    out = Path(out)
    tmp = out.with_name(out.name + f".tmp{os.getpid()}")
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           f"-I{INCLUDE}",
           # packed-fp32 VALU forms stay off: the kernels are written for the
           # scalar forms and do not rely on v_pk_*_f32
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           *extra_flags, str(src), "-o", str(tmp)]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + proc.stderr[-4000:])
    os.replace(tmp, out)
    return out


def build_probe() -> Path:
    """Compile the streaming-read probe (csrc/hbm_probe.hip)."""
    return build_library(PROBE_LIB, src=PROBE_SRC)


if __name__ == "__main__":
    print(build_library())
    print(build_probe())
