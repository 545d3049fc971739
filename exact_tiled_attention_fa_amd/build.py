"""Build libfa.so (gfx950) in-tree with hipcc, and the benchmark's
matrix-core probe as a library of its own (libfa_probe.so, not part of the
attention ABI).

    python -m exact_tiled_attention_fa_amd.build [-v]

Every source is compiled for gfx950 only.  Packed-fp32 VALU instructions are
disabled for device code (``-Xclang -target-feature -Xclang -packed-fp32-ops``):
the kernels are written with scalar float arithmetic and must not be turned
into v_pk_* fp32 forms by the compiler.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
OUT_DIR = PKG / "_lib"
LIB = OUT_DIR / "libfa.so"
OBJ_DIR = ROOT / "_build"

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_decode.hip", "fa_decode_noalloc.hip", "fa_bwd.hip",
           "fa_fwd_fp8.hip"]
PROBE_SOURCES = ["probe/mfma_probe.hip", "probe/rate_probe.hip", "probe/rate_probe_vgpr.hip"]
# Per-source extra flags.  The decode kernels keep their MFMA accumulators in
# ArchVGPRs: with the compiler's default split they live in AccVGPRs across
# the key loop and are copied out and back every step (about 300 moves per
# kernel), and the int8 instances need a fourth of the file more registers.
EXTRA_FLAGS = {"probe/rate_probe_vgpr.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "fa_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
PROBE_LIB = OUT_DIR / "libfa_probe.so"
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = (res.stdout or "") + (res.stderr or "")
    # hipcc's host pass does not know the packed-fp32 feature; drop that warning only.
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln or "error" in ln]
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))


def _obj(src: str) -> Path:
    return OBJ_DIR / (src.replace("/", "_").replace(".", "_") + ".o")


def _link(objs, lib: Path, verbose: bool) -> None:
    tmp = lib.with_suffix(".so.tmp")
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)],
         verbose)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> Path:
    """Compile every source and link libfa.so and libfa_probe.so; always
    rebuilds.  Returns the path of libfa.so."""
    OUT_DIR.mkdir(parents=True, exist_ok=True)
    OBJ_DIR.mkdir(parents=True, exist_ok=True)
    cc = hipcc()
    cmds = []
    for src in SOURCES + PROBE_SOURCES:
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([cc, *common_flags(), *EXTRA_FLAGS.get(src, []), *lang, "-c", str(CSRC / src),
                     "-o", str(_obj(src))])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    _link([_obj(s) for s in SOURCES], LIB, verbose)
    _link([_obj(s) for s in PROBE_SOURCES], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
