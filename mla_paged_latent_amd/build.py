"""Build the HIP library (gfx950) in-tree: mla_paged_latent_amd/libmla_paged_latent.so.

    python -m mla_paged_latent_amd.build [--verbose]

hipcc compiles every csrc/*.hip file for gfx950 and links one shared object
with a plain C ABI (include/mla_paged_latent.h). No GPU is needed to build.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libmla_paged_latent.so"
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off: the compiler keeps to scalar/vector fp32 forms
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

# Per-source extra flags. The wide decode kernel uses the VGPR form of the
# matrix ops, so its output accumulators can be rescaled in place.
FILE_FLAGS = {
    # matrix-op accumulators in VGPRs: the online-softmax rescale multiplies them in
    # place instead of the loop copying them between AGPRs and VGPRs every step
    "mla_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "mla_decode_wide.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "mla_decode_wide_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(CSRC.glob("*.hip"))


def build(verbose: bool = False, out: Path = LIB, extra_flags=(), objdir: Path | None = None) -> Path:
    """Compile and link; always rebuilds. Returns the library path."""
    objdir = Path(objdir) if objdir is not None else ROOT / "_build" / "obj"
    objdir.mkdir(parents=True, exist_ok=True)
    objs = []
    cc = hipcc()
    for src in sources():
        obj = objdir / (src.stem + ".o")
        cmd = [cc, *HIPCC_FLAGS, *FILE_FLAGS.get(src.name, []), *extra_flags, "-I", str(ROOT / "include"), "-c", str(src), "-o", str(obj)]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed on %s:\n%s" % (src.name, msg))
        if verbose and msg.strip():
            print(msg, flush=True)
        objs.append(str(obj))
    tmp = out.with_name(out.name + ".tmp%d" % os.getpid())
    cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    path = build(verbose="--verbose" in sys.argv)
    print(path)
