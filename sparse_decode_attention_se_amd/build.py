"""Build libse.so (HIP, gfx950) in place next to this file.

    python -m sparse_decode_attention_se_amd.build

Every source in csrc/ is compiled by hipcc for gfx950 and linked into one shared library. Packed fp32 vector
instructions are disabled for the device code, and MFMA results are kept in VGPRs.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libse.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# -amdgpu-mfma-vgpr-form: MFMA results go to ordinary VGPRs (the vector code reads them there); operands that only
# the MFMAs read may still sit in the accumulation registers
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form", "-shared"]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(x for x in res.stderr.splitlines() if "packed-fp32-ops" not in x)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile each source to an object (in parallel), then link libse.so."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(HERE, "..", "include")]
    objs = [os.path.join(objdir, os.path.basename(s)[:-4] + ".o") for s in sources()]
    cmds = [[HIPCC, *FLAGS[:-1], "-c", *inc, s, "-o", o] for s, o in zip(sources(), objs)]
    cmds = [[x for x in c if x != "-shared"] for c in cmds]
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
