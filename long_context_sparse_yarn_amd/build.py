"""Build libsinkattn.so for gfx950 in-tree (hipcc, no JIT cache).

    python long_context_sparse_yarn_amd/build.py [--verbose]

(Run it as a script, not with -m: importing it through the package would
first load the library it is about to build.)

Every call compiles from scratch.  Flags: -O3, gfx950 only, and the packed
fp32 instructions disabled on the device (-packed-fp32-ops).
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsinkattn.so")
BUILD = os.path.join(HERE, "_build")
SOURCES = ["sinkattn_abi.hip", "rope.hip", "append.hip", "prefill.hip", "decode.hip", "qkv.hip", "moe.hip",
           "attn_f32.hip", "sample.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    "-mcode-object-version=5",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    # drop the host pass's notice about the device-only target feature
    noise = ("packed-fp32-ops", "not a recognized feature", "warning generated",
             "warnings generated")
    err = "\n".join(l for l in r.stderr.splitlines() if l and not any(n in l for n in noise))
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for s in SOURCES:
        o = os.path.join(BUILD, s.replace(".hip", ".o"))
        objs.append(o)
        cmds.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
    with ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    # --no-undefined: a kernel whose host-side launch stub went missing fails here, not at load
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-Wl,--no-undefined", *objs, "-o", tmp],
         verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
