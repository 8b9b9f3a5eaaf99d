"""Build the C-ABI shared library ``libattn.so`` for gfx950 with hipcc, and the
benchmark's MFMA-only probe ``libmfma_probe.so`` (a measurement aid loaded only
by bench.py, not part of the attention boundary).

Run ``python -m head_attention_amd.build`` (or call ``build()``); the libraries
are written next to this file, in-tree, so that they travel with the source tree.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libattn.so")
SOURCES = [os.path.join(HERE, "csrc", "attn_fwd.hip"), os.path.join(HERE, "csrc", "attn_bwd.hip"),
           os.path.join(HERE, "csrc", "merge_host.cpp")]
PROBE_LIB = os.path.join(HERE, "libmfma_probe.so")
PROBE_SOURCES = [os.path.join(HERE, "csrc", "mfma_probe.hip")]

# Packed fp32 VALU forms are disabled for every HIP translation unit.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(HERE, "csrc"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def _link(sources, out, verbose):
    tmp = out + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + sources + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile both libraries (always); returns the path of libattn.so."""
    _link(SOURCES, LIB, verbose)
    _link(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
