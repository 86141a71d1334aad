"""Builds the HIP libraries in-tree for gfx950 with hipcc: libmsa_indexer.so (the decode pass)
and libmsa_probe.so (the streaming-ceiling probe bench.py measures beside it)."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCE = os.path.join(HERE, "csrc", "msa_indexer.hip")
PROBE_SOURCE = os.path.join(HERE, "csrc", "stream_probe.hip")
INCLUDE = os.path.join(ROOT, "include")
ARCH = "gfx950"


def library_path() -> str:
    return os.path.join(HERE, "libmsa_indexer.so")


def probe_library_path() -> str:
    return os.path.join(HERE, "libmsa_probe.so")


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Wall", "-Wno-unused-function",
        # Keep hipcc from emitting packed fp32 instructions (v_pk_fma_f32 and friends).
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}",
    ]


def _compile(source: str, out: str, verbose: bool, extra: list[str] | None) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *compile_flags(), *(extra or []), source, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{msg}")
    if verbose and msg.strip():
        print(msg, flush=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, extra: list[str] | None = None, out: str | None = None) -> str:
    """Compiles libmsa_indexer.so (to `out` if given); without `out`, also libmsa_probe.so."""
    path = _compile(SOURCE, out or library_path(), verbose, extra)
    if out is None:
        _compile(PROBE_SOURCE, probe_library_path(), verbose, extra)
    return path


if __name__ == "__main__":
    print(build(verbose=True))
