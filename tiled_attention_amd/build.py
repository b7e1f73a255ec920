"""Build libattn.so for gfx950 with hipcc (in-tree, no JIT cache).

Usage: python -m tiled_attention_amd.build [-v]
Each source compiles to an object under tiled_attention_amd/_build/ in
parallel, then one link produces tiled_attention_amd/libattn.so. Every call
rebuilds everything.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libattn.so")
SOURCES = ["api.cpp", "fwd_mfma.hip", "fwd_f32.hip", "paged.hip", "quant.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-command-line-argument",
    # MFMA accumulators stay in VGPRs: the softmax reads and rescales them
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _hipcc():
    for cand in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.sep not in cand or os.path.exists(cand):
            return cand
    return "hipcc"


def _compile(src, extra, verbose):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON_FLAGS + extra
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def build(verbose=False, extra_flags=()):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags), verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


def resource_usage(src):
    """Per-kernel register, scratch and spill figures of one source, from the
    compiler's kernel-resource-usage remarks (a compile to a throw-away
    object). Returns {kernel name: {field: int}}."""
    import re
    import tempfile
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [_hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", os.path.join(tmp, "x.o")] + \
            COMMON_FLAGS + ["-Rpass-analysis=kernel-resource-usage"]
        res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    out, cur = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^]]*\])?: (\d+)", line)
        if m and cur is not None:
            out[cur][m.group(1).strip()] = int(m.group(2))
    return out


def assembly(src):
    """The gfx950 assembly the compiler writes for one source (a throw-away
    compile with -S)."""
    import tempfile
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "x.s")
        cmd = [_hipcc(), "-x", "hip", "-S", "--cuda-device-only", os.path.join(CSRC, src), "-o", out] + COMMON_FLAGS
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc -S failed for {src}:\n{res.stderr}")
        with open(out) as f:
            return f.read()


if __name__ == "__main__":
    flags = [a for a in sys.argv[1:] if a != "-v"]
    print(build(verbose="-v" in sys.argv, extra_flags=flags))
