"""Build libpa.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m decode_attention_paged_pa_amd.build

Flags: -O3, no fast-math (fp32 division and the FP8 quantisation steps must
be IEEE correctly rounded), f32 denormals kept, packed-fp32 instructions
disabled, code object v5 so that the HIP runtime bundled with PyTorch loads it.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libpa.so")
SOURCES = ["pa_api.cpp", "pa_decode.hip", "pa_append.hip", "pa_evict.hip", "pa_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def hipcc_flags():
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
        "-mcode-object-version=5", "-fno-gpu-flush-denormals-to-zero",
        "-fhip-fp32-correctly-rounded-divide-sqrt",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I" + os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function",
    ]


def build(verbose=False, extra_flags=(), out_path=None, src_dir=None, link_flags=()):
    """Compile every source and link libpa.so; raises on failure.

    extra_flags (e.g. -D tuning knobs), link_flags, out_path and src_dir serve
    parameter sweeps, instrumented host builds and comparisons with other
    versions of the sources.
    """
    out_path = out_path or LIB_PATH
    src_dir = src_dir or CSRC
    out_dir = os.path.dirname(out_path)
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    obj_dir = os.path.join(out_dir, "obj_" + os.path.basename(out_path).replace(".", "_"))
    os.makedirs(obj_dir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(obj_dir, src + ".o")
        lang = ["-x", "hip"]
        cmd = [HIPCC] + hipcc_flags() + list(extra_flags) + lang + [
            "-c", os.path.join(src_dir, src), "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = out_path + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + list(link_flags) + objs
    _run(cmd, verbose)
    os.replace(tmp, out_path)
    return out_path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in p.stderr.splitlines() if noise not in l)
    if p.returncode != 0:
        raise RuntimeError("build failed: %s\n%s" % (" ".join(cmd), err))
    if verbose and err.strip():
        print(err, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose=True))
