"""Builds libssd.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Each translation unit compiles in parallel; the shared library is linked next
to this file, where the Python binding loads it.
"""
import concurrent.futures
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libssd.so")
SOURCES = ["ssd_api.hip", "ssd_meta.hip", "ssd_scan_bf16.hip", "ssd_scan_f32.hip",
           "ssd_scan_split_bf16.hip", "ssd_scan_ws_bf16.hip", "ssd_decode.hip", "ssd_conv1d.hip", "ssd_gdn.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         # no packed-fp32 instructions anywhere in the device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         f"-I{INCLUDE}"]


# per-source compiler flags (none at present)
SOURCE_FLAGS = {}


def _compile(src, obj):
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(out=LIB, jobs=4):
    """Compile every source and link `out`; returns its path."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(_compile, SOURCES, objs))
    tmp = out + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
