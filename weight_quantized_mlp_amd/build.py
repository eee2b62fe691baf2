"""Build libwqmlp.so (gfx950 only) in-tree with hipcc.

Every source is compiled for gfx950 with packed-FP32 instruction selection
disabled, then linked into ``weight_quantized_mlp_amd/libwqmlp.so``.  Runs
without a GPU (hipcc cross-compiles).
"""
import concurrent.futures
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["abi.cpp", "gemv.hip", "gemv_fast.hip", "mfma.hip", "moe.hip", "pack.hip", "probe.hip"]
LIB = os.path.join(HERE, "libwqmlp.so")
ARCH = "gfx950"
FLAGS = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument", f"-I{os.path.join(ROOT, 'include')}"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# Host-only sanitizers (AddressSanitizer + UndefinedBehaviorSanitizer on the host code of every source; the
# gfx950 code objects are built as usual).  Used by the CPU test that runs the ABI checks under them.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src, obj, hipcc, extra=()):
    cmd = [hipcc, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + FLAGS + list(extra)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=False, sanitize=False, out=None):
    """Build the library.  sanitize=True adds the host-side sanitizers (SAN_FLAGS) and writes to `out`
    (default _build/san/libwqmlp.so) instead of the in-tree library."""
    hipcc = _hipcc()
    bdir = os.path.join(ROOT, "_build", "san" if sanitize else "")
    os.makedirs(bdir, exist_ok=True)
    lib = (out or os.path.join(bdir, "libwqmlp.so")) if sanitize else LIB
    extra = SAN_FLAGS if sanitize else ()
    objs = [os.path.join(bdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        list(ex.map(lambda a: _compile(a[0], a[1], hipcc, extra), zip(SOURCES, objs)))
    tmp = lib + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if sanitize:
        cmd += ["-fsanitize=address,undefined", "-shared-libsan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True)
