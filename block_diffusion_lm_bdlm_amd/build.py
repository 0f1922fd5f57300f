"""Build the shared libraries in-tree with hipcc for gfx950.

  libbdattn.so   BDLM attention (include/bdattn.h)
  libbdvocab.so  streaming vocabulary loss (include/bdvocab.h), linked with
                 hipBLASLt for its two plain GEMMs

Every translation unit is compiled as HIP (the host ABI shares the planning
functions with the kernels) and linked into a shared library next to this
file.  Packed-fp32 instructions are disabled for the device code.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbdattn.so")
VOCAB_LIB = os.path.join(HERE, "libbdvocab.so")
BUILD = os.path.join(HERE, "_build")
SOURCES = ["bdattn.cpp", "static_fwd.cpp", "fwd.hip", "fwd_f32.hip", "pack.hip", "dq.hip", "dkdv.hip", "merge.hip"]
VOCAB_SOURCES = ["bdvocab.cpp", "vocab_rows.hip"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
VOCAB_LINK = ["-L", os.path.join(ROCM, "lib"), "-lhipblaslt", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
# Per-file code generation options for the bf16 kernels: every matrix
# product is a compiler builtin in the VGPR form, so scores feed vector code
# with no AGPR -> VGPR copies and the compiler places every wait state
# around the products.  The global->LDS copies set M0 in inline assembly;
# these files make no other use of M0, so the reserved-register warning is
# off.
_MFMA_VGPR = ["-mllvm", "-amdgpu-mfma-vgpr-form", "-Wno-inline-asm"]
EXTRA = {"dkdv.hip": _MFMA_VGPR, "fwd.hip": _MFMA_VGPR, "dq.hip": _MFMA_VGPR}
ARCH = os.environ.get("BDATTN_ARCH", "gfx950")


def _hipcc():
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.sep not in cand or os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src, build_dir=BUILD, host_flags=()):
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    host = [x for f in host_flags for x in ("-Xarch_host", f)]
    cmd = [_hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + _flags() + EXTRA.get(src, []) + host
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln)
    return obj, warn


def _link(objs, out, extra=()):
    tmp = out + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + list(objs) + list(extra)
    subprocess.run(cmd, check=True, capture_output=not verbose_link[0])
    os.replace(tmp, out)


verbose_link = [False]


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    verbose_link[0] = verbose
    srcs = SOURCES + VOCAB_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        results = dict(zip(srcs, ex.map(_compile, srcs)))
    for _, warn in results.values():
        if warn.strip() and verbose:
            print(warn, file=sys.stderr)
    _link([results[x][0] for x in SOURCES], LIB)
    _link([results[x][0] for x in VOCAB_SOURCES], VOCAB_LIB, VOCAB_LINK)
    return LIB


def build_sanitized(out_dir, sanitizers=("address", "undefined")):
    """libbdattn.so with the host code built under the given sanitizers
    (device code unchanged), into out_dir, for the CPU sanitizer job: the
    host planner, argument validation and workspace carving run under
    AddressSanitizer / UndefinedBehaviorSanitizer there.  The library then
    needs the clang sanitizer runtime preloaded."""
    os.makedirs(out_dir, exist_ok=True)
    flags = ["-fsanitize=" + ",".join(sanitizers), "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        results = list(ex.map(lambda x: _compile(x, out_dir, flags), SOURCES))
    out = os.path.join(out_dir, "libbdattn.so")
    host_link = [x for f in flags for x in ("-Xarch_host", f)] + ["-shared-libsan"]
    _link([r[0] for r in results], out, host_link)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
