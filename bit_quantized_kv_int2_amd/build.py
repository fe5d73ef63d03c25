"""Build the HIP library libkvq.so in-tree for gfx950 (hipcc cross-compiles
without a GPU). Each source is compiled to its own object (in parallel), then
linked."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkvq.so")
# debug build: every kernel fills its LDS with all-ones bytes before use
POISON_LIB = os.path.join(PKG, "libkvq_poison.so")
SOURCES = ["kvq_api.hip", "kvq_pack.hip", "kvq_decode.hip", "kvq_decode_tg.hip", "kvq_bf16.hip",
           "kvq_stream.hip", "kvq_append.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fno-fast-math",
    # no packed-fp32 instructions (v_pk_*_f32) in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# The decode kernels never produce or consume NaN (masked scores are -inf and
# every exp2 argument is finite or -inf). Without NaN semantics the IEEE mode
# bit can be cleared, so float max needs no operand canonicalisation and a
# DPP row rotation folds into the max itself.
EXTRA_FLAGS = {"kvq_decode.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
               "kvq_decode_tg.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
               # the issue probe's products keep their accumulators in VGPRs
               # (no accumulator-register copies inside its timed loops)
               "kvq_stream.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(hipcc, src, obj, defines):
    cmd = [hipcc, *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), *defines,
           "-I" + os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj]
    return subprocess.run(cmd, capture_output=True, text=True)


def build(verbose: bool = False, poison: bool = False) -> str:
    """Build libkvq.so, or with poison=True the LDS poison-fill debug build
    libkvq_poison.so (same sources and entry points, KVQ_POISON_LDS defined)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    lib_path = POISON_LIB if poison else LIB
    defines = ["-DKVQ_POISON_LDS"] if poison else []
    tag = f".tmp{os.getpid()}" + ("p" if poison else "")
    objs = [os.path.join(PKG, os.path.splitext(s)[0] + tag + ".o") for s in SOURCES]
    try:
        with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            results = list(ex.map(lambda so: _compile(hipcc, *so, defines), zip(SOURCES, objs)))
        for src, r in zip(SOURCES, results):
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n" + r.stdout + r.stderr)
            if verbose and r.stderr:
                print(r.stderr)
        tmp = lib_path + tag
        r = subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc link failed:\n" + r.stdout + r.stderr)
        os.replace(tmp, lib_path)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return lib_path


if __name__ == "__main__":
    print(build(verbose=True))
