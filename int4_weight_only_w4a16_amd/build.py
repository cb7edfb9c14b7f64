"""Build libw4a16.so in-tree with hipcc for gfx950 (host packer + C ABI + HIP kernels).

Each source compiles to its own object in parallel (the GEMV template is
instantiated once per activation-row count M in gemv_m1.hip .. gemv_m8.hip),
then hipcc links the shared library."""
import concurrent.futures
import os
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libw4a16.so")
SOURCES = ["api.cpp", "pack.cpp", "quantize.cpp", "w4a16_kernels.hip", "gemm_kernel.hip", "a8_kernels.hip", "noalloc.hip", "chain.hip"] + [f"gemv_m{m}.hip" for m in range(1, 9)]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 VALU ops (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    # gfx950 can hand a kernel its first 14 argument dwords in SGPRs: the
    # kernels list what they need at entry first, so they start without a
    # scalar load (0.24 us less per dependent launch in the decode step).
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    return res.returncode, noise


def build(verbose=False, jobs=None):
    """Compile every source into LIBRARY (always recompiles)."""
    jobs = jobs or min(8, os.cpu_count() or 1)
    with tempfile.TemporaryDirectory(prefix="w4a16_build_") as tmp:
        objs, cmds = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            objs.append(obj)
            cmds.append([hipcc()] + HIPCC_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c",
                                                   os.path.join(CSRC, src), "-o", obj])
        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as pool:
            results = list(pool.map(_run, cmds))
        for src, (rc, noise) in zip(SOURCES, results):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(noise))
            if verbose and noise:
                print("\n".join(noise))
        out = LIBRARY + ".tmp"
        rc, noise = _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", out, "-lpthread"])
        if rc != 0:
            raise RuntimeError("hipcc link failed:\n" + "\n".join(noise))
    os.replace(out, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
