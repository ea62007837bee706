"""Build libmxgemm.so (the gfx950 HIP library) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
# the host side of the C ABI, then one translation unit per kernel family
# (each holds that family's template instantiations), compiled in parallel
SRCS = ["k_large_exact.hip", "k_large_exact_b.hip", "k_large_native.hip", "k_large_e2m1.hip",
        "k_stream.hip", "k_skinny_fp8.hip", "k_skinny_e2m1.hip", "k_quant.hip", "mxgemm.hip"]
OUT = os.path.join(HERE, "libmxgemm.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off (the compiler would otherwise form them
    # from float2 arithmetic in the epilogue)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmxgemm.so)")


def build(out: str = OUT, extra=(), jobs: int = None) -> str:
    """Compile every translation unit to an object (at most `jobs` at once,
    default: the CPU count, up to 8), then link libmxgemm.so."""
    import concurrent.futures
    import tempfile
    cc = hipcc()
    jobs = jobs or min(8, os.cpu_count() or 1)
    with tempfile.TemporaryDirectory(prefix="mxgemm_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            cmd = [cc, *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                   "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            return src, obj, r
        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(compile_one, SRCS))
        failed = [(src, r) for src, _, r in results if r.returncode != 0]
        for src, _, r in results:
            # hipcc's host pass does not know the device-only feature flag
            msg = [ln for ln in (r.stdout + r.stderr).splitlines()
                   if "is not a recognized feature for this target" not in ln]
            if msg:
                print(f"--- {src}\n" + "\n".join(msg))
        if failed:
            raise RuntimeError("hipcc failed on " + ", ".join(src for src, _ in failed))
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC",
               *[obj for _, obj, _ in results], "-o", out + ".tmp"]
        subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
