"""Compile the HIP library for gfx950 into blocked_prefill_amd/librt_prefill.so (in-tree).

Each source is compiled to its own object (in parallel), then the objects are
linked into the shared library."""
import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "librt_prefill.so")
PROBE = os.path.join(HERE, "librt_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          # packed-fp32 instructions stay out of the device code
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument"]
# Per-source code-generation options. The attention kernels keep their MFMA
# accumulators in ordinary VGPRs: the softmax reads every score, and
# accumulation registers would cost a copy per score plus occupancy.
EXTRA = {
    "update.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "backward.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}
# the host pass warns that it does not know the packed-fp32 feature; that is harmless
NOISE = "is not a recognized feature for this target"


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in r.stderr.splitlines() if NOISE not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="rt_build_") as tmp:
        jobs = []
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            jobs.append((src, obj, [HIPCC, *COMMON, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]))
        workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
        with ThreadPoolExecutor(workers) as ex:
            for f in [ex.submit(_run, cmd, verbose) for _, _, cmd in jobs]:
                f.result()
        _run([HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", *[o for _, o, _ in jobs], "-o", LIB + ".tmp"],
             verbose)
    os.replace(LIB + ".tmp", LIB)
    # the benchmark's bandwidth probes (a separate library: not part of the layer's path)
    _run([HIPCC, *COMMON, "-shared", os.path.join(HERE, "probe", "stream_ceiling.hip"), "-o", PROBE + ".tmp"],
         verbose)
    os.replace(PROBE + ".tmp", PROBE)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
