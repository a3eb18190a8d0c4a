"""Build libsfi.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: python -m sparse_kv_cache_sfi_amd.build   (or __graft_entry__.build()).
Always recompiles every source; objects go to sparse_kv_cache_sfi_amd/_build/.
"""
import concurrent.futures as cf
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsfi.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-fvisibility=hidden",
    # Packed fp32 instructions stay off: the device code is written as plain fp32.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(HERE, "..", "include"),
    # Per-kernel register, LDS and scratch figures (checked below).
    "-Rpass-analysis=kernel-resource-usage",
]


# The MFMA kernels keep their accumulators in architectural VGPRs: in the accumulation
# register form the online-softmax rescale copies every accumulator to VGPRs and back on
# every iteration, and the register budget then allows one wave per SIMD instead of two.
FILE_FLAGS = {
    "verify.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "mixed.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _resource_usage(stderr: str):
    """(other diagnostics, {kernel: {figure: value}}) from hipcc's kernel-resource-usage remarks."""
    usage, other, name, pending = {}, [], None, []
    in_remark = False
    for line in stderr.splitlines():
        # the source line and caret hipcc prints under a diagnostic ("   50 | ...", "      | ^")
        if re.match(r"^\s*\d*\s*\|", line):
            if not in_remark:
                other.append(line)
            continue
        if line.startswith("In file included from"):
            pending.append(line)   # context of the next diagnostic
            continue
        remark = "[-Rpass-analysis=kernel-resource-usage]" in line
        in_remark = remark
        if not remark:
            other.extend(pending)
        pending = []
        if remark:
            body = line.split("remark:", 1)[1].rsplit("[-Rpass", 1)[0].strip()
            key, _, val = body.partition(":")
            if key == "Function Name":
                name = val.strip()
                usage[name] = {}
            elif name is not None:
                usage[name][key.strip()] = val.strip()
            continue
        other.append(line)
    return "\n".join(other), usage


def _compile(src: str):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err, usage = _resource_usage("\n".join(l for l in p.stderr.splitlines() if noise not in l))
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    # A kernel with private (scratch) memory gets a scratch allocation at every launch,
    # which costs microseconds on kernels that take ten: none may have any.
    bad = {k: u for k, u in usage.items()
           if u.get("ScratchSize [bytes/lane]", "0") != "0" or u.get("VGPRs Spill", "0") != "0"}
    if bad:
        raise RuntimeError(f"kernels in {src} use scratch memory: " +
                           "; ".join(f"{k} ({u.get('ScratchSize [bytes/lane]')} B/lane, "
                                     f"{u.get('VGPRs Spill')} VGPRs spilled)" for k, u in bad.items()))
    return obj, usage


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        results = list(ex.map(_compile, srcs))
    objs = [o for o, _ in results]
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        for _, usage in results:
            for k, u in usage.items():
                f.write(k + " " + " ".join(f"{a}={b}" for a, b in u.items()) + "\n")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build()
