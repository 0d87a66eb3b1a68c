"""Builds libdsa.so (the HIP library) for gfx950 with hipcc, in-tree.

    python -m dynamic_sparse_attention_paged_amd.build
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdsa.so")
# diagnostic variant: the attention kernel records per-wave clocks (wave_clocks.py)
LIB_CLOCKS = os.path.join(HERE, "libdsa_clocks.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed FP32 instructions are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-Wall",
          "-I", os.path.join(ROOT, "include")]

SOURCES = ["support.hip", "index_score.hip", "index_score_mfma.hip", "index_topk_fused.hip", "index_topk_fp8.hip", "topk.hip", "attn.hip", "prefill_inv.hip", "moe.hip", "check.hip", "write.hip", "dsa_api.cpp"]


def _compile(src, obj, extra=()):
    cmd = [HIPCC] + COMMON + DEVICE_FLAGS + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC] + COMMON + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for s in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(s)[0] + ".o")
        objs.append(obj)
        procs.append((s, _compile(s, obj)))
    clk_obj = os.path.join(BUILD, "attn_clocks.o")
    procs.append(("attn.hip (wave clocks)", _compile("attn.hip", clk_obj, ["-DDSA_WAVE_CLOCKS"])))
    failed = False
    for s, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature; that warning is expected
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if p.returncode != 0:
            failed = True
            sys.stderr.write(f"--- {s} failed ---\n" + "\n".join(lines) + "\n")
        elif verbose and lines:
            sys.stderr.write(f"--- {s} ---\n" + "\n".join(lines) + "\n")
    if failed:
        raise RuntimeError("HIP compilation failed")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    tmp = LIB_CLOCKS + ".tmp"
    clk_objs = [clk_obj if os.path.basename(o) == "attn.o" else o for o in objs]
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + clk_objs
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_CLOCKS)
    return LIB


def build_synth():
    """The device filler of the synthetic-input generator (dsa_synth/)."""
    src = os.path.join(ROOT, "dsa_synth", "fill.hip")
    out = os.path.join(ROOT, "dsa_synth", "libdsa_synth.so")
    tmp = out + ".tmp"
    cmd = [HIPCC, "-O3", "-fPIC", "-shared", f"--offload-arch={ARCH}"] + DEVICE_FLAGS + [
        src, "-o", tmp]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if p.returncode != 0:
        sys.stderr.write(p.stdout.decode(errors="replace"))
        raise RuntimeError("dsa_synth build failed")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_synth())
