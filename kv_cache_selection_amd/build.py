"""Build libqsa.so (the HIP library) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libqsa.so")
OBJ_DIR = os.path.join(HERE, "_build")
SOURCES = ["api.hip", "index_score.hip", "select.hip", "gather.hip", "attention.hip", "append.hip", "hotcache.hip", "slots.hip", "multiscore.hip"]

HIPCC = os.environ.get("HIPCC", "hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-result",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# per-file additions: the multi-query scorer's epilogue reads every MFMA
# result with VALU instructions, so its MFMAs write VGPRs, not AGPRs
FILE_FLAGS = {"multiscore.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, msg))
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build() -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
