"""Build libqsa.so (the HIP library) in-tree with hipcc for gfx950.

``build(sanitize=True)`` builds a second copy, ``_build_san/libqsa.so``, whose
host code (argument checks, workspace carving, the slot pool, the launch
sequence) is instrumented with AddressSanitizer and UndefinedBehaviorSanitizer;
the device code is the same. The CPU tests run against it with clang's ASan
runtime preloaded (tests/test_sanitized.py); it is never shipped or timed.
"""
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
SAN_DIR = os.path.join(HERE, "_build_san")
SAN_OUT = os.path.join(SAN_DIR, "libqsa.so")
# host-only instrumentation: each sanitizer flag applies to the host pass
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
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


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(SAN_DIR if sanitize else OBJ_DIR, src.replace(".hip", ".o"))
    extra = SAN_FLAGS if sanitize else []
    cmd = [HIPCC, *FLAGS, *extra, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, msg))
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(sanitize: bool = False) -> str:
    out = SAN_OUT if sanitize else OUT
    os.makedirs(SAN_DIR if sanitize else OBJ_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
