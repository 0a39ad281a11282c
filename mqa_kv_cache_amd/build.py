"""Builds libgqa_attn.so in-tree with hipcc for gfx950 (no JIT, no torch extension)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgqa_attn.so")
SOURCES = ["api.cpp", "rope.hip", "decode.hip", "prefill.hip", "sparse.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, out_path: str = LIB, defines=(), extra_flags=(), link_flags=()) -> str:
    """Compile every HIP source into mqa_kv_cache_amd/libgqa_attn.so (or
    out_path, with extra -D defines or compiler flags for tuning builds);
    return its path."""
    objs = []
    build_dir = os.path.join(os.path.dirname(out_path), "_build")
    os.makedirs(build_dir, exist_ok=True)
    procs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".", "_") + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = ([HIPCC] + [f for f in FLAGS if f != "-shared"] + [f"-D{d}" for d in defines]
               + list(extra_flags) + lang
               + ["-c", os.path.join(CSRC, src), "-o", obj])
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = False
    for src, cmd, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature flag; that warning is harmless
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed = True
            sys.stderr.write(f"[build] {src} failed:\n{text}\n")
        elif verbose and text.strip():
            sys.stderr.write(f"[build] {src}:\n{text}\n")
    if failed:
        raise RuntimeError("hipcc failed")
    tmp = out_path + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + list(link_flags) + ["-o", tmp] + objs
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
