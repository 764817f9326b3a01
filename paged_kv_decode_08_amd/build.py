"""Builds libpdecode.so for gfx950 with hipcc, in-tree (next to this file)."""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpdecode.so")
# the same library with the call-timeline marks compiled in (bench.py --timeline)
LIB_TIMELINE = os.path.join(HERE, "libpdecode_timeline.so")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["decode_mfma.hip", "decode_fused.hip", "decode_multi.hip", "decode_rope_ilv.hip",
           "decode_e5m2.hip",
           "decode_valu.hip", "merge.hip", "append.hip", "ceiling.hip", "noalloc.hip", "api.cpp"]
# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in the generated code.
# atomic optimizer off: the job-queue ticket is fetched by one lane and consumed a whole job later;
# the wave-aggregated form would wait for its result at once.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def _compile(src: str, verbose: bool, extra=(), build_dir=BUILD) -> str:
    obj = os.path.join(build_dir, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + FLAGS + list(extra) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False, extra=(), out=LIB, build_dir=BUILD) -> str:
    """Compiles every source and links `out`; `extra` adds hipcc flags (e.g. -D tuning macros)."""
    os.makedirs(build_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, extra, build_dir), SOURCES))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    if "--timeline" in sys.argv[1:]:
        print(build(verbose=True, extra=["-DPDECODE_TIMELINE"], out=LIB_TIMELINE,
                    build_dir=os.path.join(BUILD, "timeline")))
    else:
        print(build(verbose=True))
