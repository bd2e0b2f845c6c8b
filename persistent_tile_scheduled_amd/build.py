"""Build libdec.so (the persistent decode engine + planner + C ABI) for gfx950, in-tree.

    python -m persistent_tile_scheduled_amd.build

Every source is compiled with hipcc for gfx950 only. Packed fp32 instructions (v_pk_fma_f32,
v_pk_mul_f32, v_pk_add_f32) are switched off for the device code with
`-Xclang -target-feature -Xclang -packed-fp32-ops`. hipcc passes that flag to both of its
compilation passes: the gfx950 device pass honours it (a float2 multiply-add compiles to one
v_pk_fma_f32 without it and to two v_fma_f32 with it), while the x86 host pass, which has no
such feature, prints "'-packed-fp32-ops' is not a recognized feature for this target
(ignoring feature)" and ignores it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdec.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function"]
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def _run(cmd):
    print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = True, out: str = LIB, defines=()) -> str:
    bdir = os.path.join(HERE, "_build" + ("_" + "_".join(d.replace("=", "") for d in defines) if defines else ""))
    os.makedirs(bdir, exist_ok=True)
    objs = []
    for src, dev in [("engine.hip", True), ("planner.cpp", False), ("api.cpp", False)]:
        obj = os.path.join(bdir, src + ".o")
        cmd = [HIPCC] + COMMON + ["-D" + d for d in defines]
        cmd += (DEVICE + ["-x", "hip"]) if dev else ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"]
        cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
        _run(cmd)
        objs.append(obj)
    tmp = out + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950"] + objs + ["-o", tmp])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build()
    sys.exit(0)
