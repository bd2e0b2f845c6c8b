"""The device build switches off packed fp32 instructions (v_pk_fma_f32, v_pk_mul_f32,
v_pk_add_f32): a float2 multiply-add compiles to one packed instruction without the build's
device flags and to two scalar ones with them, and the engine's own gfx950 code object holds
none. CPU only (hipcc cross-compiles; the engine object is the in-tree build's)."""
import os
import shutil
import subprocess

import pytest

from persistent_tile_scheduled_amd import build as BLD

LLVM = "/opt/rocm/llvm/bin"
KERNEL = r"""
#include <hip/hip_runtime.h>
__global__ void k(float2* a, const float2* b, const float2* c, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) { float2 x = a[i], y = b[i], z = c[i]; x.x = fmaf(x.x, y.x, z.x); x.y = fmaf(x.y, y.y, z.y); a[i] = x; }
}
"""
PACKED = ("v_pk_fma_f32", "v_pk_mul_f32", "v_pk_add_f32")


def _asm(tmp_path, flags):
    src = tmp_path / "k.hip"
    src.write_text(KERNEL)
    out = tmp_path / ("k_%d.s" % len(flags))
    subprocess.run([BLD.HIPCC, "-O3", "--cuda-device-only", "-S", "-o", str(out)] + flags + [str(src)],
                   check=True, capture_output=True)
    return out.read_text()


@pytest.mark.skipif(not os.path.exists(BLD.HIPCC), reason="hipcc is not installed")
def test_device_flags_switch_off_packed_fp32(tmp_path):
    plain = _asm(tmp_path, ["--offload-arch=gfx950"])
    built = _asm(tmp_path, BLD.DEVICE)
    assert "v_pk_fma_f32" in plain  # the probe does produce a packed FMA by default
    assert not any(op in built for op in PACKED)
    assert built.count("v_fma_f32") + built.count("v_fmac_f32") >= 2


def test_engine_code_object_has_no_packed_fp32(tmp_path):
    obj = os.path.join(BLD.HERE, "_build", "engine.hip.o")
    tools = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump")]
    if not os.path.exists(obj) or not all(os.path.exists(t) for t in tools):
        pytest.skip("no in-tree engine object or LLVM tools")
    fat, co = tmp_path / "fat.bin", tmp_path / "engine.co"
    subprocess.run([tools[0], "--dump-section=.hip_fatbin=" + str(fat), obj], check=True, capture_output=True)
    subprocess.run([tools[1], "--type=o", "--input=" + str(fat), "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                    "--output=" + str(co), "--unbundle"], check=True, capture_output=True)
    asm = subprocess.run([tools[2], "-d", "--no-show-raw-insn", str(co)], check=True, capture_output=True,
                         text=True).stdout
    assert "v_mfma" in asm and "global_load_lds_dwordx4" in asm  # it is the engine's code
    assert not any(op in asm for op in PACKED)
