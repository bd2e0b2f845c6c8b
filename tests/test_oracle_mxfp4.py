"""Pins of the oracle's MXFP4 expert weights (CPU only).

The pages name FP4 for the MoE experts without fixing a format; the oracle takes the OCP
Microscaling (MX) FP4 type: E2M1 elements, blocks of 32 sharing one E8M0 power-of-two scale.
Each function is held to something other than itself: the E2M1 value table as the MX format
lists it, exact powers of two for E8M0, element-by-element brute force for the packing, and
the already pinned bf16 MoE path on the same (exactly representable) values.
"""
import math

import numpy as np
import pytest

import oracle as O
import workloads
from oracle import decode_oracle as D

# E2M1 magnitudes for codes 0..7 (the MX format's FP4 table); codes 8..15 are their negatives
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_all_sixteen_codes():
    got = O.decode_e2m1(np.arange(16))
    want = E2M1_TABLE + [-v for v in E2M1_TABLE]
    assert list(got) == want
    assert math.copysign(1.0, got[8]) == -1.0  # code 8 is -0
    assert list(O.decode_e2m1(np.arange(16) + 0x30)) == want  # only the low nibble counts


def test_e8m0_powers_of_two():
    got = O.decode_e8m0(np.array([0, 1, 126, 127, 128, 200, 254, 255]))
    assert list(got[:7]) == [2.0 ** -127, 2.0 ** -126, 0.5, 1.0, 2.0, 2.0 ** 73, 2.0 ** 127]
    assert np.isnan(got[7])


def _brute_row(packed, scales):
    """Element k of one row, one at a time: nibble k % 2 of byte k // 2, times the scale of
    block k // 32."""
    k_total = 2 * len(packed)
    out = []
    for k in range(k_total):
        byte = int(packed[k // 2])
        nib = (byte >> 4) if k % 2 else (byte & 0xF)
        mag = E2M1_TABLE[nib & 7]
        out.append((-mag if nib & 8 else mag) * 2.0 ** (int(scales[k // 32]) - 127))
    return out


def test_dequant_nibble_order_and_block_scales():
    rng = np.random.default_rng(3)
    packed = rng.integers(0, 256, size=(3, 48), dtype=np.uint8)   # K = 96: three blocks
    scales = np.array([[120, 127, 131], [100, 140, 127], [127, 127, 126]], dtype=np.uint8)
    got = O.dequant_mxfp4(packed, scales)
    assert got.shape == (3, 96)
    for r in range(3):
        assert list(got[r]) == _brute_row(packed[r], scales[r])
    # a hand case: byte 0x71 holds element 0 = code 1 (0.5) and element 1 = code 7 (6)
    p = np.zeros((1, 16), dtype=np.uint8)
    p[0, 0] = 0x71
    s = np.array([[128]], dtype=np.uint8)
    row = O.dequant_mxfp4(p, s)[0]
    assert row[0] == 1.0 and row[1] == 12.0 and not row[2:].any()


def test_planted_nibble_swap_is_caught(monkeypatch):
    def swapped(packed, scales):
        p = np.asarray(packed).astype(np.int64)
        codes = np.stack([p >> 4, p & 0xF], axis=-1).reshape(p.shape[:-1] + (2 * p.shape[-1],))
        return O.decode_e2m1(codes) * np.repeat(O.decode_e8m0(scales), 32, axis=-1)
    monkeypatch.setattr(D, "dequant_mxfp4", swapped)
    rng = np.random.default_rng(4)
    packed = rng.integers(0, 256, size=(1, 16), dtype=np.uint8)
    scales = np.array([[127]], dtype=np.uint8)
    assert list(D.dequant_mxfp4(packed, scales)[0]) != _brute_row(packed[0], scales[0])


def test_quantiser_stays_within_half_a_step():
    """The input generator's MXFP4 codes decode (by the oracle) to within half an E2M1 step of
    the fp32 values they were made from, values scaled past 6 saturate at 6 (the MX scale
    2^(floor(log2 amax) - 2) puts a block's largest value in [4, 8)), and every block's
    largest code is 4 or 6: the scale choice and the rounding of the generator."""
    import torch
    g = torch.Generator().manual_seed(0)
    w = torch.randn(64, 256, generator=g) * 0.02
    q, s = workloads._quantize_mxfp4(torch, w)
    d = O.dequant_mxfp4(q.numpy(), s.numpy())
    w64 = w.double().numpy()
    sc = np.repeat(O.decode_e8m0(s.numpy()), 32, axis=1)
    v = np.abs(w64) / sc
    step = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0)) * sc
    inside = v <= 6
    assert np.all(np.abs(d - w64)[inside] <= step[inside] / 2 + 1e-12)
    assert np.all(np.abs(d)[~inside] == 6 * sc[~inside])
    nz = d != 0
    assert np.all(np.sign(d[nz]) == np.sign(w64[nz]))
    top = (np.abs(d) / sc).reshape(64, 8, 32).max(axis=2)
    assert np.all((top >= 4) & (top <= 6))


def _as_bf16_weights(cfg_mx, w_mx):
    """The same model with every MXFP4 expert matrix replaced by its decoded values as bf16
    bits (exact: an E2M1 value times a power of two has at most two significant bits)."""
    import torch
    out = {}
    for name, t in w_mx.items():
        if name.endswith(".scale"):
            continue
        if name + ".scale" in w_mx:
            v = O.dequant_mxfp4(t.numpy(), w_mx[name + ".scale"].numpy())
            b = torch.from_numpy(v).to(torch.float32).to(torch.bfloat16)
            assert np.array_equal(b.to(torch.float64).numpy(), v)
            out[name] = b
        else:
            out[name] = t
    return out


@pytest.mark.parametrize("name", ["moe_tiny_mxfp4", "moe_max_route_mxfp4"])
def test_mxfp4_moe_equals_the_bf16_path_on_the_same_values(name):
    cfg = workloads.get_config(name)
    cfg_b = dict(cfg)
    cfg_b.pop("weights")
    w, x, kv = workloads.generate(cfg, seed=5)
    wb = _as_bf16_weights(cfg, w)
    W = O.dict_weights({k: (workloads.bf16_bits(v) if v.dtype == __import__("torch").bfloat16 else v.numpy())
                        for k, v in w.items()})
    Wb = O.dict_weights({k: (workloads.bf16_bits(v) if v.dtype == __import__("torch").bfloat16 else v.numpy())
                         for k, v in wb.items()})
    kvb = workloads.bf16_bits(kv)
    a = O.forward(cfg, W, workloads.bf16_bits(x), kvb)
    b = O.forward(cfg_b, Wb, workloads.bf16_bits(x), kvb)
    assert np.array_equal(a["out"], b["out"])
    for ta, tb in zip(a["layers"], b["layers"]):
        assert np.array_equal(ta["topk"], tb["topk"])
        assert np.array_equal(ta["expert_act"], tb["expert_act"])


def test_planted_scale_bias_is_caught(monkeypatch):
    """An E8M0 decode with the wrong bias (128) changes the MoE output."""
    cfg = workloads.get_config("moe_tiny_mxfp4")
    w, x, kv = workloads.generate(cfg, seed=6)
    W = O.dict_weights({k: (workloads.bf16_bits(v) if v.dtype == __import__("torch").bfloat16 else v.numpy())
                        for k, v in w.items()})
    kvb = workloads.bf16_bits(kv)
    good = O.forward(cfg, W, workloads.bf16_bits(x), kvb)["out"]
    monkeypatch.setattr(D, "decode_e8m0", lambda b: np.ldexp(1.0, np.asarray(b).astype(np.int64) - 128))
    bad = O.forward(cfg, W, workloads.bf16_bits(x), kvb)["out"]
    assert np.linalg.norm(bad - good) > 1e-3 * np.linalg.norm(good)
