"""Pins of the oracle's FP8 weights in the latent families (CPU only).

With "weights": "fp8" an MLA or MoE model stores every linear matrix except the per-head
absorption matrices and the router as OCP FP8 E4M3 bytes with one fp32 scale per row (per row of
every expert for the stacked expert tensors). The E4M3 decode is pinned on all 256 codes in
test_oracle_pins; here the rest of the path is held to the already pinned bf16 path: with the
row scales set to powers of two, every decoded weight is exactly a bf16 value, so the FP8 model
and the bf16 model built from those values must give bit-identical results.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from oracle import decode_oracle as D


def _pow2_scales(w):
    """Row scales replaced by powers of two 2^-(5 + r % 4), a different one on neighbouring rows
    (so a scale applied along the wrong axis shows)."""
    for name in list(w):
        if name.endswith(".scale") and w[name].dtype == torch.float32:
            r = torch.arange(w[name].numel()).reshape(w[name].shape)
            w[name] = torch.pow(2.0, -(5 + (r % 4)).to(torch.float32))
    return w


def _as_bf16_weights(w):
    """Every FP8 matrix replaced by its decoded values (bytes times row scales) as bf16 bits."""
    out = {}
    for name, t in w.items():
        if name.endswith(".scale"):
            continue
        if t.dtype == torch.uint8 and name + ".scale" in w:
            v = O.decode_e4m3(t.numpy()) * w[name + ".scale"].numpy().astype(np.float64)[..., None]
            b = torch.from_numpy(v).to(torch.float32).to(torch.bfloat16)
            assert np.array_equal(b.to(torch.float64).numpy(), v), name
            out[name] = b
        else:
            out[name] = t
    return out


def _weights(w):
    return O.dict_weights({k: (workloads.bf16_bits(v) if v.dtype == torch.bfloat16 else v.numpy()) for k, v in w.items()})


@pytest.mark.parametrize("name", ["mla_tiny_fp8", "moe_tiny_fp8"])
def test_fp8_latent_model_equals_the_bf16_path_on_the_same_values(name):
    cfg = workloads.get_config(name)
    cfg_b = dict(cfg)
    cfg_b.pop("weights")
    w, x, kv = workloads.generate(cfg, seed=7)
    w = _pow2_scales(w)
    assert w["layers.0.w_uk"].dtype == torch.bfloat16 and w["layers.0.wq_a"].dtype == torch.uint8
    wb = _as_bf16_weights(w)
    kvb = workloads.bf16_bits(kv)
    a = O.forward(cfg, _weights(w), workloads.bf16_bits(x), kvb)
    b = O.forward(cfg_b, _weights(wb), workloads.bf16_bits(x), kvb)
    assert np.array_equal(a["out"], b["out"])
    for ta, tb in zip(a["layers"], b["layers"]):
        for k in ("cq_raw", "kv_a", "q_nope", "attn", "h", "ffn_out"):
            assert np.array_equal(ta[k], tb[k]), k
        if cfg["arch"] == "moe":
            assert np.array_equal(ta["topk"], tb["topk"])
            assert np.array_equal(ta["expert_act"], tb["expert_act"])


def test_planted_expert_scale_axis_is_caught(monkeypatch):
    """Expert rows scaled along the column axis instead of per row change the MoE output."""
    cfg = workloads.get_config("moe_tiny_fp8")
    w, x, kv = workloads.generate(cfg, seed=8)
    W = _weights(w)
    kvb = workloads.bf16_bits(kv)
    good = O.forward(cfg, W, workloads.bf16_bits(x), kvb)["out"]
    real = D._expert_w64

    def wrong(cfg_, W_, name, index=None):
        m = real(cfg_, W_, name, index)
        sc = np.asarray(W_(name + ".scale") if index is None else W_(name + ".scale", index), dtype=np.float64)
        raw = m / sc[..., None]
        return raw * np.resize(sc, raw.shape[-1])[None, :]
    monkeypatch.setattr(D, "_expert_w64", wrong)
    bad = O.forward(cfg, W, workloads.bf16_bits(x), kvb)["out"]
    assert np.linalg.norm(bad - good) > 1e-3 * np.linalg.norm(good)
