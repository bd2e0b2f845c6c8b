"""Pins of the oracle's multi-token verification step (gqa_verify_layer / verify_forward).

The verification step of M tokens is defined as causal block attention (token i at position
kv_len + i sees the cached positions and the block's positions up to its own). Its pin is a
different computation of the same thing: M sequential single-token decode steps of the
oracle (each already pinned against torch SDPA and closed forms), the i-th at length
kv_len + i with the cache holding the earlier tokens' bf16 k, v. Planted mistakes in the
block form (no causal mask, a token missing itself) must break that pin.
"""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import decode_oracle as OD
import workloads


def _bits_of(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _sequential(cfg, Wd, x_bits, kv_bits, M):
    """M decode steps in order, appending each step's bf16 k, v to a copy of the cache."""
    n = cfg["kv_len"]
    kv = kv_bits.copy()
    outs, layers = [], []
    for i in range(M):
        res = O.forward(cfg, O.dict_weights(Wd), x_bits[i], kv, kv_len=n + i)
        for l, t in enumerate(res["layers"]):
            kv[l, 0, :, n + i, :] = t["k_new_bits"].reshape(cfg["n_kv_heads"], -1)
            kv[l, 1, :, n + i, :] = t["v_new_bits"].reshape(cfg["n_kv_heads"], -1)
        outs.append(res["out"])
        layers.append(res["layers"])
    return np.stack(outs), layers


def _case(name, M, seed=3):
    cfg = dict(workloads.get_config(name), verify=M)
    w, x, kv = workloads.generate(cfg, seed=seed, device="cpu")
    assert tuple(x.shape) == (M, cfg["hidden"]) and kv.shape[3] == cfg["kv_len"] + M
    return cfg, {k: _bits_of(v) if v.dtype == torch.bfloat16 else v.numpy() for k, v in w.items()}, _bits_of(x), _bits_of(kv)


@pytest.mark.parametrize("name,M", [("tiny", 4), ("tiny_gain", 3), ("tiny_mha_ragged", 2), ("tiny_kv0", 4)])
def test_verify_equals_sequential_decode_steps(name, M):
    cfg, Wd, xb, kvb = _case(name, M)
    res = O.verify_forward(cfg, O.dict_weights(Wd), xb, kvb)
    outs, layers = _sequential(cfg, Wd, xb, kvb, M)
    assert np.allclose(res["out"], outs, rtol=1e-11, atol=1e-11)
    for l, t in enumerate(res["layers"]):
        for i in range(M):
            for key in ("q", "attn", "h", "ffn_act", "x_out"):
                assert np.allclose(t[key][i], layers[i][l][key], rtol=1e-11, atol=1e-11), (l, i, key)
            assert np.array_equal(t["k_new_bits"][i], layers[i][l]["k_new_bits"])
            assert np.array_equal(t["v_new_bits"][i], layers[i][l]["v_new_bits"])


def test_verify_of_one_token_is_the_decode_step():
    cfg = dict(workloads.get_config("tiny"))
    w, x, kv = workloads.generate(cfg, seed=3, device="cpu")
    Wd = {k: _bits_of(v) if v.dtype == torch.bfloat16 else v.numpy() for k, v in w.items()}
    res = O.verify_forward(cfg, O.dict_weights(Wd), _bits_of(x)[None], _bits_of(kv))
    one = O.forward(cfg, O.dict_weights(Wd), _bits_of(x), _bits_of(kv))
    assert np.array_equal(res["out"][0], one["out"])


@pytest.mark.parametrize("plant,visible", [
    ("no causal mask: every token sees the whole block", lambda n, i, M: n + M),
    ("a token misses itself", lambda n, i, M: n + i),
    ("a token also sees the next one", lambda n, i, M: min(n + i + 2, n + M)),
])
def test_planted_verify_mistakes(plant, visible, monkeypatch):
    """Wrong causal visibility in the block form breaks the sequential pin."""
    cfg, Wd, xb, kvb = _case("tiny", 3)
    monkeypatch.setattr(OD, "verify_visible", visible)
    res = O.verify_forward(cfg, O.dict_weights(Wd), xb, kvb)
    monkeypatch.undo()
    outs, _ = _sequential(cfg, Wd, xb, kvb, 3)
    assert not np.allclose(res["out"], outs, rtol=1e-6), plant
