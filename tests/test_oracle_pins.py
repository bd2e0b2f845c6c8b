"""Pins of the fp64 oracle against things other than itself.

The pages print no worked example, closed form or error bound for any step (see the
module docstring of oracle/decode_oracle.py), so every pin here comes from mathematics
(closed forms, invariants, special cases), brute force on tiny inputs, or an independent
library routine (torch CPU fp64, scipy). Each `check_*` takes the oracle module as an
argument; test_planted_mistakes re-runs them against deliberately broken copies of
oracle functions to show a plausible mistake fails at least one pin.
"""
import math
import os
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from oracle import decode_oracle as OD
import workloads

RNG = np.random.default_rng(1234)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits_of(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------------------------------
# bf16 conversions
# ----------------------------------------------------------------------------------------

def test_widen_bf16_golden_table():
    """Hand-derived bit patterns (bfloat16 = top 16 bits of an IEEE binary32)."""
    rows = []
    with open(os.path.join(GOLDEN, "bf16_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                b, v = line.split()
                rows.append((int(b, 16), float(v)))
    bits = np.array([r[0] for r in rows], dtype=np.uint16)
    want = np.array([r[1] for r in rows])
    assert np.array_equal(O.widen_bf16(bits), want)
    # and the rounding direction is the inverse on these exactly representable values
    _, back = O.round_to_bf16(want)
    assert np.array_equal(back, bits)


def test_round_to_bf16_ties_to_even_golden():
    """Halfway cases: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> even (1.0);
    1 + 3*2^-8 lies halfway between 1+2^-7 and 1+2^-6 -> even (1 + 2^-6)."""
    v, b = O.round_to_bf16(np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 1 + 2**-8 + 2**-20]))
    assert v[0] == 1.0 and b[0] == 0x3F80
    assert v[1] == 1 + 2**-6 and b[1] == 0x3F82
    assert v[2] == -1.0 and b[2] == 0xBF80
    assert v[3] == 1 + 2**-7 and b[3] == 0x3F81


def test_round_to_bf16_matches_torch():
    """torch's fp32 -> bf16 conversion (round to nearest even) on fp32-exact inputs."""
    x32 = (RNG.standard_normal(20000) * np.exp(RNG.uniform(-8, 8, 20000))).astype(np.float32)
    v, b = O.round_to_bf16(x32.astype(np.float64))
    tb = _bits_of(torch.from_numpy(x32).to(torch.bfloat16))
    assert np.array_equal(b, tb)
    assert np.array_equal(v, O.widen_bf16(tb))


# ----------------------------------------------------------------------------------------
# GEMV
# ----------------------------------------------------------------------------------------

def check_gemv(o):
    Wm = RNG.standard_normal((7, 13))
    x = RNG.standard_normal(13)
    y = o.linear(Wm, x)
    brute = [sum(Wm[i][j] * x[j] for j in range(13)) for i in range(7)]
    assert np.allclose(y, brute, rtol=1e-13, atol=1e-13)
    # identity
    assert np.array_equal(o.linear(np.eye(9), x[:9]), x[:9])
    # integer-exact: small integers are exact in any order of summation
    Wi = RNG.integers(-2, 3, (5, 600)).astype(np.float64)
    xi = RNG.integers(-3, 4, 600).astype(np.float64)
    yi = o.linear(Wi, xi)
    assert np.array_equal(yi, (Wi.astype(np.int64) @ xi.astype(np.int64)).astype(np.float64))


def test_gemv():
    check_gemv(O)


def test_linear_bits_blocks_and_transposition():
    """A bf16 matrix applied through linear_bits equals the dense product, also across
    its row blocks, and is not transposed (a non-square shape fixes the orientation)."""
    Wm = torch.randn(37, 11, dtype=torch.float32).to(torch.bfloat16)
    bits = _bits_of(Wm)
    x = RNG.standard_normal(11)
    W = O.dict_weights({"m": bits})
    want = Wm.double().numpy() @ x
    assert np.allclose(O.linear_bits(W, "m", x), want, rtol=1e-13, atol=1e-13)
    assert np.allclose(O.linear_bits(W, "m", x, rows_per_block=5), want, rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------------------------------
# FP8 E4M3 weights
# ----------------------------------------------------------------------------------------

def check_decode_e4m3(o):
    codes = np.arange(256, dtype=np.uint8)
    d = o.decode_e4m3(codes)
    # the format's fixed points: 1.0, the largest finite value, the smallest subnormal and
    # normal, the largest subnormal, signed zero, the two NaN codes
    assert d[0x38] == 1.0 and d[0xB8] == -1.0
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0
    assert d[0x01] == 2.0 ** -9 and d[0x08] == 2.0 ** -6 and d[0x07] == 7 * 2.0 ** -9
    assert d[0x00] == 0.0 and d[0x80] == 0.0 and math.copysign(1.0, d[0x80]) == -1.0
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF]) and np.sum(np.isnan(d)) == 2
    # codes 0x00..0x7E are increasing; every finite value is a multiple of 2^-9
    assert np.all(np.diff(d[:0x7F]) > 0)
    fin = d[~np.isnan(d)]
    assert np.all(fin * 512 == np.round(fin * 512))
    # a library routine: torch's float8_e4m3fn dtype, all 256 codes
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ref), np.isnan(d))
    assert np.array_equal(ref[~np.isnan(ref)], d[~np.isnan(d)])


def test_decode_e4m3():
    check_decode_e4m3(O)


def check_linear_fp8(o):
    """uint8 weights are E4M3 bytes scaled per ROW: brute-force loop, and exact small-integer
    arithmetic (a per-column scale or a transposed matrix fails both)."""
    codes = RNG.integers(0, 0x7F, size=(5, 7)).astype(np.uint8) | (RNG.integers(0, 2, size=(5, 7)) << 7).astype(np.uint8)
    scale = np.array([0.5, 2.0, 3.0, 0.25, 1.5], dtype=np.float32)
    x = RNG.standard_normal(7)
    W = o.dict_weights({"m": codes, "m.scale": scale})
    y = o.linear_bits(W, "m", x)
    for r in range(5):
        acc = 0.0
        for c in range(7):
            acc += float(scale[r]) * float(o.decode_e4m3(codes[r, c])) * x[c]
        assert abs(y[r] - acc) <= 1e-12 * max(1.0, abs(acc))
    # codes of small integers (0x40 = 2, 0x48 = 4, 0x44 = 3, 0xC0 = -2) with integer x: exact
    ci = np.array([[0x40, 0x48], [0x44, 0xC0], [0x38, 0x00]], dtype=np.uint8)
    Wi = o.dict_weights({"m": ci, "m.scale": np.array([1.0, 2.0, 4.0], dtype=np.float32)})
    assert np.array_equal(o.linear_bits(Wi, "m", np.array([3.0, 5.0])), np.array([26.0, -2.0, 12.0]))
    # row blocks give the same result
    assert np.allclose(o.linear_bits(W, "m", x, rows_per_block=2), y, rtol=1e-13, atol=0)


def test_linear_fp8():
    check_linear_fp8(O)


def test_fp8_forward_equals_bf16_forward_on_the_same_values():
    """A tiny GQA model whose FP8 rows times power-of-two scales are exactly bf16 values:
    the oracle's FP8 forward equals its (independently pinned) bf16 forward on those values,
    layer trace and logits, exactly."""
    cfg = workloads.get_config("tiny_fp8")
    w, x, kv = workloads.generate(cfg, seed=3)
    f8, b16 = {}, {}
    rng = np.random.default_rng(5)
    for s in workloads.weight_specs(cfg):
        if s.name.endswith(".scale"):
            continue
        t = w[s.name]
        if s.dtype == "fp8":
            codes = t.numpy()
            sc = np.ldexp(1.0, rng.integers(-9, -4, size=codes.shape[0])).astype(np.float32)
            f8[s.name], f8[s.name + ".scale"] = codes, sc
            vals = O.decode_e4m3(codes) * sc[:, None]
            b16[s.name] = _bits_of(torch.from_numpy(vals).to(torch.bfloat16))
            assert np.array_equal(O.widen_bf16(b16[s.name]), vals)  # exactly representable
        else:
            f8[s.name] = b16[s.name] = workloads.bf16_bits(t) if t.dtype == torch.bfloat16 else t.numpy()
    xb, kvb = workloads.bf16_bits(x), workloads.bf16_bits(kv)
    a = O.forward(cfg, O.dict_weights(f8), xb, kvb)
    b = O.forward(cfg, O.dict_weights(b16), xb, kvb)
    assert np.array_equal(a["out"], b["out"])
    for ta, tb in zip(a["layers"], b["layers"]):
        for k in ta:
            assert np.array_equal(np.asarray(ta[k]), np.asarray(tb[k])), k


# ----------------------------------------------------------------------------------------
# RMSNorm
# ----------------------------------------------------------------------------------------

def check_rmsnorm(o):
    c, eps = 0.37, 1e-5
    g = RNG.standard_normal(64)
    y = o.rmsnorm(np.full(64, c), g, eps)
    assert np.allclose(y, g * c / math.sqrt(c * c + eps), rtol=1e-14)
    u = RNG.standard_normal(300)
    # scale invariance (exact as eps -> 0)
    assert np.allclose(o.rmsnorm(5.0 * u, np.ones(300), 0.0), o.rmsnorm(u, np.ones(300), 0.0), rtol=1e-13)
    # library routine
    g2 = RNG.standard_normal(300)
    ref = F.rms_norm(torch.from_numpy(u), (300,), weight=torch.from_numpy(g2), eps=1e-5).numpy()
    assert np.allclose(o.rmsnorm(u, g2, 1e-5), ref, rtol=1e-12, atol=1e-14)
    # eps sits inside the sqrt: an all-zero-but-tiny vector is scaled by 1/sqrt(eps)
    t = np.full(8, 1e-6)
    assert np.allclose(o.rmsnorm(t, np.ones(8), 1e-2), t / math.sqrt(1e-12 + 1e-2), rtol=1e-12)


def test_rmsnorm():
    check_rmsnorm(O)


# ----------------------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------------------

def check_rope(o):
    d, theta = 64, 10000.0
    u = RNG.standard_normal(d)
    assert np.allclose(o.rope(u, 0, theta), u, rtol=0, atol=0)
    y = o.rope(u, 1234, theta)
    h = d // 2
    # norm of every (i, i+d/2) pair is preserved
    assert np.allclose(u[:h] ** 2 + u[h:] ** 2, y[:h] ** 2 + y[h:] ** 2, rtol=1e-12)
    # relative position: <R_p q, R_s k> = <R_{p-s} q, k>
    q, k = RNG.standard_normal(d), RNG.standard_normal(d)
    for p_, s_ in [(7, 3), (4096, 17), (100, 100)]:
        assert np.isclose(o.rope(q, p_, theta) @ o.rope(k, s_, theta), o.rope(q, p_ - s_, theta) @ k,
                          rtol=1e-10, atol=1e-10)
    # complex-number formulation: z_i = u_i + i u_{i+d/2} is multiplied by e^{i p theta_i}
    p_ = 513
    z = (u[:h] + 1j * u[h:]) * np.exp(1j * p_ * theta ** (-np.arange(h) * 2.0 / d))
    y = o.rope(u, p_, theta)
    assert np.allclose(y[:h], z.real, rtol=1e-12, atol=1e-12)
    assert np.allclose(y[h:], z.imag, rtol=1e-12, atol=1e-12)
    # 2-d case is a plain rotation by p radians (theta_0 = 1)
    assert np.allclose(o.rope(np.array([1.0, 0.0]), math.pi / 2, theta), [0.0, 1.0], atol=1e-15)


def test_rope():
    check_rope(O)


# ----------------------------------------------------------------------------------------
# softmax / attention / split-K
# ----------------------------------------------------------------------------------------

def check_softmax(o):
    import scipy.special
    s = RNG.standard_normal((5, 33)) * 4
    p = o.softmax(s)
    assert np.allclose(p.sum(-1), 1.0, rtol=1e-14)
    assert np.allclose(o.softmax(s + 123.0), p, rtol=1e-12)
    assert np.allclose(p, scipy.special.softmax(s, axis=-1), rtol=1e-12)


def test_softmax():
    check_softmax(O)


def check_attention(o):
    d, dv, n = 16, 12, 50
    q = RNG.standard_normal(d)
    K = RNG.standard_normal((n, d))
    V = RNG.standard_normal((n, dv))
    sc = 1 / math.sqrt(d)
    # one key returns its value
    assert np.allclose(o.attend(q, K[:1], V[:1], sc), V[0], rtol=1e-14)
    # all-equal keys give the mean of V
    assert np.allclose(o.attend(q, np.tile(K[:1], (n, 1)), V, sc), V.mean(0), rtol=1e-12)
    # one dominant score selects that row
    K2 = K.copy()
    K2[17] = 1e4 * q
    assert np.allclose(o.attend(q, K2, V, sc), V[17], rtol=1e-12)
    # library routine: torch SDPA in fp64 (default scale 1/sqrt(d))
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[None, None, None, :],
                                         torch.from_numpy(K)[None, None], torch.from_numpy(V)[None, None])
    assert np.allclose(o.attend(q, K, V, sc), ref[0, 0, 0].numpy(), rtol=1e-12, atol=1e-14)


def test_attention():
    check_attention(O)


def check_split(o):
    d, n = 32, 257
    q = RNG.standard_normal(d)
    K = RNG.standard_normal((n, d)) * 2
    V = RNG.standard_normal((n, d))
    sc = 1 / math.sqrt(d)
    full = o.attend(q, K, V, sc)
    for trial in range(20):
        cuts = sorted(set(RNG.integers(1, n, RNG.integers(0, 12)).tolist()))
        bounds = [0] + cuts + [n]
        assert np.allclose(o.attend_split(q, K, V, sc, bounds), full, rtol=1e-12, atol=1e-14)
    # length-1 chunks everywhere, and a ragged tail
    assert np.allclose(o.attend_split(q, K, V, sc, list(range(n + 1))), full, rtol=1e-12)
    assert np.allclose(o.attend_split(q, K, V, sc, [0, 256, 257]), full, rtol=1e-12)
    # merge order does not matter
    parts = [o.attend_partial(q, K[a:b], V[a:b], sc) for a, b in [(0, 100), (100, 101), (101, 257)]]
    assert np.allclose(o.merge_partials(parts[::-1]), full, rtol=1e-12)


def test_split_k():
    check_split(O)


def check_silu(o):
    assert o.silu(np.array([0.0]))[0] == 0.0
    assert np.isclose(o.silu(np.array([40.0]))[0], 40.0, rtol=1e-15)
    assert abs(o.silu(np.array([-40.0]))[0]) < 1e-15
    z = RNG.standard_normal(1000) * 5
    assert np.allclose(o.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-13, atol=1e-15)
    # silu(z) - silu(-z) = z (closed form of z*sigmoid(z))
    assert np.allclose(o.silu(z) - o.silu(-z), z, rtol=1e-12, atol=1e-12)


def test_silu():
    check_silu(O)


# ----------------------------------------------------------------------------------------
# router
# ----------------------------------------------------------------------------------------

def check_route(o):
    n = 32
    r = RNG.standard_normal(n)
    b = np.zeros(n)
    b[:8] = 10.0
    rt = o.route(r, b, 8)
    assert sorted(rt["topk"].tolist()) == list(range(8))
    assert np.isclose(rt["w"].sum(), 1.0, rtol=1e-15)
    sig = 1 / (1 + np.exp(-r))
    assert np.allclose(rt["w"], sig[rt["topk"]] / sig[rt["topk"]].sum(), rtol=1e-14)
    # listed by decreasing z
    z = sig + b
    assert np.all(np.diff(z[rt["topk"]]) <= 0)
    # ties go to the lower index: all-equal logits pick 0..k-1 in order
    rt = o.route(np.zeros(n), np.zeros(n), 5)
    assert rt["topk"].tolist() == [0, 1, 2, 3, 4]
    # exact tie between experts 20 and 3 at the boundary: the lower index wins
    r2 = np.full(n, -5.0)
    r2[[7, 9]] = 3.0
    r2[[20, 3]] = 1.0
    rt = o.route(r2, np.zeros(n), 3)
    assert rt["topk"].tolist() == [7, 9, 3]
    # top_k = n: dense mixture with weights sigma / sum sigma
    rt = o.route(r, np.zeros(n), n)
    assert sorted(rt["topk"].tolist()) == list(range(n))
    assert np.allclose(np.sort(rt["w"]), np.sort(sig / sig.sum()), rtol=1e-14)
    # the bias only selects: it never enters the weights
    rt1 = o.route(r, np.zeros(n), 4)
    rt2 = o.route(r, np.full(n, 0.3), 4)
    assert rt1["topk"].tolist() == rt2["topk"].tolist()
    assert np.allclose(rt1["w"], rt2["w"], rtol=1e-15)


def test_route():
    check_route(O)


# ----------------------------------------------------------------------------------------
# MLA
# ----------------------------------------------------------------------------------------

def _tiny_mla_weights(seed=0):
    cfg = workloads.get_config("mla_tiny")
    w, x, kv = workloads.generate(cfg, seed=seed, device="cpu")
    Wd = {k: (_bits_of(v) if v.dtype == torch.bfloat16 else v.numpy()) for k, v in w.items()}
    return cfg, O.dict_weights(Wd), _bits_of(x), _bits_of(kv)


def check_mla(o):
    cfg, W, xb, kvb = _tiny_mla_weights()
    xn = o.rmsnorm(o.widen_bf16(xb), o.widen_bf16(W("layers.0.attn_norm")), cfg["rms_eps"])
    n = cfg["kv_len"]
    out, t = o.mla_attention(cfg, W, 0, xn, kvb[0], n)
    kl = cfg["kv_lora_rank"]
    # absorbed form == naive definition
    lat = np.concatenate([o.widen_bf16(kvb[0][:n]), o.widen_bf16(t["kv_new_bits"])[None, :]], 0)
    ab = o.mla_attention_absorbed(cfg, W, 0, t["q_nope"], t["q_rope"], lat)
    assert np.allclose(ab, out, rtol=1e-11, atol=1e-13)
    # the absorbed core is MQA attention with K = [c || kpe], V = c, scale 1/sqrt(nope+rope)
    nh, dn, dr = cfg["n_q_heads"], cfg["qk_nope"], cfg["qk_rope"]
    qa = t["q_abs"].reshape(nh, kl)
    qq = np.concatenate([qa, t["q_rope"].reshape(nh, dr)], axis=1)
    ref = F.scaled_dot_product_attention(torch.from_numpy(qq)[None, :, None, :],
                                         torch.from_numpy(lat)[None, None].expand(1, nh, -1, -1),
                                         torch.from_numpy(lat[:, :kl])[None, None].expand(1, nh, -1, -1),
                                         scale=1 / math.sqrt(dn + dr))
    assert np.allclose(t["o_lat"].reshape(nh, kl), ref[0, :, 0].numpy(), rtol=1e-11, atol=1e-13)
    # the new cache entry is [RMSNorm(c) || RoPE(k_pe)] rounded to bf16
    a = t["kv_a"]
    c_ref = F.rms_norm(torch.from_numpy(a[:kl]), (kl,), eps=cfg["rms_eps"]).numpy()
    assert np.allclose(t["c_new"], c_ref * o.widen_bf16(W("layers.0.kv_norm")), rtol=1e-12)


def test_mla():
    check_mla(O)


# ----------------------------------------------------------------------------------------
# whole model against an independent torch-fp64 composition
# ----------------------------------------------------------------------------------------

def _torch_gqa_forward(cfg, w, x, kv):
    """Independent composition with torch fp64 library ops (F.rms_norm, SDPA with GQA)."""
    D = torch.float64
    d, nq, nkv, hd = cfg["hidden"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    n, eps, theta = cfg["kv_len"], cfg["rms_eps"], cfg["rope_theta"]
    h_ = x.to(D)
    inv = 1.0 / (theta ** (torch.arange(0, hd, 2, dtype=D) / hd))
    ang = n * inv
    cos, sin = torch.cos(ang), torch.sin(ang)

    def rot(t):  # t [..., hd] rotate-half via complex view of (first half, second half)
        z = torch.complex(t[..., : hd // 2], t[..., hd // 2:]) * torch.complex(cos, sin)
        return torch.cat([z.real, z.imag], dim=-1)

    outs = []
    for l in range(cfg["n_layers"]):
        p = f"layers.{l}."
        xn = F.rms_norm(h_, (d,), weight=w[p + "attn_norm"].to(D), eps=eps)
        q = rot((w[p + "wq"].to(D) @ xn).view(nq, hd))
        k = rot((w[p + "wk"].to(D) @ xn).view(nkv, hd))
        v = (w[p + "wv"].to(D) @ xn).view(nkv, hd)
        K = torch.cat([kv[l, 0, :, :n].to(D), k.to(torch.bfloat16).to(D)[:, None]], dim=1)
        V = torch.cat([kv[l, 1, :, :n].to(D), v.to(torch.bfloat16).to(D)[:, None]], dim=1)
        o = F.scaled_dot_product_attention(q[None, :, None, :], K[None], V[None], enable_gqa=True)
        hh = h_ + w[p + "wo"].to(D) @ o.reshape(-1)
        hn = F.rms_norm(hh, (d,), weight=w[p + "ffn_norm"].to(D), eps=eps)
        f = w[p + "w_down"].to(D) @ (F.silu(w[p + "w_gate"].to(D) @ hn) * (w[p + "w_up"].to(D) @ hn))
        h_ = hh + f
        outs.append(h_)
    logits = w["lm_head"].to(D) @ F.rms_norm(h_, (d,), weight=w["final_norm"].to(D), eps=eps)
    return outs, logits


@pytest.mark.parametrize("name", ["tiny", "tiny_gain", "tiny_kv0", "tiny_mha_ragged"])
def test_whole_gqa_vs_torch(name):
    cfg = workloads.get_config(name)
    w, x, kv = workloads.generate(cfg, seed=3, device="cpu")
    Wd = {k: _bits_of(v) for k, v in w.items()}
    res = O.forward(cfg, O.dict_weights(Wd), _bits_of(x), _bits_of(kv))
    outs, logits = _torch_gqa_forward(cfg, w, x, kv)
    for l, t in enumerate(res["layers"]):
        assert np.allclose(t["x_out"], outs[l].numpy(), rtol=1e-10, atol=1e-10), l
    assert np.allclose(res["out"], logits.numpy(), rtol=1e-10, atol=1e-10)


def _torch_moe_ffn(cfg, w, l, hn):
    """Independent MoE FFN: torch.topk on fp32 scores (ties resolved by an index tiebreak)."""
    D = torch.float64
    p = f"layers.{l}."
    r = w[p + "router"].to(D) @ hn
    sig = torch.sigmoid(r)
    z32 = torch.sigmoid(r.float()) + w[p + "router_bias"].float()
    n = z32.numel()
    # lexicographic (z desc, index asc): sort by index, then a stable sort by -z
    order = torch.sort(-z32, stable=True).indices
    T = order[: cfg["top_k"]]
    wts = sig[T] / sig[T].sum()

    def sw(g, u, dn, x):
        return dn.to(D) @ (F.silu(g.to(D) @ x) * (u.to(D) @ x))

    y = sw(w[p + "shared.w_gate"], w[p + "shared.w_up"], w[p + "shared.w_down"], hn)
    for e, we in zip(T.tolist(), wts):
        y = y + we * sw(w[p + "experts.w_gate"][e], w[p + "experts.w_up"][e], w[p + "experts.w_down"][e], hn)
    return y, T


@pytest.mark.parametrize("name", ["mla_tiny", "moe_tiny"])
def test_whole_mla_moe_vs_torch(name):
    """MLA/MoE layers against a torch composition of the naive MLA definition."""
    cfg = workloads.get_config(name)
    w, x, kv = workloads.generate(cfg, seed=5, device="cpu")
    Wd = {k: (_bits_of(v) if v.dtype == torch.bfloat16 else v.numpy()) for k, v in w.items()}
    res = O.forward(cfg, O.dict_weights(Wd), _bits_of(x), _bits_of(kv))
    D = torch.float64
    d, nh = cfg["hidden"], cfg["n_q_heads"]
    kl, dn, dr, dv = cfg["kv_lora_rank"], cfg["qk_nope"], cfg["qk_rope"], cfg["v_head"]
    n, eps, theta = cfg["kv_len"], cfg["rms_eps"], cfg["rope_theta"]
    inv = 1.0 / (theta ** (torch.arange(0, dr, 2, dtype=D) / dr))
    cos, sin = torch.cos(n * inv), torch.sin(n * inv)

    def rot(t):
        z = torch.complex(t[..., : dr // 2], t[..., dr // 2:]) * torch.complex(cos, sin)
        return torch.cat([z.real, z.imag], dim=-1)

    h_ = x.to(D)
    for l in range(cfg["n_layers"]):
        p = f"layers.{l}."
        xn = F.rms_norm(h_, (d,), weight=w[p + "attn_norm"].to(D), eps=eps)
        cq = F.rms_norm(w[p + "wq_a"].to(D) @ xn, (cfg["q_lora_rank"],), weight=w[p + "q_norm"].to(D), eps=eps)
        qf = (w[p + "wq_b"].to(D) @ cq).view(nh, dn + dr)
        q = torch.cat([qf[:, :dn], rot(qf[:, dn:])], dim=1)
        a = w[p + "wkv_a"].to(D) @ xn
        c_new = F.rms_norm(a[:kl], (kl,), weight=w[p + "kv_norm"].to(D), eps=eps)
        ent = torch.cat([c_new, rot(a[kl:])]).to(torch.bfloat16).to(D)
        lat = torch.cat([kv[l, :n].to(D), ent[None]], dim=0)
        C, KPE = lat[:, :kl], lat[:, kl:]
        Kh = torch.cat([torch.einsum("hdc,nc->hnd", w[p + "w_uk"].to(D), C),
                        KPE[None].expand(nh, -1, -1)], dim=2)
        Vh = torch.einsum("hdc,nc->hnd", w[p + "w_uv"].to(D), C)
        o = F.scaled_dot_product_attention(q[None, :, None, :], Kh[None], Vh[None],
                                           scale=1 / math.sqrt(dn + dr))
        hh = h_ + w[p + "wo"].to(D) @ o.reshape(-1)
        hn = F.rms_norm(hh, (d,), weight=w[p + "ffn_norm"].to(D), eps=eps)
        if cfg["arch"] == "mla":
            f = w[p + "w_down"].to(D) @ (F.silu(w[p + "w_gate"].to(D) @ hn) * (w[p + "w_up"].to(D) @ hn))
        else:
            f, T = _torch_moe_ffn(cfg, w, l, hn)
            assert res["layers"][l]["topk"].tolist() == T.tolist()
        h_ = hh + f
        assert np.allclose(res["layers"][l]["x_out"], h_.numpy(), rtol=1e-10, atol=1e-10), l
    assert np.allclose(res["out"], h_.numpy(), rtol=1e-10, atol=1e-10)


# ----------------------------------------------------------------------------------------
# planted mistakes: each broken variant must fail at least one pin
# ----------------------------------------------------------------------------------------

def _patched(**repl):
    m = types.SimpleNamespace(**{k: getattr(OD, k) for k in dir(OD) if not k.startswith("__")})
    for k, v in repl.items():
        setattr(m, k, v)
    return m


def _rope_sign_flipped(u, pos, theta):
    return OD.rope(u, -pos, theta)


def _rope_interleaved(u, pos, theta):
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    i = np.arange(d // 2)
    ang = pos * theta ** (-2.0 * i / d)
    a, b = u[..., 0::2], u[..., 1::2]
    out = np.empty_like(u)
    out[..., 0::2] = a * np.cos(ang) - b * np.sin(ang)
    out[..., 1::2] = b * np.cos(ang) + a * np.sin(ang)
    return out


def _rmsnorm_no_eps(u, g, eps):
    return OD.rmsnorm(u, g, 0.0)


def _rmsnorm_eps_outside(u, g, eps):
    u = np.asarray(u, dtype=np.float64)
    return u / (math.sqrt(float(np.mean(u * u))) + eps) * g


def _merge_no_rescale(parts):
    num = sum(a for (m, l, a) in parts)
    den = sum(l for (m, l, a) in parts)
    return num / den


def _route_ties_high(r, bias, k):
    rt = OD.route(r, bias, k)
    z32 = rt["z32"]
    order = np.lexsort((-np.arange(len(z32)), -z32))
    rt["topk"] = order[:k]
    return rt


def _route_weights_with_bias(r, bias, k):
    rt = OD.route(r, bias, k)
    z = rt["z"][rt["topk"]]
    rt["w"] = z / z.sum()
    return rt


def _silu_wrong(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(z))


def _linear_drop_last_term(Wm, x):
    return Wm[:, :-1] @ x[:-1]


@pytest.mark.parametrize("check,repl", [
    (check_rope, {"rope": _rope_sign_flipped}),
    (check_rope, {"rope": _rope_interleaved}),
    (check_rmsnorm, {"rmsnorm": _rmsnorm_no_eps}),
    (check_rmsnorm, {"rmsnorm": _rmsnorm_eps_outside}),
    (check_split, {"merge_partials": _merge_no_rescale}),
    (check_route, {"route": _route_ties_high}),
    (check_route, {"route": _route_weights_with_bias}),
    (check_silu, {"silu": _silu_wrong}),
    (check_gemv, {"linear": _linear_drop_last_term}),
])
def test_planted_mistakes(check, repl):
    broken = _patched(**repl)
    with pytest.raises(AssertionError):
        check(broken)


def _whole_gqa_mismatch(patch):
    """Run the oracle on the tiny model with one of its functions replaced and report whether
    the independent torch composition (SDPA's GQA, F.rms_norm) then disagrees with it."""
    cfg = workloads.get_config("tiny")
    w, x, kv = workloads.generate(cfg, seed=3, device="cpu")
    Wd = {k: _bits_of(v) for k, v in w.items()}
    outs, logits = _torch_gqa_forward(cfg, w, x, kv)
    name, fn = patch
    orig = getattr(OD, name)
    try:
        setattr(OD, name, fn(orig))
        res = O.forward(cfg, O.dict_weights(Wd), _bits_of(x), _bits_of(kv))
    finally:
        setattr(OD, name, orig)
    return not np.allclose(res["out"], logits.numpy(), rtol=1e-6)


def test_planted_gqa_head_to_group_map():
    """An interleaved head->group map (h % n_kv instead of contiguous groups, reading R8)
    breaks the whole-model pin: the tiny model has 4 query heads on 2 KV heads."""
    cfg = workloads.get_config("tiny")
    assert cfg["n_q_heads"] > cfg["n_kv_heads"] > 1
    assert _whole_gqa_mismatch(("kv_group", lambda orig: (lambda h, nq, nkv: h % nkv)))
    assert not _whole_gqa_mismatch(("kv_group", lambda orig: orig))  # the unplanted oracle agrees


def test_planted_missing_softmax_scale():
    """A missing 1/sqrt(head_dim) breaks the whole-model pin."""
    assert _whole_gqa_mismatch(("attend", lambda orig: (lambda q, K, V, scale: orig(q, K, V, 1.0))))
