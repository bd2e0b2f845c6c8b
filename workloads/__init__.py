"""Seeded synthetic inputs for batch-1 decode, shared by the oracle side and the HIP side.

This module holds model shapes, the canonical tensor list (names, shapes, dtypes) and
seeded random generators. It holds none of the decode arithmetic: nothing here
normalises, rotates, multiplies or attends.

The tensor list is the layout contract of the decode library: every matrix is bf16,
row-major [out_features][in_features]; norm gains are bf16 [dim]; the MoE router bias is
fp32 [n_routed]; per-head MLA up-projections are [heads][rows][kv_lora_rank].

Input recipe (the pages run trained DeepSeek/GLM/MiMo checkpoints, which are not
available; these shapes stand in for them):
  * linear weights ~ N(0, weight_std) rounded to bf16 (round-to-nearest-even);
  * norm gains = 1 ("ones") or ~ N(mean, std) for the gain-pinning variants;
  * cached K/V (or latent c||k_pe) ~ N(0, kv_std) on positions [0, kv_len), slot kv_len = 0;
  * x ~ N(0, x_std) in bf16; router bias ~ N(0, router_bias_std) in fp32.
  * configs with "weights": "fp8": every linear matrix (latent families: all but the per-head
    absorption matrices and the router, FP8_KEEP_BF16) is drawn the same way in
    fp32, then each row r is stored as E4M3 bytes of row / scale[r] (round to nearest
    even) with scale[r] = max|row| / 448 in fp32, so the row's largest value maps to the
    largest finite E4M3 magnitude. Quantisation is input generation: the decode path only
    reads bytes and scales.
  * configs with "weights": "mxfp4" (MoE only): every expert matrix (routed and shared) is
    drawn the same way in fp32, then cut into blocks of 32 consecutive columns; a block with
    largest magnitude a gets the power-of-two scale 2^(floor(log2 a) - 2) (E8M0 byte
    floor(log2 a) + 125, so the block's largest value lands in [4, 8) before rounding) and
    each value is stored as the nearest E2M1 value of w / scale (magnitudes 0, 0.5, 1, 1.5,
    2, 3, 4, 6; saturating at 6), two per byte, the even column in the low nibble.
All tensors come from one torch.Generator seeded once, drawn in the canonical order.
"""
from __future__ import annotations

import json
import os
from dataclasses import dataclass
from typing import Dict, List, Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))

BF16 = "bf16"
FP32 = "fp32"
FP8 = "fp8"     # OCP FP8 E4M3 bytes (with a per-row fp32 "<name>.scale" tensor after it)
FP4X2 = "fp4x2"  # MXFP4: E2M1 pairs, uint8 [..., K/2] (with an E8M0 "<name>.scale" [..., K/32] after it)
E8M0 = "e8m0"    # power-of-two block scales, one byte each


def load_configs() -> Dict[str, dict]:
    with open(os.path.join(_HERE, "configs.json")) as f:
        return json.load(f)["configs"]


def get_config(name: str) -> dict:
    cfgs = load_configs()
    if name not in cfgs:
        raise KeyError(f"unknown config {name!r}; known: {sorted(cfgs)}")
    cfg = dict(cfgs[name])
    cfg["name"] = name
    return cfg


@dataclass(frozen=True)
class TensorSpec:
    name: str
    shape: Tuple[int, ...]
    dtype: str          # "bf16" or "fp32"
    init: str           # "weight", "gain", "router_bias"

    @property
    def numel(self) -> int:
        n = 1
        for d in self.shape:
            n *= d
        return n

    @property
    def nbytes(self) -> int:
        return self.numel * {BF16: 2, FP8: 1, FP4X2: 1, E8M0: 1}.get(self.dtype, 4)


def _mla_attn_specs(cfg: dict, p: str) -> List[TensorSpec]:
    d = cfg["hidden"]
    nh = cfg["n_q_heads"]
    ql, kl = cfg["q_lora_rank"], cfg["kv_lora_rank"]
    dn, dr, dv = cfg["qk_nope"], cfg["qk_rope"], cfg["v_head"]
    return [
        TensorSpec(p + "attn_norm", (d,), BF16, "gain"),
        TensorSpec(p + "wq_a", (ql, d), BF16, "weight"),
        TensorSpec(p + "q_norm", (ql,), BF16, "gain"),
        TensorSpec(p + "wq_b", (nh * (dn + dr), ql), BF16, "weight"),
        TensorSpec(p + "wkv_a", (kl + dr, d), BF16, "weight"),
        TensorSpec(p + "kv_norm", (kl,), BF16, "gain"),
        TensorSpec(p + "w_uk", (nh, dn, kl), BF16, "weight"),
        TensorSpec(p + "w_uv", (nh, dv, kl), BF16, "weight"),
        TensorSpec(p + "wo", (d, nh * dv), BF16, "weight"),
    ] + _index_specs(cfg, p)


def _index_specs(cfg: dict, p: str) -> List[TensorSpec]:
    """The sparse indexer's matrices ("index_heads" H > 0): index queries from the normalised
    query latent, one index key and H head weights from the normalised layer input."""
    hi = int(cfg.get("index_heads", 0))
    if hi == 0:
        return []
    di, d, ql = cfg["index_dim"], cfg["hidden"], cfg["q_lora_rank"]
    return [
        TensorSpec(p + "idx_wq", (hi * di, ql), BF16, "weight"),
        TensorSpec(p + "idx_wk", (di, d), BF16, "weight"),
        TensorSpec(p + "idx_w", (hi, d), BF16, "weight"),
    ]


def weight_specs(cfg: dict) -> List[TensorSpec]:
    """Canonical ordered tensor list of a config (the order weights are bound in). With
    "weights": "fp8" each linear matrix is FP8 and followed by its fp32 row scales."""
    out = _weight_specs_bf16(cfg)
    if cfg.get("weights") == "mxfp4":
        if cfg["arch"] != "moe":
            raise ValueError("MXFP4 expert weights need an MoE config")
        mx: List[TensorSpec] = []
        for s in out:
            if ".experts." in s.name or ".shared." in s.name:
                mx.append(TensorSpec(s.name, s.shape[:-1] + (s.shape[-1] // 2,), FP4X2, "weight"))
                mx.append(TensorSpec(s.name + ".scale", s.shape[:-1] + (s.shape[-1] // 32,), E8M0, "scale"))
            else:
                mx.append(s)
        return mx
    if cfg.get("weights", "bf16") != "fp8":
        return out
    q: List[TensorSpec] = []
    for s in out:
        if s.init == "weight" and not s.name.endswith(FP8_KEEP_BF16):
            q.append(TensorSpec(s.name, s.shape, FP8, "weight"))
            q.append(TensorSpec(s.name + ".scale", s.shape[:-1], FP32, "scale"))
        else:
            q.append(s)
    return q


# Matrices that stay bf16 under "weights": "fp8" (latent families): the per-head absorption
# matrices (2 MB a layer, read by the attention's own loops) and the router (its logits decide
# the expert choice).
FP8_KEEP_BF16 = (".w_uk", ".w_uv", ".router")


def _weight_specs_bf16(cfg: dict) -> List[TensorSpec]:
    arch = cfg["arch"]
    d = cfg["hidden"]
    out: List[TensorSpec] = []
    for l in range(cfg["n_layers"]):
        p = f"layers.{l}."
        if arch == "gqa":
            nq, nkv, hd = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
            out += [
                TensorSpec(p + "attn_norm", (d,), BF16, "gain"),
                TensorSpec(p + "wq", (nq * hd, d), BF16, "weight"),
                TensorSpec(p + "wk", (nkv * hd, d), BF16, "weight"),
                TensorSpec(p + "wv", (nkv * hd, d), BF16, "weight"),
                TensorSpec(p + "wo", (d, nq * hd), BF16, "weight"),
            ]
        else:
            out += _mla_attn_specs(cfg, p)
        out.append(TensorSpec(p + "ffn_norm", (d,), BF16, "gain"))
        if arch in ("gqa", "mla"):
            f = cfg["ffn"]
            out += [
                TensorSpec(p + "w_gate", (f, d), BF16, "weight"),
                TensorSpec(p + "w_up", (f, d), BF16, "weight"),
                TensorSpec(p + "w_down", (d, f), BF16, "weight"),
            ]
        elif arch == "moe":
            e, ef, ns = cfg["n_routed"], cfg["expert_ffn"], cfg["n_shared"]
            out += [
                TensorSpec(p + "router", (e, d), BF16, "weight"),
                TensorSpec(p + "router_bias", (e,), FP32, "router_bias"),
                TensorSpec(p + "experts.w_gate", (e, ef, d), BF16, "weight"),
                TensorSpec(p + "experts.w_up", (e, ef, d), BF16, "weight"),
                TensorSpec(p + "experts.w_down", (e, d, ef), BF16, "weight"),
                TensorSpec(p + "shared.w_gate", (ns * ef, d), BF16, "weight"),
                TensorSpec(p + "shared.w_up", (ns * ef, d), BF16, "weight"),
                TensorSpec(p + "shared.w_down", (d, ns * ef), BF16, "weight"),
            ]
        else:
            raise ValueError(f"unknown arch {arch!r}")
    if cfg.get("vocab", 0) > 0:
        out.append(TensorSpec("final_norm", (d,), BF16, "gain"))
        out.append(TensorSpec("lm_head", (cfg["vocab"], d), BF16, "weight"))
    return out


def n_tokens(cfg: dict) -> int:
    """Tokens per step: 1 for a decode step; M > 1 for a multi-token verification step
    ("verify": M in the config), whose M tokens take positions kv_len .. kv_len + M - 1."""
    return int(cfg.get("verify", 1))


def kv_shape(cfg: dict, kv_len: Optional[int] = None) -> Tuple[int, ...]:
    """Cache layout: GQA [L][2][n_kv][kv_len+M][head_dim]; MLA/MoE [L][kv_len+1][kv_lora+rope]
    (M = tokens per step: the step writes slots kv_len .. kv_len + M - 1); with a sparse
    indexer each latent row is followed by the position's index key [index_dim]."""
    n = cfg["kv_len"] if kv_len is None else kv_len
    if cfg["arch"] == "gqa":
        return (cfg["n_layers"], 2, cfg["n_kv_heads"], n + n_tokens(cfg), cfg["head_dim"])
    return (cfg["n_layers"], n + 1, cfg["kv_lora_rank"] + cfg["qk_rope"] + int(cfg.get("index_dim", 0) if cfg.get("index_heads", 0) else 0))


def x_shape(cfg: dict) -> Tuple[int, ...]:
    m = n_tokens(cfg)
    return (m, cfg["hidden"]) if m > 1 else (cfg["hidden"],)


def out_shape(cfg: dict) -> Tuple[int, ...]:
    m = n_tokens(cfg)
    o = (cfg["vocab"],) if cfg.get("vocab", 0) > 0 else (cfg["hidden"],)
    return (m,) + o if m > 1 else o


def _quantize_e4m3_rows(torch, w32):
    """Per-row E4M3 quantisation of an fp32 [rows][cols] tensor: (bytes as uint8, fp32 scales)."""
    amax = w32.abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (w32 / scale[:, None]).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale.to(torch.float32)


_E2M1_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)  # between consecutive E2M1 magnitudes


def _quantize_mxfp4(torch, w32):
    """MXFP4 quantisation of an fp32 [rows][K] tensor (K a multiple of 32): (packed E2M1
    pairs uint8 [rows][K/2], E8M0 scales uint8 [rows][K/32])."""
    rows, k = w32.shape
    blk = w32.view(rows, k // 32, 32)
    amax = blk.abs().amax(dim=2)
    e = torch.floor(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax)))) - 2
    e = torch.where(amax > 0, e, torch.full_like(e, -127.0)).clamp_(-127, 127)
    v = blk / torch.exp2(e)[:, :, None]
    mid = torch.tensor(_E2M1_MIDPOINTS, dtype=torch.float32, device=w32.device)
    mag = torch.bucketize(v.abs().contiguous(), mid, right=True).to(torch.uint8)  # 0..7
    code = mag | torch.where(v < 0, 8, 0).to(torch.uint8)
    code = code.view(rows, k)
    packed = code[:, 0::2] | (code[:, 1::2] << 4)
    return packed.contiguous(), (e + 127).to(torch.uint8)


def weight_bytes(cfg: dict) -> int:
    return sum(s.nbytes for s in weight_specs(cfg))


# ----------------------------------------------------------------------------------------
# seeded generation (torch is used only as a random-number source and a container)
# ----------------------------------------------------------------------------------------

def _bf16_randn(torch, shape, std, gen, device, mean=0.0, chunk_elems=1 << 28):
    """N(mean, std) drawn in fp32 then rounded to bf16, generated in row chunks."""
    t = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = t.view(-1)
    n = flat.numel()
    i = 0
    while i < n:
        m = min(chunk_elems, n - i)
        tmp = torch.randn(m, generator=gen, device=device, dtype=torch.float32)
        if std != 1.0:
            tmp.mul_(std)
        if mean != 0.0:
            tmp.add_(mean)
        flat[i:i + m].copy_(tmp)
        del tmp
        i += m
    return t


def generate(cfg: dict, seed: int = 0, device="cpu", kv_len: Optional[int] = None):
    """Return (weights: dict name->tensor, x: bf16 tensor, kv: bf16 tensor) on `device`.

    Every tensor is drawn from one generator seeded with `seed`, in canonical order:
    weights (weight_specs order), then the KV cache, then x.
    """
    import torch
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    init = cfg["init"]
    weights = {}
    for s in weight_specs(cfg):
        if s.init == "scale":
            continue  # produced with its matrix
        if s.init == "weight" and s.dtype == FP4X2:
            kk = 2 * s.shape[-1]
            lead = s.shape[:-1]
            nrow = 1
            for dim in lead:
                nrow *= dim
            q = torch.empty((nrow, kk // 2), dtype=torch.uint8, device=dev)
            sc = torch.empty((nrow, kk // 32), dtype=torch.uint8, device=dev)
            rows = max(1, (1 << 26) // kk)
            for r0 in range(0, nrow, rows):
                r1 = min(nrow, r0 + rows)
                w32 = torch.randn((r1 - r0, kk), generator=gen, device=dev, dtype=torch.float32)
                w32.mul_(init["weight_std"])
                q[r0:r1], sc[r0:r1] = _quantize_mxfp4(torch, w32)
                del w32
            weights[s.name] = q.view(lead + (kk // 2,))
            weights[s.name + ".scale"] = sc.view(lead + (kk // 32,))
        elif s.init == "weight" and s.dtype == FP8:
            kk = s.shape[-1]
            nrow = s.numel // kk
            q = torch.empty((nrow, kk), dtype=torch.uint8, device=dev)
            sc = torch.empty(nrow, dtype=torch.float32, device=dev)
            rows = max(1, (1 << 26) // kk)
            for r0 in range(0, nrow, rows):
                r1 = min(nrow, r0 + rows)
                w32 = torch.randn((r1 - r0, kk), generator=gen, device=dev, dtype=torch.float32)
                w32.mul_(init["weight_std"])
                q[r0:r1], sc[r0:r1] = _quantize_e4m3_rows(torch, w32)
                del w32
            weights[s.name] = q.view(s.shape)
            weights[s.name + ".scale"] = sc.view(s.shape[:-1])
        elif s.init == "weight":
            weights[s.name] = _bf16_randn(torch, s.shape, init["weight_std"], gen, dev)
        elif s.init == "gain":
            g = init["gain"]
            if g == "ones":
                weights[s.name] = torch.ones(s.shape, dtype=torch.bfloat16, device=dev)
            else:
                weights[s.name] = _bf16_randn(torch, s.shape, g["std"], gen, dev, mean=g["mean"])
        elif s.init == "router_bias":
            weights[s.name] = torch.randn(s.shape, generator=gen, device=dev,
                                          dtype=torch.float32) * init["router_bias_std"]
        else:
            raise ValueError(s.init)
    n = cfg["kv_len"] if kv_len is None else kv_len
    kvs = kv_shape(cfg, n)  # positions [0, n) drawn, the step's own slots zero
    kv = torch.zeros(kvs, dtype=torch.bfloat16, device=dev)
    if n > 0:
        if cfg["arch"] == "gqa":
            kv[:, :, :, :n, :].copy_(_bf16_randn(torch, kvs[:3] + (n, kvs[4]),
                                                 init["kv_std"], gen, dev))
        else:
            kv[:, :n, :].copy_(_bf16_randn(torch, (kvs[0], n, kvs[2]), init["kv_std"], gen, dev))
    x = _bf16_randn(torch, x_shape(cfg), init["x_std"], gen, dev)
    return weights, x, kv


def generate_embedding(cfg: dict, seed: int = 0, device="cpu"):
    """The token embedding [vocab][hidden] (bf16 ~ N(0, x_std), the distribution of x) that a
    plan with a per-step length reads its input row from when it is given no input vector.
    Drawn from its own generator (seed + 1_000_003), so `generate` stays unchanged."""
    import torch
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed) + 1_000_003)
    return _bf16_randn(torch, (cfg["vocab"], cfg["hidden"]), cfg["init"]["x_std"], gen, dev)


def bf16_bits(t):
    """A bf16 torch tensor as a numpy uint16 array of its bit patterns (host copy)."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view("uint16")
