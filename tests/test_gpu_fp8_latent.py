"""GPU parity of the latent families (MLA, MLA + MoE) with FP8 E4M3 weights (fp32 row scales)
against the fp64 oracle, which decodes the same bytes exactly (needs an MI355X).

Every linear matrix but the per-head absorption matrices and the router is FP8; the engine
converts the bytes in hardware, applies each row's scale to the row's sum and accumulates in
fp32, so the bars are the bf16 path's tight ones: relative L2 <= TIGHT_TOL on every per-layer
trace vector and on the output, the top-k exactly the oracle's rule on the engine's own router
logits, and task-schedule coverage.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from test_gpu_parity import HostWeights, LOGIT_TOL, TIGHT_TOL, check_coverage, check_kv_slot, rel_l2
from test_gpu_parity_mla import DENSE_FFN, MLA_TRACE, MOE_FFN, check_mla_layer, check_moe_layer

pytestmark = pytest.mark.gpu


def _engine(cfg, w, **kw):
    from persistent_tile_scheduled_amd.engine import DecodeEngine
    return DecodeEngine(cfg, w, **kw)


@pytest.mark.parametrize("name,seed,kv_len", [("mla_tiny_fp8", 0, None), ("mla_tiny_fp8", 2, 0), ("mla_small_fp8", 0, None),
                                              ("moe_tiny_fp8", 0, None), ("moe_small_fp8", 1, None)])
def test_fp8_latent_full_parity(name, seed, kv_len):
    cfg = dict(workloads.get_config(name))
    if kv_len is not None:
        cfg["kv_len"] = kv_len
    print(f"[fp8-latent] {name} seed={seed} kv_len={cfg['kv_len']}", flush=True)
    w, x, kv = workloads.generate(cfg, seed=seed, device="cuda")
    eng = _engine(cfg, w)
    out = eng.step(x, kv)
    torch.cuda.synchronize()
    eng.status()
    W = HostWeights(w)
    kvb = workloads.bf16_bits(kv)
    res = O.forward(cfg, W, workloads.bf16_bits(x), kvb)
    for l, t in enumerate(res["layers"]):
        errs = check_mla_layer(eng, cfg, l, t, W, kvb, tol=TIGHT_TOL)
        print(f"[fp8-latent] layer {l}: max rel error {max(errs.values()):.2e}", flush=True)
    assert rel_l2(out.cpu().numpy(), res["out"]) <= min(LOGIT_TOL, TIGHT_TOL)
    check_coverage(eng)


@pytest.mark.parametrize("name", ["mla_8k_fp8", "moe_4k_fp8"])
def test_fp8_latent_full_size_every_layer(name):
    """The full-size stacks in the bench's launch configuration: every layer recomputed by the
    oracle from the engine's own layer input."""
    cfg = workloads.get_config(name)
    print(f"[fp8-latent] {name}: generating", flush=True)
    w, x, kv = workloads.generate(cfg, seed=0, device="cuda")
    eng = _engine(cfg, w)
    out = eng.step(x, kv)
    torch.cuda.synchronize()
    eng.status()
    W = HostWeights(w)
    n = cfg["kv_len"]
    names = MLA_TRACE + (DENSE_FFN if cfg["arch"] == "mla" else MOE_FFN)
    for l in range(cfg["n_layers"]):
        xin = (O.widen_bf16(workloads.bf16_bits(x)) if l == 0
               else eng.buffer(f"layers.{l - 1}.x_out").cpu().numpy().astype(np.float64))
        kvl = workloads.bf16_bits(kv[l])
        _, t = O.mla_layer(cfg, W, l, xin, kvl, n)
        errs = {nm: rel_l2(eng.buffer(f"layers.{l}.{nm}").cpu().numpy()[: t[nm].size], t[nm]) for nm in names}
        print(f"[fp8-latent] {name} layer {l} max rel error {max(errs.values()):.2e}", flush=True)
        assert all(v <= TIGHT_TOL for v in errs.values()), errs
        check_kv_slot(cfg, kvl[None], 0, t)
        if cfg["arch"] == "moe":
            check_moe_layer(eng, cfg, l, t, W)
        W.drop(f"layers.{l}.")
    xo = eng.buffer(f"layers.{cfg['n_layers'] - 1}.x_out").cpu().numpy()
    assert np.array_equal(out.cpu().numpy(), xo)
    check_coverage(eng)


def test_fp8_latent_plan_with_per_step_length():
    cfg = workloads.get_config("moe_tiny_fp8")
    M = 300
    w, x, kv = workloads.generate(cfg, seed=13, device="cuda", kv_len=M)
    eng = _engine(cfg, w, max_len=M)
    W = HostWeights(w)
    for p in [0, 5, M // 2, M]:
        print(f"[fp8-latent] dynamic position {p}", flush=True)
        kvb = workloads.bf16_bits(kv)
        eng.set_state(p, 0)
        out = eng.step_dynamic(kv, x).clone()
        torch.cuda.synchronize()
        eng.status()
        cfg_p = dict(cfg, kv_len=p)
        res = O.forward(cfg_p, W, workloads.bf16_bits(x), kvb, kv_len=p)
        assert rel_l2(out.cpu().numpy(), res["out"]) <= min(LOGIT_TOL, TIGHT_TOL), p
        kv_after = workloads.bf16_bits(kv)
        for l in range(cfg["n_layers"]):
            xin = (O.widen_bf16(workloads.bf16_bits(x)) if l == 0
                   else eng.buffer(f"layers.{l - 1}.x_out").cpu().numpy().astype(np.float64))
            _, t = O.mla_layer(cfg_p, W, l, xin, kv_after[l], p)
            check_mla_layer(eng, cfg_p, l, t, W, kv_after, tol=TIGHT_TOL, same_input=True)
    check_coverage(eng, steps=4)
