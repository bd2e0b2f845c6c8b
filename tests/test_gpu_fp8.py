"""GPU parity of the FP8-weight GQA engine (E4M3 rows with fp32 row scales) against the
fp64 oracle, which decodes the same bytes exactly (needs an MI355X).

Bars as for bf16 weights: relative L2 <= 1e-2 on every per-layer trace vector, <= 2e-2 on the
logits, the written cache slot within one bf16 ulp of the oracle's rounding, every task once.
The products are exact in both (an E4M3 value times a fp32 input has at most 28 significant
bits, rounded once per fp32 accumulation on the GPU), so the errors are those of bf16 weights.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from test_gpu_parity import (TRACE_GQA, HostWeights, LOGIT_TOL, _teacher_forced_check, check_coverage,
                             check_kv_slot, check_layer_trace, rel_l2)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,seed", [("tiny_fp8", 0), ("tiny_fp8", 1), ("tiny_ragged_fp8", 0), ("small_gqa_fp8", 0)])
def test_fp8_full_parity(name, seed):
    print(f"[fp8] {name} seed={seed}", flush=True)
    from persistent_tile_scheduled_amd.engine import DecodeEngine
    cfg = workloads.get_config(name)
    w, x, kv = workloads.generate(cfg, seed=seed, device="cuda")
    assert w["layers.0.wq"].dtype == torch.uint8
    eng = DecodeEngine(cfg, w)
    out = eng.step(x, kv)
    torch.cuda.synchronize()
    eng.status()
    W = HostWeights(w)
    kvb = workloads.bf16_bits(kv)
    res = O.forward(cfg, W, workloads.bf16_bits(x), kvb)
    for l, t in enumerate(res["layers"]):
        check_layer_trace(eng, l, t, TRACE_GQA)
        check_kv_slot(cfg, kvb, l, t, same_input=(l == 0))
    err = rel_l2(out.cpu().numpy(), res["out"])
    print(f"[fp8] {name}: logits rel error {err:.3e}", flush=True)
    assert err <= LOGIT_TOL
    check_coverage(eng)


def test_fp8_plan_rejects_stage_launches():
    from persistent_tile_scheduled_amd.binding import DecError
    from persistent_tile_scheduled_amd.engine import DecodeEngine
    cfg = workloads.get_config("tiny_fp8")
    w, x, kv = workloads.generate(cfg, seed=0, device="cuda")
    eng = DecodeEngine(cfg, w)
    with pytest.raises(DecError):
        eng.step_stages(x, kv)


def test_8b_4k_fp8_sampled_layers():
    _teacher_forced_check("8b_4k_fp8", [0, 1, 31])
