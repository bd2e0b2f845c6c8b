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


def test_fp8_plan_with_per_step_length():
    """FP8 weights in a plan that reads its position per step: positions 0, 1, L/2 and L
    against the oracle decoding the same bytes, then three greedy steps that start from the
    embedding row of the token the previous step chose (teacher-forced on the engine's tokens
    and cache). The token is the argmax of the engine's own fp32 logits, lowest index first."""
    from persistent_tile_scheduled_amd.engine import DecodeEngine
    cfg = workloads.get_config("tiny_fp8")
    M = cfg["kv_len"]
    w, x, kv = workloads.generate(cfg, seed=6, device="cuda", kv_len=M)
    w["embed"] = workloads.generate_embedding(cfg, seed=6, device="cuda")
    eng = DecodeEngine(cfg, w, max_len=M)
    W = HostWeights(w)
    argmax_low = lambda v: int(np.flatnonzero(v == v.max())[0])
    steps = 0
    for p in [0, 1, M // 2, M]:
        print(f"[fp8 dynamic] position {p}", flush=True)
        kvb = workloads.bf16_bits(kv)
        eng.set_state(p, 3)
        got = eng.step_dynamic(kv, x).clone().cpu().numpy()
        eng.status()
        steps += 1
        st = eng.read_state()
        assert st[0] == p + 1 and st[2] == 1 and st[1] == argmax_low(got), st
        res = O.forward(dict(cfg, kv_len=p), W, workloads.bf16_bits(x), kvb, kv_len=p)
        for l, t in enumerate(res["layers"]):
            check_layer_trace(eng, l, t, TRACE_GQA)
        assert rel_l2(got, res["out"]) <= LOGIT_TOL, p
    emb = workloads.bf16_bits(w["embed"])
    tok, p0 = 5, M - 3
    eng.set_state(p0, tok)
    for i in range(3):
        print(f"[fp8 greedy] step {i} token {tok}", flush=True)
        kvb = workloads.bf16_bits(kv)
        got = eng.step_dynamic(kv).clone().cpu().numpy()
        eng.status()
        steps += 1
        st = eng.read_state()
        assert st[0] == p0 + i + 1 and st[1] == argmax_low(got), st
        res = O.forward(dict(cfg, kv_len=p0 + i), W, emb[tok], kvb, kv_len=p0 + i)
        assert rel_l2(got, res["out"]) <= LOGIT_TOL, i
        tok = st[1]
    check_coverage(eng, steps=steps)
