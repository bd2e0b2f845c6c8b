"""The step as one launch per stage (dec_step_stages), eagerly and as a replayed HIP graph
(needs an MI355X).

Bars: the per-stage step meets the same oracle bars as the single persistent launch (relative
L2 <= 1e-2 on every per-layer trace vector, <= 2e-2 on the output, top-k exact for MoE) and
every task runs exactly once per step; the per-stage and persistent outputs agree to fp32
reordering (split-K sums into shared accumulators land in run-dependent order); each graph
replay, with eager work and synchronisation between replays, matches the eager per-stage
result to the same bar.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from test_gpu_parity import (TRACE_GQA, HostWeights, LOGIT_TOL, check_coverage, check_kv_slot,
                             check_layer_trace, rel_l2)
from test_gpu_parity_mla import check_mla_layer

pytestmark = pytest.mark.gpu

# Two runs of the same kernels differ by the order in which split-K partial sums land in
# shared accumulators (fp32 reordering, ~1e-7 relative); where such a value is then rounded to
# bf16 (the appended cache entries, which the step's attention reads back), a rounding can
# land one bf16 ulp (2^-8 relative) apart and carry into later layers. Bar between two runs:
REORDER_TOL = 1e-3


def _engine(cfg, w):
    from persistent_tile_scheduled_amd.engine import DecodeEngine
    return DecodeEngine(cfg, w)


@pytest.mark.parametrize("name", ["tiny", "tiny_mha_ragged", "small_gqa", "mla_tiny", "moe_tiny"])
def test_stage_launches_match_oracle(name):
    print(f"[stages] {name}", flush=True)
    cfg = workloads.get_config(name)
    w, x, kv = workloads.generate(cfg, seed=3, device="cuda")
    eng = _engine(cfg, w)
    assert eng.n_stages > 1
    out = eng.step_stages(x, kv).clone()
    torch.cuda.synchronize()
    eng.status()
    check_coverage(eng, steps=1)
    W = HostWeights(w)
    kvb = workloads.bf16_bits(kv)
    res = O.forward(cfg, W, workloads.bf16_bits(x), kvb)
    for l, t in enumerate(res["layers"]):
        if cfg["arch"] == "gqa":
            check_layer_trace(eng, l, t, TRACE_GQA)
            check_kv_slot(cfg, kvb, l, t, same_input=(l == 0))
        else:
            check_mla_layer(eng, cfg, l, t, W, kvb)
    assert rel_l2(out.cpu().numpy(), res["out"]) <= LOGIT_TOL
    # the persistent launch on the same inputs (its slot write repeats the same values)
    out2 = eng.step(x, kv).clone()
    torch.cuda.synchronize()
    eng.status()
    check_coverage(eng, steps=2)
    assert rel_l2(out2.cpu().numpy(), res["out"]) <= LOGIT_TOL
    err = rel_l2(out2.cpu().numpy(), out.cpu().numpy())
    print(f"[stages] {name}: per-stage vs persistent rel L2 {err:.3e}", flush=True)
    assert err <= REORDER_TOL


def test_stage_range_validation():
    from persistent_tile_scheduled_amd.binding import DecError
    cfg = workloads.get_config("tiny")
    w, x, kv = workloads.generate(cfg, seed=0, device="cuda")
    eng = _engine(cfg, w)
    ns = eng.n_stages
    for lo, hi in [(-1, 1), (0, 0), (2, 1), (0, ns + 1)]:
        with pytest.raises(DecError):
            eng.plan.step_stages(x.data_ptr(), kv.data_ptr(), eng.out.data_ptr(), lo, hi, eng.stream.cuda_stream)
    # two ranges covering the step: a multi-stage (cooperative) launch, then the rest
    mid = ns // 2
    eng.plan.step_stages(x.data_ptr(), kv.data_ptr(), eng.out.data_ptr(), 0, mid, eng.stream.cuda_stream)
    eng.plan.step_stages(x.data_ptr(), kv.data_ptr(), eng.out.data_ptr(), mid, ns, eng.stream.cuda_stream)
    a = eng.out.clone()
    eng.step(x, kv)
    torch.cuda.synchronize()
    eng.status()
    check_coverage(eng, steps=2)
    assert rel_l2(eng.out.cpu().numpy(), a.cpu().numpy()) <= REORDER_TOL


@pytest.mark.parametrize("name", ["tiny", "moe_tiny"])
def test_stage_graph_replays(name):
    print(f"[graph] {name}", flush=True)
    cfg = workloads.get_config(name)
    w, x, kv = workloads.generate(cfg, seed=4, device="cuda")
    eng = _engine(cfg, w)
    ref = eng.step_stages(x, kv).clone()
    torch.cuda.synchronize()
    g = eng.capture_stages(x, kv)
    torch.cuda.synchronize()
    eng.status()
    steps = 1
    for rep in range(4):
        eng.out.fill_(float("nan"))
        junk = torch.randn(1 << 16, device="cuda").sum()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        eng.status()
        steps += 1
        assert float(junk) == float(junk)
        got = eng.out.cpu().numpy()
        assert np.all(np.isfinite(got)), rep
        assert rel_l2(got, ref.cpu().numpy()) <= REORDER_TOL, rep
    # capture itself runs nothing; every replay ran every task once
    check_coverage(eng, steps=steps)
