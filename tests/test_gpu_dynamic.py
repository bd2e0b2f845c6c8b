"""Plans whose position is read per step (dec_plan_create_dynamic / dec_step_dynamic) against
the fp64 oracle (needs an MI355X).

Bars: as for fixed-length plans -- relative L2 <= 1e-2 on every per-layer trace vector and
<= 2e-2 on the logits at each position, the written cache slot within one bf16 ulp of the
oracle's rounding, every task once per step. The greedy token is integer work decided by
floating point: it must equal the argmax of the engine's own fp32 logits exactly (lowest
index among equals), and the oracle's fp64 argmax wherever the oracle's top-2 margin exceeds
what the fp32 logits can move. Generation is teacher-forced on the engine's tokens and cache,
so one near-tie cannot derail the comparison of later steps.
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

MARGIN = 1e-3  # relative to the logit scale: fp32 logits move the top-2 gap by far less


def _engine(cfg, w, max_len):
    from persistent_tile_scheduled_amd.engine import DecodeEngine
    return DecodeEngine(cfg, w, max_len=max_len)


def _argmax_low(v):
    v = np.asarray(v)
    return int(np.flatnonzero(v == v.max())[0])


@pytest.mark.parametrize("name", ["tiny", "tiny_mha_ragged", "small_gqa"])
def test_positions_of_one_plan_match_oracle(name):
    cfg = workloads.get_config(name)
    M = cfg["kv_len"]
    w, x, kv = workloads.generate(cfg, seed=11, device="cuda", kv_len=M)
    w["embed"] = workloads.generate_embedding(cfg, seed=11, device="cuda") if cfg.get("vocab", 0) > 0 else None
    if w["embed"] is None:
        del w["embed"]
    eng = _engine(cfg, w, M)
    W = HostWeights(w)
    steps = 0
    for p in [0, 1, M // 3, M - 1, M]:
        print(f"[dynamic] {name} position {p}", flush=True)
        kvb = workloads.bf16_bits(kv)  # the cache as this step sees it
        eng.set_state(p, 0)
        out = eng.step_dynamic(kv, x).clone()
        torch.cuda.synchronize()
        eng.status()
        steps += 1
        st = eng.read_state()
        assert st[0] == p + 1 and st[2] == 1, st
        cfg_p = dict(cfg, kv_len=p)
        res = O.forward(cfg_p, W, workloads.bf16_bits(x), kvb, kv_len=p)
        for l, t in enumerate(res["layers"]):
            check_layer_trace(eng, l, t, TRACE_GQA)
            check_kv_slot(cfg_p, workloads.bf16_bits(kv), l, t, same_input=(l == 0))
        got = out.cpu().numpy()
        assert rel_l2(got, res["out"]) <= LOGIT_TOL, p
        if cfg.get("vocab", 0) > 0:
            assert st[1] == _argmax_low(got), (st, _argmax_low(got))
    check_coverage(eng, steps=steps)


@pytest.mark.parametrize("name,max_len", [("mla_tiny", 1000), ("moe_tiny", 300)])
def test_latent_positions_of_one_plan_match_oracle(name, max_len):
    """Latent-attention plans with a per-step length. The splits are planned for max_len + 1
    positions (16 for mla_tiny at 1000, 5 for moe_tiny at 300), so the small positions leave
    some splits empty; every position must still match the oracle, top-k included."""
    cfg = workloads.get_config(name)
    w, x, kv = workloads.generate(cfg, seed=13, device="cuda", kv_len=max_len)
    eng = _engine(cfg, w, max_len)
    W = HostWeights(w)
    steps = 0
    for p in [0, 1, 5, 63, 64, max_len // 2, max_len - 1, max_len]:
        print(f"[dynamic] {name} position {p}", flush=True)
        kvb = workloads.bf16_bits(kv)
        eng.set_state(p, 0)
        out = eng.step_dynamic(kv, x).clone()
        torch.cuda.synchronize()
        eng.status()
        steps += 1
        st = eng.read_state()
        assert st[0] == p + 1 and st[2] == 1, st
        cfg_p = dict(cfg, kv_len=p)
        kv_after = workloads.bf16_bits(kv)  # slot p written; positions [0, p) as the step saw them
        # each layer against the oracle's layer from the engine's own layer input, so the bars
        # hold per layer rather than for error carried through the stack
        for l in range(cfg["n_layers"]):
            xin = (O.widen_bf16(workloads.bf16_bits(x)) if l == 0
                   else eng.buffer(f"layers.{l - 1}.x_out").cpu().numpy().astype(np.float64))
            _, t = O.mla_layer(cfg_p, W, l, xin, kv_after[l], p)
            check_mla_layer(eng, cfg_p, l, t, W, kv_after, same_input=True)
        # and the whole step end to end
        res = O.forward(cfg_p, W, workloads.bf16_bits(x), kvb, kv_len=p)
        assert rel_l2(out.cpu().numpy(), res["out"]) <= LOGIT_TOL, p
    check_coverage(eng, steps=steps)


def test_latent_dynamic_equals_fixed_plan_at_its_length():
    """At position kv_len the latent plan with a per-step length computes what the fixed plan
    for kv_len does (same split count when max_len + 1 rounds to the same number of splits)."""
    from persistent_tile_scheduled_amd.engine import DecodeEngine
    print("[dynamic] mla_small: per-step-length plan against the fixed plan", flush=True)
    cfg = workloads.get_config("mla_small")
    n = cfg["kv_len"]
    w, x, kv = workloads.generate(cfg, seed=5, device="cuda")
    a = DecodeEngine(cfg, w).step(x, kv).clone()
    dyn = _engine(cfg, w, n + 20)
    kv2 = torch.zeros(workloads.kv_shape(cfg, n + 20), dtype=torch.bfloat16, device="cuda")
    kv2[:, :n + 1, :].copy_(kv[:, :n + 1, :])
    dyn.set_state(n, 0)
    b = dyn.step_dynamic(kv2, x).clone()
    torch.cuda.synchronize()
    dyn.status()
    assert rel_l2(b.cpu().numpy(), a.cpu().numpy()) <= 1e-3


def test_dynamic_equals_fixed_plan_at_its_length():
    """At position kv_len the dynamic plan computes what the fixed plan for kv_len does."""
    from persistent_tile_scheduled_amd.engine import DecodeEngine
    cfg = workloads.get_config("small_gqa")
    n = cfg["kv_len"]
    w, x, kv = workloads.generate(cfg, seed=5, device="cuda")
    fixed = DecodeEngine(cfg, w)
    a = fixed.step(x, kv).clone()
    w["embed"] = workloads.generate_embedding(cfg, seed=5, device="cuda")
    dyn = _engine(cfg, w, n + 37)
    kv2 = torch.zeros(workloads.kv_shape(cfg, n + 37), dtype=torch.bfloat16, device="cuda")
    kv2[:, :, :, :n + 1, :].copy_(kv[:, :, :, :n + 1, :])
    dyn.set_state(n, 0)
    b = dyn.step_dynamic(kv2, x).clone()
    torch.cuda.synchronize()
    dyn.status()
    assert rel_l2(b.cpu().numpy(), a.cpu().numpy()) <= 1e-3


def test_greedy_generation_matches_oracle():
    cfg = workloads.get_config("tiny")
    p0, T = cfg["kv_len"], 10
    M = p0 + T
    w, _, kv = workloads.generate(cfg, seed=21, device="cuda", kv_len=M)
    w["embed"] = workloads.generate_embedding(cfg, seed=21, device="cuda")
    emb = workloads.bf16_bits(w["embed"])
    eng = _engine(cfg, w, M)
    W = HostWeights(w)
    tok = 7
    eng.set_state(p0, tok)
    for i in range(T):
        p = p0 + i
        print(f"[greedy] step {i} position {p} token {tok}", flush=True)
        kvb = workloads.bf16_bits(kv)
        out = eng.step_dynamic(kv).clone()  # input: the embedding row of the state's token
        torch.cuda.synchronize()
        eng.status()
        st = eng.read_state()
        got = out.cpu().numpy()
        assert st[0] == p + 1 and st[2] == i + 1, st
        assert st[1] == _argmax_low(got)
        res = O.forward(dict(cfg, kv_len=p), W, emb[tok], kvb, kv_len=p)
        want = res["out"]
        assert rel_l2(got, want) <= LOGIT_TOL, i
        top = np.sort(want)[::-1]
        if top[0] - top[1] > MARGIN * np.abs(want).max():
            assert st[1] == _argmax_low(want), (i, st[1], _argmax_low(want))
        tok = st[1]
    check_coverage(eng, steps=T)


def test_back_to_back_steps_advance_the_state():
    """T steps issued with no host synchronisation: the device state carries position, token
    and step count from one to the next, and every task ran T times."""
    cfg = workloads.get_config("tiny")
    p0, T = 3, 20
    w, x, kv = workloads.generate(cfg, seed=2, device="cuda", kv_len=p0 + T)
    w["embed"] = workloads.generate_embedding(cfg, seed=2, device="cuda")
    eng = _engine(cfg, w, p0 + T)
    eng.set_state(p0, 1)
    for _ in range(T):
        eng.step_dynamic(kv)
    torch.cuda.synchronize()
    eng.status()
    st = eng.read_state()
    assert st[0] == p0 + T and st[2] == T, st
    assert st[1] == _argmax_low(eng.out.cpu().numpy())
    check_coverage(eng, steps=T)


def test_state_out_of_range_is_reported_and_harmless():
    from persistent_tile_scheduled_amd.binding import DecError
    cfg = workloads.get_config("tiny")
    M = 40
    w, x, kv = workloads.generate(cfg, seed=3, device="cuda", kv_len=M)
    w["embed"] = workloads.generate_embedding(cfg, seed=3, device="cuda")
    eng = _engine(cfg, w, M)
    for pos, tok in [(M + 1, 0), (-1, 0), (5, cfg["vocab"])]:
        eng.set_state(pos, tok)
        eng.step_dynamic(kv)  # x = None: the token must be a valid row
        with pytest.raises(DecError) as ei:
            eng.status()
        assert ei.value.status == -3, ei.value
        assert eng.read_state()[:3] == [pos, tok, 0]
        eng.plan.reset(eng.stream.cuda_stream)
    eng.set_state(5, 3)
    eng.step_dynamic(kv)
    torch.cuda.synchronize()
    eng.status()
    assert eng.read_state()[0] == 6
    check_coverage(eng, steps=1)
