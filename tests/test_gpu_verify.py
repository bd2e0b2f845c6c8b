"""GPU parity of verification steps -- M tokens at positions kv_len .. kv_len + M - 1 in one
launch -- against the fp64 oracle's causal block (oracle.verify_forward / gqa_verify_layer,
pinned on the CPU against M sequential decode steps). Bars as for single-token steps, per
token: relative L2 error <= TIGHT_TOL on every trace vector and the logits; each of the M
written cache slots within one bf16 ulp plus the fp32 accumulation error of the oracle's
rounding; every planned task once, and in dependency order.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from test_gpu_parity import (TIGHT_TOL, HostWeights, _engine, _slot_close, _slot_rel, check_coverage, rel_l2)

pytestmark = pytest.mark.gpu

TRACE = ("q", "attn", "h", "ffn_act", "ffn_out", "x_out")


def vcfg(name, m, **over):
    cfg = dict(workloads.get_config(name))
    cfg.update(over)
    cfg["verify"] = m
    return cfg


def check_trace_m(eng, l, t, m, tol=TIGHT_TOL):
    """Every trace vector of layer l, token by token."""
    worst = {}
    for key in TRACE:
        want = np.asarray(t[key]).reshape(m, -1)
        got = eng.buffer(f"layers.{l}.{key}").cpu().numpy()[: want.size].reshape(m, -1)
        errs = [rel_l2(got[i], want[i]) for i in range(m)]
        worst[key] = max(errs)
        assert worst[key] <= tol, (l, key, errs)
    return worst


def check_slots_m(cfg, kvl_bits, t, m, same_input=True):
    """The M cache slots the step wrote in one layer (kvl_bits [2][n_kv][kv_len + M][hd])."""
    n = cfg["kv_len"]
    chk = _slot_close if same_input else _slot_rel
    for i in range(m):
        chk(kvl_bits[0, :, n + i, :].reshape(-1), np.asarray(t["k_new_bits"])[i], ("k", i))
        chk(kvl_bits[1, :, n + i, :].reshape(-1), np.asarray(t["v_new_bits"])[i], ("v", i))


def run_verify(cfg, seed):
    w, x, kv = workloads.generate(cfg, seed=seed, device="cuda")
    eng = _engine()(cfg, w)
    assert eng.n_tokens == cfg["verify"]
    out = eng.step(x, kv)
    torch.cuda.synchronize()
    eng.status()
    return eng, w, x, kv, out


@pytest.mark.parametrize("name,m,seed", [
    ("tiny", 4, 0), ("tiny", 2, 1), ("tiny_gain", 3, 2), ("tiny_kv0", 3, 0), ("tiny_mha_ragged", 4, 0),
    ("small_gqa", 3, 0), ("small_gqa", 4, 5), ("tiny_hd256_g3", 4, 4)])
def test_verify_small_full_parity(name, m, seed):
    """Whole steps of small models end to end: per-token traces of every layer, the M new
    cache slots of every layer and the M rows of logits. The cases cover one and two blocks of
    8 query columns per KV group (small_gqa and tiny_hd256_g3 at M >= 3 have 12 or 16), an
    empty cache (tiny_kv0: the block attends only to itself) and ragged widths."""
    cfg = vcfg(name, m)
    print(f"[verify] {name} M={m} seed={seed}", flush=True)
    eng, w, x, kv, out = run_verify(cfg, seed)
    W = HostWeights(w)
    kvb = workloads.bf16_bits(kv)
    res = O.verify_forward(cfg, W, workloads.bf16_bits(x), kvb)
    for l, t in enumerate(res["layers"]):
        check_trace_m(eng, l, t, m)
        check_slots_m(cfg, kvb[l], t, m, same_input=(l == 0))
    got = out.cpu().numpy()
    assert got.shape == (m, cfg["vocab"])
    for i in range(m):
        assert rel_l2(got[i], res["out"][i]) <= TIGHT_TOL, i
    check_coverage(eng)


def test_verify_steps_in_a_row():
    """Two verification steps on one plan with different inputs and a cache that differs in
    its cached part: both match the oracle (epochs and counters carry across steps)."""
    cfg = vcfg("small_gqa", 4)
    eng, w, x, kv, out = run_verify(cfg, 11)
    W = HostWeights(w)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    for step in range(2):
        print(f"[verify] steps in a row: step {step}", flush=True)
        xs = (torch.randn(4, cfg["hidden"], generator=g, device="cuda") * (1 + step)).to(torch.bfloat16)
        kv[:, :, :, : cfg["kv_len"], :] = (torch.randn(kv[:, :, :, : cfg["kv_len"], :].shape, generator=g,
                                                       device="cuda") * 0.5).to(torch.bfloat16)
        o = eng.step(xs, kv).clone()
        torch.cuda.synchronize()
        eng.status()
        res = O.verify_forward(cfg, W, workloads.bf16_bits(xs), workloads.bf16_bits(kv))
        for i in range(4):
            assert rel_l2(o.cpu().numpy()[i], res["out"][i]) <= TIGHT_TOL, (step, i)
    check_coverage(eng, steps=3)


def _teacher_forced_verify(name, m, layers):
    """Full-size model in the bench's launch configuration: the oracle recomputes each listed
    layer for the M tokens from the GPU's own layer inputs; the LM head rows are checked from
    the GPU's final hidden states."""
    cfg = vcfg(name, m)
    print(f"[verify] {name} M={m}: generating", flush=True)
    eng, w, x, kv, out = run_verify(cfg, 0)
    W = HostWeights(w)
    n = cfg["kv_len"]
    for l in layers:
        xin = (O.widen_bf16(workloads.bf16_bits(x)) if l == 0 else
               eng.buffer(f"layers.{l - 1}.x_out").cpu().numpy().astype(np.float64).reshape(m, -1))
        kvl = workloads.bf16_bits(kv[l])
        _, t = O.gqa_verify_layer(cfg, W, l, xin, kvl, n)
        worst = check_trace_m(eng, l, t, m)
        print(f"[verify] layer {l} worst per-token rel errors {worst}", flush=True)
        check_slots_m(cfg, kvl, t, m)
        W.drop(f"layers.{l}.")
    xf = eng.buffer(f"layers.{cfg['n_layers'] - 1}.x_out").cpu().numpy().astype(np.float64).reshape(m, -1)
    got = out.cpu().numpy()
    for i in range(m):
        err = rel_l2(got[i], O.head(cfg, W, xf[i])["out"])
        print(f"[verify] token {i} logits rel error {err:.3e}", flush=True)
        assert err <= TIGHT_TOL
    n_pairs = check_coverage(eng)
    print(f"[verify] {name} M={m}: dependency order checked on {n_pairs} pairs", flush=True)


def test_8b_4k_verify4_every_layer():
    _teacher_forced_verify("8b_4k", 4, list(range(32)))


def test_8b_4k_verify2_sampled_layers():
    _teacher_forced_verify("8b_4k", 2, [0, 1, 15, 31])
