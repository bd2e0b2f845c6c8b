"""The allocation-free binding (dec_plan_bind_scratch): a plan bound to the library's static
per-device workspace computes the same step as the same plan bound to a caller-allocated
workspace (needs an MI355X).

Two calls in a row share one static array: a larger model first, then a smaller one, whose
binding must clear what the first left behind; the first plan is then refused until it is
bound again.
"""
import numpy as np
import pytest
import torch

import workloads
from test_gpu_parity import TIGHT_TOL, rel_l2

pytestmark = pytest.mark.gpu


def _engine(cfg, w, **kw):
    from persistent_tile_scheduled_amd.engine import DecodeEngine
    return DecodeEngine(cfg, w, **kw)


def _step(eng, x, kv):
    out = eng.step(x, kv).clone()
    torch.cuda.synchronize()
    eng.status()
    return out.cpu().numpy()


def test_static_workspace_matches_allocated_workspace():
    from persistent_tile_scheduled_amd import binding as B
    engines = []
    for name in ("small_gqa", "tiny"):  # the second call's plan and inputs are smaller
        cfg = workloads.get_config(name)
        print(f"[no-alloc] {name}", flush=True)
        w, x, kv = workloads.generate(cfg, seed=5, device="cuda")
        kv_ref = kv.clone()
        ref = _step(_engine(cfg, w), x, kv_ref)
        eng = _engine(cfg, w, static_workspace=True)
        got = _step(eng, x, kv)
        err = rel_l2(got, ref)
        print(f"[no-alloc] {name}: rel L2 vs the allocated workspace {err:.3e}", flush=True)
        assert err <= TIGHT_TOL, (name, err)
        assert torch.equal(kv, kv_ref), name  # the same cache slot written
        got2 = _step(eng, x, kv)  # a second step on the static workspace (epochs advance)
        assert rel_l2(got2, ref) <= TIGHT_TOL, name
        engines.append(eng)
    # the first plan no longer owns the static workspace
    cfg = workloads.get_config("small_gqa")
    w, x, kv = workloads.generate(cfg, seed=5, device="cuda")
    with pytest.raises(B.DecError) as ei:
        engines[0].step(x, kv)
    assert B.STATUS[ei.value.status] == "DEC_E_UNBOUND"


def test_static_workspace_rejects_an_oversized_plan():
    """A plan whose workspace exceeds the static array is refused with DEC_E_CAPACITY."""
    from persistent_tile_scheduled_amd import binding as B
    cfg = workloads.get_config("tiny")
    plan = B.Plan(cfg, max_len=1_000_000)  # a RoPE row per position: 256 MB of tables
    assert plan.sizes()["workspace_bytes"] > 64 << 20
    with pytest.raises(B.DecError) as ei:
        plan.bind_scratch([16] * len(plan.weight_descs()))
    assert B.STATUS[ei.value.status] == "DEC_E_CAPACITY"
