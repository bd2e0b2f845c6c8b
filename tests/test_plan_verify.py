"""Host-side tests of verification-step plans (dec_plan_create_verify on a described device):
M tokens at positions kv_len .. kv_len + M - 1 in one step. No GPU and no compute call."""
import collections
import math

import pytest

import workloads
from persistent_tile_scheduled_amd import binding as B
from test_plan_cpu import MI355X, simulate

CASES = [("tiny", 2), ("tiny", 4), ("tiny_kv0", 3), ("tiny_mha_ragged", 4), ("small_gqa", 2), ("small_gqa", 3),
         ("tiny_hd256_g3", 4), ("8b_4k", 2), ("8b_4k", 4), ("8b_32k", 4)]


def vplan(name, m, dev=MI355X):
    cfg = dict(workloads.get_config(name))
    cfg["verify"] = m
    return B.Plan(cfg, device=dev, n_tokens=m), cfg


@pytest.mark.parametrize("name,m", CASES)
def test_verify_plan_drains_and_covers(name, m):
    p, cfg = vplan(name, m)
    tasks = p.tasks()
    order = simulate(p)
    assert sorted(order) == sorted(t["id"] for t in tasks)
    r = cfg["n_q_heads"] // cfg["n_kv_heads"]
    n_blocks = math.ceil(m * r / 8)  # attention column blocks per split
    hd, d = cfg["head_dim"], cfg["hidden"]
    expect = {"QKV": (r + 2) * hd // 2, "ATTN": cfg["kv_len"] + m, "OPROJ_G": d, "GATEUP": cfg["ffn"], "DOWN": d,
              "HINIT": d, "LMHEAD": cfg["vocab"]}
    cov = collections.defaultdict(list)
    for t in tasks:
        ty = B.TASK_TYPES[t["type"]]
        grp = t["aux0"] if ty in ("QKV", "OPROJ_G") else (t["aux0"], t["aux3"]) if ty == "ATTN" else 0
        cov[(t["layer"], ty, grp)].append((t["unit_begin"], t["unit_end"]))
        rows = t["unit_end"] - t["unit_begin"]
        # each GEMV task keeps m results per row in the 1024-float LDS row table
        if ty in ("QKV", "GATEUP"):
            assert 2 * rows * m <= 1024, (ty, rows)
        elif ty in ("OPROJ_G", "DOWN", "LMHEAD"):
            assert rows * m <= 1024, (ty, rows)
        if ty == "ATTN":
            assert 0 <= t["aux3"] < n_blocks
            assert t["kv_staged"] == 0  # no K/V staging by the QKV task in a verification step
    for (layer, ty, grp), rs in cov.items():
        rs.sort()
        at = 0
        for a, b in rs:
            assert a == at and b > a, (layer, ty, grp)
            at = b
        assert at == expect[ty], (layer, ty, grp)
    for layer in range(cfg["n_layers"]):
        for g in range(cfg["n_kv_heads"]):
            blocks = {k[2][1] for k in cov if k[0] == layer and k[1] == "ATTN" and k[2][0] == g}
            assert blocks == set(range(n_blocks))


@pytest.mark.parametrize("name,m", CASES)
def test_verify_plan_sizes(name, m):
    p, cfg = vplan(name, m)
    s = p.sizes()
    assert workloads.n_tokens(cfg) == m
    assert s["x_bytes"] == math.prod(workloads.x_shape(cfg)) * 2 == m * cfg["hidden"] * 2
    assert s["out_bytes"] == math.prod(workloads.out_shape(cfg)) * 4 == m * cfg["vocab"] * 4
    assert s["kv_bytes"] == math.prod(workloads.kv_shape(cfg)) * 2
    kv_row = 2 * cfg["n_kv_heads"] * cfg["head_dim"] * 2
    assert s["algorithmic_bytes_per_step"] == s["weight_bytes"] + cfg["n_layers"] * (cfg["kv_len"] + m) * kv_row
    assert p.grid()[2] <= 160 * 1024
    bufs = p.buffers()
    assert bufs["layers.0.q"]["count"] == m * cfg["n_q_heads"] * cfg["head_dim"]
    assert bufs["layers.0.x_out"]["count"] == m * cfg["hidden"]
    assert bufs["layers.0.h"]["count"] == m * cfg["hidden"]


def test_verify_column_blocks_share_an_xcd():
    """The column blocks of one attention split read the same K/V rows: they run on one XCD."""
    p, cfg = vplan("8b_4k", 4)
    split_xcd = collections.defaultdict(set)
    for t in p.tasks():
        if B.TASK_TYPES[t["type"]] == "ATTN":
            split_xcd[(t["layer"], t["aux0"], t["aux1"])].add(t["xcd"])
    assert split_xcd and all(len(v) == 1 for v in split_xcd.values())


def test_one_token_verify_plan_is_the_decode_plan():
    cfg = workloads.get_config("small_gqa")
    a = B.Plan(cfg, device=MI355X).tasks()
    b = B.Plan(cfg, device=MI355X, n_tokens=1).tasks()
    assert a == b


@pytest.mark.parametrize("name,m,status", [
    ("tiny", 0, "DEC_E_INVAL"), ("tiny", 5, "DEC_E_INVAL"), ("mla_tiny", 2, "DEC_E_SHAPE"),
    ("moe_tiny", 2, "DEC_E_SHAPE"), ("tiny_fp8", 2, "DEC_E_SHAPE")])
def test_verify_plan_errors(name, m, status):
    with pytest.raises(B.DecError) as e:
        vplan(name, m)
    assert B.STATUS[e.value.status] == status


def test_verify_plan_rejects_a_dynamic_length():
    with pytest.raises(ValueError):
        B.Plan(workloads.get_config("tiny"), device=MI355X, max_len=100, n_tokens=2)
