"""Host-side tests of the C ABI and the ahead-of-time planner (no GPU needed).

The library is loaded and its planner runs on a described device (dec_plan_create_for), so
these run on a machine without a GPU. No compute entry point is called here.
"""
import collections
import os
import re

import pytest

import workloads
from persistent_tile_scheduled_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MI355X = B.device_info()
GQA_CONFIGS = ["tiny", "tiny_gain", "tiny_kv0", "tiny_mha_ragged", "small_gqa", "8b_4k", "8b_32k", "tiny_hd256_g3",
               "tiny_fp8", "tiny_ragged_fp8", "small_gqa_fp8", "8b_4k_fp8"]
MLA_CONFIGS = ["mla_tiny", "mla_small", "mla_8k", "moe_tiny", "moe_small", "moe_4k", "moe_wide_tiny", "moe_max_route",
               "moe_tiny_mxfp4", "moe_small_mxfp4", "moe_4k_mxfp4", "moe_max_route_mxfp4",
               "mla_tiny_fp8", "mla_small_fp8", "mla_8k_fp8", "moe_tiny_fp8", "moe_small_fp8", "moe_4k_fp8",
               "mla_tiny_sparse", "mla_small_sparse", "moe_tiny_sparse", "mla_32k_sparse"]


def plan(name, dev=MI355X, **over):
    cfg = dict(workloads.get_config(name))
    cfg.update(over)
    return B.Plan(cfg, device=dev), cfg


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "dec.h")).read()
    declared = set(re.findall(r"^\s*(?:dec_status|int64_t|const char\*)\s+(dec_\w+)\s*\(", hdr, re.M))
    assert len(declared) >= 20
    L = B.lib()
    for name in sorted(declared):
        assert hasattr(L, name), name
    assert declared == set(B.ABI_SYMBOLS)


@pytest.mark.parametrize("name", GQA_CONFIGS + MLA_CONFIGS)
def test_weight_list_matches_input_layout(name):
    p, cfg = plan(name)
    got = [(d["name"], d["shape"], d["dtype"]) for d in p.weight_descs()]
    want = [(s.name, s.shape, s.dtype) for s in workloads.weight_specs(cfg)]
    assert got == want
    assert p.sizes()["weight_bytes"] == sum(s.nbytes for s in workloads.weight_specs(cfg))


def test_algorithmic_bytes():
    # weights once + KV positions [0, kv_len] once (the step attends over kv_len + 1 positions)
    p, cfg = plan("8b_4k")
    s = p.sizes()
    assert s["weight_bytes"] == 15_009_849_344
    assert s["algorithmic_bytes_per_step"] == 15_009_849_344 + 32 * 2 * 8 * 4097 * 128 * 2
    p, cfg = plan("8b_32k")
    assert p.sizes()["algorithmic_bytes_per_step"] == 15_009_849_344 + 32 * 2 * 8 * 32769 * 128 * 2
    assert p.sizes()["kv_bytes"] == 32 * 2 * 8 * 32769 * 128 * 2


@pytest.mark.parametrize("over,status", [
    ({"hidden": 260}, "DEC_E_SHAPE"),
    ({"n_q_heads": 6, "n_kv_heads": 4}, "DEC_E_SHAPE"),
    ({"n_q_heads": 16, "n_kv_heads": 2}, "DEC_E_SHAPE"),     # 8 q heads per KV head: unsupported
    ({"head_dim": 48}, "DEC_E_SHAPE"),
    ({"ffn": 0}, "DEC_E_SHAPE"),
    ({"rms_eps": 0.0}, "DEC_E_SHAPE"),
    ({"kv_len": -1}, "DEC_E_CAPACITY"),
    ({"q_lora_rank": 64}, "DEC_E_SHAPE"),                      # MLA field on a GQA shape
])
def test_shape_errors(over, status):
    with pytest.raises(B.DecError) as e:
        plan("tiny", **over)
    assert B.STATUS[e.value.status] == status


def test_abi_version_and_device_errors():
    cfg = workloads.get_config("tiny")
    s = B.shape_from_config(cfg)
    s.abi_version = 99
    with pytest.raises(B.DecError) as e:
        B.Plan(s, 128, device=MI355X)
    assert B.STATUS[e.value.status] == "DEC_E_INVAL"
    with pytest.raises(B.DecError) as e:
        plan("tiny", dev=B.device_info(gfx_arch=942))
    assert B.STATUS[e.value.status] == "DEC_E_DEVICE"
    with pytest.raises(B.DecError) as e:
        plan("tiny", dev=B.device_info(lds=64 * 1024))
    assert B.STATUS[e.value.status] == "DEC_E_OCCUPANCY"
    with pytest.raises(B.DecError) as e:
        plan("tiny", dev=B.device_info(max_threads=256))
    assert B.STATUS[e.value.status] == "DEC_E_OCCUPANCY"


def test_step_before_bind_and_null_arguments():
    p, _ = plan("tiny")
    with pytest.raises(B.DecError) as e:
        p.step(0x1000, 0x1000, 0x1000)
    assert B.STATUS[e.value.status] == "DEC_E_UNBOUND"
    L = B.lib()
    import ctypes as C
    assert L.dec_plan_create(None, 0, None) == -1
    assert L.dec_plan_destroy(None) == 0
    with pytest.raises(B.DecError) as e:
        p.bind([0] * len(p.weight_descs()), 0, 0)
    assert B.STATUS[e.value.status] == "DEC_E_INVAL"
    with pytest.raises(B.DecError) as e:
        p.bind([0x100] * 3, 0x1000, 1 << 30)
    assert B.STATUS[e.value.status] == "DEC_E_INVAL"
    with pytest.raises(B.DecError) as e:
        p.set_watchdog(0)
    assert B.STATUS[e.value.status] == "DEC_E_INVAL"


def _expected_units(cfg, ttype):
    n1 = cfg["kv_len"] + 1
    g = cfg.get
    return {
        "QKV": (cfg["n_q_heads"] // max(g("n_kv_heads", 1), 1) + 2) * g("head_dim", 0) // 2,
        "ATTN": n1, "OPROJ": cfg["hidden"], "OPROJ_G": cfg["hidden"], "DOWN": cfg["hidden"],
        "GATEUP": g("ffn", 0), "HINIT": cfg["hidden"],
        "LMHEAD": cfg["vocab"],
        # MLA: [W_DQ; W_DKV] rows, W_UQ row pairs, the latent row, (head, 64-column) blocks
        "MLA_A": g("q_lora_rank", 0) + g("kv_lora_rank", 0) + g("qk_rope", 0) + (g("index_dim", 0) + g("index_heads", 0) if g("index_heads", 0) else 0),
        "MLA_B": cfg["n_q_heads"] * (g("qk_nope", 0) // 2 + g("qk_rope", 0) // 2),
        "MLA_KVAPP": g("kv_lora_rank", 0) + g("qk_rope", 0),
        "MLA_ABSORB": cfg["n_q_heads"] * g("kv_lora_rank", 0) // 64,
        "MLA_UV": cfg["n_q_heads"] * g("kv_lora_rank", 0) // 64,
        "MLA_ATTN": min(n1, g("index_topk", 0)) if g("index_heads", 0) else n1,  # (with the indexer: entries of the selected list)
        # the sparse indexer: index-query rows, scored positions, the one top-T task
        "IDX_Q": g("index_heads", 0) * g("index_dim", 0), "IDX_SCORE": n1, "IDX_TOPK": n1,
        # MoE: router rows, shared gate/up pairs, the top-k over all experts, routed pairs
        "ROUTER": g("n_routed", 0), "TOPK": g("n_routed", 0),
        "SHARED_GU": g("n_shared", 0) * g("expert_ffn", 0),
        "EXPERT_GU": g("top_k", 0) * g("expert_ffn", 0), "MOE_DOWN": cfg["hidden"],
    }[ttype]


def simulate(p):
    """Run one step of the static schedule on the CPU: every workgroup walks its list in order
    and a task runs once all its counters have reached their per-step totals. Returns the
    execution order; raises if the schedule stalls (a deadlock)."""
    tasks = p.tasks()
    deps = p.deps()
    n_wg = p.grid()[0]
    lists = collections.defaultdict(list)
    for t in tasks:
        lists[t["wg"]].append(t)
    for w in lists:
        lists[w].sort(key=lambda t: t["list_pos"])
    ctr = collections.Counter()
    tickets = collections.Counter()
    pos = {w: 0 for w in range(n_wg)}
    done = []
    progress = True
    while progress:
        progress = False
        for w in range(n_wg):
            while pos[w] < len(lists[w]):
                t = lists[w][pos[w]]
                if not all(ctr[deps[t["dep_first"] + k][0]] >= deps[t["dep_first"] + k][1] for k in range(t["n_deps"])):
                    break
                if t["signal"] >= 0:
                    ctr[t["signal"]] += 1
                if t["signal2"] >= 0:  # ticket merge: the last of the group's splits signals
                    tickets[t["signal"]] += 1
                    n_splits = sum(1 for u in tasks if u["signal"] == t["signal"])
                    if tickets[t["signal"]] == n_splits:
                        ctr[t["signal2"]] += 1
                done.append(t["id"])
                pos[w] += 1
                progress = True
    stuck = [w for w in range(n_wg) if pos[w] < len(lists[w])]
    if stuck:
        raise AssertionError(f"schedule stalls: {len(stuck)} workgroups blocked")
    return done


STAGES = {
    "gqa": ("QKV", "ATTN", "OPROJ_G", "GATEUP", "DOWN"),
    "mla": ("MLA_A", "MLA_B", "MLA_KVAPP", "MLA_ABSORB", "MLA_ATTN", "MLA_UV", "OPROJ", "GATEUP", "DOWN"),
    "moe": ("MLA_A", "MLA_B", "MLA_KVAPP", "MLA_ABSORB", "MLA_ATTN", "MLA_UV", "OPROJ", "ROUTER", "SHARED_GU",
            "TOPK", "EXPERT_GU", "MOE_DOWN"),
}


@pytest.mark.parametrize("name", ["tiny", "tiny_kv0", "tiny_mha_ragged", "small_gqa", "8b_4k"] + MLA_CONFIGS)
def test_schedule_drains_and_covers(name):
    p, cfg = plan(name)
    tasks = p.tasks()
    order = simulate(p)
    assert sorted(order) == sorted(t["id"] for t in tasks)  # each task exactly once
    # unit coverage per (layer, type, group): ranges tile [0, expected) exactly once
    cov = collections.defaultdict(list)
    for t in tasks:
        ty = B.TASK_TYPES[t["type"]]
        grp = t["aux0"] if ty in ("QKV", "ATTN", "OPROJ_G") else 0
        cov[(t["layer"], ty, grp)].append((t["unit_begin"], t["unit_end"]))
    for (layer, ty, grp), rs in cov.items():
        rs.sort()
        at = 0
        for a, b in rs:
            assert a == at and b > a, (layer, ty, grp)
            at = b
        assert at == _expected_units(cfg, ty), (layer, ty)
    n_layers = cfg["n_layers"]
    for layer in range(n_layers):
        for ty in STAGES[cfg["arch"]]:
            assert (layer, ty, 0) in cov, (layer, ty)
    if cfg["vocab"] > 0:
        assert (n_layers, "LMHEAD", 0) in cov
    else:
        assert not any(k[1] == "LMHEAD" for k in cov)


def test_lists_in_stage_order_and_deps_point_back():
    p, _ = plan("small_gqa")
    tasks = p.tasks()
    deps = p.deps()
    producers = collections.defaultdict(list)
    for t in tasks:
        if t["signal"] >= 0:
            producers[t["signal"]].append(t)
        if t["signal2"] >= 0:
            producers[t["signal2"]].append(t)
    by_wg = collections.defaultdict(list)
    for t in tasks:
        by_wg[t["wg"]].append(t)
    for w, lst in by_wg.items():
        lst.sort(key=lambda t: t["list_pos"])
        assert [t["stage"] for t in lst] == sorted(t["stage"] for t in lst)
    for t in tasks:
        for k in range(t["n_deps"]):
            c, total = deps[t["dep_first"] + k]
            assert producers[c], "waits on a counter nobody signals"
            assert all(pt["stage"] < t["stage"] for pt in producers[c])
            n_sig = sum(1 for pt in producers[c] if pt["signal"] == c)
            assert total == (1 if n_sig == 0 else n_sig)


@pytest.mark.parametrize("name", ["tiny", "8b_4k", "mla_small", "moe_small"])
def test_stage_count_for_stage_launches(name):
    """dec_step_stages launches stage ranges: the plan's stage count covers every task's
    stage, every stage holds tasks, and a one-stage launch never waits on its own tasks
    (the dependency check above, over all configurations' stage numbers)."""
    p, _ = plan(name)
    tasks = p.tasks()
    ns = p.n_stages()
    stages = {t["stage"] for t in tasks}
    assert ns == max(stages) + 1
    assert stages == set(range(ns))
    producers = collections.defaultdict(list)
    for t in tasks:
        for c in (t["signal"], t["signal2"]):
            if c >= 0:
                producers[c].append(t["stage"])
    deps = p.deps()
    for t in tasks:
        for k in range(t["n_deps"]):
            c, _ = deps[t["dep_first"] + k]
            assert max(producers[c]) < t["stage"]


@pytest.mark.parametrize("name,max_len", [("tiny", 200), ("small_gqa", 3000), ("8b_4k", 4096), ("8b_32k", 32768)])
def test_dynamic_plan_layout(name, max_len):
    """A plan with a per-step length: the fixed plan's weight list plus the token embedding
    (when there is an LM head), the cache sized for max_len + 1 slots, the LM-head tasks
    signalling one argmax task that comes last, and the attention splits planned over
    max_len + 1 positions (staged in LDS where the largest split fits)."""
    cfg = dict(workloads.get_config(name))
    p = B.Plan(cfg, device=MI355X, max_len=max_len)
    fixed = B.Plan(dict(cfg, kv_len=max_len), device=MI355X)
    names = [d["name"] for d in p.weight_descs()]
    want = [d["name"] for d in fixed.weight_descs()] + (["embed"] if cfg["vocab"] > 0 else [])
    assert names == want
    if cfg["vocab"] > 0:
        e = p.weight_descs()[-1]
        assert tuple(e["shape"]) == (cfg["vocab"], cfg["hidden"]) and e["dtype"] == "bf16"
    sz = p.sizes()
    assert sz["kv_bytes"] == 2 * cfg["n_layers"] * 2 * cfg["n_kv_heads"] * (max_len + 1) * cfg["head_dim"]
    # a step reads one embedding row, not the table: the same bytes as the fixed plan plus a row
    emb_row = cfg["hidden"] * 2 if cfg["vocab"] > 0 else 0
    assert sz["algorithmic_bytes_per_step"] == fixed.sizes()["algorithmic_bytes_per_step"] + emb_row
    tasks = p.tasks()
    am = [t for t in tasks if t["type"] == 20]
    lm = [t for t in tasks if t["type"] == 6]
    if cfg["vocab"] > 0:
        assert len(am) == 1 and am[0]["stage"] == max(t["stage"] for t in tasks)
        assert all(t["signal"] >= 0 for t in lm)
        assert sorted(t["aux0"] for t in lm) == list(range(len(lm)))
        assert am[0]["aux0"] == len(lm)
    else:
        assert not am
    att = [t for t in tasks if t["type"] == 2]
    ends = sorted((t["layer"], t["aux0"], t["unit_begin"], t["unit_end"]) for t in att if t["layer"] == 0)
    assert max(e[3] for e in ends) == max_len + 1
    if name in ("8b_4k", "small_gqa"):
        assert any(t["kv_staged"] > 0 for t in att)


@pytest.mark.parametrize("name,max_len", [("mla_tiny", 300), ("moe_tiny", 100), ("mla_8k", 8192)])
def test_dynamic_latent_plan_layout(name, max_len):
    """Latent-attention plans with a per-step length: the fixed plan's weights, a latent cache
    of max_len + 1 slots, and the attention splits planned over max_len + 1 positions, split
    a1 of a2 covering [(n+1) a1 / a2, (n+1) (a1+1) / a2) at position n."""
    cfg = dict(workloads.get_config(name))
    p = B.Plan(cfg, device=MI355X, max_len=max_len)
    fixed = B.Plan(dict(cfg, kv_len=max_len), device=MI355X)
    assert [d["name"] for d in p.weight_descs()] == [d["name"] for d in fixed.weight_descs()]
    KR = cfg["kv_lora_rank"] + cfg["qk_rope"]
    assert p.sizes()["kv_bytes"] == 2 * cfg["n_layers"] * (max_len + 1) * KR
    att = sorted((t["aux1"], t["unit_begin"], t["unit_end"], t["aux2"])
                 for t in p.tasks() if t["type"] == 11 and t["layer"] == 0)
    S = att[0][3]
    assert [a[0] for a in att] == list(range(S))
    for sp, u0, u1, s_ in att:
        assert s_ == S and u0 == (max_len + 1) * sp // S and u1 == (max_len + 1) * (sp + 1) // S


def test_dynamic_plan_errors():
    with pytest.raises(B.DecError) as ei:
        B.Plan(dict(workloads.get_config("mla_tiny"), weights="mxfp4"), device=MI355X, max_len=100)  # MXFP4: MoE only
    assert ei.value.status == -2
    with pytest.raises(B.DecError):
        B.Plan(workloads.get_config("tiny"), device=MI355X, max_len=-1)


def test_fp8_weights_plan():
    """FP8 plans: each linear matrix is uint8 E4M3 followed by its fp32 row scales; the bytes
    per step drop accordingly; other families and unaligned widths are refused. A plan with a
    per-step length has the same matrices plus a bf16 token embedding."""
    p, cfg = plan("8b_4k_fp8")
    q, _ = plan("8b_4k")
    d = {x["name"]: x for x in p.weight_descs()}
    assert d["layers.0.wq"]["dtype"] == "fp8" and tuple(d["layers.0.wq.scale"]["shape"]) == (4096,)
    assert d["layers.0.attn_norm"]["dtype"] == "bf16" and d["lm_head"]["dtype"] == "fp8"
    names = [x["name"] for x in p.weight_descs()]
    assert names.index("layers.0.w_down.scale") == names.index("layers.0.w_down") + 1
    a, b = p.sizes()["algorithmic_bytes_per_step"], q.sizes()["algorithmic_bytes_per_step"]
    kv = 32 * 4097 * 2 * 8 * 128 * 2
    assert a - kv == (b - kv - sum(x["bytes"] for x in p.weight_descs() if x["dtype"] == "bf16")) // 2 + \
        sum(x["bytes"] for x in p.weight_descs() if x["dtype"] != "fp8")
    for over in [{"hidden": 520}, {"ffn": 1000}]:
        with pytest.raises(B.DecError) as ei:
            plan("tiny_fp8", **over)
        assert ei.value.status == -2
    with pytest.raises(B.DecError) as ei:
        plan("mla_tiny", weights="fp8", q_lora_rank=104)  # FP8 rows need widths that are multiples of 16
    assert ei.value.status == -2
    dyn = B.Plan(workloads.get_config("tiny_fp8"), device=MI355X, max_len=200)
    dd = {x["name"]: x for x in dyn.weight_descs()}
    assert dd["layers.0.wq"]["dtype"] == "fp8" and dd["embed"]["dtype"] == "bf16"


def test_chiplet_placement_8b():
    """Each KV-head group's QKV rows and attention splits run on the workgroups of one XCD."""
    p, cfg = plan("8b_4k")
    for t in p.tasks():
        ty = B.TASK_TYPES[t["type"]]
        if ty in ("QKV", "ATTN", "OPROJ_G"):
            assert t["xcd"] == t["aux0"], t
    # and every workgroup gets work in every dense stage
    per_stage = collections.defaultdict(set)
    for t in p.tasks():
        per_stage[(t["layer"], B.TASK_TYPES[t["type"]])].add(t["wg"])
    for (layer, ty), wgs in per_stage.items():
        if ty in ("OPROJ_G", "GATEUP", "DOWN", "QKV", "ATTN", "LMHEAD"):
            assert len(wgs) == 256, (layer, ty, len(wgs))


@pytest.mark.parametrize("n_cu,n_xcd", [(64, 2), (80, 4), (8, 8), (304, 8)])
def test_other_device_shapes(n_cu, n_xcd):
    p, cfg = plan("small_gqa", dev=B.device_info(n_cu=n_cu, n_xcd=n_xcd))
    assert p.grid()[0] == n_cu
    simulate(p)


def test_buffers_cover_trace():
    p, cfg = plan("tiny")
    bufs = p.buffers()
    for l in range(cfg["n_layers"]):
        for nm in ("q", "kv_new", "attn", "h", "ffn_act", "ffn_out", "x_out"):
            assert f"layers.{l}.{nm}" in bufs
    ws = p.sizes()["workspace_bytes"]
    for b in bufs.values():
        assert b["offset"] % 256 == 0 and b["offset"] + b["count"] * 4 <= ws


@pytest.mark.parametrize("over,status", [
    ({"n_q_heads": 17}, "DEC_E_SHAPE"),          # more heads than one MFMA tile folds
    ({"kv_lora_rank": 96}, "DEC_E_SHAPE"),       # latent width not a multiple of 64
    ({"kv_lora_rank": 1024}, "DEC_E_SHAPE"),     # above 512
    ({"qk_rope": 12}, "DEC_E_SHAPE"),
    ({"v_head": 12}, "DEC_E_SHAPE"),
    ({"head_dim": 64}, "DEC_E_SHAPE"),            # GQA field on an MLA shape
    ({"n_routed": 16}, "DEC_E_SHAPE"),            # MoE field on a dense MLA shape
])
def test_mla_shape_errors(over, status):
    with pytest.raises(B.DecError) as e:
        plan("mla_tiny", **over)
    assert B.STATUS[e.value.status] == status


@pytest.mark.parametrize("over", [{"top_k": 17}, {"top_k": 0}, {"expert_ffn": 12}, {"ffn": 64}])
def test_moe_shape_errors(over):
    with pytest.raises(B.DecError) as e:
        plan("moe_tiny", **over)
    assert B.STATUS[e.value.status] == "DEC_E_SHAPE"


def test_mla_algorithmic_bytes():
    """MLA: every weight once + latent rows [0, kv_len]; MoE: routed experts count top_k of
    n_routed per layer."""
    p, cfg = plan("mla_8k")
    s = p.sizes()
    row = (cfg["kv_lora_rank"] + cfg["qk_rope"]) * 2
    assert s["algorithmic_bytes_per_step"] == s["weight_bytes"] + cfg["n_layers"] * (cfg["kv_len"] + 1) * row
    assert s["kv_bytes"] == cfg["n_layers"] * (cfg["kv_len"] + 1) * row
    p, cfg = plan("moe_4k")
    s = p.sizes()
    per_expert = 3 * cfg["expert_ffn"] * cfg["hidden"] * 2
    unused = cfg["n_layers"] * (cfg["n_routed"] - cfg["top_k"]) * per_expert
    row = (cfg["kv_lora_rank"] + cfg["qk_rope"]) * 2
    assert s["algorithmic_bytes_per_step"] == s["weight_bytes"] - unused + cfg["n_layers"] * (cfg["kv_len"] + 1) * row
    # MXFP4 experts: half a byte per element plus one scale byte per 32
    p, cfg = plan("moe_4k_mxfp4")
    s = p.sizes()
    per_expert = 3 * cfg["expert_ffn"] * cfg["hidden"] // 2 + 3 * cfg["expert_ffn"] * cfg["hidden"] // 32
    unused = cfg["n_layers"] * (cfg["n_routed"] - cfg["top_k"]) * per_expert
    assert s["algorithmic_bytes_per_step"] == s["weight_bytes"] - unused + cfg["n_layers"] * (cfg["kv_len"] + 1) * row


def test_fp8_latent_plan():
    """FP8 latent-family plans: every linear matrix but w_uk, w_uv and the router is E4M3
    bytes followed by fp32 row scales (one per row of every expert); the bytes per step count
    the chosen experts' bytes and scales."""
    p, cfg = plan("moe_4k_fp8")
    d = {x["name"]: x for x in p.weight_descs()}
    E, F, H = cfg["n_routed"], cfg["expert_ffn"], cfg["hidden"]
    for n in ("wq_a", "wq_b", "wkv_a", "wo", "experts.w_gate", "shared.w_down"):
        assert d["layers.0." + n]["dtype"] == "fp8" and d["layers.0." + n + ".scale"]["dtype"] == "fp32", n
    for n in ("w_uk", "w_uv", "router"):
        assert d["layers.0." + n]["dtype"] == "bf16", n
    assert tuple(d["layers.0.experts.w_down.scale"]["shape"]) == (E, H)
    s = p.sizes()
    per_expert = 3 * F * H + 2 * F * 4 + H * 4
    unused = cfg["n_layers"] * (E - cfg["top_k"]) * per_expert
    row = (cfg["kv_lora_rank"] + cfg["qk_rope"]) * 2
    assert s["algorithmic_bytes_per_step"] == s["weight_bytes"] - unused + cfg["n_layers"] * (cfg["kv_len"] + 1) * row


def test_sparse_indexer_plan():
    """Sparse-indexer plans: the indexer's three matrices after wo, a cache row of latent plus
    index key, the index tasks in their own stages, attention splits over the selected list,
    and the bytes per step counting every index key but only the selected latent rows."""
    p, cfg = plan("mla_32k_sparse")
    d = {x["name"]: x for x in p.weight_descs()}
    H, DI, T, n = cfg["index_heads"], cfg["index_dim"], cfg["index_topk"], cfg["kv_len"]
    assert tuple(d["layers.0.idx_wq"]["shape"]) == (H * DI, cfg["q_lora_rank"])
    assert tuple(d["layers.0.idx_wk"]["shape"]) == (DI, cfg["hidden"]) and tuple(d["layers.0.idx_w"]["shape"]) == (H, cfg["hidden"])
    KR = cfg["kv_lora_rank"] + cfg["qk_rope"]
    s = p.sizes()
    assert s["kv_bytes"] == cfg["n_layers"] * (n + 1) * (KR + DI) * 2
    assert s["algorithmic_bytes_per_step"] == s["weight_bytes"] + cfg["n_layers"] * ((n + 1) * DI * 2 + T * KR * 2)
    tasks = p.tasks()
    stage = {ty: {t["stage"] for t in tasks if t["type"] == ty and t["layer"] == 0} for ty in (7, 21, 22, 23, 11)}
    assert max(stage[7]) < min(stage[21]) and max(stage[21]) < min(stage[22]) < min(stage[23]) < min(stage[11])
    att = sorted((t["unit_begin"], t["unit_end"]) for t in tasks if t["type"] == 11 and t["layer"] == 0)
    assert att[0][0] == 0 and att[-1][1] == T and len(att) == T // 16
    top = [t for t in tasks if t["type"] == 23 and t["layer"] == 0]
    assert len(top) == 1
    # the splits of the selected list go to the XCDs in turn, on distinct workgroups, and no
    # absorb task (which every split waits for) sits behind the selection on its workgroup
    att_t = sorted((t for t in tasks if t["type"] == 11 and t["layer"] == 0), key=lambda t: t["aux1"])
    assert [t["xcd"] for t in att_t] == [i % 8 for i in range(len(att_t))]
    assert len({t["wg"] for t in att_t}) == len(att_t) and top[0]["wg"] not in {t["wg"] for t in att_t}
    assert all(t["wg"] != top[0]["wg"] for t in tasks if t["type"] == 10)
    for name, over in [("tiny", {"index_heads": 4, "index_dim": 32, "index_topk": 8}),
                       ("mla_tiny_sparse", {"index_dim": 48}), ("mla_tiny_sparse", {"index_heads": 80}),
                       ("mla_tiny_sparse", {"weights": "fp8"}), ("mla_tiny", {"index_topk": 8})]:
        with pytest.raises(B.DecError) as ei:
            plan(name, **over)
        assert ei.value.status == -2, (name, over)


def test_mxfp4_expert_plan():
    """MXFP4 expert plans: each expert matrix (routed and shared) is packed E2M1 pairs
    [.., cols / 2] followed by its E8M0 scales [.., cols / 32]; every other weight stays bf16;
    other families and widths that are not multiples of 32 are refused."""
    p, cfg = plan("moe_4k_mxfp4")
    d = {x["name"]: x for x in p.weight_descs()}
    names = [x["name"] for x in p.weight_descs()]
    E, F, H = cfg["n_routed"], cfg["expert_ffn"], cfg["hidden"]
    assert d["layers.0.experts.w_gate"]["dtype"] == "fp4x2" and tuple(d["layers.0.experts.w_gate"]["shape"]) == (E, F, H // 2)
    assert d["layers.0.experts.w_down.scale"]["dtype"] == "e8m0" and tuple(d["layers.0.experts.w_down.scale"]["shape"]) == (E, H, F // 32)
    assert tuple(d["layers.0.shared.w_down"]["shape"]) == (H, F // 2)
    assert names.index("layers.0.shared.w_up.scale") == names.index("layers.0.shared.w_up") + 1
    assert d["layers.0.router"]["dtype"] == "bf16" and d["layers.0.wq_a"]["dtype"] == "bf16"
    for name, over in [("moe_tiny_mxfp4", {"expert_ffn": 48}), ("moe_tiny_mxfp4", {"hidden": 264}), ("mla_tiny", {"weights": "mxfp4"}),
                       ("tiny", {"weights": "mxfp4"})]:
        with pytest.raises(B.DecError) as ei:
            plan(name, **over)
        assert ei.value.status == -2


def test_mla_attention_splits():
    """Latent attention splits tile the positions, at least 64 per split where the cache
    allows, at most one per workgroup, and the W_UV merge tasks cover every (head, block)."""
    for name in ("mla_tiny", "mla_8k", "moe_4k"):
        p, cfg = plan(name)
        n1 = cfg["kv_len"] + 1
        for layer in range(cfg["n_layers"]):
            sp = sorted((t["unit_begin"], t["unit_end"]) for t in p.tasks()
                        if t["layer"] == layer and B.TASK_TYPES[t["type"]] == "MLA_ATTN")
            S = len(sp)
            assert S == min(256, max(1, -(-n1 // 64)))
            assert sp[0][0] == 0 and sp[-1][1] == n1
            assert len({t["wg"] for t in p.tasks() if t["layer"] == layer and B.TASK_TYPES[t["type"]] == "MLA_ATTN"}) == S


def test_moe_topk_after_router_on_one_workgroup():
    p, cfg = plan("moe_4k")
    tasks = p.tasks()
    for layer in range(cfg["n_layers"]):
        tk = [t for t in tasks if t["layer"] == layer and B.TASK_TYPES[t["type"]] == "TOPK"]
        assert len(tk) == 1
        routers = [t for t in tasks if t["layer"] == layer and B.TASK_TYPES[t["type"]] == "ROUTER"]
        assert tk[0]["wg"] == max(t["wg"] for t in routers)
        # the routed-expert tasks wait for the top-k first (aux2 = 1 leading dependency), so
        # they can prefetch their rows before the rest of their wait
        deps = p.deps()
        for t in tasks:
            if t["layer"] == layer and B.TASK_TYPES[t["type"]] in ("EXPERT_GU", "MOE_DOWN"):
                assert t["aux2"] == 1 and deps[t["dep_first"]][0] == tk[0]["signal"], t


def test_mla_append_runs_alone():
    """The latent-cache append's workgroup has no W_UQ rows in the same stage."""
    p, cfg = plan("mla_8k")
    for layer in range(cfg["n_layers"]):
        app = [t for t in p.tasks() if t["layer"] == layer and B.TASK_TYPES[t["type"]] == "MLA_KVAPP"]
        assert len(app) == 1
        assert not any(t["wg"] == app[0]["wg"] and t["layer"] == layer and B.TASK_TYPES[t["type"]] == "MLA_B"
                       for t in p.tasks())


@pytest.mark.parametrize("name,expect", [("8b_4k", "all"), ("small_gqa", "all"), ("tiny_mha_ragged", "some"),
                                         ("8b_32k", "none"), ("tiny_kv0", "none")])
def test_attention_kv_staging(name, expect):
    """A staged attention split directly follows, in its workgroup's list, the QKV task that
    copies its cached K/V rows into LDS; the rows staged are exactly the split's cached
    positions (the new position, if the split holds it, is the one row left)."""
    p, cfg = plan(name)
    n = cfg["kv_len"]
    tasks = sorted(p.tasks(), key=lambda t: (t["wg"], t["list_pos"]))
    att = [t for t in tasks if B.TASK_TYPES[t["type"]] == "ATTN"]
    staged = 0
    for i, t in enumerate(tasks):
        if B.TASK_TYPES[t["type"]] != "ATTN" or t["kv_staged"] == 0:
            continue
        staged += 1
        q = tasks[i - 1]
        assert q["wg"] == t["wg"] and B.TASK_TYPES[q["type"]] == "QKV" and q["layer"] == t["layer"]
        assert q["kv_staged"] == t["kv_staged"] == min(t["unit_end"], n) - t["unit_begin"]
    n_qkv = sum(1 for t in tasks if B.TASK_TYPES[t["type"]] == "QKV" and t["kv_staged"] > 0)
    assert n_qkv == staged
    if expect == "all":
        assert staged == len(att)
    elif expect == "some":
        assert 0 < staged < len(att)
    else:
        assert staged == 0


@pytest.mark.parametrize("n_cu,n_xcd", [(80, 8), (96, 4), (64, 1), (304, 8), (7, 1)])
def test_sparse_plans_on_other_devices(n_cu, n_xcd):
    """Sparse-indexer plans for other compute-unit and XCD counts: the schedule drains, every
    task runs once, and the attention splits of the selected list sit on distinct workgroups."""
    dev = B.device_info(n_cu=n_cu, n_xcd=n_xcd)
    for name in ("mla_tiny_sparse", "moe_tiny_sparse", "mla_32k_sparse"):
        p = B.Plan(workloads.get_config(name), device=dev)
        tasks = p.tasks()
        assert sorted(simulate(p)) == sorted(t["id"] for t in tasks), name
        att = [t["wg"] for t in tasks if B.TASK_TYPES[t["type"]] == "MLA_ATTN" and t["layer"] == 0]
        assert att and len(set(att)) == len(att) and max(att) < n_cu, name
