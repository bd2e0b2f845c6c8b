"""GPU parity of the sparse indexer (latent family; reading R24) against the fp64 oracle.

The selection is integer work decided in fp32: the engine's selected positions must equal the
oracle's rule (top T by score, ties to the lower position, increasing order) applied to the
engine's own scores, exactly; the engine's scores must match the oracle's within the tight bar;
and the engine's selection must equal the oracle's own wherever the score gap at the boundary
exceeds what fp32 scores can move. The rest of the layer is then compared with the oracle run on
the engine's selection (several selections are correct at a near-tie; the layer's values are
unique given one), every trace vector at the tight bar, plus the appended index key's bf16 bits.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from oracle import decode_oracle as D
from test_gpu_parity import HostWeights, LOGIT_TOL, TIGHT_TOL, _slot_close, check_coverage, check_kv_slot, rel_l2
from test_gpu_parity_mla import DENSE_FFN, MLA_TRACE, MOE_FFN, check_moe_layer

pytestmark = pytest.mark.gpu

MARGIN = 1e-4  # relative score gap at the selection boundary above which the fp64 oracle must agree


def _engine(cfg, w, **kw):
    from persistent_tile_scheduled_amd.engine import DecodeEngine
    return DecodeEngine(cfg, w, **kw)


def check_sparse_layer(eng, cfg, W, l, xin, kvl, n):
    """Layer l from the engine's own layer input xin and the cache rows kvl (bf16 bits after the
    step). Returns the max relative error over the trace."""
    T = cfg["index_topk"]
    sc = eng.buffer(f"layers.{l}.idx_scores").cpu().numpy()[: n + 1]
    sel = eng.buffer(f"layers.{l}.idx_sel").cpu().view(torch.int32).numpy()[: min(T, n + 1)].astype(np.int64)
    assert np.array_equal(sel, O.select_positions(sc, T)), (l, "selection is not the rule on the engine's scores")
    _, t = O.mla_layer(cfg, W, l, xin, kvl, n)
    errs = {"idx_scores": rel_l2(sc, t["idx_scores"])}
    for nm in ("idx_q", "idx_w", "idx_k"):
        errs[nm] = rel_l2(eng.buffer(f"layers.{l}.{nm}").cpu().numpy()[: t[nm].size], t[nm])
    if t["idx_margin"][0] > MARGIN:
        assert np.array_equal(sel, t["idx_sel"]), (l, "selection differs from the oracle's at margin", t["idx_margin"][0])
    else:
        print(f"[sparse] layer {l}: near-tie at the boundary (margin {t['idx_margin'][0]:.2e})", flush=True)
    # the rest of the layer from the engine's selection
    real = D.select_positions
    try:
        D.select_positions = lambda s, T_: sel
        _, t = O.mla_layer(cfg, W, l, xin, kvl, n)
    finally:
        D.select_positions = real
    names = MLA_TRACE + (DENSE_FFN if cfg["arch"] == "mla" else MOE_FFN)
    for nm in names:
        errs[nm] = rel_l2(eng.buffer(f"layers.{l}.{nm}").cpu().numpy()[: t[nm].size], t[nm])
    bad = {k: v for k, v in errs.items() if v > TIGHT_TOL}
    assert not bad, (l, bad)
    KR = cfg["kv_lora_rank"] + cfg["qk_rope"]
    _slot_close(kvl[n, KR:KR + cfg["index_dim"]], t["idx_k_bits"], ("index key", l))
    check_kv_slot(cfg, kvl[None, :, :KR], 0, t)
    if cfg["arch"] == "moe":
        check_moe_layer(eng, cfg, l, t, W)
    return max(errs.values())


def _layer_inputs(eng, x, l):
    return (O.widen_bf16(workloads.bf16_bits(x)) if l == 0
            else eng.buffer(f"layers.{l - 1}.x_out").cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("name,seed,kv_len", [("mla_tiny_sparse", 0, None),   # 48 of 101 positions
                                              ("mla_tiny_sparse", 1, 30),     # 31 positions, T = 48: all of them
                                              ("mla_tiny_sparse", 2, 47),     # exactly T
                                              ("mla_small_sparse", 0, None),  # 256 of 778
                                              ("moe_tiny_sparse", 0, None)])  # with the MoE FFN
def test_sparse_parity(name, seed, kv_len):
    cfg = dict(workloads.get_config(name))
    if kv_len is not None:
        cfg["kv_len"] = kv_len
    n = cfg["kv_len"]
    print(f"[sparse] {name} seed={seed} kv_len={n}", flush=True)
    w, x, kv = workloads.generate(cfg, seed=seed, device="cuda")
    eng = _engine(cfg, w)
    out = eng.step(x, kv)
    torch.cuda.synchronize()
    eng.status()
    W = HostWeights(w)
    for l in range(cfg["n_layers"]):
        e = check_sparse_layer(eng, cfg, W, l, _layer_inputs(eng, x, l), workloads.bf16_bits(kv[l]), n)
        print(f"[sparse] layer {l}: max rel error {e:.2e}", flush=True)
    xo = eng.buffer(f"layers.{cfg['n_layers'] - 1}.x_out").cpu().numpy()
    assert np.array_equal(out.cpu().numpy(), xo)
    check_coverage(eng)


def test_sparse_32k_every_layer():
    """The full-size MLA stack at 32768 positions with 64 index heads keeping 2048 positions, in
    the bench's launch configuration."""
    cfg = workloads.get_config("mla_32k_sparse")
    n = cfg["kv_len"]
    print("[sparse] mla_32k_sparse: generating", flush=True)
    w, x, kv = workloads.generate(cfg, seed=0, device="cuda")
    eng = _engine(cfg, w)
    eng.step(x, kv)
    torch.cuda.synchronize()
    eng.status()
    W = HostWeights(w)
    for l in range(cfg["n_layers"]):
        e = check_sparse_layer(eng, cfg, W, l, _layer_inputs(eng, x, l), workloads.bf16_bits(kv[l]), n)
        print(f"[sparse] mla_32k_sparse layer {l}: max rel error {e:.2e}", flush=True)
        W.drop(f"layers.{l}.")
    check_coverage(eng)


def test_sparse_plan_with_per_step_length():
    """One plan for positions up to 300 (T = 48): positions below and at T (everything is
    selected), just above, and the largest."""
    cfg = workloads.get_config("mla_tiny_sparse")
    M = 300
    w, x, kv = workloads.generate(cfg, seed=9, device="cuda", kv_len=M)
    eng = _engine(cfg, w, max_len=M)
    W = HostWeights(w)
    for p in [0, 20, 47, 48, 150, M]:
        print(f"[sparse] dynamic position {p}", flush=True)
        eng.set_state(p, 0)
        eng.step_dynamic(kv, x)
        torch.cuda.synchronize()
        eng.status()
        cfg_p = dict(cfg, kv_len=p)
        for l in range(cfg["n_layers"]):
            check_sparse_layer(eng, cfg_p, W, l, _layer_inputs(eng, x, l), workloads.bf16_bits(kv[l]), p)
    check_coverage(eng, steps=6)


def _topk_chunk(eng):
    """Scores per LDS chunk of the top-T task (its first type-specific field)."""
    ty = {v: k for k, v in __import__("persistent_tile_scheduled_amd.binding", fromlist=["TASK_TYPES"]).TASK_TYPES.items()}
    return [t["aux0"] for t in eng.plan.tasks() if t["type"] == ty["IDX_TOPK"]][0]


def test_sparse_topk_in_chunks():
    """Caches longer than one LDS chunk of scores: the selection runs chunk by chunk. A plan for
    up to 90000 positions, stepped at exactly one full chunk, one position more (a second chunk
    of one score), and a length spanning three chunks."""
    cfg = workloads.get_config("mla_tiny_sparse")
    M = 90000
    w, x, kv = workloads.generate(cfg, seed=4, device="cuda", kv_len=M)
    eng = _engine(cfg, w, max_len=M)
    C = _topk_chunk(eng)
    assert 256 <= C < M // 2 and C % 256 == 0, C
    W = HostWeights(w)
    steps = 0
    for p in [C - 1, C, M]:
        print(f"[sparse] chunked top-T: chunk {C}, position {p}", flush=True)
        eng.set_state(p, 0)
        eng.step_dynamic(kv, x)
        steps += 1
        torch.cuda.synchronize()
        eng.status()
        cfg_p = dict(cfg, kv_len=p)
        for l in range(cfg["n_layers"]):
            check_sparse_layer(eng, cfg_p, W, l, _layer_inputs(eng, x, l), workloads.bf16_bits(kv[l]), p)
    check_coverage(eng, steps=steps)


@pytest.mark.parametrize("distinct", [5, 1])
def test_sparse_topk_ties(distinct):
    """Planted exact ties: the cached index keys repeat `distinct` rows (position p holds row
    p % distinct), so the scores take distinct + 1 values (the new position's key is this
    step's) and the selection boundary falls inside a group of equal scores, which must be taken
    at the lowest positions."""
    cfg = dict(workloads.get_config("mla_tiny_sparse"), kv_len=500)
    n = cfg["kv_len"]
    KR = cfg["kv_lora_rank"] + cfg["qk_rope"]
    DI = cfg["index_dim"]
    w, x, kv = workloads.generate(cfg, seed=5, device="cuda")
    for l in range(cfg["n_layers"]):
        rows = kv[l][:distinct, KR:KR + DI].clone()
        idx = torch.arange(n, device=kv[l].device) % distinct
        kv[l][:n, KR:KR + DI] = rows[idx]
    print(f"[sparse] ties: {distinct} distinct cached index keys", flush=True)
    eng = _engine(cfg, w)
    eng.step(x, kv)
    torch.cuda.synchronize()
    eng.status()
    W = HostWeights(w)
    for l in range(cfg["n_layers"]):
        sc = eng.buffer(f"layers.{l}.idx_scores").cpu().numpy()[:n + 1]
        assert len(np.unique(sc)) <= distinct + 1, (l, len(np.unique(sc)))
        check_sparse_layer(eng, cfg, W, l, _layer_inputs(eng, x, l), workloads.bf16_bits(kv[l]), n)
    check_coverage(eng)
