"""Pins of the oracle's sparse indexer (reading R24; CPU only).

The audit page names the indexer (64 index heads selecting the top-2048 cache positions) but
no formula; the oracle scores every position with I_s = sum_j w_j max(0, q_j . k_s) and lets
attention read only the top-T positions. Each part is held to something other than itself:
element-by-element loops for the scores, constructed score vectors for the selection rule
(ties, ranks, short caches), and the already pinned dense MLA layer -- which the sparse layer
must reproduce exactly when every position is selected, and up to rounding when the positions
it drops are given probability zero in the dense layer.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from oracle import decode_oracle as D


def _W(w):
    return O.dict_weights({k: (workloads.bf16_bits(v) if v.dtype == torch.bfloat16 else v.numpy()) for k, v in w.items()})


def test_index_scores_against_loops():
    rng = np.random.default_rng(3)
    H, d, N = 5, 7, 11
    q, w, K = rng.normal(size=(H, d)), rng.normal(size=H), rng.normal(size=(N, d))
    want = np.zeros(N)
    for s in range(N):
        for j in range(H):
            dot = 0.0
            for c in range(d):
                dot += q[j, c] * K[s, c]
            want[s] += w[j] * (dot if dot > 0 else 0.0)
    assert np.allclose(O.index_scores(q, w, K), want, rtol=1e-12, atol=1e-12)
    # a head whose dot products are all negative contributes nothing (the ReLU)
    Kp, qn = np.abs(K), -np.abs(q)
    assert np.all(O.index_scores(qn, w, Kp) == 0.0)
    assert np.allclose(O.index_scores(np.vstack([q, qn]), np.concatenate([w, w]), Kp), O.index_scores(q, w, Kp))


def test_selection_rule():
    s = np.array([0.5, 2.0, 2.0, -1.0, 2.0, 3.0, 0.5], dtype=np.float32)
    assert O.select_positions(s, 1).tolist() == [5]
    assert O.select_positions(s, 3).tolist() == [1, 2, 5]          # a three-way tie at 2.0: the lower two
    assert O.select_positions(s, 4).tolist() == [1, 2, 4, 5]
    assert O.select_positions(s, 6).tolist() == [0, 1, 2, 4, 5, 6]  # the tie at 0.5 fits whole
    assert O.select_positions(s, 7).tolist() == list(range(7))
    assert O.select_positions(s, 100).tolist() == list(range(7))   # a short cache: everything
    rng = np.random.default_rng(0)
    v = rng.normal(size=1000)
    top = np.argsort(-v, kind="stable")[:64]
    assert O.select_positions(v, 64).tolist() == sorted(top.tolist())


def test_planted_rank_by_position_is_caught():
    """Taking the first T positions instead of the T best fails the rule above."""
    s = np.array([0.1, 0.2, 5.0, 4.0], dtype=np.float32)
    assert O.select_positions(s, 2).tolist() == [2, 3]
    assert np.arange(2).tolist() != O.select_positions(s, 2).tolist()


def test_all_positions_selected_equals_dense():
    """With index_topk >= kv_len + 1 the sparse layer attends every position and must give the
    dense layer's values exactly (the index weights only add trace entries)."""
    cfg = dict(workloads.get_config("mla_tiny_sparse"), index_topk=1000)
    dense = dict(cfg)
    for k in ("index_heads", "index_dim", "index_topk"):
        dense.pop(k)
    w, x, kv = workloads.generate(cfg, seed=2)
    W = _W(w)
    kvb = workloads.bf16_bits(kv)
    a = O.forward(cfg, W, workloads.bf16_bits(x), kvb)
    b = O.forward(dense, W, workloads.bf16_bits(x), kvb)
    assert np.array_equal(a["out"], b["out"])
    assert a["layers"][0]["idx_sel"].tolist() == list(range(cfg["kv_len"] + 1))


def test_sparse_equals_dense_when_dropped_positions_cannot_matter():
    """One query head. The cached positions the indexer drops get latent rows c = 0 and
    k_pe = -1e4 q_rope, so the dense layer gives them probability exactly 0 (exp underflows);
    their index keys are unchanged, so the selection is too. The dense layer over that cache
    must then match the sparse layer, which never reads them."""
    base = dict(workloads.get_config("mla_tiny_sparse"), n_q_heads=1, n_layers=1)
    dense = {k: v for k, v in base.items() if not k.startswith("index_")}
    kl, dr = base["kv_lora_rank"], base["qk_rope"]
    n = base["kv_len"]
    for seed in range(20):
        w, x, kv = workloads.generate(base, seed=seed)
        W = _W(w)
        kvb = workloads.bf16_bits(kv)
        a = O.forward(base, W, workloads.bf16_bits(x), kvb)
        t = a["layers"][0]
        sel = t["idx_sel"]
        if sel[-1] != n:
            continue  # the new position (computed in the layer) must be among the selected
        drop = np.setdiff1d(np.arange(n), sel)
        q_rope = t["q_rope"].reshape(-1)
        kv2 = kv.clone()
        kv2[0, drop, :kl] = 0
        kv2[0, drop, kl:kl + dr] = torch.from_numpy(-1e4 * q_rope).to(torch.bfloat16)
        kvb2 = workloads.bf16_bits(kv2)
        a2 = O.forward(base, W, workloads.bf16_bits(x), kvb2)
        assert a2["layers"][0]["idx_sel"].tolist() == sel.tolist()
        assert np.array_equal(a2["out"], a["out"])   # the sparse layer never reads the dropped rows
        b = O.forward(dense, W, workloads.bf16_bits(x), kvb2)
        assert np.allclose(b["layers"][0]["attn"], t["attn"], rtol=1e-12, atol=1e-14)
        assert np.allclose(b["out"], a["out"], rtol=1e-12, atol=1e-12)
        return
    pytest.fail("no seed put the new position among the selected")


def test_planted_missing_relu_changes_the_selection(monkeypatch):
    cfg = workloads.get_config("mla_small_sparse")
    w, x, kv = workloads.generate(cfg, seed=4)
    W = _W(w)
    kvb = workloads.bf16_bits(kv)
    good = O.forward(cfg, W, workloads.bf16_bits(x), kvb)["layers"][0]["idx_sel"]
    monkeypatch.setattr(D, "index_scores", lambda q, wi, K: (np.asarray(K) @ np.asarray(q).T) @ np.asarray(wi))
    bad = O.forward(cfg, W, workloads.bf16_bits(x), kvb)["layers"][0]["idx_sel"]
    assert good.tolist() != bad.tolist()
