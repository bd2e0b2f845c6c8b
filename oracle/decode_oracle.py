"""fp64 CPU oracle for one batch-1 decode step -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.

Only the tests, the bench's CPU-baseline leg and the package's smoke check may import this
module. It shares no code with the HIP path: it is plain NumPy in float64, written from
the textbook definitions of the operations.

What the pages fix, and what they leave open
--------------------------------------------
The pages describe a persistent, tile-scheduled decode engine and name the fused
operations it runs, but print no formula, listing or worked example:
  * "Static Compilation for LLM Inference: from ASIC Graph Compile to Persistent Engine
    Kernel", section 5.4 (table of XLA/TVM assumptions): at batch 1 every GEMM is
    memory-bound and Norm+GEMM+Attention should be fused; the fused kernel
    rmsnorm_projx_wqkvia is named there.
  * same page, section 5.3 and the section 11 reference list: FlashAttention's IO-aware
    tiling with online softmax (FA1) and sequence-dimension parallelism (FA2), the basis
    of the split-K decode attention.
  * same page, section 5.5 (static compile vs dynamic serving table): the KV cache grows
    by one position per token; MoE routing is input dependent.
  * the tile-ai/TileRT audit page, paragraphs on the fused-op names
    (RMSNormProjxWqkvia, UnProjOAllReduce, ExpertDownAllReduce,
    ExpertSelectUpGateSiLU), on batch 1 (max_batch_size = 1, FlashSparseMLA) and on
    TokenSpeed's MLA q-head folding.
So every formula below is the plain standard reading (Llama-style pre-norm GQA with
rotate-half RoPE and SwiGLU; DeepSeek-style MLA with a latent KV cache and a sigmoid
top-k router). The readings taken where the pages are silent:
  R1  per-layer math: the textbook forms in this file.
  R2  the cache holds kv_len past positions; the step writes slot kv_len and attends over
      kv_len+1 positions; the RoPE position of the new token is p = kv_len.
  R3  cached K (and the MLA k_pe) are stored post-RoPE; cached MLA c is stored normalised.
  R4  RoPE pairs (i, i + d/2) ("rotate half"), theta_i = theta^(-2i/d), no scaling.
  R7  softmax scale 1/sqrt(head_dim) (GQA) and 1/sqrt(qk_nope + qk_rope) (MLA).
  R8  GQA head h reads KV head floor(h * n_kv / n_q).
  R9  router: sigma = sigmoid(W_r x); selection on sigma + bias; top-k with ties to the
      lower index; weights sigma_T / sum(sigma_T); shared experts with weight 1.
  R11 the KV cache is bf16: the appended entry is the new k/v (or c/k_pe) rounded to
      bf16 (round to nearest even), and attention reads the cache, new slot included.
  R13 MLA/MoE configs have no LM head and no final norm: the output is the last hidden
      state.
  R24 sparse indexer (the audit page: 64 index heads select the top-2048 KV positions; no
      formula): index key k = W_k x^ (appended to the cache as bf16 after the latent row),
      head weights w = W_w x^, index queries q_j = (W_q c_q)_j from the normalised query
      latent; score I_s = sum_j w_j max(0, q_j . k_s) over every position s (the ReLU-gated,
      head-weighted form of the DeepSeek lightning indexer those weights come from); the top-T
      positions by score (fp32, ties to the lower position) are the only ones attention reads.
Where floating point decides an integer (the top-k set), the decision is taken in fp32,
the precision of the GPU kernel: fp64 router logits are rounded to fp32, and the
sigmoid, the bias add and the comparisons run in fp32.

Weights are passed as a callable W(name, index=None) returning a NumPy array: uint16 bf16
bit patterns for bf16 tensors, float32 for the router bias. `index` selects one expert of
a stacked expert tensor, so the MoE oracle reads only the experts it routes to.

Low-precision weights (the pages name the lever -- fewer bytes per token -- not a format): a linear matrix given as uint8 is OCP
FP8 E4M3 bytes, and W(name + ".scale") holds one fp32 scale per row; the matrix the layer
multiplies by is scale[r] * e4m3(bytes[r, c]), decoded exactly (decode_e4m3). In the latent
families every linear matrix but the per-head absorption matrices (w_uk, w_uv) and the
router may be FP8 this way; a stacked expert tensor has one scale per row of every expert.
"""
from __future__ import annotations

import math
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

# ----------------------------------------------------------------------------------------
# bf16 bit patterns <-> float64
# ----------------------------------------------------------------------------------------


def widen_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (a bf16 is the top half of an fp32)."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        b = b.view(np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode_e4m3(bits) -> np.ndarray:
    """OCP FP8 E4M3 ("FN") byte -> float64, exactly: sign bit, 4 exponent bits with bias 7,
    3 mantissa bits; exponent 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN; there are
    no infinities (the largest finite magnitude is 1.75 * 2^8 = 448)."""
    b = np.asarray(bits).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    out = sign * mag
    return np.where((e == 0xF) & ((b & 0x7) == 0x7), np.nan, out)


def round_to_bf16(x) -> Tuple[np.ndarray, np.ndarray]:
    """Round float64 values to the nearest bf16 (ties to even), directly from float64.

    A bf16 keeps 8 significant bits. With x = m * 2^e, 0.5 <= |m| < 1 (frexp), the nearest
    bf16 is round_half_even(m * 2^8) * 2^(e-8). Returns (values as float64, uint16 bits).
    Valid for finite values inside the normal bf16 range, which is all this oracle needs.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    v = np.ldexp(np.round(np.ldexp(m, 8)), e - 8)   # np.round: half to even
    bits = (v.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return v, bits


def decode_e2m1(codes) -> np.ndarray:
    """FP4 E2M1 nibble (its low 4 bits) -> float64, exactly: bit 3 the sign, bits 2..1 an
    exponent with bias 1, bit 0 the mantissa; exponent 0 encodes the subnormals 0 and 0.5 (so
    m * 2^-1), otherwise (1 + m/2) * 2^(e-1). No infinities or NaN; the largest magnitude is 6.
    (The element format of the OCP Microscaling (MX) FP4 type; the pages name FP4 expert weights
    without fixing a format.)"""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    mag = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int64)))
    return sign * mag


def decode_e8m0(bits) -> np.ndarray:
    """E8M0 scale byte -> 2^(s - 127) (the MX shared block scale: an exponent only); s = 255
    is NaN."""
    b = np.asarray(bits).astype(np.int64)
    return np.where(b == 0xFF, np.nan, np.ldexp(1.0, (b - 127).astype(np.int64)))


MX_BLOCK = 32  # elements sharing one E8M0 scale


def dequant_mxfp4(packed, scales) -> np.ndarray:
    """MXFP4 rows -> float64. packed: uint8 [..., K/2], byte i holding element 2i in its low
    nibble and element 2i+1 in its high nibble; scales: uint8 [..., K/32]. Element k is
    E2M1(k) * E8M0(scales[k // 32])."""
    p = np.asarray(packed).astype(np.int64)
    codes = np.stack([p & 0xF, p >> 4], axis=-1).reshape(p.shape[:-1] + (2 * p.shape[-1],))
    vals = decode_e2m1(codes)
    sc = decode_e8m0(np.asarray(scales))
    return vals * np.repeat(sc, MX_BLOCK, axis=-1)


def _w64(W: Callable, name: str, index=None) -> np.ndarray:
    a = W(name) if index is None else W(name, index)
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return widen_bf16(a)
    return a.astype(np.float64)


# ----------------------------------------------------------------------------------------
# the operations (textbook definitions)
# ----------------------------------------------------------------------------------------


def rmsnorm(u: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm(u; g) = u / sqrt(mean(u^2) + eps) * g, mean over the whole vector.

    The pages name the fused RMSNorm + QKV op ("Static Compilation ..." section 5.4;
    the TileRT audit page's RMSNormProjxWqkvia) without a formula; this is the standard one.
    """
    u = np.asarray(u, dtype=np.float64)
    return u / math.sqrt(float(np.mean(u * u)) + eps) * g


def rope(u: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotate-half RoPE of one head vector u (length d) at position pos.

    theta_i = theta^(-2i/d) for i < d/2; the pair (u_i, u_{i+d/2}) is rotated by pos*theta_i:
        u'_i       = u_i cos - u_{i+d/2} sin
        u'_{i+d/2} = u_{i+d/2} cos + u_i sin
    (reading R4; the pages do not define RoPE).
    """
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    ang = pos * theta ** (-2.0 * i / d)
    c, s = np.cos(ang), np.sin(ang)
    a, b = u[..., :half], u[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def linear(Wm: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y = W x with W row-major [out][in] (a library matrix-vector product)."""
    return Wm @ x


def linear_bits(W: Callable, name: str, x: np.ndarray, index=None,
                rows_per_block: int = 1 << 16) -> np.ndarray:
    """y = W x for a matrix given by name: bf16 bits, or FP8 E4M3 bytes with one fp32 scale
    per row (W(name + ".scale")). Rows are widened a block at a time so a 1 GB LM head never
    needs its whole fp64 copy in memory. Each output element is still one full dot product
    of its row."""
    bits = W(name) if index is None else W(name, index)
    bits = np.asarray(bits)
    if bits.dtype == np.uint8:
        scale = np.asarray(W(name + ".scale") if index is None else W(name + ".scale", index), dtype=np.float64)
        widen = lambda r0, r1: decode_e4m3(bits[r0:r1]) * scale[r0:r1, None]
    else:
        widen = lambda r0, r1: widen_bf16(bits[r0:r1])
    n = bits.shape[0]
    if n <= rows_per_block:
        return linear(widen(0, n), x)
    out = np.empty(n, dtype=np.float64)
    for r0 in range(0, n, rows_per_block):
        r1 = min(n, r0 + rows_per_block)
        out[r0:r1] = linear(widen(r0, r1), x)
    return out


def softmax(s: np.ndarray) -> np.ndarray:
    """softmax over the last axis; the max is subtracted first (a value-preserving shift)."""
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def kv_group(h: int, n_q: int, n_kv: int) -> int:
    """The KV head query head h reads under grouped-query attention: contiguous groups of
    n_q / n_kv query heads share one KV head (reading R8)."""
    return (h * n_kv) // n_q


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """One query against n keys: o = softmax(scale * K q) V.  K [n][d], V [n][dv]."""
    p = softmax(scale * (K @ q))
    return p @ V


def attend_partial(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Online-softmax partial of one chunk of positions (FlashAttention's tiling,
    "Static Compilation ..." section 5.3): m = max s, l = sum e^(s-m), a = sum e^(s-m) V."""
    s = scale * (K @ q)
    m = float(np.max(s))
    e = np.exp(s - m)
    return m, float(np.sum(e)), e @ V


def merge_partials(parts: Sequence[Tuple[float, float, np.ndarray]]) -> np.ndarray:
    """Merge split-K partials: o = sum_c e^(m_c-M) a_c / sum_c e^(m_c-M) l_c, M = max m_c."""
    M = max(p[0] for p in parts)
    num = sum(math.exp(m - M) * a for (m, l, a) in parts)
    den = sum(math.exp(m - M) * l for (m, l, a) in parts)
    return num / den


def attend_split(q, K, V, scale, bounds: Sequence[int]) -> np.ndarray:
    """Split-K (flash-decoding) attention: positions cut at `bounds` (0 = b0 < ... < bk = n),
    one partial per chunk, then the merge. Equal to attend() in exact arithmetic."""
    parts = [attend_partial(q, K[a:b], V[a:b], scale) for a, b in zip(bounds[:-1], bounds[1:])]
    return merge_partials(parts)


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + e^-z)."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu(Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray, x: np.ndarray):
    """SwiGLU FFN: a = silu(W_g x) * (W_u x); y = W_d a. Returns (a, y)."""
    a = silu(Wg @ x) * (Wu @ x)
    return a, Wd @ a


def route(r: np.ndarray, bias: np.ndarray, top_k: int):
    """Sigmoid top-k router (reading R9), decision in fp32.

    sigma = sigmoid(r); z = sigma + bias; T = indices of the top_k largest z, ties to the
    lower index, listed by decreasing z; w_e = sigma_e / sum_{T} sigma. The selection is
    made on fp32 values (fp64 logits rounded to fp32, then fp32 sigmoid and add), as the
    GPU makes it. The weights are computed in fp64.
    Returns dict(sigma, z, topk, w, margin) where margin is the fp64 gap between the
    k-th and (k+1)-th largest z (inf when top_k equals the expert count).
    """
    r = np.asarray(r, dtype=np.float64)
    b = np.asarray(bias, dtype=np.float64)
    r32 = r.astype(np.float32)
    one = np.float32(1.0)
    sig32 = one / (one + np.exp(-r32))
    z32 = (sig32 + b.astype(np.float32)).astype(np.float32)
    order = np.argsort(-z32, kind="stable")          # stable: equal z keep lower index first
    T = order[:top_k].astype(np.int64)
    sigma = 1.0 / (1.0 + np.exp(-r))
    z = sigma + b
    zs = np.sort(z)[::-1]
    margin = float(zs[top_k - 1] - zs[top_k]) if top_k < len(z) else float("inf")
    w = sigma[T] / np.sum(sigma[T])
    return {"sigma": sigma, "z": z, "z32": z32, "topk": T, "w": w, "margin": margin}


# ----------------------------------------------------------------------------------------
# layers
# ----------------------------------------------------------------------------------------


def gqa_layer(cfg: dict, W: Callable, l: int, x: np.ndarray, kv_layer, kv_len: int):
    """One pre-norm GQA decoder layer at position p = kv_len.

    kv_layer: bf16 bits [2][n_kv][>=kv_len][head_dim] (positions [0, kv_len) are read).
    Returns (x_next, trace dict).
    """
    p = f"layers.{l}."
    d, nq, nkv, hd = cfg["hidden"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    eps, theta = cfg["rms_eps"], cfg["rope_theta"]
    pos = kv_len
    t: Dict[str, np.ndarray] = {"x_in": x}
    xn = rmsnorm(x, _w64(W, p + "attn_norm"), eps)
    t["xn"] = xn
    q = linear_bits(W, p + "wq", xn).reshape(nq, hd)
    k = linear_bits(W, p + "wk", xn).reshape(nkv, hd)
    v = linear_bits(W, p + "wv", xn).reshape(nkv, hd)
    q = rope(q, pos, theta)
    k = rope(k, pos, theta)
    t["q"], t["k_new"], t["v_new"] = q.reshape(-1), k.reshape(-1), v.reshape(-1)
    k16, kbits = round_to_bf16(k)
    v16, vbits = round_to_bf16(v)
    t["k_new_bits"], t["v_new_bits"] = kbits.reshape(-1), vbits.reshape(-1)
    kvl = np.asarray(kv_layer)
    scale = 1.0 / math.sqrt(hd)
    o = np.empty((nq, hd))
    for g in range(nkv):
        Kc = np.concatenate([widen_bf16(kvl[0, g, :kv_len]), k16[g][None, :]], axis=0)
        Vc = np.concatenate([widen_bf16(kvl[1, g, :kv_len]), v16[g][None, :]], axis=0)
        for h in range(nq):
            if kv_group(h, nq, nkv) == g:
                o[h] = attend(q[h], Kc, Vc, scale)
    t["attn"] = o.reshape(-1)
    h_ = x + linear_bits(W, p + "wo", t["attn"])
    t["h"] = h_
    hn = rmsnorm(h_, _w64(W, p + "ffn_norm"), eps)
    t["hn"] = hn
    a = silu(linear_bits(W, p + "w_gate", hn)) * linear_bits(W, p + "w_up", hn)
    t["ffn_act"] = a
    f = linear_bits(W, p + "w_down", a)
    t["ffn_out"] = f
    xo = h_ + f
    t["x_out"] = xo
    return xo, t


def verify_visible(kv_len: int, i: int, M: int) -> int:
    """Causal visibility in a block of M new tokens: token i (position kv_len + i) attends the
    first kv_len + i + 1 positions of the cache, itself included, none of the later tokens."""
    return kv_len + i + 1


def gqa_verify_layer(cfg: dict, W: Callable, l: int, X: np.ndarray, kv_layer, kv_len: int):
    """One pre-norm GQA layer for M tokens at once (a multi-token verification step): token i
    sits at position p_i = kv_len + i, and attends causally, over the cached positions
    [0, kv_len) and the block's own positions up to and including p_i. Every token's new k, v
    is appended to the cache (rounded to bf16, reading R11) before any attention reads it.
    The pages name multi-token prediction and speculative verification as the multi-token
    lever (the TileRT talk, practice section) without a formula; this is the causal block
    attention that M sequential decode steps compute (pinned against them).

    X: [M][hidden]. kv_layer: bf16 bits [2][n_kv][>=kv_len][head_dim].
    Returns (X_next [M][hidden], trace dict of [M][...] arrays).
    """
    p = f"layers.{l}."
    X = np.asarray(X, dtype=np.float64)
    M = X.shape[0]
    nq, nkv, hd = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    eps, theta = cfg["rms_eps"], cfg["rope_theta"]
    g_attn, g_ffn = _w64(W, p + "attn_norm"), _w64(W, p + "ffn_norm")
    t: Dict[str, np.ndarray] = {"x_in": X}
    xn = np.stack([rmsnorm(X[i], g_attn, eps) for i in range(M)])
    q = np.stack([linear_bits(W, p + "wq", xn[i]).reshape(nq, hd) for i in range(M)])
    k = np.stack([linear_bits(W, p + "wk", xn[i]).reshape(nkv, hd) for i in range(M)])
    v = np.stack([linear_bits(W, p + "wv", xn[i]).reshape(nkv, hd) for i in range(M)])
    q = np.stack([rope(q[i], kv_len + i, theta) for i in range(M)])
    k = np.stack([rope(k[i], kv_len + i, theta) for i in range(M)])
    t["q"] = q.reshape(M, -1)
    k16, kbits = round_to_bf16(k)
    v16, vbits = round_to_bf16(v)
    t["k_new_bits"], t["v_new_bits"] = kbits.reshape(M, -1), vbits.reshape(M, -1)
    kvl = np.asarray(kv_layer)
    scale = 1.0 / math.sqrt(hd)
    o = np.empty((M, nq, hd))
    for g in range(nkv):
        # the cache as the block leaves it: cached rows, then the M appended rows
        Kc = np.concatenate([widen_bf16(kvl[0, g, :kv_len]), k16[:, g]], axis=0)
        Vc = np.concatenate([widen_bf16(kvl[1, g, :kv_len]), v16[:, g]], axis=0)
        for i in range(M):
            m = verify_visible(kv_len, i, M)
            for h in range(nq):
                if kv_group(h, nq, nkv) == g:
                    o[i, h] = attend(q[i, h], Kc[:m], Vc[:m], scale)
    t["attn"] = o.reshape(M, -1)
    H = X + np.stack([linear_bits(W, p + "wo", t["attn"][i]) for i in range(M)])
    t["h"] = H
    hn = np.stack([rmsnorm(H[i], g_ffn, eps) for i in range(M)])
    a = np.stack([silu(linear_bits(W, p + "w_gate", hn[i])) * linear_bits(W, p + "w_up", hn[i]) for i in range(M)])
    t["ffn_act"] = a
    f = np.stack([linear_bits(W, p + "w_down", a[i]) for i in range(M)])
    t["ffn_out"] = f
    t["x_out"] = H + f
    return t["x_out"], t


def verify_forward(cfg: dict, W: Callable, x_bits, kv, kv_len: Optional[int] = None):
    """A verification step of M tokens (GQA family): x_bits bf16 bits [M][hidden]; kv
    indexable by layer (cache bits, positions [0, kv_len) read). Returns
    {"layers": [trace...], "out": [M][vocab] logits (or [M][hidden] last hidden states)}."""
    n = cfg["kv_len"] if kv_len is None else kv_len
    X = widen_bf16(np.asarray(x_bits))
    traces: List[Dict[str, np.ndarray]] = []
    for l in range(cfg["n_layers"]):
        X, t = gqa_verify_layer(cfg, W, l, X, kv[l], n)
        traces.append(t)
    outs = np.stack([head(cfg, W, X[i])["out"] for i in range(X.shape[0])])
    return {"layers": traces, "x_final": X, "out": outs}


def index_scores(q_idx: np.ndarray, w_idx: np.ndarray, K_idx: np.ndarray) -> np.ndarray:
    """Sparse-indexer scores (reading R24): I_s = sum_j w_j * max(0, q_j . k_s) over the H index
    heads j, for every position s. q_idx [H][d], w_idx [H], K_idx [N][d] -> [N]."""
    return np.maximum(np.asarray(K_idx) @ np.asarray(q_idx).T, 0.0) @ np.asarray(w_idx)


def select_positions(scores, T: int) -> np.ndarray:
    """The T positions with the largest scores, ties to the lower position, returned in
    increasing position order; every position when there are at most T (reading R24)."""
    s = np.asarray(scores)
    n = s.shape[0]
    if n <= T:
        return np.arange(n)
    order = np.lexsort((np.arange(n), -s.astype(np.float64)))  # by score descending, then position
    return np.sort(order[:T])


def mla_attention(cfg: dict, W: Callable, l: int, xn: np.ndarray, kv_layer, kv_len: int,
                  absorbed_trace: bool = True):
    """MLA attention of one layer (naive definition), plus the absorbed-form intermediates.

    Definition (naive): with latent cache rows [c_j || kpe_j],
        k_{h,j} = [W_UK,h c_j || kpe_j],  v_{h,j} = W_UV,h c_j,
        s_{h,j} = q_h . k_{h,j} / sqrt(qk_nope + qk_rope),  o_h = sum_j softmax(s_h)_j v_{h,j}.
    Absorbed form (same value, what a decode kernel computes; TokenSpeed's q-head folding on
    the TileRT audit page treats all heads as rows of one contraction over the latent):
        qa_h = W_UK,h^T q_nope,h;  s_{h,j} = (qa_h . c_j + q_rope,h . kpe_j)/sqrt(...);
        ol_h = sum_j p_{h,j} c_j;  o_h = W_UV,h ol_h.
    Returns (o [n_heads*v_head], trace).
    """
    p = f"layers.{l}."
    nh = cfg["n_q_heads"]
    ql, kl = cfg["q_lora_rank"], cfg["kv_lora_rank"]
    dn, dr, dv = cfg["qk_nope"], cfg["qk_rope"], cfg["v_head"]
    eps, theta = cfg["rms_eps"], cfg["rope_theta"]
    pos = kv_len
    t: Dict[str, np.ndarray] = {}
    cq_raw = linear_bits(W, p + "wq_a", xn)
    cq = rmsnorm(cq_raw, _w64(W, p + "q_norm"), eps)
    t["cq_raw"], t["cq"] = cq_raw, cq
    qf = linear_bits(W, p + "wq_b", cq).reshape(nh, dn + dr)
    q_nope = qf[:, :dn]
    q_rope = rope(qf[:, dn:], pos, theta)
    t["q_nope"], t["q_rope"] = q_nope.reshape(-1), q_rope.reshape(-1)
    a = linear_bits(W, p + "wkv_a", xn)
    t["kv_a"] = a
    c_new = rmsnorm(a[:kl], _w64(W, p + "kv_norm"), eps)
    kpe_new = rope(a[kl:], pos, theta)
    t["c_new"], t["kpe_new"] = c_new, kpe_new
    ent16, ent_bits = round_to_bf16(np.concatenate([c_new, kpe_new]))
    t["kv_new_bits"] = ent_bits
    kvl = np.asarray(kv_layer)
    lat = np.concatenate([widen_bf16(kvl[:kv_len, :kl + dr]), ent16[None, :]], axis=0)  # [n+1][kl+dr]
    if cfg.get("index_heads", 0):
        # sparse indexer (reading R24): the new position's index key is appended (bf16), every
        # position is scored, and attention reads only the selected positions' latent rows
        hi, di, T = cfg["index_heads"], cfg["index_dim"], cfg["index_topk"]
        k_idx = linear_bits(W, p + "idx_wk", xn)
        k16, k_bits = round_to_bf16(k_idx)
        w_idx = linear_bits(W, p + "idx_w", xn)
        q_idx = linear_bits(W, p + "idx_wq", cq).reshape(hi, di)
        K_idx = np.concatenate([widen_bf16(kvl[:kv_len, kl + dr:kl + dr + di]), k16[None, :]], axis=0)
        sc = index_scores(q_idx, w_idx, K_idx)
        sc32 = sc.astype(np.float32)  # the selection is decided in fp32 (the kernel's precision)
        sel = select_positions(sc32, T)
        t["idx_k"], t["idx_k_bits"], t["idx_w"], t["idx_q"] = k_idx, k_bits, w_idx, q_idx.reshape(-1)
        t["idx_scores"], t["idx_sel"] = sc, sel
        srt = np.sort(sc32.astype(np.float64))[::-1]
        t["idx_margin"] = np.array([(srt[T - 1] - srt[T]) / max(np.max(np.abs(srt)), 1e-300) if len(srt) > T else np.inf])
        lat = lat[sel]
    C, KPE = lat[:, :kl], lat[:, kl:]
    Wuk = _w64(W, p + "w_uk")   # [nh][dn][kl]
    Wuv = _w64(W, p + "w_uv")   # [nh][dv][kl]
    scale = 1.0 / math.sqrt(dn + dr)
    o = np.empty((nh, dv))
    for h in range(nh):
        Kh = np.concatenate([C @ Wuk[h].T, KPE], axis=1)     # [n+1][dn+dr]
        Vh = C @ Wuv[h].T                                     # [n+1][dv]
        o[h] = attend(np.concatenate([q_nope[h], q_rope[h]]), Kh, Vh, scale)
    t["attn"] = o.reshape(-1)
    if absorbed_trace:
        qa = np.einsum("hdc,hd->hc", Wuk, q_nope)             # [nh][kl]
        ol = np.empty((nh, kl))
        for h in range(nh):
            s = scale * (C @ qa[h] + KPE @ q_rope[h])
            ol[h] = softmax(s) @ C
        t["q_abs"] = qa.reshape(-1)
        t["o_lat"] = ol.reshape(-1)
    return o.reshape(-1), t


def mla_attention_absorbed(cfg: dict, W: Callable, l: int, q_nope, q_rope, lat) -> np.ndarray:
    """Absorbed-form MLA attention core from given q parts and latent rows lat [n][kl+dr]."""
    p = f"layers.{l}."
    nh, kl = cfg["n_q_heads"], cfg["kv_lora_rank"]
    dn, dr = cfg["qk_nope"], cfg["qk_rope"]
    Wuk = _w64(W, p + "w_uk")
    Wuv = _w64(W, p + "w_uv")
    C, KPE = lat[:, :kl], lat[:, kl:]
    scale = 1.0 / math.sqrt(dn + dr)
    qn = np.asarray(q_nope).reshape(nh, dn)
    qr = np.asarray(q_rope).reshape(nh, dr)
    out = []
    for h in range(nh):
        qa = Wuk[h].T @ qn[h]
        pr = softmax(scale * (C @ qa + KPE @ qr[h]))
        out.append(Wuv[h] @ (pr @ C))
    return np.concatenate(out)


def _expert_w64(cfg: dict, W: Callable, name: str, index=None) -> np.ndarray:
    """An expert matrix as float64: bf16 bits, (weights "fp8") E4M3 rows each times its fp32
    scale in name + ".scale", or (weights "mxfp4") MXFP4 rows with the E8M0 scales in
    name + ".scale"."""
    if cfg.get("weights") == "fp8":
        sc = np.asarray(W(name + ".scale") if index is None else W(name + ".scale", index), dtype=np.float64)
        return decode_e4m3(W(name) if index is None else W(name, index)) * sc[..., None]
    if cfg.get("weights") != "mxfp4":
        return _w64(W, name, index)
    sc = W(name + ".scale") if index is None else W(name + ".scale", index)
    return dequant_mxfp4(W(name) if index is None else W(name, index), sc)


def moe_ffn(cfg: dict, W: Callable, l: int, hn: np.ndarray):
    """MoE FFN (reading R9): y = SwiGLU_shared(hn) + sum_{e in T} w_e SwiGLU_e(hn). With
    weights "mxfp4" every expert matrix (routed and shared) is MXFP4 (reading R22)."""
    p = f"layers.{l}."
    k = cfg["top_k"]
    t: Dict[str, np.ndarray] = {}
    r = linear_bits(W, p + "router", hn)
    rt = route(r, np.asarray(W(p + "router_bias"), dtype=np.float64), k)
    t["router_logits"] = r
    t["topk"] = rt["topk"]
    t["topk_w"] = rt["w"]
    t["topk_margin"] = np.array([rt["margin"]])
    a_s, y_s = swiglu(_expert_w64(cfg, W, p + "shared.w_gate"), _expert_w64(cfg, W, p + "shared.w_up"),
                      _expert_w64(cfg, W, p + "shared.w_down"), hn)
    t["shared_act"], t["shared_out"] = a_s, y_s
    y = y_s.copy()
    acts = []
    for e, we in zip(rt["topk"], rt["w"]):
        a_e, y_e = swiglu(_expert_w64(cfg, W, p + "experts.w_gate", int(e)),
                          _expert_w64(cfg, W, p + "experts.w_up", int(e)),
                          _expert_w64(cfg, W, p + "experts.w_down", int(e)), hn)
        acts.append(a_e)
        y = y + we * y_e
    t["expert_act"] = np.concatenate(acts) if acts else np.zeros(0)
    return y, t


def mla_layer(cfg: dict, W: Callable, l: int, x: np.ndarray, kv_layer, kv_len: int):
    """One MLA layer (config arch "mla": dense SwiGLU FFN; "moe": MoE FFN)."""
    p = f"layers.{l}."
    eps = cfg["rms_eps"]
    t: Dict[str, np.ndarray] = {"x_in": x}
    xn = rmsnorm(x, _w64(W, p + "attn_norm"), eps)
    t["xn"] = xn
    o, ta = mla_attention(cfg, W, l, xn, kv_layer, kv_len)
    t.update(ta)
    h_ = x + linear_bits(W, p + "wo", o)
    t["h"] = h_
    hn = rmsnorm(h_, _w64(W, p + "ffn_norm"), eps)
    t["hn"] = hn
    if cfg["arch"] == "mla":
        a = silu(linear_bits(W, p + "w_gate", hn)) * linear_bits(W, p + "w_up", hn)
        t["ffn_act"] = a
        f = linear_bits(W, p + "w_down", a)
    else:
        f, tm = moe_ffn(cfg, W, l, hn)
        t.update(tm)
    t["ffn_out"] = f
    xo = h_ + f
    t["x_out"] = xo
    return xo, t


def layer(cfg: dict, W: Callable, l: int, x: np.ndarray, kv_layer, kv_len: int):
    if cfg["arch"] == "gqa":
        return gqa_layer(cfg, W, l, x, kv_layer, kv_len)
    return mla_layer(cfg, W, l, x, kv_layer, kv_len)


def head(cfg: dict, W: Callable, x: np.ndarray) -> Dict[str, np.ndarray]:
    """Final RMSNorm + LM head (configs with a vocabulary); otherwise the output is x."""
    if cfg.get("vocab", 0) > 0:
        xn = rmsnorm(x, _w64(W, "final_norm"), cfg["rms_eps"])
        return {"final_xn": xn, "out": linear_bits(W, "lm_head", xn)}
    return {"out": np.asarray(x, dtype=np.float64)}


def forward(cfg: dict, W: Callable, x_bits, kv, kv_len: Optional[int] = None,
            layers: Optional[Sequence[int]] = None):
    """One decode step. x_bits: bf16 bits [hidden]; kv: indexable by layer, giving that
    layer's cache bits (see gqa_layer / mla_layer). Returns {"layers": [trace...], "out": ...}.

    `layers` limits the run to a prefix of the stack (for bounded timing samples); the head
    is applied only when the whole stack ran.
    """
    n = cfg["kv_len"] if kv_len is None else kv_len
    L = cfg["n_layers"]
    todo = list(range(L)) if layers is None else list(layers)
    x = widen_bf16(x_bits)
    traces: List[Dict[str, np.ndarray]] = []
    for l in todo:
        x, t = layer(cfg, W, l, x, kv[l], n)
        traces.append(t)
    res = {"layers": traces, "x_final": x}
    if len(todo) == L:
        res.update(head(cfg, W, x))
    return res


def dict_weights(d: Dict[str, np.ndarray]) -> Callable:
    """Adapt a dict of arrays to the W(name, index=None) accessor."""
    def W(name, index=None):
        a = d[name]
        return a if index is None else a[index]
    return W
