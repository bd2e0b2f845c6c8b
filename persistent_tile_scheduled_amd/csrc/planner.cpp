// planner.cpp -- ahead-of-time planner of one batch-1 decode step.
//
// The step is unrolled, layer by layer, into stages of tile tasks ("Static Compilation for
// LLM Inference ...", section 1: the whole model is compiled ahead of time into one
// persistent engine kernel; section 5.6: Fleet's task graph is fixed at compile time;
// TileRT talk, section on breaking kernel boundaries: tile-level tasks start as soon as
// their own dependencies are met). Each stage's work is cut into one task per workgroup
// (one workgroup per CU), every task lists the dependency counters it waits on, and names
// the counter it increments when done. Placement is chiplet-aware (the TileRT audit page's
// Fleet paragraph: one XCD and its 4 MB L2 as an explicit scheduling unit): the tasks of
// one KV-head group -- its QKV rows and its attention splits -- run on the workgroups of
// one XCD, so the group's q/k/v stay in that XCD's L2.
#include "planner.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <set>
#include <tuple>
#include <sstream>

namespace dec {
namespace {

constexpr int kMinPosPerSplit = 16;
constexpr int kRowsCap = kMaxTaskRows;     // rows of one GEMV task (LDS row tables)
#ifndef DEC_STAGE_COUNTERS
#define DEC_STAGE_COUNTERS 8
#endif
constexpr int kStageCounters = DEC_STAGE_COUNTERS;  // completion counters per stage (at least one per XCD)
#ifndef DEC_ODD_XCD_SPEED
#define DEC_ODD_XCD_SPEED 0.92
#endif
constexpr double kOddXcdSpeed = DEC_ODD_XCD_SPEED;  // relative streaming speed of XCDs 1, 3, 5, 7
constexpr int kMinPosMla = 64;             // positions per latent-attention split (at least)
constexpr int kMinPosMlaSparse = 16;       // the same over the indexer's selected positions
constexpr int kIdxPos = 128;               // positions per sparse-indexer score task (at least)
constexpr int64_t kMergeFloats = 17000;    // LDS floats for one group's attention partials

int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

struct PTask {
  TaskDesc d;
  int stage;
  std::vector<int32_t> deps;
};

struct Builder {
  const dec_model_shape& s;
  int64_t n;  // kv_len (dynamic plans: the largest position a step may have)
  bool dyn;
  int nt;     // tokens per step (> 1: a verification step)
  const dec_device_info& dev;
  PlanData& P;
  std::string& err;
  int n_wg = 0, n_xcd = 1;
  int stage = 0;
  int next_id = 0;
  std::vector<std::vector<PTask>> per_wg;
  std::vector<std::pair<std::string, std::pair<int64_t, int32_t>>> acts;  // name -> (float off, dtype)
  std::vector<int64_t> act_counts;
  int64_t act_floats = 0;
  int64_t xs_floats_max = 0;  // largest staged input vector (padded)
  int64_t scratch_floats = 1024;
  int64_t mla_lds = 0;        // LDS floats (after the header) the latent-attention tasks use

  Builder(const dec_model_shape& s_, int64_t n_, bool dyn_, int nt_, const dec_device_info& d_, PlanData& p_, std::string& e_)
      : s(s_), n(n_), dyn(dyn_), nt(nt_), dev(d_), P(p_), err(e_) {}

  // A verification step keeps every activation per token ([nt][width]); its GEMV tasks hold
  // nt results per row, so they take at most kRowsCap / nt rows.
  int rows_cap() const { return kRowsCap / nt; }
  int64_t act_t(const std::string& name, int64_t count) { return act(name, count * nt); }
  // a verification GEMV stages the input of all nt tokens at once (RMSNormed inputs, merged
  // attention), or at least one chunk per token (column phases)
  void need_xs_t(int64_t K, bool whole) { xs_floats_max = std::max<int64_t>(xs_floats_max, nt * (whole ? align_up(K, kChunkCols) : kChunkCols)); }

  int xcd(int w) const { return w % n_xcd; }
  // Completion counters of a stage: nsc of them, workgroup w signalling counter w % nsc (so a
  // counter's producers share an XCD). More counters mean fewer atomic increments queued on
  // one address when a stage's workgroups finish together; consumers poll one lane each.
  int nsc = 8;
  int slot(int w) const { return w % nsc; }

  int counter(int count) {
    int base = (int)P.counter_total.size();
    P.counter_total.resize(base + count, 0);
    return base;
  }
  std::vector<int32_t> all_of(int base, int count) const {
    std::vector<int32_t> v;
    for (int i = 0; i < count; ++i)
      if (P.counter_total[base + i] > 0) v.push_back(base + i);
    return v;
  }
  int64_t act(const std::string& name, int64_t count, int32_t dtype = DEC_DTYPE_FP32) {
    int64_t off = act_floats;
    acts.push_back({name, {off, dtype}});
    act_counts.push_back(count);
    act_floats += align_up(count, 64);  // 256-byte aligned buffers
    return off;
  }
  // staged input vectors are zero-padded to the GEMV's chunk: 512 bf16 or 1024 FP8 columns
  int64_t chunk_cols() const { return fp8() ? 2 * kChunkCols : kChunkCols; }
  void need_xs(int64_t K) { xs_floats_max = std::max<int64_t>(xs_floats_max, align_up(K, chunk_cols())); }

  int add(int w, int32_t type, int layer, int u0, int u1, std::vector<int32_t> deps, int signal,
          int signal2 = -1, int a0 = 0, int a1 = 0, int a2 = 0, int a3 = 0, int a4 = 0, int a5 = 0,
          int a6 = 0) {
    PTask t;
    std::memset(&t.d, 0, sizeof(t.d));
    t.d.type = type;
    t.d.layer = layer;
    t.d.signal = signal;
    t.d.signal2 = signal2;
    t.d.id = next_id++;
    t.d.u0 = u0;
    t.d.u1 = u1;
    t.d.a0 = a0; t.d.a1 = a1; t.d.a2 = a2; t.d.a3 = a3; t.d.a4 = a4; t.d.a5 = a5; t.d.a6 = a6;
    t.stage = stage;
    t.deps = std::move(deps);
    if (signal >= 0) P.counter_total[signal] += 1;
    per_wg[w].push_back(std::move(t));
    return per_wg[w].back().d.id;
  }

  // Cut `units` units over the workgroups in `wgs` (balanced, contiguous); a workgroup whose
  // share exceeds `cap` gets several consecutive tasks.
  template <class F>
  void spread(const std::vector<int>& wgs, int units, int cap, F&& emit) {
    int m = (int)wgs.size();
    for (int i = 0; i < m; ++i) {
      int u0 = (int)((int64_t)units * i / m), u1 = (int)((int64_t)units * (i + 1) / m);
      for (int a = u0; a < u1; a += cap) emit(wgs[i], a, std::min(u1, a + cap));
    }
  }

  // Like spread, but workgroup i's share is proportional to speed(i). Used for the long
  // 4096-column streams (gate/up, LM head), which run measurably slower on the odd XCDs of
  // MI355X (about 8 %, independent of which rows an XCD gets); equal finishing times shorten
  // the wait of the stage that follows.
  template <class F>
  void spread_weighted(const std::vector<int>& wgs, int units, int cap, F&& emit) {
    const int m = (int)wgs.size();
    std::vector<double> c(m + 1, 0.0);
    for (int i = 0; i < m; ++i) c[i + 1] = c[i] + speed(wgs[i]);
    for (int i = 0; i < m; ++i) {
      int u0 = (int)std::llround(units * c[i] / c[m]), u1 = (int)std::llround(units * c[i + 1] / c[m]);
      for (int a = u0; a < u1; a += cap) emit(wgs[i], a, std::min(u1, a + cap));
    }
  }
  double speed(int w) const { return (n_xcd == 8 && (xcd(w) & 1)) ? kOddXcdSpeed : 1.0; }

  std::vector<int> all_wgs() const {
    std::vector<int> v(n_wg);
    for (int i = 0; i < n_wg; ++i) v[i] = i;
    return v;
  }
  // Workgroups ordered by XCD, cut into `g` contiguous sets (set i -> XCD-local when g | n_xcd).
  std::vector<std::vector<int>> xcd_sets(int g) const {
    std::vector<int> order = all_wgs();
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return xcd(a) < xcd(b); });
    std::vector<std::vector<int>> sets(g);
    for (int i = 0; i < g; ++i) {
      int a = (int)((int64_t)n_wg * i / g), b = (int)((int64_t)n_wg * (i + 1) / g);
      sets[i].assign(order.begin() + a, order.begin() + b);
    }
    return sets;
  }

  bool fail(dec_status st, const std::string& m, dec_status* out) {
    err = m;
    *out = st;
    return false;
  }

  bool check_shape(dec_status* st) {
    const dec_model_shape& q = s;
    if (q.abi_version != DEC_ABI_VERSION) return fail(DEC_E_INVAL, "abi_version mismatch", st);
    if (q.n_layers < 1 || q.hidden < 8 || q.hidden % 8) return fail(DEC_E_SHAPE, "need n_layers >= 1 and hidden a positive multiple of 8", st);
    if (q.vocab < 0) return fail(DEC_E_SHAPE, "vocab < 0", st);
    if (q.weight_format != DEC_WEIGHTS_BF16 && q.weight_format != DEC_WEIGHTS_FP8_E4M3 && q.weight_format != DEC_WEIGHTS_MXFP4)
      return fail(DEC_E_SHAPE, "unknown weight_format", st);
    if (q.index_heads < 0 || q.index_dim < 0 || q.index_topk < 0) return fail(DEC_E_SHAPE, "negative sparse-indexer field", st);
    if (q.index_heads > 0) {
      if (q.arch == DEC_ARCH_GQA) return fail(DEC_E_SHAPE, "the sparse indexer is for the latent families", st);
      if (q.index_heads > 64 || q.index_dim < 32 || q.index_dim > 128 || q.index_dim % 32 || q.index_topk < 1)
        return fail(DEC_E_SHAPE, "sparse indexer: index_heads <= 64, index_dim a multiple of 32 up to 128, index_topk >= 1", st);
      if (q.weight_format != DEC_WEIGHTS_BF16) return fail(DEC_E_SHAPE, "sparse indexer: bf16 weights only", st);
    } else if (q.index_dim || q.index_topk) {
      return fail(DEC_E_SHAPE, "index_dim / index_topk set without index_heads", st);
    }
    if (q.weight_format == DEC_WEIGHTS_MXFP4) {
      if (q.arch != DEC_ARCH_MOE) return fail(DEC_E_SHAPE, "MXFP4 weights: MoE family only (the expert matrices)", st);
      if (q.hidden % 32 || q.expert_ffn % 32)
        return fail(DEC_E_SHAPE, "MXFP4 expert weights need hidden and expert_ffn multiples of 32", st);
    }
    if (q.weight_format == DEC_WEIGHTS_FP8_E4M3) {
      if (q.arch == DEC_ARCH_GQA && (q.hidden % 16 || q.ffn % 16 || (q.n_q_heads * q.head_dim) % 16))
        return fail(DEC_E_SHAPE, "FP8 weights need hidden, ffn and n_q_heads * head_dim multiples of 16", st);
      if (q.arch != DEC_ARCH_GQA && (q.hidden % 16 || q.ffn % 16 || q.q_lora_rank % 16 || (q.n_q_heads * q.v_head) % 16 ||
                                     q.expert_ffn % 16))
        return fail(DEC_E_SHAPE, "FP8 weights need hidden, ffn, q_lora_rank, n_q_heads * v_head and expert_ffn multiples of 16", st);
    }
    if (!(q.rms_eps > 0.f) || !(q.rope_theta > 1.0)) return fail(DEC_E_SHAPE, "need rms_eps > 0 and rope_theta > 1", st);
    if (n < 0) return fail(DEC_E_CAPACITY, "kv_len < 0", st);
    if (n > (1 << 22)) return fail(DEC_E_CAPACITY, "kv_len above 4194304", st);
    if (nt < 1 || nt > kMaxVerifyTokens) return fail(DEC_E_INVAL, "tokens per step must be 1.." + std::to_string(kMaxVerifyTokens), st);
    if (nt > 1 && (q.arch != DEC_ARCH_GQA || q.weight_format != DEC_WEIGHTS_BF16 || dyn))
      return fail(DEC_E_SHAPE, "verification steps: GQA family, bf16 weights, fixed length only", st);
    if (q.arch == DEC_ARCH_GQA) {
      if (q.n_q_heads < 1 || q.n_kv_heads < 1 || q.n_q_heads % q.n_kv_heads)
        return fail(DEC_E_SHAPE, "GQA needs n_q_heads a positive multiple of n_kv_heads", st);
      if (q.n_q_heads / q.n_kv_heads > 4) return fail(DEC_E_SHAPE, "more than 4 query heads per KV head", st);
      if (q.head_dim != 32 && q.head_dim != 64 && q.head_dim != 128 && q.head_dim != 256)
        return fail(DEC_E_SHAPE, "head_dim must be 32, 64, 128 or 256", st);
      if (q.ffn < 8 || q.ffn % 8) return fail(DEC_E_SHAPE, "ffn must be a positive multiple of 8", st);
      if (q.q_lora_rank || q.kv_lora_rank || q.qk_nope || q.qk_rope || q.v_head || q.n_routed || q.n_shared || q.top_k || q.expert_ffn)
        return fail(DEC_E_SHAPE, "GQA shape with MLA/MoE fields set", st);
    } else if (q.arch == DEC_ARCH_MLA || q.arch == DEC_ARCH_MOE) {
      if (q.n_q_heads < 1 || q.n_q_heads > kMlaHeads) return fail(DEC_E_SHAPE, "MLA needs 1..16 query heads", st);
      if (q.n_kv_heads || q.head_dim) return fail(DEC_E_SHAPE, "MLA shape with GQA fields set", st);
      if (q.q_lora_rank < 8 || q.q_lora_rank % 8) return fail(DEC_E_SHAPE, "q_lora_rank must be a positive multiple of 8", st);
      if (q.kv_lora_rank < kMlaColBlock || q.kv_lora_rank % kMlaColBlock || q.kv_lora_rank > 512)
        return fail(DEC_E_SHAPE, "kv_lora_rank must be a multiple of 64, at most 512", st);
      if (q.qk_nope < 8 || q.qk_nope % 8 || q.qk_rope < 8 || q.qk_rope % 8 || q.qk_rope > 128)
        return fail(DEC_E_SHAPE, "qk_nope and qk_rope must be multiples of 8 (qk_rope <= 128)", st);
      if (q.v_head < 8 || q.v_head % 8) return fail(DEC_E_SHAPE, "v_head must be a positive multiple of 8", st);
      if (q.arch == DEC_ARCH_MLA) {
        if (q.ffn < 8 || q.ffn % 8) return fail(DEC_E_SHAPE, "ffn must be a positive multiple of 8", st);
        if (q.n_routed || q.n_shared || q.top_k || q.expert_ffn) return fail(DEC_E_SHAPE, "MLA shape with MoE fields set", st);
      } else {
        if (q.ffn) return fail(DEC_E_SHAPE, "MoE shape with a dense ffn", st);
        if (q.n_routed < 1 || q.top_k < 1 || q.top_k > q.n_routed || q.top_k > 64 || q.n_routed > 4096)
          return fail(DEC_E_SHAPE, "MoE needs 1 <= top_k <= min(n_routed, 64), n_routed <= 4096", st);
        if (q.n_shared < 0 || q.expert_ffn < 8 || q.expert_ffn % 8) return fail(DEC_E_SHAPE, "bad n_shared / expert_ffn", st);
      }
    } else {
      return fail(DEC_E_SHAPE, "unknown arch", st);
    }
    return true;
  }

  void add_weight(const std::string& name, int32_t dtype, std::vector<int64_t> dims) {
    int64_t e = 1;
    for (auto d : dims) e *= d;
    const int64_t es = dtype == DEC_DTYPE_BF16 ? 2 : (dtype == DEC_DTYPE_FP8 || dtype == DEC_DTYPE_FP4X2 || dtype == DEC_DTYPE_E8M0) ? 1 : 4;
    P.weights.push_back({name, dtype, dims, e * es});
  }
  bool fp8() const { return s.weight_format == DEC_WEIGHTS_FP8_E4M3; }
  bool mx4() const { return s.weight_format == DEC_WEIGHTS_MXFP4; }
  // An expert matrix [.., rows, cols]: bf16, or MXFP4 (packed pairs [.., rows, cols / 2]) followed
  // by its E8M0 block scales [.., rows, cols / 32] (the engine finds them at the index + 1).
  void add_expert(const std::string& name, std::vector<int64_t> dims) {
    if (fp8()) {  // E4M3 bytes and one fp32 scale per row of every expert
      std::vector<int64_t> sc(dims.begin(), dims.end() - 1);
      add_weight(name, DEC_DTYPE_FP8, dims);
      add_weight(name + ".scale", DEC_DTYPE_FP32, sc);
      return;
    }
    if (!mx4()) {
      add_weight(name, DEC_DTYPE_BF16, dims);
      return;
    }
    std::vector<int64_t> q = dims, sc = dims;
    q.back() /= 2;
    sc.back() /= 32;
    add_weight(name, DEC_DTYPE_FP4X2, q);
    add_weight(name + ".scale", DEC_DTYPE_E8M0, sc);
  }
  // A linear matrix [rows][cols]: bf16, or FP8 bytes followed by the fp32 row scales (the
  // engine finds the scales at the matrix's weight index + 1).
  void add_matrix(const std::string& name, int64_t rows, int64_t cols) {
    if (!fp8()) {
      add_weight(name, DEC_DTYPE_BF16, {rows, cols});
      return;
    }
    add_weight(name, DEC_DTYPE_FP8, {rows, cols});
    add_weight(name + ".scale", DEC_DTYPE_FP32, {rows});
  }

  // Canonical weight order: the bind order of the ABI.
  void weight_list(std::vector<LayerDesc>& L) {
    const int d = s.hidden;
    for (int l = 0; l < s.n_layers; ++l) {
      std::string p = "layers." + std::to_string(l) + ".";
      LayerDesc& ld = L[l];
      for (int i = 0; i < LW_COUNT; ++i) ld.w[i] = -1;
      auto W = [&](int slot, const std::string& nm, int32_t dt, std::vector<int64_t> dims) {
        ld.w[slot] = (int)P.weights.size();
        add_weight(p + nm, dt, dims);
      };
      auto M = [&](int slot, const std::string& nm, int64_t rows, int64_t cols) {
        ld.w[slot] = (int)P.weights.size();
        add_matrix(p + nm, rows, cols);
      };
      if (s.arch == DEC_ARCH_GQA) {
        W(LW_ATTN_NORM, "attn_norm", DEC_DTYPE_BF16, {d});
        M(LW_WQ, "wq", (int64_t)s.n_q_heads * s.head_dim, d);
        M(LW_WK, "wk", (int64_t)s.n_kv_heads * s.head_dim, d);
        M(LW_WV, "wv", (int64_t)s.n_kv_heads * s.head_dim, d);
        M(LW_WO, "wo", d, (int64_t)s.n_q_heads * s.head_dim);
      } else {
        const int nh = s.n_q_heads;
        W(LW_ATTN_NORM, "attn_norm", DEC_DTYPE_BF16, {d});
        // (FP8: every linear matrix but the per-head absorption matrices and the router)
        M(LW_WQA, "wq_a", s.q_lora_rank, d);
        W(LW_QNORM, "q_norm", DEC_DTYPE_BF16, {s.q_lora_rank});
        M(LW_WQB, "wq_b", (int64_t)nh * (s.qk_nope + s.qk_rope), s.q_lora_rank);
        M(LW_WKVA, "wkv_a", s.kv_lora_rank + s.qk_rope, d);
        W(LW_KVNORM, "kv_norm", DEC_DTYPE_BF16, {s.kv_lora_rank});
        W(LW_WUK, "w_uk", DEC_DTYPE_BF16, {nh, s.qk_nope, s.kv_lora_rank});
        W(LW_WUV, "w_uv", DEC_DTYPE_BF16, {nh, s.v_head, s.kv_lora_rank});
        M(LW_WO, "wo", d, (int64_t)nh * s.v_head);
        if (s.index_heads > 0) {  // the sparse indexer's matrices
          W(LW_IDXQ, "idx_wq", DEC_DTYPE_BF16, {(int64_t)s.index_heads * s.index_dim, s.q_lora_rank});
          W(LW_IDXK, "idx_wk", DEC_DTYPE_BF16, {s.index_dim, d});
          W(LW_IDXW, "idx_w", DEC_DTYPE_BF16, {s.index_heads, d});
        }
      }
      W(LW_FFN_NORM, "ffn_norm", DEC_DTYPE_BF16, {d});
      if (s.arch == DEC_ARCH_MOE) {
        const int64_t E = s.n_routed, F = s.expert_ffn, S = (int64_t)s.n_shared * s.expert_ffn;
        W(LW_ROUTER, "router", DEC_DTYPE_BF16, {E, d});
        W(LW_RBIAS, "router_bias", DEC_DTYPE_FP32, {E});
        auto X = [&](int slot, const std::string& nm, std::vector<int64_t> dims) {
          ld.w[slot] = (int)P.weights.size();
          add_expert(p + nm, dims);
        };
        X(LW_EGATE, "experts.w_gate", {E, F, d});
        X(LW_EUP, "experts.w_up", {E, F, d});
        X(LW_EDOWN, "experts.w_down", {E, d, F});
        X(LW_SGATE, "shared.w_gate", {S, d});
        X(LW_SUP, "shared.w_up", {S, d});
        X(LW_SDOWN, "shared.w_down", {d, S});
      } else {
        M(LW_GATE, "w_gate", s.ffn, d);
        M(LW_UP, "w_up", s.ffn, d);
        M(LW_DOWN, "w_down", d, s.ffn);
      }
    }
    if (s.vocab > 0) {
      P.w_final_norm = (int)P.weights.size();
      add_weight("final_norm", DEC_DTYPE_BF16, {d});
      P.w_lm_head = (int)P.weights.size();
      add_matrix("lm_head", s.vocab, d);
      if (dyn) {  // a step without an input vector starts from its token's embedding row
        P.w_embed = (int)P.weights.size();
        add_weight("embed", DEC_DTYPE_BF16, {s.vocab, d});
      }
    }
  }

  // An attention split whose workgroup runs the same layer's QKV task just before it gets
  // its cached K/V rows staged into LDS by that task (QKV: a3 = group, a4 = split index,
  // a5 = split count; attention: a3 = 1). Only where both LDS regions are already there and
  // the rows fit the fixed DMA count -- for a dynamic plan, the most rows a split has at any
  // position up to the largest; the split's other rows (at most the new position) are loaded
  // after the dependency wait.
  // The regions grow the LDS plan when the whole plan still fits the device; otherwise only
  // splits that fit the regions other stages already need are staged.
  void stage_attention_kv() {
    const int hd = s.head_dim;
    const int64_t koff = kv_stage_k_off(s.hidden, (int)chunk_cols()), voff = kv_stage_v_off(hd);
    auto candidate = [&](const TaskDesc& q, const TaskDesc& a) -> int64_t {  // LDS floats per region, or 0
      if (a.type != T_ATTN || q.type != T_QKV || q.layer != a.layer) return 0;
      const int64_t cnt = dyn ? (n + 1 + a.a2 - 1) / a.a2 : (int64_t)split_cached(n, a.a1, a.a2);
      if (cnt <= 0) return 0;
      if (2 * ((cnt * hd / 2 + 255) / 256) > (int64_t)(kWaves - 1) * kKvStageDma) return 0;
      // the matrix-core attention merges its waves below the V rows (kWaves x 4 x (hd + 4)
      // floats, the region's offset) and assembles the partial (r x (hd + 4)) below the K rows
      const int64_t r = s.n_q_heads / s.n_kv_heads;
      if (r * (hd + 4) > koff) return 0;
      return align_up((cnt + 1) * hd / 2, 256);  // + the new row; DMA granularity
    };
    int64_t need = 0;
    for (int w = 0; w < n_wg; ++w)
      for (size_t i = 1; i < per_wg[w].size(); ++i)
        need = std::max(need, candidate(per_wg[w][i - 1].d, per_wg[w][i].d));
    if (need == 0) return;
    const int64_t xs2 = std::max(xs_floats_max, koff + need), scr2 = std::max(scratch_floats, voff + need);
    if (align_up(4 * lds_floats(xs2, scr2), 1024) <= dev.lds_bytes_per_cu) {
      xs_floats_max = xs2;
      scratch_floats = scr2;
    }
    for (int w = 0; w < n_wg; ++w)
      for (size_t i = 1; i < per_wg[w].size(); ++i) {
        TaskDesc& a = per_wg[w][i].d;
        TaskDesc& q = per_wg[w][i - 1].d;
        const int64_t fl = candidate(q, a);
        if (fl == 0 || koff + fl > xs_floats_max || voff + fl > scratch_floats) continue;
        q.a3 = a.a0;
        q.a4 = a.a1;
        q.a5 = a.a2;
        a.a3 = 1;
      }
  }
  // LDS floats of the GQA plan: header, staged vector, row results, row tables, gains, scratch
  int64_t lds_floats(int64_t xs, int64_t scr) const {
    const int64_t gmax = std::max<int64_t>({(int64_t)s.hidden, (int64_t)s.q_lora_rank, (int64_t)s.kv_lora_rank});
    // (+ the FP8 row-scale table: kMaxTaskRows floats; MXFP4: a scale pointer per row)
    return 64 + xs + kYsFloats + (int64_t)kMaxTaskRows * (fp8() ? 16 : mx4() ? 20 : 12) / 4 + align_up(gmax / 2, 256) + scr;
  }

  // ---------------------------------------------------------------- GQA layer stages
  std::vector<int32_t> hinit_deps;  // layer 0: counters of the h = x init tasks
  std::vector<int64_t> h_acc;       // GQA: per-layer h accumulators

  std::vector<int32_t> build_gqa_layer(int l, std::vector<int32_t> prev, int64_t x_in) {
    LayerDesc& L = P.layers[l];
    const int d = s.hidden, nq = s.n_q_heads, nkv = s.n_kv_heads, hd = s.head_dim, f = s.ffn;
    const int r = nq / nkv;
    std::string p = "layers." + std::to_string(l) + ".";
    for (int i = 0; i < LA_COUNT; ++i) L.act[i] = -1;
    L.act[LA_X_IN] = (int)x_in;
    L.act[LA_Q] = (int)act_t(p + "q", (int64_t)nq * hd);
    L.act[LA_KVNEW] = (int)act_t(p + "kv_new", 2LL * nkv * hd);
    L.act[LA_ATTN] = (int)act_t(p + "attn", (int64_t)nq * hd);
    L.act[LA_H] = (int)h_acc[l];
    L.act[LA_ACT] = (int)act_t(p + "ffn_act", f);
    L.act[LA_FFN_OUT] = (int)act_t(p + "ffn_out", d);
    L.act[LA_X_OUT] = (int)act_t(p + "x_out", d);
    if (nt == 1) {
      need_xs(d); need_xs((int64_t)nq * hd); need_xs(f);
    } else {
      need_xs_t(d, true); need_xs_t((int64_t)r * hd, true); need_xs_t(f, false);
      // the attention stages its query columns in xs (each copy lands in 256-float blocks)
      // and assembles its split record there
      xs_floats_max = std::max<int64_t>(xs_floats_max, align_up((int64_t)kMaxVerifyCols * (hd + 4) + 256, 256));
    }
    auto sets = xcd_sets(nkv);

    // QKV: per KV group g, units = (r q heads + k + v) * hd/2 RoPE row pairs.
    ++stage;
    const int qkv = counter(nkv);
    const int U = (r + 2) * hd / 2;
    for (int g = 0; g < nkv; ++g)
      spread(sets[g], U, rows_cap() / 2, [&](int w, int a, int b) { add(w, T_QKV, l, a, b, prev, qkv + g, -1, g); });

    // attention splits over the n + nt positions: one per workgroup of the group's set, or,
    // in a verification step whose group has more than kMaxVerifyCols query columns (nt * r),
    // one task per (split, block of kMaxVerifyCols columns) on consecutive workgroups of the
    // set (one XCD: the column blocks of a split read the same K/V rows)
    ++stage;
    const int att = counter(nkv);
    const int C = nt * r;                                          // query columns per group
    const int CG = nt > 1 ? (C + kMaxVerifyCols - 1) / kMaxVerifyCols : 1;  // column blocks
    const int64_t npos = n + nt;
    int smax = 1;
    std::vector<int> S(nkv);
    for (int g = 0; g < nkv; ++g) {
      // the O-projection merges a group's partials from one LDS burst: cap the split count
      const int64_t cap = std::max<int64_t>(1, kMergeFloats / ((int64_t)C * (hd + 4)));
      S[g] = (int)std::min<int64_t>({std::max<int64_t>(1, (int64_t)sets[g].size() / CG), cap,
                                     std::max<int64_t>(1, (npos + kMinPosPerSplit - 1) / kMinPosPerSplit)});
      smax = std::max(smax, S[g]);
    }
    const int64_t pstride = (int64_t)C * (hd + 4);  // per split: C x (m, l, pad, pad, acc[hd])
    const int64_t part = act(p + "attn_partials", (int64_t)nkv * smax * pstride);
    L.act[LA_PART] = (int)part;
    // attention task: one partial per wave, per-wave stride sized for up to 4 heads (a
    // verification step's: kMaxVerifyCols columns)
    scratch_floats = std::max<int64_t>(scratch_floats, (int64_t)kWaves * (nt > 1 ? kMaxVerifyCols : 4) * (hd + 4) + 64);
    scratch_floats = std::max<int64_t>(scratch_floats, align_up((int64_t)smax * pstride, 256) + (int64_t)smax * C + 64);
    for (int g = 0; g < nkv; ++g)
      for (int sp = 0; sp < S[g]; ++sp) {
        int p0 = (int)(npos * sp / S[g]), p1 = (int)(npos * (sp + 1) / S[g]);
        for (int cg = 0; cg < CG; ++cg)
          add(sets[g][(sp * CG + cg) % sets[g].size()], T_ATTN, l, p0, p1, {qkv + g}, att + g, -1, g, sp, S[g], 0,
              (int)(part + (int64_t)g * smax * pstride), cg);
      }

    // per group: merge the group's splits, then W_o rows x the group's r*hd columns (split-K
    // over groups), added into h, which holds the residual x already (written by the previous
    // layer's down tasks, or by the layer-0 init tasks)
    ++stage;
    const int ctr_o = counter(nsc);
    for (int g = 0; g < nkv; ++g) {
      std::vector<int32_t> dg = {att + g};
      dg.insert(dg.end(), hinit_deps.begin(), hinit_deps.end());
      spread(sets[g], d, rows_cap(), [&](int w, int a, int b) {
        add(w, T_OPROJ_G, l, a, b, dg, ctr_o + slot(w), -1, g, 0, S[g], 0, (int)(part + (int64_t)g * smax * pstride));
      });
    }
    return ffn_dense(l, all_of(ctr_o, nsc));
  }

  std::vector<int32_t> ffn_dense(int l, std::vector<int32_t> deps_h) {
    const int d = s.hidden, f = s.ffn;
    ++stage;
    const int ctr_gu = counter(nsc);
    spread_weighted(all_wgs(), f, rows_cap() / 2, [&](int w, int a, int b) { add(w, T_GATEUP, l, a, b, deps_h, ctr_gu + slot(w)); });
    ++stage;
    const int ctr_dn = counter(nsc);
    const int last = (l == s.n_layers - 1 && s.vocab == 0) ? 1 : 0;
    const int hnext = (s.arch == DEC_ARCH_GQA && l + 1 < s.n_layers) ? (int)h_acc[l + 1] : -1;
    spread(all_wgs(), d, rows_cap(), [&](int w, int a, int b) {
      add(w, T_DOWN, l, a, b, all_of(ctr_gu, nsc), ctr_dn + slot(w), -1, last, hnext);
    });
    return all_of(ctr_dn, nsc);
  }

  // ---------------------------------------------------------------- MLA / MoE layer stages
  std::vector<int32_t> build_mla_layer(int l, std::vector<int32_t> prev, int64_t x_in) {
    LayerDesc& L = P.layers[l];
    const int d = s.hidden, nh = s.n_q_heads, ql = s.q_lora_rank, kl = s.kv_lora_rank;
    const int dn = s.qk_nope, dr = s.qk_rope, dv = s.v_head;
    const int KR = kl + dr, KP = (int)align_up(KR, 32), NKS = KP / 32;
    std::string p = "layers." + std::to_string(l) + ".";
    for (int i = 0; i < LA_COUNT; ++i) L.act[i] = -1;
    L.act[LA_X_IN] = (int)x_in;
    L.act[LA_CQ] = (int)act(p + "cq_raw", ql);
    L.act[LA_KVA] = (int)act(p + "kv_a", KR);
    L.act[LA_QNOPE] = (int)act(p + "q_nope", (int64_t)nh * dn);
    L.act[LA_QROPE] = (int)act(p + "q_rope", (int64_t)nh * dr);
    L.act[LA_KVNEW] = (int)act(p + "kv_new", KR);
    L.act[LA_QABS] = (int)act(p + "q_abs", (int64_t)nh * kl);
    L.act[LA_QOP] = (int)act(p + "q_operand", (int64_t)NKS * 512, DEC_DTYPE_I32);
    L.act[LA_OLAT] = (int)act(p + "o_lat", (int64_t)nh * kl);
    L.act[LA_ATTN] = (int)act(p + "attn", (int64_t)nh * dv);
    L.act[LA_H] = (int)act(p + "h", d);
    L.act[LA_FFN_OUT] = (int)act(p + "ffn_out", d);
    L.act[LA_X_OUT] = (int)act(p + "x_out", d);
    need_xs(d); need_xs(ql); need_xs(KR); need_xs((int64_t)nh * dv);
    const int HI = s.index_heads, DI = HI ? s.index_dim : 0;
    const int64_t m_sel = HI ? std::min<int64_t>(s.index_topk, n + 1) : n + 1;  // positions attention reads
    if (HI) {
      L.act[LA_IDXK] = (int)act(p + "idx_k", DI);
      L.act[LA_IDXW] = (int)act(p + "idx_w", HI);
      L.act[LA_IDXQ] = (int)act(p + "idx_q", (int64_t)HI * DI);
      L.act[LA_IDXS] = (int)act(p + "idx_scores", n + 1);
      L.act[LA_IDXSEL] = (int)act(p + "idx_sel", m_sel, DEC_DTYPE_I32);
      // score task: the queries (fp32), their MFMA operand (bf16 hi + lo, 16-head tiles), weights
      need_xs((int64_t)HI * DI + (int64_t)((HI + 15) / 16) * (DI / 32) * 2 * 256 + 64);
    }

    // A: [W_DQ; W_DKV] rows from the normalised layer input (with the indexer: then the rows of
    // W_k and W_w, whose results are the new index key and the head weights)
    ++stage;
    const int ca = counter(nsc);
    spread(all_wgs(), ql + KR + DI + HI, kRowsCap, [&](int w, int a, int b) { add(w, T_MLA_A, l, a, b, prev, ca + slot(w)); });
    auto da = all_of(ca, nsc);

    // B: W_UQ row pairs (nope pairs, then RoPE pairs, per head); the latent-cache append
    // (which also clears the attention output that the W_UV tasks accumulate into)
    ++stage;
    const int cb = counter(nsc), ckv = counter(1);
    const int UH = dn / 2 + dr / 2;
    // the append runs alone on the last workgroup, so that no W_UQ task (which every absorb
    // task waits for) queues behind it
    add(n_wg - 1, T_MLA_KVAPP, l, 0, KR, da, ckv);
    std::vector<int> bw = all_wgs();
    if (n_wg > 1) bw.pop_back();
    // the sparse indexer's query rows go ahead of W_UQ in each list: the scores and the
    // selection after them are the longer path to the attention (the absorb tasks after W_UQ
    // finish well before the selection)
    const int cq = HI ? counter(nsc) : -1;
    if (HI) spread(bw, HI * DI, kRowsCap, [&](int w, int a, int b) { add(w, T_IDX_Q, l, a, b, da, cq + slot(w)); });
    spread(bw, nh * UH, kRowsCap / 2, [&](int w, int a, int b) { add(w, T_MLA_B, l, a, b, da, cb + slot(w)); });
    auto db = all_of(cb, nsc);

    // the sparse indexer: index-query rows (above), scores of every position, the top-T
    int ctop = -1;
    if (HI) {
      ++stage;
      const int csc = counter(nsc);
      std::vector<int32_t> dsc = da;
      auto dq = all_of(cq, nsc);
      dsc.insert(dsc.end(), dq.begin(), dq.end());
      // positions [0, n] in NS ranges, cut at run time from the step's position (a plan with a
      // per-step length scores fewer positions at smaller positions)
      const int NS = (int)std::min<int64_t>(n_wg, std::max<int64_t>(1, (n + 1 + kIdxPos - 1) / kIdxPos));
      for (int i = 0; i < NS; ++i) {
        const int w = (int)((int64_t)i * n_wg / NS);
        add(w, T_IDX_SCORE, l, (int)((n + 1) * i / NS), (int)((n + 1) * (i + 1) / NS), dsc, csc + slot(w), -1, 0, i, NS);
      }
      // top-T: the scores in LDS in chunks of C (all of them when they fit beside the histogram
      // and the scan words, in the LDS region after the header)
      ++stage;
      ctop = counter(1);
      const int64_t room = ((int64_t)dev.lds_bytes_per_cu / 4 - 64 - kIdxBins - 64) / 256 * 256;
      // (a device with less LDS than that fails the plan's LDS check)
      const int64_t C = std::min<int64_t>(align_up(n + 1, 256), std::max<int64_t>(room, 256));
      add(n_wg - 1, T_IDX_TOPK, l, 0, (int)(n + 1), all_of(csc, nsc), ctop, -1, (int)C);
      mla_lds = std::max<int64_t>(mla_lds, C + kIdxBins + 64);
    }

    // absorb: q_abs[h][c-block] = W_UK[h]^T q_nope[h], one (head, 64-column block) per task
    ++stage;
    const int cabs = counter(nsc);
    const int nblk = nh * (kl / kMlaColBlock);
    // (with the indexer, not on the top-T workgroup: every attention split waits for every
    // absorb task, and one queued behind the selection would hold them all)
    spread(HI ? bw : all_wgs(), nblk, 1, [&](int w, int a, int b) { add(w, T_MLA_ABSORB, l, a, b, db, cabs + slot(w)); });

    // latent attention: S position splits, all heads folded into one MFMA tile
    ++stage;
    const int catt = counter(nsc);
    const int minpos = HI ? kMinPosMlaSparse : kMinPosMla;
    const int S = (int)std::min<int64_t>(n_wg, std::max<int64_t>(1, (m_sel + minpos - 1) / minpos));
    const int Sp = (S + 1) & ~1;  // per-head stride of the (M, Lr) table (16-byte rows)
    const int64_t pml = act(p + "attn_ml", (int64_t)nh * Sp * 2);
    const int64_t part = act(p + "attn_partials", (int64_t)S * nh * kl);
    L.act[LA_PML] = (int)pml;
    L.act[LA_PART] = (int)part;
    std::vector<int32_t> dat = all_of(cabs, nsc);
    dat.insert(dat.end(), db.begin(), db.end());
    dat.push_back(ckv);
    if (HI) dat.push_back(ctop);
    // (with the indexer a split is a range of the selected-position list, not of positions)
    for (int sp = 0; sp < S; ++sp) {
      int w = (int)((int64_t)sp * n_wg / S);
      // the indexer's few splits gather scattered rows: one per XCD in turn (workgroup w runs
      // on XCD w mod n_xcd), not every split on the XCDs an even stride lands on
      if (HI && n_xcd > 0 && (int64_t)n_xcd * ((S + n_xcd - 1) / n_xcd) <= n_wg) w = (sp % n_xcd) + n_xcd * (sp / n_xcd) * (n_wg / n_xcd / ((S + n_xcd - 1) / n_xcd));
      int p0 = (int)(m_sel * sp / S), p1 = (int)(m_sel * (sp + 1) / S);
      add(w, T_MLA_ATTN, l, p0, p1, dat, catt + slot(w), -1, 0, sp, S, 0, (int)pml, (int)part);
    }
    // LDS: q operand + one latent chunk + P operand + softmax statistics (+ the split's slice
    // of the selected positions)
    mla_lds = std::max<int64_t>(mla_lds, (int64_t)NKS * 512 + (int64_t)kMlaChunk * KP / 2 + (kMlaChunk / 32) * 512 + 256 +
                                             (HI ? align_up((m_sel + S - 1) / S + 1, 64) : 0));

    // W_UV: per (head, column block) merge the splits, multiply, add into o[h]
    ++stage;
    const int cuv = counter(nsc);
    spread(all_wgs(), nblk, 1, [&](int w, int a, int b) {
      add(w, T_MLA_UV, l, a, b, all_of(catt, nsc), cuv + slot(w), -1, 0, 0, S, 0, (int)pml, (int)part);
    });
    mla_lds = std::max<int64_t>(mla_lds, align_up(2LL * Sp, 256) + align_up(S, 4) / 4 * 256 + align_up(S, 64) + 8 * 64 + 64);

    // O projection + residual
    ++stage;
    const int co = counter(nsc);
    spread(all_wgs(), d, kRowsCap, [&](int w, int a, int b) { add(w, T_OPROJ, l, a, b, all_of(cuv, nsc), co + slot(w)); });
    auto dh = all_of(co, nsc);

    if (s.arch == DEC_ARCH_MLA) {
      L.act[LA_ACT] = (int)act(p + "ffn_act", s.ffn);
      need_xs(s.ffn);
      return ffn_dense(l, dh);
    }
    return ffn_moe(l, dh);
  }

  std::vector<int32_t> ffn_moe(int l, std::vector<int32_t> dh) {
    LayerDesc& L = P.layers[l];
    const int d = s.hidden, E = s.n_routed, K = s.top_k, F = s.expert_ffn, SF = s.n_shared * s.expert_ffn;
    std::string p = "layers." + std::to_string(l) + ".";
    L.act[LA_RLOGIT] = (int)act(p + "router_logits", E);
    L.act[LA_TOPK] = (int)act(p + "topk", 2LL * K, DEC_DTYPE_I32);
    L.act[LA_SACT] = (int)act(p + "shared_act", std::max(SF, 1));
    L.act[LA_ACT] = (int)act(p + "expert_act", (int64_t)K * F);
    if (!mx4()) {
      need_xs((int64_t)(s.n_shared + K) * align_up(F, chunk_cols()));
    } else {
      // MXFP4 segments are padded to 256 columns (the staging copy's unit); a wave's
      // 2048-column chunk may read past the last segment (those lanes' products are dropped),
      // and the gate/up input is padded to 2048 columns
      need_xs((int64_t)(s.n_shared + K - 1) * align_up(F, 256) + 2048);
      need_xs(align_up(d, 2048));
    }
    need_xs(3 * align_up(E, 256));  // top-k: z, sigma, bias

    // E1: router rows on a few workgroups, the shared expert's gate/up on the rest
    ++stage;
    const int cr = counter(nsc), cs = counter(nsc);
    int nr = std::max(1, std::min(n_wg / 4, (E + 3) / 4));
    if (SF == 0) nr = n_wg;
    std::vector<int> rw, sw;
    for (int w = 0; w < n_wg; ++w) (w < nr ? rw : sw).push_back(w);
    spread(rw, E, kRowsCap, [&](int w, int a, int b) { add(w, T_ROUTER, l, a, b, dh, cr + slot(w)); });
    if (SF > 0) spread(sw, SF, kRowsCap / 2, [&](int w, int a, int b) { add(w, T_SHARED_GU, l, a, b, dh, cs + slot(w)); });

    // E2: top-k on one workgroup
    ++stage;
    const int ct = counter(1);
    add(nr - 1, T_TOPK, l, 0, E, all_of(cr, nsc), ct);

    // E3: routed experts' gate/up (the expert id is read from the top-k result)
    ++stage;
    const int ce = counter(nsc);
    // a2 = 1: the first dependency (the top-k) decides the rows, which are prefetched before
    // the rest of the wait
    spread(all_wgs(), K * F, kRowsCap / 2, [&](int w, int a, int b) { add(w, T_EXPERT_GU, l, a, b, {ct}, ce + slot(w), -1, 0, 0, 1); });

    // E4: down projections of the shared and routed experts, weighted, + residual
    ++stage;
    const int cd = counter(nsc);
    std::vector<int32_t> dd = {ct};  // first: the top-k, which decides the rows (a2 = 1)
    auto de_ = all_of(ce, nsc), ds_ = all_of(cs, nsc);
    dd.insert(dd.end(), de_.begin(), de_.end());
    dd.insert(dd.end(), ds_.begin(), ds_.end());
    const int last = (l == s.n_layers - 1 && s.vocab == 0) ? 1 : 0;
    spread(all_wgs(), d, kRowsCap / (s.n_shared + K), [&](int w, int a, int b) { add(w, T_MOE_DOWN, l, a, b, dd, cd + slot(w), -1, last, 0, 1); });
    return all_of(cd, nsc);
  }

  bool run(dec_status* st) {
    if (!check_shape(st)) return false;
    if (dev.gfx_arch != 950) return fail(DEC_E_DEVICE, "device is not gfx950", st);
    if (dev.n_cu < 1 || dev.n_xcd < 1 || dev.n_cu % dev.n_xcd) return fail(DEC_E_DEVICE, "bad CU/XCD counts", st);
    n_wg = dev.n_cu;
    n_xcd = dev.n_xcd;
    nsc = (int)std::min<int64_t>(n_wg, align_up(std::max(n_xcd, kStageCounters), n_xcd));
    per_wg.assign(n_wg, {});
    P.shape = s;
    P.kv_len = n;
    P.dynamic = dyn;
    P.ntok = nt;
    P.dev = dev;
    P.n_wg = n_wg;
    P.layers.assign(s.n_layers, LayerDesc{});
    weight_list(P.layers);

    std::vector<int32_t> prev;
    int64_t x_in = -1;
    if (s.arch == DEC_ARCH_GQA) {
      // h accumulators: allocated up front so each layer's down tasks can initialise the next
      for (int l = 0; l < s.n_layers; ++l) P.layers[l].act[LA_H] = -1;
      for (int l = 0; l < s.n_layers; ++l) h_acc.push_back(act_t("layers." + std::to_string(l) + ".h", s.hidden));
      ++stage;
      const int ci = counter(nsc);
      spread(all_wgs(), s.hidden, kRowsCap, [&](int w, int a, int b) { add(w, T_HINIT, 0, a, b, {}, ci + slot(w), -1, (int)h_acc[0]); });
      hinit_deps = all_of(ci, nsc);
    }
    for (int l = 0; l < s.n_layers; ++l) {
      prev = (s.arch == DEC_ARCH_GQA) ? build_gqa_layer(l, prev, x_in) : build_mla_layer(l, prev, x_in);
      x_in = P.layers[l].act[LA_X_OUT];
    }
    P.x_final = (int)x_in;
    if (s.vocab > 0) {
      ++stage;
      if (!dyn) {
        spread_weighted(all_wgs(), s.vocab, rows_cap(), [&](int w, int a, int b) { add(w, T_LMHEAD, s.n_layers, a, b, prev, -1); });
      } else {
        // each LM-head task also leaves its best (logit, index) in slot a0; one task then
        // picks the step's token from those pairs
        const int ctr_lm = counter(nsc);
        int n_lm = 0;
        std::vector<std::tuple<int, int, int>> parts;
        spread_weighted(all_wgs(), s.vocab, kRowsCap, [&](int w, int a, int b) { parts.emplace_back(w, a, b); });
        const int64_t best = act("lm_best", 2LL * (int64_t)parts.size());
        for (auto& pt : parts)
          add(std::get<0>(pt), T_LMHEAD, s.n_layers, std::get<1>(pt), std::get<2>(pt), prev,
              ctr_lm + slot(std::get<0>(pt)), -1, n_lm++, (int)best);
        ++stage;
        add(0, T_ARGMAX, s.n_layers, 0, 1, all_of(ctr_lm, nsc), -1, -1, n_lm, (int)best);
      }
    }

    if (s.arch == DEC_ARCH_GQA && nt == 1) stage_attention_kv();

    // flatten per-workgroup lists, resolve dependency entries
    P.wg_begin.assign(n_wg + 1, 0);
    for (int w = 0; w < n_wg; ++w) {
      P.wg_begin[w] = (int)P.tasks.size();
      int pos = 0;
      for (auto& t : per_wg[w]) {
        if ((int)t.deps.size() > kMaxDepsPerTask) return fail(DEC_E_PLAN, "too many dependencies", st);
        t.d.dep_first = (int)P.deps.size();
        t.d.dep_count = (int)t.deps.size();
        for (int c : t.deps) P.deps.push_back({c, P.counter_total[c]});
        P.tasks.push_back(t.d);
        P.info.push_back({t.stage, w, pos++});
      }
    }
    P.wg_begin[n_wg] = (int)P.tasks.size();
    P.n_log = next_id;
    // number the stages that hold tasks 0, 1, ...; then, per workgroup, where each stage's
    // tasks begin in its list (lists are in stage order), so that a launch can run a range of
    // stages only
    {
      std::vector<int> used;
      for (auto& i : P.info) used.push_back(i.stage);
      std::sort(used.begin(), used.end());
      used.erase(std::unique(used.begin(), used.end()), used.end());
      for (auto& i : P.info) i.stage = (int32_t)(std::lower_bound(used.begin(), used.end(), i.stage) - used.begin());
      P.n_stages = (int32_t)used.size();
    }
    P.stage_first.assign((size_t)n_wg * (P.n_stages + 1), 0);
    for (int w = 0; w < n_wg; ++w) {
      int i = P.wg_begin[w];
      for (int sg = 0; sg <= P.n_stages; ++sg) {
        while (i < P.wg_begin[w + 1] && P.info[i].stage < sg) ++i;
        P.stage_first[(size_t)w * (P.n_stages + 1) + sg] = i;
      }
    }

    // RoPE table in double precision: the row of the step's position (a verification step: of
    // each of its positions n .. n + nt - 1), or (dynamic) one row per position 0..max_len
    const int rope_dim = (s.arch == DEC_ARCH_GQA) ? s.head_dim : s.qk_rope;
    P.rope_half = rope_dim / 2;
    P.rope_rows = dyn ? (int32_t)(n + 1) : nt;
    P.rope_cs.assign((size_t)P.rope_rows * 2 * P.rope_half, 0.f);
    for (int64_t row = 0; row < P.rope_rows; ++row) {
      const int64_t pos = dyn ? row : n + row;
      float* cs = P.rope_cs.data() + (size_t)row * 2 * P.rope_half;
      for (int i = 0; i < P.rope_half; ++i) {
        long double ang = (long double)pos * powl((long double)s.rope_theta, -2.0L * i / rope_dim);
        cs[i] = (float)cosl(ang);
        cs[P.rope_half + i] = (float)sinl(ang);
      }
    }
    const double qk = (s.arch == DEC_ARCH_GQA) ? s.head_dim : (s.qk_nope + s.qk_rope);
    P.attn_scale_log2 = (float)(1.0 / std::sqrt(qk) * 1.4426950408889634);

    // LDS: staged input vector + per-row results + reduction scratch
    const int64_t header = 64;  // LDS flag words ahead of the staged vector
    const int64_t gmax = std::max<int64_t>({(int64_t)s.hidden, (int64_t)s.q_lora_rank, (int64_t)s.kv_lora_rank});
    const int64_t gs = align_up(gmax / 2, 256);  // bf16 gains, DMA granularity 256 floats
    P.gs_floats = gs;
    int64_t lds = 4 * lds_floats(xs_floats_max, scratch_floats);
    if (s.arch != DEC_ARCH_GQA) {
      // the latent-attention, absorb and W_UV tasks use the whole region after the header
      const int64_t absorb = align_up(s.qk_nope, 256) + (int64_t)kMlaColBlock * 64 + 64;
      lds = std::max<int64_t>(lds, 4 * (header + std::max(mla_lds, absorb)));
    }
    lds = std::max<int64_t>(align_up(lds, 1024), kLdsMin);
    P.lds_bytes = (int32_t)lds;
    P.xs_floats = xs_floats_max;
    if (lds > dev.lds_bytes_per_cu) return fail(DEC_E_OCCUPANCY, "plan needs " + std::to_string(lds) + " B of LDS per workgroup", st);
    if (kThreads > dev.max_threads_per_cu) return fail(DEC_E_OCCUPANCY, "device runs fewer than 512 threads per CU", st);

    // workspace layout
    int64_t o = 0;
    auto take = [&](int64_t bytes) { int64_t r = o; o = align_up(o + bytes, 256); return r; };
    P.off_ctl = take(CTL_WORDS * 4);
    P.off_counters = take((int64_t)P.counter_total.size() * kCounterStride * 4);
    P.off_tasks = take((int64_t)P.tasks.size() * sizeof(TaskDesc));
    P.off_wgb = take((int64_t)(n_wg + 1) * 4);
    P.off_stf = take((int64_t)P.stage_first.size() * 4);
    P.off_deps = take((int64_t)std::max<size_t>(P.deps.size(), 1) * sizeof(DepEntry));
    P.off_wptr = take((int64_t)P.weights.size() * 8);
    P.off_layers = take((int64_t)P.layers.size() * sizeof(LayerDesc));
    P.off_rope = take((int64_t)P.rope_cs.size() * 4 + 4);
    P.off_log = take((int64_t)P.n_log * sizeof(TaskLog));
    P.off_act = take(act_floats * 4);
    P.ws_bytes = o;
    P.act_floats = act_floats;
    for (size_t i = 0; i < acts.size(); ++i)
      P.buffers.push_back({acts[i].first, acts[i].second.second, P.off_act + acts[i].second.first * 4, act_counts[i]});
    P.buffers.push_back({"task_log", DEC_DTYPE_I32, P.off_log, (int64_t)P.n_log * (int64_t)(sizeof(TaskLog) / 4)});
    P.buffers.push_back({"control", DEC_DTYPE_I32, P.off_ctl, CTL_WORDS});

    // bytes the method must read per step: every dense weight once (routed experts: only
    // the top_k chosen; the token embedding: one row), and positions [0, kv_len + ntok) of
    // the cache once
    P.weight_bytes = 0;
    for (auto& w : P.weights) P.weight_bytes += w.bytes;
    int64_t alg = P.weight_bytes;
    if (s.arch == DEC_ARCH_MOE) {  // the routed experts' bytes (matrices and block scales), per expert
      int64_t routed = 0;
      for (auto& w : P.weights)
        if (w.name.rfind("layers.0.experts.", 0) == 0) routed += w.bytes;
      alg -= (int64_t)s.n_layers * (s.n_routed - s.top_k) * (routed / s.n_routed);
    }
    if (P.w_embed >= 0)  // a step reads one row of the token embedding, not the table
      alg -= (int64_t)(s.vocab - 1) * s.hidden * 2;
    int64_t kv_row = (s.arch == DEC_ARCH_GQA) ? 2LL * s.n_kv_heads * s.head_dim * 2 : (int64_t)(s.kv_lora_rank + s.qk_rope) * 2;
    if (s.index_heads > 0)  // every position's index key, and the latent rows of the selected positions only
      alg += (int64_t)s.n_layers * ((n + 1) * (int64_t)s.index_dim * 2 + std::min<int64_t>(s.index_topk, n + 1) * kv_row);
    else
      alg += (int64_t)s.n_layers * (n + nt) * kv_row;
    P.alg_bytes = alg;

    std::string v = validate_plan(P);
    if (!v.empty()) return fail(DEC_E_PLAN, "plan validation: " + v, st);
    return true;
  }
};

}  // namespace

dec_status build_plan(const dec_model_shape& shape, int64_t kv_len, const dec_device_info& dev, PlanData* out,
                      std::string* err, bool dynamic, int ntok) {
  *out = PlanData{};
  dec_status st = DEC_OK;
  Builder b(shape, kv_len, dynamic, ntok, dev, *out, *err);
  if (!b.run(&st)) return st;
  return DEC_OK;
}

std::string validate_plan(const PlanData& p) {
  std::ostringstream e;
  const int nt = (int)p.tasks.size();
  // (1) each workgroup's list is in nondecreasing stage order
  for (int w = 0; w < p.n_wg; ++w)
    for (int i = p.wg_begin[w] + 1; i < p.wg_begin[w + 1]; ++i)
      if (p.info[i].stage < p.info[i - 1].stage) { e << "wg " << w << " list not in stage order"; return e.str(); }
  // (1b) an attention split with staged K/V rows directly follows the QKV task that stages
  //      them, in the same workgroup, for the same group, first position and row count
  for (int w = 0; w < p.n_wg; ++w)
    for (int i = p.wg_begin[w]; i < p.wg_begin[w + 1]; ++i) {
      const TaskDesc& a = p.tasks[i];
      if (a.type != T_ATTN || a.a3 == 0) continue;
      const TaskDesc* q = (i > p.wg_begin[w]) ? &p.tasks[i - 1] : nullptr;
      if (!q || q->type != T_QKV || q->layer != a.layer || q->a3 != a.a0 || q->a4 != a.a1 || q->a5 != a.a2 ||
          a.a3 != 1 || a.u0 != split_begin(p.kv_len, a.a1, a.a2) || a.u1 != split_begin(p.kv_len, a.a1 + 1, a.a2)) {
        e << "task " << a.id << ": staged K/V rows without a matching QKV task";
        return e.str();
      }
    }
  // (2) every counter waited on is produced only by tasks of earlier stages, and its
  //     per-step total equals its producers' count (merged counters: exactly one merge)
  std::vector<int> prod_stage_max(p.counter_total.size(), -1), prod_count(p.counter_total.size(), 0);
  std::vector<int> merge_count(p.counter_total.size(), 0);
  for (int i = 0; i < nt; ++i) {
    const TaskDesc& t = p.tasks[i];
    if (t.signal >= 0) {
      prod_stage_max[t.signal] = std::max(prod_stage_max[t.signal], p.info[i].stage);
      prod_count[t.signal]++;
    }
    if (t.signal2 >= 0) prod_stage_max[t.signal2] = std::max(prod_stage_max[t.signal2], p.info[i].stage);
  }
  std::set<int> merged;
  for (int i = 0; i < nt; ++i) if (p.tasks[i].signal2 >= 0) merged.insert(p.tasks[i].signal2);
  for (size_t c = 0; c < p.counter_total.size(); ++c) {
    uint32_t want = merged.count((int)c) ? 1u : (uint32_t)prod_count[c];
    if (p.counter_total[c] != want) { e << "counter " << c << " total " << p.counter_total[c] << " != producers " << want; return e.str(); }
  }
  for (int i = 0; i < nt; ++i) {
    const TaskDesc& t = p.tasks[i];
    if (t.dep_count > kMaxDepsPerTask) { e << "task " << t.id << " has too many deps"; return e.str(); }
    for (int k = 0; k < t.dep_count; ++k) {
      const DepEntry& d = p.deps[t.dep_first + k];
      if (d.counter < 0 || d.counter >= (int)p.counter_total.size()) { e << "task " << t.id << " bad counter"; return e.str(); }
      if (d.per_step == 0) { e << "task " << t.id << " waits on a counter nobody signals"; return e.str(); }
      if (prod_stage_max[d.counter] >= p.info[i].stage) { e << "task " << t.id << " waits on a same-or-later stage"; return e.str(); }
      if (d.per_step != p.counter_total[d.counter]) { e << "task " << t.id << " dep total mismatch"; return e.str(); }
    }
  }
  // (3) unit coverage: for each (layer, type[, group]) the tasks' [u0, u1) ranges tile the
  //     unit space exactly once
  struct Key { int layer, type, grp; bool operator<(const Key& o) const { return std::tie(layer, type, grp) < std::tie(o.layer, o.type, o.grp); } };
  std::map<Key, std::vector<std::pair<int, int>>> ranges;
  for (int i = 0; i < nt; ++i) {
    const TaskDesc& t = p.tasks[i];
    // (attention of a verification step: each column block tiles the positions once)
    int grp = (t.type == T_QKV || t.type == T_OPROJ_G) ? t.a0 : t.type == T_ATTN ? t.a0 * 64 + t.a5 : 0;
    ranges[{t.layer, t.type, grp}].push_back({t.u0, t.u1});
  }
  const dec_model_shape& s = p.shape;
  const int64_t n1 = p.kv_len + p.ntok;
  auto expected = [&](int type) -> int64_t {
    switch (type) {
      case T_QKV: return (int64_t)(s.n_q_heads / s.n_kv_heads + 2) * s.head_dim / 2;
      case T_ATTN: return n1;
      case T_MLA_ATTN: return s.index_heads ? std::min<int64_t>(s.index_topk, n1) : n1;  // (list entries with an indexer)
      case T_IDX_SCORE: case T_IDX_TOPK: return n1;
      case T_IDX_Q: return (int64_t)s.index_heads * s.index_dim;
      case T_OPROJ: case T_OPROJ_G: case T_DOWN: case T_MOE_DOWN: case T_HINIT: return s.hidden;
      case T_GATEUP: return s.ffn;
      case T_LMHEAD: return s.vocab;
      case T_ARGMAX: return 1;
      case T_MLA_A: return (int64_t)s.q_lora_rank + s.kv_lora_rank + s.qk_rope + (s.index_heads ? s.index_dim + s.index_heads : 0);
      case T_MLA_B: return (int64_t)s.n_q_heads * (s.qk_nope / 2 + s.qk_rope / 2);
      case T_MLA_KVAPP: return (int64_t)s.kv_lora_rank + s.qk_rope;
      case T_MLA_ABSORB: case T_MLA_UV: return (int64_t)s.n_q_heads * (s.kv_lora_rank / kMlaColBlock);
      case T_ROUTER: case T_TOPK: return s.n_routed;
      case T_SHARED_GU: return (int64_t)s.n_shared * s.expert_ffn;
      case T_EXPERT_GU: return (int64_t)s.top_k * s.expert_ffn;
    }
    return -1;
  };
  std::set<std::pair<int, int>> seen;  // (layer, type) present
  for (auto& kv : ranges) {
    auto v = kv.second;
    std::sort(v.begin(), v.end());
    int64_t at = 0;
    for (auto& r : v) {
      if (r.first != at || r.second <= r.first) { e << "coverage gap/overlap in layer " << kv.first.layer << " type " << kv.first.type; return e.str(); }
      at = r.second;
    }
    if (at != expected(kv.first.type)) { e << "coverage of type " << kv.first.type << " in layer " << kv.first.layer << " ends at " << at; return e.str(); }
    seen.insert({kv.first.layer, kv.first.type});
  }
  // every layer has its full set of stages
  std::vector<int> need;
  if (s.arch == DEC_ARCH_GQA) need = {T_QKV, T_ATTN, T_OPROJ_G, T_GATEUP, T_DOWN};
  else {
    need = {T_MLA_A, T_MLA_B, T_MLA_KVAPP, T_MLA_ABSORB, T_MLA_ATTN, T_MLA_UV, T_OPROJ};
    if (s.index_heads) { need.push_back(T_IDX_Q); need.push_back(T_IDX_SCORE); need.push_back(T_IDX_TOPK); }
    if (s.arch == DEC_ARCH_MLA) { need.push_back(T_GATEUP); need.push_back(T_DOWN); }
    else { need.push_back(T_ROUTER); need.push_back(T_TOPK); need.push_back(T_EXPERT_GU); need.push_back(T_MOE_DOWN);
           if (s.n_shared > 0) need.push_back(T_SHARED_GU); }
  }
  for (int l = 0; l < s.n_layers; ++l)
    for (int t : need)
      if (!seen.count({l, t})) { e << "layer " << l << " lacks task type " << t; return e.str(); }
  if (s.vocab > 0 && !seen.count({s.n_layers, (int)T_LMHEAD})) return "no LM head tasks";
  return "";
}

}  // namespace dec
