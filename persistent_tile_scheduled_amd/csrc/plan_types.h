// plan_types.h -- data shared by the host planner and the persistent engine kernel.
//
// The planner (planner.cpp) unrolls a whole decode step into tile tasks and writes, into
// the caller's workspace, the tables below; the engine (engine.hip) walks them. Nothing
// here depends on HIP, so the planner builds and is tested on a host without a GPU.
#pragma once
#include <stdint.h>

namespace dec {

constexpr int kThreads = 512;          // 8 wave64 per workgroup, one workgroup per CU
constexpr int kWaves = kThreads / 64;
constexpr int kChunkCols = 512;        // one wave-wide 16-byte load covers 512 bf16 columns
constexpr int kCounterStride = 32;     // u32 slots per counter (128 B: one counter per line)
constexpr int kMaxDepsPerTask = 64;    // one poller lane per dependency counter
constexpr int kYsFloats = 1024;        // per-task GEMV row results staged in LDS
constexpr int kMaxTaskRows = 1024;     // rows of one GEMV task (row-pointer table in LDS)
constexpr int kLdsMin = 96 * 1024;     // > half a CU's LDS: forces one workgroup per CU
constexpr int kMaxVerifyTokens = 4;    // tokens of one verification step
constexpr int kMaxVerifyCols = 8;      // query columns (tokens x heads of a KV group) of its attention
// Latent (MLA) attention on the matrix cores: all query heads (at most 16) are the 16 columns
// of one bf16 MFMA 16x16x32 tile, positions its rows, the latent dimension its contraction.
constexpr int kMlaHeads = 16;          // query heads folded into one MFMA tile
constexpr int kMlaChunk = 64;          // positions per LDS-resident latent chunk
constexpr int kMlaColBlock = 64;       // latent columns per absorb / W_UV task
constexpr int kIdxBins = 2048;          // histogram bins of one top-T radix pass (11-bit digits)
// GQA: a workgroup's QKV task can put the cached K/V rows of the attention split that
// follows it into LDS (issued by the streaming waves with their row prefetch, ahead of the
// dependency wait). Each streaming wave issues kKvStageDma 1-KB LDS DMA chunks (K and V
// together). K rows go after the staged hidden vector in xs, V rows after the attention merge
// slots in the scratch region; both offsets are in floats.
constexpr int kKvStageDma = 12;
// (cc: the staged vector's padding, kChunkCols columns for bf16 weights, twice that for FP8)
constexpr int kv_stage_k_off(int hidden, int cc = kChunkCols) { return (hidden + cc - 1) / cc * cc; }
constexpr int kv_stage_v_off(int hd) { return kWaves * 4 * (hd + 4) + 64; }

// Task types. Every type runs the same five phases: issue loads of its static operand
// (weights, cached KV) -> wait on its dependency counters -> stage its dynamic input
// (activations) in LDS -> compute while streaming -> store and signal.
enum TaskType : int32_t {
  T_QKV = 1,         // GQA: attention RMSNorm + W_q/W_k/W_v row pairs + RoPE + KV append
  T_ATTN = 2,        // GQA: split-K attention partial over a position range
  T_OPROJ = 3,       // W_o rows + residual (GQA and MLA)
  T_GATEUP = 4,      // FFN RMSNorm + W_gate/W_up rows + SwiGLU
  T_DOWN = 5,        // W_down rows + residual
  T_LMHEAD = 6,      // final RMSNorm + LM-head rows
  T_MLA_A = 7,       // attention RMSNorm + [W_DQ; W_DKV] rows
  T_MLA_B = 8,       // q RMSNorm + W_UQ row pairs + RoPE on the q_rope part
  T_MLA_KVAPP = 9,   // kv RMSNorm + RoPE on k_pe + latent-cache append
  T_MLA_ABSORB = 10, // q_abs[h] = W_UK[h]^T q_nope[h], one column block per task
  T_MLA_ATTN = 11,   // latent attention partial over a position range (MFMA)
  T_MLA_UV = 12,     // merge of one head's splits over a latent column block + W_UV[h] times
                     // that block, added into o[h] with agent-scope atomics
  T_ROUTER = 13,     // FFN RMSNorm + router rows
  T_SHARED_GU = 14,  // FFN RMSNorm + shared-expert gate/up rows + SwiGLU
  T_TOPK = 15,       // sigmoid, top-k selection, normalised weights
  T_EXPERT_GU = 16,  // routed-expert gate/up rows + SwiGLU (expert chosen at run time)
  T_MOE_DOWN = 17,   // shared + routed down rows, weighted sum + residual
  T_OPROJ_G = 18,    // GQA: merge one KV group's attention splits + W_o rows x that group's columns,
                     // added into h with agent-scope atomics
  T_HINIT = 19,      // GQA layer 0: h = x (the accumulator the per-group O-projections add into)
  T_ARGMAX = 20,     // greedy choice: the largest logit over the LM-head tasks' best (value,
                     // index) pairs, written to the step state (length-per-step plans)
  T_IDX_Q = 21,      // sparse indexer: index-query rows W_q c_q (normalised query latent)
  T_IDX_SCORE = 22,  // sparse indexer: scores of a range of positions (bf16 MFMA over the index keys)
  T_IDX_TOPK = 23,   // sparse indexer: the top-T positions (radix select), in increasing order
  T_NUM_TYPES
};

// One task, 64 bytes. u0/u1 = the range of units (rows, row pairs, positions, column
// blocks) it owns; a0..a6 are type-specific.
struct alignas(16) TaskDesc {
  int32_t type, layer, dep_first, dep_count;
  int32_t signal, signal2, id, u0;
  int32_t u1, a0, a1, a2;
  int32_t a3, a4, a5, a6;
};
static_assert(sizeof(TaskDesc) == 64, "task descriptor size");

struct DepEntry {
  int32_t counter;     // counter index
  uint32_t per_step;   // increments the counter receives in one step
};

// Per-layer indices: weights (into the bound weight-pointer table) and activation buffers
// (float offsets from the workspace base; -1 = absent).
enum LayerW : int32_t {
  LW_ATTN_NORM = 0, LW_WQ, LW_WK, LW_WV, LW_WO, LW_FFN_NORM, LW_GATE, LW_UP, LW_DOWN,
  LW_WQA, LW_QNORM, LW_WQB, LW_WKVA, LW_KVNORM, LW_WUK, LW_WUV,
  LW_ROUTER, LW_RBIAS, LW_EGATE, LW_EUP, LW_EDOWN, LW_SGATE, LW_SUP, LW_SDOWN,
  LW_IDXQ, LW_IDXK, LW_IDXW,  // sparse indexer: W_q [H*d][ql], W_k [d][hidden], W_w [H][hidden]
  LW_COUNT
};
enum LayerA : int32_t {
  LA_X_IN = 0,   // layer input (fp32); -1 for layer 0 (the bf16 step input x)
  LA_Q,          // GQA: q post-RoPE [nq*hd]
  LA_KVNEW,      // GQA: new k, v (fp32) [2][nkv][hd]; MLA: new latent row [kl+dr]
  LA_ATTN,       // attention output before W_o [nq*hd] / [nh*dv]
  LA_H,          // residual after attention [hidden]
  LA_ACT,        // SwiGLU activation [ffn] (MoE: routed experts [top_k][eff])
  LA_FFN_OUT,    // FFN branch output [hidden]
  LA_X_OUT,      // layer output [hidden]
  LA_PART,       // attention split partials
  LA_CQ,         // MLA: W_DQ output before q RMSNorm [ql]
  LA_KVA,        // MLA: W_DKV output [kl+dr]
  LA_QNOPE,      // MLA: [nh][dn]
  LA_QROPE,      // MLA: post-RoPE [nh][dr]
  LA_QABS,       // MLA: absorbed query [nh][kl]
  LA_OLAT,       // MLA: attention output in latent space [nh][kl]
  LA_RLOGIT,     // MoE: router logits [n_routed]
  LA_TOPK,       // MoE: int32 [top_k] expert ids, then fp32 [top_k] weights
  LA_SACT,       // MoE: shared-expert activation [ns*eff]
  LA_QOP,        // MLA: scaled [q_abs | q_rope] as bf16 hi/lo pairs in MFMA B-operand order
  LA_PML,        // MLA: split partial (m, l) [nh][S][2]
  LA_IDXK,       // sparse indexer: the new index key (fp32) [d]
  LA_IDXW,       // sparse indexer: head weights [H]
  LA_IDXQ,       // sparse indexer: index queries [H][d]
  LA_IDXS,       // sparse indexer: scores of positions [0, n] (fp32)
  LA_IDXSEL,     // sparse indexer: the selected positions (int32, increasing) [min(T, n + 1)]
  LA_COUNT
};

struct LayerDesc {
  int32_t w[LW_COUNT];
  int32_t act[LA_COUNT];
};

// Per-task execution log written by the engine (one slot per task id, 64 bytes). Times are
// s_memrealtime (100 MHz, one clock for the whole device) low words.
struct TaskLog {
  uint32_t execs;      // incremented once per execution (atomic)
  uint32_t epoch;      // epoch of the last execution
  uint32_t wg;         // workgroup that ran it
  uint32_t xcd;        // hardware XCC id read by that workgroup
  uint32_t t_start;    // task start (static loads issued just after)
  uint32_t t_ready;    // dependencies satisfied
  uint32_t t_end;      // completion (after the counter increment)
  uint32_t t_mid;      // attention: end of the position loop
  uint32_t t_staged;   // input vector staged in LDS
  uint32_t t_streamed; // all rows streamed
  uint32_t t_signal;   // just before the counter increment (read back before the increment is
                       // issued): a consumer that saw the increment passed its wait later
  uint32_t t_aux[5];   // type-specific stamps (vector-ALU attention: lane merge, wave merge)
};

// Control words at the start of the workspace (each on its own 128-byte line).
enum CtlWord : int32_t {
  CTL_EPOCH = 0,       // steps completed since bind/reset
  CTL_DONE = 32,       // workgroups finished in the current step
  CTL_STATUS = 64,     // 0 ok, else (status, task id, counter, observed) at +0..+3
  CTL_ABORT = 96,      // nonzero: a workgroup hit the watchdog; everyone drains out
  CTL_WORDS = 128
};

// Kernel arguments (passed by value).
struct EngineArgs {
  char* ws;                    // workspace base
  const TaskDesc* tasks;
  const int32_t* wg_begin;     // [n_wg + 1] task ranges per workgroup
  const int32_t* stage_first;  // [n_wg][n_stages + 1]: first task of each stage in a workgroup's list
  const DepEntry* deps;
  const uint64_t* wptr;        // bound weight pointers
  const LayerDesc* layers;
  uint32_t* counters;
  uint32_t* ctl;
  TaskLog* log;
  const float* rope_cs;        // rows of (cos[rope_half], sin[rope_half]): one row, at the step's
                               // position, or (length-per-step plans) one per position 0..max_len
  int32_t* state;              // length-per-step plans: {position, token, steps, 0}; else null
  const uint16_t* x;           // step input, bf16 [hidden]
  uint16_t* kv;                // KV cache, bf16
  float* out;                  // logits / last hidden
  float* act;                  // activation region (layer act offsets are relative to it)
  int64_t watchdog_ticks;      // s_memrealtime ticks (100 MHz) allowed per wait
  int32_t arch, n_layers, hidden, vocab;
  int32_t nq, nkv, hd, ffn;
  int32_t ql, kl, dn, dr, dv;
  int32_t n_routed, n_shared, top_k, eff;
  int32_t kv_len;              // the plan's length (a plan with a per-step length: its largest
                               // position); cache slots per (layer, K/V, head) = kv_len + 1
  int32_t n_wg, rope_half, w_final_norm, w_lm_head, x_final;
  int32_t n_stages;            // stages of the plan
  int32_t w_embed;             // weight index of the token embedding (-1: none)
  int32_t wfmt;                // weight format: 0 bf16, 1 FP8 E4M3 rows with fp32 row scales
  int32_t stage_lo, stage_hi;  // this launch runs the tasks of stages [stage_lo, stage_hi)
  int32_t xs_floats;           // LDS floats reserved for the staged input vector
  uint32_t act_bytes;          // size of the activation region
  int32_t gs_floats;           // LDS floats reserved for norm gains
  float eps, attn_scale_log2;  // softmax scale * log2(e)
  int32_t ntok;                // tokens per step (1: decode; 2..4: a verification step)
  int32_t idx_h, idx_d, idx_t; // sparse indexer: heads, key width, positions kept (idx_h = 0: dense)
  int32_t kvrow;               // latent family: cache row width (kl + dr, + idx_d with an indexer)
};

}  // namespace dec
