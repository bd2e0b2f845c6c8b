// planner.h -- ahead-of-time planner of one batch-1 decode step (host only, no HIP).
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/dec.h"
#include "plan_types.h"

namespace dec {

struct WeightSpec {
  std::string name;
  int32_t dtype;
  std::vector<int64_t> dims;
  int64_t bytes;
};

struct BufferSpec {
  std::string name;
  int32_t dtype;
  int64_t offset;   // bytes from the workspace base
  int64_t count;    // elements
};

struct TaskInfo {   // planner-side description of one task (introspection / validation)
  int32_t stage;
  int32_t wg;
  int32_t list_pos;
};

struct PlanData {
  dec_model_shape shape{};
  int64_t kv_len = 0;
  dec_device_info dev{};
  int32_t n_wg = 0, threads = kThreads, lds_bytes = 0;

  std::vector<WeightSpec> weights;
  std::vector<TaskDesc> tasks;        // grouped by workgroup, in list order
  std::vector<TaskInfo> info;         // parallel to tasks
  std::vector<int32_t> wg_begin;      // n_wg + 1
  int32_t n_stages = 0;
  std::vector<int32_t> stage_first;   // [n_wg][n_stages + 1]: first task index of each stage
  std::vector<DepEntry> deps;
  std::vector<uint32_t> counter_total;
  std::vector<LayerDesc> layers;
  std::vector<float> rope_cs;         // cos then sin, rope_half each
  std::vector<BufferSpec> buffers;
  int32_t n_log = 0;                  // task ids + ticket-merge ids
  int64_t xs_floats = 0;              // LDS floats for the largest staged input vector
  int64_t gs_floats = 0;              // LDS floats for norm gains (bf16 pairs)
  int32_t rope_half = 0;
  int32_t rope_rows = 1;              // rows of the RoPE table (positions 0..max_len when dynamic)
  bool dynamic = false;               // the step's position is read from device memory
  int32_t ntok = 1;                   // tokens per step (> 1: a verification step of that many)
  int32_t w_final_norm = -1, w_lm_head = -1, x_final = -1, w_embed = -1;
  float attn_scale_log2 = 0.f;

  // workspace layout (bytes)
  int64_t off_ctl = 0, off_counters = 0, off_tasks = 0, off_wgb = 0, off_stf = 0, off_deps = 0,
          off_wptr = 0, off_layers = 0, off_rope = 0, off_log = 0, off_act = 0, ws_bytes = 0;
  int64_t act_floats = 0;

  int64_t weight_bytes = 0, alg_bytes = 0;
};

// Validate the shape and build the plan. Returns DEC_OK or an error (message in *err).
// dynamic: kv_len is the largest position a step may have (max_len); each step reads its
// position (and, without an input vector, its token) from device memory.
// ntok > 1: a verification step of ntok tokens at positions kv_len .. kv_len + ntok - 1 (GQA,
// bf16 weights, fixed length only).
dec_status build_plan(const dec_model_shape& shape, int64_t kv_len, const dec_device_info& dev,
                      PlanData* out, std::string* err, bool dynamic = false, int ntok = 1);

// Positions [p0, p1) of attention split sp of S over the positions 0..n (n + 1 of them).
inline int split_begin(int64_t n, int sp, int S) { return (int)((n + 1) * sp / S); }
// Cached rows of that split (positions below n) an attention task can have staged in LDS.
inline int split_cached(int64_t n, int sp, int S) {
  const int p0 = split_begin(n, sp, S), p1 = split_begin(n, sp + 1, S);
  return (int)std::min<int64_t>(p1, n) - p0;
}

// Structural checks of a built plan: list order vs stage order, producers before
// consumers, counter totals, unit coverage. Returns an empty string when all hold.
std::string validate_plan(const PlanData& p);

}  // namespace dec
