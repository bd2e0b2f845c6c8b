// api.cpp -- the C ABI declared in include/dec.h: plan lifecycle, binding, the per-token
// launch and status reporting. The planner is host-only; this file is the only place that
// calls the HIP runtime.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dec.h"
#include "planner.h"

extern "C" hipError_t dec_engine_launch(const dec::EngineArgs* args, int n_wg, int lds_bytes, int run, bool cooperative,
                                        hipStream_t stream);
extern "C" hipError_t dec_engine_occupancy(int arch, int wfmt, int ntok, int idx, int lds_bytes, int* blocks_per_cu);
extern "C" hipError_t dec_scratch_current(void** ptr, size_t* bytes);
extern "C" hipError_t dec_stream_read_launch(const void* buf, int64_t bytes, int n_wg, uint32_t* sink, hipStream_t stream);

struct dec_plan {
  dec::PlanData P;
  bool bound = false;
  char* ws = nullptr;
  std::vector<uint64_t> wptr;   // sized at planning, filled by bind (bind allocates nothing)
  dec::EngineArgs args{};
  int64_t watchdog_us = 2000000;
  int scratch_dev = -1;         // bound to this device's static workspace (dec_plan_bind_scratch)
};

namespace {

thread_local std::string g_err;

// The plan bound to each device's static workspace (dec_plan_bind_scratch); a plan that was
// bound there before another one no longer owns the memory and may not run.
constexpr int kMaxScratchDevices = 64;
std::mutex g_owner_mu;
dec_plan* g_scratch_owner[kMaxScratchDevices] = {};

void release_scratch(dec_plan* p) {
  if (p->scratch_dev < 0) return;
  std::lock_guard<std::mutex> lock(g_owner_mu);
  if (g_scratch_owner[p->scratch_dev] == p) g_scratch_owner[p->scratch_dev] = nullptr;
  p->scratch_dev = -1;
}

dec_status fail(dec_status s, const std::string& m) {
  g_err = m;
  return s;
}

dec_status hip_fail(hipError_t e, const char* what) {
  return fail(DEC_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

void fill_args(dec_plan* p) {
  const dec::PlanData& P = p->P;
  const dec_model_shape& s = P.shape;
  dec::EngineArgs& a = p->args;
  char* ws = p->ws;
  a.ws = ws;
  a.tasks = reinterpret_cast<const dec::TaskDesc*>(ws + P.off_tasks);
  a.wg_begin = reinterpret_cast<const int32_t*>(ws + P.off_wgb);
  a.stage_first = reinterpret_cast<const int32_t*>(ws + P.off_stf);
  a.deps = reinterpret_cast<const dec::DepEntry*>(ws + P.off_deps);
  a.wptr = reinterpret_cast<const uint64_t*>(ws + P.off_wptr);
  a.layers = reinterpret_cast<const dec::LayerDesc*>(ws + P.off_layers);
  a.counters = reinterpret_cast<uint32_t*>(ws + P.off_counters);
  a.ctl = reinterpret_cast<uint32_t*>(ws + P.off_ctl);
  a.log = reinterpret_cast<dec::TaskLog*>(ws + P.off_log);
  a.rope_cs = reinterpret_cast<const float*>(ws + P.off_rope);
  a.act = reinterpret_cast<float*>(ws + P.off_act);
  a.x = nullptr;
  a.kv = nullptr;
  a.out = nullptr;
  a.watchdog_ticks = p->watchdog_us * 100;  // s_memrealtime runs at 100 MHz
  a.arch = s.arch;
  a.n_layers = s.n_layers;
  a.hidden = s.hidden;
  a.vocab = s.vocab;
  a.nq = s.n_q_heads;
  a.nkv = s.n_kv_heads;
  a.hd = s.head_dim;
  a.ffn = s.ffn;
  a.ql = s.q_lora_rank;
  a.kl = s.kv_lora_rank;
  a.dn = s.qk_nope;
  a.dr = s.qk_rope;
  a.dv = s.v_head;
  a.n_routed = s.n_routed;
  a.n_shared = s.n_shared;
  a.top_k = s.top_k;
  a.eff = s.expert_ffn;
  a.kv_len = (int32_t)P.kv_len;
  a.n_wg = P.n_wg;
  a.rope_half = P.rope_half;
  a.w_final_norm = P.w_final_norm;
  a.w_lm_head = P.w_lm_head;
  a.x_final = P.x_final;
  a.xs_floats = (int32_t)P.xs_floats;
  a.n_stages = P.n_stages;
  a.stage_lo = 0;
  a.stage_hi = P.n_stages;
  a.state = nullptr;
  a.w_embed = P.w_embed;
  a.wfmt = s.weight_format;
  a.act_bytes = (uint32_t)(P.act_floats * 4);
  a.gs_floats = (int32_t)P.gs_floats;
  a.eps = s.rms_eps;
  a.attn_scale_log2 = P.attn_scale_log2;
  a.ntok = P.ntok;
  a.idx_h = s.index_heads;
  a.idx_d = s.index_heads ? s.index_dim : 0;
  a.idx_t = s.index_topk;
  a.kvrow = s.kv_lora_rank + s.qk_rope + a.idx_d;
}

void copy_name(char* dst, const std::string& s) {
  std::memset(dst, 0, 64);
  std::strncpy(dst, s.c_str(), 63);
}

}  // namespace

namespace {

// A plan bound to a device's static workspace runs only while it still owns it, on that device.
dec_status check_scratch_owner(dec_plan* plan) {
  if (plan->scratch_dev < 0) return DEC_OK;
  {
    std::lock_guard<std::mutex> lock(g_owner_mu);
    if (g_scratch_owner[plan->scratch_dev] != plan)
      return fail(DEC_E_UNBOUND, "another plan has been bound to this device's static workspace since");
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != plan->scratch_dev)
    return fail(DEC_E_DEVICE, "the plan is bound to the static workspace of device " + std::to_string(plan->scratch_dev) +
                                  ", the current device is " + std::to_string(dev));
  return DEC_OK;
}

// One launch of the tasks of stages [lo, hi): cooperative (co-resident grid) when it spans
// several stages, whose tasks wait on each other; a plain launch for one stage.
// The plan's kernel must fit one workgroup per CU with the plan's LDS size; on failure the plan
// is destroyed.
dec_status check_occupancy(dec_plan** out) {
  int per_cu = 0;
  const dec::PlanData& P = (*out)->P;
  hipError_t e = dec_engine_occupancy(P.shape.arch, P.shape.weight_format, P.ntok, P.shape.index_heads > 0, P.lds_bytes, &per_cu);
  if (e != hipSuccess || per_cu < 1) {
    dec_plan_destroy(*out);
    *out = nullptr;
    if (e != hipSuccess) return hip_fail(e, "occupancy query");
    return fail(DEC_E_OCCUPANCY, "the engine kernel cannot be resident with the plan's LDS size");
  }
  return DEC_OK;
}

dec_status launch_stages(dec_plan* plan, const void* x, void* kv, void* out, int32_t lo, int32_t hi, void* stream) {
  if (!plan) return fail(DEC_E_INVAL, "null plan");
  if (!plan->bound) return fail(DEC_E_UNBOUND, "step before dec_plan_bind");
  if (dec_status st = check_scratch_owner(plan)) return st;
  if (!x || !kv || !out) return fail(DEC_E_INVAL, "null x/kv/out");
  if (reinterpret_cast<uintptr_t>(x) % 8 || reinterpret_cast<uintptr_t>(kv) % 16 || reinterpret_cast<uintptr_t>(out) % 4)
    return fail(DEC_E_INVAL, "x must be 8-byte, kv 16-byte and out 4-byte aligned");
  if (plan->P.dynamic) return fail(DEC_E_INVAL, "a plan with a per-step length runs with dec_step_dynamic");
  if ((plan->P.shape.weight_format != DEC_WEIGHTS_BF16 || plan->P.ntok > 1 || plan->P.shape.index_heads > 0) && (lo != 0 || hi != plan->P.n_stages))
    return fail(DEC_E_INVAL, "low-precision, verification and sparse-indexer plans run whole steps only (dec_step)");
  if (lo < 0 || hi > plan->P.n_stages || lo >= hi)
    return fail(DEC_E_INVAL, "stage range [" + std::to_string(lo) + ", " + std::to_string(hi) + ") not inside [0, " +
                                 std::to_string(plan->P.n_stages) + ")");
  plan->args.x = static_cast<const uint16_t*>(x);
  plan->args.kv = static_cast<uint16_t*>(kv);
  plan->args.out = static_cast<float*>(out);
  plan->args.watchdog_ticks = plan->watchdog_us * 100;
  plan->args.stage_lo = lo;
  plan->args.stage_hi = hi;
  plan->args.state = nullptr;
  const bool whole = lo == 0 && hi == plan->P.n_stages;
  hipError_t e = dec_engine_launch(&plan->args, plan->P.n_wg, plan->P.lds_bytes, whole ? 0 : 1, hi - lo > 1,
                                   reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    if (e == hipErrorCooperativeLaunchTooLarge) return fail(DEC_E_OCCUPANCY, "persistent grid cannot be co-resident");
    return hip_fail(e, "engine launch");
  }
  return DEC_OK;
}

}  // namespace

extern "C" {

const char* dec_last_error(void) { return g_err.c_str(); }

dec_status dec_device_query(dec_device_info* out) {
  if (!out) return fail(DEC_E_INVAL, "null output");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipDeviceProp_t pr;
  e = hipGetDeviceProperties(&pr, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  std::memset(out, 0, sizeof(*out));
  int gfx = 0;
  if (std::strncmp(pr.gcnArchName, "gfx", 3) == 0) gfx = (int)std::strtol(pr.gcnArchName + 3, nullptr, 10);
  out->gfx_arch = gfx;
  out->n_cu = pr.multiProcessorCount;
  out->n_xcd = (pr.multiProcessorCount % 32 == 0 && pr.multiProcessorCount >= 32) ? pr.multiProcessorCount / 32 : 1;
  out->lds_bytes_per_cu = (int32_t)pr.maxSharedMemoryPerMultiProcessor;
  out->max_threads_per_cu = pr.maxThreadsPerMultiProcessor;
  return DEC_OK;
}

dec_status dec_plan_create_for(const dec_model_shape* shape, int64_t kv_len, const dec_device_info* dev,
                               dec_plan** out) {
  if (!shape || !dev || !out) return fail(DEC_E_INVAL, "null argument");
  *out = nullptr;
  dec_plan* p = new dec_plan();
  std::string err;
  dec_status st = dec::build_plan(*shape, kv_len, *dev, &p->P, &err);
  if (st != DEC_OK) {
    delete p;
    return fail(st, err);
  }
  p->wptr.assign(p->P.weights.size(), 0);
  *out = p;
  return DEC_OK;
}

dec_status dec_plan_create(const dec_model_shape* shape, int64_t kv_len, dec_plan** out) {
  if (!shape || !out) return fail(DEC_E_INVAL, "null argument");
  dec_device_info dev;
  dec_status st = dec_device_query(&dev);
  if (st != DEC_OK) return st;
  if (dev.gfx_arch != 950) return fail(DEC_E_DEVICE, "current device is gfx" + std::to_string(dev.gfx_arch) + ", need gfx950");
  st = dec_plan_create_for(shape, kv_len, &dev, out);
  if (st != DEC_OK) return st;
  return check_occupancy(out);
}

dec_status dec_plan_destroy(dec_plan* plan) {
  if (plan) release_scratch(plan);
  delete plan;
  return DEC_OK;
}

int64_t dec_plan_n_weights(const dec_plan* plan) { return plan ? (int64_t)plan->P.weights.size() : -1; }

dec_status dec_plan_weight_desc(const dec_plan* plan, int64_t i, dec_tensor_desc* out) {
  if (!plan || !out) return fail(DEC_E_INVAL, "null argument");
  if (i < 0 || i >= (int64_t)plan->P.weights.size()) return fail(DEC_E_INVAL, "weight index out of range");
  const dec::WeightSpec& w = plan->P.weights[i];
  std::memset(out, 0, sizeof(*out));
  copy_name(out->name, w.name);
  out->dtype = w.dtype;
  out->rank = (int32_t)w.dims.size();
  for (size_t k = 0; k < w.dims.size() && k < 4; ++k) out->dims[k] = w.dims[k];
  out->bytes = w.bytes;
  return DEC_OK;
}

dec_status dec_plan_sizes(const dec_plan* plan, dec_sizes* out) {
  if (!plan || !out) return fail(DEC_E_INVAL, "null argument");
  const dec::PlanData& P = plan->P;
  const dec_model_shape& s = P.shape;
  const int64_t nt = P.ntok;  // tokens per step
  out->x_bytes = nt * s.hidden * 2;
  if (s.arch == DEC_ARCH_GQA)
    out->kv_bytes = (int64_t)s.n_layers * 2 * s.n_kv_heads * (P.kv_len + nt) * s.head_dim * 2;
  else
    out->kv_bytes = (int64_t)s.n_layers * (P.kv_len + nt) * (s.kv_lora_rank + s.qk_rope + (s.index_heads ? s.index_dim : 0)) * 2;
  out->out_bytes = nt * (s.vocab > 0 ? s.vocab : s.hidden) * 4;
  out->workspace_bytes = P.ws_bytes;
  out->weight_bytes = P.weight_bytes;
  out->algorithmic_bytes_per_step = P.alg_bytes;
  return DEC_OK;
}

int64_t dec_plan_n_tasks(const dec_plan* plan) { return plan ? (int64_t)plan->P.tasks.size() : -1; }

dec_status dec_plan_tasks(const dec_plan* plan, dec_task_desc* buf, int64_t cap, int64_t* n) {
  if (!plan || !n) return fail(DEC_E_INVAL, "null argument");
  const dec::PlanData& P = plan->P;
  *n = (int64_t)P.tasks.size();
  if (!buf) return DEC_OK;
  if (cap < *n) return fail(DEC_E_CAPACITY, "task buffer too small");
  for (size_t i = 0; i < P.tasks.size(); ++i) {
    const dec::TaskDesc& t = P.tasks[i];
    dec_task_desc& d = buf[i];
    std::memset(&d, 0, sizeof(d));
    d.id = t.id;
    d.type = t.type;
    d.layer = t.layer;
    d.stage = P.info[i].stage;
    d.wg = P.info[i].wg;
    d.xcd = P.info[i].wg % P.dev.n_xcd;
    d.list_pos = P.info[i].list_pos;
    d.unit_begin = t.u0;
    d.unit_end = t.u1;
    d.aux0 = t.a0;
    d.aux1 = t.a1;
    d.n_deps = t.dep_count;
    d.dep_first = t.dep_first;
    d.signal = t.signal;
    d.signal2 = t.signal2;
    d.aux2 = t.a2;
    d.kv_staged = (t.type == dec::T_QKV && t.a5 > 0)    ? dec::split_cached(plan->P.kv_len, t.a4, t.a5)
                  : (t.type == dec::T_ATTN && t.a3 > 0) ? dec::split_cached(plan->P.kv_len, t.a1, t.a2)
                                                        : 0;
    d.aux3 = (t.type == dec::T_ATTN) ? t.a5 : 0;
  }
  return DEC_OK;
}

int64_t dec_plan_n_deps(const dec_plan* plan) { return plan ? (int64_t)plan->P.deps.size() : -1; }

dec_status dec_plan_deps(const dec_plan* plan, int32_t* buf, int64_t cap, int64_t* n) {
  if (!plan || !n) return fail(DEC_E_INVAL, "null argument");
  *n = (int64_t)plan->P.deps.size();
  if (!buf) return DEC_OK;
  if (cap < 2 * *n) return fail(DEC_E_CAPACITY, "dep buffer too small");
  for (size_t i = 0; i < plan->P.deps.size(); ++i) {
    buf[2 * i] = plan->P.deps[i].counter;
    buf[2 * i + 1] = (int32_t)plan->P.deps[i].per_step;
  }
  return DEC_OK;
}

int64_t dec_plan_n_counters(const dec_plan* plan) { return plan ? (int64_t)plan->P.counter_total.size() : -1; }

int64_t dec_plan_n_buffers(const dec_plan* plan) { return plan ? (int64_t)plan->P.buffers.size() : -1; }

dec_status dec_plan_buffer_desc(const dec_plan* plan, int64_t i, dec_buffer_desc* out) {
  if (!plan || !out) return fail(DEC_E_INVAL, "null argument");
  if (i < 0 || i >= (int64_t)plan->P.buffers.size()) return fail(DEC_E_INVAL, "buffer index out of range");
  const dec::BufferSpec& b = plan->P.buffers[i];
  std::memset(out, 0, sizeof(*out));
  copy_name(out->name, b.name);
  out->dtype = b.dtype;
  out->offset = b.offset;
  out->count = b.count;
  return DEC_OK;
}

dec_status dec_plan_grid(const dec_plan* plan, int32_t* n_wg, int32_t* threads, int32_t* lds) {
  if (!plan || !n_wg || !threads || !lds) return fail(DEC_E_INVAL, "null argument");
  *n_wg = plan->P.n_wg;
  *threads = plan->P.threads;
  *lds = plan->P.lds_bytes;
  return DEC_OK;
}

}  // extern "C"

namespace {

// Binding without any host or device allocation: the weight pointers go into the plan's
// pre-sized table, the plan's tables are copied region by region from the plan's own arrays,
// and the control words, counters, task log and activations are cleared.
dec_status bind_impl(dec_plan* plan, const void* const* weights, int64_t n, char* ws, int64_t workspace_bytes, void* stream) {
  dec::PlanData& P = plan->P;
  if (n != (int64_t)P.weights.size())
    return fail(DEC_E_INVAL, "expected " + std::to_string(P.weights.size()) + " weights, got " + std::to_string(n));
  if (workspace_bytes < P.ws_bytes) return fail(DEC_E_CAPACITY, "workspace smaller than dec_sizes.workspace_bytes");
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(DEC_E_INVAL, "workspace not 256-byte aligned");
  if (plan->wptr.size() != P.weights.size()) return fail(DEC_E_PLAN, "weight table not sized at planning");
  for (int64_t i = 0; i < n; ++i) {
    if (!weights[i]) return fail(DEC_E_INVAL, "weight " + P.weights[i].name + " is null");
    if (reinterpret_cast<uintptr_t>(weights[i]) % 16) return fail(DEC_E_INVAL, "weight " + P.weights[i].name + " not 16-byte aligned");
    plan->wptr[i] = reinterpret_cast<uint64_t>(weights[i]);
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto put = [&](int64_t off, const void* src, size_t bytes) {
    return bytes ? hipMemcpyAsync(ws + off, src, bytes, hipMemcpyHostToDevice, s) : hipSuccess;
  };
  auto clear = [&](int64_t off, int64_t end) { return end > off ? hipMemsetAsync(ws + off, 0, (size_t)(end - off), s) : hipSuccess; };
  hipError_t e = clear(P.off_ctl, P.off_tasks);  // control words and counters
  if (e == hipSuccess) e = put(P.off_tasks, P.tasks.data(), P.tasks.size() * sizeof(dec::TaskDesc));
  if (e == hipSuccess) e = put(P.off_wgb, P.wg_begin.data(), P.wg_begin.size() * 4);
  if (e == hipSuccess) e = put(P.off_stf, P.stage_first.data(), P.stage_first.size() * 4);
  if (e == hipSuccess) e = put(P.off_deps, P.deps.data(), P.deps.size() * sizeof(dec::DepEntry));
  if (e == hipSuccess) e = put(P.off_wptr, plan->wptr.data(), plan->wptr.size() * 8);
  if (e == hipSuccess) e = put(P.off_layers, P.layers.data(), P.layers.size() * sizeof(dec::LayerDesc));
  if (e == hipSuccess) e = put(P.off_rope, P.rope_cs.data(), P.rope_cs.size() * 4);
  if (e == hipSuccess) e = clear(P.off_log, P.ws_bytes);  // task log and activations
  if (e != hipSuccess) return hip_fail(e, "upload plan tables");
  e = hipStreamSynchronize(s);  // the plan's host arrays may change after a later call
  if (e != hipSuccess) return hip_fail(e, "bind synchronise");
  plan->ws = ws;
  fill_args(plan);
  plan->bound = true;
  return DEC_OK;
}

}  // namespace

extern "C" {

dec_status dec_plan_bind(dec_plan* plan, const void* const* weights, int64_t n, void* workspace,
                         int64_t workspace_bytes, void* stream) {
  if (!plan || !weights || !workspace) return fail(DEC_E_INVAL, "null argument");
  release_scratch(plan);
  plan->bound = false;
  return bind_impl(plan, weights, n, static_cast<char*>(workspace), workspace_bytes, stream);
}

dec_status dec_plan_bind_scratch(dec_plan* plan, const void* const* weights, int64_t n, void* stream) {
  if (!plan || !weights) return fail(DEC_E_INVAL, "null argument");
  void* ws = nullptr;
  size_t bytes = 0;
  hipError_t e = dec_scratch_current(&ws, &bytes);
  if (e != hipSuccess) return hip_fail(e, "static workspace lookup");
  if (plan->P.ws_bytes > (int64_t)bytes)
    return fail(DEC_E_CAPACITY, "the plan needs " + std::to_string(plan->P.ws_bytes) + " bytes of workspace; the static workspace holds " +
                                    std::to_string(bytes));
  int dev = -1;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxScratchDevices) return fail(DEC_E_DEVICE, "device index out of range");
  release_scratch(plan);
  plan->bound = false;
  {
    std::lock_guard<std::mutex> lock(g_owner_mu);
    g_scratch_owner[dev] = nullptr;  // the memory is being overwritten: no plan owns it meanwhile
  }
  dec_status st = bind_impl(plan, weights, n, static_cast<char*>(ws), (int64_t)bytes, stream);
  if (st != DEC_OK) return st;
  std::lock_guard<std::mutex> lock(g_owner_mu);
  g_scratch_owner[dev] = plan;
  plan->scratch_dev = dev;
  return DEC_OK;
}

dec_status dec_step(dec_plan* plan, const void* x, void* kv, void* out, void* stream) {
  if (!plan) return fail(DEC_E_INVAL, "null plan");
  return launch_stages(plan, x, kv, out, 0, plan->P.n_stages, stream);
}

int64_t dec_plan_n_stages(const dec_plan* plan) { return plan ? (int64_t)plan->P.n_stages : -1; }

dec_status dec_plan_create_dynamic(const dec_model_shape* shape, int64_t max_len, const dec_device_info* dev,
                                   dec_plan** out) {
  if (!shape || !out) return fail(DEC_E_INVAL, "null argument");
  *out = nullptr;
  dec_device_info cur;
  if (!dev) {
    dec_status st = dec_device_query(&cur);
    if (st != DEC_OK) return st;
    if (cur.gfx_arch != 950) return fail(DEC_E_DEVICE, "current device is gfx" + std::to_string(cur.gfx_arch) + ", need gfx950");
    dev = &cur;
  }
  dec_plan* p = new dec_plan();
  std::string err;
  dec_status st = dec::build_plan(*shape, max_len, *dev, &p->P, &err, true);
  if (st != DEC_OK) {
    delete p;
    return fail(st, err);
  }
  p->wptr.assign(p->P.weights.size(), 0);
  *out = p;
  return DEC_OK;
}

dec_status dec_plan_create_verify(const dec_model_shape* shape, int64_t kv_len, int32_t n_tokens, const dec_device_info* dev,
                                  dec_plan** out) {
  if (!shape || !out) return fail(DEC_E_INVAL, "null argument");
  *out = nullptr;
  dec_device_info cur;
  const bool query = !dev;
  if (query) {
    dec_status st = dec_device_query(&cur);
    if (st != DEC_OK) return st;
    if (cur.gfx_arch != 950) return fail(DEC_E_DEVICE, "current device is gfx" + std::to_string(cur.gfx_arch) + ", need gfx950");
    dev = &cur;
  }
  dec_plan* p = new dec_plan();
  std::string err;
  dec_status st = dec::build_plan(*shape, kv_len, *dev, &p->P, &err, false, n_tokens);
  if (st != DEC_OK) {
    delete p;
    return fail(st, err);
  }
  p->wptr.assign(p->P.weights.size(), 0);
  *out = p;
  return query ? check_occupancy(out) : DEC_OK;
}

dec_status dec_step_dynamic(dec_plan* plan, const void* x, void* kv, void* out, int32_t* state, void* stream) {
  if (!plan) return fail(DEC_E_INVAL, "null plan");
  if (!plan->bound) return fail(DEC_E_UNBOUND, "step before dec_plan_bind");
  if (!plan->P.dynamic) return fail(DEC_E_INVAL, "dec_step_dynamic needs a plan from dec_plan_create_dynamic");
  if (dec_status st = check_scratch_owner(plan)) return st;
  if (!kv || !out || !state) return fail(DEC_E_INVAL, "null kv/out/state");
  if (!x && plan->P.w_embed < 0) return fail(DEC_E_INVAL, "no input vector and no token embedding (vocab == 0)");
  if (reinterpret_cast<uintptr_t>(x) % 8 || reinterpret_cast<uintptr_t>(kv) % 16 || reinterpret_cast<uintptr_t>(out) % 4 ||
      reinterpret_cast<uintptr_t>(state) % 16)
    return fail(DEC_E_INVAL, "x must be 8-byte, kv and state 16-byte and out 4-byte aligned");
  plan->args.x = static_cast<const uint16_t*>(x);
  plan->args.kv = static_cast<uint16_t*>(kv);
  plan->args.out = static_cast<float*>(out);
  plan->args.watchdog_ticks = plan->watchdog_us * 100;
  plan->args.stage_lo = 0;
  plan->args.stage_hi = plan->P.n_stages;
  plan->args.state = state;
  hipError_t e = dec_engine_launch(&plan->args, plan->P.n_wg, plan->P.lds_bytes, 2, true, reinterpret_cast<hipStream_t>(stream));
  plan->args.state = nullptr;
  if (e != hipSuccess) {
    if (e == hipErrorCooperativeLaunchTooLarge) return fail(DEC_E_OCCUPANCY, "persistent grid cannot be co-resident");
    return hip_fail(e, "engine launch");
  }
  return DEC_OK;
}

dec_status dec_step_stages(dec_plan* plan, const void* x, void* kv, void* out, int32_t stage_lo, int32_t stage_hi,
                           void* stream) {
  return launch_stages(plan, x, kv, out, stage_lo, stage_hi, stream);
}

dec_status dec_stream_read(const void* buf, int64_t bytes, void* sink, int64_t sink_bytes, void* stream) {
  if (!buf || !sink) return fail(DEC_E_INVAL, "null argument");
  if (bytes < 16 || bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16)
    return fail(DEC_E_INVAL, "the buffer must be 16-byte aligned and a positive multiple of 16 bytes");
  dec_device_info dev;
  dec_status st = dec_device_query(&dev);
  if (st != DEC_OK) return st;
  if (sink_bytes < (int64_t)dev.n_cu * dec::kThreads * 4 || reinterpret_cast<uintptr_t>(sink) % 4)
    return fail(DEC_E_CAPACITY, "sink must hold n_cu * 512 4-byte words");
  hipError_t e = dec_stream_read_launch(buf, bytes, dev.n_cu, static_cast<uint32_t*>(sink), reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stream-read launch");
  return DEC_OK;
}

dec_status dec_plan_status(dec_plan* plan, void* stream) {
  if (!plan) return fail(DEC_E_INVAL, "null plan");
  if (!plan->bound) return fail(DEC_E_UNBOUND, "plan not bound");
  if (dec_status st = check_scratch_owner(plan)) return st;
  hipError_t e = hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "status synchronise");
  uint32_t st[4] = {0, 0, 0, 0};
  e = hipMemcpy(st, plan->ws + plan->P.off_ctl + dec::CTL_STATUS * 4, sizeof(st), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "status read");
  if (st[0] == 7u)
    return fail(DEC_E_TIMEOUT, "watchdog: task " + std::to_string(st[1]) + " timed out waiting on counter " +
                                   std::to_string(st[2]) + " (value " + std::to_string(st[3]) + ")");
  if (st[0] == 8u)
    return fail(DEC_E_CAPACITY, "step state out of range: position " + std::to_string((int32_t)st[1]) + " (largest " +
                                    std::to_string(plan->P.kv_len) + "), token " + std::to_string((int32_t)st[2]));
  if (st[0] != 0u) return fail(DEC_E_PLAN, "unknown device status " + std::to_string(st[0]));
  return DEC_OK;
}

dec_status dec_plan_reset(dec_plan* plan, void* stream) {
  if (!plan) return fail(DEC_E_INVAL, "null plan");
  if (!plan->bound) return fail(DEC_E_UNBOUND, "plan not bound");
  if (dec_status st = check_scratch_owner(plan)) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dec::PlanData& P = plan->P;
  hipError_t e = hipMemsetAsync(plan->ws + P.off_ctl, 0, (size_t)(P.off_tasks - P.off_ctl), s);  // ctl + counters
  if (e == hipSuccess) e = hipMemsetAsync(plan->ws + P.off_log, 0, (size_t)(P.off_act - P.off_log), s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reset");
  return DEC_OK;
}

dec_status dec_plan_set_watchdog(dec_plan* plan, int64_t microseconds) {
  if (!plan) return fail(DEC_E_INVAL, "null plan");
  if (microseconds < 1) return fail(DEC_E_INVAL, "watchdog must be >= 1 us");
  plan->watchdog_us = microseconds;
  return DEC_OK;
}

}  // extern "C"
