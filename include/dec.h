/* dec.h -- C ABI of a batch-1 LLM decode step run as ONE persistent, tile-scheduled
 * kernel on an AMD Instinct MI355X (gfx950).
 *
 * What the calls implement. The pages behind this library ("Static Compilation for LLM
 * Inference: from ASIC Graph Compile to Persistent Engine Kernel", sections 1, 5.6 and 6;
 * the tile-ai/TileRT audit page, blog-vs-code table; the TileRT talk transcript, section on
 * breaking kernel boundaries) describe a decode step that is statically compiled ahead of
 * time: every shape is known, the whole layer stack is unrolled into tile-level tasks,
 * and one long-lived kernel executes them, starting each task as soon as its producers
 * are done instead of launching one kernel per operator. The TileRT audit page also fixes
 * the interface habits followed here: prepare once and then run per token, weights bound
 * before the first run, batch fixed at 1 (max_batch_size = 1), an externally produced KV
 * cache passed in as a raw buffer (inject_cache), and any shape change meaning a rebuild.
 *
 * Call sequence:
 *   dec_plan_create(shape, kv_len, &plan)     -- host-only planning (no device memory)
 *   dec_plan_sizes / dec_plan_weight_desc     -- what the caller must allocate
 *   dec_plan_bind(plan, weights, n, ws, bytes, stream)  -- once
 *   dec_step(plan, x, kv, out, stream)        -- once per token: exactly one kernel launch
 *   dec_plan_status(plan, stream)             -- optional: sync and read the device status
 *   dec_plan_destroy(plan)
 *
 * Ownership: the caller allocates and frees every device buffer (weights, workspace, x,
 * kv, out). The plan keeps the raw pointers given to bind until destroy or the next bind.
 * The library never allocates or frees device memory at run time. The only allocation the
 * library makes is the opaque host-side plan object; its code object also holds one static
 * 64 MiB workspace per device, for dec_plan_bind_scratch.
 *
 * Errors: every call validates synchronously and returns a negative dec_status on error
 * without aborting; dec_last_error() then holds a message (thread-local). dec_step is
 * asynchronous: a device-side failure (a dependency wait that exceeds the watchdog) is
 * recorded in a sticky status word in the workspace; dec_plan_status reports it and
 * dec_plan_reset clears it.
 *
 * Concurrency: the steps of one plan must be serialised (one stream, or explicit
 * ordering): its dependency counters and epoch live in its workspace. Different plans
 * with different workspaces may run concurrently.
 *
 * The `stream` arguments are hipStream_t values passed as void* (NULL = default stream).
 */
#ifndef DEC_H_
#define DEC_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DEC_ABI_VERSION 3

typedef struct dec_plan dec_plan;   /* opaque, library-owned host object */

typedef enum {
  DEC_OK = 0,
  DEC_E_INVAL = -1,      /* null pointer, bad index, wrong abi_version, wrong weight count */
  DEC_E_SHAPE = -2,      /* unsupported or inconsistent model shape */
  DEC_E_CAPACITY = -3,   /* a size exceeds what the plan supports (kv_len, workspace) */
  DEC_E_DEVICE = -4,     /* current device is not gfx950 / no device */
  DEC_E_OCCUPANCY = -5,  /* the persistent grid cannot be co-resident on this device */
  DEC_E_HIP = -6,        /* a HIP runtime call failed (message holds hipGetErrorString) */
  DEC_E_TIMEOUT = -7,    /* device watchdog: a dependency wait exceeded its budget */
  DEC_E_UNBOUND = -8,    /* dec_step before dec_plan_bind */
  DEC_E_PLAN = -9        /* planner self-validation failed (internal error) */
} dec_status;

typedef enum {
  DEC_WEIGHTS_BF16 = 0,      /* every matrix bf16 */
  DEC_WEIGHTS_FP8_E4M3 = 1,  /* every family: each linear matrix as OCP FP8 E4M3 bytes
                                [rows][cols] (stacked experts [E][rows][cols]), followed in the
                                weight list by "<name>.scale", fp32 [rows] ([E][rows]): row r of
                                the matrix is scale[r] * e4m3(bytes[r][:]). GQA: wq, wk, wv, wo,
                                w_gate, w_up, w_down, lm_head; latent families: every linear
                                matrix but the per-head absorption matrices w_uk, w_uv and the
                                router. cols must be a multiple of 16. Norm gains (and "embed")
                                stay bf16. The pages name the lever (fewer bytes moved per
                                token), not a format; the audit page names an FP8 dequantisation
                                fused into the attention's input projection. */
  DEC_WEIGHTS_MXFP4 = 2      /* MoE only: every expert matrix (experts.w_gate / w_up / w_down and
                                shared.w_gate / w_up / w_down) in the OCP Microscaling FP4 format:
                                E2M1 elements packed two per byte, uint8 [..][cols / 2], element 2i
                                in the low nibble of byte i, followed in the weight list by
                                "<name>.scale", E8M0 bytes uint8 [..][cols / 32]: element k of a row
                                is e2m1(k) * 2^(scale[k / 32] - 127). hidden and expert_ffn must be
                                multiples of 32. Every other weight stays bf16. The TileRT talk's
                                practice section reports FP4 experts with the other modules kept
                                at their precision; it names no format, this is the one gfx950
                                converts in hardware. Whole-step launches only. */
} dec_weight_format;

typedef enum {
  DEC_ARCH_GQA = 0,      /* Llama-style pre-norm decoder: GQA attention + SwiGLU FFN */
  DEC_ARCH_MLA = 1,      /* latent-KV (MLA) attention + dense SwiGLU FFN */
  DEC_ARCH_MOE = 2       /* latent-KV (MLA) attention + routed/shared expert FFN */
} dec_arch;

/* Model shape (plain data, no pointers). Fields unused by an arch must be 0.
 *   GQA: n_q_heads, n_kv_heads, head_dim, ffn.
 *   MLA: n_q_heads, q_lora_rank, kv_lora_rank, qk_nope, qk_rope, v_head, ffn.
 *   MOE: the MLA fields (ffn = 0) plus n_routed, n_shared, top_k, expert_ffn.
 * vocab > 0 adds a final RMSNorm + LM head (out = fp32 logits); vocab == 0 means
 * out = the last hidden state (fp32, no final norm). Batch is always 1. */
typedef struct dec_model_shape {
  int32_t abi_version;   /* must be DEC_ABI_VERSION */
  int32_t arch;          /* dec_arch */
  int32_t n_layers, hidden, vocab;
  int32_t n_q_heads, n_kv_heads, head_dim, ffn;
  int32_t q_lora_rank, kv_lora_rank, qk_nope, qk_rope, v_head;
  int32_t n_routed, n_shared, top_k, expert_ffn;
  float rms_eps;
  int32_t weight_format; /* dec_weight_format (0: bf16) */
  double rope_theta;
  /* Sparse indexer (latent families, bf16 weights; index_heads = 0: dense attention): per
   * layer an index key k = W_k x^ (appended to the cache after the position's latent row),
   * index_heads head weights w = W_w x^ and queries q_j = (W_q c_q)_j; every position s gets
   * the score I_s = sum_j w_j max(0, q_j . k_s), and attention reads only the index_topk
   * positions with the largest scores (ties to the lower position; all positions when there
   * are at most index_topk). index_heads <= 64, index_dim a multiple of 32 up to 128. (The
   * TileRT audit page's sparse_index: 64 index heads selecting the top-2048 KV positions.) */
  int32_t index_heads, index_dim, index_topk;
  int32_t reserved1;
} dec_model_shape;

/* Description of the device the plan is built for. dec_plan_create fills it from the
 * current HIP device; dec_plan_create_for takes it explicitly (host-only planning). */
typedef struct dec_device_info {
  int32_t gfx_arch;            /* 950 for gfx950 */
  int32_t n_cu;                /* compute units (256 on MI355X) */
  int32_t n_xcd;               /* chiplets (8 on MI355X); workgroup w runs on XCD w % n_xcd */
  int32_t lds_bytes_per_cu;    /* 163840 on gfx950 */
  int32_t max_threads_per_cu;  /* waves per CU * 64 */
  int32_t reserved0;
} dec_device_info;

typedef enum {
  DEC_DTYPE_BF16 = 0, DEC_DTYPE_FP32 = 1, DEC_DTYPE_I32 = 2, DEC_DTYPE_FP8 = 3,
  DEC_DTYPE_FP4X2 = 4,  /* two E2M1 elements per byte (dims count bytes) */
  DEC_DTYPE_E8M0 = 5    /* one power-of-two block scale per byte */
} dec_dtype;

typedef struct dec_tensor_desc {
  char name[64];           /* e.g. "layers.3.wq" */
  int32_t dtype;           /* dec_dtype */
  int32_t rank;            /* 1..4 */
  int64_t dims[4];         /* row-major; unused dims = 0 */
  int64_t bytes;
} dec_tensor_desc;

typedef struct dec_sizes {
  int64_t x_bytes;         /* bf16 [hidden] */
  int64_t kv_bytes;        /* see dec_step */
  int64_t out_bytes;       /* fp32 [vocab] or fp32 [hidden] */
  int64_t workspace_bytes; /* library-owned device scratch, caller-allocated, 256-B aligned */
  int64_t weight_bytes;    /* sum over the weight list */
  int64_t algorithmic_bytes_per_step; /* weights (active experts only) + KV positions read */
} dec_sizes;

/* One statically planned task, as the planner emitted it (for coverage checks). */
typedef struct dec_task_desc {
  int32_t id, type, layer, stage;
  int32_t wg, xcd, list_pos;
  int32_t unit_begin, unit_end;   /* rows / units / positions the task owns (type-specific) */
  int32_t aux0, aux1;             /* type-specific: group, split, head, ...; the top-T task: aux0 =
                                     scores per LDS chunk of its selection */
  int32_t n_deps, dep_first;      /* counters waited on (see dec_plan_deps) */
  int32_t signal;                 /* counter incremented on completion (-1: none) */
  int32_t signal2;                /* second counter (-1: none) */
  int32_t aux2;                   /* type-specific: split count; for the routed-expert tasks the
                                     number of leading dependencies (the router) that decide
                                     their rows */
  int32_t kv_staged;              /* GQA QKV and attention tasks: cached K/V rows of the
                                     attention split that the workgroup's QKV task copies into
                                     LDS for the attention task right after it (0: none) */
  int32_t aux3;                   /* attention tasks of a verification step: the block of 8
                                     query columns (token * heads per group + head) they take */
} dec_task_desc;

/* A named fp32 (or i32) buffer inside the workspace holding an intermediate of the last
 * step (per-layer activations, router choice, task log). Offsets are in bytes. */
typedef struct dec_buffer_desc {
  char name[64];
  int32_t dtype;
  int32_t reserved0;
  int64_t offset;
  int64_t count;           /* elements */
} dec_buffer_desc;

/* ---- planning (host only; no device memory is touched) ---- */

/* Plan for the current HIP device: unroll the whole layer stack for this shape and cache
 * length into tile tasks, dependency counters and per-workgroup lists, ahead of time ("Static
 * Compilation for LLM Inference", section 1: the model compiled once into one engine; section
 * 5.6: a static schedule rather than a dynamic dispatcher). Errors: SHAPE, CAPACITY (kv_len < 0
 * or too large), DEVICE (not gfx950), OCCUPANCY, INVAL (null). */
dec_status dec_plan_create(const dec_model_shape* shape, int64_t kv_len, struct dec_plan** out);
/* Plan for an explicitly described device (CPU-only testing and cross-planning). */
dec_status dec_plan_create_for(const dec_model_shape* shape, int64_t kv_len,
                               const dec_device_info* dev, struct dec_plan** out);
/* Free the host-side plan (the caller's device buffers are not touched). NULL is a no-op. */
dec_status dec_plan_destroy(struct dec_plan* plan);

/* The weight list in bind order (the layout contract). */
int64_t dec_plan_n_weights(const struct dec_plan* plan);
dec_status dec_plan_weight_desc(const struct dec_plan* plan, int64_t i, dec_tensor_desc* out);
dec_status dec_plan_sizes(const struct dec_plan* plan, dec_sizes* out);

/* Introspection of the static schedule. */
int64_t dec_plan_n_tasks(const struct dec_plan* plan);
dec_status dec_plan_tasks(const struct dec_plan* plan, dec_task_desc* buf, int64_t cap, int64_t* n);
/* counters: buf[2*i] = counter index, buf[2*i+1] = increments per step, for dep entry i */
int64_t dec_plan_n_deps(const struct dec_plan* plan);
dec_status dec_plan_deps(const struct dec_plan* plan, int32_t* buf, int64_t cap, int64_t* n);
int64_t dec_plan_n_counters(const struct dec_plan* plan);
int64_t dec_plan_n_buffers(const struct dec_plan* plan);
dec_status dec_plan_buffer_desc(const struct dec_plan* plan, int64_t i, dec_buffer_desc* out);
/* Grid the step launches: n_wg workgroups of `threads` threads, `lds` bytes of LDS each. */
dec_status dec_plan_grid(const struct dec_plan* plan, int32_t* n_wg, int32_t* threads, int32_t* lds);

/* ---- device side ---- */

/* Bind caller-owned weight buffers (n == dec_plan_n_weights, in weight_desc order, each
 * 16-byte aligned) and a workspace of >= workspace_bytes (256-byte aligned). Uploads the
 * task table and zeroes counters/status on `stream` (asynchronously): the "prepare once"
 * half of the prepare-then-run interface on the TileRT audit page (weights bound before the
 * first run). Errors: INVAL, HIP. */
dec_status dec_plan_bind(struct dec_plan* plan, const void* const* weights, int64_t n,
                         void* workspace, int64_t workspace_bytes, void* stream);

/* Allocation-free binding, for callers that cannot allocate device memory (code under stream
 * capture, tight serving loops, harnesses that forbid hipMalloc): as dec_plan_bind, but the
 * workspace is the library's own static device array on the current device (64 MiB per GPU,
 * held from the first such call on a device until the process ends). Nothing is allocated on
 * the host or the device; the plan's tables are copied in and the control words, counters,
 * task log and activations are cleared, and the call synchronises `stream`.
 * The array is shared by every plan bound to it on that device: binding another plan there
 * takes it over, after which the earlier plan's calls fail with DEC_E_UNBOUND until it is
 * bound again. Steps of plans bound to it must not overlap on one GPU (they would race on the
 * same memory), and they must run with that device current (else DEC_E_DEVICE). The
 * workspace-size contract is the same as for dec_plan_bind (dec_sizes.workspace_bytes).
 * Errors: INVAL (null, weight count or alignment), CAPACITY (the plan needs more than the
 * static array holds), DEVICE, HIP. */
dec_status dec_plan_bind_scratch(struct dec_plan* plan, const void* const* weights, int64_t n, void* stream);

/* Run one decode step: ONE kernel launch on `stream` (the per-token run of the audit page's
 * prepare-then-run interface; the single engine launch of "Static Compilation for LLM
 * Inference", sections 1 and 6, in place of one launch per operator).
 *   x   : bf16 [hidden], the new token's input hidden state (read only).
 *   kv  : bf16 cache. GQA: [n_layers][2][n_kv_heads][kv_len+1][head_dim] (K then V);
 *         MLA/MOE: [n_layers][kv_len+1][kv_lora_rank + qk_rope] (c || k_pe).
 *         Positions [0, kv_len) are read; slot kv_len of every layer is written with the
 *         new token's post-RoPE k / v (resp. normalised c || post-RoPE k_pe).
 *   out : fp32 [vocab] logits, or fp32 [hidden] last hidden state when vocab == 0.
 * Errors: UNBOUND, INVAL (null or misaligned), HIP (launch failure). */
dec_status dec_step(struct dec_plan* plan, const void* x, void* kv, void* out, void* stream);

/* The same step split into several launches, for measuring what the single persistent launch
 * saves (the launch-per-operator execution that the Static Compilation page and the TileRT
 * talk, section on breaking kernel boundaries, set against one engine kernel). The plan's tasks
 * fall into dec_plan_n_stages() stages in dependency order: every task waits only on tasks of
 * earlier stages. dec_step_stages runs the tasks of stages [stage_lo, stage_hi) in ONE launch
 * on `stream`: a plain launch for a single stage (nothing in it waits on anything in the same
 * launch), a cooperative one for several. One step is either one dec_step, or calls covering
 * [0, n_stages) in increasing, consecutive ranges on one stream with nothing of another step in
 * between; the step's last call (stage_hi == n_stages) completes it. The x, kv and out arguments
 * must be the same for all calls of a step. The launches read and write the same buffers as
 * dec_step and give the same results; they contain no host synchronisation or memory set, so
 * a stream capture of them (a HIP graph) replays a whole step.
 * Errors: UNBOUND, INVAL (null, misaligned, or a range outside [0, n_stages) or empty), HIP. */
int64_t dec_plan_n_stages(const struct dec_plan* plan);
dec_status dec_step_stages(struct dec_plan* plan, const void* x, void* kv, void* out, int32_t stage_lo,
                           int32_t stage_hi, void* stream);

/* ---- a plan whose length is read per step ----
 * The pages fix every shape ahead of time, while the cache grows by one position per token
 * (Static Compilation page, sections 5.5 and 7.1: static shapes against a growing KV cache;
 * TileRT audit page: any shape change means a rebuild). This plan is built once for a largest
 * position max_len; each step reads its position from device memory, so one plan and one
 * bound workspace serve a whole generation.
 *
 * dec_plan_create_dynamic: as dec_plan_create_for (dev == NULL: the current device, which must
 * be gfx950), with kv_len replaced by max_len. The attention split count is planned for
 * max_len; at a shorter position the same splits are shorter (a split may be empty and
 * contributes nothing). dec_plan_sizes reports kv_bytes for max_len + 1 slots and the
 * algorithmic bytes of a step at position max_len. When vocab > 0 the weight list ends with
 * "embed" bf16 [vocab][hidden], the token embedding (bf16 also with FP8 weights: a row is
 * read, not multiplied). Every family (GQA, MLA, MLA + MoE) and both weight formats have these
 * plans. Errors: as dec_plan_create_for.
 *
 * dec_step_dynamic: one step, ONE kernel launch on `stream`.
 *   state : device int32[4], 16-byte aligned, caller-owned: {position p, token, steps, 0}.
 *           The step reads p (0 <= p <= max_len): positions [0, p) of the cache are read and
 *           slot p is written, with RoPE at position p. When x is NULL the input vector is
 *           the embedding row of `token` (0 <= token < vocab). At the end of the step the
 *           kernel writes p + 1 to state[0], adds 1 to state[2] and, when vocab > 0, writes
 *           the greedy choice (the index of the largest logit, the lowest among equals) to
 *           state[1]. Consecutive calls therefore run a greedy generation loop on the device
 *           with no host work between tokens.
 *   x     : bf16 [hidden] or NULL (needs vocab > 0).
 *   kv    : bf16 [n_layers][2][n_kv_heads][max_len + 1][head_dim] (GQA), or the latent
 *           cache bf16 [n_layers][max_len + 1][kv_lora_rank + qk_rope] (MLA, MoE).
 *   out   : as dec_step.
 * An out-of-range position or token makes the whole step do nothing (state unchanged); the
 * sticky status then reports DEC_E_CAPACITY with the values read (dec_plan_status).
 * dec_step and dec_step_stages reject these plans, and dec_step_dynamic other plans (INVAL).
 * Errors: UNBOUND, INVAL (null kv/out/state, x NULL without an embedding, misalignment), HIP. */
dec_status dec_plan_create_dynamic(const dec_model_shape* shape, int64_t max_len, const dec_device_info* dev,
                                   struct dec_plan** out);
dec_status dec_step_dynamic(struct dec_plan* plan, const void* x, void* kv, void* out, int32_t* state, void* stream);

/* ---- a verification step of several tokens ----
 * More tokens per step for the same weight bytes: the step that checks a block of draft
 * tokens (multi-token prediction or another speculative scheme) runs the model on n_tokens
 * consecutive tokens at once (TileRT talk write-ups, sections on production results with MTP-3
 * and on raising the tokens produced per byte read). Every weight row is read once for all
 * tokens; attention is causal inside the block.
 *
 * dec_plan_create_verify: a plan for n_tokens (1 .. 4) tokens at positions kv_len ..
 * kv_len + n_tokens - 1. GQA family with bf16 weights only; dev == NULL plans for the current
 * device (which must be gfx950) and checks that the kernel fits it, as dec_plan_create; a
 * given dev plans without touching a GPU, as dec_plan_create_for. The plan runs with dec_step
 * (whole steps only: dec_step_stages accepts only the full range [0, n_stages)):
 *   x   : bf16 [n_tokens][hidden], token i's input vector in row i.
 *   kv  : bf16 [n_layers][2][n_kv_heads][kv_len + n_tokens][head_dim]. Positions [0, kv_len)
 *         are read; slots kv_len + i are written with token i's post-RoPE k / v (RoPE at
 *         position kv_len + i). Token i attends to positions [0, kv_len + i].
 *   out : fp32 [n_tokens][vocab] (vocab == 0: [n_tokens][hidden]), token i's row i.
 * dec_plan_sizes reports x, kv and out bytes for these shapes, and as algorithmic bytes every
 * weight once plus kv_len + n_tokens cache positions per layer. Token i's results equal those
 * of i + 1 single-token steps run in order, up to rounding order.
 * Errors: as dec_plan_create_for; INVAL for n_tokens outside 1..4, SHAPE for another family,
 * FP8 weights. */
dec_status dec_plan_create_verify(const dec_model_shape* shape, int64_t kv_len, int32_t n_tokens,
                                  const dec_device_info* dev, struct dec_plan** out);

/* (Control calls: no passage of the pages covers them; they report and clear the device-side
 * watchdog that keeps a stuck dependency wait from hanging the persistent kernel.)
 * Synchronise `stream` and read the sticky device status word: DEC_OK, DEC_E_TIMEOUT (the
 * failing task id is in dec_last_error()) or DEC_E_CAPACITY (a dec_step_dynamic state out of
 * range). */
dec_status dec_plan_status(struct dec_plan* plan, void* stream);
/* Re-zero counters, epoch and status (after a timeout). */
dec_status dec_plan_reset(struct dec_plan* plan, void* stream);
/* Device watchdog budget for one dependency wait, in microseconds (default 2 000 000). */
dec_status dec_plan_set_watchdog(struct dec_plan* plan, int64_t microseconds);

/* The HBM read ceiling of the current device for the engine's access pattern, to set a step's
 * achieved bandwidth against: one launch in which every compute unit's workgroup streams a
 * contiguous share of `bytes` at `buf` with 16-byte non-temporal loads, as many in flight per
 * wave as the engine's weight ring, folding what it reads into one word per thread of `sink`
 * (n_cu * 512 words). The pages' premise is that a batch-1 decode step is bound by memory
 * bandwidth ("Static Compilation for LLM Inference", section 5.4); this is that bound as the
 * engine's loads meet it. Asynchronous on `stream`; time it with events.
 * Errors: INVAL (null, unaligned, bytes not a positive multiple of 16), CAPACITY (sink too
 * small), DEVICE, HIP. */
dec_status dec_stream_read(const void* buf, int64_t bytes, void* sink, int64_t sink_bytes, void* stream);

const char* dec_last_error(void);
/* Describe the current HIP device (gfx arch, CU/XCD counts, LDS). */
dec_status dec_device_query(dec_device_info* out);

#ifdef __cplusplus
}
#endif
#endif /* DEC_H_ */
