// engine.hip -- the persistent, tile-scheduled decode engine for gfx950 (MI355X).
//
// One launch runs a whole batch-1 decode step. Every workgroup (one per CU, 8 wave64)
// walks its statically planned task list. A task
//   1. issues the loads of its static operand (weight rows, cached K/V) into registers,
//   2. waits on its dependency counters (one wave polls with agent-scope loads; a workgroup
//      barrier does not drain the loads issued in step 1, so they stay in flight),
//   3. stages its dynamic input vector in LDS (with RMSNorm where the step needs it),
//   4. streams the rest of its rows with a double-buffered register ring, reducing each
//      row with wave-wide sums,
//   5. runs its epilogue (RoPE + KV append, SwiGLU, residual), stores, and signals its
//      counter after an agent-scope release.
// This is the pages' execution model: ahead-of-time compiled tile tasks in one persistent
// engine kernel that start as soon as their producers finish ("Static Compilation for LLM
// Inference ...", sections 1, 5.6 and 6; the TileRT talk's section on breaking kernel
// boundaries), with the cross-chiplet synchronisation done through memory with
// release/acquire and atomic adds (same page, section 7.4, on AMD's buffer_wbl2 /
// flat_atomic_add with scope bits). The first page's section 5.2 notes that a megakernel's
// register budget is the maximum over its task types and leaves one wave per SIMD; this
// engine runs two waves per SIMD and hides HBM latency with many outstanding 16-byte loads
// per lane instead of occupancy. Batch-1 GEMVs are memory-bound (section 5.4), so the row
// dot products run on the vector ALUs in fp32, not on MFMA.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <map>
#include <mutex>
#include <type_traits>

#include "plan_types.h"

namespace dec {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ small helpers

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest even (NaN stays NaN): gfx950's v_cvt_pk_bf16_f32
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// two values -> one bf16 pair (a in the low half), one instruction
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const bf2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// wave-uniform value (lets the compiler keep it in SGPRs and branch on it with scalar code)
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int wave_id() { return uni((int)(threadIdx.x >> 6)); }

// 16-byte non-temporal load through the global (not flat) address space, so it counts only
// against vmcnt and never against the LDS counter
typedef const u4 __attribute__((address_space(1)))* gu4p;
__device__ __forceinline__ u4 ldg_nt(const void* p) { return __builtin_nontemporal_load((gu4p)p); }

// Data exchanged between workgroups is written and read with agent-coherent (SC1) buffer
// accesses: an SC1 store is complete only once it is visible at agent scope, and an SC1 load
// never returns a stale line from this XCD's L2. A producer therefore publishes with
// "s_waitcnt vmcnt(0); barrier; atomic add", and a consumer needs no cache invalidation --
// neither the L2 write-back (buffer_wbl2) of an agent-scope release fence nor the L2
// invalidate (buffer_inv) of an acquire fence, which measure 1-9 us each on MI355X.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kSC0 = 1;           // cache-policy bit SC0: the load misses in the compute unit's L1
constexpr int kSC1 = 16;          // cache-policy bit SC1 (agent scope)
constexpr int kCoh = kSC0 | kSC1; // loads of the new cache row: agent-coherent, and missing in L1
constexpr int kNT = 2;            // cache-policy bit NT (streamed once: non-temporal)
// Cache policy of loads of produced data (activations written in this step). A reader reads an
// address only after all of its writers have signalled. A value written once per step by plain
// (SC1, write-through) stores may sit in the writer's L1 and its XCD's L2, but only as the value
// itself: such data is loaded with SC0 (missing in L1, which could also hold lines of this
// workgroup's earlier steps' tasks) and served by the XCD's L2, where the 32 workgroups of an XCD
// share one fetch of a broadcast vector. A buffer that is first stored and then accumulated with
// agent-scope atomics -- the GQA residual h (initialised by the previous layer's down
// projection, then added into by the per-group O-projections) and the latent-attention output
// (cleared by the latent-row append, then added into by the W_UV tasks) -- can leave the stored,
// pre-atomic line in the storing workgroup's L1 and its XCD's L2, since the atomics of the other
// workgroups do not update those copies: its readers load it agent-coherently (kCoh), from
// beyond every L2. (Found as one O-projection row that read whole heads of the latent output as
// the zeros its own workgroup had stored.)
constexpr int kActCpol = kSC0;
constexpr int kVmcnt0 = 0x0F70;   // s_waitcnt vmcnt(0) (expcnt, lgkmcnt unconstrained)
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ float cld(rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kActCpol));
}
__device__ __forceinline__ u4 cld4u(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kActCpol); }
// a word of an atomically accumulated buffer (see kActCpol)
__device__ __forceinline__ float cld_coh(rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kCoh));
}
__device__ __forceinline__ f4 cld4(rsrc_t r, uint32_t off) { return __builtin_bit_cast(f4, cld4u(r, off)); }
__device__ __forceinline__ void cst(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, kSC1);
}
__device__ __forceinline__ void cst16(rsrc_t r, uint32_t off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, kSC1);
}
__device__ __forceinline__ void cst4(rsrc_t r, uint32_t off, f4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, off, 0, kSC1);
}

typedef const void __attribute__((address_space(1)))* gvp;
typedef void __attribute__((address_space(3)))* lvp;

// One wave instruction of LDS DMA (16 bytes per lane from `src` to LDS at lds_dst + 16 * lane),
// written so that the compiler does not track it: each caller waits for it explicitly
// (s_waitcnt vmcnt) before the copied data is read. Tracked, the compiler would make every wave
// wait at the next barrier for all of its own loads in flight (a barrier publishes LDS writes),
// which would drain the weight prefetch that the other waves hold across the staging step. The
// instruction has no destination register; M0 (the LDS base) is saved and restored around it,
// and one wait state separates its write from the DMA that reads it. COH selects the cache
// policy: false -- SC0, missing in L1 and served by the XCD's L2 (produced data written once per
// step); true -- SC0 SC1, agent-coherent (data that other XCDs update with atomics, see kActCpol).
static_assert(kActCpol == kSC0, "the untracked LDS DMA is written with the SC0 cache policy");
template <bool COH = false>
__device__ __forceinline__ void lds_dma16(const void* src, float* lds_dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lvp)lds_dst);
  uint32_t saved;
  if constexpr (COH)
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off sc0 sc1\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(src), "s"(base)
                 : "memory");
  else
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off sc0\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(src), "s"(base)
                 : "memory");
}

// Wave-wide LDS DMA of `nfloats` floats (a multiple of 4) of produced data from global memory
// into LDS; lane l of instruction j lands at dst[j*256 + 4l]. Lanes past the end re-read the
// last 16 bytes and land in dst[nfloats, round_up(nfloats, 256)), which the destination must
// have room for. Completion is counted by vmcnt, which the caller waits for.
template <bool COH = false>
__device__ __forceinline__ void dma_to_lds(float* dst, const float* src, int nfloats) {
  const int lane = threadIdx.x & 63;
  for (int j = 0; j * 256 < nfloats; ++j) {
    int i = j * 256 + lane * 4;
    i = i < nfloats ? i : nfloats - 4;
    lds_dma16<COH>(src + i, dst + j * 256);
  }
}

// The same copy split over all waves of the workgroup (1-KB chunk j by wave j % 8): for copies
// longer than one wave keeps in flight. Every wave must call it; each waits for its own part
// (after its own loads issued earlier), and the caller's barrier publishes the whole.
template <bool COH = false>
__device__ __forceinline__ void dma_to_lds_all(float* dst, const float* src, int nfloats) {
  const int lane = threadIdx.x & 63;
  for (int j = (int)(threadIdx.x >> 6); j * 256 < nfloats; j += kWaves) {
    int i = j * 256 + lane * 4;
    i = i < nfloats ? i : nfloats - 4;
    lds_dma16<COH>(src + i, dst + j * 256);
  }
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
}

__device__ __forceinline__ uint64_t now() { return __builtin_amdgcn_s_memrealtime(); }

// The per-task execution log (one 64-byte record per task and step). Level 1 (the default)
// records what the coverage and dependency-order checks read: the execution count, the
// workgroup and XCD, and three clock reads by wave 0 -- task start, the moment its dependency
// wait succeeded, and its completion stamp just before its counter increment. Each clock read
// is a scalar memory operation whose result is awaited only where the wave waits anyway.
// Level 2 adds the per-phase stamps used to analyse a step (staged, streamed, sub-phases, end);
// those sit on the critical path. Level 0 leaves the log out.
#ifndef DEC_TASK_LOG
#define DEC_TASK_LOG 1
#endif
constexpr bool kTaskLog = DEC_TASK_LOG >= 1;
constexpr bool kTaskLogDetail = DEC_TASK_LOG >= 2;
__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xfu;
}

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Cross-lane sums with DPP (VALU lane permutes, no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
constexpr int kQuadSwap1 = 0xB1;      // quad_perm(1,0,3,2): lane ^ 1
constexpr int kQuadSwap2 = 0x4E;      // quad_perm(2,3,0,1): lane ^ 2
constexpr int kRowHalfMirror = 0x141; // reverse within 8-lane halves of a row
constexpr int kRowMirror = 0x140;     // reverse within a 16-lane row

// Sum over aligned groups of W lanes (W = 1..64, a power of two); every lane of a group
// gets the group's sum.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  if (W >= 2) v += dpp<kQuadSwap1>(v);
  if (W >= 4) v += dpp<kQuadSwap2>(v);
  if (W >= 8) v += dpp<kRowHalfMirror>(v);   // after the quad sums: quad q gets quad q^1
  if (W >= 16) v += dpp<kRowMirror>(v);      // after the 8-lane sums: half h gets half h^1
  if (W >= 32) v += __shfl_xor(v, 16, 64);
  if (W >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}
// Full 64-lane sum, returned wave-uniform.
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  const int b = __float_as_int(v);
  return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) + __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(b, 32)) + __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}

// Full 64-lane maximum, returned wave-uniform.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<kQuadSwap1>(v));
  v = fmaxf(v, dpp<kQuadSwap2>(v));
  v = fmaxf(v, dpp<kRowHalfMirror>(v));
  v = fmaxf(v, dpp<kRowMirror>(v));
  const int b = __float_as_int(v);
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)), __int_as_float(__builtin_amdgcn_readlane(b, 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)), __int_as_float(__builtin_amdgcn_readlane(b, 48))));
}

// 2^x with the hardware instruction alone (no denormal-range scaling): results below 2^-126
// come out as 0. The softmax weights use it with x <= 0 relative to a running maximum, so it
// only drops terms smaller than 2^-126 of the largest one.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ uint64_t uni64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
template <class T>
__device__ __forceinline__ const T* wp(const EngineArgs& A, int idx) {
  return reinterpret_cast<const T*>(uni64(A.wptr[idx]));
}

// ------------------------------------------------------------------ per-workgroup state

struct Blk {
  rsrc_t act;     // coherent view of the activation region (byte offsets = 4 * float offsets)
  uint32_t epoch;
  uint32_t t_ready, t_staged, t_streamed;
  uint32_t t_sub[3];  // sub-phase stamps of the current task (thread 0; logged as t_aux[2..4])
  float norm;         // 1 / rms of the staged input (RMSNorm applied to the row results), else 1
  int* flags;     // LDS: [0] wait status, [1] ticket result
  float* xs;      // LDS: staged input vector
  float* ys;      // LDS: per-row results of the current task
  float* scr;     // LDS: reduction scratch
  uint64_t* rowp; // LDS: row pointers of the current GEMV task
  int* xoffp;     // LDS: per-row input offsets of the current GEMV task
  float* scl;     // LDS: per-row weight scales of the current GEMV task (FP8 weights)
  uint64_t* srowp; // LDS: per-row block-scale pointers of the current GEMV task (MXFP4 weights)
  float* gs;      // LDS: norm gains (bf16) of the current task
  float* actp;    // the activation region (generic pointer, for LDS DMA)
  int n;                // the step's position: cached positions [0, n), the new token's slot n
  const uint16_t* x;    // the step's input vector (bf16 [hidden])
  const float* rope;    // RoPE (cos, sin) row of position n
};

// Positions [split_pos(n, sp, S), split_pos(n, sp + 1, S)) of attention split sp of S over
// the positions 0..n (the planner cuts static plans the same way).
__device__ __forceinline__ int split_pos(int n, int sp, int S) { return (int)(((int64_t)n + 1) * sp / S); }

struct NoEarly {
  __device__ __forceinline__ void operator()() const {}
};

// Wait until every dependency counter of `t` has reached this step's target. Wave 0 polls
// (one lane per counter, agent-scope loads); the other waves wait at the barrier with their
// loads in flight. `early` runs on wave 0 once the wait has succeeded, before that barrier:
// loads it issues enter the memory queue ahead of whatever the released waves issue next.
// Returns false when the step is being aborted (watchdog).
template <class EarlyF = NoEarly>
__device__ __forceinline__ bool wait_deps(const EngineArgs& A, Blk& b, const TaskDesc& t, int d0 = 0, int d1 = -1,
                                          EarlyF&& early = EarlyF{}) {
  if (d1 < 0) d1 = t.dep_count;
  const int nd = d1 - d0;  // waits on dependencies [d0, d1) of the task
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int status = 0;
    if (nd > 0) {
      const DepEntry* dl = A.deps + t.dep_first + d0;
      const uint32_t* cp = A.ctl;  // any valid address for idle lanes
      uint32_t target = 0;
      if (lane < nd) {
        const DepEntry d = dl[lane];
        cp = A.counters + (size_t)d.counter * kCounterStride;
        target = (b.epoch + 1u) * d.per_step;
      }
      const uint64_t t0 = now();
      uint32_t spins = 0;
      while (true) {
        const bool ok = (lane >= nd) || ((int32_t)(ld_agent(cp) - target) >= 0);
        if (__all(ok)) break;
        if ((++spins & 7u) == 0u) {  // the clock and the abort word every 8th round
          const bool late = (now() - t0) > (uint64_t)A.watchdog_ticks;
          const uint32_t ab = ld_agent(A.ctl + CTL_ABORT);
          if (ab || late) {
            if (!ab && lane == 0) {
              uint32_t zero = 0;
              if (__hip_atomic_compare_exchange_strong(A.ctl + CTL_STATUS, &zero, 7u, __ATOMIC_RELAXED,
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                st_agent(A.ctl + CTL_STATUS + 1, (uint32_t)t.id);
                st_agent(A.ctl + CTL_STATUS + 2, (uint32_t)A.deps[t.dep_first].counter);
                st_agent(A.ctl + CTL_STATUS + 3, ld_agent(A.counters + (size_t)A.deps[t.dep_first].counter * kCounterStride));
              }
              st_agent(A.ctl + CTL_ABORT, 1u);
            }
            status = 1;
            break;
          }
        }
        __builtin_amdgcn_s_sleep(1);
      }
      // no cache invalidate: produced data is read with SC1 loads; the workgroup-scope fence
      // only keeps the compiler from hoisting those loads above the poll
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    if (kTaskLog) b.t_ready = (uint32_t)now();  // the wait has succeeded (wave 0)
    if (__builtin_amdgcn_readfirstlane(status) == 0) early();
    if (lane == 0) b.flags[0] = status;
  }
  __syncthreads();
  return b.flags[0] == 0;
}

// The producer's completion stamp (wave 0): the clock is read before the wait for the task's
// stores, and that wait also covers the read (lgkmcnt), so the read has returned -- and the time
// it holds has passed -- before the counter increment is issued: every consumer that sees the
// increment passed its wait (and stamped t_ready) after this time.
constexpr int kVmLgkm0 = 0x0070;  // s_waitcnt vmcnt(0) lgkmcnt(0)
__device__ __forceinline__ uint32_t store_wait_stamp() {
  uint32_t ts = 0;
  if (kTaskLog) ts = (uint32_t)now();
  __builtin_amdgcn_s_waitcnt(kTaskLog ? kVmLgkm0 : kVmcnt0);
  return ts;
}

// Every wave waits for its own SC1 stores to complete, then the barrier, then one counter
// increment: the produced data is visible at agent scope before the counter moves. Returns
// the completion stamp (meaningful in wave 0).
__device__ __forceinline__ uint32_t signal(const EngineArgs& A, int ctr) {
  const uint32_t ts = store_wait_stamp();
  __syncthreads();
  if (threadIdx.x == 0 && ctr >= 0) add_agent(A.counters + (size_t)ctr * kCounterStride, 1u);
  return ts;
}

// After a GEMV task, whose results wave 0 stored alone: wave 0 waits for its stores and
// increments the counter, while the other waves go straight on to the next task and issue
// its prefetch (the next task's barriers keep the LDS hand-over in order: its input is
// staged by wave 0, and its row results are written only after its staging barrier).
__device__ __forceinline__ uint32_t signal_w0(const EngineArgs& A, int ctr) {
  if (threadIdx.x < 64) {
    const uint32_t ts = store_wait_stamp();
    if (threadIdx.x == 0 && ctr >= 0) add_agent(A.counters + (size_t)ctr * kCounterStride, 1u);
    return ts;
  }
  return 0u;
}

__device__ __forceinline__ int pad512(int k) { return (k + kChunkCols - 1) / kChunkCols * kChunkCols; }
// A staged input padded to whole GEMV chunks of weights with ES bytes each (512 or 1024
// columns; 2048 for MXFP4, ES = 0).
template <int ES>
__device__ __forceinline__ int padc(int k) {
  constexpr int c = ES == 0 ? 2048 : 1024 / (ES ? ES : 1);
  return (k + c - 1) / c * c;
}
// The fp32 row scales of an FP8 matrix: the weight after it in the bound list.
template <int ES>
__device__ __forceinline__ const float* wscale(const EngineArgs& A, int idx) { return ES == 1 ? wp<float>(A, idx + 1) : nullptr; }

// The longest input one wave copies alone, the moment its wait succeeds (32 1-KB chunks of LDS
// DMA); a longer one (the down projections' 14336 floats, the per-group merge of 32 split
// partials) is copied by all waves in turn, which was measured faster on the 8B model (3130
// against 3182 us per step with 60-chunk single-wave copies).
#ifndef DEC_EARLY_DMA_FLOATS
#define DEC_EARLY_DMA_FLOATS 8192
#endif
constexpr int kEarlyDmaFloats = DEC_EARLY_DMA_FLOATS;

// Staging of a task's input vector into xs[0, K) (zero-padded to padK), in three parts so that
// every load goes out as early as it may:
//   before -- wave 0, ahead of the dependency wait: the norm gains (weights, known statically);
//   early  -- wave 0, the moment the wait succeeds and before the barrier that releases the
//             other waves: the LDS DMA of the activation vector, which thus enters the compute
//             unit's memory queue ahead of the ring batch those waves issue next (the unit
//             returns its loads roughly in issue order);
//   finish -- every wave: completes the copy, zero-pads, and with a gain g stores g * x.
// The source is the activation region at float offset `off`, or the bf16 step input s16 when
// off < 0 (converted to fp32 by wave 0 in `finish`). With a gain the step's RMSNorm,
// x / sqrt(mean(x^2) + eps) * g (eps inside the square root, mean over K), is applied as
// 1 / rms to each row result of the GEMV (W (g x) / rms = W RMSNorm(x)); the sum of squares
// is taken by all waves while they apply the gains. `inplace` instead leaves the normalised
// vector itself in xs (a consumer that reads the vector, not a GEMV).
struct StageVec {
  int off;
  const uint16_t* s16;
  int K, padK;
  const uint16_t* gain;
  float eps;
  bool inplace;
  bool coh;  // the vector is an atomically accumulated buffer: read it agent-coherently (kActCpol)
  __device__ __forceinline__ bool early_ok() const { return off >= 0 && K <= kEarlyDmaFloats; }
  __device__ __forceinline__ void before(Blk& b) const {  // wave 0
    if (gain) dma_to_lds(b.gs, (const float*)gain, K / 2);
  }
  __device__ __forceinline__ void early(Blk& b) const {  // wave 0
    if (early_ok()) {
      if (coh) dma_to_lds<true>(b.xs, b.actp + off, K);
      else dma_to_lds(b.xs, b.actp + off, K);
    }
  }
  __device__ __forceinline__ void finish(Blk& b) const {
    if (off >= 0 && !early_ok()) {  // too long for one wave
      if (coh) dma_to_lds_all<true>(b.xs, b.actp + off, K);
      else dma_to_lds_all(b.xs, b.actp + off, K);
    }
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      if (off < 0) {
        // the bf16 step input (layer 0): batched loads, converted to fp32
        for (int i0 = lane * 4; i0 < K; i0 += 64 * 4 * 4) {
          f4 v[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * 256;
            const uint2 x = *(const uint2*)(s16 + (i < K ? i : 0));
            v[u] = f4{bf_lo(x.x), bf_hi(x.x), bf_lo(x.y), bf_hi(x.y)};
          }
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (i0 + u * 256 < K) *(f4*)(b.xs + i0 + u * 256) = v[u];
        }
      }
      __builtin_amdgcn_s_waitcnt(kVmcnt0);  // wave 0's copies (vector, gains) have landed
      if (kTaskLogDetail && lane == 0) b.t_sub[0] = (uint32_t)now();
    }
    // a copy by all waves whose last 1-KB block is partial also writes words [K, K rounded up
    // to 256) (its clamped lanes): every wave's copy must have landed before they are cleared
    if (off >= 0 && !early_ok() && (K & 255)) __syncthreads();
    if (threadIdx.x < 64)
      for (int i = K + (int)threadIdx.x; i < padK; i += 64) b.xs[i] = 0.f;
    __syncthreads();
    b.norm = 1.f;
    if (gain) {
      const uint16_t* g16 = reinterpret_cast<const uint16_t*>(b.gs);
      float ss = 0.f;
      for (int i = threadIdx.x * 4; i < K; i += kThreads * 4) {
        const uint2 g = *(const uint2*)(g16 + i);
        f4 v = *(f4*)(b.xs + i);
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        v.x *= bf_lo(g.x);
        v.y *= bf_hi(g.x);
        v.z *= bf_lo(g.y);
        v.w *= bf_hi(g.y);
        *(f4*)(b.xs + i) = v;
      }
      ss = wave_sum(ss);
      float* part = reinterpret_cast<float*>(b.flags) + 8;  // per-wave sums of squares
      if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
      __syncthreads();
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) tot += part[w];
      b.norm = 1.0f / sqrtf(tot / (float)K + eps);
      if (kTaskLogDetail && threadIdx.x == 0) b.t_sub[1] = (uint32_t)now();
      if (inplace) {
        for (int i = threadIdx.x; i < K; i += kThreads) b.xs[i] *= b.norm;
        __syncthreads();
      }
    }
  }
};

__device__ __forceinline__ StageVec stage_vec(int off, const uint16_t* s16, int K, int padK, const uint16_t* gain, float eps,
                                              bool inplace = false, bool coh = false) {
  return StageVec{off, s16, K, padK, gain, eps, inplace, coh};
}

// All three parts in a row, for a task that is not a GEMV (it calls wait_deps itself).
__device__ __forceinline__ void stage_now(Blk& b, const StageVec& sv) {
  if (threadIdx.x < 64) {
    sv.before(b);
    sv.early(b);
  }
  sv.finish(b);
}

// A custom staging step (all in `finish`); the GEMV's row results are not rescaled.
template <class F>
struct StageFn {
  F f;
  __device__ __forceinline__ void before(Blk&) const {}
  __device__ __forceinline__ void early(Blk&) const {}
  __device__ __forceinline__ void finish(Blk& b) const {
    f();
    b.norm = 1.f;
  }
};
template <class F>
__device__ __forceinline__ StageFn<F> stage_fn(F f) { return StageFn<F>{f}; }

// ------------------------------------------------------------------ streaming row GEMV

#ifndef DEC_NB
#define DEC_NB 8
#endif
constexpr int NB = DEC_NB;  // 16-byte chunks per batch per lane (NB KB per wave per batch)
#ifndef DEC_NB_FP8
#define DEC_NB_FP8 6
#endif
// chunks per batch of a GEMV stream by weight format: an FP8 chunk spans twice the columns of a
// bf16 one, and batches of six measured faster for FP8 rows than batches of eight
constexpr int batch_chunks(int es) { return es == 1 ? DEC_NB_FP8 : NB; }
#ifndef DEC_RING_QKV
#define DEC_RING_QKV 2
#endif
#ifndef DEC_RING_OPROJ
#define DEC_RING_OPROJ 2
#endif
constexpr int kRingQKV = DEC_RING_QKV;      // register ring depth of the QKV tasks
constexpr int kRingOproj = DEC_RING_OPROJ;  // register ring depth of the per-group O-projection
constexpr int kRingFfn = 3;  // gate/up and (GQA) down: three batches in flight cover more of the stage boundary


// One wave load is 16 bytes per lane: 8 bf16, 16 FP8 (E4M3) or 32 MXFP4 (E2M1) weights.
// ES = bytes per weight (2 bf16, 1 FP8), or 0 for MXFP4: a lane's 16 bytes are then exactly one
// block of 32 elements sharing one E8M0 scale byte (loaded beside the weights, `sb`), element
// 2i in the low nibble of byte i. A chunk (one wave load) spans kCols columns.
template <int ES>
struct Chunk {
  static constexpr int kCols = ES == 0 ? 2048 : 1024 / (ES ? ES : 1);  // columns per chunk
  static constexpr int kLane = ES == 0 ? 32 : 16 / (ES ? ES : 1);      // columns per lane
  // bytes of `cols` consecutive weights of a row
  __device__ static __forceinline__ size_t bytes(int cols) { return ES == 0 ? (size_t)cols / 2 : (size_t)cols * ES; }
  // acc0/acc1 += the lane's weights . x (xp: the lane's kLane inputs in LDS)
  // MXFP4: a lane's 32 inputs are 128 bytes of LDS, 128 bytes from the next lane's, so lanes
  // reading the same quad of their inputs together would all hit the same four banks. Each lane
  // instead takes its eight quads starting at its own quad `rot` (lanes 8 apart differ by one,
  // so any 8 or 16 consecutive lanes read distinct banks), and its weights are rotated to match.
  __device__ static __forceinline__ int rot_of(int lane) { return (lane + (lane >> 3)) & 7; }
  // quad J of the rotated weights (bytes 2 (J & 1), 2 (J & 1) + 1 of r[J / 2]) times input quad (J + rot) & 7
  template <int J>
  __device__ static __forceinline__ void quad(const uint32_t (&r)[4], float sc, const float* xp, int rot, float& acc0, float& acc1) {
    const f4 x = *(const f4*)(xp + 4 * ((J + rot) & 7));
    const f2 e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r[J >> 1], sc, 2 * (J & 1));
    const f2 e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r[J >> 1], sc, 2 * (J & 1) + 1);
    acc0 = fmaf(e0.x, x.x, acc0);
    acc1 = fmaf(e0.y, x.y, acc1);
    acc0 = fmaf(e1.x, x.z, acc0);
    acc1 = fmaf(e1.y, x.w, acc1);
  }
  __device__ static __forceinline__ void dot(const u4& w, uint32_t sb, const float* xp, float& acc0, float& acc1, int rot = 0) {
    if constexpr (ES == 0) {
      // hardware E2M1 -> fp32 conversion of one byte (two elements) per instruction, scaled by
      // the block's power of two 2^(sb - 127)
      const float sc = __builtin_amdgcn_ldexpf(1.0f, (int)(sb & 0xffu) - 127);
      // rotate the eight 16-bit quads: quad j of r[] is quad (j + rot) & 7 of w
      const bool r4 = rot & 4, r2 = rot & 2, r1 = rot & 1;
      const uint32_t b0 = r4 ? w.z : w.x, b1 = r4 ? w.w : w.y, b2 = r4 ? w.x : w.z, b3 = r4 ? w.y : w.w;
      const uint32_t c0 = r2 ? b1 : b0, c1 = r2 ? b2 : b1, c2 = r2 ? b3 : b2, c3 = r2 ? b0 : b3;
      const uint32_t r[4] = {r1 ? __builtin_amdgcn_alignbit(c1, c0, 16) : c0, r1 ? __builtin_amdgcn_alignbit(c2, c1, 16) : c1,
                             r1 ? __builtin_amdgcn_alignbit(c3, c2, 16) : c2, r1 ? __builtin_amdgcn_alignbit(c0, c3, 16) : c3};
      quad<0>(r, sc, xp, rot, acc0, acc1);
      quad<1>(r, sc, xp, rot, acc0, acc1);
      quad<2>(r, sc, xp, rot, acc0, acc1);
      quad<3>(r, sc, xp, rot, acc0, acc1);
      quad<4>(r, sc, xp, rot, acc0, acc1);
      quad<5>(r, sc, xp, rot, acc0, acc1);
      quad<6>(r, sc, xp, rot, acc0, acc1);
      quad<7>(r, sc, xp, rot, acc0, acc1);
    } else if constexpr (ES == 2) {
      const f4 x0 = *(const f4*)xp, x1 = *(const f4*)(xp + 4);
      acc0 = fmaf(bf_lo(w.x), x0.x, acc0);
      acc1 = fmaf(bf_hi(w.x), x0.y, acc1);
      acc0 = fmaf(bf_lo(w.y), x0.z, acc0);
      acc1 = fmaf(bf_hi(w.y), x0.w, acc1);
      acc0 = fmaf(bf_lo(w.z), x1.x, acc0);
      acc1 = fmaf(bf_hi(w.z), x1.y, acc1);
      acc0 = fmaf(bf_lo(w.w), x1.z, acc0);
      acc1 = fmaf(bf_hi(w.w), x1.w, acc1);
    } else {
      // hardware E4M3 -> fp32 conversion, two bytes per instruction (bytes 0, 1 of the
      // selected 16-bit half are the lower two columns)
      const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f4 x = *(const f4*)(xp + 4 * q);
        const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[q], false);
        const f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wd[q], true);
        acc0 = fmaf(lo.x, x.x, acc0);
        acc1 = fmaf(lo.y, x.y, acc1);
        acc0 = fmaf(hi.x, x.z, acc0);
        acc1 = fmaf(hi.y, x.w, acc1);
      }
    }
  }
};

// Streams the rows [ja, jb) of a task through a register double buffer. Row j has K
// columns (ES bytes each) starting at rowp[j] (an LDS table filled by fill_rows) and is
// dotted with xs[xoff[j] + c].
template <int ES>
struct StreamT {
  using C = Chunk<ES>;
  static constexpr int BN = batch_chunks(ES);  // chunks per batch
  const uint64_t* rowp;
  const uint64_t* srowp;  // MXFP4: the rows' scale pointers
  const int* xoffp;
  int jb, K, cpr, lane;
  int lj, lc;
  const uint8_t* lrow;
  const uint8_t* lsrow;
  int cj, cc, cxo;
  float acc0, acc1;

  __device__ __forceinline__ void init(const uint64_t* rp, const uint64_t* srp, const int* xp, int ja, int jb_, int K_,
                                       int lane_) {
    rowp = rp;
    srowp = srp;
    xoffp = xp;
    jb = jb_;
    K = K_;
    lane = lane_;
    cpr = (K + C::kCols - 1) / C::kCols;
    lj = ja;
    lc = 0;
    lrow = (ja < jb) ? (const uint8_t*)uni64(rowp[ja]) : nullptr;
    lsrow = (ES == 0 && ja < jb) ? (const uint8_t*)uni64(srowp[ja]) : nullptr;
    cj = ja;
    cc = 0;
    cxo = (ja < jb) ? uni(xoffp[ja]) : 0;
    acc0 = acc1 = 0.f;
  }
  __device__ __forceinline__ void load(u4 (&bf)[BN], uint32_t (&sb)[BN]) {
#pragma unroll
    for (int i = 0; i < BN; ++i) {
      if (lj < jb) {
        int col = lc * C::kCols + lane * C::kLane;
        const bool in = col < K;
        col = in ? col : 0;  // masked lanes re-read the row start (bf16/FP8: xs is zero there)
        bf[i] = ldg_nt(lrow + C::bytes(col));
        if constexpr (ES == 0) sb[i] = __builtin_nontemporal_load(lsrow + (in ? lc * 64 + lane : 0));
        if (++lc == cpr) {
          lc = 0;
          if (++lj < jb) {
            lrow = (const uint8_t*)uni64(rowp[lj]);
            if constexpr (ES == 0) lsrow = (const uint8_t*)uni64(srowp[lj]);
          }
        }
      }
    }
  }
  template <class Emit>
  __device__ __forceinline__ void consume(const u4 (&bf)[BN], const uint32_t (&sb)[BN], const float* xs, Emit& emit) {
#pragma unroll
    for (int i = 0; i < BN; ++i) {
      if (cj < jb) {
        if constexpr (ES == 0) {
          // lanes past the row's end hold no elements (the staged input is not padded to whole
          // 2048-column chunks): their products are dropped
          float p0 = 0.f, p1 = 0.f;
          C::dot(bf[i], sb[i], xs + cxo + cc * C::kCols + lane * C::kLane, p0, p1, C::rot_of(lane));
          const bool in = cc * C::kCols + lane * C::kLane < K;
          acc0 += in ? p0 : 0.f;
          acc1 += in ? p1 : 0.f;
        } else {
          C::dot(bf[i], 0u, xs + cxo + cc * C::kCols + lane * C::kLane, acc0, acc1);
        }
        if (++cc == cpr) {
          emit(cj, wave_sum(acc0 + acc1));
          acc0 = acc1 = 0.f;
          cc = 0;
          if (++cj < jb) cxo = uni(xoffp[cj]);
        }
      }
    }
  }
};

// Like Stream, but over a range of the task's flattened (row, chunk) sequence: chunk f is
// chunk f % cpr of row f / cpr, and a wave's range [fa, fb) may start and end inside a row.
// Each row's partial dot product over the chunks the wave holds is emitted when its part of
// the row ends. Used where a task has few, long rows: whole rows per wave would leave the
// waves up to a row apart (3 rows against 2 for 16 rows over 7 waves), and the last waves
// alone could not keep enough loads in flight.
template <int ES>
struct StreamFlatT {
  using C = Chunk<ES>;
  static constexpr int BN = batch_chunks(ES);  // chunks per batch
  static_assert(ES != 0, "MXFP4 rows stream whole rows per wave (StreamT)");
  const uint64_t* rowp;
  const int* xoffp;
  int fb, K, cpr, lane;
  int lf, lj, lc;
  const uint8_t* lrow;
  int cf, cj, cc, cxo;
  float acc0, acc1;

  __device__ __forceinline__ void init(const uint64_t* rp, const uint64_t*, const int* xp, int fa, int fb_, int K_,
                                       int lane_) {
    rowp = rp;
    xoffp = xp;
    fb = fb_;
    K = K_;
    lane = lane_;
    cpr = (K + C::kCols - 1) / C::kCols;
    const int j0 = fa / cpr, c0 = fa - j0 * cpr;
    lf = cf = fa;
    lj = cj = j0;
    lc = cc = c0;
    lrow = (fa < fb) ? (const uint8_t*)uni64(rowp[j0]) : nullptr;
    cxo = (fa < fb) ? uni(xoffp[j0]) : 0;
    acc0 = acc1 = 0.f;
  }
  __device__ __forceinline__ void load(u4 (&bf)[BN], uint32_t (&)[BN]) {
#pragma unroll
    for (int i = 0; i < BN; ++i) {
      if (lf < fb) {
        int col = lc * C::kCols + lane * C::kLane;
        col = col < K ? col : 0;  // masked lanes re-read the row start; xs is zero there
        bf[i] = ldg_nt(lrow + C::bytes(col));
        ++lf;
        if (++lc == cpr) {
          lc = 0;
          ++lj;
          if (lf < fb) lrow = (const uint8_t*)uni64(rowp[lj]);
        }
      }
    }
  }
  template <class Emit>
  __device__ __forceinline__ void consume(const u4 (&bf)[BN], const uint32_t (&)[BN], const float* xs, Emit& emit) {
#pragma unroll
    for (int i = 0; i < BN; ++i) {
      if (cf < fb) {
        C::dot(bf[i], 0u, xs + cxo + cc * C::kCols + lane * C::kLane, acc0, acc1);
        ++cf;
        const bool row_end = ++cc == cpr;
        if (row_end || cf == fb) {
          emit(cj, wave_sum(acc0 + acc1));
          acc0 = acc1 = 0.f;
          if (row_end) {
            cc = 0;
            ++cj;
            if (cf < fb) cxo = uni(xoffp[cj]);
          }
        }
      }
    }
  }
};

using Stream = StreamT<2>;
using StreamFlat = StreamFlatT<2>;

// Each wave writes the row pointers / input offsets of its own rows (no barrier needed:
// LDS accesses of one wave are ordered).
template <int ES = 2, class RM>
__device__ __forceinline__ void fill_rows(const RM& rm, int ja, int jb, uint64_t* rowp, int* xoffp, uint64_t* srowp = nullptr) {
  for (int j = ja + (int)(threadIdx.x & 63); j < jb; j += 64) {
    rowp[j] = (uint64_t)(uintptr_t)rm.row(j);
    xoffp[j] = rm.xoff(j);
    if constexpr (ES == 0) srowp[j] = (uint64_t)(uintptr_t)rm.srow(j);
  }
}

// Work split over the waves of a workgroup. Wave 0 polls the dependency counters, and a
// poll cannot complete before that wave's earlier loads (vmcnt counts in issue order), so
// wave 0 streams nothing: it polls, helps stage the input vector and signals, while waves
// 1..7 prefetch and stream. Returns the start of wave `w`'s part of [0, n).
__device__ __forceinline__ int wave_start(int n, int w) {
  return (w == 0) ? 0 : (int)(((int64_t)n * (w - 1)) / (kWaves - 1));
}

// The shared skeleton of every GEMV task. Rows are split over the waves in whole groups of
// G rows (G consecutive rows are summed into one result ys[j / G]). With `prefetch`, the
// row map may not depend on anything this task waits for: the first two batches are issued
// before the dependency wait.
// R is the depth of the register ring (batches of NB chunks): all R batches are in flight when
// the wait begins. The big FFN and LM-head stages use R = 2; the small, latency-bound stages
// of the attention block use a deeper ring, so that most or all of a workgroup's rows are
// already loading while it waits.
// `pre_deps` > 0: the row map depends on the task's first pre_deps dependencies (the MoE
// expert choice). The task waits for those, runs `pre` (wave 0 puts what the row map reads
// into LDS), then issues its prefetch (such a task passes prefetch = true) before waiting
// for the rest. `prefetch` must be a compile-time constant at every call: with loads issued
// on two alternative paths the compiler cannot count the loads in flight, and the stream
// loop would wait for all of them before every batch.
// `issue` runs on every wave once the input is staged, before the stream: it may start loads
// of data the next task needs. (Issued earlier, such loads would sit in the compute unit's
// memory queue ahead of the staging loads, which wait for the dependency.)
struct NoPre {
  __device__ __forceinline__ void operator()() const {}
};
// FLAT: the waves split the rows' chunks evenly (StreamFlat; G must be 1) and the partial
// row sums meet in ys through LDS float atomics (two waves at most share a row, so the sum
// does not depend on their order); otherwise each wave streams whole groups of G rows.
template <int R = 2, bool FLAT = false, int ES = 2, class RM, class StageT, class EpiF, class PreF = NoPre,
          class IssueF = NoPre>  // R in [2, 4]; ES: bytes per weight (2 bf16, 1 FP8 with row scales)
__device__ __forceinline__ bool run_gemv(const EngineArgs& A, Blk& b, const TaskDesc& t, const RM& rm, int nrows,
                                         int K, int G, bool prefetch, const StageT& stage, EpiF&& epi, int pre_deps = 0,
                                         PreF&& pre = PreF{}, IssueF&& issue = IssueF{}) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int ng = nrows / G;
  int ja, jb, fa, fb;
  if constexpr (FLAT) {
    const int cpr = (K + Chunk<ES>::kCols - 1) / Chunk<ES>::kCols, nf = nrows * cpr;
    fa = wave_start(nf, wave);
    fb = wave_start(nf, wave + 1);
    ja = fa / cpr;
    jb = (fb + cpr - 1) / cpr;
  } else {
    ja = wave_start(ng, wave) * G;
    jb = wave_start(ng, wave + 1) * G;
    fa = ja;
    fb = jb;
  }
  typename std::conditional<FLAT, StreamFlatT<ES>, StreamT<ES>>::type s;
  constexpr int BN = batch_chunks(ES);
  u4 buf[R][BN];
  uint32_t sbuf[R][BN];  // MXFP4 block scales (unused for the other formats)
  if (threadIdx.x < 64) stage.before(b);
  if (pre_deps > 0) {
    if (!wait_deps(A, b, t, 0, pre_deps)) return false;
    pre();
    __syncthreads();
  }
  if constexpr (ES == 1) {
    // FP8 rows: wave 0 (no weight loads in flight) puts the task's row scales into LDS (after
    // `pre`, which stages what a run-time row map reads); the barrier of the dependency wait
    // publishes them
    if (threadIdx.x < 64)
      for (int j = (int)threadIdx.x; j < nrows; j += 64) b.scl[j] = rm.scale(j);
  }
  if (prefetch) {
    fill_rows<ES>(rm, ja, jb, b.rowp, b.xoffp, b.srowp);
    s.init(b.rowp, b.srowp, b.xoffp, fa, fb, K, lane);
#pragma unroll
    for (int k = 0; k < R; ++k) s.load(buf[k], sbuf[k]);
  }
  // wave 0 issues the input's copy the moment the wait succeeds (StageVec::early)
  if (!wait_deps(A, b, t, pre_deps, -1, [&] { stage.early(b); })) return false;
  if constexpr (FLAT)
    for (int i = threadIdx.x; i < ng; i += kThreads) b.ys[i] = 0.f;  // row sums (the stage's barrier orders this)
  stage.finish(b);
  const float nrm = b.norm;
  if (kTaskLogDetail && threadIdx.x == 0) b.t_staged = (uint32_t)now();
  issue();
  if (!prefetch) {
    fill_rows<ES>(rm, ja, jb, b.rowp, b.xoffp, b.srowp);
    s.init(b.rowp, b.srowp, b.xoffp, fa, fb, K, lane);
#pragma unroll
    for (int k = 0; k < R; ++k) s.load(buf[k], sbuf[k]);
  }
  float gacc = 0.f;
  auto emit = [&](int j, float v) {
    v *= nrm;                              // 1 / rms of a normalised input (else 1)
    if constexpr (ES == 1) v *= b.scl[j];  // G == 1 for FP8 rows
    if constexpr (FLAT) {
      if (lane == 0) atomicAdd(b.ys + j, v);
    } else {
      gacc += v;
      if (j % G == G - 1) {
        if (lane == 0) b.ys[j / G] = gacc;
        gacc = 0.f;
      }
    }
  };
  auto more = [&] {
    if constexpr (FLAT) return s.cf < fb;
    else return s.cj < jb;
  };
  while (more()) {
    s.consume(buf[0], sbuf[0], b.xs, emit);
    s.load(buf[0], sbuf[0]);
    if (!more()) break;
    s.consume(buf[1], sbuf[1], b.xs, emit);
    s.load(buf[1], sbuf[1]);
    if constexpr (R > 2) {
      if (!more()) break;
      s.consume(buf[2], sbuf[2], b.xs, emit);
      s.load(buf[2], sbuf[2]);
    }
    if constexpr (R > 3) {
      if (!more()) break;
      s.consume(buf[3], sbuf[3], b.xs, emit);
      s.load(buf[3], sbuf[3]);
    }
  }
  __syncthreads();
  if (kTaskLogDetail && threadIdx.x == 0) b.t_streamed = (uint32_t)now();
  if (threadIdx.x < 64) epi();  // wave 0 stores the results (see signal_w0)
  return true;
}

// ------------------------------------------------------------------ row maps

// a when sel is false, else b: by arithmetic on the addresses (a per-lane choice between two
// pointers written as a select is placed in scratch memory by the compiler)
__device__ __forceinline__ const uint8_t* pick2(bool sel, const void* a, const void* b) {
  const uintptr_t x = (uintptr_t)a;
  return (const uint8_t*)(x + (uintptr_t)sel * ((uintptr_t)b - x));
}

// Row maps give each task row's address; es = bytes per weight (2 bf16, 1 FP8), and for FP8
// rows `scale` reads the row's fp32 scale.
struct RmPlain {  // rows r0 + j of a [*, K] matrix
  const void* W;
  int K, r0;
  int es = 2;
  const float* S = nullptr;
  __device__ __forceinline__ const void* row(int j) const { return (const uint8_t*)W + (size_t)(r0 + j) * K * es; }
  __device__ __forceinline__ float scale(int j) const { return S[r0 + j]; }
  __device__ __forceinline__ int xoff(int) const { return 0; }
};

struct RmGateUp {  // unit u -> (gate row u, up row u)
  const void *Wg, *Wu;
  int K, u0;
  int es = 2;
  const float *Sg = nullptr, *Su = nullptr;
  __device__ __forceinline__ const void* row(int j) const {
    const uintptr_t g = (uintptr_t)Wg;
    const uintptr_t base = g + (uintptr_t)(j & 1) * ((uintptr_t)Wu - g);
    return (const uint8_t*)base + (size_t)(u0 + (j >> 1)) * K * es;
  }
  __device__ __forceinline__ float scale(int j) const { return ((j & 1) ? Su : Sg)[u0 + (j >> 1)]; }
  __device__ __forceinline__ int xoff(int) const { return 0; }
};

// GQA QKV: within KV group g, unit u = (slot, i): slot < r -> q head g*r+slot, slot == r ->
// k head g, slot == r+1 -> v head g; the unit's two rows are i and i + hd/2 of that head
// (the pair RoPE rotates together).
struct RmQKV {
  const void *wq, *wk, *wv;
  int g, r, hd, hh, K, u0;
  int es = 2;
  const float *sq = nullptr, *sk = nullptr, *sv = nullptr;
  // the matrix (0 q, 1 k, 2 v) and row of task row j
  __device__ __forceinline__ void where(int j, int& m, int& row) const {
    const int u = u0 + (j >> 1);
    const int slot = u / hh, i = u - slot * hh;
    const int rr = i + (j & 1) * hh;
    m = slot < r ? 0 : slot - r + 1;
    row = slot < r ? (g * r + slot) * hd + rr : g * hd + rr;
  }
  // (the matrix is picked by arithmetic on the addresses, not by indexing a pointer table,
  // which the compiler would place in scratch memory)
  static __device__ __forceinline__ uintptr_t pick(int m, const void* a, const void* b, const void* c) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b, z = (uintptr_t)c;
    return x + (uintptr_t)(m >= 1) * (y - x) + (uintptr_t)(m >= 2) * (z - y);
  }
  __device__ __forceinline__ const void* row(int j) const {
    int m, rw;
    where(j, m, rw);
    return (const uint8_t*)pick(m, wq, wk, wv) + (size_t)rw * K * es;
  }
  __device__ __forceinline__ float scale(int j) const {
    int m, rw;
    where(j, m, rw);
    return ((const float*)pick(m, sq, sk, sv))[rw];
  }
  __device__ __forceinline__ int xoff(int) const { return 0; }
};

// ------------------------------------------------------------------ GQA tasks


// With KV (a5 > 0 rows): the streaming waves also put cached K/V rows [a4, a4 + a5) of KV
// group a3 -- the attention split this workgroup runs next -- into LDS, behind their row
// prefetch. Every streaming wave issues exactly kKvStageDma 1-KB chunks (indices past the
// end repeat the last chunk; lanes past a region's end re-read its last 16 bytes), so the
// number of loads in flight is the same on every path through the stream loop.
// LDS DMA of the cached K and V rows [p0, p0 + rows) of KV group g of a layer: K rows to
// xs + kv_stage_k_off(hidden), V rows to scr + kv_stage_v_off(hd), as 1-KB chunks. Called by
// waves 1..7 (slot = wave - 1); each issues kKvStageDma chunks (slots past the last chunk
// re-load it), which covers up to 7 * kKvStageDma chunks of K and V together.
__device__ __forceinline__ void kv_stage_dma(const EngineArgs& A, Blk& b, int layer, int g, int p0, int rows, int slot) {
  const int lane = threadIdx.x & 63, hd = A.hd;
  const int hw = hd / 2, nfl = rows * hw, nch = (nfl + 255) / 256;
  if (rows <= 0) return;
  const size_t n1 = (size_t)A.kv_len + 1;
  const float* ks = reinterpret_cast<const float*>(A.kv + (((size_t)layer * 2 + 0) * A.nkv + g) * n1 * hd) + (size_t)p0 * hw;
  const float* vs = reinterpret_cast<const float*>(A.kv + (((size_t)layer * 2 + 1) * A.nkv + g) * n1 * hd) + (size_t)p0 * hw;
  float* kd = b.xs + kv_stage_k_off(A.hidden, A.wfmt ? 2 * kChunkCols : kChunkCols);
  float* vd = b.scr + kv_stage_v_off(hd);
#pragma unroll
  for (int k = 0; k < kKvStageDma; ++k) {
    int c = slot + (kWaves - 1) * k;
    c = c < 2 * nch ? c : 2 * nch - 1;
    const bool isv = c >= nch;
    const int cc = isv ? c - nch : c;
    int f = cc * 256 + lane * 4;
    f = f < nfl ? f : nfl - 4;
    __builtin_amdgcn_global_load_lds((gvp)((isv ? vs : ks) + f), (lvp)((isv ? vd : kd) + cc * 256), 16, 0, 0);
  }
}

template <bool KV, int ES>
__device__ __forceinline__ bool task_qkv(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int K = A.hidden, hd = A.hd, hh = hd / 2, r = A.nq / A.nkv, g = t.a0;
  const RmQKV rm{wp<uint8_t>(A, L.w[LW_WQ]), wp<uint8_t>(A, L.w[LW_WK]), wp<uint8_t>(A, L.w[LW_WV]), g, r, hd, hh, K, t.u0,
                 ES, wscale<ES>(A, L.w[LW_WQ]), wscale<ES>(A, L.w[LW_WK]), wscale<ES>(A, L.w[LW_WV])};
  const int xin = L.act[LA_X_IN];
  auto issue = [&] {
    if constexpr (KV) {
      const int wave = wave_id();
      if (wave == 0) return;  // wave 0 stages the input vector: no loads ahead of it
      const int p0 = split_pos(b.n, t.a4, t.a5), p1 = split_pos(b.n, t.a4 + 1, t.a5);
      kv_stage_dma(A, b, t.layer, t.a3, p0, (p1 < b.n ? p1 : b.n) - p0, wave - 1);
    }
  };
  return run_gemv<kRingQKV, false, ES>(
      A, b, t, rm, 2 * (t.u1 - t.u0), K, 1, true,
      stage_vec(xin, b.x, K, padc<ES>(K), wp<uint16_t>(A, L.w[LW_ATTN_NORM]), A.eps),
      [&] {
        const int n = b.n;
        const size_t lay = (size_t)2 * A.nkv * (A.kv_len + 1) * hd;  // cache elements per layer
        const rsrc_t kvr = make_rsrc(A.kv + (size_t)t.layer * lay, (uint32_t)(lay * 2));
        for (int i = threadIdx.x; i < t.u1 - t.u0; i += 64) {
          const int u = t.u0 + i, slot = u / hh, k = u - slot * hh;
          float a = b.ys[2 * i], c = b.ys[2 * i + 1];
          if (slot <= r) {  // RoPE on q and k
            const float cs = b.rope[k], sn = b.rope[A.rope_half + k];
            const float a2 = a * cs - c * sn;
            c = c * cs + a * sn;
            a = a2;
          }
          if (slot < r) {
            const uint32_t q = (uint32_t)(L.act[LA_Q] + (g * r + slot) * hd);
            cst(b.act, (q + k) * 4u, a);
            cst(b.act, (q + k + hh) * 4u, c);
          } else {
            const int sel = slot - r;  // 0: k, 1: v
            const uint32_t kn = (uint32_t)(L.act[LA_KVNEW] + (sel * A.nkv + g) * hd);
            cst(b.act, (kn + k) * 4u, a);
            cst(b.act, (kn + k + hh) * 4u, c);
            const uint32_t row = (uint32_t)(((size_t)(sel * A.nkv + g) * (A.kv_len + 1) + n) * hd);
            cst16(kvr, (row + k) * 2u, f2bf(a));
            cst16(kvr, (row + k + hh) * 2u, f2bf(c));
          }
        }
      },
      0, NoPre{}, issue);
}

// Merge S split partials (m, l, acc[hd]) of H heads into xs[h*hd + d] =
// sum_s e^(m_s-M) acc_s[d] / sum_s e^(m_s-M) l_s (base-2 exponents), zero-padding xs up to
// padK: the staging step of the per-group O-projection (a StageVec-like step: `early` is wave
// 0's LDS DMA of all S*H partials the moment the wait succeeds, when they fit one wave's
// outstanding loads; otherwise every wave copies a part in `finish`). The merge then runs from
// LDS. With o_off >= 0 wave 0 also stores the merged vector there.
struct StageMerge {
  int parts_off, S, H, hd, padK, o_off;
  __device__ __forceinline__ int n() const { return S * H * (hd + 4); }
  __device__ __forceinline__ void before(Blk&) const {}
  __device__ __forceinline__ void early(Blk& b) const {  // wave 0
    if (n() <= kEarlyDmaFloats) dma_to_lds(b.scr, b.actp + parts_off, n());
  }
  __device__ __forceinline__ void finish(Blk& b) const;
};

__device__ __forceinline__ void StageMerge::finish(Blk& b) const {
  const int ps = hd + 4;                    // m, l, 2 pad, acc[hd]
  const int n = S * H * ps;
  float* P = b.scr;                         // [S][H][ps]
  float* w = P + ((n + 255) & ~255);        // [S][H] merge weights
  b.norm = 1.f;
  if (n > kEarlyDmaFloats) dma_to_lds_all(P, b.actp + parts_off, n);
  else if (threadIdx.x < 64) __builtin_amdgcn_s_waitcnt(kVmcnt0);  // wave 0's early copy
  for (int i = H * hd + (int)threadIdx.x; i < padK; i += kThreads) b.xs[i] = 0.f;
  if (kTaskLogDetail && threadIdx.x == 0) b.t_sub[0] = (uint32_t)now();
  __syncthreads();
  if (kTaskLogDetail && threadIdx.x == 0) b.t_sub[1] = (uint32_t)now();
  // merge weights w[s][h] = 2^(m_s - M) / sum_s 2^(m_s - M) l_s: wave h (h < 8) owns heads
  // h, h + 8, ...; lanes run over the splits (an empty split has m = -inf and weight 0)
  for (int h = wave_id(); h < H; h += kWaves) {
    const int lane = threadIdx.x & 63;
    float M = -INFINITY;
    for (int sp = lane; sp < S; sp += 64) M = fmaxf(M, P[(sp * H + h) * ps]);
    M = wave_max(M);
    float den = 0.f;
    for (int sp = lane; sp < S; sp += 64) den = fmaf(ex2(P[(sp * H + h) * ps] - M), P[(sp * H + h) * ps + 1], den);
    const float inv = 1.0f / wave_sum(den);
    for (int sp = lane; sp < S; sp += 64) w[sp * H + h] = ex2(P[(sp * H + h) * ps] - M) * inv;
  }
  __syncthreads();
  if (kTaskLogDetail && threadIdx.x == 0) b.t_sub[2] = (uint32_t)now();
  // the weighted sums, eight independent accumulators per output
  for (int i = threadIdx.x; i < H * hd; i += kThreads) {
    const int h = i / hd, d = i - h * hd;
    const float* pp = P + h * ps + 4 + d;
    const float* ww = w + h;
    const int st = H * ps;
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = 0.f;
    int sp = 0;
    for (; sp + 8 <= S; sp += 8) {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = fmaf(ww[(sp + k) * H], pp[(sp + k) * st], v[k]);
    }
    for (; sp < S; ++sp) v[0] = fmaf(ww[sp * H], pp[sp * st], v[0]);
    b.xs[i] = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
  }
  __syncthreads();
  if (o_off >= 0 && threadIdx.x < 64)
    for (int i = threadIdx.x * 4; i < H * hd; i += 256) cst4(b.act, (uint32_t)(o_off + i) * 4u, *(const f4*)(b.xs + i));
}

// Split-K attention of one KV group over positions [u0, u1): the group's R query heads share
// every K/V load. A group of LPP = hd/8 lanes holds one position's row (8 dims per lane);
// one wave instruction covers 64/LPP consecutive positions. Online softmax in base 2 per
// head; partials are merged across the lane groups of a wave (cross-lane exchanges), then
// across waves (LDS); the O-projection tasks merge the splits. The cached positions stream
// through two register blocks with one kind of load and no divergent branch, so the
// compiler's wait for a block does not also wait for the other block in flight; the first
// two blocks are loaded before the dependency wait. The new position (slot kv_len, written
// by this step's QKV tasks) is folded in after the loop, read with agent-coherent loads.
template <int R, int LPP>
__device__ __forceinline__ bool task_attn(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  constexpr int GPW = 64 / LPP, NP = 3, PER_BLK = NP * GPW;
  const LayerDesc& L = A.layers[t.layer];
  const int hd = LPP * 8, r = A.nq / A.nkv, g = t.a0, n = b.n, n1 = A.kv_len + 1;
  const int wave = wave_id(), lane = threadIdx.x & 63, grp = lane / LPP, sub = lane - grp * LPP;
  const int p0 = split_pos(n, t.a1, t.a2), np = split_pos(n, t.a1 + 1, t.a2) - p0;
  const int q0 = p0 + wave_start(np, wave), q1 = p0 + wave_start(np, wave + 1);
  const int qc = q1 < n ? q1 : n;  // cached positions [q0, qc)
  const uint16_t* Kb = A.kv + (((size_t)t.layer * 2 + 0) * A.nkv + g) * (size_t)n1 * hd;
  const uint16_t* Vb = A.kv + (((size_t)t.layer * 2 + 1) * A.nkv + g) * (size_t)n1 * hd;
  const int nblk = (qc > q0) ? (qc - q0 + PER_BLK - 1) / PER_BLK : 0;
  // buffer loads bounded at row qc: rows past the wave's cached range read as zero (and are
  // masked), so a block needs one lane offset and a uniform block offset, nothing clamped
  const rsrc_t kr = make_rsrc(Kb, (uint32_t)(qc * hd * 2)), vr = make_rsrc(Vb, (uint32_t)(qc * hd * 2));
  const uint32_t lo = (uint32_t)(((q0 + grp) * hd + sub * 8) * 2);
  u4 ka[NP], va[NP], kb[NP], vb[NP];
  auto load = [&](int blk, u4(&kk)[NP], u4(&vv)[NP]) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int so = (blk * NP + i) * GPW * hd * 2;
      kk[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, lo, so, kNT);
      vv[i] = __builtin_amdgcn_raw_buffer_load_b128(vr, lo, so, kNT);
    }
  };
  load(0, ka, va);
  load(1, kb, vb);
  if (!wait_deps(A, b, t)) return false;

  // the group's queries, fetched by wave 0 (no loads in flight) into LDS and scaled there by
  // softmax scale * log2(e); the blocks read them from LDS (no registers held across the loop)
  if (threadIdx.x < 64) {
    dma_to_lds(b.ys, b.actp + L.act[LA_Q] + g * r * hd, r * hd);
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < r * hd; i += kThreads) b.ys[i] *= A.attn_scale_log2;
  __syncthreads();
  float m[R], l[R], acc[R][8];
#pragma unroll
  for (int h = 0; h < R; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[h][d] = 0.f;
  }
  // fold one block in: lane group grp's row i is position base + i GPW + grp, part of the
  // wave's work when it lies in [lo, hi). Heads past r repeat head r - 1 and are never stored.
  auto step = [&](int base, int lo, int hi, const u4(&kk)[NP], const u4(&vv)[NP]) {
    float s[R][NP];
    int qo = sub * 8;
    asm volatile("" : "+v"(qo));  // re-read q per block: keeps the reads from being hoisted into registers
#pragma unroll
    for (int h = 0; h < R; ++h) {
      const float* qh = b.ys + (h < r ? h : r - 1) * hd + qo;
      const f4 qa = *(const f4*)qh, qb = *(const f4*)(qh + 4);
      const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const u4 kw = kk[i];
        const float kf[8] = {bf_lo(kw.x), bf_hi(kw.x), bf_lo(kw.y), bf_hi(kw.y),
                             bf_lo(kw.z), bf_hi(kw.z), bf_lo(kw.w), bf_hi(kw.w)};
        float p = 0.f;
#pragma unroll
        for (int d = 0; d < 8; ++d) p = fmaf(qv[d], kf[d], p);
        s[h][i] = p;
      }
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int pos = base + i * GPW + grp;
      const bool valid = pos >= lo && pos < hi;
#pragma unroll
      for (int h = 0; h < R; ++h) {
        const float p = group_sum<LPP>(s[h][i]);
        s[h][i] = valid ? p : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < R; ++h) {
      float mb = s[h][0];
#pragma unroll
      for (int i = 1; i < NP; ++i) mb = fmaxf(mb, s[h][i]);
      const float mn = fmaxf(m[h], mb);
      const float mr = (mn == -INFINITY) ? 0.f : mn;  // nothing seen yet: every factor is 0
      const float alpha = ex2(m[h] - mr);
      l[h] *= alpha;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[h][d] *= alpha;
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const float p = ex2(s[h][i] - mr);
        l[h] += p;
        const u4 vw = vv[i];
        acc[h][0] = fmaf(p, bf_lo(vw.x), acc[h][0]);
        acc[h][1] = fmaf(p, bf_hi(vw.x), acc[h][1]);
        acc[h][2] = fmaf(p, bf_lo(vw.y), acc[h][2]);
        acc[h][3] = fmaf(p, bf_hi(vw.y), acc[h][3]);
        acc[h][4] = fmaf(p, bf_lo(vw.z), acc[h][4]);
        acc[h][5] = fmaf(p, bf_hi(vw.z), acc[h][5]);
        acc[h][6] = fmaf(p, bf_lo(vw.w), acc[h][6]);
        acc[h][7] = fmaf(p, bf_hi(vw.w), acc[h][7]);
      }
      m[h] = mn;
    }
  };
  // the loads are unconditional (blocks past the end read zeros without touching memory) and
  // the scheduler may not move one block's work across the other's loads, so the compiler's
  // wait before each block leaves the next block in flight
  for (int blk = 0; blk < nblk; blk += 2) {
    step(q0 + blk * PER_BLK, q0, qc, ka, va);
    load(blk + 2, ka, va);
    __builtin_amdgcn_sched_barrier(0);
    step(q0 + (blk + 1) * PER_BLK, q0, qc, kb, vb);
    load(blk + 3, kb, vb);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (q0 <= n && n < q1) {
    // the new position: every lane group reads row n (agent scope: other workgroups wrote it
    // in this step), lane group 0 of row 0 folds it in
    const rsrc_t kn = make_rsrc(Kb, (uint32_t)(n1 * hd * 2)), vn = make_rsrc(Vb, (uint32_t)(n1 * hd * 2));
    const uint32_t off = (uint32_t)(n * hd + sub * 8) * 2u;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      ka[i] = __builtin_amdgcn_raw_buffer_load_b128(kn, off, 0, kCoh);
      va[i] = __builtin_amdgcn_raw_buffer_load_b128(vn, off, 0, kCoh);
    }
    step(n, n, n + 1, ka, va);
  }
  const uint32_t t_mid = kTaskLogDetail ? (uint32_t)now() : 0u;
  // merge the wave's lane groups (the same dims of different positions) with cross-lane
  // exchanges: partials (m, l, acc) of lanes L and L ^ X combine as
  // M = max, l = l e^(m - M) + l' e^(m' - M), acc likewise (base 2); afterwards every lane
  // group holds the wave's partial
#pragma unroll 1
  for (int X = LPP; X < 64; X <<= 1) {
#pragma unroll
    for (int h = 0; h < R; ++h) {
      if (h >= r) continue;
      const float om = __shfl_xor(m[h], X, 64), ol = __shfl_xor(l[h], X, 64);
      const float M = fmaxf(m[h], om);
      const float ca = (m[h] == -INFINITY) ? 0.f : exp2f(m[h] - M);
      const float cb = (om == -INFINITY) ? 0.f : exp2f(om - M);
      l[h] = l[h] * ca + ol * cb;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[h][d] = acc[h][d] * ca + __shfl_xor(acc[h][d], X, 64) * cb;
      m[h] = M;
    }
  }
  // lane group 0 of each wave writes the wave's partial: slot = wave, [slot][R][ps] with
  // ps = hd + 4 (m, l, 2 pad, acc[hd]); the compile-time slot stride keeps the merge's LDS
  // addresses in instruction offsets
  constexpr int NS = kWaves, ps = hd + 4, SS = R * ps;
  if (grp == 0) {
    float* gp = b.scr + wave * SS;
#pragma unroll
    for (int h = 0; h < R; ++h) {
      if (h >= r) continue;
      if (sub == 0) {
        gp[h * ps] = m[h];
        gp[h * ps + 1] = l[h];
      }
#pragma unroll
      for (int d = 0; d < 8; ++d) gp[h * ps + 4 + sub * 8 + d] = acc[h][d];
    }
  }
  __syncthreads();
  const uint32_t t_lanes = kTaskLogDetail ? (uint32_t)now() : 0u;
  // workgroup partial (M, den, sum of weighted acc) -> LDS (xs), then wave 0 stores it; each
  // thread recomputes its head's merge weights over the NS wave slots
#pragma unroll 1
  for (int i = threadIdx.x; i < r * hd; i += kThreads) {
    const int h = i / hd, d = i - h * hd;
    float M = -INFINITY;
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) M = fmaxf(M, b.scr[sl * SS + h * ps]);
    float v = 0.f, den = 0.f;
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
      const float ms = b.scr[sl * SS + h * ps];
      const float e = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
      v = fmaf(e, b.scr[sl * SS + h * ps + 4 + d], v);
      den = fmaf(e, b.scr[sl * SS + h * ps + 1], den);
    }
    b.xs[h * ps + 4 + d] = v;
    if (d == 0) {
      b.xs[h * ps] = M;
      b.xs[h * ps + 1] = den;
      b.xs[h * ps + 2] = 0.f;
      b.xs[h * ps + 3] = 0.f;
    }
  }
  const uint32_t gpart = (uint32_t)(t.a4 + t.a1 * r * ps);
  __syncthreads();
  const uint32_t t_merged = kTaskLogDetail ? (uint32_t)now() : 0u;
  if (threadIdx.x < 64)
    for (int i = threadIdx.x * 4; i < r * ps; i += 256) cst4(b.act, (gpart + i) * 4u, *(const f4*)(b.xs + i));
  if (kTaskLogDetail && threadIdx.x == 0) {
    A.log[t.id].t_aux[0] = t_lanes;
    A.log[t.id].t_aux[1] = t_merged;
    A.log[t.id].t_mid = t_mid;
  }
  return true;
}

template <int R>
__device__ __forceinline__ bool task_attn_hd(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  switch (A.hd) {
    case 32: return task_attn<R, 4>(A, b, t);
    case 64: return task_attn<R, 8>(A, b, t);
    case 128: return task_attn<R, 16>(A, b, t);
    default: return task_attn<R, 32>(A, b, t);
  }
}

template <int ES>
__device__ __forceinline__ bool task_oproj(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int K = (A.arch == 0) ? A.nq * A.hd : A.nq * A.dv;
  const RmPlain rm{wp<uint8_t>(A, L.w[LW_WO]), K, t.u0, ES, wscale<ES>(A, L.w[LW_WO])};
  const int xin = L.act[LA_X_IN];
  return run_gemv<2, false, ES>(
      A, b, t, rm, t.u1 - t.u0, K, 1, true,
      stage_vec(L.act[LA_ATTN], nullptr, K, padc<ES>(K), nullptr, 0.f, false, A.arch != 0),
      [&] {
        for (int i = threadIdx.x; i < t.u1 - t.u0; i += 64) {
          const int rr = t.u0 + i;
          const float res = xin >= 0 ? cld(b.act, (uint32_t)(xin + rr) * 4u) : bf16f(b.x[rr]);
          cst(b.act, (uint32_t)(L.act[LA_H] + rr) * 4u, res + b.ys[i]);
        }
      });
}

struct RmCols {  // rows r0 + j of a [*, ld] matrix, columns starting at c0
  const void* W;
  int ld, r0, c0;
  int es = 2;
  const float* S = nullptr;
  __device__ __forceinline__ const void* row(int j) const { return (const uint8_t*)W + ((size_t)(r0 + j) * ld + c0) * es; }
  __device__ __forceinline__ float scale(int j) const { return S[r0 + j]; }
  __device__ __forceinline__ int xoff(int) const { return 0; }
};

// Rows [u0, u1) of W_o times the merged attention output of KV group g (its r*hd columns):
// one term of h = x + sum_g W_o[:, g] o_g. The group's split partials are merged while
// staging; the first task of the group also stores the merged o_g (the attention output).
template <int ES>
__device__ __forceinline__ bool task_oproj_g(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int r = A.nq / A.nkv, hd = A.hd, g = t.a0, K = r * hd;
  const RmCols rm{wp<uint8_t>(A, L.w[LW_WO]), A.nq * hd, t.u0, g * K, ES, wscale<ES>(A, L.w[LW_WO])};
  return run_gemv<kRingOproj, false, ES>(
      A, b, t, rm, t.u1 - t.u0, K, 1, true,
      StageMerge{t.a4, t.a2, r, hd, padc<ES>(K), t.u0 == 0 ? L.act[LA_ATTN] + g * K : -1},
      [&] {
        float* h = b.actp + L.act[LA_H] + t.u0;
        for (int i = threadIdx.x; i < t.u1 - t.u0; i += 64)
          __hip_atomic_fetch_add(h + i, b.ys[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      });
}

// Layer 0: h = x (widened), the accumulator the per-group O-projections add into.
__device__ __forceinline__ bool task_hinit(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  for (int i = threadIdx.x; i < t.u1 - t.u0; i += kThreads) cst(b.act, (uint32_t)(t.a0 + t.u0 + i) * 4u, bf16f(b.x[t.u0 + i]));
  return true;
}


template <int ES>
__device__ __forceinline__ bool task_gateup(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int K = A.hidden;
  const RmGateUp rm{wp<uint8_t>(A, L.w[LW_GATE]), wp<uint8_t>(A, L.w[LW_UP]), K, t.u0, ES, wscale<ES>(A, L.w[LW_GATE]),
                    wscale<ES>(A, L.w[LW_UP])};
  return run_gemv<kRingFfn, false, ES>(
      A, b, t, rm, 2 * (t.u1 - t.u0), K, 1, true,
      stage_vec(L.act[LA_H], nullptr, K, padc<ES>(K), wp<uint16_t>(A, L.w[LW_FFN_NORM]), A.eps, false, A.arch == 0),
      [&] {
        for (int i = threadIdx.x; i < t.u1 - t.u0; i += 64)
          cst(b.act, (uint32_t)(L.act[LA_ACT] + t.u0 + i) * 4u, silu(b.ys[2 * i]) * b.ys[2 * i + 1]);
      });
}

template <bool FLAT, int ES>
__device__ __forceinline__ bool task_down(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int K = A.ffn;
  const RmPlain rm{wp<uint8_t>(A, L.w[LW_DOWN]), K, t.u0, ES, wscale<ES>(A, L.w[LW_DOWN])};
  return run_gemv<FLAT ? kRingFfn : 2, FLAT, ES>(
      A, b, t, rm, t.u1 - t.u0, K, 1, true,
      stage_vec(L.act[LA_ACT], nullptr, K, padc<ES>(K), nullptr, 0.f),
      [&] {
        for (int i = threadIdx.x; i < t.u1 - t.u0; i += 64) {
          const int rr = t.u0 + i;
          const float y = b.ys[i];
          const float hr = A.arch == 0 ? cld_coh(b.act, (uint32_t)(L.act[LA_H] + rr) * 4u) : cld(b.act, (uint32_t)(L.act[LA_H] + rr) * 4u);
          const float xo = hr + y;
          cst(b.act, (uint32_t)(L.act[LA_FFN_OUT] + rr) * 4u, y);
          if (t.a1 >= 0) cst(b.act, (uint32_t)(t.a1 + rr) * 4u, xo);  // next layer's h starts at x
          cst(b.act, (uint32_t)(L.act[LA_X_OUT] + rr) * 4u, xo);
          if (t.a0) A.out[rr] = xo;
        }
      });
}

// Wave-wide (value, index) maximum, ties to the lower index; every lane ends with the result.
__device__ __forceinline__ void best_pair(float& v, int& i) {
#pragma unroll
  for (int x = 1; x < 64; x <<= 1) {
    const float ov = __shfl_xor(v, x, 64);
    const int oi = __shfl_xor(i, x, 64);
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
  }
}

// Selection keys: one unsigned 64-bit key per (score, index) whose order is the order of the
// scores, the lower index first among equal scores. High word: the fp32 bits mapped to an
// unsigned order (negative values bit-inverted, positive values with the sign bit set; -0
// taken as +0, as the float compare does); low word: the inverted index. NaN gets key 0,
// which is also the mark of an empty or retired slot, so a maximum is one 64-bit compare
// with no tie branch.
__device__ __forceinline__ uint64_t sel_key(float v, int i) {
  const uint32_t u = __float_as_uint(v) == 0x80000000u ? 0u : __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  const uint32_t m = v == v ? 0xffffffffu : 0u;
  return ((uint64_t)(o & m) << 32) | ((uint32_t)~i & m);
}
__device__ __forceinline__ int sel_index(uint64_t k) { return (int)~(uint32_t)k; }
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t k) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)k, CTRL, 0xf, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(k >> 32), CTRL, 0xf, 0xf, true);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
// Largest key of the wave, returned wave-uniform: DPP exchanges within each 16-lane row (the
// lane pairings of group_sum), then the four row maxima.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
  k = umax64(k, dpp64<kQuadSwap1>(k));
  k = umax64(k, dpp64<kQuadSwap2>(k));
  k = umax64(k, dpp64<kRowHalfMirror>(k));
  k = umax64(k, dpp64<kRowMirror>(k));
  uint64_t r[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    r[q] = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), 16 * q) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k, 16 * q);
  return umax64(umax64(r[0], r[1]), umax64(r[2], r[3]));
}

template <bool GREEDY, int ES>
__device__ __forceinline__ bool task_lmhead(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const int K = A.hidden;
  const RmPlain rm{wp<uint8_t>(A, A.w_lm_head), K, t.u0, ES, wscale<ES>(A, A.w_lm_head)};
  return run_gemv<2, false, ES>(
      A, b, t, rm, t.u1 - t.u0, K, 1, true,
      stage_vec(A.x_final, nullptr, K, padc<ES>(K), wp<uint16_t>(A, A.w_final_norm), A.eps),
      [&] {
        for (int i = threadIdx.x; i < t.u1 - t.u0; i += 64) A.out[t.u0 + i] = b.ys[i];
        if constexpr (GREEDY) {  // this task's largest logit (lowest index among equals) -> slot a0
          float bv = -INFINITY;
          int bi = 0x7fffffff;
          for (int i = threadIdx.x; i < t.u1 - t.u0; i += 64)
            if (b.ys[i] > bv) { bv = b.ys[i]; bi = t.u0 + i; }
          best_pair(bv, bi);
          if (threadIdx.x == 0) {
            cst(b.act, (uint32_t)(t.a1 + 2 * t.a0) * 4u, bv);
            cst(b.act, (uint32_t)(t.a1 + 2 * t.a0 + 1) * 4u, __int_as_float(bi));
          }
        }
      });
}

// Greedy choice of the next token: the largest of the LM-head tasks' best logits (the lowest
// index among equal values), written to the step state as the next step's token.
__device__ __forceinline__ bool task_argmax(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  if (!wait_deps(A, b, t)) return false;
  if (threadIdx.x < 64) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int i = threadIdx.x; i < t.a0; i += 64) {
      const float v = cld(b.act, (uint32_t)(t.a1 + 2 * i) * 4u);
      const int k = __float_as_int(cld(b.act, (uint32_t)(t.a1 + 2 * i + 1) * 4u));
      if (v > bv || (v == bv && k < bi)) { bv = v; bi = k; }
    }
    best_pair(bv, bi);
    if (threadIdx.x == 0) st_agent(reinterpret_cast<uint32_t*>(A.state) + 1, (uint32_t)(bi == 0x7fffffff ? 0 : bi));
  }
  return true;
}


// ------------------------------------------------------------------ MLA tasks
//
// Latent attention in the absorbed form (TileRT audit page, TokenSpeed MLA paragraph: the
// query heads are folded into the rows of one contraction over the shared latent cache):
//   q_abs[h] = W_UK[h]^T q_nope[h];  s[h][j] = (q_abs[h] . c_j + q_rope[h] . kpe_j) / sqrt(dn + dr)
//   o_lat[h] = sum_j softmax(s[h])_j c_j;  o[h] = W_UV[h] o_lat[h]
// At 16 heads x (kl + dr) the attention does ~30 flop per latent byte, so it runs on the
// matrix cores: bf16 MFMA 16x16x32, with the fp32 operands that are not bf16 (the scaled
// query and the probabilities) split into bf16 hi + lo parts so that the products keep
// about 16 mantissa bits.

typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f4 mfma_bf16(u4 a, u4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8_t, a), __builtin_bit_cast(bf8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t bf_pair(uint16_t lo, uint16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

// fp32 x as a bf16 pair hi + lo (hi = x rounded, lo = the rest rounded): about 16 mantissa
// bits of x, enough for operands whose other side is exact bf16
__device__ __forceinline__ void split_bf16(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = pk_bf16(x0, x1);
  lo = pk_bf16(x0 - bf_lo(hi), x1 - bf_hi(hi));
}
// eight values (a, then b) times s as the hi and lo halves of one bf16 MFMA operand
__device__ __forceinline__ void split_bf16x8(f4 a, f4 b, float s, u4& hi, u4& lo) {
  uint32_t h[4], l[4];
  split_bf16(a.x * s, a.y * s, h[0], l[0]);
  split_bf16(a.z * s, a.w * s, h[1], l[1]);
  split_bf16(b.x * s, b.y * s, h[2], l[2]);
  split_bf16(b.z * s, b.w * s, h[3], l[3]);
  hi = u4{h[0], h[1], h[2], h[3]};
  lo = u4{l[0], l[1], l[2], l[3]};
}

// GQA attention of one KV group over a split whose K/V rows are in LDS -- the cached rows
// copied by the workgroup's QKV task, the new position (when the split holds it) copied in
// by wave 0 after the dependency wait -- on the matrix cores. Each wave takes 16-position
// tiles of the split in turn and keeps a flash-style running softmax per head:
//   scores S = K q~^T (bf16 MFMA 16x16x32): rows = the tile's positions, columns = the group's
//     r <= 4 query heads (the rest zero), q~ = q * scale * log2(e) as hi + lo bf16 operands,
//     K exact;
//   m = running max, P = 2^(S - m), l = running sum, O rescaled by 2^(m_old - m);
//   O += P V (bf16 MFMA 16x16x16): the score tile's registers are, element for element, the
//     A operand (rows = heads, k = positions), P as hi + lo parts; V gathered from its rows.
// The eight waves' (m, l, O) are then merged through LDS into the split partial
// (m, l, 0, 0, unnormalised o[hd]) per head -- the record the lane-group path writes -- which
// wave 0 alone stores (the task signals like a GEMV). Positions past the split read its last
// row (finite values, probability 0).
typedef short s4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f4 mfma_bf16_k16(uint2 a, uint2 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4_t, a), __builtin_bit_cast(s4_t, b), c, 0, 0, 0);
}
// One 16-position tile of an attention split on the matrix cores, folded into the calling
// wave's running softmax state (m, l: lane's head hl; o: rows = heads 4 q4 + i, column
// 16 ct + hl). K and V hold the tile's rows from row 16 tile on (rows of HD bf16); rows at or
// past nv are not part of the split (read as row nv - 1, probability 0).
template <int HD>
__device__ __forceinline__ void attn_tile(const uint16_t* Ks, const uint16_t* Vs, int tile, int nv, int r, int hl, int q4,
                                          const u4 (&qh)[HD / 32], const u4 (&ql)[HD / 32], float& m, float& l,
                                          f4 (&o)[HD / 16]) {
  constexpr int NKS = HD / 32, NCT = HD / 16;
  int pos = 16 * tile + hl;
  pos = pos < nv ? pos : nv - 1;
  const uint16_t* arow = Ks + (size_t)pos * HD + 8 * q4;
  f4 dh = f4{0.f, 0.f, 0.f, 0.f}, dl = dh;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const u4 a = *reinterpret_cast<const u4*>(arow + 32 * ks);
    dh = mfma_bf16(a, qh[ks], dh);
    dl = mfma_bf16(a, ql[ks], dl);
  }
  const f4 d = dh + dl;  // S[position 16 tile + 4 q4 + i][head hl]
  const int pq = 16 * tile + 4 * q4;
  float sv[4], mt = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sv[i] = (pq + i < nv && hl < r) ? d[i] : -INFINITY;
    mt = fmaxf(mt, sv[i]);
  }
  mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
  const float mn = fmaxf(m, mt);  // -inf only for heads past r
  const float al = (m == -INFINITY) ? 0.f : ex2(m - mn);
  float pv[4], ls = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pv[i] = (sv[i] == -INFINITY) ? 0.f : ex2(sv[i] - mn);
    ls += pv[i];
  }
  ls += __shfl_xor(ls, 16, 64);
  ls += __shfl_xor(ls, 32, 64);
  l = l * al + ls;
  m = mn;
  // rescale O rows (heads 0..3 live in lanes q4 = 0; lane i holds head i's factor)
  const int alb = __float_as_int(al);
  const f4 a4 = f4{__int_as_float(__builtin_amdgcn_readlane(alb, 0)), __int_as_float(__builtin_amdgcn_readlane(alb, 1)),
                   __int_as_float(__builtin_amdgcn_readlane(alb, 2)), __int_as_float(__builtin_amdgcn_readlane(alb, 3))};
  uint2 ph, plo;
  {
    uint32_t h0, h1, l0, l1;
    split_bf16(pv[0], pv[1], h0, l0);
    split_bf16(pv[2], pv[3], h1, l1);
    ph = uint2{h0, h1};
    plo = uint2{l0, l1};
  }
  const uint16_t* vrow = Vs + hl;
  int vp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) vp[i] = (pq + i < nv ? pq + i : nv - 1) * HD;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const uint16_t* vc = vrow + 16 * ct;
    const uint2 bv = uint2{bf_pair(vc[vp[0]], vc[vp[1]]), bf_pair(vc[vp[2]], vc[vp[3]])};
    o[ct] *= a4;
    o[ct] = mfma_bf16_k16(ph, bv, o[ct]);
    o[ct] = mfma_bf16_k16(plo, bv, o[ct]);
  }
}

// The eight waves' (m, l, O) -> LDS slots -> the split partial (m, l, 0, 0, unnormalised o) per
// head, which wave 0 stores.
template <int HD>
__device__ __forceinline__ void attn_finish(const EngineArgs& A, Blk& b, const TaskDesc& t, int r, int hl, int q4, float m,
                                            float l, const f4 (&o)[HD / 16]) {
  constexpr int NCT = HD / 16, ps = HD + 4, SS = 4 * ps;
  const int wave = wave_id();
  // this wave's (m, l, O) -> slot `wave`: [wave][head < 4][m, l, 0, 0, o[HD]]
  float* slot = b.scr + wave * SS;
  if (q4 == 0 && hl < r) {
    slot[hl * ps] = m;
    slot[hl * ps + 1] = l;
  }
  if (q4 == 0) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < r) slot[i * ps + 4 + 16 * ct + hl] = o[ct][i];
  }
  __syncthreads();
  // merge the waves: xs[h * ps] = (M, sum_w e_w l_w, 0, 0, sum_w e_w O_w), e_w = 2^(m_w - M)
  for (int i = threadIdx.x; i < r * HD; i += kThreads) {
    const int h = i / HD, d = i - h * HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, b.scr[w * SS + h * ps]);
    float v = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = b.scr[w * SS + h * ps];
      const float e = (mw == -INFINITY) ? 0.f : ex2(mw - M);
      v = fmaf(e, b.scr[w * SS + h * ps + 4 + d], v);
      den = fmaf(e, b.scr[w * SS + h * ps + 1], den);
    }
    b.xs[h * ps + 4 + d] = v;
    if (d == 0) *reinterpret_cast<f4*>(b.xs + h * ps) = f4{M, den, 0.f, 0.f};
  }
  __syncthreads();
  if (kTaskLogDetail && threadIdx.x == 0) A.log[t.id].t_mid = (uint32_t)now();
  if (threadIdx.x < 64) {  // wave 0 stores the partial (see signal_w0)
    const uint32_t gpart = (uint32_t)(t.a4 + t.a1 * r * ps);
    for (int i = threadIdx.x * 4; i < r * ps; i += 256) cst4(b.act, (gpart + i) * 4u, *(const f4*)(b.xs + i));
  }
}

template <int HD>
__device__ __forceinline__ bool task_attn_mfma(const EngineArgs& A, Blk& b, const TaskDesc& t, bool self_stage) {
  constexpr int NKS = HD / 32, NCT = HD / 16;
  const LayerDesc& L = A.layers[t.layer];
  const int r = A.nq / A.nkv, g = t.a0;
  const int p0 = split_pos(b.n, t.a1, t.a2), p1 = split_pos(b.n, t.a1 + 1, t.a2), np = p1 - p0;
  const int c = (p1 < b.n ? p1 : b.n) - p0;  // cached rows, staged in LDS; row c (if < np) is the new position
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));  // keeps lane-derived LDS addresses inside the task (not hoisted and spilled)
  const int wave = wave_id(), hl = lane & 15, q4 = lane >> 4;
  uint16_t* Ks = reinterpret_cast<uint16_t*>(b.xs + kv_stage_k_off(A.hidden, A.wfmt ? 2 * kChunkCols : kChunkCols));  // [np][HD]
  uint16_t* Vs = reinterpret_cast<uint16_t*>(b.scr + kv_stage_v_off(HD));       // [np][HD]
  // the cached rows were copied into LDS by the QKV task just before this one, or, in a launch
  // that does not run that task, are copied here; this wave's DMA has landed once vmcnt is 0,
  // and the barrier in the wait publishes it to the other waves
  if (self_stage && wave > 0) kv_stage_dma(A, b, t.layer, g, p0, c, wave - 1);
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  if (!wait_deps(A, b, t)) return false;
  // every wave loads q~ in B-operand order itself: lane L of k-step ks holds head L % 16,
  // dims 32 ks + 8 (L / 16) + e (zero past r)
  f4 qa[NKS], qb[NKS];
  const uint32_t qo = (uint32_t)(L.act[LA_Q] + (g * r + (hl < r ? hl : 0)) * HD + 8 * q4) * 4u;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    qa[ks] = cld4(b.act, qo + ks * 128u);
    qb[ks] = cld4(b.act, qo + ks * 128u + 16u);
  }
  if (wave == 0 && c < np && lane < HD / 8) {  // row c: the new position, written by this step's QKV tasks
    const size_t n1 = (size_t)A.kv_len + 1, off = (size_t)(p0 + c) * HD + lane * 8;
    const uint16_t* kb = A.kv + (((size_t)t.layer * 2 + 0) * A.nkv + g) * n1 * HD;
    const uint16_t* vb = A.kv + (((size_t)t.layer * 2 + 1) * A.nkv + g) * n1 * HD;
    __builtin_amdgcn_global_load_lds((gvp)(kb + off), (lvp)(Ks + (size_t)c * HD), 16, 0, kCoh);
    __builtin_amdgcn_global_load_lds((gvp)(vb + off), (lvp)(Vs + (size_t)c * HD), 16, 0, kCoh);
  }
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  if (kTaskLogDetail && threadIdx.x == 0) b.t_sub[0] = (uint32_t)now();
  u4 qh[NKS], ql[NKS];
  const float sc = (hl < r) ? A.attn_scale_log2 : 0.f;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) split_bf16x8(qa[ks], qb[ks], sc, qh[ks], ql[ks]);
  __syncthreads();
  float m = -INFINITY, l = 0.f;
  f4 o[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) o[ct] = f4{0.f, 0.f, 0.f, 0.f};
  const int ntile = (np + 15) >> 4;
  for (int tile = wave; tile < ntile; tile += kWaves) attn_tile<HD>(Ks, Vs, tile, np, r, hl, q4, qh, ql, m, l, o);
  if (kTaskLogDetail && threadIdx.x == 0) b.t_sub[1] = (uint32_t)now();
  attn_finish<HD>(A, b, t, r, hl, q4, m, l, o);
  return true;
}

// The scaled query q~ = [q_abs | q_rope] * softmax scale * log2(e), as the B operand of the
// score MFMA (k = latent dimension, n = head): lane L of k-step ks holds k = 32 ks + 8 (L/16)
// + 0..7 of head L % 16, first the bf16 hi parts (block 2 ks), then the lo parts (2 ks + 1).
__device__ __forceinline__ void qop_store(const Blk& b, int qop, int h, int k, float v) {
  const int ks = k >> 5, L = h + 16 * ((k & 31) >> 3), j = k & 7;
  const uint16_t hi = f2bf(v), lo = f2bf(v - bf16f(hi));
  const uint32_t i0 = (uint32_t)(((ks * 2) * 64 + L) * 8 + j);
  cst16(b.act, (uint32_t)qop * 4u + i0 * 2u, hi);
  cst16(b.act, (uint32_t)qop * 4u + (i0 + 512u) * 2u, lo);
}

struct RmMlaA {  // rows [0, ql) of W_DQ, then the rows of W_DKV (KR), then W_k (DI), W_w (HI)
  const void *wqa, *wkva;
  int K, ql, r0;
  int es = 2;
  const float *sqa = nullptr, *skva = nullptr;  // FP8: row scales
  const void *wik = nullptr, *wiw = nullptr;    // sparse indexer (bf16)
  int KR = 0, DI = 0;
  __device__ __forceinline__ const void* row(int j) const {
    const int r = r0 + j;
    const int s1 = r >= ql, s2 = r >= ql + KR, s3 = r >= ql + KR + DI;
    const int off = s1 * ql + s2 * KR + s3 * DI;
    return pick2(s2, pick2(s1, wqa, wkva), pick2(s3, wik, wiw)) + (size_t)(r - off) * K * es;
  }
  __device__ __forceinline__ float scale(int j) const {
    const int r = r0 + j;
    return r < ql ? sqa[r] : skva[r - ql];
  }
  __device__ __forceinline__ int xoff(int) const { return 0; }
};

// x^ = RMSNorm(x); [cq_raw | kv_a] = [W_DQ; W_DKV] x^
template <int ES, bool IDX>
__device__ __forceinline__ bool task_mla_a(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int K = A.hidden, ql = A.ql, KR = A.kl + A.dr, DI = IDX ? A.idx_d : 0;
  const RmMlaA rm{wp<uint8_t>(A, L.w[LW_WQA]), wp<uint8_t>(A, L.w[LW_WKVA]), K, ql, t.u0, ES, wscale<ES>(A, L.w[LW_WQA]),
                  wscale<ES>(A, L.w[LW_WKVA]), DI ? wp<uint8_t>(A, L.w[LW_IDXK]) : nullptr,
                  DI ? wp<uint8_t>(A, L.w[LW_IDXW]) : nullptr, KR, DI};
  return run_gemv<2, false, ES>(
      A, b, t, rm, t.u1 - t.u0, K, 1, true,
      stage_vec(L.act[LA_X_IN], b.x, K, padc<ES>(K), wp<uint16_t>(A, L.w[LW_ATTN_NORM]), A.eps),
      [&] {
        for (int i = threadIdx.x; i < t.u1 - t.u0; i += 64) {
          const int r = t.u0 + i;
          if (r < ql + KR) {
            const int off = r < ql ? L.act[LA_CQ] + r : L.act[LA_KVA] + (r - ql);
            cst(b.act, (uint32_t)off * 4u, b.ys[i]);
          } else if (IDX && r < ql + KR + DI) {
            // the new index key: traced, and appended to the cache (bf16) after the latent row
            const int k = r - ql - KR;
            cst(b.act, (uint32_t)(L.act[LA_IDXK] + k) * 4u, b.ys[i]);
            uint16_t* row = A.kv + ((size_t)t.layer * (A.kv_len + 1) + b.n) * A.kvrow + KR;
            const rsrc_t rr = make_rsrc(row, (uint32_t)DI * 2u);
            cst16(rr, (uint32_t)k * 2u, f2bf(b.ys[i]));
          } else if (IDX) {
            cst(b.act, (uint32_t)(L.act[LA_IDXW] + r - ql - KR - DI) * 4u, b.ys[i]);
          }
        }
      });
}

// W_UQ row pairs: unit (head h, i) is rows (i, i + dn/2) of the head's nope part for
// i < dn/2, else the RoPE pair (dn + k, dn + k + dr/2), k = i - dn/2.
struct RmMlaB {
  const uint8_t* W;
  int K, dn, dr, uh, u0;
  int es = 2;
  const float* S = nullptr;  // FP8: row scales
  __device__ __forceinline__ int rix(int j) const {  // the task row's row of W_UQ
    const int u = u0 + (j >> 1), h = u / uh, i = u - h * uh, hn = dn >> 1;
    const int rr = i < hn ? i + (j & 1) * hn : dn + (i - hn) + (j & 1) * (dr >> 1);
    return h * (dn + dr) + rr;
  }
  __device__ __forceinline__ const void* row(int j) const { return W + (size_t)rix(j) * K * es; }
  __device__ __forceinline__ float scale(int j) const { return S[rix(j)]; }
  __device__ __forceinline__ int xoff(int) const { return 0; }
};

// cq = RMSNorm(cq_raw); [q_nope | q_rope] = W_UQ cq, RoPE on q_rope
template <int ES>
__device__ __forceinline__ bool task_mla_b(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int K = A.ql, dn = A.dn, dr = A.dr, uh = dn / 2 + dr / 2;
  const RmMlaB rm{wp<uint8_t>(A, L.w[LW_WQB]), K, dn, dr, uh, t.u0, ES, wscale<ES>(A, L.w[LW_WQB])};
  return run_gemv<2, false, ES>(
      A, b, t, rm, 2 * (t.u1 - t.u0), K, 1, true,
      stage_vec(L.act[LA_CQ], nullptr, K, padc<ES>(K), wp<uint16_t>(A, L.w[LW_QNORM]), A.eps),
      [&] {
        for (int i = threadIdx.x; i < t.u1 - t.u0; i += 64) {
          const int u = t.u0 + i, h = u / uh, k = u - h * uh;
          const float a = b.ys[2 * i], c = b.ys[2 * i + 1];
          if (k < dn / 2) {
            cst(b.act, (uint32_t)(L.act[LA_QNOPE] + h * dn + k) * 4u, a);
            cst(b.act, (uint32_t)(L.act[LA_QNOPE] + h * dn + k + dn / 2) * 4u, c);
          } else {
            const int kk = k - dn / 2;
            const float cs = b.rope[kk], sn = b.rope[A.rope_half + kk];
            const float a2 = a * cs - c * sn, c2 = c * cs + a * sn;
            cst(b.act, (uint32_t)(L.act[LA_QROPE] + h * dr + kk) * 4u, a2);
            cst(b.act, (uint32_t)(L.act[LA_QROPE] + h * dr + kk + dr / 2) * 4u, c2);
            qop_store(b, L.act[LA_QOP], h, A.kl + kk, a2 * A.attn_scale_log2);
            qop_store(b, L.act[LA_QOP], h, A.kl + kk + dr / 2, c2 * A.attn_scale_log2);
          }
        }
      });
}

// The new latent row: c = RMSNorm(kv_a[:kl]), kpe = RoPE(kv_a[kl:]), appended to the cache at
// position kv_len as bf16. Also clears o (the W_UV tasks accumulate into it).
__device__ __forceinline__ bool task_mla_kvapp(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int kl = A.kl, dr = A.dr, KR = kl + dr, n = b.n;
  if (!wait_deps(A, b, t)) return false;
  stage_now(b, stage_vec(L.act[LA_KVA], nullptr, kl, pad512(kl), wp<uint16_t>(A, L.w[LW_KVNORM]), A.eps, true));
  const rsrc_t rowr = make_rsrc(A.kv + ((size_t)t.layer * (A.kv_len + 1) + n) * A.kvrow, (uint32_t)KR * 2u);
  for (int i = threadIdx.x; i < kl; i += kThreads) {
    const float v = b.xs[i];
    cst(b.act, (uint32_t)(L.act[LA_KVNEW] + i) * 4u, v);
    cst16(rowr, (uint32_t)i * 2u, f2bf(v));
  }
  for (int k = threadIdx.x; k < dr / 2; k += kThreads) {
    const float a = cld(b.act, (uint32_t)(L.act[LA_KVA] + kl + k) * 4u);
    const float c = cld(b.act, (uint32_t)(L.act[LA_KVA] + kl + k + dr / 2) * 4u);
    const float cs = b.rope[k], sn = b.rope[A.rope_half + k];
    const float a2 = a * cs - c * sn, c2 = c * cs + a * sn;
    cst(b.act, (uint32_t)(L.act[LA_KVNEW] + kl + k) * 4u, a2);
    cst(b.act, (uint32_t)(L.act[LA_KVNEW] + kl + k + dr / 2) * 4u, c2);
    cst16(rowr, (uint32_t)(kl + k) * 2u, f2bf(a2));
    cst16(rowr, (uint32_t)(kl + k + dr / 2) * 2u, f2bf(c2));
  }
  for (int i = threadIdx.x; i < A.nq * A.dv; i += kThreads) cst(b.act, (uint32_t)(L.act[LA_ATTN] + i) * 4u, 0.f);
  return true;
}

// q_abs[h][c0, c0 + 64) = sum_d W_UK[h][d][c0 + c] q_nope[h][d]. Thread t owns 8 columns
// (t % 8) of rows d = t / 8 + 64 i; the 64 row groups are summed through LDS.
__device__ __forceinline__ bool task_mla_absorb(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int kl = A.kl, dn = A.dn, nb = kl / kMlaColBlock;
  const int h = t.u0 / nb, c0 = (t.u0 - h * nb) * kMlaColBlock;
  const uint16_t* W = wp<uint16_t>(A, L.w[LW_WUK]) + (size_t)h * dn * kl + c0;
  const int q = threadIdx.x & 7, dg = threadIdx.x >> 3;
  u4 w0 = u4{0u, 0u, 0u, 0u}, w1 = w0;
  if (dg < dn) w0 = ldg_nt(W + (size_t)dg * kl + 8 * q);
  if (dg + 64 < dn) w1 = ldg_nt(W + (size_t)(dg + 64) * kl + 8 * q);
  if (!wait_deps(A, b, t)) return false;
  float* qn = b.xs;                                   // [align_up(dn, 256)]
  float* red = b.xs + ((dn + 255) & ~255);            // [64][64]
  if (threadIdx.x < 64) {
    dma_to_lds(qn, b.actp + L.act[LA_QNOPE] + h * dn, dn);
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
  }
  __syncthreads();
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  auto fma8 = [&](u4 w, float x) {
    acc[0] = fmaf(bf_lo(w.x), x, acc[0]); acc[1] = fmaf(bf_hi(w.x), x, acc[1]);
    acc[2] = fmaf(bf_lo(w.y), x, acc[2]); acc[3] = fmaf(bf_hi(w.y), x, acc[3]);
    acc[4] = fmaf(bf_lo(w.z), x, acc[4]); acc[5] = fmaf(bf_hi(w.z), x, acc[5]);
    acc[6] = fmaf(bf_lo(w.w), x, acc[6]); acc[7] = fmaf(bf_hi(w.w), x, acc[7]);
  };
  if (dg < dn) fma8(w0, qn[dg]);
  if (dg + 64 < dn) fma8(w1, qn[dg + 64]);
  for (int d = dg + 128; d < dn; d += 64) fma8(ldg_nt(W + (size_t)d * kl + 8 * q), qn[d]);
#pragma unroll
  for (int j = 0; j < 8; ++j) red[dg * 64 + 8 * q + j] = acc[j];
  __syncthreads();
  if (threadIdx.x < 64) {
    const int c = threadIdx.x;
    float v0 = 0.f, v1 = 0.f;
    for (int g = 0; g < 64; g += 2) {
      v0 += red[g * 64 + c];
      v1 += red[(g + 1) * 64 + c];
    }
    const float v = v0 + v1;
    cst(b.act, (uint32_t)(L.act[LA_QABS] + h * kl + c0 + c) * 4u, v);
    qop_store(b, L.act[LA_QOP], h, c0 + c, v * A.attn_scale_log2);
  }
  return true;
}

// One split of the latent attention: positions [u0, u1) of the layer's latent cache, all
// heads at once. Per chunk of kMlaChunk positions (DMA'd into LDS, row stride KP = kl + dr
// rounded up to 32):
//   scores  S^T[pos][h] = LAT[pos][:] . q~[h][:]   (waves 0..3, one 16-position tile each)
//   online softmax per head in base 2 (running max M and sum Lr in LDS)
//   PV      O[h][c] += P[h][pos] LAT[pos][c]       (wave w: latent column tiles w + 8 i)
// P goes through LDS in the A-operand order; the latent's B operand for PV (8 positions of
// one column per lane) is gathered from the LDS chunk. The unnormalised split partial
// (O, M, Lr) is stored for the W_UV tasks, which merge the splits.
template <bool IDX>
__device__ __forceinline__ bool task_mla_attn(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int kl = A.kl, KR = kl + A.dr, KP = (KR + 31) & ~31, NKS = KP >> 5, nh = A.nq;
  // split a1 of a2 over positions [0, n]; a plan with a per-step length can leave a split
  // empty at small positions: it then stores the neutral partial (M = -inf, Lr = 0, O = 0).
  // With the sparse indexer the split is a range of the list of selected positions
  // (increasing), of length m = min(T, n + 1).
  const bool sparse = IDX && A.idx_h > 0;
  const int n = b.n, m = sparse ? (A.idx_t < n + 1 ? A.idx_t : n + 1) : n + 1;
  const int p0 = split_pos(m - 1, t.a1, t.a2), p1 = split_pos(m - 1, t.a1 + 1, t.a2);
  const int wave = wave_id(), lane = threadIdx.x & 63, hl = lane & 15, g = lane >> 4;
  const int KS = IDX ? A.kvrow : KR;  // cache row stride (elements)
  const uint16_t* lat = A.kv + (size_t)t.layer * (A.kv_len + 1) * KS;
  u4* QL = reinterpret_cast<u4*>(b.xs);                                   // [NKS][2][64]
  uint16_t* LAT = reinterpret_cast<uint16_t*>(b.xs + NKS * 512);          // [kMlaChunk][KP]
  u4* PA = reinterpret_cast<u4*>(b.xs + NKS * 512 + kMlaChunk * KP / 2);  // [kMlaChunk/32][2][64]
  float* ST = b.xs + NKS * 512 + kMlaChunk * KP / 2 + (kMlaChunk / 32) * 512;
  float* TMAX = ST;            // [4][16]
  float* TSUM = ST + 64;       // [4][16]
  float* MR = ST + 128;        // [16] running max
  float* LR = ST + 144;        // [16] running sum
  float* AL = ST + 160;        // [16] rescale of the previous chunks
  int* SELS = reinterpret_cast<int*>(ST + 256);  // sparse: the split's selected positions
  const int segs_row = KP >> 3, nseg = kMlaChunk * segs_row;
  // positions [c0, c0 + kMlaChunk) into LAT; rows past the split repeat its last position
  // (finite values: their probabilities are 0); pad columns are zeroed after arrival
  // A chunk that holds the new position (written by another workgroup in this step) is read
  // with agent-coherent (SC1) loads: a short latent row can share its cache line with rows
  // this XCD read, and cached, earlier in the step.
  auto dma_chunk = [&](int c0, int w0) {  // issued by waves w0..7
    if (wave < w0) return;
    const int ce = c0 + kMlaChunk < p1 ? c0 + kMlaChunk : p1;
    const bool coh = sparse ? SELS[ce - 1 - p0] == n : ce > n;  // (the list increases: n can only be last)
    for (int j = wave - w0; j * 64 < nseg; j += kWaves - w0) {
      const int q = j * 64 + lane, row = q / segs_row, sc = q - row * segs_row;
      int pos = c0 + row;
      pos = pos < p1 ? pos : p1 - 1;
      if (sparse) {  // (clamped: a position the selection wrote is always in [0, n])
        pos = SELS[pos - p0];
        pos = pos < 0 ? 0 : (pos > n ? n : pos);
      }
      const int col = (sc * 8 < KR) ? sc * 8 : 0;
      if (coh)
        __builtin_amdgcn_global_load_lds((gvp)(lat + (size_t)pos * KS + col), (lvp)(LAT + j * 512), 16, 0, kCoh);
      else
        __builtin_amdgcn_global_load_lds((gvp)(lat + (size_t)pos * KS + col), (lvp)(LAT + j * 512), 16, 0, kActCpol);
    }
  };
  auto zero_pad = [&](int w0) {  // each wave zeroes the pad slots of its own copies
    if (KP == KR || wave < w0) return;
    for (int j = wave - w0; j * 64 < nseg; j += kWaves - w0) {
      const int q = j * 64 + lane, row = q / segs_row, sc = q - row * segs_row;
      if (sc * 8 >= KR) *reinterpret_cast<u4*>(LAT + (size_t)q * 8) = u4{0u, 0u, 0u, 0u};
    }
  };
  // a chunk of cached positions only (< kv_len) can be fetched before the wait (not by
  // wave 0, whose dependency polls would queue behind the copies)
  // (with the indexer the positions are known only once the selection is done: no prefetch)
  const bool pre = !sparse && (p0 + kMlaChunk < p1 ? p0 + kMlaChunk : p1) <= n;
  if (pre && p1 > p0) dma_chunk(p0, 1);
  if (!wait_deps(A, b, t)) return false;
  if (sparse && p1 > p0) {  // the split's slice of the selected positions into LDS
    for (int i = threadIdx.x; i < p1 - p0; i += kThreads)
      SELS[i] = __float_as_int(cld(b.act, (uint32_t)(L.act[LA_IDXSEL] + p0 + i) * 4u));
    __syncthreads();
  }
  if (!pre && p1 > p0) dma_chunk(p0, 0);
  if (wave == 0) dma_to_lds(reinterpret_cast<float*>(QL), b.actp + L.act[LA_QOP], NKS * 512);
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  zero_pad(pre ? 1 : 0);
  if (threadIdx.x < 16) {
    MR[threadIdx.x] = -INFINITY;
    LR[threadIdx.x] = 0.f;
  }
  __syncthreads();
  const int nct = kl >> 4;  // latent column tiles of 16
  f4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = p0; c0 < p1; c0 += kMlaChunk) {
    if (c0 != p0) {
      __syncthreads();  // the previous chunk's LAT and PA are no longer read
      dma_chunk(c0, 0);
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      zero_pad(0);
      __syncthreads();
    }
    const int nt = (p1 - c0 < kMlaChunk) ? p1 - c0 : kMlaChunk;
    float sv[4];
    if (wave < kMlaChunk / 16) {
      f4 d = f4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* arow = LAT + (size_t)(16 * wave + hl) * KP + 8 * g;
      // two k-steps per round (the MFMAs are convergent: no compiler remainder loop), then the odd one
      int ks = 0;
      for (; ks + 2 <= NKS; ks += 2) {
        const u4 a0 = *reinterpret_cast<const u4*>(arow + ks * 32);
        const u4 a1 = *reinterpret_cast<const u4*>(arow + ks * 32 + 32);
        d = mfma_bf16(a0, QL[(ks * 2) * 64 + lane], d);
        d = mfma_bf16(a0, QL[(ks * 2 + 1) * 64 + lane], d);
        d = mfma_bf16(a1, QL[(ks * 2 + 2) * 64 + lane], d);
        d = mfma_bf16(a1, QL[(ks * 2 + 3) * 64 + lane], d);
      }
      if (ks < NKS) {
        const u4 a = *reinterpret_cast<const u4*>(arow + ks * 32);
        d = mfma_bf16(a, QL[(ks * 2) * 64 + lane], d);
        d = mfma_bf16(a, QL[(ks * 2 + 1) * 64 + lane], d);
      }
      // lane: head hl, chunk positions 16 wave + 4 g + i
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = (16 * wave + 4 * g + i < nt) ? d[i] : -INFINITY;
        mx = fmaxf(mx, sv[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (lane < 16) TMAX[wave * 16 + lane] = mx;
    }
    __syncthreads();
    if (wave < kMlaChunk / 16) {
      float mn = MR[hl];
#pragma unroll
      for (int tt = 0; tt < kMlaChunk / 16; ++tt) mn = fmaxf(mn, TMAX[tt * 16 + hl]);
      float pv[4], ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = (sv[i] == -INFINITY) ? 0.f : ex2(sv[i] - mn);
        ps += pv[i];
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      if (lane < 16) TSUM[wave * 16 + lane] = ps;
      uint16_t hi[4], lo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hi[i] = f2bf(pv[i]);
        lo[i] = f2bf(pv[i] - bf16f(hi[i]));
      }
      // A operand of PV: k-step wave/2, lane hl + 16 * (position / 8), element position % 8
      const int Lp = hl + 16 * (2 * (wave & 1) + (g >> 1));
      uint16_t* pa = reinterpret_cast<uint16_t*>(PA) + ((size_t)((wave >> 1) * 2) * 64 + Lp) * 8 + 4 * (g & 1);
      *reinterpret_cast<uint2*>(pa) = uint2{bf_pair(hi[0], hi[1]), bf_pair(hi[2], hi[3])};
      *reinterpret_cast<uint2*>(pa + 64 * 8) = uint2{bf_pair(lo[0], lo[1]), bf_pair(lo[2], lo[3])};
    }
    __syncthreads();
    if (threadIdx.x < 16) {
      const int h = threadIdx.x;
      const float mo = MR[h];
      float mn = mo, ts = 0.f;
#pragma unroll
      for (int tt = 0; tt < kMlaChunk / 16; ++tt) {
        mn = fmaxf(mn, TMAX[tt * 16 + h]);
        ts += TSUM[tt * 16 + h];
      }
      const float al = (mo == -INFINITY) ? 0.f : ex2(mo - mn);
      LR[h] = LR[h] * al + ts;
      MR[h] = mn;
      AL[h] = al;
    }
    __syncthreads();
    // PV: D rows = heads 4 g + i, column = latent 16 ct + hl
    const f4 al4 = *reinterpret_cast<const f4*>(AL + 4 * g);
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) acc[jt] *= al4;
#pragma unroll 1
    for (int kk = 0; kk < kMlaChunk / 32; ++kk) {
      if (32 * kk >= nt) break;
      const u4 ah = PA[(kk * 2) * 64 + lane], alo = PA[(kk * 2 + 1) * 64 + lane];
      const uint16_t* bcol = LAT + (size_t)(32 * kk + 8 * g) * KP + hl;
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const int ct = wave + kWaves * jt;
        if (ct < nct) {
          const uint16_t* bp = bcol + 16 * ct;
          const u4 bb = u4{bf_pair(bp[0], bp[KP]), bf_pair(bp[2 * KP], bp[3 * KP]),
                           bf_pair(bp[4 * KP], bp[5 * KP]), bf_pair(bp[6 * KP], bp[7 * KP])};
          acc[jt] = mfma_bf16(ah, bb, acc[jt]);
          acc[jt] = mfma_bf16(alo, bb, acc[jt]);
        }
      }
    }
  }
  // unnormalised split partial: O[s][h][c], and (M, Lr) per head
  const int sidx = t.a1, S = t.a2;
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    const int ct = wave + kWaves * jt;
    if (ct < nct) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * g + i;
        if (h < nh) cst(b.act, (uint32_t)(t.a5 + (sidx * nh + h) * kl + 16 * ct + hl) * 4u, acc[jt][i]);
      }
    }
  }
  const int Sp = (S + 1) & ~1;  // per-head stride of the (M, Lr) table
  if (threadIdx.x < nh) {
    cst(b.act, (uint32_t)(t.a4 + (threadIdx.x * Sp + sidx) * 2) * 4u, MR[threadIdx.x]);
    cst(b.act, (uint32_t)(t.a4 + (threadIdx.x * Sp + sidx) * 2 + 1) * 4u, LR[threadIdx.x]);
  }
  return true;
}

// Merge of head h's S split partials over the latent columns [c0, c0 + 64):
//   o_lat[h][c] = sum_s 2^(M_s - M) O_s[h][c] / sum_s 2^(M_s - M) Lr_s[h]
// then o[h] += W_UV[h][:, c0:c0+64] o_lat[h][c0:c0+64] with agent-scope float atomics.
__device__ __forceinline__ bool task_mla_uv(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int kl = A.kl, dv = A.dv, nh = A.nq, S = t.a2, nb = kl / kMlaColBlock;
  const int h = t.u0 / nb, c0 = (t.u0 - h * nb) * kMlaColBlock;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const uint16_t* W = wp<uint16_t>(A, L.w[LW_WUV]) + (size_t)h * dv * kl + c0;
  const int nitems = dv * 8;  // (row j, 8 columns q) items
  const int i0 = threadIdx.x, i1 = threadIdx.x + kThreads;
  u4 w0 = u4{0u, 0u, 0u, 0u}, w1 = w0;
  if (i0 < nitems) w0 = ldg_nt(W + (size_t)(i0 >> 3) * kl + 8 * (i0 & 7));
  if (i1 < nitems) w1 = ldg_nt(W + (size_t)(i1 >> 3) * kl + 8 * (i1 & 7));
  if (!wait_deps(A, b, t)) return false;
  const int Sp = (S + 1) & ~1;
  float* MLs = b.xs;                                  // [2 Sp] (M, Lr) of head h per split
  float* ACs = MLs + ((2 * Sp + 255) & ~255);         // [S][64] split partials of this block
  float* Ws = ACs + ((S + 3) / 4) * 256;              // [S] merge weights
  float* red = Ws + ((S + 63) & ~63);                 // [8][64]
  float* ol = red + 512;                              // [64]
  if (wave == 0) dma_to_lds(MLs, b.actp + t.a4 + h * Sp * 2, 2 * Sp);
  for (int j = wave; j * 4 < S; j += kWaves) {
    int sp = 4 * j + (lane >> 4);
    sp = sp < S ? sp : S - 1;
    const float* src = b.actp + t.a5 + ((size_t)sp * nh + h) * kl + c0 + 4 * (lane & 15);
    __builtin_amdgcn_global_load_lds((gvp)src, (lvp)(ACs + j * 256), 16, 0, kActCpol);
  }
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  __syncthreads();
  if (wave == 0) {
    float M = -INFINITY;
    for (int sp = lane; sp < S; sp += 64) M = fmaxf(M, MLs[2 * sp]);
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) M = fmaxf(M, __shfl_xor(M, k, 64));
    float den = 0.f;
    for (int sp = lane; sp < S; sp += 64) {
      const float e = exp2f(MLs[2 * sp] - M);
      Ws[sp] = e;
      den += e * MLs[2 * sp + 1];
    }
    den = wave_sum(den);
    if (lane == 0) b.flags[2] = __float_as_int(1.0f / den);
  }
  __syncthreads();
  {
    const int c = threadIdx.x & 63;
    float v = 0.f;
    for (int sp = threadIdx.x >> 6; sp < S; sp += kWaves) v = fmaf(Ws[sp], ACs[sp * 64 + c], v);
    red[(threadIdx.x >> 6) * 64 + c] = v;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) v += red[k * 64 + threadIdx.x];
    v *= __int_as_float(b.flags[2]);
    ol[threadIdx.x] = v;
    cst(b.act, (uint32_t)(L.act[LA_OLAT] + h * kl + c0 + threadIdx.x) * 4u, v);
  }
  __syncthreads();
  float* o = b.actp + L.act[LA_ATTN] + h * dv;
  auto item = [&](int i, u4 w) {
    const float* x = ol + 8 * (i & 7);
    float v = bf_lo(w.x) * x[0];
    v = fmaf(bf_hi(w.x), x[1], v);
    v = fmaf(bf_lo(w.y), x[2], v);
    v = fmaf(bf_hi(w.y), x[3], v);
    v = fmaf(bf_lo(w.z), x[4], v);
    v = fmaf(bf_hi(w.z), x[5], v);
    v = fmaf(bf_lo(w.w), x[6], v);
    v = fmaf(bf_hi(w.w), x[7], v);
    v = group_sum<8>(v);
    if ((i & 7) == 0) __hip_atomic_fetch_add(o + (i >> 3), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  if (i0 < nitems) item(i0, w0);
  if (i1 < nitems) item(i1, w1);
  for (int i = threadIdx.x + 2 * kThreads; i < nitems; i += kThreads) item(i, ldg_nt(W + (size_t)(i >> 3) * kl + 8 * (i & 7)));
  return true;
}


// ------------------------------------------------------------------ MoE tasks
//
// Sparse FFN of the MoE layers: a sigmoid router picks top_k of n_routed experts (TileRT
// audit page, the MoE-routing paragraph: the expert choice is made on the device, so the
// expert tasks read their weight pointers from the router's output at run time); one or
// more shared experts run on every token, during the routing wait.

// hn = RMSNorm(h); r = W_router hn
__device__ __forceinline__ bool task_router(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int K = A.hidden;
  const RmPlain rm{wp<uint16_t>(A, L.w[LW_ROUTER]), K, t.u0};
  return run_gemv(
      A, b, t, rm, t.u1 - t.u0, K, 1, true,
      stage_vec(L.act[LA_H], nullptr, K, pad512(K), wp<uint16_t>(A, L.w[LW_FFN_NORM]), A.eps),
      [&] {
        for (int i = threadIdx.x; i < t.u1 - t.u0; i += 64) cst(b.act, (uint32_t)(L.act[LA_RLOGIT] + t.u0 + i) * 4u, b.ys[i]);
      });
}

// Expert matrices in MXFP4 (ES = 0): rows of K / 2 packed bytes, and K / 32 E8M0 scale bytes
// per row in the weight bound after the matrix. Unit u -> (gate row u, up row u) of the
// shared experts' [ns * eff, hidden] matrices.
struct RmGateUp4 {
  const uint8_t *Wg, *Wu, *Sg, *Su;
  int K, u0;
  __device__ __forceinline__ const void* row(int j) const {
    return pick2(j & 1, Wg, Wu) + (size_t)(u0 + (j >> 1)) * (K / 2);
  }
  __device__ __forceinline__ const void* srow(int j) const {
    return pick2(j & 1, Sg, Su) + (size_t)(u0 + (j >> 1)) * (K / 32);
  }
  __device__ __forceinline__ int xoff(int) const { return 0; }
};

// shared experts' gate/up rows (rows of [ns * eff, hidden] matrices) + SwiGLU
template <int ES, class RM>
__device__ __forceinline__ bool shared_gu(const EngineArgs& A, Blk& b, const TaskDesc& t, const RM& rm) {
  const LayerDesc& L = A.layers[t.layer];
  const int K = A.hidden;
  return run_gemv<2, false, ES>(
      A, b, t, rm, 2 * (t.u1 - t.u0), K, 1, true,
      stage_vec(L.act[LA_H], nullptr, K, padc<ES>(K), wp<uint16_t>(A, L.w[LW_FFN_NORM]), A.eps),
      [&] {
        for (int i = threadIdx.x; i < t.u1 - t.u0; i += 64)
          cst(b.act, (uint32_t)(L.act[LA_SACT] + t.u0 + i) * 4u, silu(b.ys[2 * i]) * b.ys[2 * i + 1]);
      });
}
template <int ES>
__device__ __forceinline__ bool task_shared_gu(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  if constexpr (ES == 0) {
    const RmGateUp4 rm{wp<uint8_t>(A, L.w[LW_SGATE]), wp<uint8_t>(A, L.w[LW_SUP]), wp<uint8_t>(A, L.w[LW_SGATE] + 1),
                       wp<uint8_t>(A, L.w[LW_SUP] + 1), A.hidden, t.u0};
    return shared_gu<ES>(A, b, t, rm);
  } else {
    const RmGateUp rm{wp<uint8_t>(A, L.w[LW_SGATE]), wp<uint8_t>(A, L.w[LW_SUP]), A.hidden, t.u0, ES,
                      wscale<ES>(A, L.w[LW_SGATE]), wscale<ES>(A, L.w[LW_SUP])};
    return shared_gu<ES>(A, b, t, rm);
  }
}

// sigma = sigmoid(r), z = sigma + bias (fp32). The top_k experts by z, ties to the lower
// index, in decreasing order of z: expert e goes to slot rank(e) = #{f : z_f > z_e or
// (z_f == z_e and f < e)} when that is below top_k. Weights w = sigma_T / sum(sigma_T).
// Output: int32 ids[top_k], then fp32 w[top_k].
__device__ __forceinline__ bool task_topk(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int E = A.n_routed, K = A.top_k;
  if (!wait_deps(A, b, t)) return false;
  float* z = b.xs;                       // [E]
  float* sg = b.xs + ((E + 255) & ~255);  // [E]
  float* bias = sg + ((E + 255) & ~255);  // [E]
  int* ids = reinterpret_cast<int*>(b.ys);  // [top_k] chosen experts in rank order
  if (threadIdx.x < 64) {
    dma_to_lds(z, b.actp + L.act[LA_RLOGIT], E & ~3);
    dma_to_lds(bias, wp<float>(A, L.w[LW_RBIAS]), E & ~3);
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    for (int e = (E & ~3) + (int)threadIdx.x; e < E; e += 64) {
      z[e] = cld(b.act, (uint32_t)(L.act[LA_RLOGIT] + e) * 4u);
      bias[e] = wp<float>(A, L.w[LW_RBIAS])[e];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < ((E + 3) & ~3); e += kThreads) {
    if (e < E) {
      const float s = 1.0f / (1.0f + expf(-z[e]));
      sg[e] = s;
      z[e] = s + bias[e];
    } else {
      z[e] = -INFINITY;  // padding: never ranks above a real expert
    }
  }
  __syncthreads();
  // wave 0 picks the K largest z in K rounds. Each lane keeps the largest selection key of the
  // scores it owns (e = lane, lane + 64, ...); the wave-wide maximum names the round's
  // winner, whose owner retires it (NaN in LDS: key 0) and rescans its own scores. The picks
  // come out in decreasing z, lower index first among equal values.
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    // a lane's scores four at a time: z spans E rounded up to 256 floats, so the four reads
    // stay inside it, and slots at or past E count as empty
    auto scan = [&]() {
      uint64_t m = 0;
      for (int e0 = lane; e0 < E; e0 += 256) {
        float a[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = z[e0 + 64 * j];
#pragma unroll
        for (int j = 0; j < 4; ++j) m = umax64(m, e0 + 64 * j < E ? sel_key(a[j], e0 + 64 * j) : 0ull);
      }
      return m;
    };
    uint64_t lk = scan();
    for (int k = 0; k < K; ++k) {
      const uint64_t w = wave_max_key(lk);
      const int bi = w == 0 ? 0 : sel_index(w);  // (key 0 only if every remaining score is NaN)
      if (lane == 0) ids[k] = bi;
      if (lane == (bi & 63)) {
        z[bi] = __int_as_float(0x7fc00000);
        lk = scan();
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {  // lane k < K holds pick k (top_k <= 64)
    const int k = threadIdx.x;
    const int id = k < K ? ids[k] : 0;
    const float s = k < K ? sg[id] : 0.f;
    const float sum = wave_sum(s);
    if (k < K) {
      cst(b.act, (uint32_t)(L.act[LA_TOPK] + k) * 4u, __int_as_float(id));
      cst(b.act, (uint32_t)(L.act[LA_TOPK] + K + k) * 4u, s / sum);
    }
  }
  return true;
}

// Routed experts' gate/up: unit u = (slot k, row i) -> rows i of W_gate[e_k], W_up[e_k];
// the expert ids are read once the top-k task has signalled, then the rows are prefetched.
template <int ES = 2>
struct RmExpertGU {
  const uint8_t *Wg, *Wu;
  const int* ids;  // LDS
  int K, F, u0;
  const uint8_t *Sg = nullptr, *Su = nullptr;  // MXFP4: the block scales; FP8: the fp32 row scales
  __device__ __forceinline__ size_t rix(int j) const {  // the row's index in [E * F] rows
    const int u = u0 + (j >> 1), k = u / F, i = u - k * F;
    return (size_t)ids[k] * F + i;
  }
  __device__ __forceinline__ const void* row(int j) const {
    const uintptr_t g = (uintptr_t)Wg;
    const uintptr_t base = g + (uintptr_t)(j & 1) * ((uintptr_t)Wu - g);
    return (const uint8_t*)base + rix(j) * (ES == 0 ? K / 2 : (size_t)K * ES);
  }
  __device__ __forceinline__ float scale(int j) const { return ((const float*)pick2(j & 1, Sg, Su))[rix(j)]; }
  __device__ __forceinline__ const void* srow(int j) const { return pick2(j & 1, Sg, Su) + rix(j) * (K / 32); }
  __device__ __forceinline__ int xoff(int) const { return 0; }
};

// The chosen expert ids into LDS (clamped to the expert range so that a bad id cannot
// address outside the weights).
__device__ __forceinline__ void stage_ids(const EngineArgs& A, const LayerDesc& L, Blk& b, int* ids) {
  if (threadIdx.x < (unsigned)A.top_k) {
    int e = __float_as_int(cld(b.act, (uint32_t)(L.act[LA_TOPK] + threadIdx.x) * 4u));
    e = e < 0 ? 0 : (e >= A.n_routed ? A.n_routed - 1 : e);
    ids[threadIdx.x] = e;
  }
}

template <int ES>
__device__ __forceinline__ bool task_expert_gu(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int K = A.hidden, F = A.eff;
  int* ids = reinterpret_cast<int*>(b.scr);
  const RmExpertGU<ES> rm{wp<uint8_t>(A, L.w[LW_EGATE]), wp<uint8_t>(A, L.w[LW_EUP]), ids, K, F, t.u0,
                          ES != 2 ? wp<uint8_t>(A, L.w[LW_EGATE] + 1) : nullptr,
                          ES != 2 ? wp<uint8_t>(A, L.w[LW_EUP] + 1) : nullptr};
  return run_gemv<2, false, ES>(
      A, b, t, rm, 2 * (t.u1 - t.u0), K, 1, true,
      stage_vec(L.act[LA_H], nullptr, K, padc<ES>(K), wp<uint16_t>(A, L.w[LW_FFN_NORM]), A.eps),
      [&] {
        for (int i = threadIdx.x; i < t.u1 - t.u0; i += 64)
          cst(b.act, (uint32_t)(L.act[LA_ACT] + t.u0 + i) * 4u, silu(b.ys[2 * i]) * b.ys[2 * i + 1]);
      },
      t.a2, [&] { stage_ids(A, L, b, ids); });
}

// Down projections: output row r sums G = ns + top_k segments of eff columns: segment s < ns
// is shared expert s (columns s*eff.. of W_sdown[r]), segment ns + k is W_down[e_k][r]. The
// staged input holds the shared activations and the routed ones pre-scaled by w_k, one
// segment per 512-aligned slot.
template <int ES = 2>
struct RmMoeDown {
  const uint8_t *Ws, *Wd;
  const int* ids;  // LDS
  int ns, G, F, Fp, d, r0;
  const uint8_t *Ss = nullptr, *Sd = nullptr;  // MXFP4: the block scales; FP8: the fp32 row scales
  // element offset of task row j's segment: shared experts' segments lie side by side in one
  // row of W_sdown; a routed expert's is a row of its own W_down
  __device__ __forceinline__ bool shared(int j) const { return j % G < ns; }
  __device__ __forceinline__ size_t eoff(int j) const {
    const int q = j / G, sgm = j - q * G, r = r0 + q;
    if (sgm < ns) return (size_t)r * ns * F + (size_t)sgm * F;
    return ((size_t)ids[sgm - ns] * d + r) * F;
  }
  __device__ __forceinline__ const void* row(int j) const {
    return pick2(!shared(j), Ws, Wd) + (ES == 0 ? eoff(j) / 2 : eoff(j) * ES);
  }
  // FP8: a shared expert's segment is part of one row r of W_sdown (scale r); a routed one is
  // row r of its expert's W_down
  __device__ __forceinline__ float scale(int j) const {
    const int q = j / G, sgm = j - q * G, r = r0 + q;
    return shared(j) ? ((const float*)Ss)[r] : ((const float*)Sd)[(size_t)ids[sgm - ns] * d + r];
  }
  __device__ __forceinline__ const void* srow(int j) const { return pick2(!shared(j), Ss, Sd) + eoff(j) / 32; }
  __device__ __forceinline__ int xoff(int j) const { return (j % G) * Fp; }
};

// MXFP4 segments are padded to 256 columns, the unit of the staging copy (one 1-KB LDS DMA),
// not to whole 2048-column chunks: lanes past a segment's end drop their products (StreamT).
template <int ES>
__device__ __forceinline__ bool task_moe_down(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int F = A.eff, Fp = ES == 0 ? (F + 255) / 256 * 256 : padc<ES>(F), ns = A.n_shared, Kt = A.top_k, G = ns + Kt, d = A.hidden;
  int* ids = reinterpret_cast<int*>(b.scr);
  float* wk = b.scr + 64;
  const RmMoeDown<ES> rm{wp<uint8_t>(A, L.w[LW_SDOWN]), wp<uint8_t>(A, L.w[LW_EDOWN]), ids, ns, G, F, Fp, d, t.u0,
                         ES != 2 ? wp<uint8_t>(A, L.w[LW_SDOWN] + 1) : nullptr,
                         ES != 2 ? wp<uint8_t>(A, L.w[LW_EDOWN] + 1) : nullptr};
  return run_gemv<2, false, ES>(
      A, b, t, rm, G * (t.u1 - t.u0), F, G, true,
      stage_fn([&] {
        {
          // the G input segments (8 KB each at eff = 2048) are copied by the waves in turn: one
          // wave alone would issue more copies than it can keep in flight
          const int wave = wave_id();
          if (threadIdx.x < 64)
            for (int k = threadIdx.x; k < Kt; k += 64) wk[k] = cld(b.act, (uint32_t)(L.act[LA_TOPK] + Kt + k) * 4u);
          for (int sg = wave; sg < G; sg += kWaves) {
            const float* src = b.actp + (sg < ns ? L.act[LA_SACT] + sg * F : L.act[LA_ACT] + (sg - ns) * F);
            dma_to_lds(b.xs + sg * Fp, src, F);
          }
          __builtin_amdgcn_s_waitcnt(kVmcnt0);  // (a wave's copies land after its own prefetch)
        }
        __syncthreads();
        for (int sg = 0; sg < G; ++sg) {
          const float w = sg < ns ? 1.0f : wk[sg - ns];
          for (int c = threadIdx.x; c < Fp; c += kThreads) {
            float* x = b.xs + sg * Fp + c;
            *x = c < F ? *x * w : 0.f;
          }
        }
        __syncthreads();
      }),
      [&] {
        for (int i = threadIdx.x; i < t.u1 - t.u0; i += 64) {
          const int rr = t.u0 + i;
          const float y = b.ys[i];
          const float xo = cld(b.act, (uint32_t)(L.act[LA_H] + rr) * 4u) + y;
          cst(b.act, (uint32_t)(L.act[LA_FFN_OUT] + rr) * 4u, y);
          cst(b.act, (uint32_t)(L.act[LA_X_OUT] + rr) * 4u, xo);
          if (t.a0) A.out[rr] = xo;
        }
      },
      t.a2, [&] { stage_ids(A, L, b, ids); });
}


// ------------------------------------------------------------------ sparse indexer
//
// The TileRT audit page's sparse_index: index heads score every cached position and attention
// reads only the top-T of them. Per layer (reading of the oracle): index key k = W_k x^ and head
// weights w = W_w x^ come out of the T_MLA_A rows (the key is appended to the cache after the
// position's latent row), index queries q_j = (W_q c_q)_j out of T_IDX_Q; T_IDX_SCORE computes
// I_s = sum_j w_j max(0, q_j . k_s) for a range of positions on the matrix cores, T_IDX_TOPK
// selects the T largest (ties to the lower position) in increasing position order, and the
// latent attention splits that list.

// index queries: rows of W_q [H * DI][ql] times the normalised query latent
__device__ __forceinline__ bool task_idx_q(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int K = A.ql;
  const RmPlain rm{wp<uint8_t>(A, L.w[LW_IDXQ]), K, t.u0};
  return run_gemv(
      A, b, t, rm, t.u1 - t.u0, K, 1, true,
      stage_vec(L.act[LA_CQ], nullptr, K, pad512(K), wp<uint16_t>(A, L.w[LW_QNORM]), A.eps),
      [&] {
        for (int i = threadIdx.x; i < t.u1 - t.u0; i += 64) cst(b.act, (uint32_t)(L.act[LA_IDXQ] + t.u0 + i) * 4u, b.ys[i]);
      });
}

// Scores of positions [p0, p1) (range a1 of a2 over [0, n], cut at run time). The queries
// become the B operand of bf16 MFMA 16x16x32 (16 heads per tile, k = the key's dimensions,
// fp32 split into bf16 hi + lo); 16 positions' keys are the A operand, exact bf16, loaded from
// the cache straight into registers. For each head tile the 16 x 16 score tile gets the ReLU and
// the head weights, and the sum over heads is a 16-lane reduction.
__device__ __forceinline__ bool task_idx_score(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int H = A.idx_h, DI = A.idx_d, NKI = DI / 32, HT = (H + 15) / 16, KR = A.kl + A.dr, n = b.n;
  const int p0 = split_pos(n, t.a1, t.a2), p1 = split_pos(n, t.a1 + 1, t.a2);
  const int wave = wave_id(), lane = threadIdx.x & 63;
  float* QF = b.xs;                                      // [H][DI] fp32
  u4* QB = reinterpret_cast<u4*>(b.xs + H * DI);         // [HT][NKI][hi, lo][64 lanes]
  float* WI = b.xs + H * DI + HT * NKI * 2 * 256;        // [64] head weights (0 past H)
  if (!wait_deps(A, b, t)) return false;
  dma_to_lds_all(QF, b.actp + L.act[LA_IDXQ], H * DI);
  if (threadIdx.x < 64) WI[lane] = lane < H ? cld(b.act, (uint32_t)(L.act[LA_IDXW] + lane) * 4u) : 0.f;
  __syncthreads();
  for (int e = threadIdx.x; e < HT * NKI * 64; e += kThreads) {
    const int Ll = e & 63, ks = (e >> 6) % NKI, ht = (e >> 6) / NKI;
    const int hh = 16 * ht + (Ll & 15), k0 = 32 * ks + 8 * (Ll >> 4);
    const f4 z = f4{0.f, 0.f, 0.f, 0.f};
    const f4 a = hh < H ? *reinterpret_cast<const f4*>(QF + hh * DI + k0) : z;
    const f4 c = hh < H ? *reinterpret_cast<const f4*>(QF + hh * DI + k0 + 4) : z;
    u4 hi, lo;
    split_bf16x8(a, c, 1.0f, hi, lo);
    QB[((ht * NKI + ks) * 2 + 0) * 64 + Ll] = hi;
    QB[((ht * NKI + ks) * 2 + 1) * 64 + Ll] = lo;
  }
  __syncthreads();
  // the layer's cache rows as one buffer (key of position p at element p * kvrow + KR)
  const rsrc_t kr = make_rsrc(A.kv + (size_t)t.layer * (A.kv_len + 1) * A.kvrow, (uint32_t)((A.kv_len + 1) * A.kvrow * 2));
  for (int base = p0 + 16 * wave; base < p1; base += 16 * kWaves) {
    int pos = base + (lane & 15);
    pos = pos < p1 ? pos : p1 - 1;
    const uint32_t off = (uint32_t)(pos * A.kvrow + KR + 8 * (lane >> 4)) * 2u;
    // the key of position n was written in this step by another workgroup: read it coherently
    const bool has_new = base + 16 > n;
    u4 ka[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < NKI) {
        if (has_new)
          ka[ks] = __builtin_amdgcn_raw_buffer_load_b128(kr, off + 64u * ks, 0, kCoh);
        else
          ka[ks] = __builtin_amdgcn_raw_buffer_load_b128(kr, off + 64u * ks, 0, kActCpol);
      }
    }
    f4 acc = f4{0.f, 0.f, 0.f, 0.f};
    for (int ht = 0; ht < HT; ++ht) {
      f4 d = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (ks < NKI) {
          d = mfma_bf16(ka[ks], QB[((ht * NKI + ks) * 2 + 0) * 64 + lane], d);
          d = mfma_bf16(ka[ks], QB[((ht * NKI + ks) * 2 + 1) * 64 + lane], d);
        }
      }
      const float w = WI[16 * ht + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, fmaxf(d[i], 0.f), acc[i]);
    }
    // lane: head 16 ht + lane % 16, positions base + 4 (lane / 16) + i
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = group_sum<16>(acc[i]);
    if ((lane & 15) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = base + 4 * (lane >> 4) + i;
        if (p < p1) cst(b.act, (uint32_t)(L.act[LA_IDXS] + p) * 4u, acc[i] + 0.f);  // (+0: no -0 scores)
      }
    }
  }
  return true;
}

// An fp32 score as an unsigned key with the same order.
__device__ __forceinline__ uint32_t score_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of v over the workgroup's threads (thread order), and the total;
// scratch: 8 words.
__device__ __forceinline__ int block_excl_scan(int v, int* scratch, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int pre = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int c = scratch[w];
    pre += w < wave ? c : 0;
    total += c;
  }
  __syncthreads();
  return pre + incl - v;
}

// The top T of the N = n + 1 scores, ties to the lower position, written in increasing position
// order (all positions when N <= T). The scores go to LDS as order-preserving unsigned keys'
// sources, in chunks of C (once, when N <= C). A min/max pass finds the bits every key shares;
// radix passes of up to 11 bits below them narrow the prefix of the T-th largest key and how many
// of the keys with that prefix are still to take, until either the whole bucket is taken or every
// bit is fixed. A last pass compacts: each thread scans a contiguous block of positions (an odd
// number of them, so that the block starts fall in distinct LDS banks) and the block prefix sums
// give each taken position its slot.
__device__ __forceinline__ bool task_idx_topk(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int N = b.n + 1, T = A.idx_t, C = t.a0;
  if (!wait_deps(A, b, t)) return false;
  const uint32_t sel = (uint32_t)L.act[LA_IDXSEL] * 4u;
  if (N <= T) {
    for (int i = threadIdx.x; i < N; i += kThreads) cst(b.act, sel + (uint32_t)i * 4u, __int_as_float(i));
    return true;
  }
  constexpr int kBins = kIdxBins;
  float* SC = b.xs;                                                // [C] one chunk of scores
  uint32_t* hist = reinterpret_cast<uint32_t*>(b.xs + C);          // [kBins]
  int* misc = reinterpret_cast<int*>(b.xs + C + kBins);            // [0..2] choice, [8..15] scan, [16..31] min/max
  const float* src = b.actp + L.act[LA_IDXS];
  const int nch = (N + C - 1) / C, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  static_assert(kBins == 4 * kThreads, "the bin scan gives each thread four bins");
  // DMA of chunk c into SC; `chunk` returns chunk c's length, loading it unless the one chunk
  // is resident
  auto fetch = [&](int c) {
    const int c0 = c * C, cnt = N - c0 < C ? N - c0 : C;
    __syncthreads();  // the previous chunk's readers are done
    dma_to_lds_all(SC, src + c0, (cnt + 3) & ~3);
    __syncthreads();
    return cnt;
  };
  auto chunk = [&](int c) { return nch == 1 ? N : fetch(c); };
  // f(key) for the chunk's keys i = thread, thread + kThreads, ...: eight LDS reads in flight
  // per thread (one at a time, each read's latency was paid in full: 3.6 us per pass over 32769)
  auto strided = [&](int cnt, auto&& f) {
    int i = threadIdx.x;
    for (; i + 7 * kThreads < cnt; i += 8 * kThreads) {
      uint32_t k[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) k[u] = score_key(SC[i + u * kThreads]);
#pragma unroll
      for (int u = 0; u < 8; ++u) f(k[u]);
    }
    for (; i < cnt; i += kThreads) f(score_key(SC[i]));
  };
  // f(masked key, i) for i = i0 .. i1 - 1 in order, eight reads in flight
  auto in_order = [&](int i0, int i1, uint32_t m, auto&& f) {
    int i = i0;
    for (; i + 8 <= i1; i += 8) {
      uint32_t k[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) k[u] = score_key(SC[i + u]) & m;
#pragma unroll
      for (int u = 0; u < 8; ++u) f(k[u], i + u);
    }
    for (; i < i1; ++i) f(score_key(SC[i]) & m, i);
  };
  if (nch == 1) fetch(0);
  if (kTaskLogDetail && threadIdx.x == 0) b.t_sub[0] = (uint32_t)now();
  // the keys' common high bits
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int c = 0; c < nch; ++c)
    strided(chunk(c), [&](uint32_t k) {
      kmin = k < kmin ? k : kmin;
      kmax = k > kmax ? k : kmax;
    });
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t a = (uint32_t)__shfl_xor((int)kmin, d, 64), c = (uint32_t)__shfl_xor((int)kmax, d, 64);
    kmin = a < kmin ? a : kmin;
    kmax = c > kmax ? c : kmax;
  }
  if (lane == 0) {
    misc[16 + wave] = (int)kmin;
    misc[24 + wave] = (int)kmax;
  }
  __syncthreads();
  kmin = 0xffffffffu;
  kmax = 0u;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t a = (uint32_t)misc[16 + w], c = (uint32_t)misc[24 + w];
    kmin = a < kmin ? a : kmin;
    kmax = c > kmax ? c : kmax;
  }
  // bits at and above `lo` are fixed: keys whose masked value exceeds `prefix` are all taken, and
  // `need` of those equal to it
  if (kTaskLogDetail && threadIdx.x == 0) b.t_sub[1] = (uint32_t)now();
  int lo = kmin == kmax ? 0 : 32 - __builtin_clz(kmin ^ kmax);
  uint32_t mask = lo >= 32 ? 0u : ~((1u << lo) - 1u), prefix = kmax & mask;
  int need = T;
  while (lo > 0) {
    const int width = lo < 11 ? lo : 11, shift = lo - width;
    const uint32_t dm = (1u << width) - 1u;
    for (int i = threadIdx.x; i < kBins; i += kThreads) hist[i] = 0u;
    __syncthreads();
    for (int c = 0; c < nch; ++c)
      strided(chunk(c), [&](uint32_t k) {
        if ((k & mask) == prefix) atomicAdd(hist + ((k >> shift) & dm), 1u);
      });
    __syncthreads();
    // thread j holds bins kBins-1-4j .. kBins-4-4j (from the top)
    uint32_t h[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) h[q] = hist[kBins - 1 - 4 * (int)threadIdx.x - q];
    const int sum = (int)(h[0] + h[1] + h[2] + h[3]);
    int tot;
    int before = block_excl_scan(sum, misc + 8, tot);  // keys in higher bins than this thread's
    if (before < need && need <= before + sum) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (need <= before + (int)h[q]) {
          misc[0] = kBins - 1 - 4 * (int)threadIdx.x - q;
          misc[1] = need - before;
          misc[2] = (int)h[q];
          break;
        }
        before += (int)h[q];
      }
    }
    __syncthreads();
    prefix |= (uint32_t)misc[0] << shift;
    mask |= dm << shift;
    need = misc[1];
    lo = shift;
    const bool whole = need == misc[2];
    __syncthreads();
    if (whole) break;
  }
  if (kTaskLogDetail && threadIdx.x == 0) b.t_sub[2] = (uint32_t)now();
  // compaction, chunk by chunk in position order
  int eq_seen = 0, out_seen = 0;
  for (int c = 0; c < nch; ++c) {
    const int cnt = chunk(c), c0 = c * C;
    const int B = ((cnt + kThreads - 1) / kThreads) | 1;
    const int i0 = (int)threadIdx.x * B < cnt ? (int)threadIdx.x * B : cnt, i1 = i0 + B < cnt ? i0 + B : cnt;
    int gt = 0, eq = 0;
    in_order(i0, i1, mask, [&](uint32_t k, int) {
      gt += k > prefix;
      eq += k == prefix;
    });
    int eq_tot, out_tot;
    const int eqb = eq_seen + block_excl_scan(eq, misc + 8, eq_tot);
    int take = need - eqb;
    take = take < 0 ? 0 : (take > eq ? eq : take);
    int out = out_seen + block_excl_scan(gt + take, misc + 8, out_tot);
    in_order(i0, i1, mask, [&](uint32_t k, int i) {
      if (k > prefix || (k == prefix && take-- > 0)) cst(b.act, sel + (uint32_t)(out++) * 4u, __int_as_float(c0 + i));
    });
    eq_seen += eq_tot;
    out_seen += out_tot;
  }
  return true;
}


// ------------------------------------------------------------------ multi-token verification
//
// A verification step of MT tokens at positions n .. n + MT - 1 (the check of draft tokens in
// speculative decoding, or the tokens of multi-token prediction; the TileRT talk, practice
// section): every weight row is read once for all MT tokens, so each GEMV becomes a skinny GEMM
// of MT columns, computed on the vector ALUs as MT dot products per row. Activations are
// [MT][width] in the workspace and [MT][padded width] in LDS; an input too wide to stage for
// all MT tokens at once (the down projection's) is staged and streamed in column phases, the
// row sums adding up in LDS across phases. Attention is causal within the block: token i sees
// the cached positions and the block's positions n .. n + i.

// Per-token 1/rms of a verification step's staged inputs: LDS words after the staging flags
// (written in the staging step, read in the epilogue; 1 where there is no RMSNorm).
__device__ __forceinline__ float* token_norms(const Blk& b) { return reinterpret_cast<float*>(b.flags) + 48; }

// Staging of columns [k0, k0 + kw) of MT vectors (token i at float offset off + i * stride, or
// the bf16 step input x + i * stride when off < 0) into xs[i * pw + c], zero-padded to pw. With
// a gain (never phased: kw == K) each token is RMSNormed: xs holds g * x and the per-token 1/rms goes to LDS (token_norms).
template <int MT>
struct StageM {
  int off, stride;
  const uint16_t* s16;
  int K, k0, kw, pw;
  const uint16_t* gain;
  float eps;
  bool coh;
  __device__ __forceinline__ bool early_ok() const { return off >= 0 && MT * kw <= kEarlyDmaFloats; }
  __device__ __forceinline__ void before(Blk& b) const {  // wave 0
    if (gain) dma_to_lds(b.gs, (const float*)gain, K / 2);
  }
  __device__ __forceinline__ void early(Blk& b) const {  // wave 0
    if (!early_ok()) return;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if (coh) dma_to_lds<true>(b.xs + i * pw, b.actp + off + i * stride + k0, kw);
      else dma_to_lds(b.xs + i * pw, b.actp + off + i * stride + k0, kw);
    }
  }
  __device__ __forceinline__ void finish(Blk& b) const {
    if (off >= 0 && !early_ok()) {
      // every wave copies a share: 1-KB chunk j of token i by wave (i * chunks + j) % 8
      const int nch = (kw + 255) / 256, lane = threadIdx.x & 63;
      for (int q = (int)(threadIdx.x >> 6); q < MT * nch; q += kWaves) {
        const int i = q / nch, j = q - i * nch;
        int c = j * 256 + lane * 4;
        c = c < kw ? c : kw - 4;
        if (coh) lds_dma16<true>(b.actp + off + i * stride + k0 + c, b.xs + i * pw + j * 256);
        else lds_dma16(b.actp + off + i * stride + k0 + c, b.xs + i * pw + j * 256);
      }
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
    }
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      if (off < 0) {  // the bf16 step inputs (layer 0)
        for (int i = 0; i < MT; ++i)
          for (int c = lane * 4; c < kw; c += 256) {
            const uint2 x = *(const uint2*)(s16 + (size_t)i * stride + k0 + c);
            *(f4*)(b.xs + i * pw + c) = f4{bf_lo(x.x), bf_hi(x.x), bf_lo(x.y), bf_hi(x.y)};
          }
      }
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
    }
    // (as in StageVec: the clamped lanes of another wave's partial last block write past kw)
    if (off >= 0 && !early_ok() && (kw & 255)) __syncthreads();
    if (threadIdx.x < 64)
      for (int i = 0; i < MT; ++i)
        for (int c = kw + (int)threadIdx.x; c < pw; c += 64) b.xs[i * pw + c] = 0.f;
    __syncthreads();
    float* nrm = token_norms(b);
    if (threadIdx.x < MT) nrm[threadIdx.x] = 1.f;
    if (gain) {
      const uint16_t* g16 = reinterpret_cast<const uint16_t*>(b.gs);
      float* part = reinterpret_cast<float*>(b.flags) + 8;  // [wave][MT] sums of squares
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        float ss = 0.f;
        for (int c = threadIdx.x * 4; c < K; c += kThreads * 4) {
          const uint2 g = *(const uint2*)(g16 + c);
          f4 v = *(f4*)(b.xs + i * pw + c);
          ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
          v.x *= bf_lo(g.x);
          v.y *= bf_hi(g.x);
          v.z *= bf_lo(g.y);
          v.w *= bf_hi(g.y);
          *(f4*)(b.xs + i * pw + c) = v;
        }
        ss = wave_sum(ss);
        if ((threadIdx.x & 63) == 0) part[(threadIdx.x >> 6) * MT + i] = ss;
      }
      __syncthreads();
      if (threadIdx.x < MT) {
        float tot = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) tot += part[w * MT + threadIdx.x];
        nrm[threadIdx.x] = 1.0f / sqrtf(tot / (float)K + eps);
      }
    }
  }
};

// Streams chunks [ca, cb) of the task's rows (bf16, 512 columns per chunk) over a flattened
// (row, chunk) range [fa, fb), dotting each with the MT staged vectors (xs[i * pw + column -
// ca * 512]); each row's partial sums are added into ys[row * MT + i] with LDS atomics when the
// wave's part of the row ends.
template <int MT>
struct StreamM {
  const uint64_t* rowp;
  int fb, K, ca, cpr, pw, lane;
  int lf, lj, lc;
  const uint8_t* lrow;
  int cf, cj, cc;
  float acc[MT][2];
  __device__ __forceinline__ void init(const uint64_t* rp, int fa, int fb_, int K_, int ca_, int cb_, int pw_, int lane_) {
    rowp = rp;
    fb = fb_;
    K = K_;
    ca = ca_;
    cpr = cb_ - ca_;
    pw = pw_;
    lane = lane_;
    const int j0 = fa / cpr, c0 = fa - j0 * cpr;
    lf = cf = fa;
    lj = cj = j0;
    lc = cc = c0;
    lrow = (fa < fb) ? (const uint8_t*)uni64(rowp[j0]) : nullptr;
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[i][0] = acc[i][1] = 0.f;
  }
  __device__ __forceinline__ void load(u4 (&bf)[NB]) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (lf < fb) {
        int col = (ca + lc) * kChunkCols + lane * 8;
        col = col < K ? col : 0;  // masked lanes re-read the row start; xs is zero there
        bf[i] = ldg_nt(lrow + (size_t)col * 2);
        ++lf;
        if (++lc == cpr) {
          lc = 0;
          ++lj;
          if (lf < fb) lrow = (const uint8_t*)uni64(rowp[lj]);
        }
      }
    }
  }
  __device__ __forceinline__ void consume(const u4 (&bf)[NB], const float* xs, float* ys) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (cf < fb) {
        const u4 w = bf[k];
        const float wf[8] = {bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y), bf_lo(w.z), bf_hi(w.z), bf_lo(w.w), bf_hi(w.w)};
        const float* xp = xs + cc * kChunkCols + lane * 8;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const f4 x0 = *(const f4*)(xp + i * pw), x1 = *(const f4*)(xp + i * pw + 4);
          acc[i][0] = fmaf(wf[0], x0.x, acc[i][0]);
          acc[i][1] = fmaf(wf[1], x0.y, acc[i][1]);
          acc[i][0] = fmaf(wf[2], x0.z, acc[i][0]);
          acc[i][1] = fmaf(wf[3], x0.w, acc[i][1]);
          acc[i][0] = fmaf(wf[4], x1.x, acc[i][0]);
          acc[i][1] = fmaf(wf[5], x1.y, acc[i][1]);
          acc[i][0] = fmaf(wf[6], x1.z, acc[i][0]);
          acc[i][1] = fmaf(wf[7], x1.w, acc[i][1]);
        }
        ++cf;
        const bool row_end = ++cc == cpr;
        if (row_end || cf == fb) {
#pragma unroll
          for (int i = 0; i < MT; ++i) {
            const float v = wave_sum(acc[i][0] + acc[i][1]);
            if (lane == 0) atomicAdd(ys + cj * MT + i, v);
            acc[i][0] = acc[i][1] = 0.f;
          }
          if (row_end) {
            cc = 0;
            ++cj;
          }
        }
      }
      // one chunk at a time: MT tokens' x reads of several chunks held at once would not fit
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// The verification GEMV: rows [0, nrows) of the row map against MT staged vectors of K
// columns, in column phases of at most A.xs_floats / MT floats each; every wave takes an even
// share of each phase's (row, chunk) pairs. Returns with ys[row * MT + i] complete (before
// 1/rms) and wave 0 running `epi`.
template <int MT, class RM, class StageF, class EpiF>
__device__ __forceinline__ bool run_gemv_m(const EngineArgs& A, Blk& b, const TaskDesc& t, const RM& rm, int nrows, int K,
                                           StageF&& stage_of, EpiF&& epi) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int cfull = (K + kChunkCols - 1) / kChunkCols;
  const int cph_max = A.xs_floats / (MT * kChunkCols);  // chunks per phase (the planner keeps it >= 1)
  const int nph = (cfull + cph_max - 1) / cph_max;
  StreamM<MT> s;
  u4 buf[2][NB];
  auto phase_range = [&](int p, int& ca, int& cb) {
    ca = (int)((int64_t)cfull * p / nph);
    cb = (int)((int64_t)cfull * (p + 1) / nph);
  };
  auto start = [&](int p) {
    int ca, cb;
    phase_range(p, ca, cb);
    const int nf = nrows * (cb - ca), fa = wave_start(nf, wave), fb = wave_start(nf, wave + 1);
    s.init(b.rowp, fa, fb, K, ca, cb, (cb - ca) * kChunkCols, lane);
    s.load(buf[0]);
    s.load(buf[1]);
  };
  // row pointers of every row (each wave writes a share; the staging barrier publishes them)
  for (int j = (int)threadIdx.x; j < nrows; j += kThreads) b.rowp[j] = (uint64_t)(uintptr_t)rm.row(j);
  __syncthreads();
  int ca0, cb0;
  phase_range(0, ca0, cb0);
  const auto st0 = stage_of(ca0, cb0);
  if (threadIdx.x < 64) st0.before(b);
  start(0);
  if (!wait_deps(A, b, t, 0, -1, [&] { st0.early(b); })) return false;
  for (int i = threadIdx.x; i < nrows * MT; i += kThreads) b.ys[i] = 0.f;  // (the staging barrier orders this)
  st0.finish(b);
  for (int p = 0; p < nph; ++p) {
    if (p > 0) {
      __syncthreads();  // every wave is done with the previous phase's columns
      int ca, cb;
      phase_range(p, ca, cb);
      start(p);
      // (a short copy is wave 0's, issued in early(): during the wait for phase 0, here now)
      const auto st = stage_of(ca, cb);
      if (threadIdx.x < 64) st.early(b);
      st.finish(b);
    }
    while (s.cf < s.fb) {
      s.consume(buf[0], b.xs, b.ys);
      s.load(buf[0]);
      if (s.cf >= s.fb) break;
      s.consume(buf[1], b.xs, b.ys);
      s.load(buf[1]);
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) epi();
  return true;
}

template <int MT>
__device__ __forceinline__ float token_norm(const Blk& b, int tk) { return token_norms(b)[tk]; }

template <int MT>
__device__ __forceinline__ bool task_qkv_v(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int K = A.hidden, hd = A.hd, hh = hd / 2, r = A.nq / A.nkv, g = t.a0;
  const RmQKV rm{wp<uint8_t>(A, L.w[LW_WQ]), wp<uint8_t>(A, L.w[LW_WK]), wp<uint8_t>(A, L.w[LW_WV]), g, r, hd, hh, K, t.u0};
  const int xin = L.act[LA_X_IN];
  return run_gemv_m<MT>(
      A, b, t, rm, 2 * (t.u1 - t.u0), K,
      [&](int ca, int cb) {
        return StageM<MT>{xin, K, b.x, K, ca * kChunkCols, K, pad512(K), wp<uint16_t>(A, L.w[LW_ATTN_NORM]), A.eps, false};
      },
      [&] {
        const int n = b.n;
        const size_t nslot = (size_t)A.kv_len + MT;
        const size_t lay = (size_t)2 * A.nkv * nslot * hd;  // cache elements per layer
        const rsrc_t kvr = make_rsrc(A.kv + (size_t)t.layer * lay, (uint32_t)(lay * 2));
        for (int e = threadIdx.x; e < (t.u1 - t.u0) * MT; e += 64) {
          const int i = e / MT, tk = e - i * MT;
          const int u = t.u0 + i, slot = u / hh, k = u - slot * hh;
          const float nv = token_norm<MT>(b, tk);
          float a = b.ys[(2 * i) * MT + tk] * nv, c = b.ys[(2 * i + 1) * MT + tk] * nv;
          if (slot <= r) {  // RoPE at the token's position (row tk of the table)
            const float* rope = b.rope + (size_t)tk * 2 * A.rope_half;
            const float cs = rope[k], sn = rope[A.rope_half + k];
            const float a2 = a * cs - c * sn;
            c = c * cs + a * sn;
            a = a2;
          }
          if (slot < r) {
            const uint32_t q = (uint32_t)(L.act[LA_Q] + tk * A.nq * hd + (g * r + slot) * hd);
            cst(b.act, (q + k) * 4u, a);
            cst(b.act, (q + k + hh) * 4u, c);
          } else {
            const int sel = slot - r;  // 0: k, 1: v
            const uint32_t kn = (uint32_t)(L.act[LA_KVNEW] + tk * 2 * A.nkv * hd + (sel * A.nkv + g) * hd);
            cst(b.act, (kn + k) * 4u, a);
            cst(b.act, (kn + k + hh) * 4u, c);
            const uint32_t row = (uint32_t)(((size_t)(sel * A.nkv + g) * nslot + n + tk) * hd);
            cst16(kvr, (row + k) * 2u, f2bf(a));
            cst16(kvr, (row + k + hh) * 2u, f2bf(c));
          }
        }
      });
}

// Causal split-K attention of one KV group for MT tokens over positions [p0, p1) of the
// n + MT positions (the block's own positions at n .. n + MT - 1). Of the group's C = MT * r
// query columns (column c: token c / r, head c % r of the group), the task takes the R columns
// from c0 = a5 * R on (a plan with C > R gives each split ceil(C / R) tasks); they share every
// K/V load, as in task_attn: lane groups of hd / 8 lanes hold a position's row, base-2 online
// softmax per column. Cached positions (< n) are seen by every column; block position n + j
// only by the columns of tokens i >= j. The partial (m, l, 2 pad, acc[hd]) of each column goes
// to its row of the split's record [C][hd + 4].
template <int MT, int R, int LPP>
__device__ __forceinline__ bool task_attn_v(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  constexpr int GPW = 64 / LPP, NP = 2, PER_BLK = NP * GPW;
  const LayerDesc& L = A.layers[t.layer];
  const int hd = LPP * 8, r = A.nq / A.nkv, g = t.a0, n = b.n;
  const int C = MT * r, c0 = t.a5 * R, nc = C - c0 < R ? C - c0 : R;  // this task's columns
  const int n1 = A.kv_len + MT;  // cache slots per (layer, K/V, head)
  const int wave = wave_id(), lane = threadIdx.x & 63, grp = lane / LPP, sub = lane - grp * LPP;
  const int p0 = t.u0, np = t.u1 - t.u0;
  const int q0 = p0 + wave_start(np, wave), q1 = p0 + wave_start(np, wave + 1);
  const int qc = q1 < n ? q1 : n;  // cached positions [q0, qc)
  const uint16_t* Kb = A.kv + (((size_t)t.layer * 2 + 0) * A.nkv + g) * (size_t)n1 * hd;
  const uint16_t* Vb = A.kv + (((size_t)t.layer * 2 + 1) * A.nkv + g) * (size_t)n1 * hd;
  const int nblk = (qc > q0) ? (qc - q0 + PER_BLK - 1) / PER_BLK : 0;
  const rsrc_t kr = make_rsrc(Kb, (uint32_t)((qc > 0 ? qc : 0) * hd * 2)), vr = make_rsrc(Vb, (uint32_t)((qc > 0 ? qc : 0) * hd * 2));
  const uint32_t lo = (uint32_t)(((q0 + grp) * hd + sub * 8) * 2);
  u4 ka[NP], va[NP], kb[NP], vb[NP];
  auto load = [&](int blk, u4(&kk)[NP], u4(&vv)[NP]) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int so = (blk * NP + i) * GPW * hd * 2;
      kk[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, lo, so, kNT);
      vv[i] = __builtin_amdgcn_raw_buffer_load_b128(vr, lo, so, kNT);
    }
  };
  load(0, ka, va);
  load(1, kb, vb);
  if (!wait_deps(A, b, t)) return false;
  // the R query vectors, scaled by softmax scale * log2(e), into LDS (xs: the split record is
  // assembled there only after every wave is done with them); columns past the task's nc repeat
  // its last one and are never seen
  float* qs = b.xs;
  if (threadIdx.x < 64) {
    for (int j = 0; j < R; ++j) {
      const int c = c0 + (j < nc ? j : nc - 1), tk = c / r, h = c - tk * r;
      dma_to_lds(qs + j * hd, b.actp + L.act[LA_Q] + tk * A.nq * hd + (g * r + h) * hd, hd);
    }
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < R * hd; i += kThreads) qs[i] *= A.attn_scale_log2;
  __syncthreads();
  float m[R], l[R], acc[R][8];
#pragma unroll
  for (int h = 0; h < R; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[h][d] = 0.f;
  }
  // fold one block in; `vis` = the last block position (relative to n) column c may see
  // (columns of token i see block positions up to n + i; cached positions are all visible)
  auto step = [&](int base, int lo_, int hi_, const u4(&kk)[NP], const u4(&vv)[NP]) {
    float s[R][NP];
    int qo = sub * 8;
    asm volatile("" : "+v"(qo));
#pragma unroll
    for (int h = 0; h < R; ++h) {
      const float* qh = qs + h * hd + qo;
      const f4 qa = *(const f4*)qh, qb = *(const f4*)(qh + 4);
      const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const u4 kw = kk[i];
        const float kf[8] = {bf_lo(kw.x), bf_hi(kw.x), bf_lo(kw.y), bf_hi(kw.y), bf_lo(kw.z), bf_hi(kw.z), bf_lo(kw.w), bf_hi(kw.w)};
        float p = 0.f;
#pragma unroll
        for (int d = 0; d < 8; ++d) p = fmaf(qv[d], kf[d], p);
        s[h][i] = p;
      }
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int pos = base + i * GPW + grp;
      const bool valid = pos >= lo_ && pos < hi_;
#pragma unroll
      for (int h = 0; h < R; ++h) {
        const float p = group_sum<LPP>(s[h][i]);
        // a block position n + j is visible to the columns of tokens j and later
        const bool seen = valid && h < nc && (pos < n || pos - n <= (c0 + h) / r);
        s[h][i] = seen ? p : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < R; ++h) {
      float mb = s[h][0];
#pragma unroll
      for (int i = 1; i < NP; ++i) mb = fmaxf(mb, s[h][i]);
      const float mn = fmaxf(m[h], mb);
      const float mr = (mn == -INFINITY) ? 0.f : mn;
      const float alpha = ex2(m[h] - mr);
      l[h] *= alpha;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[h][d] *= alpha;
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const float p = ex2(s[h][i] - mr);
        l[h] += p;
        const u4 vw = vv[i];
        acc[h][0] = fmaf(p, bf_lo(vw.x), acc[h][0]);
        acc[h][1] = fmaf(p, bf_hi(vw.x), acc[h][1]);
        acc[h][2] = fmaf(p, bf_lo(vw.y), acc[h][2]);
        acc[h][3] = fmaf(p, bf_hi(vw.y), acc[h][3]);
        acc[h][4] = fmaf(p, bf_lo(vw.z), acc[h][4]);
        acc[h][5] = fmaf(p, bf_hi(vw.z), acc[h][5]);
        acc[h][6] = fmaf(p, bf_lo(vw.w), acc[h][6]);
        acc[h][7] = fmaf(p, bf_hi(vw.w), acc[h][7]);
      }
      m[h] = mn;
    }
  };
  for (int blk = 0; blk < nblk; blk += 2) {
    step(q0 + blk * PER_BLK, q0, qc, ka, va);
    load(blk + 2, ka, va);
    __builtin_amdgcn_sched_barrier(0);
    step(q0 + (blk + 1) * PER_BLK, q0, qc, kb, vb);
    load(blk + 3, kb, vb);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the block's own positions in this wave's range, one at a time (agent-coherent loads: other
  // workgroups wrote them in this step)
  const rsrc_t kn = make_rsrc(Kb, (uint32_t)(n1 * hd * 2)), vn = make_rsrc(Vb, (uint32_t)(n1 * hd * 2));
  for (int pj = (q0 > n ? q0 : n); pj < q1; ++pj) {
    const uint32_t off = (uint32_t)(pj * hd + sub * 8) * 2u;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      ka[i] = __builtin_amdgcn_raw_buffer_load_b128(kn, off, 0, kCoh);
      va[i] = __builtin_amdgcn_raw_buffer_load_b128(vn, off, 0, kCoh);
    }
    step(pj, pj, pj + 1, ka, va);
  }
  // merge the wave's lane groups, then the waves, into the split record (as task_attn)
#pragma unroll 1
  for (int X = LPP; X < 64; X <<= 1) {
#pragma unroll
    for (int h = 0; h < R; ++h) {
      const float om = __shfl_xor(m[h], X, 64), ol = __shfl_xor(l[h], X, 64);
      const float M = fmaxf(m[h], om);
      const float ca = (m[h] == -INFINITY) ? 0.f : exp2f(m[h] - M);
      const float cb = (om == -INFINITY) ? 0.f : exp2f(om - M);
      l[h] = l[h] * ca + ol * cb;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[h][d] = acc[h][d] * ca + __shfl_xor(acc[h][d], X, 64) * cb;
      m[h] = M;
    }
  }
  constexpr int ps = LPP * 8 + 4, SS = R * ps;
  if (grp == 0) {
    float* gp = b.scr + wave * SS;
#pragma unroll
    for (int h = 0; h < R; ++h) {
      if (sub == 0) {
        gp[h * ps] = m[h];
        gp[h * ps + 1] = l[h];
      }
#pragma unroll
      for (int d = 0; d < 8; ++d) gp[h * ps + 4 + sub * 8 + d] = acc[h][d];
    }
  }
  __syncthreads();
#pragma unroll 1
  for (int i = threadIdx.x; i < nc * hd; i += kThreads) {
    const int h = i / hd, d = i - h * hd;
    float M = -INFINITY;
#pragma unroll
    for (int sl = 0; sl < kWaves; ++sl) M = fmaxf(M, b.scr[sl * SS + h * ps]);
    float v = 0.f, den = 0.f;
#pragma unroll
    for (int sl = 0; sl < kWaves; ++sl) {
      const float ms = b.scr[sl * SS + h * ps];
      const float e = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
      v = fmaf(e, b.scr[sl * SS + h * ps + 4 + d], v);
      den = fmaf(e, b.scr[sl * SS + h * ps + 1], den);
    }
    b.xs[h * ps + 4 + d] = v;
    if (d == 0) *reinterpret_cast<f4*>(b.xs + h * ps) = f4{M, den, 0.f, 0.f};
  }
  __syncthreads();
  const uint32_t gpart = (uint32_t)(t.a4 + (t.a1 * C + c0) * ps);
  if (threadIdx.x < 64)
    for (int i = threadIdx.x * 4; i < nc * ps; i += 256) cst4(b.act, (gpart + i) * 4u, *(const f4*)(b.xs + i));
  return true;
}

template <int MT>
__device__ __forceinline__ bool task_attn_v_hd(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  constexpr int R = kMaxVerifyCols;  // query columns per task (held per lane)
  switch (A.hd) {
    case 32: return task_attn_v<MT, R, 4>(A, b, t);
    case 64: return task_attn_v<MT, R, 8>(A, b, t);
    case 128: return task_attn_v<MT, R, 16>(A, b, t);
    default: return task_attn_v<MT, R, 32>(A, b, t);
  }
}

// Merge of a group's split records for the MT tokens (columns c = token * r + head) into the
// per-token O-projection inputs xs[token * pw + head * hd + d] (zero-padded to pw), staged like
// StageMerge; the first task of the group also stores the attention output of every token.
template <int MT>
struct StageMergeM {
  int parts_off, S, r, hd, pw, o_off, o_stride;  // o_off < 0: no store
  __device__ __forceinline__ int n() const { return S * MT * r * (hd + 4); }
  __device__ __forceinline__ void before(Blk&) const {}
  __device__ __forceinline__ void early(Blk& b) const {  // wave 0
    if (n() <= kEarlyDmaFloats) dma_to_lds(b.scr, b.actp + parts_off, n());
  }
  __device__ __forceinline__ void finish(Blk& b) const {
    const int H = MT * r, ps = hd + 4, nf = n();
    float* P = b.scr;                      // [S][H][ps]
    float* w = P + ((nf + 255) & ~255);   // [S][H] merge weights
    if (nf > kEarlyDmaFloats) dma_to_lds_all(P, b.actp + parts_off, nf);
    else if (threadIdx.x < 64) __builtin_amdgcn_s_waitcnt(kVmcnt0);
    for (int i = threadIdx.x; i < MT * pw; i += kThreads)
      if (i - (i / pw) * pw >= r * hd) b.xs[i] = 0.f;
    __syncthreads();
    for (int h = wave_id(); h < H; h += kWaves) {
      const int lane = threadIdx.x & 63;
      float M = -INFINITY;
      for (int sp = lane; sp < S; sp += 64) M = fmaxf(M, P[(sp * H + h) * ps]);
#pragma unroll
      for (int k = 1; k < 64; k <<= 1) M = fmaxf(M, __shfl_xor(M, k, 64));
      float den = 0.f;
      for (int sp = lane; sp < S; sp += 64) den += exp2f(P[(sp * H + h) * ps] - M) * P[(sp * H + h) * ps + 1];
      den = wave_sum(den);
      const float inv = 1.0f / den;
      for (int sp = lane; sp < S; sp += 64) w[sp * H + h] = exp2f(P[(sp * H + h) * ps] - M) * inv;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < H * hd; i += kThreads) {
      const int h = i / hd, d = i - h * hd;
      float v = 0.f;
      for (int sp = 0; sp < S; ++sp) v = fmaf(w[sp * H + h], P[(sp * H + h) * ps + 4 + d], v);
      const int tk = h / r;
      b.xs[tk * pw + (h - tk * r) * hd + d] = v;
    }
    if (threadIdx.x < MT) token_norms(b)[threadIdx.x] = 1.f;
    __syncthreads();
    if (o_off >= 0 && threadIdx.x < 64)
      for (int tk = 0; tk < MT; ++tk)
        for (int i = threadIdx.x * 4; i < r * hd; i += 256)
          cst4(b.act, (uint32_t)(o_off + tk * o_stride + i) * 4u, *(const f4*)(b.xs + tk * pw + i));
  }
};

template <int MT>
__device__ __forceinline__ bool task_oproj_g_v(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int r = A.nq / A.nkv, hd = A.hd, g = t.a0, K = r * hd;
  const RmCols rm{wp<uint8_t>(A, L.w[LW_WO]), A.nq * hd, t.u0, g * K};
  return run_gemv_m<MT>(
      A, b, t, rm, t.u1 - t.u0, K,
      [&](int, int) {
        return StageMergeM<MT>{t.a4, t.a2, r, hd, pad512(K), t.u0 == 0 ? L.act[LA_ATTN] + g * K : -1, A.nq * hd};
      },
      [&] {
        for (int e = threadIdx.x; e < (t.u1 - t.u0) * MT; e += 64) {
          const int i = e / MT, tk = e - i * MT;
          __hip_atomic_fetch_add(b.actp + L.act[LA_H] + tk * A.hidden + t.u0 + i, b.ys[e], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        }
      });
}

// Layer 0: h[token] = x[token] (widened), the accumulators the per-group O-projections add into.
template <int MT>
__device__ __forceinline__ bool task_hinit_v(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  for (int tk = 0; tk < MT; ++tk)
    for (int i = threadIdx.x; i < t.u1 - t.u0; i += kThreads)
      cst(b.act, (uint32_t)(t.a0 + tk * A.hidden + t.u0 + i) * 4u, bf16f(b.x[(size_t)tk * A.hidden + t.u0 + i]));
  return true;
}

template <int MT>
__device__ __forceinline__ bool task_gateup_v(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int K = A.hidden;
  const RmGateUp rm{wp<uint8_t>(A, L.w[LW_GATE]), wp<uint8_t>(A, L.w[LW_UP]), K, t.u0};
  return run_gemv_m<MT>(
      A, b, t, rm, 2 * (t.u1 - t.u0), K,
      [&](int ca, int) {
        return StageM<MT>{L.act[LA_H], K, nullptr, K, ca * kChunkCols, K, pad512(K), wp<uint16_t>(A, L.w[LW_FFN_NORM]), A.eps, true};
      },
      [&] {
        for (int e = threadIdx.x; e < (t.u1 - t.u0) * MT; e += 64) {
          const int i = e / MT, tk = e - i * MT;
          const float nv = token_norm<MT>(b, tk);
          const float gv = b.ys[(2 * i) * MT + tk] * nv, uv = b.ys[(2 * i + 1) * MT + tk] * nv;
          cst(b.act, (uint32_t)(L.act[LA_ACT] + tk * A.ffn + t.u0 + i) * 4u, silu(gv) * uv);
        }
      });
}

template <int MT>
__device__ __forceinline__ bool task_down_v(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const LayerDesc& L = A.layers[t.layer];
  const int K = A.ffn;
  const RmPlain rm{wp<uint8_t>(A, L.w[LW_DOWN]), K, t.u0};
  return run_gemv_m<MT>(
      A, b, t, rm, t.u1 - t.u0, K,
      [&](int ca, int cb) {
        const int k0 = ca * kChunkCols, k1 = cb * kChunkCols < K ? cb * kChunkCols : K;
        return StageM<MT>{L.act[LA_ACT], K, nullptr, K, k0, k1 - k0, (cb - ca) * kChunkCols, nullptr, 0.f, false};
      },
      [&] {
        for (int e = threadIdx.x; e < (t.u1 - t.u0) * MT; e += 64) {
          const int i = e / MT, tk = e - i * MT, rr = t.u0 + i, d = A.hidden;
          const float y = b.ys[e];
          const float xo = cld_coh(b.act, (uint32_t)(L.act[LA_H] + tk * d + rr) * 4u) + y;
          cst(b.act, (uint32_t)(L.act[LA_FFN_OUT] + tk * d + rr) * 4u, y);
          if (t.a1 >= 0) cst(b.act, (uint32_t)(t.a1 + tk * d + rr) * 4u, xo);  // next layer's h starts at x
          cst(b.act, (uint32_t)(L.act[LA_X_OUT] + tk * d + rr) * 4u, xo);
          if (t.a0) A.out[(size_t)tk * d + rr] = xo;
        }
      });
}

template <int MT>
__device__ __forceinline__ bool task_lmhead_v(const EngineArgs& A, Blk& b, const TaskDesc& t) {
  const int K = A.hidden;
  const RmPlain rm{wp<uint8_t>(A, A.w_lm_head), K, t.u0};
  return run_gemv_m<MT>(
      A, b, t, rm, t.u1 - t.u0, K,
      [&](int ca, int) {
        return StageM<MT>{A.x_final, K, nullptr, K, ca * kChunkCols, K, pad512(K), wp<uint16_t>(A, A.w_final_norm), A.eps, false};
      },
      [&] {
        for (int e = threadIdx.x; e < (t.u1 - t.u0) * MT; e += 64) {
          const int i = e / MT, tk = e - i * MT;
          A.out[(size_t)tk * A.vocab + t.u0 + i] = b.ys[e] * token_norm<MT>(b, tk);
        }
      });
}

}  // namespace

// ------------------------------------------------------------------ the engine

// The task walk, instantiated once per model family so that each kernel's register
// allocation covers only the task types it runs: GQA (MLA = false) and MLA / MLA + MoE.
// What one launch runs: a whole step of a fixed-length plan (the product path), a range of
// stages of one, or a whole step of a plan with a per-step length. Each is its own kernel, so
// the one-launch step carries none of the others' code.
enum RunKind : int { kRunStep = 0, kRunStages = 1, kRunDynamic = 2 };

// The kernel argument block, re-read through a pointer the compiler cannot see through: each
// task loads the arguments it uses (scalar loads, cached) instead of keeping every argument
// of the persistent loop live in scalar registers.
__device__ __forceinline__ const EngineArgs& args_view() {
  typedef const EngineArgs __attribute__((address_space(4)))* CArgsP;
  CArgsP p = (CArgsP)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return *(const EngineArgs*)p;
}

// ES: the weights' element format -- GQA: every linear matrix (2 bf16, 1 FP8); latent family:
// 2 bf16, 1 FP8 (every linear matrix but the absorption matrices and the router), 0 MXFP4
// experts (every other matrix bf16).
// IDX: the latent family with the sparse indexer (its tasks are compiled into their own kernels,
// so the dense kernels' register allocation does not carry them).
template <bool MLA, int RUN, int ES = 2, int MT = 1, bool IDX = false>
__device__ __forceinline__ void engine_body(const EngineArgs& A) {
  constexpr int ED = ES == 1 ? 1 : 2;  // the latent family's non-expert matrices
  extern __shared__ f4 lds4[];
  float* lds = reinterpret_cast<float*>(lds4);
  Blk b;
  b.flags = reinterpret_cast<int*>(lds);
  b.xs = lds + 64;
  b.ys = b.xs + A.xs_floats;
  b.rowp = reinterpret_cast<uint64_t*>(b.ys + kYsFloats);
  b.xoffp = reinterpret_cast<int*>(b.rowp + kMaxTaskRows);
  b.scl = reinterpret_cast<float*>(b.xoffp + kMaxTaskRows);
  b.srowp = reinterpret_cast<uint64_t*>(b.scl);  // (MXFP4 scale pointers: in place of the FP8 scales)
  b.gs = b.scl + (ES == 1 ? kMaxTaskRows : ES == 0 ? 2 * kMaxTaskRows : 0);
  b.scr = b.gs + A.gs_floats;
  b.actp = A.act;
  b.act = make_rsrc(A.act, A.act_bytes);
  b.epoch = ld_agent(A.ctl + CTL_EPOCH);
  b.t_ready = b.t_staged = b.t_streamed = 0;
  b.t_sub[0] = b.t_sub[1] = b.t_sub[2] = 0;
  b.n = A.kv_len;
  b.x = A.x;
  b.rope = A.rope_cs;
  if constexpr (RUN == kRunDynamic) {
    // the step's position (and, without an input vector, its token), written by the
    // previous step's last workgroup or by the caller; every workgroup reads the same values
    // and, if they are out of range, the whole step does nothing (sticky status 8)
    // (wave-uniform values: every lane loads the same word; readfirstlane lets the compiler
    // keep them, and everything computed from them, in scalar registers)
    const int n = __builtin_amdgcn_readfirstlane((int)ld_agent(reinterpret_cast<const uint32_t*>(A.state)));
    const int tok = __builtin_amdgcn_readfirstlane((int)ld_agent(reinterpret_cast<const uint32_t*>(A.state) + 1));
    if (n < 0 || n > A.kv_len || (!A.x && (tok < 0 || tok >= A.vocab))) {
      if (blockIdx.x == 0 && threadIdx.x == 0) {
        uint32_t zero = 0;
        if (__hip_atomic_compare_exchange_strong(A.ctl + CTL_STATUS, &zero, 8u, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)) {
          st_agent(A.ctl + CTL_STATUS + 1, (uint32_t)n);
          st_agent(A.ctl + CTL_STATUS + 2, (uint32_t)tok);
        }
      }
      return;
    }
    b.n = n;
    if (!A.x) b.x = wp<uint16_t>(A, A.w_embed) + (size_t)tok * A.hidden;
    b.rope = A.rope_cs + (size_t)n * 2 * A.rope_half;
  }
  const uint32_t xcc = xcc_id();
  const int wg = blockIdx.x;
  const int rq = A.nkv > 0 ? A.nq / A.nkv : 1;
  // a launch runs the tasks of stages [stage_lo, stage_hi) of this workgroup's list; a step is
  // one launch of all stages, or launches of consecutive ranges in order (every dependency
  // lies in an earlier stage, so a one-stage launch never waits on its own tasks)
  const bool all_stages = RUN != kRunStages || (A.stage_lo == 0 && A.stage_hi == A.n_stages);
  int ti0 = A.wg_begin[wg], ti1 = A.wg_begin[wg + 1];
  if (RUN == kRunStages && !all_stages) {
    const int32_t* sf = A.stage_first + (size_t)wg * (A.n_stages + 1);
    ti0 = sf[A.stage_lo];
    ti1 = sf[A.stage_hi];
  }
  for (int ti = ti0; ti < ti1; ++ti) {
    const EngineArgs& A = args_view();
    const TaskDesc t = A.tasks[ti];
    const uint32_t t0 = (kTaskLog && threadIdx.x < 64) ? (uint32_t)now() : 0u;
    bool ok = true, gemv = true;
    int sig = t.signal;
    if constexpr (!MLA && MT > 1) {
      // a verification step of MT tokens (GQA, bf16, whole steps)
      switch (t.type) {
        case T_QKV: ok = task_qkv_v<MT>(A, b, t); break;
        case T_ATTN: gemv = false; ok = task_attn_v_hd<MT>(A, b, t); break;
        case T_OPROJ_G: ok = task_oproj_g_v<MT>(A, b, t); break;
        case T_HINIT: gemv = false; ok = task_hinit_v<MT>(A, b, t); break;
        case T_GATEUP: ok = task_gateup_v<MT>(A, b, t); break;
        case T_DOWN: ok = task_down_v<MT>(A, b, t); break;
        case T_LMHEAD: ok = task_lmhead_v<MT>(A, b, t); break;
        default: ok = false; break;
      }
    } else if constexpr (!MLA) {
      switch (t.type) {
        // K/V rows pass from a QKV task to the attention split after it through LDS only when
        // one launch runs both (a launch of all stages)
        case T_QKV: ok = (t.a5 > 0 && all_stages) ? task_qkv<true, ES>(A, b, t) : task_qkv<false, ES>(A, b, t); break;
        case T_ATTN:
          gemv = false;
          if (t.a3 > 0) {
            gemv = true;  // wave 0 alone stores the partial
            switch (A.hd) {
              case 32: ok = task_attn_mfma<32>(A, b, t, !all_stages); break;
              case 64: ok = task_attn_mfma<64>(A, b, t, !all_stages); break;
              case 128: ok = task_attn_mfma<128>(A, b, t, !all_stages); break;
              default: ok = task_attn_mfma<256>(A, b, t, !all_stages); break;
            }
          }
          else ok = rq <= 1 ? task_attn_hd<1>(A, b, t) : rq <= 2 ? task_attn_hd<2>(A, b, t) : task_attn_hd<4>(A, b, t);
          break;
        case T_OPROJ_G: ok = task_oproj_g<ES>(A, b, t); break;
        case T_HINIT: gemv = false; ok = task_hinit(A, b, t); break;
        case T_GATEUP: ok = task_gateup<ES>(A, b, t); break;
        case T_DOWN: ok = task_down<true, ES>(A, b, t); break;
        case T_LMHEAD: ok = task_lmhead<RUN == kRunDynamic, ES>(A, b, t); break;
        case T_ARGMAX:
          gemv = false;
          if constexpr (RUN == kRunDynamic) ok = task_argmax(A, b, t);
          else ok = false;
          break;
        default: ok = false; break;
      }
    } else {
      switch (t.type) {
        case T_MLA_A: ok = task_mla_a<ED, IDX>(A, b, t); break;
        case T_MLA_B: ok = task_mla_b<ED>(A, b, t); break;
        case T_MLA_KVAPP: gemv = false; ok = task_mla_kvapp(A, b, t); break;
        case T_MLA_ABSORB: gemv = false; ok = task_mla_absorb(A, b, t); break;
        case T_MLA_ATTN: gemv = false; ok = task_mla_attn<IDX>(A, b, t); break;
        case T_MLA_UV: gemv = false; ok = task_mla_uv(A, b, t); break;
        case T_OPROJ: ok = task_oproj<ED>(A, b, t); break;
        case T_GATEUP: ok = task_gateup<ED>(A, b, t); break;
        case T_DOWN: ok = task_down<false, ED>(A, b, t); break;
        case T_LMHEAD: ok = task_lmhead<RUN == kRunDynamic, ED>(A, b, t); break;
        case T_ARGMAX:
          gemv = false;
          if constexpr (RUN == kRunDynamic) ok = task_argmax(A, b, t);
          else ok = false;
          break;
        case T_ROUTER: ok = task_router(A, b, t); break;
        case T_SHARED_GU: ok = task_shared_gu<ES>(A, b, t); break;
        case T_TOPK: gemv = false; ok = task_topk(A, b, t); break;
        case T_EXPERT_GU: ok = task_expert_gu<ES>(A, b, t); break;
        case T_MOE_DOWN: ok = task_moe_down<ES>(A, b, t); break;
        case T_IDX_Q:
          if constexpr (IDX) ok = task_idx_q(A, b, t);
          else ok = false;
          break;
        case T_IDX_SCORE:
          gemv = false;
          if constexpr (IDX) ok = task_idx_score(A, b, t);
          else ok = false;
          break;
        case T_IDX_TOPK:
          gemv = false;
          if constexpr (IDX) ok = task_idx_topk(A, b, t);
          else ok = false;
          break;
        default: ok = false; break;
      }
    }
    if (!ok) break;
    const uint32_t t_sig = gemv ? signal_w0(A, sig) : signal(A, sig);
    if (kTaskLog && threadIdx.x == 0) {
      TaskLog* lg = A.log + t.id;
      add_agent(&lg->execs, 1u);
      lg->epoch = b.epoch;
      lg->wg = (uint32_t)wg;
      lg->xcd = xcc;
      lg->t_start = t0;
      lg->t_ready = b.t_ready;
      lg->t_end = kTaskLogDetail ? (uint32_t)now() : 0u;
      lg->t_staged = b.t_staged;
      lg->t_streamed = b.t_streamed;
      lg->t_signal = t_sig;
      lg->t_aux[2] = b.t_sub[0];
      lg->t_aux[3] = b.t_sub[1];
      lg->t_aux[4] = b.t_sub[2];
      b.t_sub[0] = b.t_sub[1] = b.t_sub[2] = 0;
    }
  }
  // the last workgroup to finish the step's last launch advances the epoch for the next step
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  __syncthreads();
  if (threadIdx.x == 0 && (RUN != kRunStages || A.stage_hi == A.n_stages)) {
    const uint32_t d = add_agent(A.ctl + CTL_DONE, 1u);
    if (d == (uint32_t)A.n_wg - 1u) {
      st_agent(A.ctl + CTL_DONE, 0u);
      add_agent(A.ctl + CTL_EPOCH, 1u);
      if constexpr (RUN == kRunDynamic) {  // every workgroup has read the position: advance it
        uint32_t* st = reinterpret_cast<uint32_t*>(A.state);
        st_agent(st, (uint32_t)(b.n + 1));
        st_agent(st + 2, ld_agent(st + 2) + 1u);
      }
    }
  }
}

extern "C" __global__ void __launch_bounds__(kThreads, 1) dec_engine_gqa(EngineArgs A) { engine_body<false, kRunStep>(A); }
extern "C" __global__ void __launch_bounds__(kThreads, 1) dec_engine_mla(EngineArgs A) { engine_body<true, kRunStep>(A); }
extern "C" __global__ void __launch_bounds__(kThreads, 1) dec_engine_gqa_stages(EngineArgs A) {
  engine_body<false, kRunStages>(A);
}
extern "C" __global__ void __launch_bounds__(kThreads, 1) dec_engine_mla_stages(EngineArgs A) {
  engine_body<true, kRunStages>(A);
}
extern "C" __global__ void __launch_bounds__(kThreads, 1) dec_engine_gqa_dyn(EngineArgs A) {
  engine_body<false, kRunDynamic>(A);
}
extern "C" __global__ void __launch_bounds__(kThreads, 1) dec_engine_mla_dyn(EngineArgs A) {
  engine_body<true, kRunDynamic>(A);
}
extern "C" __global__ void __launch_bounds__(kThreads, 1) dec_engine_mla_sp(EngineArgs A) {
  engine_body<true, kRunStep, 2, 1, true>(A);
}
extern "C" __global__ void __launch_bounds__(kThreads, 1) dec_engine_mla_sp_dyn(EngineArgs A) {
  engine_body<true, kRunDynamic, 2, 1, true>(A);
}
extern "C" __global__ void __launch_bounds__(kThreads, 1) dec_engine_mla_f8(EngineArgs A) {
  engine_body<true, kRunStep, 1>(A);
}
extern "C" __global__ void __launch_bounds__(kThreads, 1) dec_engine_mla_f8_dyn(EngineArgs A) {
  engine_body<true, kRunDynamic, 1>(A);
}
extern "C" __global__ void __launch_bounds__(kThreads, 1) dec_engine_mla_x4(EngineArgs A) {
  engine_body<true, kRunStep, 0>(A);
}
extern "C" __global__ void __launch_bounds__(kThreads, 1) dec_engine_mla_x4_dyn(EngineArgs A) {
  engine_body<true, kRunDynamic, 0>(A);
}
extern "C" __global__ void __launch_bounds__(kThreads, 1) dec_engine_gqa_f8(EngineArgs A) {
  engine_body<false, kRunStep, 1>(A);
}
extern "C" __global__ void __launch_bounds__(kThreads, 1) dec_engine_gqa_f8_dyn(EngineArgs A) {
  engine_body<false, kRunDynamic, 1>(A);
}
extern "C" __global__ void __launch_bounds__(kThreads, 1) dec_engine_gqa_v2(EngineArgs A) {
  engine_body<false, kRunStep, 2, 2>(A);
}
extern "C" __global__ void __launch_bounds__(kThreads, 1) dec_engine_gqa_v3(EngineArgs A) {
  engine_body<false, kRunStep, 2, 3>(A);
}
extern "C" __global__ void __launch_bounds__(kThreads, 1) dec_engine_gqa_v4(EngineArgs A) {
  engine_body<false, kRunStep, 2, 4>(A);
}

}  // namespace dec

// Host-side launch (used by the C ABI in api.cpp). run: 0 a whole step, 1 a range of stages,
// 2 a whole step of a plan with a per-step length; ntok > 1: a verification step (run 0).
static const void* engine_fn(int arch, int run, int wfmt = 0, int ntok = 1, bool idx = false) {
  if (idx && arch != 0) return run == 2 ? (const void*)dec::dec_engine_mla_sp_dyn : (const void*)dec::dec_engine_mla_sp;
  if (ntok == 2) return (const void*)dec::dec_engine_gqa_v2;
  if (ntok == 3) return (const void*)dec::dec_engine_gqa_v3;
  if (ntok == 4) return (const void*)dec::dec_engine_gqa_v4;
  if (wfmt == 2) return run == 2 ? (const void*)dec::dec_engine_mla_x4_dyn : (const void*)dec::dec_engine_mla_x4;
  if (wfmt == 1 && arch != 0) return run == 2 ? (const void*)dec::dec_engine_mla_f8_dyn : (const void*)dec::dec_engine_mla_f8;
  if (wfmt) return run == 2 ? (const void*)dec::dec_engine_gqa_f8_dyn : (const void*)dec::dec_engine_gqa_f8;
  if (run == 1) return arch == 0 ? (const void*)dec::dec_engine_gqa_stages : (const void*)dec::dec_engine_mla_stages;
  if (run == 2) return arch == 0 ? (const void*)dec::dec_engine_gqa_dyn : (const void*)dec::dec_engine_mla_dyn;
  return arch == 0 ? (const void*)dec::dec_engine_gqa : (const void*)dec::dec_engine_mla;
}

extern "C" __attribute__((visibility("hidden"))) hipError_t dec_engine_launch(const dec::EngineArgs* args, int n_wg, int lds_bytes,
                                                                         int run, bool cooperative, hipStream_t stream) {
  // the dynamic-LDS limit each kernel has been given so far
  static std::mutex mu;
  static std::map<const void*, int> configured_lds;
  const int k = args->arch == 0 ? 0 : 1;
  const bool idx = args->idx_h > 0;
  // MXFP4 experts and the sparse indexer: the latent family; FP8, MXFP4 or the indexer: no
  // stage launches
  if (run < 0 || run > 2 || (args->wfmt == 2 && k != 1) || ((args->wfmt || idx) && run == 1) || (idx && (k != 1 || args->wfmt)))
    return hipErrorInvalidValue;
  if (args->ntok > 1 && (k != 0 || run != 0 || args->wfmt || args->ntok > dec::kMaxVerifyTokens)) return hipErrorInvalidValue;
  const void* fn = engine_fn(args->arch, run, args->wfmt, args->ntok, idx);
  {
    std::lock_guard<std::mutex> lock(mu);
    int& have = configured_lds.emplace(fn, -1).first->second;
    if (have < lds_bytes) {
      hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
      if (e != hipSuccess) return e;
      have = lds_bytes;
    }
  }
  void* kargs[] = {const_cast<dec::EngineArgs*>(args)};
  if (!cooperative)  // one stage: no task waits on another of the same launch
    return hipLaunchKernel(fn, dim3(n_wg), dim3(dec::kThreads), kargs, (size_t)lds_bytes, stream);
  return hipLaunchCooperativeKernel(fn, dim3(n_wg), dim3(dec::kThreads), kargs, (unsigned)lds_bytes, stream);
}

extern "C" __attribute__((visibility("hidden"))) hipError_t dec_engine_occupancy(int arch, int wfmt, int ntok, int idx,
                                                                               int lds_bytes, int* blocks_per_cu) {
  const void* fn = engine_fn(arch, 0, wfmt, ntok, idx != 0);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, dec::kThreads, (size_t)lds_bytes);
}

// ------------------------------------------------------------------ stream-read ceiling
//
// The HBM read rate this part reaches with the engine's access pattern, as a reference for
// the step's achieved bandwidth: every workgroup (one per CU, 8 waves) streams a contiguous
// share of a buffer with 16-byte non-temporal loads, two batches of eight 1-KB wave loads in
// flight per wave (the engine's weight ring), and folds what it reads into one word per
// thread so that no load is dropped.
namespace dec {
__global__ void __launch_bounds__(kThreads, 1) dec_stream_read_kernel(const u4* buf, int64_t n16, uint32_t* sink) {
  const int64_t per_wg = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per_wg, hi = lo + per_wg < n16 ? lo + per_wg : n16;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t acc = 0;
  // chunk c of the workgroup's share: 64 consecutive 16-byte words; wave w takes chunks w, w + 8, ...
  const int64_t nchunk = hi > lo ? (hi - lo + 63) / 64 : 0;
  auto addr = [&](int64_t c) {
    int64_t i = lo + c * 64 + lane;
    return buf + (i < hi ? i : hi - 1);
  };
  u4 a[NB], b[NB];
  int64_t c = wave;
  auto load = [&](u4 (&r)[NB], int64_t c0) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int64_t ck = c0 + (int64_t)k * kWaves;
      r[k] = ck < nchunk ? ldg_nt(addr(ck)) : u4{0u, 0u, 0u, 0u};
    }
  };
  auto fold = [&](const u4 (&r)[NB]) {
#pragma unroll
    for (int k = 0; k < NB; ++k) acc += r[k].x ^ r[k].y ^ r[k].z ^ r[k].w;
  };
  load(a, c);
  load(b, c + (int64_t)NB * kWaves);
  for (; c < nchunk; c += (int64_t)2 * NB * kWaves) {
    fold(a);
    load(a, c + (int64_t)2 * NB * kWaves);
    fold(b);
    load(b, c + (int64_t)3 * NB * kWaves);
  }
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}
}  // namespace dec

// One stream-read launch over `bytes` (a multiple of 16) at `buf`, n_wg workgroups; `sink`
// receives n_wg * 512 words.
extern "C" __attribute__((visibility("hidden"))) hipError_t dec_stream_read_launch(const void* buf, int64_t bytes, int n_wg,
                                                                                 uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(dec::dec_stream_read_kernel, dim3(n_wg), dim3(dec::kThreads), 0, stream,
                     static_cast<const dec::u4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

// ------------------------------------------------------------------ the static workspace
//
// For callers that cannot allocate device memory (code under stream capture, serving loops,
// harnesses that forbid allocation): one workspace per GPU in a file-scope device array, which
// dec_plan_bind_scratch binds a plan to instead of a caller-allocated workspace. Each GPU the
// library runs on holds its copy until the process ends. Host code never passes the array's
// name to the device: it uses the address hipGetSymbolAddress returns for the current device,
// looked up once per device and kept.
namespace {
constexpr size_t kScratchBytes = (size_t)64 << 20;  // 64 MiB: the 8B model's plan needs 30 MB, the MLA model's 39 MB
static __device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// The current device's copy of the static workspace: its device address and size.
extern "C" __attribute__((visibility("hidden"))) hipError_t dec_scratch_current(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = kScratchBytes;
  return hipSuccess;
}
