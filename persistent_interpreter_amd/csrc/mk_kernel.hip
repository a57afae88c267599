// mk_kernel.hip -- the persistent decode megakernel for gfx950 (MI355X).
//
// One workgroup per compute unit runs an interpreter over the queue of
// instructions the host planned for it (megakernel chapter "L'interpréteur
// sur GPU", section 3.2).  Dependencies between instructions on different
// compute units are counters in global memory that producers increment and
// consumers wait on (section 3.4).  Weights of the upcoming instructions
// stream into a ring of 16 KB LDS pages while the current instruction
// computes or waits (section 3.3: pages freed by one instruction are refilled
// for the next at once).
//
// Roles of the waves of a workgroup (the loader/compute/storer split of the
// section 3.2 template, recast for CDNA4, which has no TMA and no warp
// specialisation hardware):
//   * 3 loader waves (kNLW) walk the queue's weight streams in order and copy them
//     global -> LDS with direct-to-LDS 128-bit loads, several pages in
//     flight, refilling a page as soon as every compute wave released it;
//   * 1 sync wave walks the same queue, waits on each instruction's counter
//     groups, and writes the instruction's fp32 input vector (the RMSNorm'd
//     residual, the attention output or an MLP chunk) into a small LDS ring;
//   * 8 compute waves walk the same queue, take the pages' rows in turn,
//     do the dot products and the instruction's epilogue, and the last wave
//     to finish an instruction increments its counter groups.
//
// Cross-CU data (activations, partials, the new K/V slot) is written and
// read with device-coherent (sc1) accesses and counters are incremented only
// after the writer's stores completed (s_waitcnt vmcnt(0)); no L2-wide
// writeback or invalidate is used.  Every wait is bounded by a watchdog.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "mk_layout.hpp"
#include "mk_plan.hpp"

namespace mk {

typedef unsigned u4 __attribute__((ext_vector_type(4)));
// Global memory is always accessed through address-space-1 pointers: a
// generic (flat) access would count against the LDS wait counter too, so a
// later wait for an LDS flag would stall until a global store is
// acknowledged.
#define GAS __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ GAS T *G(T *p) { return (GAS T *)p; }
template <class T>
__device__ __forceinline__ const GAS T *G(const T *p) { return (const GAS T *)p; }
typedef float f4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

extern "C" __shared__ __align__(16) char smem[];

__device__ __forceinline__ uint32_t &lds_u32(int off) { return *reinterpret_cast<uint32_t *>(smem + off); }

// --------------------------------------------------------------------------
// bf16 helpers
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Step s of a launch (step_off = s) runs with the launch's epoch, tag and
// greedy target moved on by s, and writes logits row block s.  Only
// step_off changes between steps: every other argument stays the launch's
// own, which the compiler may re-load instead of keeping in registers.
__device__ __forceinline__ uint32_t step_tag(const Args &a) { return a.tag + (uint32_t)a.step_off; }
__device__ __forceinline__ uint32_t step_epoch(const Args &a) { return a.epoch + (uint32_t)a.step_off; }
__device__ __forceinline__ uint32_t step_amax_target(const Args &a) {
  return a.amax_target + (uint32_t)a.step_off * a.n_lm;
}
__device__ __forceinline__ float *step_logits(const Args &a) {
  return a.logits + (size_t)a.step_off * (size_t)a.batch * (size_t)a.ctx->V;
}

// --------------------------------------------------------------------------
// device-coherent accesses (relaxed agent-scope atomics -> sc1)
__device__ __forceinline__ float ld_c(const float *p) {
  return __uint_as_float(__hip_atomic_load(G(reinterpret_cast<const uint32_t *>(p)), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ float2 ld_c2(const float *p) {
  uint64_t v = __hip_atomic_load(G(reinterpret_cast<const uint64_t *>(p)), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}
__device__ __forceinline__ void st_c(float *p, float v) {
  __hip_atomic_store(G(reinterpret_cast<uint32_t *>(p)), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_c16(uint16_t *p, uint16_t v) {
  __hip_atomic_store(G(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint16_t ld_c16(const uint16_t *p) {
  return __hip_atomic_load(G(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_cu(const uint32_t *p) {
  return __hip_atomic_load(G(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Non-atomic device-coherent (sc1) loads/stores through buffer resources:
// the same cache policy as the atomics above, but the compiler may keep many
// in flight.  Ordering against counters/flags is explicit (waitcnt, LDS
// flags, compiler barriers around the waits).
constexpr int kSC1 = 16;  // cache-policy bits: sc1
// The weight stream is read once per step: nontemporal loads keep it from
// displacing the activations, partials and counters in the caches (3 % per
// step on the Llama-1B shape).
#ifndef MK_WPOL
#define MK_WPOL 2
#endif
constexpr int kWPol = MK_WPOL;  // cache-policy bits of the weight stream (2 = nt)
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t rsrc(const void *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ f4 ldc4(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSC1));
}
__device__ __forceinline__ u4 ldc4u(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSC1));
}
__device__ __forceinline__ float ldc1(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kSC1));
}
__device__ __forceinline__ uint16_t ldc16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kSC1);
}

// Tagged activation words: value in the low half, the step's tag in the
// high half, written as one 64-bit store.  Each word is its own flag: the
// producer (a QKV epilogue: q and the new K/V slot) stores them with no
// counter and no wait for their acknowledgement, and a consumer re-reads any
// word whose tag is not yet this step's.
__device__ __forceinline__ void st_tag(uint64_t *p, float v, uint32_t tag) {
  __hip_atomic_store(G(p), ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ldt(rsrc_t r, uint32_t word) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, word * 8, 0, kSC1);
  return ((uint64_t)v[1] << 32) | v[0];
}
__device__ __forceinline__ float tval(uint64_t w) { return __uint_as_float((uint32_t)w); }
__device__ __forceinline__ bool tok(uint64_t w, uint32_t tag) { return (uint32_t)(w >> 32) == tag; }

// Wake every sleeping wave of the workgroup (after publishing an LDS flag).
__device__ __forceinline__ void wake() { asm volatile("s_wakeup" ::: "memory"); }
#ifndef MK_PRIO
#define MK_PRIO 0  // wave issue priorities by role (s_setprio)
#endif
#ifndef MK_BPRIO
#define MK_BPRIO 1  // the same for the batched kernel
#endif
#ifndef MK_WSLEEP
#define MK_WSLEEP 1  // counter polls: s_sleep units (64 clocks) between polls
#endif
#ifndef MK_ARB
#define MK_ARB 16  // attention: K/V rows in flight per batch beyond the prefetched ones (head_dim 64)
#endif
#ifndef MK_TSLEEP
#define MK_TSLEEP 1  // tagged-word re-reads: s_sleep units between them
#endif
#ifndef MK_LSLEEP
#define MK_LSLEEP 1  // loader waiting for a free ring slot: s_sleep units between checks
#endif
#ifndef MK_FSLEEP
#define MK_FSLEEP 4  // page-sentinel spins: s_sleep units between polls
#endif
// LDS-flag spins: s_sleep units between polls (measured on the Llama-1B
// shape: 1, 2, 3, 4, 6, 10, 20 give 948, 944, 942, 940, 944, 952, 964 us)
#ifndef MK_SLEEP
#define MK_SLEEP 4
#endif

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Ordering of the cross-CU protocol.  A producer's results are written with
// device-coherent (sc1) stores, which complete at the device's coherence
// point; `s_waitcnt vmcnt(0)` waits for their acknowledgements before the
// counter increment is issued, so every result is visible device-wide before
// the increment is (the release half).  A consumer's poll is a device-
// coherent load whose value decides a branch, so the wave issues nothing
// after the poll until its value has returned, and everything it reads of
// other CUs' results afterwards is again a device-coherent load, which reads
// the coherence point rather than a possibly stale cached copy (the acquire
// half, for exactly the locations the consumer reads).  What the hardware
// does not need, the compiler still could break: relaxed atomics do not stop
// it from moving a later plain (buffer) load above the poll, so every poll
// exit is a compiler fence.  MK_ACQ=1 adds the memory model's own agent-scope
// acquire fence at every poll exit and a release fence before every counter
// increment (measured on the Llama-1B shape at batch 1: 1855 us a step
// against 903 us, the fences writing back and invalidating caches at every
// hop).
#ifndef MK_ACQ
#define MK_ACQ 0
#endif
__device__ __forceinline__ void poll_exit() {
#if MK_ACQ
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#else
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
#endif
}
__device__ __forceinline__ void before_signal() {
#if MK_ACQ
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
#else
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
#endif
}
// LDS flags order data within the workgroup: a compiler fence suffices (LDS
// operations of one wave complete in order).
__device__ __forceinline__ void lds_poll_exit() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// LDS control words for the C++ roles (sync and compute waves)
// Flags are wave-uniform: the value is moved to a scalar register so every
// branch on it is a scalar branch, not an exec-mask region.
__device__ __forceinline__ uint32_t lds_ld(int off) {
  return __builtin_amdgcn_readfirstlane(
      __hip_atomic_load(&lds_u32(off), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
}
// Per-lane load (lanes may read different words).
__device__ __forceinline__ uint32_t lds_ld_lane(int off) {
  return __hip_atomic_load(&lds_u32(off), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(int off, uint32_t v) {
  __hip_atomic_store(&lds_u32(off), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// --------------------------------------------------------------------------
// 64-lane reductions with DPP (quad perms, row rotates, row broadcasts)
template <int CTRL, int RM>
__device__ __forceinline__ float dpp0(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, RM, 0xf, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp0<0xb1, 0xf>(v);    // quad_perm [1,0,3,2]
  v += dpp0<0x4e, 0xf>(v);    // quad_perm [2,3,0,1]
  v += dpp0<0x124, 0xf>(v);   // row_ror:4
  v += dpp0<0x128, 0xf>(v);   // row_ror:8
  v += dpp0<0x142, 0xa>(v);   // row_bcast:15 into rows 1, 3
  v += dpp0<0x143, 0xc>(v);   // row_bcast:31 into rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_max(float v) {
  // all lanes hold valid values; the identity for the bcast steps is -inf
  auto mx = [](float a, float b) { return fmaxf(a, b); };
  v = mx(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0xb1, 0xf, 0xf, false)));
  v = mx(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x4e, 0xf, 0xf, false)));
  v = mx(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x124, 0xf, 0xf, false)));
  v = mx(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x128, 0xf, 0xf, false)));
  v = mx(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x142, 0xa, 0xf, false)));
  v = mx(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x143, 0xc, 0xf, false)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

struct Env {
  const DevCtx *__restrict__ cp;  // device context (scalar loads)
  uint64_t *trace;                // this workgroup's records, or null
  const Instr *q;    // this workgroup's queue
  uint32_t nq;       // its length
  int cu;
  int pos0;          // batch 1: this step's position (positions[0] + step_off)
  int flags;         // MK_FLAG_* of the handle
};

// MK_FLAG_PERTURB: a seeded pseudo-random delay (0..31 sleeps of 64 clocks)
// before each instruction of each wave, different for every step (tag),
// workgroup, instruction and wave, so that the same schedule runs under
// other interleavings.
constexpr int kFlagPerturb = 4;
__device__ __forceinline__ void perturb(const Env &e, uint32_t tag, uint32_t qi, uint32_t wave) {
  if (!(e.flags & kFlagPerturb)) return;
  uint32_t x = tag * 0x9E3779B9u ^ (uint32_t)e.cu * 0x85EBCA6Bu ^ qi * 0xC2B2AE35u ^ wave * 0x27D4EB2Fu;
  x ^= x >> 15;
  x *= 0x2C1B3C6Du;
  x ^= x >> 12;
  for (uint32_t i = __builtin_amdgcn_readfirstlane(x & 31u); i > 0; --i) __builtin_amdgcn_s_sleep(1);
}

__device__ __forceinline__ int64_t now() { return (int64_t)wall_clock64(); }

// Trace record per queued instruction (100 MHz wall clock):
//   [0] op | layer << 8 | unit << 24
//   [1] sync wave: waits of the first activation piece satisfied
//   [2] compute wave 0 passed the unit's gate
//   [3] last compute wave: epilogue done, about to signal
//   [4] sync wave: started the instruction (before its waits)
//   [5] sync wave: first activation piece published
//   [6] last compute wave: its own pieces done, epilogue starting
//   [7] sync wave: last activation piece published
constexpr int kTraceWords = 8;
__device__ __forceinline__ void trace_put(const Env &e, uint32_t qi, int word, uint64_t v) {
  if (e.trace) G(e.trace)[(size_t)qi * kTraceWords + word] = v;
}
// timestamp record: the clock is only read when tracing
__device__ __forceinline__ void trace_now(const Env &e, uint32_t qi, int word) {
  if (e.trace) G(e.trace)[(size_t)qi * kTraceWords + word] = (uint64_t)now();
}

// Record the first device error and make every wave of this workgroup exit.
__device__ void raise_error(const Env &e, uint32_t code, uint32_t info) {
  GAS uint32_t *st = G(e.cp->status);
  if (__hip_atomic_load(st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
    uint32_t zero = 0;
    if (__hip_atomic_compare_exchange_strong(st, &zero, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT)) {
      __hip_atomic_store(st + 1, info, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(st + 2, (uint32_t)e.cu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  lds_st(L_ABORT, 1);
}

// Spin on an LDS condition with the abort flag and the watchdog.
// Watchdog for spin loops.  The clock (s_memrealtime) is a scalar-memory
// round trip of about a microsecond under load, so it is read only every 256
// polls and the deadline is set lazily at the first such read: a short wait
// never touches the clock.
struct Watchdog {
  int64_t deadline = 0;
  // true when the budget is exhausted
  __device__ __forceinline__ bool expired(int64_t budget) {
    const int64_t t = now();
    if (deadline == 0) {
      deadline = t + budget;
      return false;
    }
    return t > deadline;
  }
};

// Waits on LDS flags sleep between polls; the producer of every flag
// executes s_wakeup, so a waiter normally resumes right after the flag is
// set and polling does not flood the LDS queue or the issue slots.
template <class F>
__device__ __forceinline__ bool spin_lds(const Env &e, F cond, uint32_t info) {
  if (cond()) {
    lds_poll_exit();
    return true;
  }
  Watchdog wd;
  for (uint32_t it = 1;; ++it) {
    __builtin_amdgcn_s_sleep(MK_SLEEP);
    if (cond()) {
      lds_poll_exit();
      return true;
    }
    if ((it & 63) == 0) {
      if (lds_ld(L_ABORT)) return false;
      if (wd.expired(e.cp->watchdog_ticks)) {
        raise_error(e, 0xA0000000u | info, 0);
        return false;
      }
    }
  }
}

// The same with a short sleep: for waits whose producer cannot wake the
// waiter (a page sentinel written by a direct-to-LDS load).
template <class F>
__device__ __forceinline__ bool spin_lds_fast(const Env &e, F cond, uint32_t info) {
  if (cond()) {
    lds_poll_exit();
    return true;
  }
  Watchdog wd;
  for (uint32_t it = 1;; ++it) {
    __builtin_amdgcn_s_sleep(MK_FSLEEP);
    if (cond()) {
      lds_poll_exit();
      return true;
    }
    if ((it & 255) == 0) {
      if (lds_ld(L_ABORT)) return false;
      if (wd.expired(e.cp->watchdog_ticks)) {
        raise_error(e, 0xA0000000u | info, 0);
        return false;
      }
    }
  }
}

// Re-run `load` (it re-reads tagged words and returns, per lane, whether all
// of them carry this step's tag) until every lane is satisfied.
template <class F>
__device__ __forceinline__ bool until_tagged(const Env &e, F load, uint32_t info) {
  Watchdog wd;
  for (uint32_t it = 0;; ++it) {
    if (__all(load())) {
      poll_exit();
      return true;
    }
    if ((it & 63) == 63) {
      if (lds_ld(L_ABORT)) return false;
      if (wd.expired(e.cp->watchdog_ticks)) {
        raise_error(e, 0xD0000000u | info, 0);
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(MK_TSLEEP);
  }
}

// --------------------------------------------------------------------------
// Weight pieces: piece (k, r) of instruction d is K-range k of unit row
// r = i*ipw + s (see Instr).  Pure arithmetic on descriptor fields plus, for
// tabulated units, a load from the row table: the loader must not issue
// vector loads whose waits would drain its outstanding direct-to-LDS loads,
// so on its fast path these are scalar (uniform index, read-only table).
__device__ __forceinline__ const char *piece_addr(const Instr &d, const uint64_t *__restrict__ rowtab,
                                                  uint32_t k, uint32_t r) {
  uint64_t base;
  if (d.tab >= 0) base = rowtab[d.tab + r];
  else if (d.ipw == 2) base = ((r & 1) ? d.w1 : d.w0) + (uint64_t)(d.item0 + (r >> 1)) * d.rowb;
  else base = d.w0 + (uint64_t)(d.item0 + r) * d.rowb;
  return reinterpret_cast<const char *>(base) + (size_t)k * d.pb;
}

__device__ __forceinline__ bool is_gemv(uint8_t op) {
  return op == OP_QKV || op == OP_O || op == OP_FFN || op == OP_DOWN || op == OP_LM;
}

// --------------------------------------------------------------------------
// Loader waves.  All of their LDS accesses are inline asm so the compiler's
// wait-count insertion never ties them to the outstanding direct-to-LDS
// loads; page completion is tracked with explicit vmcnt waits.
__device__ __forceinline__ uint32_t lds_addr(int off) {
  return (uint32_t)(uintptr_t)((LDS_AS char *)smem + off);
}
__device__ __forceinline__ uint32_t asm_lds_ld(uint32_t off) {
  off = lds_addr((int)off);
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(off) : "memory");
  return v;
}
template <int N>
__device__ __forceinline__ void wait_vm_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// --------------------------------------------------------------------------
// Paged attention.  The K/V rows a split has from earlier steps (its
// positions below p) are read-only during a step, like the weights, so the
// loader streams them through the same page ring ahead of the unit's
// dependency wait (the megakernel chapter "L'interpréteur sur GPU", section
// 3.3: the next instruction's inputs load while the current one computes).
// A page holds RPP rows: 8 wave-loads of K, then 8 of V.  K row t of a page
// sits in wave-load t / RPL, its 16-byte chunk c at position c ^ (t & 7) of
// the row, so a wave reading one chunk of 8 consecutive rows (one lane per
// row) hits 8 different bank groups; V rows are stored as they are.
// Attention descriptors of paged plans carry RPP in `ppp` (0: the register
// path of attn_body).
__device__ __forceinline__ size_t kv_off(const DevCtx &c, int l, int t, int b, int g, int s) {
  return lay::kv(c.max_batch, c.nkv, c.max_seq, c.hd, l, t, b, g, s);
}

__device__ __forceinline__ void attn_geom(const Args &a, const Instr &d, int p, int &lo, int &hi, uint32_t &nr) {
  lo = (int)d.aux1 * a.split_len;
  hi = min(lo + a.split_len, p + 1);
  nr = (uint32_t)max(0, min(hi, p) - lo);  // rows before p: from the cache
}
__device__ __forceinline__ uint32_t attn_pages(const Args &a, const Instr &d, int p) {
  int lo, hi;
  uint32_t nr;
  attn_geom(a, d, p, lo, hi, nr);
  return (nr + d.ppp - 1) / d.ppp;
}
template <int CPR>
__device__ __forceinline__ void load_kv_page(const char *Kb, const char *Vb, uint32_t jp, uint32_t nr,
                                             LDS_AS char *slot, int lane) {
  constexpr uint32_t RPL = 64 / CPR, RPP = 8 * RPL, RB = CPR * 16;
  const uint32_t t0 = (uint32_t)lane / CPR, cp = (uint32_t)lane % CPR;
#pragma unroll
  for (uint32_t jj = 0; jj < 8; ++jj) {
    const uint32_t t = jj * RPL + t0;
    uint32_t r = jp * RPP + t;
    if (r >= nr) r = 0;  // past the split's rows: re-read its first row
    __builtin_amdgcn_global_load_lds(Kb + (size_t)r * RB + (cp ^ (t & 7)) * 16, (LDS_AS void *)(slot + jj * 1024),
                                     16, 0, kSC1);
  }
#pragma unroll
  for (uint32_t jj = 0; jj < 8; ++jj) {
    const uint32_t t = jj * RPL + t0;
    uint32_t r = jp * RPP + t;
    if (r >= nr) r = 0;
    __builtin_amdgcn_global_load_lds(Vb + (size_t)r * RB + cp * 16, (LDS_AS void *)(slot + 8192 + jj * 1024), 16,
                                     0, kSC1);
  }
}

#ifndef MK_SDEPTH
#define MK_SDEPTH 3
#endif
constexpr int kSentDepth = MK_SDEPTH;  // pages in flight per loader wave (17 loads each, <= 63)
static_assert(kSentDepth >= 1 && 17 * kSentDepth <= 63, "load counter range");
// Each loader wave keeps up to kSentDepth pages in flight (17 loads each: 16
// weight loads and the page's sentinel).  A page is never published by the
// loader: its sentinel lands after its data, so the loader only waits for a
// free ring slot (compute waves' releases) and, to bound its load counter,
// for its oldest page once kSentDepth are in flight.
// A later step of a launch streams K/V pages only once the sync wave has
// seen the step's tokens counted (L_TOKOK; see wait_tokens for what that
// orders).  Weight pages need no such wait.
__device__ __forceinline__ bool loader_tok_gate(const Env &e, bool &tok_ok, uint32_t qi) {
  if (tok_ok) return true;
  Watchdog wd;
  for (uint32_t it = 1;; ++it) {
    if (__builtin_amdgcn_readfirstlane(asm_lds_ld(L_TOKOK))) {
      tok_ok = true;
      return true;
    }
    __builtin_amdgcn_s_sleep(MK_LSLEEP);
    if ((it & 63) == 0) {
      if (__builtin_amdgcn_readfirstlane(asm_lds_ld(L_ABORT))) return false;
      if (wd.expired(e.cp->watchdog_ticks)) {
        raise_error(e, 0xB8000000u | qi, 0);
        return false;
      }
    }
  }
}

template <bool PAGED>
__device__ __forceinline__ void loader_role(const Env &e, const Args &a, int lw) {
  const int lane = lane_id();
  const uint32_t P = (uint32_t)e.cp->ring_pages;
  int npend = 0;
  auto min_cons = [&]() -> uint32_t {
    uint32_t v = lane < kNCW ? asm_lds_ld(L_CONS + 4 * lane) : 0xffffffffu;
    // minimum over lanes 0..7 with readlanes (no LDS-unit cross-lane ops)
    uint32_t m = __builtin_amdgcn_readlane(v, 0);
#pragma unroll
    for (int i = 1; i < kNCW; ++i) m = min(m, (uint32_t)__builtin_amdgcn_readlane(v, i));
    return m;
  };
  uint32_t n = 0;  // global page index
  bool tok_ok = a.step_off == 0;
  for (uint32_t qi = 0; qi < e.nq; ++qi) {
    const Instr d = e.q[qi];
    perturb(e, step_tag(a), qi, (uint32_t)(threadIdx.x >> 6));
    if (PAGED && d.op == OP_ATTN) {
      if (!loader_tok_gate(e, tok_ok, qi)) {
        wait_vm0();
        return;
      }
      int lo, hi;
      uint32_t nr;
      attn_geom(a, d, e.pos0, lo, hi, nr);
      const uint32_t np = (nr + d.ppp - 1) / d.ppp;
      const DevCtx &c = *e.cp;
      const char *Kb = reinterpret_cast<const char *>(a.kv + kv_off(c, d.layer, 0, (int)d.b, (int)d.aux0, lo));
      const char *Vb = reinterpret_cast<const char *>(a.kv + kv_off(c, d.layer, 1, (int)d.b, (int)d.aux0, lo));
      for (uint32_t jp = 0; jp < np; ++jp, ++n) {
        if ((int)(n % kNLW) != lw) continue;
        if (n >= P && min_cons() < n - P + 1) {
          const uint32_t need = n - P + 1;
          Watchdog wd;
          for (uint32_t it = 1;; ++it) {
            __builtin_amdgcn_s_sleep(MK_LSLEEP);
            if (min_cons() >= need) break;
            if ((it & 63) == 0) {
              if (__builtin_amdgcn_readfirstlane(asm_lds_ld(L_ABORT))) { wait_vm0(); return; }
              if (wd.expired(e.cp->watchdog_ticks)) { raise_error(e, 0xB0000000u | qi, n); wait_vm0(); return; }
            }
          }
        }
        if (npend == kSentDepth) {
          wait_vm_n<17 * (kSentDepth - 1)>();
          --npend;
        }
        LDS_AS char *slot = (LDS_AS char *)smem + L_RING + (n % P) * kPageBytes;
        if (c.hd == 64) load_kv_page<8>(Kb, Vb, jp, nr, slot, lane);
        else load_kv_page<16>(Kb, Vb, jp, nr, slot, lane);
        __builtin_amdgcn_global_load_lds(a.iota + n, (LDS_AS void *)(smem + L_SENT + (n % P) * kSentBytes), 4, 0, 0);
        ++npend;
      }
      continue;
    }
    if (!is_gemv(d.op)) continue;
    const uint32_t per = d.n_items * d.ipw;
    const uint32_t npieces = per * d.nk;
    for (uint32_t p = 0; p < d.pages; ++p, ++n) {
      if ((int)(n % kNLW) != lw) continue;
      if (n >= P && min_cons() < n - P + 1) {
        // slot n % P is free once every compute wave released page n - P
        const uint32_t need = n - P + 1;
        Watchdog wd;
        for (uint32_t it = 1;; ++it) {
          __builtin_amdgcn_s_sleep(MK_LSLEEP);
          if (min_cons() >= need) break;
          if ((it & 63) == 0) {
            if (__builtin_amdgcn_readfirstlane(asm_lds_ld(L_ABORT))) { wait_vm0(); return; }
            if (wd.expired(e.cp->watchdog_ticks)) { raise_error(e, 0xB0000000u | qi, n); wait_vm0(); return; }
          }
        }
      }
      if (npend == kSentDepth) {
        wait_vm_n<17 * (kSentDepth - 1)>();  // the oldest page of this wave has landed
        --npend;
      }
      // issue exactly 16 wave-loads (1 KB each) for page p into slot n % P,
      // then its sentinel; unused tail loads re-read the page's first piece
      LDS_AS char *slot = (LDS_AS char *)smem + L_RING + (n % P) * kPageBytes;
      const uint32_t t0 = p * d.ppp;
      const uint32_t cnt = min((uint32_t)d.ppp, npieces - t0);
      uint32_t k = t0 / per, r = t0 - k * per;
      const char *first = piece_addr(d, a.rowtab, k, r);
      if (d.pb >= 1024) {
        const uint32_t lpp = d.pb >> 10;  // wave-loads per piece
        uint32_t j = 0;
        for (uint32_t q = 0; q < cnt; ++q) {
          const char *src = piece_addr(d, a.rowtab, k, r) + lane * 16;
          LDS_AS char *dst = slot + j * 1024;
          uint32_t sub = 0;
          // the immediate offset moves both the global source and the LDS
          // destination, so four loads share one M0 and one address
          for (; sub + 4 <= lpp; sub += 4, src += 4096, dst += 4096) {
            __builtin_amdgcn_global_load_lds(src, (LDS_AS void *)dst, 16, 0, kWPol);
            __builtin_amdgcn_global_load_lds(src, (LDS_AS void *)dst, 16, 1024, kWPol);
            __builtin_amdgcn_global_load_lds(src, (LDS_AS void *)dst, 16, 2048, kWPol);
            __builtin_amdgcn_global_load_lds(src, (LDS_AS void *)dst, 16, 3072, kWPol);
          }
          for (; sub < lpp; ++sub, src += 1024, dst += 1024)
            __builtin_amdgcn_global_load_lds(src, (LDS_AS void *)dst, 16, 0, kWPol);
          j += lpp;
          if (++r == per) { r = 0; ++k; }
        }
        for (; j < 16; ++j)
          __builtin_amdgcn_global_load_lds(first + lane * 16, (LDS_AS void *)(slot + j * 1024), 16, 0, kWPol);
      } else {
        const uint32_t sh = 31 - __builtin_clz(d.pb);  // pb is a power of two
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const uint32_t o = (uint32_t)j * 1024 + lane * 16;
          const uint32_t q = o >> sh, within = o & (d.pb - 1);
          const uint32_t t = t0 + q;
          const char *src = first;
          if (t < npieces) {
            const uint32_t kk = t / per;
            src = piece_addr(d, a.rowtab, kk, t - kk * per) + within;
          }
          __builtin_amdgcn_global_load_lds(src, (LDS_AS void *)(slot + j * 1024), 16, 0, kWPol);
        }
      }
      __builtin_amdgcn_global_load_lds(a.iota + n, (LDS_AS void *)(smem + L_SENT + (n % P) * kSentBytes), 4, 0, 0);
      ++npend;
    }
  }
  wait_vm0();
}

// --------------------------------------------------------------------------
// Sync wave: counter waits and activation pieces.

// Poll one counter group until each of its counter slots reached
// target * epoch.  Lane i polls slot i (i < nslot).
__device__ __forceinline__ bool wait_group(const Env &e, const Args &a, const Wait &wt, uint32_t qi) {
  const int lane = lane_id();
  const uint32_t grp = wt.grp;
  const bool mine = lane < (int)wt.nslot;
  const uint32_t *cp = a.ctr + ((size_t)grp * kSlots + (lane & (kSlots - 1))) * kCtrStride;
  const uint32_t need = mine ? a.grp_target[grp * kSlots + lane] * step_epoch(a) : 0u;
  Watchdog wd;
  for (uint32_t it = 0;; ++it) {
    bool ok = true;
    if (mine) ok = (int32_t)(ld_cu(cp) - need) >= 0;
    if (__all(ok)) {
      poll_exit();
      return true;
    }
    if ((it & 63) == 63) {
      if (lds_ld(L_ABORT)) return false;
      if (ld_cu(&e.cp->status[0]) != 0) { lds_st(L_ABORT, 1); return false; }
      if (wd.expired(e.cp->watchdog_ticks)) {
        raise_error(e, 0xC0000000u | grp, qi);
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(MK_WSLEEP);
  }
}

// Token b of this step, read once per step by the sync wave (the only
// reader).  Step 0's are the caller's; those of step s > 0 were written
// during the launch by another workgroup and are read device-coherently.
__device__ __forceinline__ int32_t ld_tok(const Args &a, int b) {
  if (a.step_off == 0) return a.tokens[b];
  return (int32_t)ld_cu(reinterpret_cast<const uint32_t *>(a.next_tok) + b);
}

// Step s > 0 of a launch reads the tokens step s - 1 chose: wait until its
// finisher has counted them (the token counter reaches tok_base + s).  The
// finisher ran after every unit of step s - 1, so this wait also orders the
// K/V rows that step wrote before their reads in this step, provided their
// stores were acknowledged before some signal on the way to the finisher: a
// QKV epilogue does not wait for its stores (no counter follows it), and its
// wave acknowledges them at the end of its next attention or reduction unit,
// which every workgroup of the Llama-1B and Qwen3-8B schedules has; where a
// workgroup has none, the rest of the step outlasting the stores is what
// orders them.  L_TOKOK tells the workgroup's other waves.
__device__ __forceinline__ bool wait_tokens(const Env &e, const Args &a) {
  if (a.step_off == 0) return true;
  const uint32_t *tc = a.amax_ctr + kTokWord;
  const uint32_t need = a.tok_base + (uint32_t)a.step_off;
  Watchdog wd;
  for (uint32_t it = 0;; ++it) {
    if ((int32_t)(ld_cu(tc) - need) >= 0) {
      poll_exit();
      lds_st(L_TOKOK, 1);
      wake();
      return true;
    }
    if ((it & 63) == 63) {
      if (lds_ld(L_ABORT)) return false;
      if (ld_cu(&e.cp->status[0]) != 0) { lds_st(L_ABORT, 1); return false; }
      if (wd.expired(e.cp->watchdog_ticks)) {
        raise_error(e, 0xC8000000u | (uint32_t)a.step_off, 0);
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(MK_WSLEEP);
  }
}

// Input vector source of the RMSNorm'd instructions.
__device__ __forceinline__ void norm_src(const Env &e, const Instr &d, int b, int32_t tok,
                                         const float *&h, const uint16_t *&emb, const uint16_t *&w) {
  const DevCtx &c = *e.cp;
  h = nullptr;
  emb = nullptr;
  if (d.op == OP_QKV) {
    w = G(c.layers)[d.layer].attn_norm;
    if (d.layer == 0) emb = c.embed + (size_t)tok * c.H;
    else h = c.h_buf + lay::h(c.max_batch, c.H, 2 * d.layer, b);
  } else if (d.op == OP_FFN) {
    w = G(c.layers)[d.layer].ffn_norm;
    h = c.h_buf + lay::h(c.max_batch, c.H, 2 * d.layer + 1, b);
  } else {  // OP_LM
    w = c.final_norm;
    h = c.h_buf + lay::h(c.max_batch, c.H, 2 * c.L, b);
  }
}

__device__ __forceinline__ void sync_role(const Env &e, const Args &a) {
  const DevCtx &c = *e.cp;
  const int lane = lane_id();
  if (!wait_tokens(e, a)) return;
  // inputs are validated once per workgroup before anything depends on them
  for (int b = 0; b < a.batch; ++b) {
    int32_t tk = ld_tok(a, b), ps = a.positions[b] + a.step_off;
    if (tk < 0 || tk >= c.V) { raise_error(e, 0xE1000000u, (uint32_t)b); return; }
    if (ps < 0 || ps >= c.max_seq) { raise_error(e, 0xE2000000u, (uint32_t)b); return; }
  }
  const int b = 0;
  const int32_t tok = ld_tok(a, b);
  const int pos = e.pos0;
  uint32_t seq = 0;
  float rs = 0.f;
  for (uint32_t qi = 0; qi < e.nq; ++qi) {
    const Instr d = e.q[qi];
    perturb(e, step_tag(a), qi, (uint32_t)(threadIdx.x >> 6));
    const uint32_t nx = is_gemv(d.op) ? d.nk : 1;
    const bool normed = d.op == OP_QKV || d.op == OP_FFN || d.op == OP_LM;
    float *accs = reinterpret_cast<float *>(smem + L_ACC + (qi & (kAccSlots - 1)) * kAccFloats * 4);

    // Step-invariant inputs are fetched before the unit's dependency waits,
    // so that their round trips overlap the wait: the norm weights of the
    // first activation piece, and for QKV the RoPE cos/sin of position p
    // for the unit's pairs (staged in the upper half of its result slot,
    // once the unit that used the slot before has finished its epilogue).
    const float *h = nullptr;
    const uint16_t *emb = nullptr, *nw = nullptr;
    uint64_t *nwl = reinterpret_cast<uint64_t *>(smem + L_NW);  // norm weights, 4 per word
    auto stage_norm_weights = [&](uint32_t k0) {
      for (uint32_t i = (uint32_t)lane * 4; i < d.kc; i += 256)
        nwl[i >> 2] = *G(reinterpret_cast<const uint64_t *>(nw + k0 + i));
    };
    if (normed) {
      norm_src(e, d, b, tok, h, emb, nw);
      stage_norm_weights(0);
    }
    // Unit qi shares its LDS result slot and its completion counter with
    // unit qi - kAccSlots, whose epilogue must have finished before this
    // unit's slot is written (RoPE values, residual rows, below) and before
    // its ready flag lets the compute waves use either: every compute wave
    // passes that flag before it touches them.
    if (qi >= (uint32_t)kAccSlots &&
        !spin_lds(e, [&]() { return lds_ld(L_EPI) + kAccSlots > qi; }, 0x500 | qi))
      return;
    if (d.op == OP_QKV) {
      const uint32_t half = (uint32_t)c.hd >> 1, ppg = (uint32_t)(c.G + 2) * half;
      for (uint32_t i = (uint32_t)lane; i < d.n_items; i += 64) {
        const uint32_t ii = ((d.item0 + i) % ppg) % half;
        const uint64_t cs = *G(reinterpret_cast<const uint64_t *>(c.rope + lay::rope(c.hd, pos, (int)ii)));
        accs[kAccFloats / 2 + 2 * i] = __uint_as_float((uint32_t)cs);
        accs[kAccFloats / 2 + 2 * i + 1] = __uint_as_float((uint32_t)(cs >> 32));
      }
    }

    uint32_t wi = 0;
    if (lane == 0) trace_now(e, qi, 4);
    // O and DOWN units of at most 64 rows (but layer 0's O, whose residual
    // is the bf16 embedding row): the activation pieces are plain fp32
    // copies of attn / a and the residual rows copies of h, so they go to
    // LDS by direct-to-LDS loads, two pieces in flight; the counter waits of
    // piece k + 1 overlap the loads of piece k.  A piece is exactly 8
    // wave-loads (1 KB each; lanes past the piece re-read its start), piece
    // 0 one more for the residual rows, so `vmcnt` tells when the older of
    // two pieces has landed.
    const bool dma_pieces = (d.op == OP_DOWN || (d.op == OP_O && d.layer > 0)) && d.n_items <= 64;
    if (dma_pieces) {
      const float *src = d.op == OP_O ? c.attn_buf + lay::attn(c.max_batch, c.nq, c.hd, d.layer, b)
                                      : c.a_buf + lay::a(c.max_batch, c.F, d.layer, b);
      const float *res = c.h_buf + lay::h(c.max_batch, c.H, d.op == OP_O ? 2 * d.layer : 2 * d.layer + 1, b) +
                         d.item0 + lane;
      LDS_AS char *accl = (LDS_AS char *)smem + L_ACC + (qi & (kAccSlots - 1)) * kAccFloats * 4;
      auto issue = [&](uint32_t k, uint32_t sq) {
        if (k == 0 && lane < (int)d.n_items) __builtin_amdgcn_global_load_lds(res, (LDS_AS void *)accl, 4, 0, kSC1);
        LDS_AS char *slot = (LDS_AS char *)smem + L_XS + (sq % kNXS) * kXSlotBytes;
        const float *base = src + (size_t)k * d.kc;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t f = (uint32_t)(j * 256 + lane * 4);
          __builtin_amdgcn_global_load_lds(base + (f < d.kc ? f : 0u), (LDS_AS void *)(slot + j * 1024), 16, 0, kSC1);
        }
      };
      // piece 0's waits, then the pipeline (later pieces' waits inside it)
      while (wi < d.wait_n) {
        const Wait wt = a.waits[d.wait_off + wi];
        if (wt.before_k > 0) break;
        if (!wait_group(e, a, wt, qi)) return;
        ++wi;
      }
      if (lane == 0) {
        trace_put(e, qi, 0, (uint64_t)d.op | ((uint64_t)d.layer << 8) | ((uint64_t)d.unit << 24));
        trace_now(e, qi, 1);
      }
      int64_t t_first = 0, t_last = 0;  // trace words 5 and 7, stored after the loop
      uint32_t issued = 0, done = 0;
      while (done < nx) {
        if (issued < nx && issued - done < (uint32_t)kNXS) {
          while (wi < d.wait_n) {
            const Wait wt = a.waits[d.wait_off + wi];
            if (wt.before_k > issued) break;
            if (!wait_group(e, a, wt, qi)) { wait_vm0(); return; }
            ++wi;
          }
          const uint32_t sq = seq + issued;
          if (sq >= (uint32_t)kNXS) {
            const uint32_t need = sq - kNXS + 1;
            auto freed = [&]() {
              uint32_t v = lane < kNCW ? lds_ld_lane(L_XCONS + 4 * lane) : 0xffffffffu;
              uint32_t m = __builtin_amdgcn_readlane(v, 0);
#pragma unroll
              for (int i = 1; i < kNCW; ++i) m = min(m, (uint32_t)__builtin_amdgcn_readlane(v, i));
              return m >= need;
            };
            if (!spin_lds(e, freed, 0x100 | qi)) { wait_vm0(); return; }
          }
          issue(issued, sq);
          ++issued;
        } else {
          if (issued - done >= 2) wait_vm_n<8>();
          else wait_vm0();
          if (lane == 0) lds_st(L_XREADY, seq + done + 1);
          wake();
          if (done == 0) t_first = now();
          if (done + 1 == nx) t_last = now();
          ++done;
        }
      }
      if (lane == 0) {
        trace_put(e, qi, 5, (uint64_t)t_first);
        trace_put(e, qi, 7, (uint64_t)t_last);
      }
      seq += nx;
    }
    // (a `continue` above instead of this test makes the compiler spill)
    if (!dma_pieces)
    for (uint32_t k = 0; k < nx; ++k, ++seq) {
      while (wi < d.wait_n) {
        const Wait wt = a.waits[d.wait_off + wi];
        if (wt.before_k > k) break;
        if (!wait_group(e, a, wt, qi)) return;
        ++wi;
      }
      if (seq >= (uint32_t)kNXS) {
        const uint32_t need = seq - kNXS + 1;
        auto freed = [&]() {
          uint32_t v = lane < kNCW ? lds_ld_lane(L_XCONS + 4 * lane) : 0xffffffffu;
          uint32_t m = __builtin_amdgcn_readlane(v, 0);
#pragma unroll
          for (int i = 1; i < kNCW; ++i) m = min(m, (uint32_t)__builtin_amdgcn_readlane(v, i));
          return m >= need;
        };
        if (!spin_lds(e, freed, 0x100 | qi)) return;
      }
      float *xs = reinterpret_cast<float *>(smem + L_XS + (seq % kNXS) * kXSlotBytes);
      if (k == 0 && lane == 0) {
        trace_put(e, qi, 0, (uint64_t)d.op | ((uint64_t)d.layer << 8) | ((uint64_t)d.unit << 24));
        trace_now(e, qi, 1);
      }
      if (normed) {
        const rsrc_t hr = rsrc(h ? (const void *)h : (const void *)emb);
        // one batch of up to 2048 elements (8 x 4 per lane) in flight
        auto load_batch = [&](uint32_t e0, f4 (&v)[8]) {
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const uint32_t i = e0 + (uint32_t)(lane + 64 * m) * 4;
            if (i < (uint32_t)c.H) {
              if (emb) {
                const uint64_t uu = *G(reinterpret_cast<const uint64_t *>(emb + i));
                v[m] = f4{bf_lo((uint32_t)uu), bf_hi((uint32_t)uu), bf_lo((uint32_t)(uu >> 32)),
                          bf_hi((uint32_t)(uu >> 32))};
              } else {
                v[m] = ldc4(hr, i * 4);
              }
            } else {
              v[m] = f4{0.f, 0.f, 0.f, 0.f};
            }
          }
        };
        f4 hv[8];
        if (k == 0) {
          float ss = 0.f;
          for (uint32_t e0 = 0; e0 < (uint32_t)c.H; e0 += 2048) {
            load_batch(e0, hv);
#pragma unroll
            for (int m = 0; m < 8; ++m) ss += hv[m].x * hv[m].x + hv[m].y * hv[m].y + hv[m].z * hv[m].z + hv[m].w * hv[m].w;
          }
          ss = wave_sum(ss);
          rs = 1.0f / sqrtf(ss / (float)c.H + c.eps);
        }
        // pieces hold at most 2048 elements; the last batch loaded is still
        // in hv when H <= 2048 (then nk == 1)
        const uint32_t k0 = k * d.kc;
        if (c.H > 2048 || k0 != 0) load_batch(k0, hv);
        if (k > 0) stage_norm_weights(k0);
        // one base address per lane, the 8 chunks at immediate offsets
        const uint64_t *nwp = nwl + lane;
        f4 *xp = reinterpret_cast<f4 *>(xs) + lane;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const uint32_t i = (uint32_t)(lane + 64 * m) * 4;
          if (i < d.kc) {
            const f4 v = hv[m];
            const uint64_t w4 = nwp[64 * m];
            const uint32_t w0 = (uint32_t)w4, w1 = (uint32_t)(w4 >> 32);
            f4 o = {v.x * rs * bf_lo(w0), v.y * rs * bf_hi(w0), v.z * rs * bf_lo(w1), v.w * rs * bf_hi(w1)};
            xp[64 * m] = o;
          }
        }
      } else if (d.op == OP_O || d.op == OP_DOWN) {
        // the activation piece and (first piece) the unit's residual rows,
        // loaded together: one round trip
        const float *src = d.op == OP_O ? c.attn_buf + lay::attn(c.max_batch, c.nq, c.hd, d.layer, b)
                                        : c.a_buf + lay::a(c.max_batch, c.F, d.layer, b);
        const rsrc_t sr = rsrc(src + k * d.kc);
        f4 v[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const uint32_t i = (uint32_t)(lane + 64 * m) * 4;
          if (i < d.kc) v[m] = ldc4(sr, i * 4);
        }
        if (k == 0) {
          float rv[kAccFloats / 64];
          if (d.op == OP_O && d.layer == 0) {
            const GAS uint16_t *er = G(c.embed) + (size_t)tok * c.H + d.item0;
#pragma unroll
            for (int m = 0; m < kAccFloats / 64; ++m) {
              const uint32_t r = (uint32_t)(lane + 64 * m);
              rv[m] = r < d.n_items ? bf16f(er[r]) : 0.f;
            }
          } else {
            const int idx = d.op == OP_O ? 2 * d.layer : 2 * d.layer + 1;
            const rsrc_t rr = rsrc(c.h_buf + lay::h(c.max_batch, c.H, idx, b) + d.item0);
#pragma unroll
            for (int m = 0; m < kAccFloats / 64; ++m) {
              const uint32_t r = (uint32_t)(lane + 64 * m);
              rv[m] = r < d.n_items ? ldc1(rr, r * 4) : 0.f;
            }
          }
#pragma unroll
          for (int m = 0; m < kAccFloats / 64; ++m) {
            const uint32_t r = (uint32_t)(lane + 64 * m);
            if (r < d.n_items) accs[r] = rv[m];
          }
        }
        f4 *xp = reinterpret_cast<f4 *>(xs) + lane;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const uint32_t i = (uint32_t)(lane + 64 * m) * 4;
          if (i < d.kc) xp[64 * m] = v[m];
        }
      }
      wait_lgkm0();
      if (lane == 0) lds_st(L_XREADY, seq + 1);
      wake();
      if (k == 0 && lane == 0) trace_now(e, qi, 5);
      if (k + 1 == nx && lane == 0) trace_now(e, qi, 7);
    }
  }
}

// --------------------------------------------------------------------------
// Compute waves.

// Dot product of one weight piece (bf16, in LDS) with the activation piece
// held in registers: lane l owns 16-byte groups l, l+64, l+128, l+192.
// The page reads are one inline-asm block: the compiler's wait-count pass,
// seeing the loaders' direct-to-LDS loads in the same kernel, would otherwise
// put a vmcnt(0) before each read and make every row wait for the wave's
// outstanding global stores.  Lanes past the piece read other LDS bytes of
// the ring (in bounds) and are zeroed.
__device__ __forceinline__ float dot_piece(const char *piece, const float (&xr)[32], uint32_t n16) {
  const int lane = lane_id();
  const uint32_t addr = (uint32_t)(uintptr_t)((LDS_AS const char *)piece) + (uint32_t)lane * 16;
  u4 w[4];
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:1024\n\t"
      "ds_read_b128 %2, %4 offset:2048\n\t"
      "ds_read_b128 %3, %4 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3])  // early-clobber: later reads use addr
      : "v"(addr));
  if (n16 < 256) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if ((uint32_t)lane + 64u * m >= n16) w[m] = u4{0u, 0u, 0u, 0u};
  }
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    a0 = fmaf(bf_lo(w[m].x), xr[m * 8 + 0], a0);
    a1 = fmaf(bf_hi(w[m].x), xr[m * 8 + 1], a1);
    a0 = fmaf(bf_lo(w[m].y), xr[m * 8 + 2], a0);
    a1 = fmaf(bf_hi(w[m].y), xr[m * 8 + 3], a1);
    a0 = fmaf(bf_lo(w[m].z), xr[m * 8 + 4], a0);
    a1 = fmaf(bf_hi(w[m].z), xr[m * 8 + 5], a1);
    a0 = fmaf(bf_lo(w[m].w), xr[m * 8 + 6], a0);
    a1 = fmaf(bf_hi(w[m].w), xr[m * 8 + 7], a1);
  }
  return wave_sum(a0 + a1);
}

__device__ __forceinline__ void load_x(const float *xs, uint32_t n16, float (&xr)[32]) {
  const int lane = lane_id();
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t g = (uint32_t)lane + 64u * m;
    if (g < n16) {
      f4 p = *reinterpret_cast<const f4 *>(xs + g * 8);
      f4 q = *reinterpret_cast<const f4 *>(xs + g * 8 + 4);
      xr[m * 8 + 0] = p.x; xr[m * 8 + 1] = p.y; xr[m * 8 + 2] = p.z; xr[m * 8 + 3] = p.w;
      xr[m * 8 + 4] = q.x; xr[m * 8 + 5] = q.y; xr[m * 8 + 6] = q.z; xr[m * 8 + 7] = q.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) xr[m * 8 + i] = 0.f;
    }
  }
}


// Epilogue of a finished GEMV instruction, run by its last compute wave
// over the staged row results R (LDS): row i*ipw + s of the unit.  The
// outputs of 64 rows go out in one vector store.
//   QKV : RoPE on q/k pairs (i, i + hd/2), q -> fp32 scratch, k/v -> bf16
//         cache slot p;   O, DOWN: R already holds residual + dot;
//   FFN : a = silu(gate) * up;   LM: logits.
// Greedy order of (logit, vocabulary index) pairs: larger logit first, the
// lower index among equal logits; a NaN ranks above every number (the
// first NaN wins), as in the usual argmax of a float array.
__device__ __forceinline__ bool amax_better(float v, uint32_t i, float bv, uint32_t bi) {
  const bool vn = v != v, bn = bv != bv;
  if (vn || bn) return vn && (!bn || i < bi);
  return v > bv || (v == bv && i < bi);
}
// Butterfly over the 64 lanes: every lane ends with the wave's best pair.
__device__ __forceinline__ void amax_reduce(float &bv, uint32_t &bi) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const uint32_t oi = (uint32_t)__shfl_xor((int)bi, off);
    if (amax_better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
}

__device__ __forceinline__ void unit_epilogue(const Env &e, const Args &a, const Instr &d, const float *R) {
  const DevCtx &c = *e.cp;
  const int lane = lane_id();
  const int b = 0;
  for (uint32_t i = (uint32_t)lane; i < d.n_items; i += 64) {
    switch (d.op) {
      case OP_QKV: {
        const float v0 = R[2 * i], v1 = R[2 * i + 1];
        const uint32_t half = (uint32_t)c.hd >> 1;
        const uint32_t ppg = (uint32_t)(c.G + 2) * half;
        const uint32_t pp = d.item0 + i;
        const uint32_t g = pp / ppg;
        const uint32_t rr = pp - g * ppg;
        const uint32_t hs = rr / half;
        const uint32_t ii = rr - hs * half;
        const int p = e.pos0;
        if (hs <= (uint32_t)c.G && c.qk_norm) {
          // per-head q/k RMSNorm needs the whole head, which spans several
          // units: q and k leave raw (un-normed, un-rotated) and the
          // attention units norm and rotate them (and write K to the cache)
          uint64_t *dst = hs < (uint32_t)c.G
                              ? c.q_buf + lay::q(c.max_batch, c.nq, c.hd, d.layer, b, (int)(g * c.G + hs))
                              : c.kvn_buf + lay::kvn(c.max_batch, c.nkv, c.hd, d.layer, b, (int)g, 0);
          st_tag(dst + ii, v0, step_tag(a));
          st_tag(dst + ii + half, v1, step_tag(a));
        } else if (hs <= (uint32_t)c.G) {
          const float cs = R[kAccFloats / 2 + 2 * i], sn = R[kAccFloats / 2 + 2 * i + 1];
          const float r0 = v0 * cs - v1 * sn, r1 = v1 * cs + v0 * sn;
          if (hs < (uint32_t)c.G) {
            uint64_t *q = c.q_buf + lay::q(c.max_batch, c.nq, c.hd, d.layer, b, (int)(g * c.G + hs));
            st_tag(q + ii, r0, step_tag(a));
            st_tag(q + ii + half, r1, step_tag(a));
          } else {
            uint16_t *k = a.kv + kv_off(c, d.layer, 0, b, g, p);
            const uint16_t k0 = f2bf(r0), k1 = f2bf(r1);
            st_c16(k + ii, k0);
            st_c16(k + ii + half, k1);
            uint64_t *kn = c.kvn_buf + lay::kvn(c.max_batch, c.nkv, c.hd, d.layer, b, (int)g, 0);
            st_tag(kn + ii, bf16f(k0), step_tag(a));
            st_tag(kn + ii + half, bf16f(k1), step_tag(a));
          }
        } else {
          uint16_t *v = a.kv + kv_off(c, d.layer, 1, b, g, p);
          const uint16_t u0 = f2bf(v0), u1 = f2bf(v1);
          st_c16(v + ii, u0);
          st_c16(v + ii + half, u1);
          uint64_t *vn = c.kvn_buf + lay::kvn(c.max_batch, c.nkv, c.hd, d.layer, b, (int)g, 1);
          st_tag(vn + ii, bf16f(u0), step_tag(a));
          st_tag(vn + ii + half, bf16f(u1), step_tag(a));
        }
        break;
      }
      case OP_O:
        st_c(c.h_buf + lay::h(c.max_batch, c.H, 2 * d.layer + 1, b) + d.item0 + i, R[i]);
        break;
      case OP_FFN: {
        const float gt = R[2 * i], up = R[2 * i + 1];
        st_c(c.a_buf + lay::a(c.max_batch, c.F, d.layer, b) + d.item0 + i, gt / (1.0f + expf(-gt)) * up);
        break;
      }
      case OP_DOWN:
        st_c(c.h_buf + lay::h(c.max_batch, c.H, 2 * d.layer + 2, b) + d.item0 + i, R[i]);
        break;
      default:  // OP_LM
        G(step_logits(a))[lay::logits(c.V, b) + d.item0 + i] = R[i];
        break;
    }
  }
  if (d.op == OP_LM && a.next_tok) {
    // this unit's greedy candidate; each lane visits its rows in ascending
    // order, so strict comparisons keep the lowest index among equals
    float bv = -INFINITY;
    uint32_t bi = 0xffffffffu;
    for (uint32_t i = (uint32_t)lane; i < d.n_items; i += 64) {
      const float v = R[i];
      if (amax_better(v, d.item0 + i, bv, bi)) {
        bv = v;
        bi = d.item0 + i;
      }
    }
    amax_reduce(bv, bi);
    if (lane == 0) st_tag(a.amax + d.unit, bv, bi);
  }
}

// The greedy finisher's tokens: device-coherent stores (a later step of the
// launch reads them on other CUs), acknowledged before the token counter
// counts the step.  Positions are written by the launch's last step only,
// so a caller may pass the same buffer as positions and next_positions.
__device__ __forceinline__ void st_tok(int32_t *p, int32_t v) {
  __hip_atomic_store(G(reinterpret_cast<uint32_t *>(p)), (uint32_t)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void count_tokens(const Args &a) {
  wait_vm0();
  before_signal();
  if (lane_id() == 0)
    __hip_atomic_fetch_add(G(a.amax_ctr + kTokWord), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The last LM unit of the step to count itself picks the greedy token from
// every unit's candidate (each acknowledged before its unit counted) and
// writes it with the next position.
__device__ __forceinline__ void lm_greedy_finish(const Env &e, const Args &a) {
  const int lane = lane_id();
  uint32_t o = 0;
  before_signal();
  if (lane == 0)
    o = __hip_atomic_fetch_add(G(a.amax_ctr), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  o = __builtin_amdgcn_readfirstlane(o);
  if (o + 1u != step_amax_target(a)) return;
  poll_exit();  // the candidates read below were acknowledged before their units counted
  const rsrc_t r = rsrc(a.amax);
  float bv = -INFINITY;
  uint32_t bi = 0xffffffffu;
  for (uint32_t u = (uint32_t)lane; u < a.n_lm; u += 64) {
    const uint64_t w = ldt(r, u);
    const float v = tval(w);
    const uint32_t i = (uint32_t)(w >> 32);
    if (amax_better(v, i, bv, bi)) {
      bv = v;
      bi = i;
    }
  }
  amax_reduce(bv, bi);
  if (lane == 0) {
    st_tok(a.next_tok, (int32_t)bi);
    if (a.step_off + 1 == (int32_t)a.n_steps) G(a.next_pos)[0] = e.pos0 + 1;
  }
  count_tokens(a);
}

// I2 on registers (head_dim 64, splits of at most PF positions beyond the
// prefetch; the paged body takes every other case).  The first PF
// positions of the split that precede p are step-invariant (written by
// earlier steps), so their K/V are loaded before the unit's dependency
// gate; q and the new slot p are loaded after it.
template <int DPL, class Gate>
__device__ bool attn_body(const Env &e, const Args &a, const Instr &d, int h, int p, Gate gate) {
  const DevCtx &c = *e.cp;
  const int lane = lane_id();
  const int b = (int)d.b, g = (int)d.aux0, s = (int)d.aux1;
  const int j = g * c.G + h;
  constexpr int hd = 64 * DPL, PF = 20 / DPL;  // prefetch depth (register budget)
  const int lo = s * a.split_len;
  const int hi = min(lo + a.split_len, p + 1);
  const int nt0 = max(0, min(hi - lo, PF));
  const rsrc_t Kr = rsrc(a.kv + kv_off(c, d.layer, 0, b, g, lo));
  const rsrc_t Vr = rsrc(a.kv + kv_off(c, d.layer, 1, b, g, lo));
  uint16_t kk[PF][DPL], vv[PF][DPL];
  if (nt0 > 0) {
#pragma unroll
    for (int t = 0; t < PF; ++t) {
      const int tt = min(t, nt0 - 1);  // in bounds; unused beyond nt0
#pragma unroll
      for (int m = 0; m < DPL; ++m) {
        kk[t][m] = ldc16(Kr, (uint32_t)(tt * hd + lane + 64 * m) * 2);
        vv[t][m] = ldc16(Vr, (uint32_t)(tt * hd + lane + 64 * m) * 2);
      }
    }
  }
  if (!gate()) return false;
  // rows an earlier step of this launch wrote (positions from p - step_off
  // on) are complete only once the gate has passed: load them again
  if (a.step_off > 0 && lo + nt0 > p - a.step_off) {
#pragma unroll
    for (int t = 0; t < PF; ++t) {
      const int tt = min(t, nt0 - 1);
#pragma unroll
      for (int m = 0; m < DPL; ++m) {
        kk[t][m] = ldc16(Kr, (uint32_t)(tt * hd + lane + 64 * m) * 2);
        vv[t][m] = ldc16(Vr, (uint32_t)(tt * hd + lane + 64 * m) * 2);
      }
    }
  }
  float mrun = -INFINITY, lrun = 0.f, o[DPL], q[DPL];
  uint16_t kp[DPL], vp[DPL];
#pragma unroll
  for (int m = 0; m < DPL; ++m) o[m] = 0.f;
  if (lo < hi) {
    // lane = head dimension (dims lane + 64*m) for q, K and V
    const rsrc_t qr = rsrc(c.q_buf + lay::q(c.max_batch, c.nq, hd, d.layer, b, j));
    // the new slot p (written this step) comes from the tagged copy, never
    // from the cache
    const rsrc_t nr = rsrc(c.kvn_buf + lay::kvn(c.max_batch, c.nkv, hd, d.layer, b, g, 0));
    const bool has_p = p < hi;
    auto load = [&]() -> bool {
      bool ok = true;
#pragma unroll
      for (int m = 0; m < DPL; ++m) {
        const uint64_t wq = ldt(qr, (uint32_t)(lane + 64 * m));
        q[m] = tval(wq);
        ok = ok && tok(wq, step_tag(a));
        kp[m] = vp[m] = 0;
        if (has_p) {
          const uint64_t wk = ldt(nr, (uint32_t)(lane + 64 * m)), wv = ldt(nr, (uint32_t)(hd + lane + 64 * m));
          kp[m] = (uint16_t)((uint32_t)wk >> 16);  // exact: K and V arrive rounded to bf16
          vp[m] = (uint16_t)((uint32_t)wv >> 16);
          ok = ok && tok(wk, step_tag(a)) && tok(wv, step_tag(a));
        }
      }
      return ok;
    };
    if (!until_tagged(e, load, 0x800 | d.unit)) return false;
    // first PF positions from the prefetched registers
    {
      float sc = -INFINITY;
#pragma unroll
      for (int t = 0; t < PF; ++t) {
        const bool isp = lo + t == p;
        float pr = 0.f;
#pragma unroll
        for (int m = 0; m < DPL; ++m) pr = fmaf(q[m], bf16f(isp ? kp[m] : kk[t][m]), pr);
        const float st = wave_sum(pr) * c.attn_scale;
        if (lane == t && t < nt0) sc = st;
      }
      const float cm = wave_max(sc);
      const float pt = lane < nt0 ? expf(sc - cm) : 0.f;
      lrun = wave_sum(pt);
#pragma unroll
      for (int t = 0; t < PF; ++t) {
        const bool isp = lo + t == p;
        const float wt = t < nt0 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pt), t)) : 0.f;
#pragma unroll
        for (int m = 0; m < DPL; ++m) o[m] = fmaf(wt, bf16f(isp ? vp[m] : vv[t][m]), o[m]);
      }
      mrun = cm;
    }
    // remaining positions in chunks of 64, NR rows in flight
    constexpr int NR = DPL == 1 ? MK_ARB : 8;
#pragma unroll 1
    for (int c0 = lo + PF; c0 < hi; c0 += 64) {
      const int nt = min(64, hi - c0);
      float sc = -INFINITY;
#pragma unroll 1
      for (int t0 = 0; t0 < nt; t0 += NR) {
        uint16_t k8[NR][DPL];
#pragma unroll
        for (int t = 0; t < NR; ++t) {
          const int tt = min(t0 + t, nt - 1);
#pragma unroll
          for (int m = 0; m < DPL; ++m)
            k8[t][m] = c0 + tt == p ? kp[m] : ldc16(Kr, (uint32_t)((c0 - lo + tt) * hd + lane + 64 * m) * 2);
        }
#pragma unroll
        for (int t = 0; t < NR; ++t) {
          float pr = 0.f;
#pragma unroll
          for (int m = 0; m < DPL; ++m) pr = fmaf(q[m], bf16f(k8[t][m]), pr);
          const float st = wave_sum(pr) * c.attn_scale;
          if (lane == t0 + t && t0 + t < nt) sc = st;
        }
      }
      const bool valid = lane < nt;
      const float cm = wave_max(sc);
      const float mn = fmaxf(mrun, cm);
      const float pt = valid ? expf(sc - mn) : 0.f;
      const float scale = mrun == -INFINITY ? 0.f : expf(mrun - mn);
      lrun = lrun * scale + wave_sum(pt);
#pragma unroll
      for (int m = 0; m < DPL; ++m) o[m] *= scale;
#pragma unroll 1
      for (int t0 = 0; t0 < nt; t0 += NR) {
        uint16_t v8[NR][DPL];
#pragma unroll
        for (int t = 0; t < NR; ++t) {
          const int tt = min(t0 + t, nt - 1);  // in bounds; weight 0 beyond nt
#pragma unroll
          for (int m = 0; m < DPL; ++m)
            v8[t][m] = c0 + tt == p ? vp[m] : ldc16(Vr, (uint32_t)((c0 - lo + tt) * hd + lane + 64 * m) * 2);
        }
#pragma unroll
        for (int t = 0; t < NR; ++t) {
          const float wt = t0 + t < nt
                               ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pt), min(t0 + t, 63)))
                               : 0.f;
#pragma unroll
          for (int m = 0; m < DPL; ++m) o[m] = fmaf(wt, bf16f(v8[t][m]), o[m]);
        }
      }
      mrun = mn;
    }
  }
  float *out = a.part_buf + lay::part(c.max_batch, c.nq, a.n_split, hd, d.layer, b, j, s);
#pragma unroll
  for (int m = 0; m < DPL; ++m) st_c(out + lane + 64 * m, o[m]);
  if (lane == 0) {
    st_c(out + hd, mrun);
    st_c(out + hd + 1, lrun);
  }
  return true;
}

// I2 on paged K/V (head_dim 128, and splits longer than attn_body's register
// prefetch).  All compute waves work: wave cw takes query head h = cw % G
// and every WPH-th page of the split (WPH = 8 / G waves per head), so each
// K/V page is read from HBM once and from LDS by the G waves of its heads.
// Scores run one lane per row (a whole K row against q, no cross-lane
// reduction), P.V one 16-byte V chunk per lane; each wave keeps a running
// (m, l, o) and the WPH partials of a head are merged in LDS in wave order,
// so the result does not depend on timing.  The waves of rp == 0 fetch q
// (and, in the split holding p, this step's K/V from the tagged words),
// apply the per-head q/k RMSNorm and RoPE when the model has them, write
// the rotated, rounded K of slot p to the cache (head 0's wave), stage q in
// LDS for the other waves of the head, and fold row p into their partial.
// LDS: the unit's activation slot (an attention unit takes no activation
// piece) holds q [G][hd] and the merge area [G][WPH-1][hd + 2].
template <int DPL>
__device__ bool attn_paged(const Env &e, const Args &a, const Instr &d, int cw, int p, uint32_t n, uint32_t seq,
                           uint32_t &aq_t, uint32_t &am_t, int ring, int sent, uint32_t P, int xso) {
  const DevCtx &c = *e.cp;
  const int lane = lane_id();
  constexpr int hd = 64 * DPL, CPR = hd / 8, RPL = 64 / CPR, RPP = 8 * RPL;
  const int GQ = c.G, WPH = kNCW / GQ;
  const int h = cw % GQ, rp = cw / GQ;
  const int b = (int)d.b, g = (int)d.aux0, s = (int)d.aux1, j = g * GQ + h;
  int lo, hi;
  uint32_t nr;
  attn_geom(a, d, p, lo, hi, nr);
  const uint32_t np = (nr + RPP - 1) / RPP;
  const bool has_p = p >= lo && p < hi;
  float *Q = reinterpret_cast<float *>(smem + xso);
  float *MG = Q + GQ * hd + h * (WPH - 1) * (hd + 2);
  aq_t += (uint32_t)GQ;
  am_t += (uint32_t)(GQ * (WPH - 1));
  if (!spin_lds(e, [&]() { return lds_ld(L_XREADY) > seq; }, 0x210)) return false;
  float qv[DPL], kpv[DPL];
#pragma unroll
  for (int m = 0; m < DPL; ++m) qv[m] = kpv[m] = 0.f;
  const rsrc_t nrr = rsrc(c.kvn_buf + lay::kvn(c.max_batch, c.nkv, hd, d.layer, b, g, 0));
  if (rp == 0) {
    if (lo < hi) {
      float qnw[DPL], knw[DPL], rc = 0.f, rsn = 0.f;
      if constexpr (DPL == 2) {
        if (c.qk_norm) {
          // norm weights of dims lane and lane + 64, RoPE of pair (lane, lane + 64)
          const uint16_t *qn = G(c.layers)[d.layer].q_norm, *kn = G(c.layers)[d.layer].k_norm;
#pragma unroll
          for (int m = 0; m < DPL; ++m) {
            qnw[m] = bf16f(G(qn)[lane + 64 * m]);
            knw[m] = bf16f(G(kn)[lane + 64 * m]);
          }
          const uint64_t csw = *G(reinterpret_cast<const uint64_t *>(c.rope + lay::rope(hd, p, lane)));
          rc = __uint_as_float((uint32_t)csw);
          rsn = __uint_as_float((uint32_t)(csw >> 32));
        }
      }
      const rsrc_t qr = rsrc(c.q_buf + lay::q(c.max_batch, c.nq, hd, d.layer, b, j));
      auto load = [&]() -> bool {
        bool ok = true;
#pragma unroll
        for (int m = 0; m < DPL; ++m) {
          const uint64_t wq = ldt(qr, (uint32_t)(lane + 64 * m));
          qv[m] = tval(wq);
          ok = ok && tok(wq, step_tag(a));
          if (has_p) {
            const uint64_t wk = ldt(nrr, (uint32_t)(lane + 64 * m)), wv = ldt(nrr, (uint32_t)(hd + lane + 64 * m));
            kpv[m] = tval(wk);
            ok = ok && tok(wk, step_tag(a)) && tok(wv, step_tag(a));
          }
        }
        return ok;
      };
      if (!until_tagged(e, load, 0x800 | d.unit)) return false;
      if constexpr (DPL == 2) {
        if (c.qk_norm) {
          // RMSNorm over the head (eps inside the root, weight after), RoPE of
          // (lane, lane + 64); K of slot p is rounded to bf16 like the cache
          auto norm_rope = [&](float (&u)[DPL], const float (&w)[DPL]) {
            const float ss = wave_sum(u[0] * u[0] + u[1] * u[1]);
            const float r = 1.0f / sqrtf(ss / (float)hd + c.eps);
            const float a0 = u[0] * r * w[0], a1 = u[1] * r * w[1];
            u[0] = a0 * rc - a1 * rsn;
            u[1] = a1 * rc + a0 * rsn;
          };
          norm_rope(qv, qnw);
          if (has_p) {
            norm_rope(kpv, knw);
            const uint16_t k0 = f2bf(kpv[0]), k1 = f2bf(kpv[1]);
            kpv[0] = bf16f(k0);
            kpv[1] = bf16f(k1);
            if (h == 0) {
              uint16_t *kc = a.kv + kv_off(c, d.layer, 0, b, g, p);
              st_c16(kc + lane, k0);
              st_c16(kc + lane + 64, k1);
            }
          }
        }
      }
#pragma unroll
      for (int m = 0; m < DPL; ++m) Q[h * hd + lane + 64 * m] = qv[m];
    }
    wait_lgkm0();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (lane == 0) __hip_atomic_fetch_add(&lds_u32(L_AQ), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    wake();
  } else {
    if (!spin_lds(e, [&]() { return lds_ld(L_AQ) >= aq_t; }, 0x710)) return false;
  }
  // this wave's pages: running (m, l) per head and o over the 8 dims of
  // chunk lane % CPR, summed over the rows of lane / CPR
  float m_run = -INFINITY, l_run = 0.f, o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
  const float *Qh = Q + h * hd;
  const uint32_t t = (uint32_t)lane % RPP, hh = (uint32_t)lane / RPP;  // row of a page, half of it (hd 128)
  uint32_t rel = n;
  for (uint32_t jp = (uint32_t)rp; jp < np; jp += (uint32_t)WPH) {
    const uint32_t pg = n + jp;
    if (pg > rel) {
      if (lane == 0) lds_st(L_CONS + 4 * cw, pg);
      rel = pg;
      wake();
    }
    if (!spin_lds_fast(e, [&]() { return lds_ld(sent + (pg % P) * kSentBytes) == pg; }, 0x310)) return false;
    const uint32_t pb = (uint32_t)ring + (pg % P) * kPageBytes;
    // scores: lane t against K row t (chunks hh*8 .. hh*8+7), four chunks
    // in flight at a time
    const uint32_t rowa = lds_addr((int)(pb + (t / RPL) * 1024 + (t % RPL) * CPR * 16));
    float sc0 = 0.f, sc1 = 0.f;
#pragma unroll
    for (int c0 = 0; c0 < 8; c0 += 4) {
      u4 kc[4];
      asm volatile(
          "ds_read_b128 %0, %4\n\t"
          "ds_read_b128 %1, %5\n\t"
          "ds_read_b128 %2, %6\n\t"
          "ds_read_b128 %3, %7\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(kc[0]), "=&v"(kc[1]), "=&v"(kc[2]), "=&v"(kc[3])
          : "v"(rowa + (((hh * 8 + c0 + 0) ^ (t & 7)) << 4)), "v"(rowa + (((hh * 8 + c0 + 1) ^ (t & 7)) << 4)),
            "v"(rowa + (((hh * 8 + c0 + 2) ^ (t & 7)) << 4)), "v"(rowa + (((hh * 8 + c0 + 3) ^ (t & 7)) << 4)));
#pragma unroll
      for (int ci = 0; ci < 4; ++ci) {
        const f4 q0 = *reinterpret_cast<const f4 *>(Qh + (hh * 8 + c0 + ci) * 8);
        const f4 q1 = *reinterpret_cast<const f4 *>(Qh + (hh * 8 + c0 + ci) * 8 + 4);
        sc0 = fmaf(q0.x, bf_lo(kc[ci].x), sc0);
        sc1 = fmaf(q0.y, bf_hi(kc[ci].x), sc1);
        sc0 = fmaf(q0.z, bf_lo(kc[ci].y), sc0);
        sc1 = fmaf(q0.w, bf_hi(kc[ci].y), sc1);
        sc0 = fmaf(q1.x, bf_lo(kc[ci].z), sc0);
        sc1 = fmaf(q1.y, bf_hi(kc[ci].z), sc1);
        sc0 = fmaf(q1.z, bf_lo(kc[ci].w), sc0);
        sc1 = fmaf(q1.w, bf_hi(kc[ci].w), sc1);
      }
    }
    float sc = sc0 + sc1;
    if constexpr (DPL == 2) sc += __shfl_xor(sc, 32);
    sc *= c.attn_scale;
    const bool valid = (uint32_t)lane < (uint32_t)RPP && jp * RPP + t < nr;
    const float cm = wave_max(valid ? sc : -INFINITY);
    const float mn = fmaxf(m_run, cm);
    const float pt = valid ? expf(sc - mn) : 0.f;
    const float scl = m_run == -INFINITY ? 0.f : expf(m_run - mn);
    l_run = l_run * scl + wave_sum(pt);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= scl;
    m_run = mn;
    // P.V: wave-load jv holds rows jv*RPL + lane / CPR, chunk lane % CPR
    const uint32_t va = lds_addr((int)(pb + 8192 + lane * 16));
#pragma unroll
    for (int j0 = 0; j0 < 8; j0 += 4) {
      u4 vc[4];
      asm volatile(
          "ds_read_b128 %0, %4\n\t"
          "ds_read_b128 %1, %4 offset:1024\n\t"
          "ds_read_b128 %2, %4 offset:2048\n\t"
          "ds_read_b128 %3, %4 offset:3072\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(vc[0]), "=&v"(vc[1]), "=&v"(vc[2]), "=&v"(vc[3])
          : "v"(va + j0 * 1024));
#pragma unroll
      for (int jv = 0; jv < 4; ++jv) {
        const float w = __shfl(pt, (j0 + jv) * RPL + lane / CPR);
        o[0] = fmaf(w, bf_lo(vc[jv].x), o[0]);
        o[1] = fmaf(w, bf_hi(vc[jv].x), o[1]);
        o[2] = fmaf(w, bf_lo(vc[jv].y), o[2]);
        o[3] = fmaf(w, bf_hi(vc[jv].y), o[3]);
        o[4] = fmaf(w, bf_lo(vc[jv].z), o[4]);
        o[5] = fmaf(w, bf_hi(vc[jv].z), o[5]);
        o[6] = fmaf(w, bf_lo(vc[jv].w), o[6]);
        o[7] = fmaf(w, bf_hi(vc[jv].w), o[7]);
      }
    }
  }
  // one o per chunk: lanes of the same chunk hold different rows' sums
#pragma unroll
  for (int i = 0; i < 8; ++i)
    for (int off = CPR; off < 64; off <<= 1) o[i] += __shfl_xor(o[i], off);
  if (rp == 0 && has_p) {
    // row p: this step's K and V (the tagged words this wave verified)
    float pr = 0.f;
#pragma unroll
    for (int m = 0; m < DPL; ++m) pr = fmaf(qv[m], kpv[m], pr);
    const float sp = wave_sum(pr) * c.attn_scale;
    const float mn = fmaxf(m_run, sp);
    const float scl = m_run == -INFINITY ? 0.f : expf(m_run - mn);
    const float wp = expf(sp - mn);
    l_run = l_run * scl + wp;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = fmaf(wp, tval(ldt(nrr, (uint32_t)(hd + (lane % CPR) * 8 + i))), o[i] * scl);
    m_run = mn;
  }
  // merge the head's WPH partials in wave order
  if (WPH > 1) {
    if (rp > 0) {
      float *dst = MG + (rp - 1) * (hd + 2);
      if (lane < CPR) {
#pragma unroll
        for (int i = 0; i < 8; ++i) dst[lane * 8 + i] = o[i];
      }
      if (lane == 0) {
        dst[hd] = m_run;
        dst[hd + 1] = l_run;
      }
      wait_lgkm0();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (lane == 0) __hip_atomic_fetch_add(&lds_u32(L_AM), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      wake();
    } else {
      if (!spin_lds(e, [&]() { return lds_ld(L_AM) >= am_t; }, 0x720)) return false;
      for (int r = 1; r < WPH; ++r) {
        const float *src = MG + (r - 1) * (hd + 2);
        const float mr = src[hd], lr = src[hd + 1];
        if (mr == -INFINITY) continue;  // a part with no rows
        const float M = fmaxf(m_run, mr);
        const float fa = m_run == -INFINITY ? 0.f : expf(m_run - M), fb = expf(mr - M);
        l_run = l_run * fa + lr * fb;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = o[i] * fa + (lane < CPR ? src[lane * 8 + i] : 0.f) * fb;
        m_run = M;
      }
    }
  }
  if (rp == 0) {
    if (a.n_split == 1) {
      // one split per KV head: the merged partial is the attention output
      // (no reduction instruction follows)
      float *out = c.attn_buf + lay::attn(c.max_batch, c.nq, hd, d.layer, b) + (size_t)j * hd;
      const float inv = 1.0f / l_run;
      if (lane < CPR) {
#pragma unroll
        for (int i = 0; i < 8; ++i) st_c(out + lane * 8 + i, o[i] * inv);
      }
    } else {
      float *out = a.part_buf + lay::part(c.max_batch, c.nq, a.n_split, hd, d.layer, b, j, s);
      if (lane < CPR) {
#pragma unroll
        for (int i = 0; i < 8; ++i) st_c(out + lane * 8 + i, o[i]);
      }
      if (lane == 0) {
        st_c(out + hd, m_run);
        st_c(out + hd + 1, l_run);
      }
    }
  }
  wait_lgkm0();
  if (lane == 0) lds_st(L_CONS + 4 * cw, n + np);
  wake();
  return true;
}

// I3: log-sum-exp combine of the split partials of query head (g*G + h):
// m* = max m_s, w_s = exp(m_s - m*), out = sum w_s o_s / sum w_s l_s; empty
// splits (m = -inf) get weight 0.
template <int DPL>
__device__ __forceinline__ void red_body(const Env &e, const Args &a, const Instr &d, int h) {
  const DevCtx &c = *e.cp;
  const int lane = lane_id();
  const int b = (int)d.b, g = (int)d.aux0;
  const int j = g * c.G + h;
  constexpr int hd = 64 * DPL, dpl = DPL;
  const int ns = a.n_split;
  const float *base = a.part_buf + lay::part(c.max_batch, c.nq, ns, hd, d.layer, b, j, 0);
  const rsrc_t pr = rsrc(base);
  const uint32_t rowb = (uint32_t)(hd + 4) * 4;
  // m, l of every split and the first RB splits' o in one round trip
  constexpr int RB = 32 / DPL;  // splits per round trip (all 32 at head_dim 64)
  float ms = -INFINITY, ls = 0.f;
  float ov[RB][dpl];
  if (lane < ns) {
    ms = ldc1(pr, lane * rowb + hd * 4);
    ls = ldc1(pr, lane * rowb + hd * 4 + 4);
  }
#pragma unroll
  for (int t = 0; t < RB; ++t) {
    const int ss = min(t, ns - 1);  // in bounds; weight 0 beyond ns
#pragma unroll
    for (int m = 0; m < dpl; ++m) ov[t][m] = ldc1(pr, ss * rowb + (uint32_t)(lane + 64 * m) * 4);
  }
  const float mstar = wave_max(ms);
  const float ws = ms == -INFINITY ? 0.f : expf(ms - mstar);
  const float L = wave_sum(ws * ls);
  float o[dpl];
#pragma unroll
  for (int m = 0; m < dpl; ++m) o[m] = 0.f;
#pragma unroll 1
  for (int s0 = 0; s0 < ns; s0 += RB) {
    if (s0 > 0) {
#pragma unroll
      for (int t = 0; t < RB; ++t) {
        const int ss = min(s0 + t, ns - 1);
#pragma unroll
        for (int m = 0; m < dpl; ++m) ov[t][m] = ldc1(pr, ss * rowb + (uint32_t)(lane + 64 * m) * 4);
      }
    }
#pragma unroll
    for (int t = 0; t < RB; ++t) {
      const float w = s0 + t < ns ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ws), min(s0 + t, 63))) : 0.f;
#pragma unroll
      for (int m = 0; m < dpl; ++m) o[m] = fmaf(w, ov[t][m], o[m]);
    }
  }
  float *out = c.attn_buf + lay::attn(c.max_batch, c.nq, hd, d.layer, b) + (size_t)j * hd;
#pragma unroll
  for (int m = 0; m < dpl; ++m) st_c(out + lane + 64 * m, o[m] / L);
}

template <bool PAGED>
__device__ __forceinline__ void compute_role(const Env &e, const Args &a, int cw) {
  const DevCtx &c = *e.cp;
  const int lane = lane_id();
  const uint32_t P = (uint32_t)c.ring_pages;
  float *acc = reinterpret_cast<float *>(smem + L_ACC);
  uint32_t n = 0, seq = 0, aq_t = 0, am_t = 0;
  for (uint32_t qi = 0; qi < e.nq; ++qi) {
    const Instr d = e.q[qi];
    perturb(e, step_tag(a), qi, (uint32_t)(threadIdx.x >> 6));
    const bool gv = is_gemv(d.op);
    const uint32_t nx = gv ? d.nk : 1;
    uint32_t upages = d.pages;
    // gate: the first activation piece of the instruction is produced
    auto gate = [&]() { return spin_lds(e, [&]() { return lds_ld(L_XREADY) > seq; }, 0x200 | qi); };
    if (PAGED && d.op == OP_ATTN) {
      upages = attn_pages(a, d, e.pos0);
      const int xso = L_XS + (int)((seq % kNXS) * kXSlotBytes);
      bool ok = false;
      if constexpr (PAGED)
        ok = c.hd == 64 ? attn_paged<1>(e, a, d, cw, e.pos0, n, seq, aq_t, am_t, L_RING, L_SENT, P, xso)
                        : attn_paged<2>(e, a, d, cw, e.pos0, n, seq, aq_t, am_t, L_RING, L_SENT, P, xso);
      if (!ok) return;
    } else if (!PAGED && d.op == OP_ATTN && cw < c.G) {
      // head_dim 64, splits within the register prefetch
      if constexpr (!PAGED)
        if (!attn_body<1>(e, a, d, cw, e.pos0, gate)) return;
    } else if (!gate()) {
      return;
    }
    if (cw == 0 && lane == 0) trace_now(e, qi, 2);
    // this unit's staged row results
    float *acc = reinterpret_cast<float *>(smem + L_ACC + (qi & (kAccSlots - 1)) * kAccFloats * 4);
    if (gv) {
      // This wave owns unit rows r = cw, cw + kNCW, ... and visits only its
      // own pieces, in stream order: piece t = k*per + r lies at position
      // t % ppp of the unit's page t / ppp, so consecutive pieces of a page
      // belong to different waves and a page is released after one dot of
      // each.  Pages before the next own piece are released before waiting.
      const uint32_t per = d.n_items * d.ipw;
      const uint32_t ppp = d.ppp;
      const uint32_t n16 = d.pb >> 4;
      const uint32_t r0 = (uint32_t)cw;
      const bool has_resid = d.op == OP_O || d.op == OP_DOWN;  // acc preloaded
      uint32_t rel = n, wpg = 0xffffffffu;
      float xr[32];
      for (uint32_t k = 0; k < d.nk; ++k) {
        if (k > 0) {
          if (lane == 0) lds_st(L_XCONS + 4 * cw, seq + k);
          wake();  // the sync wave may wait for this activation slot
        }
        if (r0 >= per && k > 0) continue;
        // (a wave without rows passes the first piece's flag all the same)
        if (!spin_lds(e, [&]() { return lds_ld(L_XREADY) > seq + k; }, 0x400 | qi)) return;
        if (r0 >= per) continue;
        load_x(reinterpret_cast<const float *>(smem + L_XS + ((seq + k) % kNXS) * kXSlotBytes), n16, xr);
        const uint32_t t = k * per + r0;
        uint32_t pi = t / ppp, o = t - pi * ppp;
        for (uint32_t r = r0; r < per;) {
          const uint32_t pg = n + pi;
          if (pg != wpg) {
            if (pg > rel) {
              if (lane == 0) lds_st(L_CONS + 4 * cw, pg);
              rel = pg;
              wake();  // a loader may wait for a released slot
            }
            if (!spin_lds_fast(e, [&]() { return lds_ld(L_SENT + (pg % P) * kSentBytes) == pg; }, 0x300 | qi)) return;
            wpg = pg;
          }
          float v = dot_piece(smem + L_RING + (pg % P) * kPageBytes + o * d.pb, xr, n16);
          if (k > 0 || has_resid) v = acc[r] + v;  // k order fixed: deterministic
          if (lane == 0) acc[r] = v;
          r += kNCW;
          o += kNCW;
          while (o >= ppp) {
            o -= ppp;
            ++pi;
          }
        }
      }
      wait_lgkm0();
      if (lane == 0) lds_st(L_CONS + 4 * cw, n + d.pages);
      wake();
    } else if (d.op == OP_RED) {
      if (cw < c.G) {
        if (c.hd == 64) red_body<1>(e, a, d, cw);
        else red_body<2>(e, a, d, cw);
      }
    }
    n += upages;
    seq += nx;
    if (lane == 0) lds_st(L_XCONS + 4 * cw, seq);
    wake();
    // completion: the last wave to finish runs the epilogue and signals.
    // Results that other workgroups read as tagged words (q and the new K/V
    // slot, from QKV units) need no acknowledgement; plain fp32 results are
    // acknowledged before the counter moves.
    if (!gv) wait_vm0();  // attention partials / reduction output of this wave
    wait_lgkm0();         // staged results are in LDS
    uint32_t old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(&lds_u32(L_DONE + 4 * (qi & 3)), 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old == kNCW - 1) {
#if MK_PRIO
      __builtin_amdgcn_s_setprio(3);  // the epilogue is on the critical path
#endif
      if (lane == 0) trace_now(e, qi, 6);
      if (gv) {
        unit_epilogue(e, a, d, acc);
        if (d.op != OP_QKV) wait_vm0();
      }
      if (d.op == OP_LM && a.next_tok) lm_greedy_finish(e, a);
      before_signal();
      if (lane == 0) {
        trace_now(e, qi, 3);
        lds_st(L_DONE + 4 * (qi & 3), 0);
        lds_st(L_EPI, qi + 1);
        if (d.sig0 >= 0)
          __hip_atomic_fetch_add(G(a.ctr) + ((size_t)d.sig0 * kSlots + d.slot0) * kCtrStride, 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        if (d.sig1 >= 0)
          __hip_atomic_fetch_add(G(a.ctr) + ((size_t)d.sig1 * kSlots + d.slot1) * kCtrStride, 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
#if MK_PRIO
      __builtin_amdgcn_s_setprio(1);
#endif
    }
  }
}

// ==========================================================================
// Batched steps (2 to 8 sequences).  Each GEMV instruction is then a small
// dense contraction (the sequences x the unit's weight rows x K), which the
// matrix cores take: v_mfma_f32_16x16x32_bf16 multiplies a 16 x 32 block A of
// activations by a 32 x 16 block B of weights, accumulating in fp32
// ("L'interpréteur sur GPU", section 3.6: with a batch, the projections
// become compute-shaped products).  Activations stay fp32 between
// instructions; each value x enters the product as a bf16 pair, hi = bf16(x)
// and lo = bf16(x - hi), and the 16 rows of A are the hi parts of sequences
// 0..7 (rows 0..7) and their lo parts (rows 8..15), so one MFMA forms both
// halves of every product and the result of sequence s is D[s] + D[s + 8]
// (the bf16 multi-term split of Henry, Tang and Heinecke, 2019).
//
// Weights stream through the same ring of 16 KB pages, in MFMA order: a 1 KB
// block holds 8 weight rows x 64 elements, chunk-major (slot c*8 + r holds
// elements 8c .. 8c+7 of row r).  The loader gathers a block with one
// 16-byte load per lane, so every 8 lanes read one whole 128-byte line of a
// row; a compute wave reads the B operand of 16 rows x 32 elements from two
// blocks as eight 128-byte runs, free of LDS bank conflicts.  A unit's rows
// form 16-row tiles; compute waves split the tiles, then the K steps of a
// tile, and the last wave sums the waves' partial tiles in wave order, so the
// sum order is fixed.

typedef __bf16 bf8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t phys_k(const Instr &d, uint32_t k) { return lay::mfma_phys_k(k, d.nk, d.unit); }
// The K window of a batched GEMV unit: a split-K down unit covers one MLP
// chunk [koff, koff + klen) of its rows, every other unit the whole row.
__device__ __forceinline__ bool split_down(const Instr &d) { return d.op == OP_DOWN && lay::split_n(d.aux1) > 1; }
__device__ __forceinline__ void kwin(const Instr &d, uint32_t &koff, uint32_t &klen) {
  if (split_down(d)) {
    koff = lay::split_koff(d.aux0);
    klen = lay::split_klen(d.aux0);
  } else {
    koff = 0;
    klen = d.rowb >> 1;
  }
}

// LDS layout of the batched kernel (bytes; control words as above)
constexpr int LB_AMAX = 192;    // u64[8]  running greedy best per sequence of this workgroup
constexpr int LB_ACC = 256;     // f32 [kAccSlots][kAccFloats]: residual rows [row][seq], RoPE staging
constexpr int LB_PART = LB_ACC + kAccSlots * kAccFloats * 4;  // f32 [2][kNCW][128] partial tiles
// Activation staging: a piece's fp32 inputs of up to 8 sequences (rows of
// 256 elements, 1040 bytes apart so that the 8 sequences of one k-offset
// fall in different LDS banks) and its 256 bf16 norm weights.  kInflB pieces
// are in flight while the compute waves use another: a unit's pieces cost
// one memory round trip per kInflB of them, not one each.
#ifndef MK_BINFL
#define MK_BINFL 3
#endif
constexpr int kInflB = MK_BINFL;
constexpr int kNXSB = kInflB + 1;
constexpr int kXRowB = 1040;
constexpr int kXNwB = 8 * kXRowB;                              // norm weights within a slot
constexpr int kXSlotB = kXNwB + 512;
constexpr int LB_XS = LB_PART + 2 * kNCW * 128 * 4;
constexpr int LB_RING = ((LB_XS + kNXSB * kXSlotB + 1023) / 1024) * 1024;
// the weight ring takes what is left
constexpr int kRingPagesB = (kLdsBytes - LB_RING) / (kPageBytes + kSentBytes);
static_assert(kRingPagesB >= 4, "batched ring");
constexpr int LB_SENT = LB_RING + kRingPagesB * kPageBytes;
static_assert(LB_SENT + kRingPagesB * kSentBytes <= kLdsBytes, "batched LDS budget");
static_assert(LB_AMAX + 8 * 8 <= LB_ACC && L_EPI < LB_AMAX, "control words");

__device__ __forceinline__ int seq_pos(const Args &a, const DevCtx &c, int b) {
  const int p = a.positions[b] + a.step_off;
  return (p < 0 || p >= c.max_seq) ? 0 : p;
}

typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
typedef float f2v __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to bf16 (RNE) by the hardware conversion
// (v_cvt_pk_bf16_f32), first value in the low half.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2v{a, b}, bf2v));
}

// 8 consecutive fp32 values as the A operand of one lane: their hi parts, or
// (lo) what is left of each after its hi part, both bf16 (RNE).  x - hi is
// exact in fp32.  Branch-free: every lane converts twice and keeps the
// operand of its half of the wave.
__device__ __forceinline__ u4 pack_hilo(const float (&x)[8], bool lo) {
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float x0 = x[2 * j], x1 = x[2 * j + 1];
    const uint32_t h = cvt_pk_bf16(x0, x1);
    const float r0 = x0 - __uint_as_float(h << 16), r1 = x1 - __uint_as_float(h & 0xffff0000u);
    w[j] = cvt_pk_bf16(lo ? r0 : x0, lo ? r1 : x1);
  }
  return u4{w[0], w[1], w[2], w[3]};
}

// Start of weight row r of an MFMA unit, per lane (r < rows of the unit).
// Tabulated units (QKV pairs) read the 8 row addresses of block `rb` with
// uniform (scalar) loads and pick their own: a per-lane vector load would
// join the loader's direct-to-LDS loads in its wait counter.
__device__ __forceinline__ const char *row_start(const Instr &d, const uint64_t *__restrict__ rowtab, uint32_t rb,
                                                 uint32_t R, int lane) {
  const uint32_t r = min(rb * 8 + (uint32_t)(lane & 7), R - 1);
  if (d.tab >= 0) {
    uint64_t ent[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ent[i] = rowtab[d.tab + min(rb * 8 + (uint32_t)i, R - 1)];
    uint64_t mine = ent[0];
#pragma unroll
    for (int i = 1; i < 8; ++i)
      if ((lane & 7) == i) mine = ent[i];
    return reinterpret_cast<const char *>(mine);
  }
  uint64_t base;
  if (d.ipw == 2) base = ((r & 1) ? d.w1 : d.w0) + (uint64_t)(d.item0 + (r >> 1)) * d.rowb;
  else base = d.w0 + (uint64_t)(d.item0 + r) * d.rowb;
  return reinterpret_cast<const char *>(base);
}

template <bool PAGED>
__device__ __forceinline__ void loader_role_b(const Env &e, const Args &a, int lw) {
  const int lane = lane_id();
  constexpr uint32_t P = kRingPagesB;
  const char *zero = reinterpret_cast<const char *>(e.cp->zero);
  int npend = 0;
  auto min_cons = [&]() -> uint32_t {
    uint32_t v = lane < kNCW ? asm_lds_ld(L_CONS + 4 * lane) : 0xffffffffu;
    uint32_t m = __builtin_amdgcn_readlane(v, 0);
#pragma unroll
    for (int i = 1; i < kNCW; ++i) m = min(m, (uint32_t)__builtin_amdgcn_readlane(v, i));
    return m;
  };
  uint32_t n = 0;
  bool tok_ok = a.step_off == 0;
  for (uint32_t qi = 0; qi < e.nq; ++qi) {
    const Instr d = e.q[qi];
    perturb(e, step_tag(a), qi, (uint32_t)(threadIdx.x >> 6));
    if (PAGED && d.op == OP_ATTN) {
      if (!loader_tok_gate(e, tok_ok, qi)) {
        wait_vm0();
        return;
      }
      const DevCtx &c = *e.cp;
      int lo, hi;
      uint32_t nr;
      attn_geom(a, d, seq_pos(a, c, (int)d.b), lo, hi, nr);
      const uint32_t np = (nr + d.ppp - 1) / d.ppp;
      const char *Kb = reinterpret_cast<const char *>(a.kv + kv_off(c, d.layer, 0, (int)d.b, (int)d.aux0, lo));
      const char *Vb = reinterpret_cast<const char *>(a.kv + kv_off(c, d.layer, 1, (int)d.b, (int)d.aux0, lo));
      for (uint32_t jp = 0; jp < np; ++jp, ++n) {
        if ((int)(n % kNLW) != lw) continue;
        if (n >= P && min_cons() < n - P + 1) {
          const uint32_t need = n - P + 1;
          Watchdog wd;
          for (uint32_t it = 1;; ++it) {
            __builtin_amdgcn_s_sleep(MK_LSLEEP);
            if (min_cons() >= need) break;
            if ((it & 63) == 0) {
              if (__builtin_amdgcn_readfirstlane(asm_lds_ld(L_ABORT))) { wait_vm0(); return; }
              if (wd.expired(e.cp->watchdog_ticks)) { raise_error(e, 0xB0000000u | qi, n); wait_vm0(); return; }
            }
          }
        }
        if (npend == kSentDepth) {
          wait_vm_n<17 * (kSentDepth - 1)>();
          --npend;
        }
        LDS_AS char *slot = (LDS_AS char *)smem + LB_RING + (n % P) * kPageBytes;
        if (c.hd == 64) load_kv_page<8>(Kb, Vb, jp, nr, slot, lane);
        else load_kv_page<16>(Kb, Vb, jp, nr, slot, lane);
        __builtin_amdgcn_global_load_lds(a.iota + n, (LDS_AS void *)(smem + LB_SENT + (n % P) * kSentBytes), 4, 0, 0);
        ++npend;
      }
      continue;
    }
    if (!is_gemv(d.op)) continue;
    const uint32_t R = d.n_items * d.ipw, nrb = d.ppp;
    uint32_t koff, K;
    kwin(d, koff, K);
    const uint32_t nblk = (uint32_t)d.nk * nrb * 4;
    const bool wide = lay::mfma_wide(nrb);
    const uint32_t nk = d.nk, rot = MK_BROT ? d.unit % nk : 0u;  // (the piece rotation of lay::mfma_phys_k)
    const uint32_t lane_k = 8 * (uint32_t)(lane >> 3);
    uint32_t cur_rb = 0xffffffffu;
    const char *rowp = nullptr;
    for (uint32_t p = 0; p < d.pages; ++p, ++n) {
      if ((int)(n % kNLW) != lw) continue;
      if (n >= P && min_cons() < n - P + 1) {
        const uint32_t need = n - P + 1;
        Watchdog wd;
        for (uint32_t it = 1;; ++it) {
          __builtin_amdgcn_s_sleep(MK_LSLEEP);
          if (min_cons() >= need) break;
          if ((it & 63) == 0) {
            if (__builtin_amdgcn_readfirstlane(asm_lds_ld(L_ABORT))) { wait_vm0(); return; }
            if (wd.expired(e.cp->watchdog_ticks)) { raise_error(e, 0xB0000000u | qi, n); wait_vm0(); return; }
          }
        }
      }
      if (npend == kSentDepth) {
        wait_vm_n<17 * (kSentDepth - 1)>();
        --npend;
      }
      LDS_AS char *slot = (LDS_AS char *)smem + LB_RING + (n % P) * kPageBytes;
      // the page's first block by division, the rest by stepping (block
      // order of lay::mfma_block)
      uint32_t k, kb, rb;
      lay::mfma_block(p * 16 < nblk ? p * 16 : 0u, nrb, wide, k, kb, rb);
      for (uint32_t j = 0; j < 16; ++j) {
        if (p * 16 + j >= nblk) k = kb = rb = 0;  // tail of the last page: re-read the first block
        if (rb != cur_rb) {
          cur_rb = rb;
          rowp = row_start(d, a.rowtab, rb, R, lane);
        }
        const uint32_t kp = k + rot >= nk ? k + rot - nk : k + rot;
        const uint32_t kk = kp * kMfmaKc + kb * 64 + lane_k;
        const char *src = kk < K ? rowp + (size_t)(koff + kk) * 2 : zero;
        __builtin_amdgcn_global_load_lds(src, (LDS_AS void *)(slot + j * 1024), 16, 0, kWPol);
        if (wide) {
          if (++rb == nrb) {
            rb = 0;
            if (++kb == 4) {
              kb = 0;
              ++k;
            }
          }
        } else if (++kb == 4) {
          kb = 0;
          if (++rb == nrb) {
            rb = 0;
            ++k;
          }
        }
      }
      __builtin_amdgcn_global_load_lds(a.iota + n, (LDS_AS void *)(smem + LB_SENT + (n % P) * kSentBytes), 4, 0, 0);
      ++npend;
    }
  }
  wait_vm0();
}

// Load-count wait for the batched sync wave's pipeline: the loads of the
// younger pieces in flight (at most kInflB - 1 pieces of at most
// kMaxBatch + 1 loads; piece 0 of O and DOWN adds kMaxBatch residual
// loads, but it is never a younger piece).
template <int N>
__device__ __forceinline__ void wait_vm_sel(uint32_t n) {
  if constexpr (N == 0) {
    wait_vm_n<0>();
  } else {
    if (n >= (uint32_t)N) wait_vm_n<N>();
    else wait_vm_sel<N - 1>(n);
  }
}
static_assert((kInflB - 1) * (kMaxBatch + 1) <= 63, "load counter range");
__device__ __forceinline__ void wait_vm_le(uint32_t n) { wait_vm_sel<(kInflB - 1) * (kMaxBatch + 1)>(n); }

// The batched sync wave.  For each GEMV unit it copies the activation pieces
// (fp32 rows of every sequence, and the norm weights of normed units)
// global -> LDS with direct-to-LDS loads, kInflB pieces in flight, and
// publishes each piece once it has landed.  RMSNorm's scale 1/rms is a
// factor per sequence, so the product runs on the unnormalised h (times the
// norm weight) and the epilogue applies the factor: W (rs * h * w) =
// rs * (W (h * w)).  The sync wave accumulates each sequence's sum of
// squares from the pieces as they land and stores rs before it publishes
// the unit's last piece.  O and DOWN units also get their residual rows.
__device__ __forceinline__ void sync_role_b(const Env &e, const Args &a) {
  const DevCtx &c = *e.cp;
  const int lane = lane_id();
  const int B = a.batch;
  if (!wait_tokens(e, a)) return;
  for (int b = 0; b < B; ++b) {
    int32_t tk = ld_tok(a, b), ps = a.positions[b] + a.step_off;
    if (tk < 0 || tk >= c.V) { raise_error(e, 0xE1000000u, (uint32_t)b); return; }
    if (ps < 0 || ps >= c.max_seq) { raise_error(e, 0xE2000000u, (uint32_t)b); return; }
  }
  // lane b < B holds sequence b's token for the whole step
  const int32_t tok_all = lane < B ? ld_tok(a, lane) : 0;
  const char *zero = reinterpret_cast<const char *>(c.zero);
  uint32_t seq = 0;
  for (uint32_t qi = 0; qi < e.nq; ++qi) {
    const Instr d = e.q[qi];
    perturb(e, step_tag(a), qi, (uint32_t)(threadIdx.x >> 6));
    const bool gv = is_gemv(d.op);
    const uint32_t nx = gv ? d.nk : 1;
    const bool normed = d.op == OP_QKV || d.op == OP_FFN || d.op == OP_LM;
    const bool emb_in = d.op == OP_QKV && d.layer == 0;  // bf16 embedding rows
    float *accs = reinterpret_cast<float *>(smem + LB_ACC + (qi & (kAccSlots - 1)) * kAccFloats * 4);
    // Unit qi shares its LDS result slot and its completion counter with
    // unit qi - kAccSlots, whose epilogue must have finished before this
    // unit's slot is written (RoPE values, residual rows, 1/rms, below) and
    // before its ready flags let the compute waves use either: every compute
    // wave passes such a flag before it touches them.
    if (qi >= (uint32_t)kAccSlots &&
        !spin_lds(e, [&]() { return lds_ld(L_EPI) + kAccSlots > qi; }, 0x500 | qi))
      return;
    if (d.op == OP_QKV) {
      // RoPE cos/sin of each (pair, sequence) at that sequence's position,
      // staged before the waits
      const uint32_t half = (uint32_t)c.hd >> 1, ppg = (uint32_t)(c.G + 2) * half;
      for (uint32_t x = (uint32_t)lane; x < d.n_items * (uint32_t)B; x += 64) {
        const uint32_t i = x / (uint32_t)B, b = x - i * (uint32_t)B;
        const uint32_t ii = ((d.item0 + i) % ppg) % half;
        const uint64_t cs =
            *G(reinterpret_cast<const uint64_t *>(c.rope + lay::rope(c.hd, seq_pos(a, c, (int)b), (int)ii)));
        accs[kAccFloats / 2 + 2 * x] = __uint_as_float((uint32_t)cs);
        accs[kAccFloats / 2 + 2 * x + 1] = __uint_as_float((uint32_t)(cs >> 32));
      }
    }
    if (lane == 0) trace_now(e, qi, 4);
    uint32_t wi = 0;
    if (!gv) {
      // attention and reduction units: their waits, then their piece (a
      // paged attention unit keeps q and its merge in the slot)
      while (wi < d.wait_n) {
        if (!wait_group(e, a, a.waits[d.wait_off + wi], qi)) return;
        ++wi;
      }
      if (lane == 0) {
        trace_put(e, qi, 0, (uint64_t)d.op | ((uint64_t)d.layer << 8) | ((uint64_t)d.unit << 24));
        trace_now(e, qi, 1);
      }
      if (seq >= (uint32_t)kNXSB) {
        const uint32_t need = seq - kNXSB + 1;
        auto freed = [&]() {
          uint32_t v = lane < kNCW ? lds_ld_lane(L_XCONS + 4 * lane) : 0xffffffffu;
          uint32_t m = __builtin_amdgcn_readlane(v, 0);
#pragma unroll
          for (int i = 1; i < kNCW; ++i) m = min(m, (uint32_t)__builtin_amdgcn_readlane(v, i));
          return m >= need;
        };
        if (!spin_lds(e, freed, 0x100 | qi)) return;
      }
      if (lane == 0) lds_st(L_XREADY, seq + 1);
      wake();
      ++seq;
      continue;
    }
    uint32_t koff, K;
    kwin(d, koff, K);
    // The unit's input rows: sequence b's starts at src0 + b * sstr bytes,
    // its residual row (O, DOWN) at res0 + b * rstr.  They are computed once
    // per unit into registers: the compiler treats every direct-to-LDS load
    // as a possible store, and would re-read the context with a scalar
    // round trip per sequence if the issue loop derived them from it.
    const char *src0 = zero, *res0 = zero;
    uint32_t sstr = 0, rstr = (uint32_t)c.H * 4;
    const uint16_t *nw = nullptr;
    if (d.op == OP_O) {
      src0 = reinterpret_cast<const char *>(c.attn_buf + lay::attn(c.max_batch, c.nq, c.hd, d.layer, 0));
      sstr = (uint32_t)(c.nq * c.hd) * 4;
      res0 = reinterpret_cast<const char *>(c.h_buf + lay::h(c.max_batch, c.H, 2 * d.layer, 0) + d.item0 + lane);
    } else if (d.op == OP_DOWN) {
      src0 = reinterpret_cast<const char *>(c.a_buf + lay::a(c.max_batch, c.F, d.layer, 0) + koff);
      sstr = (uint32_t)c.F * 4;
      res0 = reinterpret_cast<const char *>(c.h_buf + lay::h(c.max_batch, c.H, 2 * d.layer + 1, 0) + d.item0 + lane);
    } else {
      const float *h;
      const uint16_t *emb;
      norm_src(e, d, 0, 0, h, emb, nw);
      if (h) src0 = reinterpret_cast<const char *>(h);
      sstr = (uint32_t)c.H * 4;
    }
    // layer 0's QKV widens the bf16 embedding rows of the step's tokens
    const uint16_t *embed = c.embed;
    const uint32_t Hs = (uint32_t)c.H;
    const int32_t tok_l = emb_in ? tok_all : 0;
    const uint32_t loads = (emb_in ? 0u : (uint32_t)B) + (normed ? 1u : 0u);
    float ss = 0.f;  // sum of squares of sequence lane >> 3, over this lane's part
    auto issue = [&](uint32_t k, uint32_t sq) -> uint32_t {
      LDS_AS char *slot = (LDS_AS char *)smem + LB_XS + (sq % kNXSB) * kXSlotB;
      const uint32_t kp = phys_k(d, k);
      const uint32_t e0 = kp * kMfmaKc + 4 * (uint32_t)lane;
      uint32_t nl = 0;
      if (!emb_in) {
        const char *src = src0 + (size_t)e0 * 4;
        for (int b = 0; b < B; ++b, src += sstr) {
          __builtin_amdgcn_global_load_lds(e0 < K ? src : zero, (LDS_AS void *)(slot + b * kXRowB), 16, 0, kSC1);
          ++nl;
        }
      }
      if (normed) {
        const uint32_t w0 = kp * kMfmaKc + 8 * (uint32_t)lane;
        if (lane < 32)
          __builtin_amdgcn_global_load_lds(w0 < K ? reinterpret_cast<const char *>(nw + w0) : zero,
                                           (LDS_AS void *)(slot + kXNwB), 16, 0, 0);
        ++nl;
      }
      if (k == 0 && (d.op == OP_O || d.op == OP_DOWN)) {
        // residual rows [sequence][64]: lane r < rows takes row r
        LDS_AS char *accl = (LDS_AS char *)smem + LB_ACC + (qi & (kAccSlots - 1)) * kAccFloats * 4;
        if (!(d.op == OP_O && d.layer == 0)) {  // (layer 0's O: the bf16 embedding, below)
          const char *res = res0;
          for (int b = 0; b < B; ++b, res += rstr) {
            if (lane < (int)d.n_items)
              __builtin_amdgcn_global_load_lds(res, (LDS_AS void *)(accl + b * 64 * 4), 4, 0, kSC1);
            ++nl;
          }
        }
      }
      return nl;
    };
    // the landed piece in slot sq: embedding rows (layer 0), sums of squares
    auto land = [&](uint32_t k, uint32_t sq) {
      LDS_AS char *slot = (LDS_AS char *)smem + LB_XS + (sq % kNXSB) * kXSlotB;
      if (emb_in) {
        // bf16 embedding rows of every sequence, widened into the slot
        for (int b = 0; b < B; ++b) {
          const uint32_t e0 = phys_k(d, k) * kMfmaKc + 4 * (uint32_t)lane;
          const int32_t tk = __builtin_amdgcn_readlane(tok_l, b);
          f4 v = {0.f, 0.f, 0.f, 0.f};
          if (e0 < K) {
            const uint64_t uu = *G(reinterpret_cast<const uint64_t *>(embed + (size_t)tk * Hs + e0));
            v = f4{bf_lo((uint32_t)uu), bf_hi((uint32_t)uu), bf_lo((uint32_t)(uu >> 32)), bf_hi((uint32_t)(uu >> 32))};
          }
          *reinterpret_cast<LDS_AS f4 *>(slot + b * kXRowB + lane * 16) = v;
        }
        wait_lgkm0();
      }
      if (normed) {
        // lane l: 32 elements of sequence l >> 3
        const int b = lane >> 3;
        if (b < B) {
          const LDS_AS f4 *row = reinterpret_cast<const LDS_AS f4 *>(slot + b * kXRowB);
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const f4 v = row[m * 8 + (lane & 7)];
            ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
          }
        }
      }
    };
    int64_t t_first = 0, t_last = 0;
    uint32_t issued = 0, done = 0;
    uint32_t nl[kNXSB] = {};  // loads of each piece in flight (by piece % kNXSB)
    while (done < nx) {
      if (issued < nx && issued - done < (uint32_t)kInflB) {
        // waits of piece `issued`, then a free slot (every compute wave
        // released the piece kNXSB before it)
        while (wi < d.wait_n) {
          const Wait wt = a.waits[d.wait_off + wi];
          // (a rotated piece order takes every wait before its first piece)
          if (!MK_BROT && wt.before_k > issued) break;
          if (!wait_group(e, a, wt, qi)) { wait_vm0(); return; }
          ++wi;
        }
        if (issued == 0 && lane == 0) {
          trace_put(e, qi, 0, (uint64_t)d.op | ((uint64_t)d.layer << 8) | ((uint64_t)d.unit << 24));
          trace_now(e, qi, 1);
        }
        const uint32_t sq = seq + issued;
        if (sq >= (uint32_t)kNXSB) {
          const uint32_t need = sq - kNXSB + 1;
          auto freed = [&]() {
            uint32_t v = lane < kNCW ? lds_ld_lane(L_XCONS + 4 * lane) : 0xffffffffu;
            uint32_t m = __builtin_amdgcn_readlane(v, 0);
#pragma unroll
            for (int i = 1; i < kNCW; ++i) m = min(m, (uint32_t)__builtin_amdgcn_readlane(v, i));
            return m >= need;
          };
          if (!spin_lds(e, freed, 0x100 | qi)) { wait_vm0(); return; }
        }
        nl[issued % kNXSB] = issue(issued, sq);
        ++issued;
      } else {
        // the oldest piece in flight has landed once only the younger
        // pieces' loads are outstanding
        uint32_t younger = 0;
        for (uint32_t q = done + 1; q < issued; ++q) younger += nl[q % kNXSB];
        wait_vm_le(younger);
        land(done, seq + done);
        if (done + 1 == nx && normed) {
          // every piece is in: 1/rms of each sequence (lanes 8b .. 8b+7
          // hold sequence b's partial sums) into the unit's result slot
          ss += __shfl_xor(ss, 1);
          ss += __shfl_xor(ss, 2);
          ss += __shfl_xor(ss, 4);
          if ((lane & 7) == 0 && (lane >> 3) < B) accs[lane >> 3] = 1.0f / sqrtf(ss / (float)c.H + c.eps);
        }
        if (d.op == OP_O && d.layer == 0 && done == 0) {
          // layer 0's residual is the bf16 embedding row
          for (int b = 0; b < B; ++b) {
            const int32_t tk = __builtin_amdgcn_readlane(tok_all, b);
            if ((uint32_t)lane < d.n_items) accs[b * 64 + lane] = bf16f(G(c.embed)[(size_t)tk * c.H + d.item0 + lane]);
          }
        }
        wait_lgkm0();
        if (lane == 0) lds_st(L_XREADY, seq + done + 1);
        wake();
        if (done == 0) t_first = now();
        if (done + 1 == nx) t_last = now();
        ++done;
      }
    }
    if (lane == 0) {
      trace_put(e, qi, 5, (uint64_t)t_first);
      trace_put(e, qi, 7, (uint64_t)t_last);
    }
    seq += nx;
  }
}

// The summed result of weight row r (within the unit) for sequence s, from
// the waves' partial tiles: tile r / 16 was computed by waves t, t + T, ...
// Within a wave's partial, lanes 0..31 hold D[s][n] for s = 4*(lane/16) + j
// (register j), n = lane % 16, after the hi and lo halves were added.
__device__ __forceinline__ float tile_sum(const float *Pb, uint32_t T, uint32_t r, uint32_t s) {
  const uint32_t t = r >> 4, nn = r & 15;
  const uint32_t idx = (((s >> 2) * 16 + nn) << 2) + (s & 3);
  float v = Pb[t * 128 + idx];
  for (uint32_t w = t + T; w < (uint32_t)kNCW; w += T) v += Pb[w * 128 + idx];
  return v;
}

__device__ __forceinline__ bool unit_epilogue_b(const Env &e, const Args &a, const Instr &d, const float *accs,
                                                const float *Pb) {
  const DevCtx &c = *e.cp;
  const int lane = lane_id();
  const uint32_t B = (uint32_t)a.batch;
  const uint32_t T = ((uint32_t)d.ppp + 1) >> 1;
  if (split_down(d)) {
    // the chunk's partial rows, acknowledged, then this unit's arrival; the
    // row group's last arrival sums the chunks in chunk order onto the
    // residual (the same order whichever unit arrives last) and signals
    const uint32_t S = lay::split_n(d.aux1), sp = lay::split_s(d.aux1);
    float *dp0 = a.part_buf + lay::part_size(c.L, c.max_batch, c.nq, a.n_split, c.hd);
    for (uint32_t x = (uint32_t)lane; x < d.n_items * B; x += 64) {
      const uint32_t i = x / B, b = x - i * B;
      st_c(dp0 + lay::dpart(c.H, c.max_batch, (int)S, d.layer, (int)sp, (int)(d.item0 + i), (int)b),
           tile_sum(Pb, T, i, b));
    }
    wait_vm0();
    before_signal();
    uint32_t old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(G(a.amax_ctr) + kCtrStride + lay::split_group(d.aux1), 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old + 1u != S * step_epoch(a)) return false;
    poll_exit();
    const rsrc_t pr = rsrc(dp0);
    for (uint32_t x = (uint32_t)lane; x < d.n_items * B; x += 64) {
      const uint32_t i = x / B, b = x - i * B;
      float v = accs[b * 64 + i];
      for (uint32_t s2 = 0; s2 < S; ++s2)
        v += ldc1(pr, (uint32_t)lay::dpart(c.H, c.max_batch, (int)S, d.layer, (int)s2, (int)(d.item0 + i), (int)b) * 4);
      st_c(c.h_buf + lay::h(c.max_batch, c.H, 2 * d.layer + 2, (int)b) + d.item0 + i, v);
    }
    return true;
  }
  if (T > (uint32_t)kNCW) {
    // a wide LM unit: the waves stored the logits; merge their candidates
    // (in wave order) into the workgroup's running best per sequence
    if (!a.next_tok) return true;
    uint64_t *run = reinterpret_cast<uint64_t *>(smem + LB_AMAX);
    const uint64_t *cand = reinterpret_cast<const uint64_t *>(Pb);
    if ((uint32_t)lane < B) {
      float bv = -INFINITY;
      uint32_t bi = 0xffffffffu;
      for (int w = 0; w < kNCW; ++w) {
        const uint64_t x = cand[w * 8 + lane];
        const float v = __uint_as_float((uint32_t)x);
        const uint32_t i = (uint32_t)(x >> 32);
        if (amax_better(v, i, bv, bi)) {
          bv = v;
          bi = i;
        }
      }
      if (!(d.aux1 & 1u)) {
        const uint64_t w = run[lane];
        const float ov = __uint_as_float((uint32_t)w);
        const uint32_t oi = (uint32_t)(w >> 32);
        if (amax_better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      run[lane] = ((uint64_t)bi << 32) | __float_as_uint(bv);
      if (d.aux1 & 2u) st_tag(a.amax + (size_t)d.aux0 * B + lane, bv, bi);
    }
    wait_lgkm0();
    return true;
  }
  // normed units: the sequence's 1/rms (accs[b]); O, DOWN: residual rows
  // accs[b * 64 + row]
  for (uint32_t x = (uint32_t)lane; x < d.n_items * B; x += 64) {
    const uint32_t i = x / B, b = x - i * B;
    switch (d.op) {
      case OP_QKV: {
        const float rsb = accs[b];
        const float v0 = tile_sum(Pb, T, 2 * i, b) * rsb, v1 = tile_sum(Pb, T, 2 * i + 1, b) * rsb;
        const uint32_t half = (uint32_t)c.hd >> 1;
        const uint32_t ppg = (uint32_t)(c.G + 2) * half;
        const uint32_t pp = d.item0 + i, g = pp / ppg, rr = pp - g * ppg;
        const uint32_t hs = rr / half, ii = rr - hs * half;
        const int p = seq_pos(a, c, (int)b);
        if (hs <= (uint32_t)c.G) {
          const float cs = accs[kAccFloats / 2 + 2 * x], sn = accs[kAccFloats / 2 + 2 * x + 1];
          const float r0 = v0 * cs - v1 * sn, r1 = v1 * cs + v0 * sn;
          if (hs < (uint32_t)c.G) {
            uint64_t *q = c.q_buf + lay::q(c.max_batch, c.nq, c.hd, d.layer, (int)b, (int)(g * c.G + hs));
            st_tag(q + ii, r0, step_tag(a));
            st_tag(q + ii + half, r1, step_tag(a));
          } else {
            uint16_t *k = a.kv + kv_off(c, d.layer, 0, (int)b, (int)g, p);
            const uint16_t k0 = f2bf(r0), k1 = f2bf(r1);
            st_c16(k + ii, k0);
            st_c16(k + ii + half, k1);
            uint64_t *kn = c.kvn_buf + lay::kvn(c.max_batch, c.nkv, c.hd, d.layer, (int)b, (int)g, 0);
            st_tag(kn + ii, bf16f(k0), step_tag(a));
            st_tag(kn + ii + half, bf16f(k1), step_tag(a));
          }
        } else {
          uint16_t *v = a.kv + kv_off(c, d.layer, 1, (int)b, (int)g, p);
          const uint16_t u0 = f2bf(v0), u1 = f2bf(v1);
          st_c16(v + ii, u0);
          st_c16(v + ii + half, u1);
          uint64_t *vn = c.kvn_buf + lay::kvn(c.max_batch, c.nkv, c.hd, d.layer, (int)b, (int)g, 1);
          st_tag(vn + ii, bf16f(u0), step_tag(a));
          st_tag(vn + ii + half, bf16f(u1), step_tag(a));
        }
        break;
      }
      case OP_O:
        st_c(c.h_buf + lay::h(c.max_batch, c.H, 2 * d.layer + 1, (int)b) + d.item0 + i,
             accs[b * 64 + i] + tile_sum(Pb, T, i, b));
        break;
      case OP_FFN: {
        const float gt = tile_sum(Pb, T, 2 * i, b) * accs[b], up = tile_sum(Pb, T, 2 * i + 1, b) * accs[b];
        st_c(c.a_buf + lay::a(c.max_batch, c.F, d.layer, (int)b) + d.item0 + i, gt / (1.0f + expf(-gt)) * up);
        break;
      }
      case OP_DOWN:
        st_c(c.h_buf + lay::h(c.max_batch, c.H, 2 * d.layer + 2, (int)b) + d.item0 + i,
             accs[b * 64 + i] + tile_sum(Pb, T, i, b));
        break;
      default:  // OP_LM
        G(step_logits(a))[lay::logits(c.V, (int)b) + d.item0 + i] = tile_sum(Pb, T, i, b) * accs[b];
        break;
    }
  }
  if (d.op == OP_LM && a.next_tok) {
    // per sequence: this unit's best row, merged into the workgroup's
    // running best (LM units of a workgroup run their epilogues in queue
    // order); the workgroup's last LM unit publishes it
    uint64_t *run = reinterpret_cast<uint64_t *>(smem + LB_AMAX);
    for (uint32_t b = 0; b < B; ++b) {
      float bv = -INFINITY;
      uint32_t bi = 0xffffffffu;
      for (uint32_t i = (uint32_t)lane; i < d.n_items; i += 64) {
        const float v = tile_sum(Pb, T, i, b) * accs[b];
        if (amax_better(v, d.item0 + i, bv, bi)) {
          bv = v;
          bi = d.item0 + i;
        }
      }
      amax_reduce(bv, bi);
      if (!(d.aux1 & 1u)) {
        const uint64_t w = run[b];
        const float ov = __uint_as_float((uint32_t)w);
        const uint32_t oi = (uint32_t)(w >> 32);
        if (amax_better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if (lane == 0) run[b] = ((uint64_t)bi << 32) | __float_as_uint(bv);
      if ((d.aux1 & 2u) && lane == 0) st_tag(a.amax + (size_t)d.aux0 * B + b, bv, bi);
    }
    wait_lgkm0();
  }
  return true;
}

// The last LM workgroup of the step to count itself picks every sequence's
// greedy token from the workgroups' published candidates.
__device__ __forceinline__ void lm_greedy_finish_b(const Env &e, const Args &a) {
  const DevCtx &c = *e.cp;
  const int lane = lane_id();
  uint32_t o = 0;
  before_signal();
  if (lane == 0)
    o = __hip_atomic_fetch_add(G(a.amax_ctr), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  o = __builtin_amdgcn_readfirstlane(o);
  if (o + 1u != step_amax_target(a)) return;
  poll_exit();
  const rsrc_t r = rsrc(a.amax);
  const uint32_t B = (uint32_t)a.batch;
  for (uint32_t b = 0; b < B; ++b) {
    float bv = -INFINITY;
    uint32_t bi = 0xffffffffu;
    for (uint32_t u = (uint32_t)lane; u < a.n_lm; u += 64) {
      const uint64_t w = ldt(r, u * B + b);
      const float v = tval(w);
      const uint32_t i = (uint32_t)(w >> 32);
      if (amax_better(v, i, bv, bi)) {
        bv = v;
        bi = i;
      }
    }
    amax_reduce(bv, bi);
    if (lane == 0) {
      st_tok(a.next_tok + b, (int32_t)bi);
      if (a.step_off + 1 == (int32_t)a.n_steps) G(a.next_pos)[b] = seq_pos(a, c, (int)b) + 1;
    }
  }
  count_tokens(a);
}

// A wide LM-head unit (more than 8 row tiles): compute wave cw owns the
// whole tiles t = cw, cw + 8, ... (at most 4), so no partial tiles are summed
// across waves.  Per piece it builds the 8 A operands once and runs them
// against each of its tiles in turn; tile by tile, the waves walk the pages
// of a piece in order.  The wave then stores its rows' logits and leaves
// each sequence's best (logit, row) of its rows in the candidate area.
__device__ bool gemv_wide_b(const Env &e, const Args &a, const Instr &d, int cw, uint32_t n, uint32_t seq,
                            uint32_t qi, const float *accs, uint64_t *cand) {
  const DevCtx &c = *e.cp;
  const int lane = lane_id();
  constexpr uint32_t P = kRingPagesB;
  const uint32_t nrb = d.ppp, T = (nrb + 1) >> 1, R = d.n_items;
  const uint32_t ntw = (T - (uint32_t)cw + kNCW - 1) / kNCW;
  const bool upper = (lane & 15) >= 8;
  const uint32_t brow = (uint32_t)(((lane >> 4) * 8 + (lane & 7)) * 16);
  const int sA = lane & 7;
  const bool loA = (lane & 15) >= 8, liveA = sA < a.batch;
  const uint32_t kA = 8 * (uint32_t)(lane >> 4);
  f4 acc[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = f4{0.f, 0.f, 0.f, 0.f};
  uint32_t rel = n, v0 = 0xffffffffu, v1 = 0xffffffffu;
  for (uint32_t k = 0; k < d.nk; ++k) {
    if (k > 0) {
      if (lane == 0) lds_st(L_XCONS + 4 * cw, seq + k);
      wake();
    }
    if (!spin_lds(e, [&]() { return lds_ld(L_XREADY) > seq + k; }, 0x400 | qi)) return false;
    const uint32_t slot = (uint32_t)LB_XS + ((seq + k) % kNXSB) * kXSlotB;
    for (uint32_t kb = 0; kb < 4; ++kb) {
      // the A operands of K steps 2kb and 2kb + 1 (64 elements of the piece)
      u4 A[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t ks = 2 * kb + (uint32_t)h;
        const uint32_t xaddr = lds_addr((int)(slot + sA * kXRowB + (ks * 32 + kA) * 4));
        const uint32_t waddr = lds_addr((int)(slot + kXNwB + (ks * 32 + kA) * 2));
        u4 x0, x1, wv;
        asm volatile(
            "ds_read_b128 %0, %3\n\t"
            "ds_read_b128 %1, %3 offset:16\n\t"
            "ds_read_b128 %2, %4\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(x0), "=&v"(x1), "=&v"(wv)
            : "v"(xaddr), "v"(waddr));
        float x[8] = {__uint_as_float(x0.x), __uint_as_float(x0.y), __uint_as_float(x0.z), __uint_as_float(x0.w),
                      __uint_as_float(x1.x), __uint_as_float(x1.y), __uint_as_float(x1.z), __uint_as_float(x1.w)};
        x[0] *= bf_lo(wv.x); x[1] *= bf_hi(wv.x); x[2] *= bf_lo(wv.y); x[3] *= bf_hi(wv.y);
        x[4] *= bf_lo(wv.z); x[5] *= bf_hi(wv.z); x[6] *= bf_lo(wv.w); x[7] *= bf_hi(wv.w);
        if (!liveA) {
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = 0.f;
        }
        A[h] = pack_hilo(x, loA);
      }
#pragma unroll
      for (uint32_t r = 0; r < 4; ++r) {
        if (r >= ntw) break;
        const uint32_t t = (uint32_t)cw + kNCW * r;
        const uint32_t Llo = lay::mfma_block_index(k, kb, 2 * t, nrb, true);
        const uint32_t Lhi = lay::mfma_block_index(k, kb, min(2 * t + 1, nrb - 1), nrb, true);
        const uint32_t pgA = n + (Llo >> 4), pgB = n + (Lhi >> 4);
        if (pgA > rel) {
          if (lane == 0) lds_st(L_CONS + 4 * cw, pgA);
          rel = pgA;
          wake();
        }
        for (uint32_t pg = pgA; pg <= pgB; ++pg) {
          if (pg == v0 || pg == v1) continue;
          if (!spin_lds_fast(e, [&]() { return lds_ld(LB_SENT + (pg % P) * kSentBytes) == pg; }, 0x300 | qi))
            return false;
          v0 = v1;
          v1 = pg;
        }
        const uint32_t Lb = upper ? Lhi : Llo, pg = n + (Lb >> 4);
        const uint32_t baddr = lds_addr(LB_RING + (int)((pg % P) * kPageBytes + (Lb & 15) * 1024 + brow));
        u4 b0, b1;
        asm volatile(
            "ds_read_b128 %0, %2\n\t"
            "ds_read_b128 %1, %2 offset:512\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(b0), "=&v"(b1)
            : "v"(baddr));
        acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, A[0]), __builtin_bit_cast(bf8v, b0),
                                                        acc[r], 0, 0, 0);
        acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, A[1]), __builtin_bit_cast(bf8v, b1),
                                                        acc[r], 0, 0, 0);
      }
    }
  }
  // hi + lo halves (lanes l and l + 32), then lane l < 32 holds rows
  // t*16 + l % 16 for sequences 4*(l/16) .. 4*(l/16) + 3
  float bvv[4];
  uint32_t bii[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bvv[j] = -INFINITY;
    bii[j] = 0xffffffffu;
  }
  const uint32_t B = (uint32_t)a.batch;
#pragma unroll
  for (uint32_t r = 0; r < 4; ++r) {
    if (r >= ntw) break;
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[r][j] += __shfl_xor(acc[r][j], 32);
    const uint32_t row = ((uint32_t)cw + kNCW * r) * 16 + (uint32_t)(lane & 15);
    if (lane < 32 && row < R) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t sq = 4 * (uint32_t)(lane >> 4) + (uint32_t)j;
        if (sq < B) {
          const float v = acc[r][j] * accs[sq];
          G(step_logits(a))[lay::logits(c.V, (int)sq) + d.item0 + row] = v;
          if (amax_better(v, d.item0 + row, bvv[j], bii[j])) {
            bvv[j] = v;
            bii[j] = d.item0 + row;
          }
        }
      }
    }
  }
  if (a.next_tok) {
    // best of the 16 lanes that share a sequence group
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const float ov = __shfl_xor(bvv[j], off);
        const uint32_t oi = (uint32_t)__shfl_xor((int)bii[j], off);
        if (amax_better(ov, oi, bvv[j], bii[j])) {
          bvv[j] = ov;
          bii[j] = oi;
        }
      }
    }
    if (lane == 0 || lane == 16) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        cand[cw * 8 + 4 * (lane >> 4) + j] = ((uint64_t)bii[j] << 32) | __float_as_uint(bvv[j]);
    }
  }
  return true;
}

template <bool PAGED>
__device__ __forceinline__ void compute_role_b(const Env &e, const Args &a, int cw) {
  const DevCtx &c = *e.cp;
  const int lane = lane_id();
  constexpr uint32_t P = kRingPagesB;
  uint32_t n = 0, seq = 0, aq_t = 0, am_t = 0;
  for (uint32_t qi = 0; qi < e.nq; ++qi) {
    const Instr d = e.q[qi];
    perturb(e, step_tag(a), qi, (uint32_t)(threadIdx.x >> 6));
    const bool gv = is_gemv(d.op);
    const uint32_t nx = gv ? d.nk : 1;
    uint32_t upages = d.pages;
    auto gate = [&]() { return spin_lds(e, [&]() { return lds_ld(L_XREADY) > seq; }, 0x200 | qi); };
    if (PAGED && d.op == OP_ATTN) {
      const int p = seq_pos(a, c, (int)d.b);
      upages = attn_pages(a, d, p);
      const int xso = LB_XS + (int)((seq % kNXSB) * kXSlotB);
      bool ok = false;
      if constexpr (PAGED)
        ok = c.hd == 64 ? attn_paged<1>(e, a, d, cw, p, n, seq, aq_t, am_t, LB_RING, LB_SENT, P, xso)
                        : attn_paged<2>(e, a, d, cw, p, n, seq, aq_t, am_t, LB_RING, LB_SENT, P, xso);
      if (!ok) return;
    } else if (!PAGED && d.op == OP_ATTN && cw < c.G) {
      if constexpr (!PAGED)
        if (!attn_body<1>(e, a, d, cw, seq_pos(a, c, (int)d.b), gate)) return;
    } else if (!gv && !gate()) {
      return;
    }
    if (cw == 0 && lane == 0) trace_now(e, qi, 2);
    const float *accs = reinterpret_cast<const float *>(smem + LB_ACC + (qi & (kAccSlots - 1)) * kAccFloats * 4);
    float *Pb = reinterpret_cast<float *>(smem + LB_PART + (qi & 1) * kNCW * 128 * 4);
    if (gv && ((uint32_t)d.ppp + 1) / 2 > (uint32_t)kNCW) {
      // (the candidate area is the partial-tile buffer, last read by unit
      // qi - 2's epilogue)
      if (qi >= 2 && !spin_lds(e, [&]() { return lds_ld(L_EPI) + 1 >= qi; }, 0x600 | qi)) return;
      if (!gemv_wide_b(e, a, d, cw, n, seq, qi, accs, reinterpret_cast<uint64_t *>(Pb))) return;
      wait_lgkm0();
      if (lane == 0) lds_st(L_CONS + 4 * cw, n + d.pages);
      wake();
    } else if (gv) {
      const uint32_t nrb = d.ppp, T = (nrb + 1) >> 1;
      const uint32_t t = (uint32_t)cw % T, nwt = ((uint32_t)kNCW - 1 - t) / T + 1, kg = (uint32_t)cw / T;
      const uint32_t rb_lo = 2 * t, rb_hi = min(2 * t + 1, nrb - 1);
      const bool upper = (lane & 15) >= 8;
      // this lane's offsets within a block, and its A row: sequence sA's
      // hi (rows 0..7) or lo (rows 8..15) part, elements kA .. kA+7 of a step
      const uint32_t brow = (uint32_t)(((lane >> 4) * 8 + (lane & 7)) * 16);
      const int sA = lane & 7;
      const bool loA = (lane & 15) >= 8, liveA = sA < a.batch;
      const bool normed = d.op == OP_QKV || d.op == OP_FFN || d.op == OP_LM;
      const uint32_t kA = 8 * (uint32_t)(lane >> 4);
      f4 acc = {0.f, 0.f, 0.f, 0.f};
      uint32_t rel = n, v0 = 0xffffffffu, v1 = 0xffffffffu;
      // this wave's K steps of 32: j = kg, kg + nwt, ... (nwt <= 8, so every
      // piece k = j / 8 holds at least one of them)
      uint32_t kcur = 0xffffffffu;
      for (uint32_t j = kg; j < (uint32_t)d.nk * 8; j += nwt) {
        const uint32_t k = j >> 3, ks = j & 7;
        if (k != kcur) {
          if (k > 0) {  // every earlier piece is released
            if (lane == 0) lds_st(L_XCONS + 4 * cw, seq + k);
            wake();
          }
          if (!spin_lds(e, [&]() { return lds_ld(L_XREADY) > seq + k; }, 0x400 | qi)) return;
          kcur = k;
        }
        {
          const uint32_t L0 = (k * nrb + rb_lo) * 4 + (ks >> 1), L1 = (k * nrb + rb_hi) * 4 + (ks >> 1);
          const uint32_t pg0 = n + (L0 >> 4), pg1 = n + (L1 >> 4);
          if (pg0 > rel) {
            if (lane == 0) lds_st(L_CONS + 4 * cw, pg0);
            rel = pg0;
            wake();
          }
          if (pg0 != v0) {
            if (!spin_lds_fast(e, [&]() { return lds_ld(LB_SENT + (pg0 % P) * kSentBytes) == pg0; }, 0x300 | qi))
              return;
            v0 = pg0;
          }
          if (pg1 != v1 && pg1 != v0) {
            if (!spin_lds_fast(e, [&]() { return lds_ld(LB_SENT + (pg1 % P) * kSentBytes) == pg1; }, 0x300 | qi))
              return;
          }
          v1 = pg1;
          const uint32_t mypg = upper ? pg1 : pg0, myL = upper ? L1 : L0;
          const uint32_t slot = (uint32_t)LB_XS + ((seq + k) % kNXSB) * kXSlotB;
          const uint32_t xaddr = lds_addr((int)(slot + sA * kXRowB + (ks * 32 + kA) * 4));
          const uint32_t waddr = lds_addr((int)(slot + kXNwB + (ks * 32 + kA) * 2));
          const uint32_t baddr = lds_addr(LB_RING + (int)((mypg % P) * kPageBytes + (myL & 15) * 1024 +
                                                          ((ks & 1) * 4 * 8 * 16) + brow));
          u4 x0, x1, wv, bv;
          asm volatile(
              "ds_read_b128 %0, %4\n\t"
              "ds_read_b128 %1, %4 offset:16\n\t"
              "ds_read_b128 %2, %5\n\t"
              "ds_read_b128 %3, %6\n\t"
              "s_waitcnt lgkmcnt(0)"
              : "=&v"(x0), "=&v"(x1), "=&v"(wv), "=&v"(bv)
              : "v"(xaddr), "v"(waddr), "v"(baddr));
          float x[8] = {__uint_as_float(x0.x), __uint_as_float(x0.y), __uint_as_float(x0.z), __uint_as_float(x0.w),
                        __uint_as_float(x1.x), __uint_as_float(x1.y), __uint_as_float(x1.z), __uint_as_float(x1.w)};
          if (normed) {
            x[0] *= bf_lo(wv.x); x[1] *= bf_hi(wv.x); x[2] *= bf_lo(wv.y); x[3] *= bf_hi(wv.y);
            x[4] *= bf_lo(wv.z); x[5] *= bf_hi(wv.z); x[6] *= bf_lo(wv.w); x[7] *= bf_hi(wv.w);
          }
          if (!liveA) {
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = 0.f;
          }
          const u4 av = pack_hilo(x, loA);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, av), __builtin_bit_cast(bf8v, bv),
                                                         acc, 0, 0, 0);
        }
      }
      // hi + lo halves: rows s and s + 8 of D sit in lanes l and l + 32
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += __shfl_xor(acc[j], 32);
      // the partial-tile buffer (qi & 1) was last read by unit qi - 2's epilogue
      if (qi >= 2 && !spin_lds(e, [&]() { return lds_ld(L_EPI) + 1 >= qi; }, 0x600 | qi)) return;
      if (lane < 32) *reinterpret_cast<f4 *>(Pb + cw * 128 + lane * 4) = acc;
      wait_lgkm0();
      if (lane == 0) lds_st(L_CONS + 4 * cw, n + d.pages);
      wake();
    } else if (d.op == OP_RED) {
      if (cw < c.G) {
        if (c.hd == 64) red_body<1>(e, a, d, cw);
        else red_body<2>(e, a, d, cw);
      }
    }
    n += upages;
    seq += nx;
    if (lane == 0) lds_st(L_XCONS + 4 * cw, seq);
    wake();
    if (!gv) wait_vm0();
    wait_lgkm0();
    uint32_t old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(&lds_u32(L_DONE + 4 * (qi & 3)), 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old == kNCW - 1) {
      lds_poll_exit();  // every wave's partial tile is in LDS
      if (lane == 0) trace_now(e, qi, 6);
      bool sig = true;  // (a split-K down unit signals only as its group's last arrival)
      if (gv) {
        sig = unit_epilogue_b(e, a, d, accs, Pb);
        if (d.op != OP_QKV) wait_vm0();
      }
      if (d.op == OP_LM && a.next_tok && (d.aux1 & 2u)) {
        wait_vm0();  // the published candidates are acknowledged before counting
        lm_greedy_finish_b(e, a);
      }
      before_signal();
      if (lane == 0) {
        trace_now(e, qi, 3);
        lds_st(L_DONE + 4 * (qi & 3), 0);
        lds_st(L_EPI, qi + 1);
        if (sig && d.sig0 >= 0)
          __hip_atomic_fetch_add(G(a.ctr) + ((size_t)d.sig0 * kSlots + d.slot0) * kCtrStride, 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        if (sig && d.sig1 >= 0)
          __hip_atomic_fetch_add(G(a.ctr) + ((size_t)d.sig1 * kSlots + d.slot1) * kCtrStride, 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
      wake();
    }
  }
}

// A step's set-up on this workgroup: its queue and (batch 1) position;
// false for a workgroup with no units (nothing to wait for or produce; the
// inputs are validated by the workgroups that use them).
template <bool BATCHED>
__device__ __forceinline__ bool step_env(const Args &a, Env &e) {
  e.cp = a.ctx;
  e.cu = (int)blockIdx.x;
  const uint32_t q0 = a.q_off[e.cu], q1 = a.q_off[e.cu + 1];
  e.q = a.instr + q0;
  e.nq = q1 - q0;
  if (e.nq == 0) return false;
  e.trace = a.trace ? a.trace + 4 + (size_t)e.cu * a.trace_stride * kTraceWords : nullptr;
  e.flags = e.cp->flags;
  // batch 1: an out-of-range position is replaced by 0 so that every cache
  // access stays in bounds; the sync wave reports it as an input error and
  // the step is abandoned (batched roles read each sequence's own position)
  e.pos0 = 0;
  if (!BATCHED) {
    e.pos0 = a.positions[0] + a.step_off;
    if (e.pos0 < 0 || e.pos0 >= e.cp->max_seq) e.pos0 = 0;
  }
  return true;
}

// LDS control words (step 0's tokens are the caller's) and page sentinels
// (no page has landed: they hold an index no page has), then every wave.
template <bool BATCHED>
__device__ __forceinline__ void step_lds(const Args &a) {
  if (threadIdx.x < 64) lds_u32(threadIdx.x * 4) = threadIdx.x * 4 == L_TOKOK && a.step_off == 0 ? 1u : 0u;
  constexpr int kSentWords = (BATCHED ? kRingPagesB : kRingPages) * kSentBytes / 4;
  for (int i = (int)threadIdx.x; i < kSentWords; i += kThreads)
    lds_u32((BATCHED ? LB_SENT : L_SENT) + 4 * i) = 0xffffffffu;
  __syncthreads();
}

// Issue priorities by role, set once per launch.
template <bool BATCHED>
__device__ __forceinline__ void role_priority(int w) {
#if MK_BPRIO
  // the sync wave's activation pieces ahead of the weight stream, whose
  // loads otherwise fill the CU's memory queue first
  if (BATCHED) {
    if (w >= kNCW + kNLW) __builtin_amdgcn_s_setprio(3);
    else if (w < kNCW) __builtin_amdgcn_s_setprio(2);
  }
#endif
#if MK_PRIO
  // the sync wave (critical-path waits and activation pieces) first,
  // compute waves next, weight streaming last
  if (!BATCHED) {
    if (w >= kNCW + kNLW) __builtin_amdgcn_s_setprio(3);
    else if (w < kNCW) __builtin_amdgcn_s_setprio(1);
  }
#endif
}

constexpr int kRoleCompute = 0, kRoleLoader = 1, kRoleSync = 2;
template <bool PAGED, bool BATCHED, int ROLE>
__device__ __forceinline__ void run_role(const Env &e, const Args &a, int w) {
  if (ROLE == kRoleCompute) {
    if (BATCHED) compute_role_b<PAGED>(e, a, w);
    else compute_role<PAGED>(e, a, w);
  } else if (ROLE == kRoleLoader) {
    if (BATCHED) loader_role_b<PAGED>(e, a, w - kNCW);
    else loader_role<PAGED>(e, a, w - kNCW);
  } else {
    if (BATCHED) sync_role_b(e, a);
    else sync_role(e, a);
  }
}

// Several chained greedy steps per launch (n_steps, tok_base set).  Step s
// runs with step_off = s: its counter targets, tags, positions, tokens and
// logits rows follow from it.  Each role runs its own step loop, so that a
// wave keeps across steps only the arguments its role reads; the loops meet
// at the same barriers (set-up, end of step) in every step.
template <bool PAGED, bool BATCHED, int ROLE>
__device__ __forceinline__ void role_steps(const Args &a, int w) {
  Args as = a;
  for (int32_t s = 0;; ++s) {
    as.step_off = s;
    Env e;
    if (!step_env<BATCHED>(as, e)) return;
    step_lds<BATCHED>(as);
    run_role<PAGED, BATCHED, ROLE>(e, as, w);
    // a device error raised elsewhere ends the launch here too; one lane
    // decides, so that every wave leaves at the same step
    if (threadIdx.x == 0 && ld_cu(reinterpret_cast<const uint32_t *>(e.cp->status))) lds_u32(L_ABORT) = 1u;
    // every wave of the workgroup is through step s (and its loads)
    __syncthreads();
    if (lds_u32(L_ABORT) || (uint32_t)s + 1 >= as.n_steps) return;
  }
}
template <bool PAGED, bool BATCHED>
__device__ __forceinline__ void chained_steps(const Args &a) {
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  role_priority<BATCHED>(w);
  if (w < kNCW) role_steps<PAGED, BATCHED, kRoleCompute>(a, w);
  else if (w < kNCW + kNLW) role_steps<PAGED, BATCHED, kRoleLoader>(a, w);
  else role_steps<PAGED, BATCHED, kRoleSync>(a, w);
}

#define MK_STEP_PARAMS                                                                                              \
  const DevCtx *__restrict__ ctx, const Instr *__restrict__ instr, const uint32_t *__restrict__ q_off,             \
      const Wait *__restrict__ waits, const uint64_t *__restrict__ rowtab, uint32_t *__restrict__ ctr,             \
      const uint32_t *__restrict__ grp_target, float *__restrict__ part_buf, const uint32_t *__restrict__ iota,    \
      const int32_t *__restrict__ tokens, const int32_t *__restrict__ positions, uint16_t *__restrict__ kv,        \
      float *__restrict__ logits, uint64_t *__restrict__ trace, uint32_t trace_stride, uint32_t epoch,             \
      uint32_t tag, int32_t batch, int32_t n_split, int32_t split_len, uint64_t *__restrict__ amax,               \
      uint32_t *__restrict__ amax_ctr, int32_t *__restrict__ next_tok, int32_t *__restrict__ next_pos,            \
      uint32_t n_lm, uint32_t amax_target, uint32_t n_steps, uint32_t tok_base
#define MK_STEP_ARGS(NS)                                                                                            \
  Args { ctx, instr, q_off, waits, rowtab, ctr, grp_target, part_buf, iota, tokens, positions, kv, logits, trace,  \
         trace_stride, epoch, tag, batch, n_split, split_len, amax, amax_ctr, next_tok, next_pos, n_lm,             \
         amax_target, NS, tok_base, 0 }

// One decode step per launch.  PAGED: the plan's attention units stream
// their K/V through pages (each plan is one or the other; separate
// instantiations keep the register allocation of the register-path kernel
// unchanged).
template <bool PAGED>
__global__ void __launch_bounds__(kThreads, 1) mk_interp(MK_STEP_PARAMS) {
  const Args a = MK_STEP_ARGS(1u);
  Env e;
  e.cp = a.ctx;
  e.cu = (int)blockIdx.x;
  const uint32_t q0 = a.q_off[e.cu], q1 = a.q_off[e.cu + 1];
  e.q = a.instr + q0;
  e.nq = q1 - q0;
  // a workgroup without units has nothing to wait for or produce (the
  // inputs are validated by the workgroups that use them)
  if (e.nq == 0) return;
  e.trace = a.trace ? a.trace + 4 + (size_t)e.cu * a.trace_stride * kTraceWords : nullptr;
  e.flags = e.cp->flags;
  // the wave index is uniform within a wave: saying so keeps each role's
  // control flow on the scalar unit instead of exec-masked vector code
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  role_priority<false>(w);
  // an out-of-range position is replaced by 0 so that every cache access
  // stays in bounds; the sync wave reports it as an input error and the
  // step is abandoned
  e.pos0 = a.positions[0];
  if (e.pos0 < 0 || e.pos0 >= e.cp->max_seq) e.pos0 = 0;
  step_lds<false>(a);
  if (w < kNCW) compute_role<PAGED>(e, a, w);
  else if (w < kNCW + kNLW) loader_role<PAGED>(e, a, w - kNCW);
  else sync_role(e, a);
}

template <bool PAGED>
__global__ void __launch_bounds__(kThreads, 1) mk_interp_b(MK_STEP_PARAMS) {
  const Args a = MK_STEP_ARGS(1u);
  Env e;
  e.cp = a.ctx;
  e.cu = (int)blockIdx.x;
  const uint32_t q0 = a.q_off[e.cu], q1 = a.q_off[e.cu + 1];
  e.q = a.instr + q0;
  e.nq = q1 - q0;
  if (e.nq == 0) return;
  e.trace = a.trace ? a.trace + 4 + (size_t)e.cu * a.trace_stride * kTraceWords : nullptr;
  e.pos0 = 0;  // unused: batched roles read each sequence's own position
  e.flags = e.cp->flags;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  role_priority<true>(w);
  step_lds<true>(a);
  if (w < kNCW) compute_role_b<PAGED>(e, a, w);
  else if (w < kNCW + kNLW) loader_role_b<PAGED>(e, a, w - kNCW);
  else sync_role_b(e, a);
}

template <bool PAGED>
__global__ void __launch_bounds__(kThreads, 1) mk_interp_n(MK_STEP_PARAMS) {
  chained_steps<PAGED, false>(MK_STEP_ARGS(n_steps));
}
template <bool PAGED>
__global__ void __launch_bounds__(kThreads, 1) mk_interp_bn(MK_STEP_PARAMS) {
  chained_steps<PAGED, true>(MK_STEP_ARGS(n_steps));
}

}  // namespace mk

// --------------------------------------------------------------------------
// Host-side launch helpers (the ABI layer is plain C++).
namespace mk {

// [batched][paged][multi-step]
static const void *const kKernels[8] = {
    (const void *)mk_interp<false>,   (const void *)mk_interp_n<false>,
    (const void *)mk_interp<true>,    (const void *)mk_interp_n<true>,
    (const void *)mk_interp_b<false>, (const void *)mk_interp_bn<false>,
    (const void *)mk_interp_b<true>,  (const void *)mk_interp_bn<true>};

hipError_t kernel_setup(int *blocks_per_cu) {
  *blocks_per_cu = 1 << 30;
  for (const void *fn : kKernels) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    int nb = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, kThreads, kLdsBytes);
    if (e != hipSuccess) return e;
    if (nb < *blocks_per_cu) *blocks_per_cu = nb;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Static scratch for callers that cannot allocate (mk_decode_step_static):
// one array per GPU, held until the process ends.  Host code never passes
// the array's name to a kernel (in host code it is a stand-in, not a device
// address): set-up resolves its device address once per device with
// hipGetSymbolAddress and every use goes through that pointer.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(int device, void **ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device) return hipErrorInvalidDevice;  // the device must be current
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

// Zero `words` 32-bit words with vector stores (a kernel rather than a
// memset node, so that the step can be captured into a graph).
__global__ void __launch_bounds__(256) mk_fill_zero(uint32_t *__restrict__ p, uint32_t words) {
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < words; i += gridDim.x * 256u) p[i] = 0u;
}

hipError_t fill_zero(void *p, size_t words, hipStream_t stream) {
  const uint32_t blocks = (uint32_t)std::min<size_t>((words + 255) / 256, 1024);
  hipLaunchKernelGGL(mk_fill_zero, dim3(blocks ? blocks : 1), dim3(256), 0, stream, (uint32_t *)p,
                     (uint32_t)words);
  return hipGetLastError();
}

hipError_t kernel_launch(const Args &a0, int grid, bool cooperative, bool paged, hipStream_t stream) {
  Args a = a0;
  void *params[] = {&a.ctx, &a.instr, &a.q_off, &a.waits, &a.rowtab, &a.ctr, &a.grp_target, &a.part_buf, &a.iota,
                    &a.tokens, &a.positions, &a.kv, &a.logits, &a.trace, &a.trace_stride, &a.epoch, &a.tag,
                    &a.batch, &a.n_split, &a.split_len, &a.amax, &a.amax_ctr, &a.next_tok, &a.next_pos,
                    &a.n_lm, &a.amax_target, &a.n_steps, &a.tok_base};
  // One workgroup per CU fits (checked at create); a plain launch places all
  // of them at once on an otherwise idle device, a cooperative one also
  // waits for room when other work holds CUs (about 23 us more per launch).
  // batches of 2 or more sequences run the MFMA kernel; plans whose
  // attention streams paged K/V run that instantiation
  const void *fn = kKernels[(a.batch > 1 ? 4 : 0) + (paged ? 2 : 0) + (a.n_steps > 1 ? 1 : 0)];
  if (cooperative) return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kThreads), params, kLdsBytes, stream);
  return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), params, kLdsBytes, stream);
}

}  // namespace mk
