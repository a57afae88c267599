// mk_plan.hpp -- the instruction descriptors, wait table and device context
// shared by the host scheduler and the persistent interpreter kernel.
//
// A plan is what the host pre-schedules before launch (megakernel chapter
// "L'interpréteur sur GPU", section 3.2): for every workgroup (one per CU) a
// queue of instruction descriptors, and for every dependency a counter group
// in global memory (section 3.4).
#pragma once
#include <stdint.h>

namespace mk {

// Opcodes: the seven fused instructions of the section 3.2 table.
enum Op : uint8_t {
  OP_QKV = 1,   // RMSNorm + QKV (+ q/k norm) + RoPE, K/V written to the cache
  OP_ATTN = 2,  // split-KV attention partials (m, l, o) for one KV head
  OP_RED = 3,   // log-sum-exp reduction of the partials of one KV head
  OP_O = 4,     // O projection + residual
  OP_FFN = 5,   // RMSNorm + gate/up + SiLU
  OP_DOWN = 6,  // down projection + residual
  OP_LM = 7,    // final RMSNorm + LM head
};

constexpr int kWave = 64;
constexpr int kNCW = 8;                  // compute waves per workgroup
#ifndef MK_NLW
#define MK_NLW 3
#endif
constexpr int kNLW = MK_NLW;             // loader waves per workgroup
constexpr int kThreads = (kNCW + kNLW + 1) * kWave;  // + 1 sync wave
constexpr int kPageBytes = 16384;        // LDS page (16 KB, 16 wave-loads of 1 KB)
constexpr int kMaxKc = 2048;             // elements per weight piece (<= 4 KB)
constexpr int kXSlotBytes = kMaxKc * 4;  // one fp32 activation piece
constexpr int kNXS = 2;                  // activation slots (double buffer)
constexpr int kAccFloats = 512;          // LDS row results of one unit (rows*ipw)
constexpr int kAccSlots = 4;             // units in flight per workgroup
constexpr int kLdsBytes = 163840;        // gfx950: 160 KB per CU
#ifndef MK_CSTRIDE
#define MK_CSTRIDE 32
#endif
constexpr int kCtrStride = MK_CSTRIDE;   // uint32 spacing of counters (128 B)
// A counter group is split over up to kSlots counters so that no counter
// takes more than kAtomicsPerSlot increments per step: atomics on one
// address serialise at the memory side (a few hundred ns each under load).
constexpr int kSlots = 64;
#ifndef MK_APS
#define MK_APS 1
#endif
constexpr int kAtomicsPerSlot = MK_APS;
constexpr int kMaxSplits = 64;
// Batched (MFMA) plans: pieces of 256 elements = 8 MFMA k-steps of 32, one
// per compute wave; units of at most 64 weight rows (four 16-row tiles).
constexpr int kMfmaKc = 256;
// Attention splits of at most this many positions run on registers (head
// dim 64); longer ones, and head_dim 128, stream their K/V through pages.
constexpr int kAttnRegRows = 20;
// The static scratch of mk_decode_step_static (per GPU) and the number of
// GPUs the library keeps one for.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;
constexpr int kMaxStepsPerLaunch = 65536;  // decode steps one launch may run
constexpr int kMfmaRows = 64;
// Batched LM-head units are wider: one per workgroup, each compute wave
// owning whole 16-row tiles (at most 4 of them), so the final-normed
// activation is staged once per workgroup.
constexpr int kMfmaWideRows = 512;

// One queued instruction (96 bytes).  An instruction's weight stream is the
// sequence of pieces t = 0 .. n_items*ipw*nk - 1 in k-major order:
//   k = t / (n_items*ipw), item i = (t % (n_items*ipw)) / ipw, s = t % ipw,
// piece t is row-part (item i, sub-row s) x K-range [k*kc, (k+1)*kc).  Pieces
// are packed `ppp` per 16 KB page.
struct alignas(16) Instr {
  uint8_t op;
  uint8_t ipw;          // pieces (rows) per item: 2 for RoPE pairs / gate+up
  uint16_t layer;
  uint16_t nk;          // K pieces per row
  uint16_t ppp;         // pieces per page
  uint32_t kc;          // elements per piece
  uint32_t pb;          // bytes per piece (2*kc)
  uint32_t item0;       // first item of this unit
  uint32_t n_items;
  uint32_t pages;       // weight pages of this unit (0: no weight stream)
  uint32_t wait_off;    // first entry in the wait table
  uint32_t wait_n;      // number of wait entries
  int32_t sig0, sig1;   // counter groups signalled on completion (-1: none)
  uint32_t b;           // sequence index (attention units)
  uint32_t aux0, aux1;  // ATTN: KV head, split; RED: KV head; QKV: G, head_dim
  uint32_t unit;        // unit index within (layer, op), for tracing
  // weight stream (host-resolved so the loader reads no context): row
  // r = i*ipw + s of the unit starts at rowtab[tab + r] if tab >= 0, else at
  // (s ? w1 : w0) + (item0 + i) * rowb.  FFN: w0 = w_gate, w1 = w_up.
  uint64_t w0, w1;
  int32_t tab;          // offset into the plan's row-address table, or -1
  uint32_t rowb;        // bytes per weight row (K * 2)
  uint32_t slot0, slot1;  // counter slot of sig0 / sig1 within its group
};
static_assert(sizeof(Instr) == 96, "descriptor size");

// A wait: counter group `grp` (its `nslot` counters) must reach its per-step
// targets before the activation piece `before_k` of the instruction is
// produced.
struct Wait {
  uint32_t grp;
  uint16_t before_k;
  uint16_t nslot;
};

struct DevLayer {
  const uint16_t *attn_norm, *wq, *wk, *wv, *q_norm, *k_norm;
  const uint16_t *wo, *ffn_norm, *w_gate, *w_up, *w_down;
};

// Device context: everything the kernel needs besides the per-step
// arguments.  Lives in device memory, read with scalar loads.
struct DevCtx {
  int32_t L, H, nq, nkv, hd, F, V, G, qk_norm, tied;
  int32_t max_batch, max_seq, num_cus;
  float eps, attn_scale;
  int64_t watchdog_ticks;   // 100 MHz ticks
  const uint16_t *embed, *final_norm, *lm_head;
  const DevLayer *layers;
  float *h_buf;       // [2L+1][max_batch][H]
  float *attn_buf;    // [L][max_batch][nq*hd]
  float *a_buf;       // [L][max_batch][F]
  // tagged words (fp32 value in the low 32 bits, the step's tag above)
  uint64_t *q_buf;    // [L][max_batch][nq][hd]
  uint64_t *kvn_buf;  // [L][max_batch][nkv][2][hd] this step's K/V slot (bf16-rounded)
  const float *rope;  // [max_seq][hd/2][2] (cos, sin)
  const uint16_t *zero;  // 1 KB of zeros: weights past K in zero-padded MFMA pieces
  uint32_t *status;   // [0] error code, [1..] details
  uint64_t *trace;    // per-instruction records or NULL
  int32_t ring_pages; // LDS weight pages per workgroup
  int32_t flags;
};

// LDS layout of a workgroup (bytes).
// (bytes 0..63 unused)
constexpr int L_CONS = 64;      // u32[8]   pages released per compute wave
constexpr int L_XCONS = 96;     // u32[8]   activation pieces released per wave
constexpr int L_XREADY = 128;   // u32      activation pieces produced
constexpr int L_DONE = 132;     // u32[4]   waves finished, per unit slot
constexpr int L_ABORT = 148;    // u32      nonzero: every wave exits
constexpr int L_EPI = 152;      // u32      units whose epilogue has finished
constexpr int L_AQ = 156;       // u32      paged attention: heads whose q is staged in LDS
constexpr int L_AM = 160;       // u32      paged attention: partials written for the merge
constexpr int L_TOKOK = 164;    // u32      this step's input tokens are in (earlier steps of the launch are done)
constexpr int kMaxBatch = 8;    // sequences per step the plans are built for
constexpr int L_ACC = 256;      // fp32 row results, kAccSlots x kAccFloats
constexpr int L_XS = L_ACC + kAccSlots * kAccFloats * 4;  // activation ring
constexpr int L_RING = ((L_XS + kNXS * kXSlotBytes + 1023) / 1024) * 1024;
constexpr int kMaxRingPages = 16;
constexpr int kRingPages = (kLdsBytes - L_RING) / kPageBytes < kMaxRingPages
                               ? (kLdsBytes - L_RING) / kPageBytes : kMaxRingPages;
static_assert(kRingPages >= 4, "LDS budget");
constexpr int L_NW = L_RING + kRingPages * kPageBytes;  // bf16 norm weights of one piece
// Page sentinels: after a page's 16 weight loads the loader issues one more
// direct-to-LDS load of the page's index (from a table holding i at i) into
// the slot's sentinel (64 lanes x 4 bytes).  Loads return in issue order, so
// a sentinel equal to n means page n has landed.
constexpr int kSentBytes = 256;
constexpr int L_SENT = L_NW + kMaxKc * 2;
static_assert(L_SENT + kRingPages * kSentBytes <= kLdsBytes, "LDS budget");

// Kernel arguments of one decode step (one per-batch plan).
struct Args {
  const DevCtx *ctx;
  const Instr *instr;         // all per-CU queues back to back
  const uint32_t *q_off;      // [num_cus + 1]
  const Wait *waits;
  const uint64_t *rowtab;     // row start addresses for tabulated units
  uint32_t *ctr;              // [n_groups][kSlots][kCtrStride]
  const uint32_t *grp_target; // [n_groups][kSlots] arrivals per step
  float *part_buf;            // [L][max_batch][nq][n_split][hd + 4] (o.., m, l)
  const uint32_t *iota;       // iota[i] = i for every page index of the longest queue
  const int32_t *tokens;
  const int32_t *positions;
  uint16_t *kv;
  float *logits;
  uint64_t *trace;            // [1 + num_cus * trace_stride][4] or null
  uint32_t trace_stride;      // records per workgroup (longest queue)
  uint32_t epoch;             // this plan's launch count: counter targets scale with it
  uint32_t tag;               // this step's activation tag (handle-wide, never 0)
  int32_t batch;
  int32_t n_split, split_len;
  // greedy next token (next_tok null: off).  Each LM unit stores its
  // candidate (largest logit of its rows, lowest index among equals) as one
  // 64-bit word, logit bits | index << 32, and counts itself on amax_ctr;
  // the unit that brings the counter to amax_target reduces the candidates.
  uint64_t *amax;             // [n_lm]
  uint32_t *amax_ctr;         // one counter word, zeroed with the others
  int32_t *next_tok;          // [batch]: argmax of the step's logits
  int32_t *next_pos;          // [batch]: positions + 1
  uint32_t n_lm;              // LM units in the plan
  uint32_t amax_target;       // counter value once this step's LM units are in
  // Several greedy steps per launch: step s (0-based, step_off) runs with
  // epoch epoch + s, tag tag + s, greedy target amax_target + s * n_lm,
  // positions + s, logits row block s and (s > 0) the tokens the step
  // before wrote to next_tok; the step's finisher stores the tokens, waits
  // for their acknowledgement and counts the step on the token counter
  // (amax_ctr + kTokWord), which step s + 1's sync waves wait for
  // (>= tok_base + s + 1) before they read a token.  The other fields are
  // the launch's own.
  uint32_t n_steps;           // >= 1 (> 1 only with next_tok)
  uint32_t tok_base;          // greedy steps counted before this launch
  int32_t step_off;           // device side: this step's index s
};
// The token counter word, in the greedy arrival counter's padded block.
constexpr int kTokWord = 16;
static_assert(kTokWord > 0 && kTokWord < kCtrStride, "token counter inside the greedy counter's block");

}  // namespace mk
