/*
 * mk.h -- C ABI of the persistent decode megakernel for MI355X (gfx950).
 *
 * One call of mk_decode_step runs one decode step of a Llama-style decoder
 * (every layer, then the LM head) for 1 to 8 sequences in ONE persistent
 * kernel launch.  The method is the GPU interpreter of the megakernel chapter
 * "L'interpréteur sur GPU": each compute unit's workgroup runs a queue of
 * instructions that the host scheduled before launch (section 3.2), drawn
 * from seven fused instructions (table of section 3.2): RMSNorm + QKV + RoPE,
 * attention, attention reduction, O-projection + residual, RMSNorm +
 * up/gate + SiLU, down-projection + residual, RMSNorm + LM head.  Kernel
 * boundaries are replaced by counters in global memory (section 3.4) and the
 * next instruction's weights stream into a paged on-chip buffer while the
 * current one finishes (section 3.3).
 *
 * Conventions for every entry point:
 *   - All pointers marked "device" are HIP device pointers on the device that
 *     was current when mk_create ran; "host" pointers are ordinary memory.
 *   - Integer status: 0 = MK_OK, negative = error (see MK_ERR_*).  Errors a
 *     host check can find are returned synchronously and nothing is launched.
 *   - The library never keeps a pointer to caller host memory after a call
 *     returns, and never writes caller device memory except where stated.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define MK_OK                   0
#define MK_ERR_INVALID_ARG     (-1)  /* null pointer, out-of-range argument   */
#define MK_ERR_UNSUPPORTED     (-2)  /* shape the decomposition cannot express */
#define MK_ERR_OOM             (-3)  /* device allocation failed              */
#define MK_ERR_HIP             (-4)  /* a HIP runtime call failed             */
#define MK_ERR_NOT_CORESIDENT  (-5)  /* the grid cannot be co-resident        */
#define MK_ERR_NO_DEVICE       (-6)  /* no usable GPU                         */
#define MK_ERR_NOT_PREPARED    (-7)  /* mk_decode_step_static: the batch
                                        size's schedule is not built yet     */
#define MK_ERR_DEVICE_TIMEOUT  (-10) /* a counter wait exceeded the watchdog  */
#define MK_ERR_BAD_TOKEN       (-11) /* tokens[b] outside [0, vocab)          */
#define MK_ERR_BAD_POSITION    (-12) /* positions[b] outside [0, max_seq)     */

/* ---- flags ------------------------------------------------------------- */
#define MK_FLAG_TRACE    1u   /* record per-instruction timestamps           */
/* Launch each step as a cooperative launch.  Every step needs one
 * workgroup per CU resident at once (mk_create checks that one fits).  By
 * default a step is a plain launch, which places all of them at once when
 * nothing else runs on the device; with other work on the device set this
 * flag, so that the launch waits until the whole grid fits (about 23 us
 * more per step on MI355X).  A plain launch whose workgroups cannot all run
 * ends in the watchdog: mk_sync_status reports MK_ERR_DEVICE_TIMEOUT. */
#define MK_FLAG_COOPERATIVE 2u
/* Test instruments ("Quand ne pas le faire", section 9.3: an ordering bug of
 * a persistent kernel shows as a rare wrong token, not as a failed check):
 * MK_FLAG_PERTURB makes every wave sleep a seeded pseudo-random time (0 to
 * 31 units of 64 clocks, different for every step, workgroup, instruction
 * and wave) before each instruction, so the same schedule runs under other
 * interleavings; results must be bitwise the same.  MK_FLAG_TEST_STALL
 * raises, on the host, the target of the counter the LM units wait on by
 * one, so that wait can never complete: the step must end through the
 * watchdog (MK_ERR_DEVICE_TIMEOUT from mk_sync_status) with every wave
 * exiting.  Neither is meant for production use. */
#define MK_FLAG_PERTURB     4u
#define MK_FLAG_TEST_STALL  8u

/* ---- model and schedule configuration ---------------------------------- */
/* All sizes in elements.  The model is a pre-norm Llama-style decoder with
 * grouped-query attention, SwiGLU FFN and half-split RoPE; qk_norm adds a
 * per-head RMSNorm on q and k (Qwen3-style). */
typedef struct mk_config {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab;
  float   rms_eps, rope_theta;
  int32_t tied_embeddings;   /* 1: LM head is the embedding matrix          */
  int32_t qk_norm;           /* 1: per-head q/k RMSNorm before RoPE          */
  int32_t max_batch;         /* capacity of kv_cache and scratch (sequences) */
  int32_t max_seq;           /* KV slots per sequence                        */
  int32_t mlp_chunks;        /* counters on the up/gate -> down edge, 0 = 4  */
  int32_t kv_splits;         /* attention splits per (seq, KV head), 0 = auto*/
  int32_t num_cus;           /* workgroups (one per CU), 0 = every CU        */
  int32_t watchdog_ms;       /* bound on any single wait, 0 = 2000 ms        */
  uint32_t flags;            /* MK_FLAG_*                                    */
} mk_config;

/* Device pointers to bf16 weights, row-major [out][in] (nn.Linear layout).
 * Norm weights are [hidden] (q_norm/k_norm: [head_dim]). */
typedef struct mk_layer_weights {
  const void *attn_norm, *wq, *wk, *wv;
  const void *q_norm, *k_norm;          /* NULL unless qk_norm              */
  const void *wo, *ffn_norm, *w_gate, *w_up, *w_down;
} mk_layer_weights;

typedef struct mk_weights {
  const void *embed;                    /* [vocab][hidden]                  */
  const void *final_norm;               /* [hidden]                         */
  const void *lm_head;                  /* [vocab][hidden]; NULL iff tied   */
  const mk_layer_weights *layers;       /* host array of n_layers entries   */
} mk_weights;

typedef struct mk_handle mk_handle;

/* mk_create -- validate the configuration, query the device, allocate the
 * library's scratch (counters, activations, partials, RoPE table).  The
 * instruction schedule (chapter "L'interpréteur sur GPU", section 3.2:
 * queues are planned on the host before launch) of a batch size is built at
 * its first step and passes the static checks of mk_plan_check before it is
 * uploaded.  The scratch holds what that interpreter needs beside the
 * weights: counters in global memory zeroed before use (section 3.4) and
 * the activations that cross workgroups; the LDS page ring of section 3.3
 * lives in each launch and needs no allocation.
 *   cfg, w  : host pointers, read during the call only.  The weight device
 *             pointers inside must stay valid and unmodified until
 *             mk_destroy; the library reads them in place and never copies,
 *             repacks or writes them.
 *   out     : receives the handle (NULL on error).
 * Errors: MK_ERR_INVALID_ARG, MK_ERR_UNSUPPORTED, MK_ERR_NO_DEVICE,
 *         MK_ERR_OOM, MK_ERR_HIP, MK_ERR_NOT_CORESIDENT.  MK_ERR_UNSUPPORTED
 *         for shapes the kernels cannot run, refused before any device call:
 *         head_dim other than 64 or 128, query heads per KV head not
 *         dividing 8, qk_norm without head_dim 128, hidden or ffn_dim not a
 *         multiple of 8, kv_splits above 64, n_layers above 4096, hidden,
 *         ffn_dim or n_q_heads*head_dim above 2^20 (a descriptor holds the
 *         layer and a row's K pieces in 16 bits). */
int mk_create(const mk_config *cfg, const mk_weights *w, mk_handle **out);

/* mk_decode_step -- one decode step for sequences b < batch on `stream`
 * (asynchronous; the call returns after enqueueing): exactly one launch of
 * the persistent kernel, which runs the whole forward pass of every
 * sequence (the one-kernel definition on the index page of part 8, "Les
 * megakernels"; the seven instructions of chapter "L'interpréteur sur GPU",
 * section 3.2, with cross-workgroup dependencies through the counters of
 * section 3.4).  One sequence runs the vector-unit kernel; 2 to 8 run the
 * batched kernel (matrix-core products over the sequences; each weight is
 * read once per step for the whole batch).
 *   tokens    : device int32 [batch], the token fed at this step.
 *   positions : device int32 [batch], the KV slot of that token; slots
 *               0..positions[b]-1 must already hold the sequence's K/V.
 *   kv_cache  : device bf16 [n_layers][2][max_batch][n_kv_heads][max_seq]
 *               [head_dim] (index 0 = K after RoPE, 1 = V).  The step writes
 *               slot positions[b] of every layer for every b < batch and
 *               nothing else.
 *   logits    : device fp32 [batch][vocab], fully written.
 *   stream    : hipStream_t (NULL = the null stream).
 * One step may be in flight per handle; stream order serialises steps.
 * The handle is not thread-safe.  Device-side errors (watchdog, bad token or
 * position) are reported by mk_sync_status after the stream is synchronised.
 * Errors returned here: MK_ERR_INVALID_ARG (null pointer, batch outside
 * [1, max_batch]), MK_ERR_UNSUPPORTED (batch above 8; qk_norm with batch
 * above 1), MK_ERR_HIP, MK_ERR_OOM. */
int mk_decode_step(mk_handle *h, int32_t batch, const int32_t *tokens,
                   const int32_t *positions, void *kv_cache, float *logits,
                   void *stream);

/* mk_decode_step_greedy -- mk_decode_step plus the greedy next token,
 * computed in the same launch after the LM head: every LM unit reduces its
 * rows to one candidate and the last unit to finish reduces the candidates,
 * so no further kernel or host round trip is needed.  The pages' path ends
 * with the LM head (chapter "L'interpréteur sur GPU", table of section 3.2);
 * picking the greedy token is not described there and is taken as the
 * plainest step after it.
 *   next_tokens    : device int32 [batch]: index of the largest logit of row
 *                    b (the lowest index among equal logits; a NaN ranks
 *                    above every number), computed from the fp32 logits
 *                    this step writes.
 *   next_positions : device int32 [batch]: positions[b] + 1.
 * Both may be the same buffers as tokens and positions: every read of the
 * inputs in the launch comes before these writes, so a caller can chain
 * steps on the device with one pair of buffers.  Other arguments and errors
 * as mk_decode_step (MK_ERR_INVALID_ARG also for a null output).  The
 * outputs are unspecified after a device error. */
int mk_decode_step_greedy(mk_handle *h, int32_t batch, const int32_t *tokens,
                          const int32_t *positions, void *kv_cache,
                          float *logits, int32_t *next_tokens,
                          int32_t *next_positions, void *stream);

/* mk_decode_steps_greedy -- n_steps greedy decode steps in ONE launch:
 * step s + 1 feeds the token step s chose, at the next position, so the
 * host sees neither the steps' tokens nor a kernel boundary between them.
 * The pages count what each kernel launch costs (chapter "L'interpréteur
 * sur GPU", section 3.1) and replace the boundaries between kernels by
 * counters (section 3.4); doing the same across decode steps is not
 * described there and is taken as the plainest extension of the in-launch
 * greedy token: the step's last LM unit writes the tokens and counts the
 * step on a device counter, and the next step's workgroups start once it
 * has.
 * The results equal those of n_steps chained mk_decode_step_greedy calls
 * bit for bit.  Ordering between the steps of a launch: step s + 1 reads
 * the K/V rows step s wrote only after step s's token counter moved; the
 * stores of those rows are acknowledged before that counter moves where
 * every workgroup runs an attention or reduction unit after its QKV units
 * (the Llama-1B and Qwen3-8B schedules on 256 CUs); in schedules with fewer
 * attention units than workgroups, what orders them is the rest of the step
 * outlasting a store's acknowledgement, not a wait.
 *   n_steps        : 1 .. 65536.
 *   tokens         : device int32 [batch], the tokens of the first step.
 *   positions      : device int32 [batch], the first step's KV slots; step s
 *                    writes slot positions[b] + s of every layer, so
 *                    positions[b] + n_steps must not exceed max_seq.
 *   logits         : device fp32 [n_steps][batch][vocab], step s in row
 *                    block s, fully written.
 *   next_tokens    : device int32 [batch]: written by every step (the tokens
 *                    the next step reads), the last step's on return.  May
 *                    be the same buffer as tokens.
 *   next_positions : device int32 [batch]: positions[b] + n_steps, written by
 *                    the last step only.  May be the same buffer as
 *                    positions.
 * Errors: as mk_decode_step_greedy, and MK_ERR_INVALID_ARG for n_steps
 * outside [1, 65536].  A device error in step s (bad position, watchdog)
 * ends the launch at that step; mk_sync_status reports it and the outputs
 * of steps s and later are unspecified.  With MK_FLAG_TRACE the trace
 * buffer holds the launch's last step. */
int mk_decode_steps_greedy(mk_handle *h, int32_t batch, int32_t n_steps,
                           const int32_t *tokens, const int32_t *positions,
                           void *kv_cache, float *logits, int32_t *next_tokens,
                           int32_t *next_positions, void *stream);

/* mk_decode_step_static -- mk_decode_step_greedy for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  It calls no hipMalloc, hipFree
 * or allocating library routine: the step's scratch (its counter groups,
 * the greedy and split-K arrival counters, the attention and split-K
 * partials and the greedy candidates) is a static array of the library, one per GPU, of 32 MiB, held until the
 * process ends, and the schedule of `batch` must already exist (built by an
 * earlier mk_decode_step or mk_decode_step_greedy call of this handle with
 * the same batch size).  Each call first clears the counters with a small
 * fill kernel on `stream` (no memset node), then launches the step: two
 * kernels in stream order.
 *   next_tokens, next_positions : as mk_decode_step_greedy, or both NULL for
 *                                 a step without the greedy choice.
 *   Other arguments as mk_decode_step.
 * Every call on one GPU, from any handle, shares that GPU's array: calls
 * whose executions overlap on one GPU (several streams, several threads)
 * race and give wrong results; serialise them.  Ordinary steps of the same
 * handle use their own scratch and may be mixed with these calls freely.
 * Errors: MK_ERR_INVALID_ARG, MK_ERR_NOT_PREPARED (no schedule for this
 * batch size yet), MK_ERR_UNSUPPORTED (the schedule's scratch exceeds the
 * 32 MiB array), MK_ERR_HIP; device-side errors through mk_sync_status. */
int mk_decode_step_static(mk_handle *h, int32_t batch, const int32_t *tokens,
                          const int32_t *positions, void *kv_cache,
                          float *logits, int32_t *next_tokens,
                          int32_t *next_positions, void *stream);

/* mk_sync_status -- synchronise the device and return the first device-side
 * error of the steps since the last call (MK_OK if none): a wait that
 * outlived the watchdog (MK_ERR_DEVICE_TIMEOUT; a missing or late
 * dependency in a megakernel shows up as a hang or a rare wrong token, not
 * as a clean failure: chapter "Quand ne pas le faire", section 9.3, the
 * debugging cost), a token outside the vocabulary (MK_ERR_BAD_TOKEN) or a
 * position outside the cache (MK_ERR_BAD_POSITION); the step that found it
 * writes nothing further.  After an error the library re-zeroes its
 * counters (section 3.4 of "L'interpréteur sur GPU": counters start from
 * zero) so the next step starts clean; a decode step is idempotent (it
 * rewrites slot p and the logits), so the caller may simply run it again. */
int mk_sync_status(mk_handle *h);

/* mk_destroy -- free everything mk_create and the steps allocated: the
 * schedules of every batch size used (the host-planned queues of chapter
 * "L'interpréteur sur GPU", section 3.2), their counters (section 3.4) and
 * the activation scratch.  The caller's weights, cache and outputs are not
 * touched.  NULL-safe.  The caller must have synchronised any stream the
 * handle was used on (the library does not wait for steps in flight). */
void mk_destroy(mk_handle *h);

/* mk_strerror -- static text for a status code (never NULL). */
const char *mk_strerror(int code);

/* ---- host-only planning and diagnostics --------------------------------- */

/* Summary of a schedule built for `num_cus` workgroups without touching any
 * GPU. */
typedef struct mk_plan_report {
  int32_t num_cus, batch, kv_splits, mlp_chunks;
  int32_t n_instr;            /* descriptors over all queues                 */
  int32_t n_groups;           /* counter groups                              */
  int32_t n_pages;            /* 16 KB weight pages over all queues          */
  int32_t max_queue;          /* longest per-CU queue                        */
  int64_t weight_bytes;       /* bf16 weight bytes streamed per step         */
  int64_t max_cu_bytes;       /* largest per-CU weight stream                */
  int64_t mfma_cols_k;        /* batched plans: sum over units of weight rows
                                 padded to 16-row tiles x K padded to 256
                                 (the 16x16x32 MFMAs issue 2*16 FLOP per
                                 unit of this); 0 for batch-1 plans          */
  int32_t sim_runs;           /* interleavings simulated                     */
  int32_t sim_errors;         /* missing dependencies or deadlocks found     */
  int32_t paged_kv;           /* 1: attention units stream K/V through the
                                 LDS page ring (the kernel instantiated for
                                 paged attention runs the step); 0: the
                                 register-prefetch attention body           */
  int32_t down_splits;        /* batched plans: MLP chunks each down-
                                 projection row group is split over (its
                                 last arrival sums them); 0 = no split      */
  char    msg[256];           /* first error found, if any                   */
} mk_plan_report;

/* mk_plan_check -- build the schedule for (cfg, batch) on `num_cus`
 * workgroups, validate it statically (every read is covered by a wait on
 * every writer of that data; counter targets match their producers) and run
 * a static happens-before check (every read ordered after each of its
 * writers by the counter waits and tagged reads, never by queue order: the
 * waves of a workgroup pipeline across units), then `sim_runs` seeded
 * interleavings of the per-CU queues that respect only the counter waits
 * (some adversarial: one CU delayed, stage-reversed priorities), checking
 * that every read sees its producers finished and that no interleaving
 * deadlocks; no two units write the same elements; every unit's rows,
 * heads, splits, row-table
 * and wait entries and every recorded access must lie inside the buffers
 * they index.  `corrupt` != 0 deliberately breaks the plan (1: drop a
 * signal, 2: lower a wait target, 3: drop a wait, 4: move an attention unit
 * one split past the last, 5: let two units write the same rows) so tests
 * can check that the validator catches it.  Host only; no GPU needed.
 * Returns MK_OK if the plan is valid, MK_ERR_UNSUPPORTED for shapes the
 * decomposition rejects, MK_ERR_INVALID_ARG otherwise; rep is filled. */
int mk_plan_check(const mk_config *cfg, int32_t batch, int32_t num_cus,
                  int32_t sim_runs, int32_t corrupt, uint64_t seed,
                  mk_plan_report *rep);

/* One queued unit of a schedule, as mk_plan_units reports it. */
typedef struct mk_unit_info {
  int32_t op;       /* 1 QKV, 2 attention, 3 reduction, 4 O, 5 FFN, 6 down, 7 LM head */
  int32_t layer;
  int32_t nk;       /* activation pieces per row (projections)                       */
  int32_t pages;    /* 16 KB weight pages streamed (projections); paged attention:
                       rows per page in ppp, pages from the step's position         */
  int32_t ppp;      /* weight pieces per page, or K/V rows per page (paged attention) */
  int32_t n_items;  /* output rows (items) of the unit                               */
  int32_t ipw;      /* pieces (rows) per item: 2 for RoPE pairs and gate/up          */
  int32_t wait_n;   /* counter groups it waits on                                    */
  int32_t b;        /* sequence (attention and reduction units; 0 otherwise)          */
  int32_t aux0;     /* attention and reduction units: KV head                         */
  int32_t aux1;     /* attention units: KV split (positions [aux1*split_len, ...))    */
  int32_t split_len;/* KV positions per split (the plan's; the same for every unit)   */
} mk_unit_info;

/* mk_plan_units -- the schedule mk_plan_check builds for (cfg, batch) on
 * `num_cus` workgroups, unit by unit: the per-workgroup queues back to back,
 * workgroup c's units at [q_off[c], q_off[c + 1]).  It lets tests model
 * what happens inside a workgroup (the ordering between its loader, sync
 * and compute waves) over the library's own schedules.  Host only.
 *   units : host array of `cap` entries, or NULL with cap 0 (count only).
 *   q_off : host int32 [num_cus + 1], or NULL.
 * Returns the number of units (entries beyond cap are not written), or an
 * MK_ERR_* code. */
int mk_plan_units(const mk_config *cfg, int32_t batch, int32_t num_cus,
                  mk_unit_info *units, int32_t cap, int32_t *q_off);

/* Result of the address model below. */
typedef struct mk_addr_report {
  int64_t accesses;           /* global accesses evaluated (per lane)        */
  int32_t violations;         /* accesses outside the buffer they address    */
  char    msg[256];           /* the first violation: site, buffer, offset   */
} mk_addr_report;

/* mk_addr_check -- host model of the decode kernel's global memory accesses
 * for `steps` consecutive steps of (cfg, batch) on `num_cus` workgroups,
 * positions advancing by one per step from positions[b] and the tokens
 * fixed at tokens[b].  It builds the plan the library would upload, gives
 * every tensor and library buffer its size as mk_create and the plan upload
 * allocate them, and walks every workgroup's queue the way each role of the
 * kernel does (input checks, norm weights, RoPE rows, activation pieces,
 * residual rows, weight pieces and page sentinels, attention K/V rows and
 * the new slot, tagged q/K/V words, partials, reduction, epilogue stores,
 * greedy candidates, counters), per lane, with the kernel's own offset
 * arithmetic; every access must lie inside the buffer it addresses, and
 * every access a unit makes to an activation buffer (h, attention output,
 * MLP activation, attention partials, tagged q/K/V) must fall in a read or
 * write the plan records for that unit, the records mk_plan_check's
 * dependency checks are made on.  This is
 * the gate every new kernel path passes before it runs on a GPU (the
 * megakernel chapter "Quand ne pas le faire", section 9.3: an error of this
 * kind shows as a rare wrong token or a fault, not as a failed assertion).
 *   positions, tokens : host int32 [batch].
 *   corrupt : 0, or a planted size error for the model's self-tests: the
 *             model's copy of one buffer is one record short (1: the KV
 *             cache's last slot, 2: the last attention partial, 3: the last
 *             RoPE row, 4: the last q head, 5: the final residual row, 6:
 *             the last sequence's logits row), so a run that reaches that
 *             record must report it; or a planted record error: the plan
 *             forgets the first FFN unit's residual read (7) or the first
 *             attention unit's tagged q/K/V read (8).
 * Returns MK_OK if every access is in its buffer and recorded,
 * MK_ERR_INVALID_ARG (rep->msg names the first) otherwise, or the plan's own
 * error.  Host only. */
int mk_addr_check(const mk_config *cfg, int32_t batch, int32_t num_cus,
                  int32_t steps, const int32_t *positions,
                  const int32_t *tokens, int32_t corrupt,
                  mk_addr_report *rep);

/* mk_addr_check_launch -- the same model for ONE launch of `steps` chained
 * greedy steps (mk_decode_steps_greedy): step s writes logits row block s of
 * a [steps][batch][vocab] buffer, reads its tokens from next_tokens for
 * s > 0 (the caller's tokens for s = 0) after waiting on the token counter,
 * and its positions at positions[b] + s.  Arguments, returns and errors as
 * mk_addr_check.  Host only. */
int mk_addr_check_launch(const mk_config *cfg, int32_t batch, int32_t num_cus,
                         int32_t steps, const int32_t *positions,
                         const int32_t *tokens, int32_t corrupt,
                         mk_addr_report *rep);

/* Internal activation buffers, for stage-by-stage comparison in tests. */
#define MK_BUF_H      1   /* fp32 [2L+1][max_batch][hidden]: index 2l+1 is the
                             residual after attention of layer l, 2l+2 after
                             its FFN (index 0 unused)                         */
#define MK_BUF_Q      2   /* [L][max_batch][n_q][head_dim], after RoPE, as
                             64-bit words: fp32 value in the low 32 bits, the
                             tag of the step that wrote it in the high 32     */
#define MK_BUF_ATTN   3   /* fp32 [L][max_batch][n_q*head_dim]                 */
#define MK_BUF_A      4   /* fp32 [L][max_batch][ffn_dim], SiLU(gate)*up       */
#define MK_BUF_TRACE  5   /* uint64 trace records (MK_FLAG_TRACE)              */

/* mk_get_buffer -- device pointer and size in bytes of an internal buffer.
 * The memory belongs to the library; read it only after the step that wrote
 * it has completed.  Returns MK_ERR_INVALID_ARG for an unknown id. */
int mk_get_buffer(mk_handle *h, int32_t which, void **ptr, size_t *bytes);

/* mk_stream_read -- diagnostic: read `bytes` of device memory at `buf` once
 * with 128-bit nontemporal loads from every CU (4096 workgroups), folding
 * what each thread read into one word of `sink` so the loads cannot be
 * dropped.  The time it takes gives the chip's achievable streaming-read
 * rate, the practical ceiling of a step that reads every weight once.
 *   buf  : device, 16-byte aligned; bytes a nonzero multiple of 16.
 *   sink : device uint32 [mk_stream_read_sink_words()], overwritten.
 * Asynchronous on `stream` (hipStream_t, NULL = the null stream).
 * Errors: MK_ERR_INVALID_ARG, MK_ERR_HIP. */
int mk_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);
size_t mk_stream_read_sink_words(void);

/* mk_version -- ABI version of this header (major*100 + minor): 101 adds
 * mk_decode_step_greedy, 102 mk_stream_read, 103 mk_addr_check, the batched
 * (MFMA) kernel and mk_plan_report.mfma_cols_k, 104
 * mk_plan_report.paged_kv and .down_splits, 105 mk_decode_steps_greedy,
 * 106 mk_addr_check_launch, 107 mk_plan_units, 108 size limits that keep
 * every descriptor field in range (mk_create and mk_plan_check refuse
 * larger shapes), 109 mk_unit_info.b, .aux0, .aux1 and .split_len. */
int mk_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
