// mk_layout.hpp -- element offsets of every buffer the decode kernel
// addresses, as plain index arithmetic usable on the host and the device.
//
// The kernel forms each global address as  base + offset(...)  with the
// offsets below, and the host-side address model (mk_addr.cpp) evaluates the
// same functions for every (unit, wave, lane, step) of a plan and checks the
// result against the extent of the buffer it must fall in.  Keeping the
// arithmetic in one place means the model cannot drift from the kernel on a
// retyped formula; what the model mirrors by hand is only the loop
// structure of each instruction body.
//
// Layouts (elements, row-major):
//   kv cache  bf16 [L][2][max_batch][n_kv][max_seq][hd]   (0 = K, 1 = V)
//   h         fp32 [2L+1][max_batch][H]  (index 2l: input of layer l,
//                                         2l+1: after attention, 2L: final)
//   q         u64  [L][max_batch][n_q][hd]       tagged words
//   kvn       u64  [L][max_batch][n_kv][2][hd]   tagged words, this step's slot
//   attn      fp32 [L][max_batch][n_q*hd]
//   a         fp32 [L][max_batch][F]
//   partials  fp32 [L][max_batch][n_q][n_split][hd+4]  (o[hd], m, l, pad)
//   rope      fp32 [max_seq][hd/2][2]                  (cos, sin)
//   logits    fp32 [batch][V]
//   counters  u32  [n_groups][kSlots][kCtrStride]
#pragma once
#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define MK_HD __host__ __device__ __forceinline__
#else
#define MK_HD inline
#endif

namespace mk {
namespace lay {

MK_HD size_t kv(int MB, int nkv, int S, int hd, int l, int t, int b, int g, int s) {
  return ((((size_t)l * 2 + t) * MB + b) * nkv + g) * (size_t)S * hd + (size_t)s * hd;
}
MK_HD size_t kv_size(int L, int MB, int nkv, int S, int hd) { return (size_t)L * 2 * MB * nkv * S * hd; }

MK_HD size_t h(int MB, int H, int idx, int b) { return ((size_t)idx * MB + b) * H; }
MK_HD size_t h_size(int L, int MB, int H) { return (size_t)(2 * L + 1) * MB * H; }

MK_HD size_t q(int MB, int nq, int hd, int l, int b, int j) { return (((size_t)l * MB + b) * nq + j) * hd; }
MK_HD size_t q_size(int L, int MB, int nq, int hd) { return (size_t)L * MB * nq * hd; }

MK_HD size_t kvn(int MB, int nkv, int hd, int l, int b, int g, int t) {
  return ((((size_t)l * MB + b) * nkv + g) * 2 + t) * hd;
}
MK_HD size_t kvn_size(int L, int MB, int nkv, int hd) { return (size_t)L * MB * nkv * 2 * hd; }

MK_HD size_t attn(int MB, int nq, int hd, int l, int b) { return ((size_t)l * MB + b) * ((size_t)nq * hd); }
MK_HD size_t attn_size(int L, int MB, int nq, int hd) { return (size_t)L * MB * nq * hd; }

MK_HD size_t a(int MB, int F, int l, int b) { return ((size_t)l * MB + b) * F; }
MK_HD size_t a_size(int L, int MB, int F) { return (size_t)L * MB * F; }

// One partial record is hd + 4 floats: o[0..hd), m, l, two words of padding.
MK_HD size_t part(int MB, int nq, int ns, int hd, int l, int b, int j, int s) {
  return ((((size_t)l * MB + b) * nq + j) * ns + s) * (size_t)(hd + 4);
}
MK_HD size_t part_size(int L, int MB, int nq, int ns, int hd) { return (size_t)L * MB * nq * ns * (hd + 4); }

MK_HD size_t rope(int hd, int p, int i) { return ((size_t)p * (hd / 2) + i) * 2; }
MK_HD size_t rope_size(int S, int hd) { return (size_t)S * hd; }

MK_HD size_t logits(int V, int b) { return (size_t)b * V; }

// Batched GEMV units (MFMA): the weight stream is a sequence of 1 KB blocks,
// each 8 rows x 64 elements of one K piece (256 elements).  `nrb` row blocks
// of 8 rows.  Block L of a unit's stream holds K piece k, 64-wide chunk kb
// (0..3) of row block rb.  Ordinary units go row block by row block within a
// piece (a row block's 4 chunks together); wide units (more than 8 tiles of
// 16 rows: the batched LM head) go chunk by chunk, every row block of chunk
// kb before chunk kb + 1, so that a compute wave builds the A operands of a
// chunk once for all its tiles.
MK_HD bool mfma_wide(uint32_t nrb) { return (nrb + 1) / 2 > 8; }
MK_HD void mfma_block(uint32_t L, uint32_t nrb, bool wide, uint32_t &k, uint32_t &kb, uint32_t &rb) {
  if (wide) {
    rb = L % nrb;
    const uint32_t rest = L / nrb;
    kb = rest & 3;
    k = rest >> 2;
  } else {
    kb = L & 3;
    const uint32_t rbk = L >> 2;
    rb = rbk % nrb;
    k = rbk / nrb;
  }
}
MK_HD uint32_t mfma_block_index(uint32_t k, uint32_t kb, uint32_t rb, uint32_t nrb, bool wide) {
  return wide ? (k * 4 + kb) * nrb + rb : (k * nrb + rb) * 4 + kb;
}

// Split-K down-projection units (batched plans): unit (row group, chunk s)
// multiplies rows of W_down by one MLP chunk of the activation, K elements
// [koff, koff + klen).  aux0 = koff | klen << 16; aux1 = s | S << 4 |
// group << 8 with S the number of chunks (S <= 1: an ordinary unit over the
// whole K) and `group` the global index of its (layer, row group).  Partial
// results: fp32 [L][S][H][max_batch]; one arrival counter per group.
MK_HD uint32_t split_n(uint32_t aux1) { return (aux1 >> 4) & 15u; }
MK_HD uint32_t split_s(uint32_t aux1) { return aux1 & 15u; }
MK_HD uint32_t split_group(uint32_t aux1) { return aux1 >> 8; }
MK_HD uint32_t split_koff(uint32_t aux0) { return aux0 & 0xffffu; }
MK_HD uint32_t split_klen(uint32_t aux0) { return aux0 >> 16; }
MK_HD size_t dpart(int H, int MB, int S, int l, int s, int r, int b) {
  return (((size_t)l * S + s) * H + r) * MB + b;
}
MK_HD size_t dpart_size(int L, int S, int H, int MB) { return (size_t)L * S * H * MB; }

#ifndef MK_BROT
#define MK_BROT 1
#endif
// K-piece order of a batched GEMV unit: unit u takes its pieces starting at
// piece u mod nk, so that at any moment the units of one instruction read
// different activation pieces instead of all reading the same bytes.  The
// loader (weights) and the sync wave (activations) map a unit's logical
// piece k to the same physical piece; the compute waves only see logical
// pieces.
MK_HD uint32_t mfma_phys_k(uint32_t k, uint32_t nk, uint32_t unit) {
  if (!MK_BROT) return k;
  const uint32_t kk = k + unit % nk;
  return kk >= nk ? kk - nk : kk;
}

}  // namespace lay
}  // namespace mk
