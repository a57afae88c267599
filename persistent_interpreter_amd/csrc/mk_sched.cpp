// mk_sched.cpp -- host instruction scheduler and plan validator.
//
// The host plans every workgroup's instruction queue before launch
// (megakernel chapter "L'interpréteur sur GPU", section 3.2).  Each of the
// seven instructions is cut into units spread over the compute units; each
// dependency between units is a counter group that consumers wait on
// (section 3.4), at the granularity the data is produced (the generalisation
// closing section 3.4: dependency granularity follows production
// granularity): per KV head from QKV to attention, per (sequence, KV head)
// from attention to its reduction, per MLP chunk from up/gate to down (four
// chunks by default, the chunked example of section 3.4), and whole-vector
// edges where a RMSNorm needs every row.
#include "mk_sched.hpp"
#include "mk_layout.hpp"

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <functional>
#include <map>
#include <random>

#ifndef MK_XCDMAP
#define MK_XCDMAP 0  // 1: XCD-aware CU placement (measured neutral on the Llama-1B shape)
#endif

namespace mk {

int choose_kc(int K, int kmax) {
  // piece bytes (2*kc) must be a multiple of 1 KB or divide 1 KB so that a
  // 1 KB wave-load never straddles pieces unevenly; kc * batch fp32
  // activations must fit one LDS activation slot (kmax = 2048 / batch)
  static const int cand[] = {2048, 1536, 1024, 512, 256, 128, 64, 32, 16, 8};
  for (int kc : cand)
    if (kc <= K && kc <= kmax && K % kc == 0) return kc;
  return 0;
}

static inline uint32_t part_lo(uint64_t total, uint64_t n, uint64_t u) {
  return (uint32_t)(total * u / n);
}

namespace {

struct Unit {
  Instr in;
  int cu;
  std::vector<Wait> waits;
  std::vector<Access> reads, writes;
  std::vector<int> sigs;
};

struct Builder {
  const mk_config &c;
  int B, C;
  Plan &P;
  std::vector<Unit> units;

  Builder(const mk_config &cfg, int b, int cus, Plan &p) : c(cfg), B(b), C(cus), P(p) {}

  int group() {
    P.grp_target.resize(P.grp_target.size() + kSlots, 0);
    P.grp_producers.push_back(0);
    P.grp_nslot.push_back(0);
    return P.n_groups++;
  }

  // a split-K unit other than the first of its group: the group signals
  // once (its last arrival), with the first unit's counter slot
  static bool split_follower(const Instr &in) {
    return in.op == OP_DOWN && lay::split_n(in.aux1) > 1 && lay::split_s(in.aux1) > 0;
  }

  void add(Unit u) {
    u.in.sig0 = u.sigs.size() > 0 ? u.sigs[0] : -1;
    u.in.sig1 = u.sigs.size() > 1 ? u.sigs[1] : -1;
    if (!split_follower(u.in))
      for (int g : u.sigs) P.grp_producers[g] += 1;
    units.push_back(std::move(u));
  }

  // Once every unit exists: size each group's counter slots so that no
  // slot takes more than kAtomicsPerSlot increments, deal the producers
  // round-robin over the slots and give every wait its group's slot count.
  void assign_slots() {
    for (int g = 0; g < P.n_groups; ++g) {
      const uint32_t need = (P.grp_producers[g] + kAtomicsPerSlot - 1) / kAtomicsPerSlot;
      P.grp_nslot[g] = std::max(1u, std::min(need, (uint32_t)kSlots));
    }
    std::vector<uint32_t> next(P.n_groups, 0);
    for (size_t ui = 0; ui < units.size(); ++ui) {
      Unit &u = units[ui];
      if (split_follower(u.in)) {  // (the group's units are consecutive)
        u.in.slot0 = units[ui - 1].in.slot0;
        u.in.slot1 = units[ui - 1].in.slot1;
      } else {
        for (int i = 0; i < (int)u.sigs.size() && i < 2; ++i) {
          const int g = u.sigs[i];
          const uint32_t slot = next[g]++ % P.grp_nslot[g];
          P.grp_target[(size_t)g * kSlots + slot] += 1;
          (i == 0 ? u.in.slot0 : u.in.slot1) = slot;
        }
      }
      for (Wait &w : u.waits) w.nslot = (uint16_t)P.grp_nslot[w.grp];
    }
  }
};

Instr gemv(Op op, int layer, uint32_t item0, uint32_t n, int ipw, int K, int kc,
           uint32_t unit, bool mfma) {
  Instr in;
  std::memset(&in, 0, sizeof in);
  in.op = op;
  in.layer = (uint16_t)layer;
  in.ipw = (uint8_t)ipw;
  in.kc = (uint32_t)kc;
  in.pb = (uint32_t)(2 * kc);
  in.item0 = item0;
  in.n_items = n;
  if (mfma) {
    // MFMA stream (batched plans): pieces of kMfmaKc elements (the last one
    // zero-padded past K), 1 KB blocks of 8 rows x 64 elements (the last
    // block's rows past the unit repeat its last row), 16 blocks per page;
    // ppp holds the number of 8-row blocks
    in.nk = (uint16_t)((K + kMfmaKc - 1) / kMfmaKc);
    const uint32_t nrb = (n * ipw + 7) / 8;
    in.ppp = (uint16_t)nrb;
    const uint64_t blocks = (uint64_t)in.nk * nrb * (kMfmaKc / 64);
    in.pages = (uint32_t)((blocks + 15) / 16);
  } else {
    in.nk = (uint16_t)(K / kc);
    int ppp = kPageBytes / (int)in.pb;
    in.ppp = (uint16_t)ppp;
    uint64_t pieces = (uint64_t)n * ipw * in.nk;
    in.pages = (uint32_t)((pieces + ppp - 1) / ppp);
  }
  in.sig0 = in.sig1 = -1;
  in.tab = -1;
  in.rowb = (uint32_t)(2 * K);
  in.unit = unit;
  return in;
}

Instr plain(Op op, int layer, uint32_t unit) {
  Instr in;
  std::memset(&in, 0, sizeof in);
  in.op = op;
  in.layer = (uint16_t)layer;
  in.sig0 = in.sig1 = -1;
  in.tab = -1;
  in.unit = unit;
  return in;
}

}  // namespace

int build_plan(const mk_config &c, int B, int C, Plan &P, std::string &err) {
  P = Plan();
  const int L = c.n_layers, H = c.hidden, nq = c.n_q_heads, nkv = c.n_kv_heads;
  const int hd = c.head_dim, F = c.ffn_dim, V = c.vocab, S = c.max_seq;
  if (C < 1 || B < 1 || B > c.max_batch) {
    err = "num_cus and batch must be >= 1 and batch <= max_batch";
    return MK_ERR_INVALID_ARG;
  }
  if (B > kMaxBatch) {
    err = "batch must be <= 8 (positions and 1/rms of a step are staged in LDS)";
    return MK_ERR_UNSUPPORTED;
  }
  const int G = nq / nkv, HALF = hd / 2;
  // batched plans (MFMA) use pieces of kMfmaKc elements, the last one
  // zero-padded; batch-1 plans a divisor of K
  const bool mfma = B > 1;
  const int kc_h = mfma ? kMfmaKc : choose_kc(H, kMaxKc), kc_o = mfma ? kMfmaKc : choose_kc(nq * hd, kMaxKc);
  const int kc_f = mfma ? kMfmaKc : choose_kc(F, kMaxKc);
  if (!kc_h || !kc_o || !kc_f) {
    err = "hidden, n_q_heads*head_dim and ffn_dim must be multiples of 8";
    return MK_ERR_UNSUPPORTED;
  }
  const uint32_t PPG = (uint32_t)(G + 2) * HALF;     // QKV row pairs per KV head
  const uint32_t TP = (uint32_t)nkv * PPG;
  const int nk_f = (F + kc_f - 1) / kc_f;
  int chunks = c.mlp_chunks > 0 ? c.mlp_chunks : 4;
  chunks = std::min(chunks, nk_f);
  int n_split = c.kv_splits;
  if (n_split <= 0) {
    n_split = std::max(1, std::min(kMaxSplits, C / std::max(1, B * nkv)));
    n_split = std::min(n_split, std::max(1, (S + 15) / 16));
  }
  if (n_split > kMaxSplits) {
    err = "kv_splits must be <= 64";
    return MK_ERR_UNSUPPORTED;
  }
  const int split_len = (S + n_split - 1) / n_split;
  // attention on paged K/V (loader-streamed) for head_dim 128 and for splits
  // longer than the register path's prefetch; RPP rows per 16 KB page
  const bool paged_kv = hd == 128 || split_len > kAttnRegRows;
  const uint16_t rpp = (uint16_t)(hd == 128 ? 32 : 64);
  P.paged_kv = paged_kv;
  // a single split (paged) leaves nothing to reduce
  const bool fused_attn = paged_kv && n_split == 1;
  P.num_cus = C;
  P.batch = B;
  P.n_split = n_split;
  P.split_len = split_len;
  P.mlp_chunks = chunks;

  // units: at least one per CU (when there are rows for it), at most
  // `cap` row results per sequence-row of their LDS staging slot (QKV units
  // keep half of it for the RoPE values of their pairs)
  // units of one instruction: at least one per CU (and `at_least`), and
  // enough that the largest unit's rows * ipw * batch results fit `cap`
  // (units take ceil(rows / n) or floor(rows / n) rows)
  auto units_for = [&](uint32_t rows, uint32_t ipw, uint32_t at_least, uint32_t cap = kAccFloats) {
    uint32_t n = std::max<uint32_t>(std::min<uint32_t>((uint32_t)C, rows), at_least);
    uint32_t max_rows = std::max<uint32_t>(1, cap / (ipw * (uint32_t)B));
    // MFMA units hold at most kMfmaRows weight rows (four 16-row tiles)
    if (mfma) max_rows = std::min<uint32_t>(max_rows, (uint32_t)kMfmaRows / ipw);
    n = std::max<uint32_t>(n, (rows + max_rows - 1) / max_rows);
    return std::min<uint32_t>(n, rows);
  };
  const uint32_t n_qkv = units_for(TP, 2, (uint32_t)nkv, kAccFloats / 2);
  const uint32_t n_o = units_for(H, 1, 1), n_down = units_for(H, 1, 1);
  const uint32_t n_ffn = units_for(F, 2, (uint32_t)chunks);
  // batched: wide LM units (their results leave from registers, so the LDS
  // result-slot bound does not apply)
  const uint32_t n_lm = mfma ? std::min<uint32_t>(std::max<uint32_t>(std::min<uint32_t>((uint32_t)C, V),
                                                                     (V + kMfmaWideRows - 1) / kMfmaWideRows),
                                                  V)
                             : units_for(V, 1, 1);

  // batched: split-K down units, S = chunks per row group, row groups of at
  // most kMfmaRows rows, about one unit per workgroup
  const bool down_split = mfma && chunks > 1 && F < 65536;
  const uint32_t n_rg = down_split ? std::min<uint32_t>((uint32_t)H, std::max<uint32_t>(
                                         (uint32_t)C / (uint32_t)chunks, ((uint32_t)H + kMfmaRows - 1) / kMfmaRows))
                                   : 0;
  P.down_splits = down_split ? chunks : 0;
  P.n_down_groups = down_split ? (int)(n_rg * (uint32_t)L) : 0;
  auto chunk_k0 = [&](int ch) { return (uint32_t)((uint64_t)ch * nk_f / chunks); };
  // first element of chunk ch (F for ch == chunks)
  auto chunk_e0 = [&](int ch) { return std::min<uint32_t>(chunk_k0(ch) * kc_f, (uint32_t)F); };

  Builder bd(c, B, C, P);
  std::vector<int> g_down_prev(1, -1);
  int g_down = -1;
  for (int l = 0; l < L; ++l) {
    std::vector<int> g_attn(fused_attn ? 0 : (size_t)B * nkv), g_ffn(chunks);
    for (auto &g : g_attn) g = bd.group();
    const int g_red = bd.group(), g_o = bd.group();
    for (auto &g : g_ffn) g = bd.group();
    const int g_dn = bd.group();

    // I1: RMSNorm + QKV + RoPE.  Items are row pairs (i, i+hd/2) of one head
    // in KV-head-major order: for KV head g, its G query heads, then K, V.
    for (uint32_t u = 0; u < n_qkv; ++u) {
      uint32_t p0 = part_lo(TP, n_qkv, u), p1 = part_lo(TP, n_qkv, u + 1);
      Unit un;
      un.in = gemv(OP_QKV, l, p0, p1 - p0, 2, H, kc_h, u, mfma);
      un.in.aux0 = (uint32_t)G;
      un.in.aux1 = (uint32_t)hd;
      un.cu = (int)(u % C);
      if (l > 0) un.waits.push_back({(uint32_t)g_down, 0});
      for (int b = 0; b < B; ++b) {
        if (l > 0) un.reads.push_back({R_HOUT, (uint16_t)(l - 1), (uint32_t)b, 0, (uint32_t)H, 0});
        un.writes.push_back({R_QKV, (uint16_t)l, (uint32_t)b, p0, p1, 0});
      }
      // no counter: q and this step's K/V slot are tagged words that the
      // attention units read until every word carries the step's tag
      bd.add(std::move(un));
    }
    // I2: attention partials per (sequence, KV head, split).
    for (int b = 0; b < B; ++b)
      for (int g = 0; g < nkv; ++g)
        for (int s = 0; s < n_split; ++s) {
          uint32_t a = (uint32_t)((b * nkv + g) * n_split + s);
          Unit un;
          un.in = plain(OP_ATTN, l, a);
          un.in.ppp = paged_kv ? rpp : 0;
          un.in.b = (uint32_t)b;
          un.in.aux0 = (uint32_t)g;
          un.in.aux1 = (uint32_t)s;
          un.cu = (int)(a % C);
          un.reads.push_back({R_QKV, (uint16_t)l, (uint32_t)b, g * PPG, (g + 1) * PPG, 0, 1});
          if (fused_attn) {
            // one (paged) split per KV head: the unit merges in LDS and
            // writes the attention output itself
            un.writes.push_back({R_ATTN, (uint16_t)l, (uint32_t)b, (uint32_t)(g * G * hd),
                                 (uint32_t)((g + 1) * G * hd), 0});
            un.sigs.push_back(g_red);
          } else {
            un.writes.push_back({R_PART, (uint16_t)l, (uint32_t)b, (uint32_t)(g * n_split + s),
                                 (uint32_t)(g * n_split + s + 1), 0});
            un.sigs.push_back(g_attn[b * nkv + g]);
          }
          bd.add(std::move(un));
        }
    // I3: reduction of the partials per (sequence, KV head).
    const int n_red = fused_attn ? 0 : B * nkv;
    for (int r = 0; r < n_red; ++r) {
      int b = r / nkv, g = r % nkv;
      Unit un;
      un.in = plain(OP_RED, l, (uint32_t)r);
      un.in.b = (uint32_t)b;
      un.in.aux0 = (uint32_t)g;
      un.cu = (int)(((uint64_t)r * C / n_red) % C);
      un.waits.push_back({(uint32_t)g_attn[r], 0});
      un.reads.push_back({R_PART, (uint16_t)l, (uint32_t)b, (uint32_t)(g * n_split),
                          (uint32_t)((g + 1) * n_split), 0});
      un.writes.push_back({R_ATTN, (uint16_t)l, (uint32_t)b, (uint32_t)(g * G * hd),
                           (uint32_t)((g + 1) * G * hd), 0});
      un.sigs.push_back(g_red);
      bd.add(std::move(un));
    }
    // I4: O projection + residual, rows of H.
    for (uint32_t u = 0; u < n_o; ++u) {
      uint32_t r0 = part_lo(H, n_o, u), r1 = part_lo(H, n_o, u + 1);
      Unit un;
      un.in = gemv(OP_O, l, r0, r1 - r0, 1, nq * hd, kc_o, u, mfma);
      un.cu = (int)(u % C);
      un.waits.push_back({(uint32_t)g_red, 0});
      for (int b = 0; b < B; ++b) {
        un.reads.push_back({R_ATTN, (uint16_t)l, (uint32_t)b, 0, (uint32_t)(nq * hd), 0});
        if (l > 0) un.reads.push_back({R_HOUT, (uint16_t)(l - 1), (uint32_t)b, r0, r1, 0});
        un.writes.push_back({R_HMID, (uint16_t)l, (uint32_t)b, r0, r1, 0});
      }
      un.sigs.push_back(g_o);
      bd.add(std::move(un));
    }
    // I5: RMSNorm + gate/up + SiLU; items are FFN rows j (gate row, up row).
    for (uint32_t u = 0; u < n_ffn; ++u) {
      uint32_t j0 = part_lo(F, n_ffn, u), j1 = part_lo(F, n_ffn, u + 1);
      Unit un;
      un.in = gemv(OP_FFN, l, j0, j1 - j0, 2, H, kc_h, u, mfma);
      un.cu = (int)(u % C);
      un.waits.push_back({(uint32_t)g_o, 0});
      for (int b = 0; b < B; ++b) {
        un.reads.push_back({R_HMID, (uint16_t)l, (uint32_t)b, 0, (uint32_t)H, 0});
        un.writes.push_back({R_A, (uint16_t)l, (uint32_t)b, j0, j1, 0});
      }
      for (int ch = 0; ch < chunks; ++ch) {
        uint32_t e0 = chunk_e0(ch), e1 = chunk_e0(ch + 1);
        if (j0 < e1 && e0 < j1) un.sigs.push_back(g_ffn[ch]);
      }
      if (un.sigs.size() > 2) {
        err = "internal: an FFN unit spans more than two MLP chunks";
        return MK_ERR_UNSUPPORTED;
      }
      bd.add(std::move(un));
    }
    // I6, batched plans: split-K over the MLP chunks.  Every workgroup would
    // otherwise stage the whole activation of all sequences (F x batch fp32)
    // for a few rows; unit (row group, chunk s) stages chunk s only, waits
    // for chunk s only, and the last unit of a row group to finish sums the
    // chunks' partial rows in chunk order, adds the residual and signals.
    if (down_split) {
      for (uint32_t rg = 0; rg < n_rg; ++rg) {
        const uint32_t r0 = part_lo(H, n_rg, rg), r1 = part_lo(H, n_rg, rg + 1);
        const uint32_t group = (uint32_t)l * n_rg + rg;
        for (int ch = 0; ch < chunks; ++ch) {
          const uint32_t e0 = chunk_e0(ch), e1 = chunk_e0(ch + 1);
          Unit un;
          un.in = gemv(OP_DOWN, l, r0, r1 - r0, 1, F, kc_f, rg * chunks + (uint32_t)ch, mfma);
          un.in.nk = (uint16_t)(chunk_k0(ch + 1) - chunk_k0(ch));
          un.in.pages = (uint32_t)(((uint64_t)un.in.nk * un.in.ppp * 4 + 15) / 16);
          un.in.aux0 = e0 | ((e1 - e0) << 16);
          un.in.aux1 = (uint32_t)ch | ((uint32_t)chunks << 4) | (group << 8);
          un.cu = (int)((rg * chunks + (uint32_t)ch) % C);
          un.waits.push_back({(uint32_t)g_ffn[ch], 0});
          for (int b = 0; b < B; ++b) {
            un.reads.push_back({R_A, (uint16_t)l, (uint32_t)b, e0, e1, 0});
            un.reads.push_back({R_HMID, (uint16_t)l, (uint32_t)b, r0, r1, 0});
            un.writes.push_back({R_HOUT, (uint16_t)l, (uint32_t)b, r0, r1, 0});
          }
          un.sigs.push_back(g_dn);
          bd.add(std::move(un));
        }
      }
      g_down = g_dn;
      continue;
    }
    // I6: down projection + residual; consumes the MLP chunks in order.
    for (uint32_t u = 0; u < n_down; ++u) {
      uint32_t r0 = part_lo(H, n_down, u), r1 = part_lo(H, n_down, u + 1);
      Unit un;
      un.in = gemv(OP_DOWN, l, r0, r1 - r0, 1, F, kc_f, u, mfma);
      un.cu = (int)(u % C);
      for (int ch = 0; ch < chunks; ++ch) un.waits.push_back({(uint32_t)g_ffn[ch], chunk_k0(ch)});
      for (int b = 0; b < B; ++b) {
        for (int ch = 0; ch < chunks; ++ch)
          un.reads.push_back({R_A, (uint16_t)l, (uint32_t)b, chunk_e0(ch), chunk_e0(ch + 1), chunk_k0(ch)});
        un.reads.push_back({R_HMID, (uint16_t)l, (uint32_t)b, r0, r1, 0});
        un.writes.push_back({R_HOUT, (uint16_t)l, (uint32_t)b, r0, r1, 0});
      }
      un.sigs.push_back(g_dn);
      bd.add(std::move(un));
    }
    g_down = g_dn;
    (void)g_down_prev;
  }
  // I7: final RMSNorm + LM head.
  for (uint32_t u = 0; u < n_lm; ++u) {
    uint32_t v0 = part_lo(V, n_lm, u), v1 = part_lo(V, n_lm, u + 1);
    Unit un;
    un.in = gemv(OP_LM, L, v0, v1 - v0, 1, H, kc_h, u, mfma);
    un.in.layer = (uint16_t)L;
    un.cu = (int)(u % C);
    un.waits.push_back({(uint32_t)g_down, 0});
    for (int b = 0; b < B; ++b)
      un.reads.push_back({R_HOUT, (uint16_t)(L - 1), (uint32_t)b, 0, (uint32_t)H, 0});
    bd.add(std::move(un));
  }

  bd.assign_slots();
  // Per-CU queues in creation order (= stage order).
  std::vector<std::vector<int>> per_cu(C);
  // Workgroup w of a one-workgroup-per-CU launch runs on XCD w mod 8.  The
  // units are placed on logical CUs in blocks (QKV group g, its attention
  // splits and its reduction on logical CUs g*C/8 .. (g+1)*C/8 - 1); logical
  // CU x runs as workgroup (x / (C/8)) + 8 * (x % (C/8)), so each such block
  // shares one XCD and its L2.
  auto phys = [&](int x) {
#if MK_XCDMAP
    if (C % 8 == 0) return (x / (C / 8)) + 8 * (x % (C / 8));
#endif
    return x;
  };
  for (size_t i = 0; i < bd.units.size(); ++i) per_cu[phys(bd.units[i].cu)].push_back((int)i);
  P.q_off.assign(C + 1, 0);
  std::vector<int64_t> cu_bytes(C, 0);
  for (int cu = 0; cu < C; ++cu) {
    P.q_off[cu] = (uint32_t)P.instr.size();
    for (int ui : per_cu[cu]) {
      Unit &un = bd.units[ui];
      Instr in = un.in;
      in.wait_off = (uint32_t)P.waits.size();
      in.wait_n = (uint32_t)un.waits.size();
      for (auto &w : un.waits) P.waits.push_back(w);
      if (in.pages) {
        // K elements per row (no padding; a split unit its K window)
        const int64_t rowb = in.op == OP_DOWN && lay::split_n(in.aux1) > 1 ? 2 * (int64_t)lay::split_klen(in.aux0)
                                                                             : (int64_t)in.rowb;
        int64_t bytes = (int64_t)in.n_items * in.ipw * rowb;
        cu_bytes[cu] += bytes;
        P.weight_bytes += bytes;
        P.n_pages += (int)in.pages;
        const bool wide = mfma && in.op == OP_LM;
        if ((!wide && (int64_t)in.n_items * in.ipw * B > kAccFloats) ||
            (in.op == OP_QKV && (int64_t)in.n_items * in.ipw * B > kAccFloats / 2)) {
          err = "internal: too many rows in a unit";
          return MK_ERR_UNSUPPORTED;
        }
        if (mfma && (in.kc != (uint32_t)kMfmaKc ||
                     in.n_items * in.ipw > (uint32_t)(wide ? kMfmaWideRows : kMfmaRows))) {
          err = "internal: MFMA unit shape";
          return MK_ERR_UNSUPPORTED;
        }
      }
      P.instr.push_back(in);
      P.reads.push_back(un.reads);
      P.writes.push_back(un.writes);
    }
  }
  P.q_off[C] = (uint32_t)P.instr.size();
  P.max_cu_bytes = *std::max_element(cu_bytes.begin(), cu_bytes.end());
  // greedy candidates: the LM units of one workgroup keep a running best per
  // sequence in LDS and its last LM unit publishes it, so the arrival
  // counter counts workgroups (LM groups), not units.  aux0 = group index,
  // aux1 bit 0: first LM unit of its workgroup, bit 1: last.
  P.n_lm_groups = 0;
  for (int cu = 0; cu < C; ++cu) {
    int first = -1, last = -1;
    for (uint32_t qi = P.q_off[cu]; qi < P.q_off[cu + 1]; ++qi)
      if (P.instr[qi].op == OP_LM) {
        if (first < 0) first = (int)qi;
        last = (int)qi;
      }
    if (first < 0) continue;
    for (int qi = first; qi <= last; ++qi)
      if (P.instr[qi].op == OP_LM) {
        P.instr[qi].aux0 = (uint32_t)P.n_lm_groups;
        P.instr[qi].aux1 = (qi == first ? 1u : 0u) | (qi == last ? 2u : 0u);
      }
    ++P.n_lm_groups;
  }
  return MK_OK;
}

void resolve_streams(const mk_config &c, const mk_weights &w, Plan &P) {
  const int G = c.n_q_heads / c.n_kv_heads, hd = c.head_dim, half = hd / 2;
  const uint64_t Hb = 2ull * c.hidden;
  P.rowtab.clear();
  for (Instr &in : P.instr) {
    if (in.op == OP_ATTN || in.op == OP_RED) continue;
    in.tab = -1;
    if (in.op == OP_LM) {
      in.w0 = (uint64_t)(uintptr_t)(c.tied_embeddings ? w.embed : w.lm_head);
      continue;
    }
    const mk_layer_weights &ly = w.layers[in.layer];
    switch (in.op) {
      case OP_QKV: {
        // rows of pair (i, i + hd/2) of one head, in the pair order of the
        // unit: row r = 2*i + s
        in.tab = (int32_t)P.rowtab.size();
        const uint32_t ppg = (uint32_t)(G + 2) * half;
        for (uint32_t i = 0; i < in.n_items; ++i)
          for (uint32_t s = 0; s < 2; ++s) {
            const uint32_t pp = in.item0 + i, g = pp / ppg, rr = pp % ppg;
            const uint32_t hs = rr / half, ii = rr % half + s * half;
            uint64_t base;
            if (hs < (uint32_t)G) base = (uint64_t)(uintptr_t)ly.wq + ((uint64_t)(g * G + hs) * hd + ii) * Hb;
            else if (hs == (uint32_t)G) base = (uint64_t)(uintptr_t)ly.wk + ((uint64_t)g * hd + ii) * Hb;
            else base = (uint64_t)(uintptr_t)ly.wv + ((uint64_t)g * hd + ii) * Hb;
            P.rowtab.push_back(base);
          }
        break;
      }
      case OP_O: in.w0 = (uint64_t)(uintptr_t)ly.wo; break;
      case OP_FFN:
        in.w0 = (uint64_t)(uintptr_t)ly.w_gate;
        in.w1 = (uint64_t)(uintptr_t)ly.w_up;
        break;
      default: in.w0 = (uint64_t)(uintptr_t)ly.w_down; break;
    }
  }
  if (P.rowtab.empty()) P.rowtab.push_back(0);
}

// ---------------------------------------------------------------------------
// Validation: counter bookkeeping plus simulated interleavings.

namespace {

struct Sim {
  const Plan &P;
  int C;
  std::vector<uint32_t> target;               // per group
  std::vector<std::vector<int>> writers;      // per (read index) writer unit ids
  std::vector<std::vector<std::pair<uint32_t, int>>> read_ix;  // per unit: (phase, read list index)
  std::vector<std::vector<uint32_t>> phases;  // per unit: sorted distinct before_k
  std::vector<std::vector<int>> sig;          // per unit groups signalled

  explicit Sim(const Plan &p) : P(p), C(p.num_cus) {}
};

}  // namespace

int check_plan(const mk_config &cfg, Plan &P, int sim_runs, int corrupt, uint64_t seed,
               mk_plan_report *rep) {
  const int C = P.num_cus;
  const size_t NU = P.instr.size();
  std::string first;
  int errors = 0;
  auto fail = [&](const std::string &m) {
    if (first.empty()) first = m;
    ++errors;
  };
  std::mt19937_64 rng(seed);

  // Extents: every index an instruction or a recorded access carries stays
  // inside the buffer it addresses (the kernel forms its addresses from
  // these fields, the step's position and the lane alone).
  {
    if (corrupt == 4)
      for (Instr &in : P.instr)
        if (in.op == OP_ATTN) {
          in.aux1 = (uint32_t)P.n_split;  // one split past the last
          break;
        }
    const uint32_t H = (uint32_t)cfg.hidden, F = (uint32_t)cfg.ffn_dim, V = (uint32_t)cfg.vocab;
    const uint32_t nkv = (uint32_t)cfg.n_kv_heads, nq = (uint32_t)cfg.n_q_heads, hd = (uint32_t)cfg.head_dim;
    const uint32_t G = nq / nkv, ppg = (G + 2) * (hd / 2), ns = (uint32_t)P.n_split;
    if (P.n_split < 1 || P.n_split > kMaxSplits || P.split_len < 1 ||
        (int64_t)P.n_split * P.split_len < cfg.max_seq)
      fail("the KV splits do not cover max_seq slots");
    auto limit = [&](uint8_t op) -> uint32_t {
      switch (op) {
        case OP_QKV: return nkv * ppg;
        case OP_O: case OP_DOWN: return H;
        case OP_FFN: return F;
        case OP_LM: return V;
        default: return 0;
      }
    };
    for (size_t u = 0; u < NU; ++u) {
      const Instr &in = P.instr[u];
      if (in.layer >= (uint32_t)cfg.n_layers && in.op != OP_LM) fail("instruction layer out of range");
      if (in.b >= (uint32_t)P.batch) fail("instruction sequence out of range");
      if (in.op == OP_ATTN && (in.aux0 >= nkv || in.aux1 >= ns)) fail("attention unit head or split out of range");
      if (in.op == OP_RED && in.aux0 >= nkv) fail("reduction unit head out of range");
      if (in.op == OP_DOWN && lay::split_n(in.aux1) > 1 &&
          (lay::split_s(in.aux1) >= lay::split_n(in.aux1) || (int)lay::split_n(in.aux1) != P.down_splits ||
           lay::split_group(in.aux1) >= (uint32_t)P.n_down_groups ||
           lay::split_koff(in.aux0) + lay::split_klen(in.aux0) > F || lay::split_klen(in.aux0) == 0 ||
           (uint32_t)in.nk * kMfmaKc < lay::split_klen(in.aux0)))
        fail("split-K down unit out of range");
      const uint32_t lim = limit(in.op);
      if (lim && ((uint64_t)in.item0 + in.n_items > lim || in.n_items == 0)) fail("unit rows out of range");
      if (in.tab >= 0 && (size_t)in.tab + (size_t)in.n_items * in.ipw > P.rowtab.size())
        fail("row table entries out of range");
      if (in.wait_off + (uint64_t)in.wait_n > P.waits.size()) fail("wait entries out of range");
    }
    auto res_limit = [&](uint8_t res) -> uint32_t {
      switch (res) {
        case R_QKV: return nkv * ppg;
        case R_PART: return nkv * ns;
        case R_ATTN: return nq * hd;
        case R_HMID: case R_HOUT: return H;
        case R_A: return F;
        default: return 0;
      }
    };
    for (size_t u = 0; u < NU && u < P.reads.size(); ++u)
      for (const auto *lst : {&P.reads[u], &P.writes[u]})
        for (const Access &x : *lst) {
          const uint32_t lim = res_limit(x.res);
          if (!lim || x.lo > x.hi || x.hi > lim || x.layer >= (uint32_t)cfg.n_layers || x.b >= (uint32_t)P.batch)
            fail("a recorded access lies outside its buffer");
        }
  }

  // Deliberate corruption for validator self-tests.
  std::vector<uint32_t> target(P.n_groups, 0);
  for (int g = 0; g < P.n_groups; ++g)
    for (int x = 0; x < kSlots; ++x) target[g] += P.grp_target[(size_t)g * kSlots + x];
  std::vector<std::vector<int>> sig(NU);
  for (size_t u = 0; u < NU; ++u) {
    if (P.instr[u].sig0 >= 0) sig[u].push_back(P.instr[u].sig0);
    if (P.instr[u].sig1 >= 0) sig[u].push_back(P.instr[u].sig1);
  }
  std::vector<std::vector<Wait>> waits(NU);
  for (size_t u = 0; u < NU; ++u)
    for (uint32_t i = 0; i < P.instr[u].wait_n; ++i) waits[u].push_back(P.waits[P.instr[u].wait_off + i]);
  if (corrupt) {
    // pick a unit with both a signal and waiting consumers
    std::vector<int> cand;
    for (size_t u = 0; u < NU; ++u)
      if (!sig[u].empty() && P.instr[u].op != OP_LM) cand.push_back((int)u);
    int victim = cand.empty() ? -1 : cand[rng() % cand.size()];
    if (corrupt == 1 && victim >= 0) sig[victim].clear();
    if (corrupt == 2 && victim >= 0) target[sig[victim][0]] -= 1;
    if (corrupt == 3) {
      // a wait nothing else implies: reduction and gate/up units wait on
      // exactly the producers of what they read (other units' waits may be
      // implied through a chain, and dropping those is harmless)
      std::vector<int> w;
      for (size_t u = 0; u < NU; ++u)
        if (!waits[u].empty() && (P.instr[u].op == OP_RED || P.instr[u].op == OP_FFN)) w.push_back((int)u);
      if (!w.empty()) {
        int u = w[rng() % w.size()];
        waits[u].erase(waits[u].begin() + (rng() % waits[u].size()));
      }
    }
  }

  // Static: slot targets equal the producers dealt to each slot, every slot
  // in use, none over its atomic budget, and waits poll every used slot.
  {
    std::vector<uint32_t> cnt((size_t)P.n_groups * kSlots, 0);
    for (size_t u = 0; u < NU; ++u) {
      const Instr &in = P.instr[u];
      if (Builder::split_follower(in)) continue;  // counted with its group's first unit
      if (in.sig0 >= 0) {
        if (in.slot0 >= P.grp_nslot[in.sig0]) fail("signal slot outside its group");
        else cnt[(size_t)in.sig0 * kSlots + in.slot0]++;
      }
      if (in.sig1 >= 0) {
        if (in.slot1 >= P.grp_nslot[in.sig1]) fail("signal slot outside its group");
        else cnt[(size_t)in.sig1 * kSlots + in.slot1]++;
      }
    }
    if (cnt != P.grp_target) fail("counter targets differ from producer placement");
    for (int g = 0; g < P.n_groups; ++g)
      for (uint32_t x = 0; x < P.grp_nslot[g]; ++x) {
        const uint32_t t = P.grp_target[(size_t)g * kSlots + x];
        if (t == 0) fail("unused counter slot");
        if (t > (uint32_t)kAtomicsPerSlot && P.grp_nslot[g] < (uint32_t)kSlots) fail("slot over its atomic budget");
      }
    for (size_t u = 0; u < NU; ++u)
      for (auto &w : waits[u]) {
        if (w.grp >= (uint32_t)P.n_groups || P.grp_producers[w.grp] == 0)
          fail("wait on a group without producers");
        else if (w.nslot != P.grp_nslot[w.grp]) fail("wait polls a different slot count");
      }
  }

  // Writers of every read.
  struct Key { uint8_t res; uint16_t l; uint32_t b; };
  auto key_of = [](const Access &a) { return ((uint64_t)a.res << 48) | ((uint64_t)a.layer << 32) | a.b; };
  std::vector<std::pair<uint64_t, std::pair<uint32_t, int>>> wl;  // key -> (lo, unit)
  for (size_t u = 0; u < NU; ++u)
    for (auto &w : P.writes[u]) wl.push_back({key_of(w), {w.lo, (int)u}});
  std::sort(wl.begin(), wl.end());
  // per unit: (phase, writers) of counter-guarded reads and of tagged reads
  std::vector<std::vector<std::pair<uint32_t, std::vector<int>>>> rw(NU), rt(NU);
  for (size_t u = 0; u < NU; ++u)
    for (auto &r : P.reads[u]) {
      std::vector<int> ws;
      uint64_t k = key_of(r);
      auto it = std::lower_bound(wl.begin(), wl.end(), std::make_pair(k, std::make_pair(0u, -1)));
      for (; it != wl.end() && it->first == k; ++it) {
        int wu = it->second.second;
        for (auto &w : P.writes[wu])
          if (key_of(w) == k && w.lo < r.hi && r.lo < w.hi) { ws.push_back(wu); break; }
      }
      // every element of the read must have a writer
      std::vector<std::pair<uint32_t, uint32_t>> iv;
      for (int wu : ws)
        for (auto &w : P.writes[wu])
          if (key_of(w) == k) iv.push_back({std::max(w.lo, r.lo), std::min(w.hi, r.hi)});
      std::sort(iv.begin(), iv.end());
      uint32_t cov = r.lo;
      for (auto &p : iv)
        if (p.first <= cov) cov = std::max(cov, p.second);
      if (cov < r.hi) fail("a read has elements no unit writes");
      (r.tagged ? rt : rw)[u].push_back({r.phase, std::move(ws)});
    }

  // Every element has one writer: two units writing the same activation
  // elements would leave the step's result to whichever finished last.  (The
  // units of a split-K down group record the group's rows each; the group's
  // last arrival writes them once.)
  {
    if (corrupt == 5)  // self-test: one O unit's rows grow into the next O unit's
      for (size_t u = 0; u + 1 < NU; ++u)
        if (P.instr[u].op == OP_O && !P.writes[u].empty()) {
          bool grown = false;
          for (size_t v = u + 1; v < NU && !grown; ++v)
            if (P.instr[v].op == OP_O && P.instr[v].layer == P.instr[u].layer)
              for (auto &w : P.writes[v])
                if (key_of(w) == key_of(P.writes[u][0]) && w.lo >= P.writes[u][0].hi) {
                  P.writes[u][0].hi = w.lo + 1;
                  grown = true;
                  break;
                }
          if (grown) break;
        }
    auto one_writer = [&](int x, int y) {
      const Instr &a = P.instr[x], &b = P.instr[y];
      return x == y || (a.op == OP_DOWN && b.op == OP_DOWN && lay::split_n(a.aux1) > 1 &&
                        lay::split_n(b.aux1) > 1 && lay::split_group(a.aux1) == lay::split_group(b.aux1));
    };
    std::vector<std::pair<std::pair<uint64_t, uint32_t>, std::pair<uint32_t, int>>> ws;  // (key, lo) -> (hi, unit)
    for (size_t u = 0; u < NU; ++u)
      for (auto &w : P.writes[u]) ws.push_back({{key_of(w), w.lo}, {w.hi, (int)u}});
    std::sort(ws.begin(), ws.end());
    for (size_t i = 1; i < ws.size(); ++i)
      if (ws[i].first.first == ws[i - 1].first.first && ws[i].first.second < ws[i - 1].second.first &&
          !one_writer(ws[i].second.second, ws[i - 1].second.second)) {
        char m[200];
        std::snprintf(m, sizeof m, "units %d and %d (op %d, %d) write the same elements", ws[i - 1].second.second,
                      ws[i].second.second, P.instr[ws[i - 1].second.second].op, P.instr[ws[i].second.second].op);
        fail(m);
        break;
      }
  }

  // Happens-before, statically.  Inside a workgroup the roles pipeline: the
  // sync wave stages unit u's inputs while the compute waves may still be on
  // units u - 1 .. u - 3, so queue order orders nothing in global memory.
  // What does: a counter wait (its group's target implies every producer of
  // the group finished, and with it everything those producers waited for)
  // and a tagged read (the writer's words are there, so the writer passed
  // its own waits).  Every counter-guarded read must find each of its
  // writers among the units its waits (before the read's piece) and its
  // tagged reads imply.  (The interleavings below run each queue in order,
  // so they cannot see a missing wait on a producer of the same workgroup.)
  if (errors == 0) {
    const size_t words = (NU + 63) / 64;
    using Bits = std::vector<uint64_t>;
    std::vector<std::vector<int>> prod(P.n_groups);
    for (size_t u = 0; u < NU; ++u)
      for (int g : sig[u]) prod[g].push_back((int)u);
    std::vector<Bits> done_g(P.n_groups);
    std::vector<char> state(P.n_groups, 0);  // 0 new, 1 in progress, 2 done
    std::map<std::vector<int64_t>, Bits> pre_cache;
    auto has = [](const Bits &b, size_t i) { return (b[i >> 6] >> (i & 63)) & 1; };
    auto or_into = [](Bits &a, const Bits &b) {
      for (size_t i = 0; i < a.size(); ++i) a[i] |= b[i];
    };
    bool cyclic = false;
    std::function<const Bits &(int)> done_of;
    // units finished once unit p can start its reads: its waits' groups and
    // its tagged writers (each with what its own waits imply)
    auto pre_of = [&](int p) -> const Bits & {
      std::vector<int64_t> key;
      for (auto &w : waits[p]) key.push_back(w.grp);
      for (auto &rp : rt[p])
        for (int t : rp.second) key.push_back(-1 - (int64_t)t);
      std::sort(key.begin(), key.end());
      key.erase(std::unique(key.begin(), key.end()), key.end());
      auto it = pre_cache.find(key);
      if (it != pre_cache.end()) return it->second;
      Bits b(words, 0);
      for (int64_t k : key) {
        if (k >= 0) {
          or_into(b, done_of((int)k));
        } else {
          const int t = (int)(-1 - k);
          b[(size_t)t >> 6] |= 1ull << (t & 63);
          for (auto &w : waits[t]) or_into(b, done_of((int)w.grp));
        }
      }
      return pre_cache.emplace(key, std::move(b)).first->second;
    };
    // A group guarantees its producers (and what they waited for) only if
    // its target counts every one of them.
    done_of = [&](int g) -> const Bits & {
      if (state[g] == 2) return done_g[g];
      Bits b(words, 0);
      if (state[g] == 1) {
        cyclic = true;
        done_g[g] = std::move(b);
        return done_g[g];
      }
      state[g] = 1;
      if (target[g] >= P.grp_producers[g])
        for (int p : prod[g]) {
          b[(size_t)p >> 6] |= 1ull << (p & 63);
          or_into(b, pre_of(p));
        }
      done_g[g] = std::move(b);
      state[g] = 2;
      return done_g[g];
    };
    for (size_t u = 0; u < NU && errors == 0; ++u)
      for (auto &rp : rw[u]) {
        for (int wu : rp.second) {
          if (wu == (int)u) continue;
          bool ok = false;
          for (auto &w : waits[u])
            if (!ok && w.before_k <= rp.first && has(done_of((int)w.grp), (size_t)wu)) ok = true;
          for (auto &tp : rt[u])
            if (!ok && tp.first <= rp.first)
              for (int t : tp.second) {
                if (t == wu) ok = true;
                for (auto &w : waits[t])
                  if (!ok && has(done_of((int)w.grp), (size_t)wu)) ok = true;
                if (ok) break;
              }
          if (!ok) {
            char m[200];
            std::snprintf(m, sizeof m, "unit %zu (op %d layer %d) reads data of unit %d (op %d) no wait orders",
                          u, P.instr[u].op, P.instr[u].layer, wu, P.instr[wu].op);
            fail(m);
            break;
          }
        }
        if (errors) break;
      }
    if (cyclic) fail("the counter waits form a cycle");
  }

  // Phases of each unit: sorted distinct before_k values (always 0).
  std::vector<std::vector<uint32_t>> phases(NU);
  for (size_t u = 0; u < NU; ++u) {
    phases[u].push_back(0);
    for (auto &w : waits[u]) phases[u].push_back(w.before_k);
    std::sort(phases[u].begin(), phases[u].end());
    phases[u].erase(std::unique(phases[u].begin(), phases[u].end()), phases[u].end());
  }

  // Interleavings: each CU runs its queue strictly in order, phase by phase;
  // a phase may start once its waits' groups reached their targets.
  // split-K units signal through their group: the S-th arrival signals
  std::vector<int> sgroup(NU, -1);
  for (size_t u = 0; u < NU; ++u)
    if (P.instr[u].op == OP_DOWN && lay::split_n(P.instr[u].aux1) > 1)
      sgroup[u] = (int)lay::split_group(P.instr[u].aux1);
  int runs = 0;
  for (int run = 0; run < sim_runs && errors == 0; ++run, ++runs) {
    int strategy = run % 4;
    int delayed = (int)(rng() % C);
    std::vector<uint32_t> count(P.n_groups, 0);
    std::vector<uint32_t> arrived(std::max(1, P.n_down_groups), 0);
    std::vector<char> done(NU, 0);
    std::vector<uint32_t> pos(C), ph(C, 0);
    for (int cu = 0; cu < C; ++cu) pos[cu] = P.q_off[cu];
    size_t remaining = NU;
    std::vector<int> ready;
    while (remaining) {
      ready.clear();
      for (int cu = 0; cu < C; ++cu) {
        if (pos[cu] >= P.q_off[cu + 1]) continue;
        uint32_t u = pos[cu];
        uint32_t phase = phases[u][ph[cu]];
        bool ok = true;
        for (auto &w : waits[u])
          if (w.before_k == phase && count[w.grp] < target[w.grp]) { ok = false; break; }
        // a tagged read spins until its writers' words are there
        for (auto &rp : rt[u])
          if (ok && rp.first == phase)
            for (int wu : rp.second)
              if (!done[wu]) { ok = false; break; }
        if (ok) ready.push_back(cu);
      }
      if (ready.empty()) {
        fail("deadlock: no workgroup can make progress");
        break;
      }
      int cu;
      if (strategy == 0) cu = ready[rng() % ready.size()];
      else if (strategy == 1) {
        std::vector<int> others;
        for (int r : ready) if (r != delayed) others.push_back(r);
        cu = others.empty() ? ready[0] : others[rng() % others.size()];
      } else if (strategy == 2) {
        // earliest stage first
        cu = ready[0];
        for (int r : ready) if (pos[r] - P.q_off[r] < pos[cu] - P.q_off[cu]) cu = r;
      } else {
        // run one workgroup as far as it can go
        cu = ready[rng() % ready.size()];
        int best = -1;
        for (int r : ready) if (best < 0 || pos[r] - P.q_off[r] > pos[best] - P.q_off[best]) best = r;
        if (rng() % 2) cu = best;
      }
      uint32_t u = pos[cu];
      uint32_t phase = phases[u][ph[cu]];
      for (auto &rp : rw[u])
        if (rp.first == phase)
          for (int wu : rp.second)
            if (!done[wu]) {
              char m[200];
              std::snprintf(m, sizeof m, "unit %u (op %d layer %d) reads data of unit %d (op %d) before it finished",
                            u, P.instr[u].op, P.instr[u].layer, wu, P.instr[wu].op);
              fail(m);
              break;
            }
      if (errors) break;
      if (++ph[cu] == phases[u].size()) {
        done[u] = 1;
        --remaining;
        if (sgroup[u] < 0 || ++arrived[sgroup[u]] == (uint32_t)P.down_splits)
          for (int g : sig[u]) count[g]++;
        ph[cu] = 0;
        ++pos[cu];
      }
    }
  }
  if (rep) {
    rep->sim_runs = runs;
    rep->sim_errors = errors;
    std::snprintf(rep->msg, sizeof rep->msg, "%s", first.c_str());
  }
  return errors ? MK_ERR_INVALID_ARG : MK_OK;
}

}  // namespace mk
