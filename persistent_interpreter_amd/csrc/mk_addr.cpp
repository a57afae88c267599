// mk_addr.cpp -- host model of every global-memory access of the decode
// kernel, checked against the extent of the buffer it belongs to.
//
// For a configuration, a batch size and a run of steps (positions advancing
// by one per step, as in greedy decoding), the model builds the same plan the
// library uploads, gives every caller tensor and library buffer a synthetic
// base address (2^40 apart, so an overrun of one can never land in
// another), and walks each workgroup's queue the way each role of the kernel
// does: the sync wave's input checks, norm weights, RoPE values, activation
// pieces and residual rows; the loader waves' weight pieces and page
// sentinels; the compute waves' attention and reduction bodies, epilogues,
// greedy candidates and counter signals.  Every access is evaluated per lane
// with the offsets of mk_layout.hpp (the kernel's own arithmetic) and must
// lie inside the one buffer it addresses.  The loop structure of each body is
// mirrored from mk_kernel.hip; a change there must be made here too, and the
// tests run this model for every shape the GPU tests run.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_layout.hpp"
#include "mk_plan.hpp"
#include "mk_sched.hpp"

using namespace mk;

namespace {

constexpr int kShift = 40;

struct Model {
  struct Buf {
    std::string name;
    uint64_t bytes;
  };
  std::vector<Buf> bufs;
  int64_t n = 0;
  int bad = 0;
  std::string first;

  // Dependency records: every access of the unit being walked (`unit`, -1
  // outside units) to an activation buffer must fall in a range the plan
  // recorded as that unit's read or write, since the plan checker orders
  // exactly the recorded accesses.  The split-K partial rows after the
  // attention partials are private to a down-projection group and are not
  // recorded.
  int unit = -1;
  const Plan *plan = nullptr;
  uint64_t id_h = 0, id_attn = 0, id_a = 0, id_part = 0, id_q = 0, id_kvn = 0;
  uint64_t MB = 1, H = 1, nq = 1, hd = 1, F = 1, nkv = 1, ns = 1, G = 1, half = 1, ppg = 1, part_elems = 0;
  int64_t meta_n = 0;

  // the record found last and the absolute element interval of this
  // buffer it covers around the element asked for (accesses of one unit
  // mostly fall in the interval found just before)
  int c_unit = -1;
  uint64_t c_id = 0, c_lo = 0, c_hi = 0;

  const Access *find(uint8_t res, uint64_t layer, uint64_t b, uint64_t x) const {
    for (const auto *lst : {&plan->reads[unit], &plan->writes[unit]})
      for (const Access &r : *lst)
        if (r.res == res && r.layer == layer && r.b == b && r.lo <= x && x < r.hi) return &r;
    return nullptr;
  }
  // element e of buffer `id`: recorded for the current unit?  On success
  // [lo, hi) is an interval of elements around e that the same record covers
  bool covered(uint64_t id, uint64_t e, uint64_t &lo, uint64_t &hi) const {
    lo = e;
    hi = e + 1;
    if (id == id_h) {
      const uint64_t idx = e / (MB * H), b = (e / H) % MB, base = (idx * MB + b) * H;
      if (idx == 0) return false;  // the embedding's slot: never read or written as h
      const Access *r = (idx & 1) ? find(R_HMID, (idx - 1) / 2, b, e - base) : find(R_HOUT, idx / 2 - 1, b, e - base);
      if (!r) return false;
      lo = base + r->lo;
      hi = base + r->hi;
      return true;
    }
    if (id == id_attn || id == id_a) {
      const uint64_t row = id == id_attn ? nq * hd : F, lb = e / row, base = lb * row;
      const Access *r = find(id == id_attn ? R_ATTN : R_A, lb / MB, lb % MB, e - base);
      if (!r) return false;
      lo = base + r->lo;
      hi = base + r->hi;
      return true;
    }
    if (id == id_part) {
      if (e >= part_elems) {  // split-K partial rows: private to their group
        lo = part_elems;
        hi = ~0ull;
        return true;
      }
      const uint64_t rec = e / (hd + 4), s = rec % ns, j = (rec / ns) % nq, lb = rec / (ns * nq);
      if (!find(R_PART, lb / MB, lb % MB, (j / G) * ns + s)) return false;
      lo = rec * (hd + 4);
      hi = lo + hd + 4;
      return true;
    }
    // tagged q or this step's K/V words: QKV row pairs (i, i + hd/2) of a KV
    // head's group (its G query heads, then K, then V)
    uint64_t head, lb, pair0;
    if (id == id_q) {
      head = e / hd;
      const uint64_t j = head % nq;
      lb = head / nq;
      pair0 = (j / G) * ppg + (j % G) * half;
    } else {
      head = e / hd;  // (l, b, g, t) flattened
      const uint64_t t = head % 2, g = (head / 2) % nkv;
      lb = head / (2 * nkv);
      pair0 = g * ppg + (G + t) * half;
    }
    const uint64_t x = pair0 + (e % hd) % half;
    const Access *r = find(R_QKV, lb / MB, lb % MB, x);
    if (!r) return false;
    if (r->lo <= pair0 && pair0 + half <= r->hi) {  // the whole head
      lo = head * hd;
      hi = lo + hd;
    }
    return true;
  }
  void meta(uint64_t id, uint64_t off, uint32_t bytes, const char *site) {
    uint64_t es;
    if (id == id_h || id == id_attn || id == id_a || id == id_part) es = 4;
    else if (id == id_q || id == id_kvn) es = 8;
    else return;
    const uint64_t e0 = off / es, e1 = (off + bytes - 1) / es;
    ++meta_n;
    if (c_unit == unit && c_id == id && c_lo <= e0 && e1 < c_hi) return;
    // the first and the last element (the records are ranges of elements,
    // so an access whose ends are covered by one record is covered)
    uint64_t lo, hi, lo1, hi1;
    const bool ok0 = covered(id, e0, lo, hi);
    const bool ok1 = ok0 && (e1 < hi || covered(id, e1, lo1, hi1));
    if (ok0 && ok1) {
      c_unit = unit;
      c_id = id;
      c_lo = lo;
      c_hi = hi;
      return;
    }
    if (first.empty()) {
      char m[256];
      std::snprintf(m, sizeof m, "%s: unit %d (op %d layer %d) touches %s element %llu, which the plan "
                    "does not record for it", site, unit, (int)plan->instr[unit].op,
                    (int)plan->instr[unit].layer, bufs[id - 1].name.c_str(),
                    (unsigned long long)(ok0 ? e1 : e0));
      first = m;
    }
    ++bad;
  }

  uint64_t add(const std::string &name, uint64_t bytes) {
    bufs.push_back({name, bytes});
    return (uint64_t)bufs.size() << kShift;
  }
  // an access of `bytes` at absolute synthetic address `addr`, which must lie
  // in buffer `want` (0: any buffer, for weight streams whose tensor is
  // resolved by the plan)
  void at(uint64_t addr, uint32_t bytes, uint64_t want, const char *site) {
    ++n;
    const uint64_t id = addr >> kShift, off = addr & ((1ull << kShift) - 1);
    const bool in = id >= 1 && id <= bufs.size() && off + bytes <= bufs[id - 1].bytes &&
                    (want == 0 || (want >> kShift) == id);
    if (in && unit >= 0 && plan) meta(id, off, bytes, site);
    if (!in) {
      if (first.empty()) {
        char m[256];
        std::snprintf(m, sizeof m, "%s: %u bytes at %s+%llu (size %llu)%s%s", site, bytes,
                      id >= 1 && id <= bufs.size() ? bufs[id - 1].name.c_str() : "?", (unsigned long long)off,
                      id >= 1 && id <= bufs.size() ? (unsigned long long)bufs[id - 1].bytes : 0ull,
                      want ? ", expected in " : "", want ? bufs[(want >> kShift) - 1].name.c_str() : "");
        first = m;
      }
      ++bad;
    }
  }
  // element access into buffer `base` (element size `es`)
  void el(uint64_t base, uint64_t idx, uint32_t es, uint32_t bytes, const char *site) {
    at(base + idx * es, bytes, base, site);
  }
};

struct Bases {
  uint64_t tokens, positions, kv, logits, next_tok, next_pos;
  // the step being walked: where its tokens come from (the caller's, or for
  // step s > 0 of a launch of several steps the ones step s - 1 wrote), the
  // first logits element of its row block, and whether its sync waves wait
  // on the token counter
  uint64_t tok_src = 0, logit_off = 0;
  bool tok_wait = false;
  uint64_t h, q, kvn, attn, a, part, rope, status, ctr, target, amax, rowtab, iota;
  uint64_t embed, lm_head, final_norm, zero;
  std::vector<uint64_t> attn_norm, q_norm, k_norm, ffn_norm;
};

}  // namespace

// Paged attention (attn_paged and load_kv_page of mk_kernel.hip): the K/V
// page loads of one unit, and the compute waves' global accesses.
static void paged_kv_loads(Model &M, const Bases &B, const Plan &P, const mk_config &c, const Instr &d, int p,
                           uint32_t &n) {
  const int MB = c.max_batch, nkv = c.n_kv_heads, S = c.max_seq, hd = c.head_dim;
  const int CPR = hd / 8, RPL = 64 / CPR, RPP = 8 * RPL;
  const int lo = (int)d.aux1 * P.split_len, hi = std::min(lo + P.split_len, p + 1);
  const uint32_t nr = (uint32_t)std::max(0, std::min(hi, p) - lo);
  const uint32_t np = (nr + RPP - 1) / RPP;
  const uint64_t Kb = lay::kv(MB, nkv, S, hd, d.layer, 0, (int)d.b, (int)d.aux0, lo);
  const uint64_t Vb = lay::kv(MB, nkv, S, hd, d.layer, 1, (int)d.b, (int)d.aux0, lo);
  for (uint32_t jp = 0; jp < np; ++jp, ++n) {
    for (int kvt = 0; kvt < 2; ++kvt)
      for (uint32_t jj = 0; jj < 8; ++jj)
        for (int lane = 0; lane < 64; ++lane) {
          const uint32_t t = jj * RPL + lane / CPR, cp = lane % CPR;
          uint32_t r = jp * RPP + t;
          if (r >= nr) r = 0;
          const uint32_t ch = kvt ? cp : (cp ^ (t & 7));
          if (r >= (uint32_t)(hi - lo)) M.at(~0ull, 16, 0, "loader: K/V row outside its split");
          M.el(B.kv, (kvt ? Vb : Kb) + (uint64_t)r * hd + ch * 8, 2, 16, "loader: K/V page row");
        }
    M.el(B.iota, n, 4, 4, "loader: K/V page sentinel");
  }
}

static void paged_attn_compute(Model &M, const Bases &B, const Plan &P, const mk_config &c, const Instr &d, int p) {
  const int MB = c.max_batch, nq = c.n_q_heads, nkv = c.n_kv_heads, S = c.max_seq, hd = c.head_dim;
  const int G = nq / nkv, WPH = kNCW / G, CPR = hd / 8, DPL = hd / 64, ns = P.n_split;
  const int b = (int)d.b, g = (int)d.aux0, s = (int)d.aux1;
  const int lo = s * P.split_len, hi = std::min(lo + P.split_len, p + 1);
  const bool has_p = p >= lo && p < hi;
  for (int cw = 0; cw < kNCW; ++cw) {
    const int h = cw % G, rp = cw / G, j = g * G + h;
    if (rp != 0) continue;  // the other waves read LDS only
    for (int lane = 0; lane < 64; ++lane) {
      if (lo < hi) {
        if (c.qk_norm && DPL == 2) {
          for (int m = 0; m < DPL; ++m) {
            M.el(B.q_norm[d.layer], lane + 64 * m, 2, 2, "attn(paged): q_norm weight");
            M.el(B.k_norm[d.layer], lane + 64 * m, 2, 2, "attn(paged): k_norm weight");
          }
          M.el(B.rope, lay::rope(hd, p, lane), 4, 8, "attn(paged): RoPE of (lane, lane + 64)");
        }
        for (int m = 0; m < DPL; ++m) {
          M.el(B.q, lay::q(MB, nq, hd, d.layer, b, j) + lane + 64 * m, 8, 8, "attn(paged): tagged q");
          if (has_p) {
            M.el(B.kvn, lay::kvn(MB, nkv, hd, d.layer, b, g, 0) + lane + 64 * m, 8, 8, "attn(paged): tagged K");
            M.el(B.kvn, lay::kvn(MB, nkv, hd, d.layer, b, g, 0) + hd + lane + 64 * m, 8, 8, "attn(paged): tagged V");
          }
        }
        if (c.qk_norm && DPL == 2 && has_p && h == 0) {
          M.el(B.kv, lay::kv(MB, nkv, S, hd, d.layer, 0, b, g, p) + lane, 2, 2, "attn(paged): K store at p");
          M.el(B.kv, lay::kv(MB, nkv, S, hd, d.layer, 0, b, g, p) + lane + 64, 2, 2, "attn(paged): K store at p");
        }
      }
      if (has_p)
        for (int i = 0; i < 8; ++i)
          M.el(B.kvn, lay::kvn(MB, nkv, hd, d.layer, b, g, 0) + hd + (lane % CPR) * 8 + i, 8, 8,
               "attn(paged): V of row p");
      if (ns == 1) {
        if (lane < CPR)
          for (int i = 0; i < 8; ++i)
            M.el(B.attn, lay::attn(MB, nq, hd, d.layer, b) + (uint64_t)j * hd + lane * 8 + i, 4, 4,
                 "attn(paged): output (single split)");
      } else {
        const uint64_t out = lay::part(MB, nq, ns, hd, d.layer, b, j, s);
        if (lane < CPR)
          for (int i = 0; i < 8; ++i) M.el(B.part, out + lane * 8 + i, 4, 4, "attn(paged): partial o");
        if (lane == 0) {
          M.el(B.part, out + hd, 4, 4, "attn(paged): partial m");
          M.el(B.part, out + hd + 1, 4, 4, "attn(paged): partial l");
        }
      }
    }
  }
  M.el(B.ctr, ((uint64_t)d.sig0 * kSlots + d.slot0) * kCtrStride, 4, 4, "attn(paged): counter signal");
}

// The batched (MFMA) kernel: sync_role_b, loader_role_b, compute_role_b and
// unit_epilogue_b of mk_kernel.hip.
static void walk_batched(Model &M, const Bases &B, const Plan &P, const mk_config &c, int batch, int num_cus,
                         const std::vector<int> &pos_in, const int32_t *tokens, bool inputs_ok) {
  const int L = c.n_layers, H = c.hidden, nq = c.n_q_heads, nkv = c.n_kv_heads, hd = c.head_dim;
  const int F = c.ffn_dim, V = c.vocab, MB = c.max_batch, S = c.max_seq, G = nq / nkv, half = hd / 2;
  const int ns = P.n_split;
  std::vector<int> pos(batch);
  for (int b = 0; b < batch; ++b) pos[b] = (pos_in[b] < 0 || pos_in[b] >= S) ? 0 : pos_in[b];
  auto is_gemv = [](uint8_t op) { return op == OP_QKV || op == OP_O || op == OP_FFN || op == OP_DOWN || op == OP_LM; };
  // input vector of a normed instruction for sequence b (norm_src)
  auto norm_src = [&](const Instr &d, int b, uint64_t &h, uint64_t &emb, uint64_t &nw) {
    h = emb = 0;
    if (d.op == OP_QKV) {
      nw = B.attn_norm[d.layer];
      if (d.layer == 0) emb = B.embed + (uint64_t)tokens[b] * H * 2;
      else h = B.h + lay::h(MB, H, 2 * d.layer, b) * 4;
    } else if (d.op == OP_FFN) {
      nw = B.ffn_norm[d.layer];
      h = B.h + lay::h(MB, H, 2 * d.layer + 1, b) * 4;
    } else {
      nw = B.final_norm;
      h = B.h + lay::h(MB, H, 2 * L, b) * 4;
    }
  };
  for (int cu = 0; cu < num_cus; ++cu) {
    M.unit = -1;
    const uint32_t q0 = P.q_off[cu], q1 = P.q_off[cu + 1];
    // ---- sync wave (sync_role_b: staging pipeline)
    for (int b = 0; b < batch; ++b) {
      M.el(B.tok_src, b, 4, 4, "sync(b): tokens[b]");
      M.el(B.positions, b, 4, 4, "sync(b): positions[b]");
    }
    if (inputs_ok)
      for (uint32_t qi = q0; qi < q1; ++qi) {
        const Instr &d = P.instr[qi];
        M.unit = (int)qi;
        const bool gv = is_gemv(d.op);
        const uint32_t nx = gv ? d.nk : 1;
        const bool normed = d.op == OP_QKV || d.op == OP_FFN || d.op == OP_LM;
        const bool emb_in = d.op == OP_QKV && d.layer == 0;
        if (d.op == OP_QKV) {
          const uint32_t ppg = (uint32_t)(G + 2) * half;
          for (uint32_t x = 0; x < d.n_items * (uint32_t)batch; ++x) {
            const uint32_t i = x / batch, b = x % batch, ii = ((d.item0 + i) % ppg) % half;
            M.el(B.rope, lay::rope(hd, pos[b], (int)ii), 4, 8, "sync(b): RoPE of (pair, sequence)");
          }
        }
        for (uint32_t w = 0; w < d.wait_n; ++w) {
          const Wait &wt = P.waits[d.wait_off + w];
          for (uint32_t lane = 0; lane < wt.nslot; ++lane) {
            M.el(B.ctr, ((uint64_t)wt.grp * kSlots + lane) * kCtrStride, 4, 4, "sync(b): counter poll");
            M.el(B.target, (uint64_t)wt.grp * kSlots + lane, 4, 4, "sync(b): slot target");
          }
          M.el(B.status, 0, 4, 4, "sync(b): status poll");
        }
        if (!gv) continue;
        const bool split = d.op == OP_DOWN && lay::split_n(d.aux1) > 1;
        const uint32_t koff = split ? lay::split_koff(d.aux0) : 0u;
        const uint32_t K = split ? lay::split_klen(d.aux0) : d.rowb >> 1;
        uint64_t nw = 0;
        if (normed) {
          uint64_t h, emb;
          norm_src(d, 0, h, emb, nw);
        }
        for (uint32_t k = 0; k < nx; ++k) {
          const uint32_t kp = lay::mfma_phys_k(k, d.nk, d.unit);  // the piece logical piece k stages
          for (int lane = 0; lane < 64; ++lane) {
            const uint32_t e0 = kp * kMfmaKc + 4 * (uint32_t)lane;
            for (int b = 0; b < batch; ++b) {
              if (emb_in) {
                if (e0 < K) M.at(B.embed + ((uint64_t)tokens[b] * H + e0) * 2, 8, B.embed, "sync(b): embedding piece");
                continue;
              }
              uint64_t src, want;
              if (d.op == OP_O) { src = B.attn + lay::attn(MB, nq, hd, d.layer, b) * 4; want = B.attn; }
              else if (d.op == OP_DOWN) { src = B.a + (lay::a(MB, F, d.layer, b) + koff) * 4; want = B.a; }
              else { uint64_t emb, w; norm_src(d, b, src, emb, w); want = B.h; }
              if (e0 < K) M.at(src + (uint64_t)e0 * 4, 16, want, "sync(b): staged activation");
              else M.at(B.zero, 16, B.zero, "sync(b): zero padding");
            }
            if (normed && lane < 32) {
              const uint32_t w0 = kp * kMfmaKc + 8 * (uint32_t)lane;
              if (w0 < K) M.at(nw + (uint64_t)w0 * 2, 16, nw, "sync(b): staged norm weights");
              else M.at(B.zero, 16, B.zero, "sync(b): zero padding");
            }
          }
          if (k == 0 && (d.op == OP_O || d.op == OP_DOWN))
            for (int b = 0; b < batch; ++b)
              for (uint32_t r = 0; r < d.n_items; ++r) {
                if (d.op == OP_O && d.layer == 0)
                  M.at(B.embed + ((uint64_t)tokens[b] * H + d.item0 + r) * 2, 2, B.embed, "sync(b): embedding residual");
                else
                  M.el(B.h, lay::h(MB, H, d.op == OP_O ? 2 * d.layer : 2 * d.layer + 1, b) + d.item0 + r, 4, 4,
                       "sync(b): residual rows");
              }
        }
      }
    // ---- loader waves
    uint32_t n = 0;
    for (uint32_t qi = q0; qi < q1; ++qi) {
      const Instr &d = P.instr[qi];
      M.unit = (int)qi;
      if (d.op == OP_ATTN && d.ppp) {
        paged_kv_loads(M, B, P, c, d, pos[d.b], n);
        continue;
      }
      if (!is_gemv(d.op)) continue;
      const bool split = d.op == OP_DOWN && lay::split_n(d.aux1) > 1;
      const uint32_t koff = split ? lay::split_koff(d.aux0) : 0u;
      const uint32_t R = d.n_items * d.ipw, nrb = d.ppp, K = split ? lay::split_klen(d.aux0) : d.rowb >> 1;
      const uint32_t nblk = (uint32_t)d.nk * nrb * 4;
      const bool wide = lay::mfma_wide(nrb);
      for (uint32_t p = 0; p < d.pages; ++p, ++n) {
        for (uint32_t j = 0; j < 16; ++j) {
          uint32_t Lb = p * 16 + j;
          if (Lb >= nblk) Lb = 0;
          uint32_t k, kb, rb;
          lay::mfma_block(Lb, nrb, wide, k, kb, rb);
          k = lay::mfma_phys_k(k, d.nk, d.unit);
          if (d.tab >= 0)
            for (uint32_t i = 0; i < 8; ++i)
              M.el(B.rowtab, (uint64_t)d.tab + std::min(rb * 8 + i, R - 1), 8, 8, "loader(b): row table");
          for (int lane = 0; lane < 64; ++lane) {
            const uint32_t r = std::min(rb * 8 + (uint32_t)(lane & 7), R - 1);
            uint64_t row;
            if (d.tab >= 0) row = (size_t)d.tab + r < P.rowtab.size() ? P.rowtab[d.tab + r] : 0;
            else if (d.ipw == 2) row = ((r & 1) ? d.w1 : d.w0) + (uint64_t)(d.item0 + (r >> 1)) * d.rowb;
            else row = d.w0 + (uint64_t)(d.item0 + r) * d.rowb;
            const uint32_t kk = k * kMfmaKc + kb * 64 + 8 * (uint32_t)(lane >> 3);
            if (kk < K) {
              M.at(row + (uint64_t)(koff + kk) * 2, 16, 0, "loader(b): weight block");
              if (koff + kk + 8 > (d.rowb >> 1)) M.at(~0ull, 16, 0, "loader(b): weight block crosses its row");
            } else {
              M.at(B.zero, 16, B.zero, "loader(b): zero padding");
            }
          }
        }
        M.el(B.iota, n, 4, 4, "loader(b): page sentinel");
      }
    }
    // ---- compute waves
    if (!inputs_ok) continue;
    for (uint32_t qi = q0; qi < q1; ++qi) {
      const Instr &d = P.instr[qi];
      M.unit = (int)qi;
      const int b0 = (int)d.b;
      if (d.op == OP_ATTN && d.ppp) {
        paged_attn_compute(M, B, P, c, d, pos[b0]);
      } else if (d.op == OP_ATTN) {
        const int g = (int)d.aux0, s = (int)d.aux1;
        const int DPL = hd / 64, PF = 20 / DPL, NR = DPL == 1 ? 16 : 8;
        const int p = pos[b0];
        const int lo = s * P.split_len, hi = std::min(lo + P.split_len, p + 1);
        const int nt0 = std::max(0, std::min(hi - lo, PF));
        const uint64_t Kr = lay::kv(MB, nkv, S, hd, d.layer, 0, b0, g, lo);
        const uint64_t Vr = lay::kv(MB, nkv, S, hd, d.layer, 1, b0, g, lo);
        for (int h = 0; h < G; ++h) {
          const int j = g * G + h;
          for (int lane = 0; lane < 64; ++lane) {
            if (nt0 > 0)
              for (int t = 0; t < PF; ++t)
                for (int m = 0; m < DPL; ++m) {
                  const int tt = std::min(t, nt0 - 1);
                  M.el(B.kv, Kr + (uint64_t)tt * hd + lane + 64 * m, 2, 2, "attn(b): prefetched K");
                  M.el(B.kv, Vr + (uint64_t)tt * hd + lane + 64 * m, 2, 2, "attn(b): prefetched V");
                }
            if (lo < hi) {
              const bool has_p = p < hi;
              for (int m = 0; m < DPL; ++m) {
                M.el(B.q, lay::q(MB, nq, hd, d.layer, b0, j) + lane + 64 * m, 8, 8, "attn(b): tagged q");
                if (has_p) {
                  M.el(B.kvn, lay::kvn(MB, nkv, hd, d.layer, b0, g, 0) + lane + 64 * m, 8, 8, "attn(b): tagged K");
                  M.el(B.kvn, lay::kvn(MB, nkv, hd, d.layer, b0, g, 0) + hd + lane + 64 * m, 8, 8,
                       "attn(b): tagged V");
                }
              }
              for (int c0 = lo + PF; c0 < hi; c0 += 64) {
                const int nt = std::min(64, hi - c0);
                for (int kvt = 0; kvt < 2; ++kvt)
                  for (int t0 = 0; t0 < nt; t0 += NR)
                    for (int t = 0; t < NR; ++t) {
                      const int tt = std::min(t0 + t, nt - 1);
                      if (c0 + tt == p) continue;
                      for (int m = 0; m < DPL; ++m)
                        M.el(B.kv, (kvt ? Vr : Kr) + (uint64_t)(c0 - lo + tt) * hd + lane + 64 * m, 2, 2,
                             "attn(b): K/V row of the long split");
                    }
              }
            }
            const uint64_t out = lay::part(MB, nq, ns, hd, d.layer, b0, j, s);
            for (int m = 0; m < DPL; ++m) M.el(B.part, out + lane + 64 * m, 4, 4, "attn(b): partial o");
            if (lane == 0) {
              M.el(B.part, out + hd, 4, 4, "attn(b): partial m");
              M.el(B.part, out + hd + 1, 4, 4, "attn(b): partial l");
            }
          }
        }
        M.el(B.ctr, ((uint64_t)d.sig0 * kSlots + d.slot0) * kCtrStride, 4, 4, "attn(b): counter signal");
      } else if (d.op == OP_RED) {
        const int g = (int)d.aux0, DPL = hd / 64, RB = 32 / DPL;
        const uint32_t rowb = (uint32_t)(hd + 4) * 4;
        for (int h = 0; h < G; ++h) {
          const int j = g * G + h;
          const uint64_t base = B.part + lay::part(MB, nq, ns, hd, d.layer, b0, j, 0) * 4;
          for (int lane = 0; lane < 64; ++lane) {
            if (lane < ns) {
              M.at(base + (uint64_t)lane * rowb + hd * 4, 4, B.part, "red(b): m");
              M.at(base + (uint64_t)lane * rowb + hd * 4 + 4, 4, B.part, "red(b): l");
            }
            for (int s0 = 0; s0 < ns; s0 += RB)
              for (int t = 0; t < RB; ++t)
                for (int m = 0; m < DPL; ++m)
                  M.at(base + (uint64_t)std::min(s0 + t, ns - 1) * rowb + (uint64_t)(lane + 64 * m) * 4, 4, B.part,
                       "red(b): o");
            for (int m = 0; m < DPL; ++m)
              M.el(B.attn, lay::attn(MB, nq, hd, d.layer, b0) + (uint64_t)j * hd + lane + 64 * m, 4, 4,
                   "red(b): output");
          }
        }
        M.el(B.ctr, ((uint64_t)d.sig0 * kSlots + d.slot0) * kCtrStride, 4, 4, "red(b): counter signal");
      } else {
        for (uint32_t x = 0; x < d.n_items * (uint32_t)batch; ++x) {
          const uint32_t i = x / batch;
          const int b = (int)(x % batch);
          switch (d.op) {
            case OP_QKV: {
              const uint32_t ppg = (uint32_t)(G + 2) * half, pp = d.item0 + i, g = pp / ppg, rr = pp - g * ppg;
              const uint32_t hs = rr / half, ii = rr - hs * half;
              if (hs < (uint32_t)G) {
                const uint64_t qo = lay::q(MB, nq, hd, d.layer, b, (int)(g * G + hs));
                M.el(B.q, qo + ii, 8, 8, "epilogue(b): q word");
                M.el(B.q, qo + ii + half, 8, 8, "epilogue(b): q word");
              } else {
                const int t = hs == (uint32_t)G ? 0 : 1;
                const uint64_t ko = lay::kv(MB, nkv, S, hd, d.layer, t, b, (int)g, pos[b]);
                M.el(B.kv, ko + ii, 2, 2, "epilogue(b): K/V slot p");
                M.el(B.kv, ko + ii + half, 2, 2, "epilogue(b): K/V slot p");
                const uint64_t no = lay::kvn(MB, nkv, hd, d.layer, b, (int)g, t);
                M.el(B.kvn, no + ii, 8, 8, "epilogue(b): tagged K/V");
                M.el(B.kvn, no + ii + half, 8, 8, "epilogue(b): tagged K/V");
              }
              break;
            }
            case OP_O: M.el(B.h, lay::h(MB, H, 2 * d.layer + 1, b) + d.item0 + i, 4, 4, "epilogue(b): O"); break;
            case OP_FFN: M.el(B.a, lay::a(MB, F, d.layer, b) + d.item0 + i, 4, 4, "epilogue(b): FFN"); break;
            case OP_DOWN:
              if (lay::split_n(d.aux1) > 1) {
                // split-K: this chunk's partial row, then (as the group's
                // last arrival) every chunk's partial row
                const int S2 = (int)lay::split_n(d.aux1);
                M.el(B.part, lay::part_size(L, MB, nq, ns, hd) + lay::dpart(H, MB, S2, d.layer, (int)lay::split_s(d.aux1),
                                                                            (int)(d.item0 + i), b),
                     4, 4, "epilogue(b): split partial");
                for (int s2 = 0; s2 < S2; ++s2)
                  M.el(B.part, lay::part_size(L, MB, nq, ns, hd) + lay::dpart(H, MB, S2, d.layer, s2, (int)(d.item0 + i), b),
                       4, 4, "epilogue(b): split partials read");
              }
              M.el(B.h, lay::h(MB, H, 2 * d.layer + 2, b) + d.item0 + i, 4, 4, "epilogue(b): down");
              break;
            default: M.el(B.logits, B.logit_off + lay::logits(V, b) + d.item0 + i, 4, 4, "epilogue(b): logits"); break;
          }
        }
        if (d.op == OP_DOWN && lay::split_n(d.aux1) > 1)
          M.el(B.ctr, (uint64_t)P.n_groups * kSlots * kCtrStride + kCtrStride + lay::split_group(d.aux1), 4, 4,
               "epilogue(b): split arrival counter");
        if (d.op == OP_LM && (d.aux1 & 2u)) {
          for (int b = 0; b < batch; ++b)
            M.el(B.amax, (uint64_t)d.aux0 * batch + b, 8, 8, "epilogue(b): workgroup greedy candidate");
          M.el(B.ctr, (uint64_t)P.n_groups * kSlots * kCtrStride, 4, 4, "greedy(b): arrival counter");
          M.el(B.ctr, (uint64_t)P.n_groups * kSlots * kCtrStride + kTokWord, 4, 4, "greedy(b): token counter");
          for (int u = 0; u < P.n_lm_groups; ++u)
            for (int b = 0; b < batch; ++b) M.el(B.amax, (uint64_t)u * batch + b, 8, 8, "greedy(b): candidates");
          for (int b = 0; b < batch; ++b) {
            M.el(B.next_tok, b, 4, 4, "greedy(b): next token");
            M.el(B.next_pos, b, 4, 4, "greedy(b): next position");
          }
        }
        for (int sg : {d.sig0, d.sig1})
          if (sg >= 0) {
            const uint32_t slot = sg == d.sig0 ? d.slot0 : d.slot1;
            M.el(B.ctr, ((uint64_t)sg * kSlots + slot) * kCtrStride, 4, 4, "epilogue(b): counter signal");
          }
      }
    }
    M.el(B.status, 0, 4, 12, "raise_error: status words");
  }
}

// `steps` steps, as that many one-step launches, or (one_launch) as one
// launch of `steps` chained steps.
static int addr_check(const mk_config *cfg, int32_t batch, int32_t num_cus, int32_t steps, bool one_launch,
                      const int32_t *positions, const int32_t *tokens, int32_t corrupt, mk_addr_report *rep) {
  if (rep) std::memset(rep, 0, sizeof *rep);
  if (!cfg || !positions || !tokens || batch < 1 || num_cus < 1 || steps < 1) return MK_ERR_INVALID_ARG;
  const mk_config &c = *cfg;
  Plan P;
  std::string err;
  int rc = build_plan(c, batch, num_cus, P, err);
  if (rc) {
    if (rep) std::snprintf(rep->msg, sizeof rep->msg, "%s", err.c_str());
    return rc;
  }
  const int L = c.n_layers, H = c.hidden, nq = c.n_q_heads, nkv = c.n_kv_heads, hd = c.head_dim;
  const int F = c.ffn_dim, V = c.vocab, MB = c.max_batch, S = c.max_seq, G = nq / nkv, half = hd / 2;
  const int ns = P.n_split;
  Model M;
  Bases B;
  // caller tensors (bf16 weights, int32 inputs, the cache and the logits)
  B.embed = M.add("embed", (uint64_t)V * H * 2);
  B.lm_head = c.tied_embeddings ? B.embed : M.add("lm_head", (uint64_t)V * H * 2);
  B.final_norm = M.add("final_norm", (uint64_t)H * 2);
  std::vector<mk_layer_weights> lw(L);
  for (int l = 0; l < L; ++l) {
    auto w = [&](const char *nm, uint64_t bytes) {
      return (const void *)(uintptr_t)M.add(std::string(nm) + "[" + std::to_string(l) + "]", bytes);
    };
    lw[l].attn_norm = w("attn_norm", (uint64_t)H * 2);
    lw[l].wq = w("wq", (uint64_t)nq * hd * H * 2);
    lw[l].wk = w("wk", (uint64_t)nkv * hd * H * 2);
    lw[l].wv = w("wv", (uint64_t)nkv * hd * H * 2);
    lw[l].q_norm = c.qk_norm ? w("q_norm", (uint64_t)hd * 2) : nullptr;
    lw[l].k_norm = c.qk_norm ? w("k_norm", (uint64_t)hd * 2) : nullptr;
    lw[l].wo = w("wo", (uint64_t)H * nq * hd * 2);
    lw[l].ffn_norm = w("ffn_norm", (uint64_t)H * 2);
    lw[l].w_gate = w("w_gate", (uint64_t)F * H * 2);
    lw[l].w_up = w("w_up", (uint64_t)F * H * 2);
    lw[l].w_down = w("w_down", (uint64_t)H * F * 2);
    B.attn_norm.push_back((uint64_t)(uintptr_t)lw[l].attn_norm);
    B.q_norm.push_back((uint64_t)(uintptr_t)lw[l].q_norm);
    B.k_norm.push_back((uint64_t)(uintptr_t)lw[l].k_norm);
    B.ffn_norm.push_back((uint64_t)(uintptr_t)lw[l].ffn_norm);
  }
  mk_weights W;
  W.embed = (const void *)(uintptr_t)B.embed;
  W.lm_head = c.tied_embeddings ? nullptr : (const void *)(uintptr_t)B.lm_head;
  W.final_norm = (const void *)(uintptr_t)B.final_norm;
  W.layers = lw.data();
  resolve_streams(c, W, P);
  if (check_plan(c, P, 0, 0, 0, nullptr) != MK_OK) {
    if (rep) std::snprintf(rep->msg, sizeof rep->msg, "the plan fails its static checks");
    return MK_ERR_UNSUPPORTED;
  }
  // planted record errors: the plan forgets one read of the first FFN unit
  // (its residual input, 7) or of the first attention unit (its tagged q/K/V,
  // 8), which the walk must then report
  if (corrupt == 7 || corrupt == 8)
    for (size_t u = 0; u < P.instr.size(); ++u)
      if (P.instr[u].op == (corrupt == 7 ? OP_FFN : OP_ATTN) && !P.reads[u].empty()) {
        P.reads[u].erase(P.reads[u].begin());
        break;
      }
  B.tokens = M.add("tokens", (uint64_t)batch * 4);
  B.positions = M.add("positions", (uint64_t)batch * 4);
  // planted size errors for the model's self-tests: one record short
  const uint64_t short_kv = corrupt == 1 ? (uint64_t)hd * 2 : 0, short_part = corrupt == 2 ? (hd + 4) * 4 : 0;
  const uint64_t short_rope = corrupt == 3 ? (uint64_t)hd * 4 : 0, short_q = corrupt == 4 ? (uint64_t)hd * 8 : 0;
  const uint64_t short_h = corrupt == 5 ? (uint64_t)H * 4 : 0, short_logits = corrupt == 6 ? (uint64_t)V * 4 : 0;
  B.kv = M.add("kv_cache", lay::kv_size(L, MB, nkv, S, hd) * 2 - short_kv);
  B.logits = M.add("logits", (uint64_t)(one_launch ? steps : 1) * batch * V * 4 - short_logits);
  B.next_tok = M.add("next_tokens", (uint64_t)batch * 4);
  B.next_pos = M.add("next_positions", (uint64_t)batch * 4);
  // library buffers, sized as mk_create and the plan upload size them
  B.h = M.add("h", lay::h_size(L, MB, H) * 4 - short_h);
  B.q = M.add("q", lay::q_size(L, MB, nq, hd) * 8 - short_q);
  B.kvn = M.add("kvn", lay::kvn_size(L, MB, nkv, hd) * 8);
  B.attn = M.add("attn", lay::attn_size(L, MB, nq, hd) * 4);
  B.a = M.add("a", lay::a_size(L, MB, F) * 4);
  B.part = M.add("partials", (lay::part_size(L, MB, nq, ns, hd) +
                              (P.down_splits ? lay::dpart_size(L, P.down_splits, H, MB) : 0)) * 4 - short_part);
  B.rope = M.add("rope", lay::rope_size(S, hd) * 4 - short_rope);
  M.plan = &P;
  M.id_h = B.h >> kShift;
  M.id_q = B.q >> kShift;
  M.id_kvn = B.kvn >> kShift;
  M.id_attn = B.attn >> kShift;
  M.id_a = B.a >> kShift;
  M.id_part = B.part >> kShift;
  M.MB = (uint64_t)MB; M.H = (uint64_t)H; M.nq = (uint64_t)nq; M.hd = (uint64_t)hd; M.F = (uint64_t)F;
  M.nkv = (uint64_t)nkv; M.ns = (uint64_t)ns; M.G = (uint64_t)G; M.half = (uint64_t)half;
  M.ppg = (uint64_t)(G + 2) * half;
  M.part_elems = lay::part_size(L, MB, nq, ns, hd);
  B.status = M.add("status", 256);
  const uint64_t amax_word = (uint64_t)P.n_groups * kSlots * kCtrStride;
  B.ctr = M.add("counters", (amax_word + kCtrStride + (uint64_t)P.n_down_groups) * 4);
  B.target = M.add("targets", P.grp_target.size() * 4);
  uint32_t n_lm = 0, max_pages = 0;
  for (const Instr &in : P.instr) n_lm += in.op == OP_LM;
  for (int cu = 0; cu < num_cus; ++cu) {
    M.unit = -1;
    uint32_t np = 0;
    for (uint32_t qi = P.q_off[cu]; qi < P.q_off[cu + 1]; ++qi) {
      const Instr &in = P.instr[qi];
      np += in.op == OP_ATTN && in.ppp ? (uint32_t)((P.split_len + in.ppp - 1) / in.ppp) : in.pages;
    }
    max_pages = std::max(max_pages, np);
  }
  B.amax = M.add("amax", (uint64_t)n_lm * MB * 8);
  B.zero = M.add("zero", 1024);
  B.rowtab = M.add("rowtab", P.rowtab.size() * 8);
  B.iota = M.add("iota", ((uint64_t)max_pages + 1) * 4);

  for (int step = 0; step < steps; ++step) {
    std::vector<int> pos(batch);
    for (int b = 0; b < batch; ++b) pos[b] = positions[b] + step;
    B.tok_src = one_launch && step > 0 ? B.next_tok : B.tokens;
    B.logit_off = one_launch ? (uint64_t)step * batch * V : 0;
    B.tok_wait = one_launch && step > 0;
    if (B.tok_wait) M.el(B.ctr, amax_word + kTokWord, 4, 4, "sync: token counter wait");
    // the launch clamps an invalid position to 0 for the cache accesses (the
    // sync wave reports it and abandons the step)
    const int pos0 = (pos[0] < 0 || pos[0] >= S) ? 0 : pos[0];
    bool inputs_ok = true;
    for (int b = 0; b < batch; ++b)
      if (tokens[b] < 0 || tokens[b] >= V || pos[b] < 0 || pos[b] >= S) inputs_ok = false;
    M.el(B.positions, 0, 4, 4, "kernel start: positions[0]");

    if (batch > 1) {
      walk_batched(M, B, P, c, batch, num_cus, pos, tokens, inputs_ok);
      continue;
    }
    for (int cu = 0; cu < num_cus; ++cu) {
      M.unit = -1;
      const uint32_t q0 = P.q_off[cu], q1 = P.q_off[cu + 1];
      // ---- sync wave ----------------------------------------------------
      for (int b = 0; b < batch; ++b) {
        M.el(B.tok_src, b, 4, 4, "sync: tokens[b]");
        M.el(B.positions, b, 4, 4, "sync: positions[b]");
      }
      if (inputs_ok)
        for (uint32_t qi = q0; qi < q1; ++qi) {
          const Instr &d = P.instr[qi];
          M.unit = (int)qi;
          const bool gv = d.op == OP_QKV || d.op == OP_O || d.op == OP_FFN || d.op == OP_DOWN || d.op == OP_LM;
          const uint32_t nx = gv ? d.nk : 1;
          const bool normed = d.op == OP_QKV || d.op == OP_FFN || d.op == OP_LM;
          const int b = 0;
          uint64_t hbase = 0, emb = 0, nw = 0;
          if (normed) {
            if (d.op == OP_QKV) {
              nw = B.attn_norm[d.layer];
              if (d.layer == 0) emb = B.embed + (uint64_t)tokens[b] * H * 2;
              else hbase = B.h + lay::h(MB, H, 2 * d.layer, b) * 4;
            } else if (d.op == OP_FFN) {
              nw = B.ffn_norm[d.layer];
              hbase = B.h + lay::h(MB, H, 2 * d.layer + 1, b) * 4;
            } else {
              nw = B.final_norm;
              hbase = B.h + lay::h(MB, H, 2 * L, b) * 4;
            }
            for (uint32_t k = 0; k < nx; ++k)
              for (int lane = 0; lane < 64; ++lane)
                for (uint32_t i = (uint32_t)lane * 4; i < d.kc; i += 256)
                  M.at(nw + ((uint64_t)k * d.kc + i) * 2, 8, nw, "sync: norm weights");
          }
          if (d.op == OP_QKV) {
            const uint32_t ppg = (uint32_t)(G + 2) * half;
            for (uint32_t i = 0; i < d.n_items; ++i) {
              const uint32_t ii = ((d.item0 + i) % ppg) % half;
              M.el(B.rope, lay::rope(hd, pos0, (int)ii), 4, 8, "sync: RoPE of the unit's pairs");
            }
          }
          for (uint32_t w = 0; w < d.wait_n; ++w) {
            const Wait &wt = P.waits[d.wait_off + w];
            for (uint32_t lane = 0; lane < wt.nslot; ++lane) {
              M.el(B.ctr, ((uint64_t)wt.grp * kSlots + lane) * kCtrStride, 4, 4, "sync: counter poll");
              M.el(B.target, (uint64_t)wt.grp * kSlots + lane, 4, 4, "sync: slot target");
            }
            M.el(B.status, 0, 4, 4, "sync: status poll");
          }
          const bool dma = (d.op == OP_DOWN || (d.op == OP_O && d.layer > 0)) && d.n_items <= 64;
          if (dma) {
            const uint64_t src = d.op == OP_O ? B.attn + lay::attn(MB, nq, hd, d.layer, b) * 4
                                              : B.a + lay::a(MB, F, d.layer, b) * 4;
            const uint64_t want = d.op == OP_O ? B.attn : B.a;
            const uint64_t res =
                B.h + (lay::h(MB, H, d.op == OP_O ? 2 * d.layer : 2 * d.layer + 1, b) + d.item0) * 4;
            for (int lane = 0; lane < (int)d.n_items; ++lane) M.at(res + lane * 4, 4, B.h, "sync: residual rows");
            for (uint32_t k = 0; k < nx; ++k)
              for (int j = 0; j < 8; ++j)
                for (int lane = 0; lane < 64; ++lane) {
                  const uint32_t f = (uint32_t)(j * 256 + lane * 4);
                  M.at(src + ((uint64_t)k * d.kc + (f < d.kc ? f : 0u)) * 4, 16, want, "sync: activation piece (DMA)");
                }
          } else {
            for (uint32_t k = 0; k < nx; ++k) {
              if (normed) {
                auto batch_ld = [&](uint32_t e0) {
                  for (int lane = 0; lane < 64; ++lane)
                    for (int m = 0; m < 8; ++m) {
                      const uint32_t i = e0 + (uint32_t)(lane + 64 * m) * 4;
                      if (i >= (uint32_t)H) continue;
                      if (emb) M.at(emb + (uint64_t)i * 2, 8, B.embed, "sync: embedding row");
                      else M.at(hbase + (uint64_t)i * 4, 16, B.h, "sync: residual for the norm");
                    }
                };
                if (k == 0)
                  for (uint32_t e0 = 0; e0 < (uint32_t)H; e0 += 2048) batch_ld(e0);
                if (H > 2048 || k != 0) batch_ld(k * d.kc);
              } else if (d.op == OP_O || d.op == OP_DOWN) {
                const uint64_t src = d.op == OP_O ? B.attn + lay::attn(MB, nq, hd, d.layer, b) * 4
                                                  : B.a + lay::a(MB, F, d.layer, b) * 4;
                const uint64_t want = d.op == OP_O ? B.attn : B.a;
                for (int lane = 0; lane < 64; ++lane)
                  for (int m = 0; m < 8; ++m) {
                    const uint32_t i = (uint32_t)(lane + 64 * m) * 4;
                    if (i < d.kc) M.at(src + ((uint64_t)k * d.kc + i) * 4, 16, want, "sync: activation piece");
                  }
                if (k == 0)
                  for (int lane = 0; lane < 64; ++lane)
                    for (int m = 0; m < kAccFloats / 64; ++m) {
                      const uint32_t r = (uint32_t)(lane + 64 * m);
                      if (r >= d.n_items) continue;
                      if (d.op == OP_O && d.layer == 0)
                        M.at(B.embed + ((uint64_t)tokens[b] * H + d.item0 + r) * 2, 2, B.embed, "sync: embedding residual");
                      else
                        M.el(B.h, lay::h(MB, H, d.op == OP_O ? 2 * d.layer : 2 * d.layer + 1, b) + d.item0 + r, 4, 4,
                             "sync: residual rows");
                    }
              }
            }
          }
        }

      // ---- loader waves ---------------------------------------------------
      uint32_t n = 0;
      for (uint32_t qi = q0; qi < q1; ++qi) {
        const Instr &d = P.instr[qi];
        M.unit = (int)qi;
        if (d.op == OP_ATTN && d.ppp) {
          paged_kv_loads(M, B, P, c, d, pos0, n);
          continue;
        }
        const bool gv = d.op == OP_QKV || d.op == OP_O || d.op == OP_FFN || d.op == OP_DOWN || d.op == OP_LM;
        if (!gv) continue;
        const uint32_t per = d.n_items * d.ipw, npieces = per * d.nk;
        auto piece = [&](uint32_t k, uint32_t r) -> uint64_t {
          uint64_t base;
          if (d.tab >= 0) {
            M.el(B.rowtab, (uint64_t)d.tab + r, 8, 8, "loader: row table");
            base = (size_t)d.tab + r < P.rowtab.size() ? P.rowtab[d.tab + r] : 0;
          } else if (d.ipw == 2) {
            base = ((r & 1) ? d.w1 : d.w0) + (uint64_t)(d.item0 + (r >> 1)) * d.rowb;
          } else {
            base = d.w0 + (uint64_t)(d.item0 + r) * d.rowb;
          }
          return base + (uint64_t)k * d.pb;
        };
        for (uint32_t p = 0; p < d.pages; ++p, ++n) {
          const uint32_t t0 = p * d.ppp;
          const uint32_t cnt = std::min((uint32_t)d.ppp, npieces - t0);
          uint32_t k = t0 / per, r = t0 - k * per;
          const uint64_t first = piece(k, r);
          if (d.pb >= 1024) {
            const uint32_t lpp = d.pb >> 10;
            uint32_t j = 0;
            for (uint32_t qq = 0; qq < cnt; ++qq) {
              const uint64_t src = piece(k, r);
              const uint64_t row0 = src - (uint64_t)k * d.pb;  // the row's start: the piece must stay in its row
              for (uint32_t sub = 0; sub < lpp; ++sub)
                for (int lane = 0; lane < 64; ++lane) {
                  const uint64_t ad = src + sub * 1024 + lane * 16;
                  M.at(ad, 16, 0, "loader: weight piece");
                  if (ad + 16 > row0 + d.rowb) M.at(~0ull, 16, 0, "loader: weight piece crosses its row");
                }
              j += lpp;
              if (++r == per) { r = 0; ++k; }
            }
            for (; j < 16; ++j)
              for (int lane = 0; lane < 64; ++lane) M.at(first + lane * 16, 16, 0, "loader: tail re-read");
          } else {
            const uint32_t sh = 31 - __builtin_clz(d.pb);
            for (int j = 0; j < 16; ++j)
              for (int lane = 0; lane < 64; ++lane) {
                const uint32_t o = (uint32_t)j * 1024 + lane * 16;
                const uint32_t qq = o >> sh, within = o & (d.pb - 1);
                const uint32_t t = t0 + qq;
                uint64_t src = first;
                if (t < npieces) {
                  const uint32_t kk = t / per;
                  src = piece(kk, t - kk * per) + within;
                }
                M.at(src, 16, 0, "loader: weight piece (small)");
              }
          }
          M.el(B.iota, n, 4, 4, "loader: page sentinel");
        }
      }

      // ---- compute waves ----------------------------------------------------
      if (!inputs_ok) continue;
      for (uint32_t qi = q0; qi < q1; ++qi) {
        const Instr &d = P.instr[qi];
        M.unit = (int)qi;
        const int b = (int)d.b;
        if (d.op == OP_ATTN && d.ppp) {
          paged_attn_compute(M, B, P, c, d, pos0);
        } else if (d.op == OP_ATTN) {
          const int g = (int)d.aux0, s = (int)d.aux1;
          const int DPL = hd / 64, PF = 20 / DPL, NR = DPL == 1 ? 16 : 8;
          const int p = pos0;
          const int lo = s * P.split_len, hi = std::min(lo + P.split_len, p + 1);
          const int nt0 = std::max(0, std::min(hi - lo, PF));
          const uint64_t Kr = lay::kv(MB, nkv, S, hd, d.layer, 0, b, g, lo);
          const uint64_t Vr = lay::kv(MB, nkv, S, hd, d.layer, 1, b, g, lo);
          for (int h = 0; h < G; ++h) {
            const int j = g * G + h;
            for (int lane = 0; lane < 64; ++lane) {
              if (nt0 > 0)
                for (int t = 0; t < PF; ++t) {
                  const int tt = std::min(t, nt0 - 1);
                  for (int m = 0; m < DPL; ++m) {
                    M.el(B.kv, Kr + (uint64_t)tt * hd + lane + 64 * m, 2, 2, "attn: prefetched K");
                    M.el(B.kv, Vr + (uint64_t)tt * hd + lane + 64 * m, 2, 2, "attn: prefetched V");
                  }
                }
              if (DPL == 2 && c.qk_norm) {
                for (int m = 0; m < DPL; ++m) {
                  M.el(B.q_norm[d.layer], lane + 64 * m, 2, 2, "attn: q_norm weight");
                  M.el(B.k_norm[d.layer], lane + 64 * m, 2, 2, "attn: k_norm weight");
                }
                M.el(B.rope, lay::rope(hd, p, lane), 4, 8, "attn: RoPE of pair (lane, lane + 64)");
              }
              if (lo < hi) {
                const bool has_p = p < hi;
                for (int m = 0; m < DPL; ++m) {
                  M.el(B.q, lay::q(MB, nq, hd, d.layer, b, j) + lane + 64 * m, 8, 8, "attn: tagged q");
                  if (has_p) {
                    M.el(B.kvn, lay::kvn(MB, nkv, hd, d.layer, b, g, 0) + lane + 64 * m, 8, 8, "attn: tagged new K");
                    M.el(B.kvn, lay::kvn(MB, nkv, hd, d.layer, b, g, 0) + hd + lane + 64 * m, 8, 8,
                         "attn: tagged new V");
                  }
                }
                if (DPL == 2 && c.qk_norm && has_p && h == 0) {
                  M.el(B.kv, lay::kv(MB, nkv, S, hd, d.layer, 0, b, g, p) + lane, 2, 2, "attn: K store at p");
                  M.el(B.kv, lay::kv(MB, nkv, S, hd, d.layer, 0, b, g, p) + lane + 64, 2, 2, "attn: K store at p");
                }
                for (int c0 = lo + PF; c0 < hi; c0 += 64) {
                  const int nt = std::min(64, hi - c0);
                  for (int kvt = 0; kvt < 2; ++kvt)
                    for (int t0 = 0; t0 < nt; t0 += NR)
                      for (int t = 0; t < NR; ++t) {
                        const int tt = std::min(t0 + t, nt - 1);
                        if (c0 + tt == p) continue;
                        for (int m = 0; m < DPL; ++m)
                          M.el(B.kv, (kvt ? Vr : Kr) + (uint64_t)(c0 - lo + tt) * hd + lane + 64 * m, 2, 2,
                               "attn: K/V row of the long split");
                      }
                }
              }
              const uint64_t out = lay::part(MB, nq, ns, hd, d.layer, b, j, s);
              for (int m = 0; m < DPL; ++m) M.el(B.part, out + lane + 64 * m, 4, 4, "attn: partial o");
              if (lane == 0) {
                M.el(B.part, out + hd, 4, 4, "attn: partial m");
                M.el(B.part, out + hd + 1, 4, 4, "attn: partial l");
              }
            }
          }
          M.el(B.ctr, ((uint64_t)d.sig0 * kSlots + d.slot0) * kCtrStride, 4, 4, "attn: counter signal");
        } else if (d.op == OP_RED) {
          const int g = (int)d.aux0, DPL = hd / 64, RB = 32 / DPL;
          const uint32_t rowb = (uint32_t)(hd + 4) * 4;
          for (int h = 0; h < G; ++h) {
            const int j = g * G + h;
            const uint64_t base = B.part + lay::part(MB, nq, ns, hd, d.layer, b, j, 0) * 4;
            for (int lane = 0; lane < 64; ++lane) {
              if (lane < ns) {
                M.at(base + (uint64_t)lane * rowb + hd * 4, 4, B.part, "red: m of a split");
                M.at(base + (uint64_t)lane * rowb + hd * 4 + 4, 4, B.part, "red: l of a split");
              }
              for (int s0 = 0; s0 < ns; s0 += RB)
                for (int t = 0; t < RB; ++t) {
                  const int ss = std::min(s0 + t, ns - 1);
                  for (int m = 0; m < DPL; ++m)
                    M.at(base + (uint64_t)ss * rowb + (uint64_t)(lane + 64 * m) * 4, 4, B.part, "red: o of a split");
                }
              for (int m = 0; m < DPL; ++m)
                M.el(B.attn, lay::attn(MB, nq, hd, d.layer, b) + (uint64_t)j * hd + lane + 64 * m, 4, 4,
                     "red: attention output");
            }
          }
          M.el(B.ctr, ((uint64_t)d.sig0 * kSlots + d.slot0) * kCtrStride, 4, 4, "red: counter signal");
        } else {
          // GEMV epilogue (the last compute wave), lanes stride the items
          const int p = pos0;
          for (uint32_t i = 0; i < d.n_items; ++i) {
            switch (d.op) {
              case OP_QKV: {
                const uint32_t ppg = (uint32_t)(G + 2) * half, pp = d.item0 + i, g = pp / ppg, rr = pp - g * ppg;
                const uint32_t hs = rr / half, ii = rr - hs * half;
                if (hs <= (uint32_t)G && c.qk_norm) {
                  const uint64_t dst = hs < (uint32_t)G ? lay::q(MB, nq, hd, d.layer, b, (int)(g * G + hs))
                                                        : lay::kvn(MB, nkv, hd, d.layer, b, (int)g, 0);
                  const uint64_t buf = hs < (uint32_t)G ? B.q : B.kvn;
                  M.el(buf, dst + ii, 8, 8, "epilogue: raw q/k word");
                  M.el(buf, dst + ii + half, 8, 8, "epilogue: raw q/k word");
                } else if (hs < (uint32_t)G) {
                  const uint64_t qo = lay::q(MB, nq, hd, d.layer, b, (int)(g * G + hs));
                  M.el(B.q, qo + ii, 8, 8, "epilogue: q word");
                  M.el(B.q, qo + ii + half, 8, 8, "epilogue: q word");
                } else {
                  const int t = hs == (uint32_t)G ? 0 : 1;
                  const uint64_t ko = lay::kv(MB, nkv, S, hd, d.layer, t, b, (int)g, p);
                  M.el(B.kv, ko + ii, 2, 2, "epilogue: K/V slot p");
                  M.el(B.kv, ko + ii + half, 2, 2, "epilogue: K/V slot p");
                  const uint64_t no = lay::kvn(MB, nkv, hd, d.layer, b, (int)g, t);
                  M.el(B.kvn, no + ii, 8, 8, "epilogue: tagged K/V word");
                  M.el(B.kvn, no + ii + half, 8, 8, "epilogue: tagged K/V word");
                }
                break;
              }
              case OP_O: M.el(B.h, lay::h(MB, H, 2 * d.layer + 1, b) + d.item0 + i, 4, 4, "epilogue: O rows"); break;
              case OP_FFN: M.el(B.a, lay::a(MB, F, d.layer, b) + d.item0 + i, 4, 4, "epilogue: FFN rows"); break;
              case OP_DOWN:
                M.el(B.h, lay::h(MB, H, 2 * d.layer + 2, b) + d.item0 + i, 4, 4, "epilogue: down rows");
                break;
              default: M.el(B.logits, B.logit_off + lay::logits(V, b) + d.item0 + i, 4, 4, "epilogue: logits"); break;
            }
          }
          if (d.op == OP_LM) {
            M.el(B.amax, d.unit, 8, 8, "epilogue: greedy candidate");
            M.el(B.ctr, amax_word, 4, 4, "greedy: arrival counter");
            M.el(B.ctr, amax_word + kTokWord, 4, 4, "greedy: token counter");
            for (uint32_t u = 0; u < n_lm; ++u) M.el(B.amax, u, 8, 8, "greedy: candidates");
            M.el(B.next_tok, 0, 4, 4, "greedy: next token");
            M.el(B.next_pos, 0, 4, 4, "greedy: next position");
          }
          for (int sg : {d.sig0, d.sig1})
            if (sg >= 0) {
              const uint32_t slot = sg == d.sig0 ? d.slot0 : d.slot1;
              M.el(B.ctr, ((uint64_t)sg * kSlots + slot) * kCtrStride, 4, 4, "epilogue: counter signal");
            }
        }
      }
      // error path: status words
      M.el(B.status, 0, 4, 12, "raise_error: status words");
    }
  }
  if (rep) {
    rep->accesses = M.n;
    rep->violations = M.bad;
    std::snprintf(rep->msg, sizeof rep->msg, "%s", M.first.c_str());
  }
  return M.bad ? MK_ERR_INVALID_ARG : MK_OK;
}

extern "C" int mk_addr_check(const mk_config *cfg, int32_t batch, int32_t num_cus, int32_t steps,
                             const int32_t *positions, const int32_t *tokens, int32_t corrupt,
                             mk_addr_report *rep) {
  return addr_check(cfg, batch, num_cus, steps, false, positions, tokens, corrupt, rep);
}

extern "C" int mk_addr_check_launch(const mk_config *cfg, int32_t batch, int32_t num_cus, int32_t steps,
                                    const int32_t *positions, const int32_t *tokens, int32_t corrupt,
                                    mk_addr_report *rep) {
  return addr_check(cfg, batch, num_cus, steps, true, positions, tokens, corrupt, rep);
}
