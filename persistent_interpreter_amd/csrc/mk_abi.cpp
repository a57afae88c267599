// mk_abi.cpp -- the C ABI of include/mk.h: configuration checks, device
// buffers, per-batch plans and the single launch per decode step.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_layout.hpp"
#include "mk_plan.hpp"
#include "mk_sched.hpp"

namespace mk {
hipError_t kernel_setup(int *blocks_per_cu);
hipError_t kernel_launch(const Args &a, int grid, bool cooperative, bool paged, hipStream_t stream);
hipError_t static_scratch(int device, void **ptr);
hipError_t fill_zero(void *p, size_t words, hipStream_t stream);
}  // namespace mk

using namespace mk;

namespace {

struct DevPlan {
  Plan plan;
  Instr *d_instr = nullptr;
  uint32_t *d_qoff = nullptr;
  Wait *d_waits = nullptr;
  uint64_t *d_rowtab = nullptr;
  uint32_t *d_ctr = nullptr;
  uint32_t *d_target = nullptr;
  float *d_part = nullptr;
  uint32_t *d_iota = nullptr;
  uint64_t *d_trace = nullptr;
  uint64_t *d_amax = nullptr;  // greedy candidates, one per LM unit
  size_t ctr_bytes = 0, trace_bytes = 0;
  size_t amax_word = 0;        // index in d_ctr of the greedy arrival counter
  uint32_t trace_stride = 0;
  uint32_t epoch = 0;
  uint32_t n_lm = 0;
  uint32_t n_arrive = 0;       // greedy candidates (and arrivals) per step
  uint32_t greedy_epoch = 0;   // greedy steps since the counters were zeroed
};

template <class T>
int dev_alloc(T **p, size_t bytes) {
  if (bytes == 0) bytes = 16;
  if (hipMalloc((void **)p, bytes) != hipSuccess) {
    *p = nullptr;
    return MK_ERR_OOM;
  }
  return MK_OK;
}

template <class T>
int upload(T **p, const std::vector<T> &v) {
  int rc = dev_alloc(p, v.size() * sizeof(T));
  if (rc) return rc;
  if (!v.empty() && hipMemcpy(*p, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess)
    return MK_ERR_HIP;
  return MK_OK;
}

void free_plan(DevPlan &p) {
  hipFree(p.d_instr);
  hipFree(p.d_qoff);
  hipFree(p.d_waits);
  hipFree(p.d_rowtab);
  hipFree(p.d_ctr);
  hipFree(p.d_target);
  hipFree(p.d_part);
  hipFree(p.d_iota);
  hipFree(p.d_trace);
  hipFree(p.d_amax);
}

constexpr int kMaxLayers = 4096;
constexpr int kMaxDim = 1 << 20;

int check_config(const mk_config *c, std::string &err) {
  if (!c) { err = "null config"; return MK_ERR_INVALID_ARG; }
  if (c->n_layers < 1 || c->hidden < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 1 ||
      c->ffn_dim < 1 || c->vocab < 1 || c->max_batch < 1 || c->max_seq < 1) {
    err = "every size must be >= 1";
    return MK_ERR_INVALID_ARG;
  }
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f)) { err = "bad rms_eps or rope_theta"; return MK_ERR_INVALID_ARG; }
  if (c->n_q_heads % c->n_kv_heads) { err = "n_q_heads must be a multiple of n_kv_heads"; return MK_ERR_UNSUPPORTED; }
  if (c->head_dim != 64 && c->head_dim != 128) { err = "head_dim must be 64 or 128"; return MK_ERR_UNSUPPORTED; }
  if (kNCW % (c->n_q_heads / c->n_kv_heads)) {
    err = "query heads per KV head must divide 8 (1, 2, 4 or 8)";
    return MK_ERR_UNSUPPORTED;
  }
  if (c->qk_norm && c->head_dim != 128) { err = "q/k norm needs head_dim 128"; return MK_ERR_UNSUPPORTED; }
  if (c->hidden % 8 || c->ffn_dim % 8) { err = "hidden and ffn_dim must be multiples of 8"; return MK_ERR_UNSUPPORTED; }
  if (c->kv_splits > kMaxSplits || c->kv_splits < 0) { err = "kv_splits must be in [0, 64]"; return MK_ERR_UNSUPPORTED; }
  // a descriptor keeps the layer index (the LM head's units take n_layers)
  // and the K pieces of a row (256-element MFMA pieces) in 16 bits
  if (c->n_layers > kMaxLayers || c->hidden > kMaxDim || c->ffn_dim > kMaxDim ||
      (int64_t)c->n_q_heads * c->head_dim > kMaxDim) {
    err = "n_layers above 4096, or hidden, ffn_dim or n_q_heads*head_dim above 2^20";
    return MK_ERR_UNSUPPORTED;
  }
  if (c->mlp_chunks < 0 || c->num_cus < 0 || c->watchdog_ms < 0) { err = "negative knob"; return MK_ERR_INVALID_ARG; }
  if ((int64_t)c->vocab * c->hidden >= (1ll << 40)) { err = "model too large"; return MK_ERR_UNSUPPORTED; }
  return MK_OK;
}

}  // namespace

struct mk_handle {
  mk_config cfg;
  int device = 0;
  int num_cus = 0;
  std::vector<mk_layer_weights> layers;
  mk_weights w;
  DevCtx hctx;
  DevCtx *d_ctx = nullptr;
  DevLayer *d_layers = nullptr;
  float *h_buf = nullptr, *attn_buf = nullptr, *a_buf = nullptr;
  uint64_t *q_buf = nullptr, *kvn_buf = nullptr;  // tagged words, see DevCtx
  float *rope = nullptr;
  uint16_t *zero = nullptr;  // zeros read for weights past K in padded MFMA pieces
  uint32_t *status = nullptr;
  size_t h_bytes = 0, q_bytes = 0, attn_bytes = 0, a_bytes = 0, kvn_bytes = 0;
  std::map<int, std::unique_ptr<DevPlan>> plans;
  DevPlan *last_plan = nullptr;
  void *static_scratch = nullptr;  // this device's array for mk_decode_step_static
  uint32_t tag = 0;  // activation tag of the last step (never 0; never reset)
  bool error_pending = false;
};

extern "C" {

int mk_version(void) { return 109; }

const char *mk_strerror(int code) {
  switch (code) {
    case MK_OK: return "ok";
    case MK_ERR_INVALID_ARG: return "invalid argument";
    case MK_ERR_UNSUPPORTED: return "unsupported shape or configuration";
    case MK_ERR_OOM: return "device allocation failed";
    case MK_ERR_HIP: return "HIP runtime call failed";
    case MK_ERR_NOT_CORESIDENT: return "the persistent grid cannot be co-resident";
    case MK_ERR_NO_DEVICE: return "no usable GPU";
    case MK_ERR_NOT_PREPARED: return "the batch size's schedule is not built yet (run one ordinary step first)";
    case MK_ERR_DEVICE_TIMEOUT: return "a counter wait exceeded the watchdog";
    case MK_ERR_BAD_TOKEN: return "token id outside [0, vocab)";
    case MK_ERR_BAD_POSITION: return "position outside [0, max_seq)";
    default: return "unknown status code";
  }
}

int mk_plan_units(const mk_config *cfg, int32_t batch, int32_t num_cus, mk_unit_info *units, int32_t cap,
                  int32_t *q_off) {
  std::string err;
  int rc = check_config(cfg, err);
  if (rc != MK_OK) return rc;
  if (batch < 1 || batch > cfg->max_batch || num_cus < 1 || cap < 0 || (cap > 0 && !units))
    return MK_ERR_INVALID_ARG;
  Plan plan;
  rc = build_plan(*cfg, batch, num_cus, plan, err);
  if (rc != MK_OK) return rc;
  const int32_t n = (int32_t)plan.instr.size();
  if (q_off)
    for (int c = 0; c <= num_cus; ++c) q_off[c] = (int32_t)plan.q_off[c];
  for (int32_t i = 0; i < n && i < cap; ++i) {
    const Instr &in = plan.instr[i];
    mk_unit_info &u = units[i];
    u.op = in.op;
    u.layer = in.layer;
    u.nk = in.nk;
    u.pages = (int32_t)in.pages;
    u.ppp = in.ppp;
    u.n_items = (int32_t)in.n_items;
    u.ipw = in.ipw;
    u.wait_n = (int32_t)in.wait_n;
    const bool kv_unit = in.op == OP_ATTN || in.op == OP_RED;
    u.b = kv_unit ? (int32_t)in.b : 0;
    u.aux0 = kv_unit ? (int32_t)in.aux0 : 0;
    u.aux1 = in.op == OP_ATTN ? (int32_t)in.aux1 : 0;
    u.split_len = plan.split_len;
  }
  return n;
}

int mk_plan_check(const mk_config *cfg, int32_t batch, int32_t num_cus, int32_t sim_runs, int32_t corrupt,
                  uint64_t seed, mk_plan_report *rep) {
  std::string err;
  if (rep) std::memset(rep, 0, sizeof *rep);
  int rc = check_config(cfg, err);
  if (rc == MK_OK && (batch < 1 || batch > cfg->max_batch || num_cus < 1 || sim_runs < 0)) {
    err = "batch, num_cus or sim_runs out of range";
    rc = MK_ERR_INVALID_ARG;
  }
  Plan plan;
  if (rc == MK_OK) rc = build_plan(*cfg, batch, num_cus, plan, err);
  if (rc != MK_OK) {
    if (rep) std::snprintf(rep->msg, sizeof rep->msg, "%s", err.c_str());
    return rc;
  }
  if (rep) {
    rep->num_cus = num_cus;
    rep->batch = batch;
    rep->kv_splits = plan.n_split;
    rep->mlp_chunks = plan.mlp_chunks;
    rep->n_instr = (int32_t)plan.instr.size();
    rep->n_groups = plan.n_groups;
    rep->n_pages = plan.n_pages;
    int mq = 0;
    for (int c = 0; c < num_cus; ++c) mq = std::max(mq, (int)(plan.q_off[c + 1] - plan.q_off[c]));
    rep->max_queue = mq;
    rep->weight_bytes = plan.weight_bytes;
    rep->max_cu_bytes = plan.max_cu_bytes;
    rep->paged_kv = plan.paged_kv ? 1 : 0;
    rep->down_splits = plan.down_splits;
    rep->mfma_cols_k = 0;
    if (batch > 1)
      for (const Instr &in : plan.instr)
        if (in.pages) rep->mfma_cols_k += (int64_t)((in.ppp + 1) / 2) * 16 * in.nk * kMfmaKc;
  }
  return check_plan(*cfg, plan, sim_runs, corrupt, seed, rep);
}

int mk_create(const mk_config *cfg, const mk_weights *w, mk_handle **out) {
  if (!out) return MK_ERR_INVALID_ARG;
  *out = nullptr;
  std::string err;
  int rc = check_config(cfg, err);
  if (rc) return rc;
  if (!w || !w->embed || !w->final_norm || !w->layers) return MK_ERR_INVALID_ARG;
  if (!cfg->tied_embeddings && !w->lm_head) return MK_ERR_INVALID_ARG;
  for (int l = 0; l < cfg->n_layers; ++l) {
    const mk_layer_weights &ly = w->layers[l];
    if (!ly.attn_norm || !ly.wq || !ly.wk || !ly.wv || !ly.wo || !ly.ffn_norm || !ly.w_gate || !ly.w_up ||
        !ly.w_down)
      return MK_ERR_INVALID_ARG;
    if (cfg->qk_norm && (!ly.q_norm || !ly.k_norm)) return MK_ERR_INVALID_ARG;
  }

  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return MK_ERR_NO_DEVICE;
  auto h = std::make_unique<mk_handle>();
  h->cfg = *cfg;
  if (hipGetDevice(&h->device) != hipSuccess) return MK_ERR_HIP;
  int cus = 0, coop = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->device) != hipSuccess ||
      hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, h->device) != hipSuccess)
    return MK_ERR_HIP;
  if (!coop) return MK_ERR_NOT_CORESIDENT;
  h->num_cus = cfg->num_cus > 0 ? std::min(cfg->num_cus, cus) : cus;
  int per_cu = 0;
  if (kernel_setup(&per_cu) != hipSuccess) return MK_ERR_HIP;
  if (per_cu < 1) return MK_ERR_NOT_CORESIDENT;
  // the device address of this GPU's static scratch (resolved once per
  // device, with the device current)
  if (static_scratch(h->device, &h->static_scratch) != hipSuccess) return MK_ERR_HIP;

  h->layers.assign(w->layers, w->layers + cfg->n_layers);
  h->w = *w;
  h->w.layers = h->layers.data();

  const int L = cfg->n_layers, MB = cfg->max_batch, H = cfg->hidden, nq = cfg->n_q_heads;
  const int hd = cfg->head_dim, F = cfg->ffn_dim, S = cfg->max_seq;
  h->h_bytes = lay::h_size(L, MB, H) * 4;
  h->q_bytes = lay::q_size(L, MB, nq, hd) * 8;
  h->attn_bytes = lay::attn_size(L, MB, nq, hd) * 4;
  h->a_bytes = lay::a_size(L, MB, F) * 4;
  h->kvn_bytes = lay::kvn_size(L, MB, cfg->n_kv_heads, hd) * 8;
  std::vector<float> rope(lay::rope_size(S, hd));
  for (int p = 0; p < S; ++p)
    for (int i = 0; i < hd / 2; ++i) {
      // angle p * theta^(-2i/hd) in double, cos/sin rounded to float
      double ang = (double)p * std::pow((double)cfg->rope_theta, -2.0 * i / (double)hd);
      rope[lay::rope(hd, p, i)] = (float)std::cos(ang);
      rope[lay::rope(hd, p, i) + 1] = (float)std::sin(ang);
    }
  std::vector<DevLayer> dl(L);
  for (int l = 0; l < L; ++l) {
    const mk_layer_weights &s = w->layers[l];
    dl[l] = DevLayer{(const uint16_t *)s.attn_norm, (const uint16_t *)s.wq, (const uint16_t *)s.wk,
                     (const uint16_t *)s.wv, (const uint16_t *)s.q_norm, (const uint16_t *)s.k_norm,
                     (const uint16_t *)s.wo, (const uint16_t *)s.ffn_norm, (const uint16_t *)s.w_gate,
                     (const uint16_t *)s.w_up, (const uint16_t *)s.w_down};
  }
  if ((rc = dev_alloc(&h->h_buf, h->h_bytes)) || (rc = dev_alloc(&h->q_buf, h->q_bytes)) ||
      (rc = dev_alloc(&h->attn_buf, h->attn_bytes)) || (rc = dev_alloc(&h->a_buf, h->a_bytes)) ||
      (rc = dev_alloc(&h->kvn_buf, h->kvn_bytes)) || (rc = upload(&h->rope, rope)) ||
      (rc = dev_alloc(&h->zero, 1024)) ||
      (rc = dev_alloc(&h->status, 256)) || (rc = upload(&h->d_layers, dl))) {
    mk_destroy(h.release());
    return rc;
  }
  // tag 0 never matches a step's tag (tags start at 1)
  if (hipMemset(h->status, 0, 256) != hipSuccess || hipMemset(h->zero, 0, 1024) != hipSuccess ||
      hipMemset(h->h_buf, 0, h->h_bytes) != hipSuccess ||
      hipMemset(h->q_buf, 0, h->q_bytes) != hipSuccess || hipMemset(h->attn_buf, 0, h->attn_bytes) != hipSuccess ||
      hipMemset(h->a_buf, 0, h->a_bytes) != hipSuccess || hipMemset(h->kvn_buf, 0, h->kvn_bytes) != hipSuccess) {
    mk_destroy(h.release());
    return MK_ERR_HIP;
  }
  DevCtx &c = h->hctx;
  std::memset(&c, 0, sizeof c);
  c.L = L; c.H = H; c.nq = nq; c.nkv = cfg->n_kv_heads; c.hd = hd; c.F = F; c.V = cfg->vocab;
  c.G = nq / cfg->n_kv_heads; c.qk_norm = cfg->qk_norm; c.tied = cfg->tied_embeddings;
  c.max_batch = MB; c.max_seq = S; c.num_cus = h->num_cus;
  c.eps = cfg->rms_eps;
  c.attn_scale = (float)(1.0 / std::sqrt((double)hd));
  c.watchdog_ticks = (int64_t)(cfg->watchdog_ms > 0 ? cfg->watchdog_ms : 2000) * 100000;
  c.embed = (const uint16_t *)w->embed;
  c.final_norm = (const uint16_t *)w->final_norm;
  c.lm_head = (const uint16_t *)w->lm_head;
  c.layers = h->d_layers;
  c.h_buf = h->h_buf; c.q_buf = h->q_buf; c.attn_buf = h->attn_buf; c.a_buf = h->a_buf;
  c.kvn_buf = h->kvn_buf;
  c.rope = h->rope;
  c.zero = h->zero;
  c.status = h->status;
  c.trace = nullptr;
  c.ring_pages = kRingPages;
  c.flags = (int32_t)cfg->flags;
  std::vector<DevCtx> one(1, c);
  if ((rc = upload(&h->d_ctx, one))) {
    mk_destroy(h.release());
    return rc;
  }
  *out = h.release();
  return MK_OK;
}

// Attention partials, then the split-K down partials (batched plans).
static size_t part_bytes(const mk_config &c, const Plan &P) {
  return (lay::part_size(c.n_layers, c.max_batch, c.n_q_heads, P.n_split, c.head_dim) +
          (P.down_splits ? lay::dpart_size(c.n_layers, P.down_splits, c.hidden, c.max_batch) : 0)) *
         4;
}

static int get_plan(mk_handle *h, int batch, DevPlan **out) {
  auto it = h->plans.find(batch);
  if (it != h->plans.end()) {
    *out = it->second.get();
    return MK_OK;
  }
  // the batched (MFMA) kernel has no per-head q/k norm
  if (batch > 1 && h->cfg.qk_norm) return MK_ERR_UNSUPPORTED;
  auto dp = std::make_unique<DevPlan>();
  std::string err;
  int rc = build_plan(h->cfg, batch, h->num_cus, dp->plan, err);
  if (rc) return rc;
  resolve_streams(h->cfg, h->w, dp->plan);
  Plan &P = dp->plan;
  // no plan reaches the device without the validator's static checks
  // (coverage of every read by waits, counter targets, extents)
  if (check_plan(h->cfg, P, 0, 0, 0, nullptr) != MK_OK) return MK_ERR_UNSUPPORTED;
  // the counter groups, then one padded word: the greedy arrival counter,
  // then the arrival counters of the split-K down groups
  dp->amax_word = (size_t)P.n_groups * kSlots * kCtrStride;
  dp->ctr_bytes = (dp->amax_word + kCtrStride + (size_t)P.n_down_groups) * 4;
  for (const Instr &in : P.instr) dp->n_lm += in.op == OP_LM ? 1u : 0u;
  // greedy arrivals per step: one per LM unit (batch 1), one per workgroup
  // holding LM units (batched)
  dp->n_arrive = batch > 1 ? (uint32_t)P.n_lm_groups : dp->n_lm;
  const size_t part = part_bytes(h->cfg, P);
  // page sentinels: iota[i] = i for every page index of the longest queue
  uint32_t max_pages = 0;
  for (int c = 0; c < h->num_cus; ++c) {
    uint32_t np = 0;
    for (uint32_t q = P.q_off[c]; q < P.q_off[c + 1]; ++q) {
      const Instr &in = P.instr[q];
      // a paged attention unit streams at most a whole split
      np += in.op == OP_ATTN && in.ppp ? (uint32_t)((P.split_len + in.ppp - 1) / in.ppp) : in.pages;
    }
    max_pages = std::max(max_pages, np);
  }
  std::vector<uint32_t> iota(max_pages + 1);
  for (uint32_t i = 0; i <= max_pages; ++i) iota[i] = i;
  if ((rc = upload(&dp->d_instr, P.instr)) || (rc = upload(&dp->d_qoff, P.q_off)) ||
      (rc = upload(&dp->d_iota, iota)) ||
      (rc = upload(&dp->d_waits, P.waits)) || (rc = upload(&dp->d_rowtab, P.rowtab)) ||
      (rc = upload(&dp->d_target, P.grp_target)) || (rc = dev_alloc(&dp->d_ctr, dp->ctr_bytes)) ||
      (rc = dev_alloc(&dp->d_part, part)) ||
      (rc = dev_alloc(&dp->d_amax, (size_t)dp->n_lm * h->cfg.max_batch * 8))) {
    free_plan(*dp);
    return rc;
  }
  if (h->cfg.flags & MK_FLAG_TEST_STALL) {
    // test instrument: the last counter group (every LM unit waits on it)
    // gets one arrival more than its producers give, so that wait cannot
    // complete and the step must end in the watchdog
    std::vector<uint32_t> t = P.grp_target;
    t[(size_t)(P.n_groups - 1) * kSlots] += 1;
    if (hipMemcpy(dp->d_target, t.data(), t.size() * 4, hipMemcpyHostToDevice) != hipSuccess) {
      free_plan(*dp);
      return MK_ERR_HIP;
    }
  }
  if (hipMemset(dp->d_ctr, 0, dp->ctr_bytes) != hipSuccess || hipMemset(dp->d_part, 0, part) != hipSuccess) {
    free_plan(*dp);
    return MK_ERR_HIP;
  }
  if (h->cfg.flags & MK_FLAG_TRACE) {
    // header [num_cus, stride, words per record, 0] then
    // [num_cus][stride][8] records
    uint32_t mq = 0;
    for (int c = 0; c < h->num_cus; ++c) mq = std::max(mq, P.q_off[c + 1] - P.q_off[c]);
    dp->trace_stride = mq;
    dp->trace_bytes = (4 + (size_t)h->num_cus * mq * 8) * 8;
    std::vector<uint64_t> init(dp->trace_bytes / 8, 0);
    init[0] = (uint64_t)h->num_cus;
    init[1] = mq;
    init[2] = 8;
    if ((rc = upload(&dp->d_trace, init))) {
      free_plan(*dp);
      return rc;
    }
  }
  *out = dp.get();
  h->plans[batch] = std::move(dp);
  return MK_OK;
}

// Scratch of one step: the counter groups (with the greedy arrival counter
// after them), the attention partials and the greedy candidates, and the
// launch counts their targets are scaled by.
struct StepScratch {
  uint32_t *ctr;
  float *part;
  uint64_t *amax;
  uint32_t epoch, greedy_epoch;
};

// sc.epoch and sc.greedy_epoch are the counts of the launch's first step;
// a launch of n_steps steps runs epochs sc.epoch .. sc.epoch + n_steps - 1.
static int launch_with(mk_handle *h, DevPlan *dp, int32_t batch, const int32_t *tokens, const int32_t *positions,
                       void *kv_cache, float *logits, int32_t *next_tokens, int32_t *next_positions,
                       const StepScratch &sc, uint32_t n_steps, void *stream) {
  Args a;
  a.ctx = h->d_ctx;
  a.instr = dp->d_instr;
  a.q_off = dp->d_qoff;
  a.waits = dp->d_waits;
  a.rowtab = dp->d_rowtab;
  a.ctr = sc.ctr;
  a.grp_target = dp->d_target;
  a.part_buf = sc.part;
  a.iota = dp->d_iota;
  a.tokens = tokens;
  a.positions = positions;
  a.kv = (uint16_t *)kv_cache;
  a.logits = logits;
  a.trace = dp->d_trace;
  a.trace_stride = dp->trace_stride;
  h->last_plan = dp;
  a.epoch = sc.epoch;
  // one activation tag per step, never 0: the launch takes the next n_steps
  // values, starting again from 1 where they would wrap
  uint32_t t0 = h->tag + 1;
  if (t0 == 0 || (uint64_t)t0 + n_steps - 1 > 0xffffffffull) t0 = 1;
  a.tag = t0;
  h->tag = t0 + n_steps - 1;
  a.batch = batch;
  a.n_split = dp->plan.n_split;
  a.split_len = dp->plan.split_len;
  a.amax = sc.amax;
  a.amax_ctr = sc.ctr + dp->amax_word;
  a.next_tok = next_tokens;
  a.next_pos = next_positions;
  a.n_lm = dp->n_arrive;
  a.amax_target = next_tokens ? sc.greedy_epoch * dp->n_arrive : 0;
  a.n_steps = n_steps;
  a.tok_base = next_tokens ? sc.greedy_epoch - 1 : 0;  // greedy steps before this launch
  a.step_off = 0;
  if (kernel_launch(a, h->num_cus, (h->cfg.flags & MK_FLAG_COOPERATIVE) != 0, dp->plan.paged_kv,
                    (hipStream_t)stream) != hipSuccess)
    return MK_ERR_HIP;
  return MK_OK;
}

static int launch_step(mk_handle *h, int32_t batch, const int32_t *tokens, const int32_t *positions,
                       void *kv_cache, float *logits, int32_t *next_tokens, int32_t *next_positions,
                       uint32_t n_steps, void *stream) {
  if (!h || !tokens || !positions || !kv_cache || !logits) return MK_ERR_INVALID_ARG;
  if (batch < 1 || batch > h->cfg.max_batch) return MK_ERR_INVALID_ARG;
  if (n_steps < 1 || n_steps > (uint32_t)kMaxStepsPerLaunch || (n_steps > 1 && !next_tokens))
    return MK_ERR_INVALID_ARG;
  // One launch for the whole batch: the batch-1 kernel (GEMV on the vector
  // units) or, for 2..8 sequences, the batched kernel (MFMA), each running
  // its batch size's plan.
  DevPlan *dp = nullptr;
  int rc = get_plan(h, batch, &dp);
  if (rc) return rc;
  const uint32_t e0 = dp->epoch + 1, g0 = dp->greedy_epoch + 1;
  dp->epoch += n_steps;
  if (next_tokens) dp->greedy_epoch += n_steps;
  const StepScratch sc{dp->d_ctr, dp->d_part, dp->d_amax, e0, g0};
  rc = launch_with(h, dp, batch, tokens, positions, kv_cache, logits, next_tokens, next_positions, sc, n_steps,
                   stream);
  if (rc != MK_OK) {
    // nothing was enqueued, so the counters did not move: the next launch
    // must wait for the same targets as this one would have
    dp->epoch -= n_steps;
    if (next_tokens) dp->greedy_epoch -= n_steps;
  }
  return rc;
}

int mk_decode_step(mk_handle *h, int32_t batch, const int32_t *tokens, const int32_t *positions, void *kv_cache,
                   float *logits, void *stream) {
  return launch_step(h, batch, tokens, positions, kv_cache, logits, nullptr, nullptr, 1, stream);
}

int mk_decode_step_greedy(mk_handle *h, int32_t batch, const int32_t *tokens, const int32_t *positions,
                          void *kv_cache, float *logits, int32_t *next_tokens, int32_t *next_positions,
                          void *stream) {
  if (!next_tokens || !next_positions) return MK_ERR_INVALID_ARG;
  return launch_step(h, batch, tokens, positions, kv_cache, logits, next_tokens, next_positions, 1, stream);
}

int mk_decode_steps_greedy(mk_handle *h, int32_t batch, int32_t n_steps, const int32_t *tokens,
                           const int32_t *positions, void *kv_cache, float *logits, int32_t *next_tokens,
                           int32_t *next_positions, void *stream) {
  if (!next_tokens || !next_positions || n_steps < 1) return MK_ERR_INVALID_ARG;
  return launch_step(h, batch, tokens, positions, kv_cache, logits, next_tokens, next_positions,
                     (uint32_t)n_steps, stream);
}

int mk_decode_step_static(mk_handle *h, int32_t batch, const int32_t *tokens, const int32_t *positions,
                          void *kv_cache, float *logits, int32_t *next_tokens, int32_t *next_positions,
                          void *stream) {
  if (!h || !tokens || !positions || !kv_cache || !logits) return MK_ERR_INVALID_ARG;
  if (batch < 1 || batch > h->cfg.max_batch) return MK_ERR_INVALID_ARG;
  if ((next_tokens == nullptr) != (next_positions == nullptr)) return MK_ERR_INVALID_ARG;
  // no allocation here: the schedule must already exist, and the step's
  // scratch is this GPU's static array
  auto it = h->plans.find(batch);
  if (it == h->plans.end()) return MK_ERR_NOT_PREPARED;
  DevPlan *dp = it->second.get();
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const size_t amax_bytes = (size_t)dp->n_lm * h->cfg.max_batch * 8;
  const size_t off_part = up(dp->ctr_bytes), off_amax = off_part + up(part_bytes(h->cfg, dp->plan));
  if (off_amax + amax_bytes > kStaticScratchBytes) return MK_ERR_UNSUPPORTED;
  char *base = (char *)h->static_scratch;
  // counters start from zero on every call (the array keeps the previous
  // call's contents); a fill kernel, not a memset, so the step may be
  // captured into a graph
  if (fill_zero(base, dp->ctr_bytes / 4, (hipStream_t)stream) != hipSuccess) return MK_ERR_HIP;
  const StepScratch sc{(uint32_t *)base, (float *)(base + off_part), (uint64_t *)(base + off_amax), 1u, 1u};
  return launch_with(h, dp, batch, tokens, positions, kv_cache, logits, next_tokens, next_positions, sc, 1, stream);
}

int mk_sync_status(mk_handle *h) {
  if (!h) return MK_ERR_INVALID_ARG;
  if (hipDeviceSynchronize() != hipSuccess) return MK_ERR_HIP;
  uint32_t st[4] = {0, 0, 0, 0};
  if (hipMemcpy(st, h->status, sizeof st, hipMemcpyDeviceToHost) != hipSuccess) return MK_ERR_HIP;
  if (st[0] == 0) return MK_OK;
  // a device error: clear it and re-zero every plan's counters
  hipMemset(h->status, 0, 256);
  for (auto &kv : h->plans) {
    hipMemset(kv.second->d_ctr, 0, kv.second->ctr_bytes);
    kv.second->epoch = 0;
    kv.second->greedy_epoch = 0;
  }
  hipDeviceSynchronize();
  const uint32_t top = st[0] >> 24;
  if (top == 0xE1) return MK_ERR_BAD_TOKEN;
  if (top == 0xE2) return MK_ERR_BAD_POSITION;
  return MK_ERR_DEVICE_TIMEOUT;
}

void mk_destroy(mk_handle *h) {
  if (!h) return;
  for (auto &kv : h->plans) free_plan(*kv.second);
  hipFree(h->d_ctx);
  hipFree(h->d_layers);
  hipFree(h->h_buf);
  hipFree(h->q_buf);
  hipFree(h->attn_buf);
  hipFree(h->a_buf);
  hipFree(h->kvn_buf);
  hipFree(h->rope);
  hipFree(h->zero);
  hipFree(h->status);
  delete h;
}

int mk_get_buffer(mk_handle *h, int32_t which, void **ptr, size_t *bytes) {
  if (!h || !ptr || !bytes) return MK_ERR_INVALID_ARG;
  switch (which) {
    case MK_BUF_H: *ptr = h->h_buf; *bytes = h->h_bytes; return MK_OK;
    case MK_BUF_Q: *ptr = h->q_buf; *bytes = h->q_bytes; return MK_OK;
    case MK_BUF_ATTN: *ptr = h->attn_buf; *bytes = h->attn_bytes; return MK_OK;
    case MK_BUF_A: *ptr = h->a_buf; *bytes = h->a_bytes; return MK_OK;
    case MK_BUF_TRACE:
      if (!h->last_plan || !h->last_plan->d_trace) break;
      *ptr = h->last_plan->d_trace;
      *bytes = h->last_plan->trace_bytes;
      return MK_OK;
    default: break;
  }
  *ptr = nullptr;
  *bytes = 0;
  return MK_ERR_INVALID_ARG;
}

}  // extern "C"
