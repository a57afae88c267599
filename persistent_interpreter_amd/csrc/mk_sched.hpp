// mk_sched.hpp -- host instruction scheduler and plan validator.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_plan.hpp"

namespace mk {

// A data region touched by an instruction, for validation only:
// buffer kind x (layer, sequence) x [lo, hi) in that buffer's row/element
// units.
enum Res : uint8_t {
  R_QKV = 1,   // QKV output pairs (q rows and the K/V slot p), per (l, b)
  R_PART = 2,  // attention partials, index = kv_head * n_split + split
  R_ATTN = 3,  // attention output rows (query-head dims), per (l, b)
  R_HMID = 4,  // residual after attention, rows of H
  R_A = 5,     // SiLU(gate)*up, rows of F
  R_HOUT = 6,  // residual after the FFN, rows of H
};

struct Access {
  uint8_t res;
  uint16_t layer;
  uint32_t b;
  uint32_t lo, hi;
  uint32_t phase;  // activation piece before which the read happens (reads)
  // reads only: the data is tagged with its step and the reader re-reads
  // until every word carries this step's tag, so no counter guards it (the
  // reader waits for its writers by itself)
  uint8_t tagged;
};

struct Plan {
  int num_cus = 0, batch = 0, n_split = 0, split_len = 0, mlp_chunks = 0;
  int n_groups = 0;
  int n_lm_groups = 0;              // workgroups holding LM units
  int down_splits = 0;              // split-K down units per row group (0: none)
  int n_down_groups = 0;            // (layer, row group) arrival counters
  bool paged_kv = false;            // attention units stream K/V pages
  std::vector<Instr> instr;         // all per-CU queues back to back
  std::vector<uint32_t> q_off;      // [num_cus + 1]
  std::vector<Wait> waits;
  std::vector<uint32_t> grp_target; // [n_groups][kSlots]
  std::vector<uint32_t> grp_nslot;  // [n_groups] counters in use
  std::vector<uint32_t> grp_producers;  // [n_groups] total producer units
  std::vector<uint64_t> rowtab;     // row start addresses of tabulated units
  // validation metadata, parallel to instr
  std::vector<std::vector<Access>> reads, writes;
  int64_t weight_bytes = 0, max_cu_bytes = 0;
  int n_pages = 0;
};

// Choose the elements per weight piece for a K dimension: the largest
// divisor of K whose byte size is a multiple of 1 KB or a divisor of 1 KB,
// at most kMaxKc.  Returns 0 if none.
int choose_kc(int K, int kmax);

// Build the plan.  Returns MK_OK or an MK_ERR_* code with `err` set.
int build_plan(const mk_config &cfg, int batch, int num_cus, Plan &out,
               std::string &err);

// Fill every weight-streaming descriptor's row addressing (w0, w1, tab,
// rowb) from the model's device pointers.
void resolve_streams(const mk_config &cfg, const mk_weights &w, Plan &plan);

// Static checks plus `sim_runs` interleavings (see mk_plan_check in mk.h).
int check_plan(const mk_config &cfg, Plan &plan, int sim_runs, int corrupt,
               uint64_t seed, mk_plan_report *rep);

}  // namespace mk
