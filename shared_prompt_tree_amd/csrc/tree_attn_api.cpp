// C ABI of libtreeattn.so (declared in include/tree_attn.h).
//
// Every entry point validates its arguments on the host before the first
// HIP call, lays out the caller's workspace, and enqueues:
//   prefill      : work list, V^T copy, forward kernel
//   replay_fwd   : work list, V^T copies, forward kernel (prompt column and
//                  own branch merged in one online-softmax state)
//   replay_bwd   : work lists, K^T / Q^T / dO^T copies (the dO^T copy also
//                  forms delta = rowsum(dO o O)), dQ kernel, dK/dV kernel
//                  (prompt tiles write float32 seeds summed over every
//                  branch; own-branch tiles write dK_R, dV_R)
//   prefill_bwd  : work lists, K^T / Q^T / dO^T copies (with delta), dQ
//                  kernel, dK/dV kernel (prefill term plus the seeds)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "tree_attn.h"
#include "device_common.h"
#include "launch.h"

using namespace treeattn;

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kStaticScratchBytes = TREE_ATTN_STATIC_SCRATCH_BYTES;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }
long long pad_len(long long n) { return ceil_div(n, kPad) * kPad; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Host-side facts derived from the problem after validation.
struct Shape {
  int ng = 0, nb = 0, hq = 0, hkv = 0, d = 0, dtype = 0, hp = 1, tile_q = 0;
  size_t esz = 0;
  long long p_tokens = 0, r_tokens = 0;
  long long p_pad = 0, r_pad = 0;    // padded token totals
  long long q_items_prefill = 0, q_items_replay = 0;
  long long wq_items_prefill = 0, wq_items_replay = 0;  // with 384-row forward tiles
  long long k_items_prefill = 0, k_items_replay = 0;
  // replay key-stationary list: splits of the prompt tiles (prompt_splits)
  long long split_target = 0;  // rows one prompt split should read at most
  long long n_splits = 0;      // sum over groups of the splits
  long long part_rows = 0;     // partial-seed rows of the split groups
  int max_prompt = 0;          // longest prompt
  int col_splits_fwd = 1;      // prompt-column chunks of the replay forward launch
  int col_splits_bwd = 1;      // and of the replay dQ launch
  long long own_work = 0;      // own-branch 64-key steps over the replay query tiles
  long long own_max = 0;       // most own-branch steps of one query tile
  long long prompt_work = 0;   // prompt-column 64-key steps over the replay query tiles
  bool fused_replay = false;   // replay backward forms dQ in the dK/dV kernel
  bool fused_prefill = false;  // prefill backward likewise
};

// A replay key-stationary item reading more than the launch's total rows
// divided by this is worth splitting: with one dK/dV workgroup per compute
// unit of a 256-CU MI355X, no item then exceeds half of one CU's fair share,
// so the largest-first order can balance the launch.  Measured
// (bench.py --tile-split-sweep, five short-prompt shapes and the
// response-heavy workload): every value from 256 to 4096 is within 2-6% of
// the best split target, and 512 within 2.1% on all of them; not splitting
// costs up to 1.9x.
constexpr long long kSplitSlots = 512;

// Replay query-stationary launches (forward, dQ) may cut each prompt column
// into S chunks of whole 64-key tiles (each at least kMinChunkKeys keys);
// the chunks' partial results are merged afterwards.  S is chosen by a
// makespan model (the largest-first placement of section 3.4, Eq. 6, on 256
// compute units, scored like Eqs. 7-10 with compute and movement terms), in
// units of one 64-key step of one workgroup:
//   items      q_wgs * S, each costing its prompt chunk, its own-branch
//              tiles (last chunk only) and an item overhead;
//   makespan   max(rounds * mean item, longest item), rounds =
//              ceil(items / kQSlots) (one 8-wave workgroup per CU): the
//              critical path of largest-first list scheduling, which the
//              hardware dispatcher performs on the largest-first work list;
//   merge      2 * S * response rows * Hq * d * 4 bytes of float32 partials
//              written and read back, at a bytes-per-unit rate.
// The forward and the dQ pass are priced separately (each entry point cuts
// its own launch).  Their constants were fitted to bench.py --split-sweep:
// replay calls of five few-row shapes timed at S = 1..32 on one MI355X
// (forward: 1.7 us per unit, 6 units of overhead per workgroup, merge at
// 0.275 ms/GB; dQ pass: 2.0 us per unit, no measurable overhead, merge at
// 0.30 ms/GB; 2.7% and 3.2% rms error).  Only launches of up to
// kColSearchWgs workgroups are considered: beyond that a partial last round
// costs little.
constexpr int kMinChunkKeys = 1024;
constexpr int kMaxColSplits = 64;
constexpr long long kQSlots = 256;
constexpr long long kColSearchWgs = 8 * kQSlots;

struct ColSplitCosts {
  double item_overhead;         // units per workgroup
  double merge_bytes_per_unit;  // partial bytes merged per unit of time
};
constexpr ColSplitCosts kFwdSplitCosts{6.0, 6.2e6};
constexpr ColSplitCosts kDqSplitCosts{0.0, 6.7e6};

// Prompt-column chunks S of a replay query launch (see the model above).
int choose_col_splits(const Shape& s, const ColSplitCosts& c) {
  const long long n_hg = s.hq / s.hp;
  const long long q_wgs = s.q_items_replay * n_hg;
  const long long smax =
      std::min<long long>(kMaxColSplits, s.max_prompt / kMinChunkKeys);
  if (q_wgs == 0 || q_wgs > kColSearchWgs || smax < 2) return 1;
  const double prompt = (double)s.prompt_work * n_hg, own = (double)s.own_work * n_hg;
  const long long ptiles_max = ceil_div(s.max_prompt, kTileK);
  const double row_bytes = (double)s.r_tokens * s.hq * s.d * 4;
  int best = 1;
  double best_t = 0;
  for (long long S = 1; S <= smax; ++S) {
    const long long items = q_wgs * S;
    const double work = prompt + own + c.item_overhead * items;
    const double longest = (double)ceil_div(ptiles_max, S) + s.own_max + c.item_overhead;
    const double rounds = (double)ceil_div(items, kQSlots);
    double t = std::max(rounds * work / items, longest);
    if (S > 1) t += 2.0 * S * row_bytes / c.merge_bytes_per_unit;
    if (S == 1 || t < best_t) {
      best = (int)S;
      best_t = t;
    }
  }
  return best;
}

// dQ strategy of a backward call under TREE_ATTN_DQ_AUTO: a cost model in
// the spirit of the planner's (section 3.4, "Cost model", Eqs. 7-10: compute
// plus movement terms with constants calibrated on measured runs), on one
// GPU.  Per call, with `pairs` the valid (row, key) pairs times Hq:
//   separate  pairs * 14 d / kSepFlops          (dQ pass 6d + dK/dV 8d)
//   fused     max(pairs * 10 d / kFusedFlops,   (one pass, 10d)
//                 atomic bytes / kAtomicBytes)  (dQ added per key tile)
// where every query row adds d float32 per key tile it reads (its group's
// prompt tiles plus the causal tiles of its own segment).  The constants
// come from same-box runs of both strategies on the prompt-heavy,
// response-heavy and long-mixed workloads: the separate kernels ran at
// 1.04-1.06 PFLOP/s of executed work, the fused kernel added its dQ rows at
// 0.79-0.97 TB/s, below the time of its arithmetic, so it is bound by the
// atomics (2 bytes per pair at head_dim 128) and the model prefers the
// separate pass on every shape measured.
constexpr double kSepFlops = 1.05e15;
constexpr double kFusedFlops = 1.06e15;
constexpr double kAtomicBytes = 0.95e12;

// sum over k = 1..n of ceil(k / kTileKV): key tiles read by the rows of an
// n-token causal segment
double causal_tile_visits(long long n) {
  const long long m = n / kTileKV, q = n % kTileKV;
  return (double)kTileKV * m * (m + 1) / 2 + (double)q * (m + 1);
}

bool choose_dq_fused(const tree_attn_problem* p, const Shape& s, bool replay) {
  double pairs = 0, visits = 0;
  for (int g = 0; g < s.ng; ++g) {
    const long long P = p->prompt_cu_h[g + 1] - p->prompt_cu_h[g];
    if (!replay) {
      pairs += (double)P * (P + 1) / 2;
      visits += causal_tile_visits(P);
      continue;
    }
    for (int i = p->group_branch_cu_h[g]; i < p->group_branch_cu_h[g + 1]; ++i) {
      const long long r = p->resp_cu_h[i + 1] - p->resp_cu_h[i];
      pairs += (double)r * P + (double)r * (r + 1) / 2;
      visits += (double)r * ceil_div(P, kTileKV) + causal_tile_visits(r);
    }
  }
  const double t_sep = pairs * s.hq * 14.0 * s.d / kSepFlops;
  const double t_fused = std::max(pairs * s.hq * 10.0 * s.d / kFusedFlops,
                                  visits * s.hq * s.d * 4.0 / kAtomicBytes);
  return t_fused < t_sep;
}

int validate_problem(const tree_attn_problem* p, bool need_device, Shape& s) {
  if (!p) return TREE_ATTN_ERR_INVALID;
  if (p->dq_strategy < TREE_ATTN_DQ_AUTO || p->dq_strategy > TREE_ATTN_DQ_FUSED)
    return TREE_ATTN_ERR_INVALID;
  if (p->dq_strategy == TREE_ATTN_DQ_FUSED &&
      (p->dtype != TREE_ATTN_BF16 || p->head_dim != 128))
    return TREE_ATTN_ERR_UNSUPPORTED;
  if (p->dtype != TREE_ATTN_F32 && p->dtype != TREE_ATTN_BF16) return TREE_ATTN_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return TREE_ATTN_ERR_UNSUPPORTED;
  if (p->num_groups < 1 || p->num_branches < 0) return TREE_ATTN_ERR_INVALID;
  if (p->num_q_heads < 1 || p->num_kv_heads < 1) return TREE_ATTN_ERR_INVALID;
  if (p->num_q_heads % p->num_kv_heads != 0) return TREE_ATTN_ERR_INVALID;
  if (!(p->softmax_scale > 0.f) || !std::isfinite(p->softmax_scale)) return TREE_ATTN_ERR_INVALID;
  if (!p->prompt_cu_h || !p->group_branch_cu_h || !p->resp_cu_h) return TREE_ATTN_ERR_INVALID;
  if (need_device && (!p->prompt_cu_d || !p->group_branch_cu_d || !p->resp_cu_d))
    return TREE_ATTN_ERR_INVALID;
  const int ng = p->num_groups, nb = p->num_branches;
  if (p->prompt_cu_h[0] != 0 || p->group_branch_cu_h[0] != 0 || p->resp_cu_h[0] != 0)
    return TREE_ATTN_ERR_INVALID;
  for (int g = 0; g < ng; ++g) {
    if (p->prompt_cu_h[g + 1] < p->prompt_cu_h[g]) return TREE_ATTN_ERR_INVALID;
    if (p->group_branch_cu_h[g + 1] < p->group_branch_cu_h[g]) return TREE_ATTN_ERR_INVALID;
  }
  if (p->group_branch_cu_h[ng] != nb) return TREE_ATTN_ERR_INVALID;
  for (int i = 0; i < nb; ++i)
    if (p->resp_cu_h[i + 1] < p->resp_cu_h[i]) return TREE_ATTN_ERR_INVALID;

  s.ng = ng;
  s.nb = nb;
  s.hq = p->num_q_heads;
  s.hkv = p->num_kv_heads;
  s.d = p->head_dim;
  s.dtype = p->dtype;
  s.esz = p->dtype == TREE_ATTN_BF16 ? 2 : 4;
  const int grp = s.hq / s.hkv;
  s.hp = 1;
  while (s.hp < 16 && grp % (2 * s.hp) == 0) s.hp *= 2;
  s.tile_q = kTileQ / s.hp;
  s.p_tokens = p->prompt_cu_h[ng];
  s.r_tokens = p->resp_cu_h[nb];
  // every index the kernels form must fit in int32
  const long long lim = (1LL << 31) - 1;
  if ((s.p_tokens + s.r_tokens) * (long long)s.hq > lim) return TREE_ATTN_ERR_INVALID;
  for (int g = 0; g < ng; ++g) {
    const int len = p->prompt_cu_h[g + 1] - p->prompt_cu_h[g];
    s.max_prompt = std::max(s.max_prompt, len);
    s.p_pad += pad_len(len);
    s.q_items_prefill += ceil_div(len, s.tile_q);
    s.wq_items_prefill += ceil_div(len, kTileQWide / s.hp);
    s.k_items_prefill += ceil_div(len, kTileKV);
  }
  // Rows read by the replay key-stationary items (prompt tiles read every
  // response row of their group, an own-branch tile the rows at or after
  // it), the longest own-branch item, and from them the split target.
  long long total = 0, longest = 0;
  for (int i = 0; i < nb; ++i) {
    const int len = p->resp_cu_h[i + 1] - p->resp_cu_h[i];
    s.r_pad += pad_len(len);
    s.q_items_replay += ceil_div(len, s.tile_q);
    for (long long q = s.tile_q; q < len + s.tile_q; q += s.tile_q) {  // own keys per query tile
      const long long own = ceil_div(std::min<long long>(q, len), kTileK);
      s.own_work += own;
      s.own_max = std::max(s.own_max, own);
    }
    s.wq_items_replay += ceil_div(len, kTileQWide / s.hp);
    const long long n = ceil_div(len, kTileKV);
    s.k_items_replay += n;
    total += n * len - (long long)kTileKV * n * (n - 1) / 2;
    longest = std::max<long long>(longest, len);
  }
  for (int g = 0; g < ng; ++g) {
    const int plen = p->prompt_cu_h[g + 1] - p->prompt_cu_h[g];
    const long long rows =
        (long long)p->resp_cu_h[p->group_branch_cu_h[g + 1]] - p->resp_cu_h[p->group_branch_cu_h[g]];
    total += (long long)ceil_div(plen, kTileKV) * rows;
    for (int i = p->group_branch_cu_h[g]; i < p->group_branch_cu_h[g + 1]; ++i)
      s.prompt_work += ceil_div(p->resp_cu_h[i + 1] - p->resp_cu_h[i], s.tile_q) *
                       ceil_div(plen, kTileK);
  }
  if (p->prompt_tile_split_rows < 0) return TREE_ATTN_ERR_INVALID;
  s.split_target = p->prompt_tile_split_rows > 0
                       ? (long long)p->prompt_tile_split_rows
                       : std::max(longest, (total * s.hkv + kSplitSlots - 1) / kSplitSlots);
  for (int g = 0; g < ng; ++g) {
    const int plen = p->prompt_cu_h[g + 1] - p->prompt_cu_h[g];
    const int branches = p->group_branch_cu_h[g + 1] - p->group_branch_cu_h[g];
    const long long rows =
        (long long)p->resp_cu_h[p->group_branch_cu_h[g + 1]] - p->resp_cu_h[p->group_branch_cu_h[g]];
    const int sg = prompt_splits(branches, rows, s.split_target);
    s.n_splits += sg;
    s.k_items_replay += (long long)ceil_div(plen, kTileKV) * sg;
    if (sg > 1) s.part_rows += (long long)sg * plen;
  }
  if (s.p_pad * s.hp > lim || s.r_pad * s.hp > lim) return TREE_ATTN_ERR_INVALID;
  if (s.k_items_replay * s.hkv > lim || s.part_rows > lim)
    return TREE_ATTN_ERR_INVALID;
  if (p->prompt_col_splits < 0 || p->prompt_col_splits > kMaxColSplits) return TREE_ATTN_ERR_INVALID;
  s.col_splits_fwd = p->prompt_col_splits > 0 ? p->prompt_col_splits
                                              : choose_col_splits(s, kFwdSplitCosts);
  s.col_splits_bwd = p->prompt_col_splits > 0 ? p->prompt_col_splits
                                              : choose_col_splits(s, kDqSplitCosts);
  if (p->dq_strategy == TREE_ATTN_DQ_FUSED) {
    s.fused_replay = s.fused_prefill = true;
  } else if (p->dq_strategy == TREE_ATTN_DQ_AUTO && s.dtype == TREE_ATTN_BF16 && s.d == 128) {
    s.fused_replay = choose_dq_fused(p, s, true);
    s.fused_prefill = choose_dq_fused(p, s, false);
  }
  // every attention launch must fit one dispatch: at most 2^32 - 1
  // work-items (workgroups x threads), counting the XCD round-up
  const long long n_hg = s.hq / s.hp;
  const long long dispatch_max = (long long)UINT32_MAX;
  const long long q_prefill = std::max(s.q_items_prefill * 512, s.wq_items_prefill * 768);
  const long long q_replay =
      std::max(s.q_items_replay * std::max(s.col_splits_fwd, s.col_splits_bwd) * 512,
               s.wq_items_replay * 768);
  if ((q_prefill + 8 * 768) * n_hg > dispatch_max || (q_replay + 8 * 768) * n_hg > dispatch_max)
    return TREE_ATTN_ERR_INVALID;
  if ((std::max(s.k_items_prefill, s.k_items_replay) + 8) * s.hkv * 512 > dispatch_max)
    return TREE_ATTN_ERR_INVALID;
  // tile copies address a head group's slice of a transposed copy with a
  // 32-bit byte offset
  const long long slice = (long long)s.d * std::max(s.p_pad, s.r_pad) * s.hp * (long long)s.esz;
  if (slice > (long long)UINT32_MAX) return TREE_ATTN_ERR_INVALID;
  return TREE_ATTN_OK;
}

// Bump allocator over the caller's workspace.
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    void* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  }
};

struct MetaBufs {
  int32_t* prompt_pad;
  int32_t* resp_pad;
  int32_t* branch_group;
  int32_t* src_cu;
  int32_t* src_order;
  int32_t* split_cu;
  int32_t* split_first;
  int32_t* part_row;
  void* items;
};

MetaBufs take_meta(Carve& c, const Shape& s, long long cap, size_t item_bytes) {
  MetaBufs m;
  m.prompt_pad = static_cast<int32_t*>(c.take((s.ng + 1) * sizeof(int32_t)));
  m.resp_pad = static_cast<int32_t*>(c.take((s.nb + 1) * sizeof(int32_t)));
  m.branch_group = static_cast<int32_t*>(c.take((s.nb + 1) * sizeof(int32_t)));
  m.src_cu = static_cast<int32_t*>(c.take((s.ng + s.nb + 1) * sizeof(int32_t)));
  m.src_order = static_cast<int32_t*>(c.take((s.ng + s.nb + 1) * sizeof(int32_t)));
  m.split_cu = static_cast<int32_t*>(c.take((s.ng + 1) * sizeof(int32_t)));
  m.split_first = static_cast<int32_t*>(c.take((s.n_splits + 1) * sizeof(int32_t)));
  m.part_row = static_cast<int32_t*>(c.take((s.ng + 1) * sizeof(int32_t)));
  m.items = c.take(std::max<long long>(cap, 1) * item_bytes);
  return m;
}

// Workspace layout of one entry point.  With base == nullptr only the size
// is computed.
struct Plan {
  MetaBufs mq{}, mk{};
  void* vt_p = nullptr;   // V^T prompt  [hkv][d][p_pad]
  void* vt_r = nullptr;   // V^T response
  void* kt_p = nullptr;   // K^T prompt
  void* kt_r = nullptr;   // K^T response
  void* qt = nullptr;     // Q^T  [hq/hp][d][pad*hp]
  void* dot = nullptr;    // dO^T
  float* delta = nullptr; // [hq][tokens]
  float* part_k = nullptr;  // partial prompt seeds of split groups [part_rows][hkv][d]
  float* part_v = nullptr;
  float* o_part = nullptr;    // split prompt column: [chunks][r_tokens][hq][d]
  float* lse_part = nullptr;  // [chunks][hq][r_tokens]
  float* dq_part = nullptr;   // [chunks][r_tokens][hq][d]
  float* dq_acc = nullptr;    // fused dQ strategy: float32 dQ / scale [tokens][hq][d]
  size_t bytes = 0;
};

Plan make_plan(const Shape& s, int op, void* base) {
  Plan pl;
  Carve c(base);
  const size_t e = s.esz;
  const size_t kvT_p = (size_t)s.hkv * s.d * s.p_pad * e;
  const size_t kvT_r = (size_t)s.hkv * s.d * s.r_pad * e;
  switch (op) {
    case TREE_ATTN_OP_PREFILL:
      pl.mq = take_meta(c, s, s.q_items_prefill, sizeof(QItem));
      pl.vt_p = c.take(kvT_p);
      break;
    case TREE_ATTN_OP_REPLAY_FWD:
      pl.mq = take_meta(c, s, s.q_items_replay * s.col_splits_fwd, sizeof(QItem));
      pl.vt_p = c.take(kvT_p);
      pl.vt_r = c.take(kvT_r);
      if (s.col_splits_fwd > 1) {
        pl.o_part = static_cast<float*>(
            c.take((size_t)s.col_splits_fwd * s.r_tokens * s.hq * s.d * sizeof(float)));
        pl.lse_part = static_cast<float*>(
            c.take((size_t)s.col_splits_fwd * s.hq * s.r_tokens * sizeof(float)));
      }
      break;
    case TREE_ATTN_OP_REPLAY_BWD:
      if (s.fused_replay) {
        pl.dq_acc = static_cast<float*>(c.take((size_t)s.r_tokens * s.hq * s.d * sizeof(float)));
        pl.mk = take_meta(c, s, s.k_items_replay, sizeof(KItem));
      } else {
        pl.mq = take_meta(c, s, s.q_items_replay * s.col_splits_bwd, sizeof(QItem));
        if (s.col_splits_bwd > 1)
          pl.dq_part = static_cast<float*>(
              c.take((size_t)s.col_splits_bwd * s.r_tokens * s.hq * s.d * sizeof(float)));
        pl.mk = take_meta(c, s, s.k_items_replay, sizeof(KItem));
        pl.kt_p = c.take(kvT_p);
        pl.kt_r = c.take(kvT_r);
      }
      pl.qt = c.take((size_t)s.hq * s.d * s.r_pad * e);
      pl.dot = c.take((size_t)s.hq * s.d * s.r_pad * e);
      pl.delta = static_cast<float*>(c.take((size_t)s.hq * s.r_tokens * sizeof(float)));
      if (s.part_rows > 0) {
        const size_t part = (size_t)s.part_rows * s.hkv * s.d * sizeof(float);
        pl.part_k = static_cast<float*>(c.take(part));
        pl.part_v = static_cast<float*>(c.take(part));
      }
      break;
    case TREE_ATTN_OP_PREFILL_BWD:
      if (s.fused_prefill) {
        pl.dq_acc = static_cast<float*>(c.take((size_t)s.p_tokens * s.hq * s.d * sizeof(float)));
      } else {
        pl.mq = take_meta(c, s, s.q_items_prefill, sizeof(QItem));
        pl.kt_p = c.take(kvT_p);
      }
      pl.mk = take_meta(c, s, s.k_items_prefill, sizeof(KItem));
      pl.qt = c.take((size_t)s.hq * s.d * s.p_pad * e);
      pl.dot = c.take((size_t)s.hq * s.d * s.p_pad * e);
      pl.delta = static_cast<float*>(c.take((size_t)s.hq * s.p_tokens * sizeof(float)));
      break;
    default:
      break;
  }
  pl.bytes = c.off;
  return pl;
}

int check_ws(const Shape& s, int op, void* ws, size_t ws_bytes, Plan& pl) {
  pl = make_plan(s, op, nullptr);
  if (ws_bytes < pl.bytes) return TREE_ATTN_ERR_WORKSPACE;
  if (pl.bytes > 0 && !ws) return TREE_ATTN_ERR_INVALID;
  if (!aligned16(ws)) return TREE_ATTN_ERR_INVALID;
  pl = make_plan(s, op, ws);
  return TREE_ATTN_OK;
}

// A tensor pointer must be non-null and 16-byte aligned unless it has no
// element at all.
bool tensor_ok(const void* p, long long tokens) {
  if (tokens == 0) return true;
  return p != nullptr && aligned16(p);
}

thread_local hipError_t g_last_hip = hipSuccess;
thread_local hipEvent_t g_events[3][2] = {{nullptr, nullptr}, {nullptr, nullptr}, {nullptr, nullptr}};

int hip_status(hipError_t e) {
  if (e == hipSuccess) return TREE_ATTN_OK;
  g_last_hip = e;
  return TREE_ATTN_ERR_HIP;
}

#define TA_TRY(expr)                          \
  do {                                        \
    hipError_t e_ = (expr);                   \
    if (e_ != hipSuccess) return hip_status(e_); \
  } while (0)

hipError_t run_meta(const tree_attn_problem* p, const Shape& s, const MetaBufs& m, int mode,
                    long long cap, hipStream_t st, int tile_q = 0, int col_splits = 1) {
  MetaArgs a;
  a.mode = mode;
  a.n_groups = s.ng;
  a.n_branches = s.nb;
  a.prompt_cu = p->prompt_cu_d;
  a.group_branch_cu = p->group_branch_cu_d;
  a.resp_cu = p->resp_cu_d;
  a.prompt_pad = m.prompt_pad;
  a.resp_pad = m.resp_pad;
  a.branch_group = m.branch_group;
  a.src_cu = m.src_cu;
  a.src_order = m.src_order;
  a.items = m.items;
  a.cap = (int)cap;
  a.tile_q = tile_q > 0 ? tile_q : s.tile_q;
  a.col_splits = mode == kMetaQReplay ? col_splits : 1;
  a.split_target = mode == kMetaKReplay ? s.split_target : 0;
  a.split_cu = m.split_cu;
  a.split_first = m.split_first;
  a.part_row = m.part_row;
  return launch_meta(a, st);
}

// Transposed padded copy of `in`; with dot_with/dot_out (the dO copy of a
// backward call, O and delta) the same pass also forms the row dot.
hipError_t run_transpose(const void* in, void* out, int heads, int hp, const Shape& s, int n_seg,
                         const int32_t* seg_cu_d, const int32_t* seg_pad_d, long long pad_tokens,
                         hipStream_t st, const void* dot_with = nullptr, float* dot_out = nullptr,
                         long long dot_tokens = 0) {
  TransposeArgs t;
  t.dot_with = dot_with;
  t.dot_out = dot_out;
  t.dot_tokens = (int)dot_tokens;
  t.in = in;
  t.out = out;
  t.heads = heads;
  t.hp = hp;
  t.d = s.d;
  t.n_seg = n_seg;
  t.seg_cu = seg_cu_d;
  t.seg_pad = seg_pad_d;
  t.pad_tokens = (int)pad_tokens;
  return launch_transpose(t, s.dtype, st);
}

// Forward launch shape: the 12-wave kernel (384 rows per item) where its
// item count still gives every CU several workgroups, else 8 waves.
struct FwdShape {
  int waves, tile_q;
  long long items;
};
FwdShape fwd_shape(const Shape& s, long long items, long long wide_items) {
  if (s.dtype == TREE_ATTN_BF16 && wide_items * (s.hq / s.hp) >= kWideMinWorkgroups)
    return {12, kTileQWide / s.hp, wide_items};
  return {8, s.tile_q, items};
}

// Host checks of a replay forward call (problem, tensors); fills s.
int check_replay_fwd(const tree_attn_problem* problem, const void* k_p, const void* v_p,
                     const void* q_r, const void* k_r, const void* v_r, void* o_r, float* lse_r,
                     Shape& s) {
  const int rc = validate_problem(problem, true, s);
  if (rc != TREE_ATTN_OK) return rc;
  if (!tensor_ok(k_p, s.p_tokens) || !tensor_ok(v_p, s.p_tokens)) return TREE_ATTN_ERR_INVALID;
  for (const void* t : {q_r, k_r, v_r, static_cast<const void*>(o_r), static_cast<const void*>(lse_r)})
    if (!tensor_ok(t, s.r_tokens)) return TREE_ATTN_ERR_INVALID;
  return TREE_ATTN_OK;
}

// The replay forward's launches, with scratch laid out by pl.
int run_replay_fwd(const tree_attn_problem* problem, const Shape& s, const Plan& pl,
                   const void* k_p, const void* v_p, const void* q_r, const void* k_r,
                   const void* v_r, void* o_r, float* lse_r, hipStream_t st) {
  if (s.r_tokens == 0) return TREE_ATTN_OK;
  (void)hipGetLastError();
  const int S = s.col_splits_fwd;
  const bool split = S > 1;
  const FwdShape fs = split ? FwdShape{8, s.tile_q, s.q_items_replay * S}
                            : fwd_shape(s, s.q_items_replay, s.wq_items_replay);
  TA_TRY(run_meta(problem, s, pl.mq, kMetaQReplay, s.q_items_replay * S, st, fs.tile_q, S));
  TA_TRY(run_transpose(v_p, pl.vt_p, s.hkv, 1, s, s.ng, problem->prompt_cu_d, pl.mq.prompt_pad,
                       s.p_pad, st));
  TA_TRY(run_transpose(v_r, pl.vt_r, s.hkv, 1, s, s.nb, problem->resp_cu_d, pl.mq.resp_pad,
                       s.r_pad, st));
  FwdLaunch f;
  f.waves = fs.waves;
  f.q = q_r;
  f.o = o_r;
  f.lse = lse_r;
  f.k_a = k_p;
  f.vt_a = pl.vt_p;
  f.k_b = k_r;
  f.vt_b = pl.vt_r;
  f.items = pl.mq.items;
  f.n_items = (int)fs.items;
  f.hq = s.hq;
  f.hkv = s.hkv;
  f.hp = s.hp;
  f.d = s.d;
  f.dtype = s.dtype;
  f.lse_stride = (int)s.r_tokens;
  f.vt_a_stride = (int)s.p_pad;
  f.vt_b_stride = (int)s.r_pad;
  f.scale = problem->softmax_scale;
  f.o_part = pl.o_part;
  f.lse_part = pl.lse_part;
  TA_TRY(launch_fwd(f, st));
  if (split)  // the chunks' partial states, merged (section 3.3)
    TA_TRY(launch_lse_merge(S, (int)s.r_tokens, s.hq, s.d, s.dtype, pl.o_part,
                            pl.lse_part, o_r, lse_r, st));
  return TREE_ATTN_OK;
}

}  // namespace

// ------------------------------------------------------------ static scratch
//
// Scratch of tree_attn_replay_fwd_noalloc, for callers that cannot allocate
// device memory: one array per GPU, allocated with the code object when the
// library is loaded on that device and held until the process ends.  On the
// host the name `scratch` stands for the variable, not for its device
// address: host code only ever uses the address looked up below, once per
// device, with that device current.
// The array has external linkage: a `static` device array becomes a local
// symbol of the code object, which the HIP runtime cannot resolve from the
// host-side variable (it aborts the process instead of returning an error).
// kAlign bytes of slack let the looked-up address be rounded up to kAlign
// whatever alignment the code object gives the symbol.
namespace treeattn {
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes + kAlign];
}  // namespace treeattn

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_base[kMaxDevices] = {};

// Device address of the scratch array on the device of `stream`, which must
// be the calling thread's current device.
int static_scratch(hipStream_t stream, void** base) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (stream != nullptr) {
    int sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return hip_status(e);
    if (sdev != dev) return TREE_ATTN_ERR_INVALID;
  }
  if (dev < 0 || dev >= kMaxDevices) return TREE_ATTN_ERR_INVALID;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_base[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(treeattn::scratch));
    if (e != hipSuccess) return hip_status(e);
    if (p == nullptr) return TREE_ATTN_ERR_HIP;
    g_scratch_base[dev] = reinterpret_cast<void*>(align_up(reinterpret_cast<uintptr_t>(p)));
  }
  *base = g_scratch_base[dev];
  return TREE_ATTN_OK;
}

}  // namespace

namespace treeattn {
void kernel_events(int kind, hipEvent_t* start, hipEvent_t* stop) {
  *start = g_events[kind][0];
  *stop = g_events[kind][1];
}
}  // namespace treeattn

extern "C" {

int tree_attn_workspace_size(const tree_attn_problem* problem, int op, size_t* bytes) {
  if (!bytes) return TREE_ATTN_ERR_INVALID;
  if (op < TREE_ATTN_OP_PREFILL || op > TREE_ATTN_OP_PREFILL_BWD) return TREE_ATTN_ERR_INVALID;
  Shape s;
  const int rc = validate_problem(problem, false, s);
  if (rc != TREE_ATTN_OK) return rc;
  *bytes = make_plan(s, op, nullptr).bytes;
  return TREE_ATTN_OK;
}

int tree_attn_prefill(const tree_attn_problem* problem, const void* q_p, const void* k_p,
                      const void* v_p, void* o_p, float* lse_p, void* ws, size_t ws_bytes,
                      tree_attn_stream_t stream) {
  Shape s;
  int rc = validate_problem(problem, true, s);
  if (rc != TREE_ATTN_OK) return rc;
  for (const void* t : {q_p, k_p, v_p, static_cast<const void*>(o_p), static_cast<const void*>(lse_p)})
    if (!tensor_ok(t, s.p_tokens)) return TREE_ATTN_ERR_INVALID;
  Plan pl;
  rc = check_ws(s, TREE_ATTN_OP_PREFILL, ws, ws_bytes, pl);
  if (rc != TREE_ATTN_OK) return rc;
  if (s.p_tokens == 0) return TREE_ATTN_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const FwdShape fs = fwd_shape(s, s.q_items_prefill, s.wq_items_prefill);
  TA_TRY(run_meta(problem, s, pl.mq, kMetaQPrefill, s.q_items_prefill, st, fs.tile_q));
  TA_TRY(run_transpose(v_p, pl.vt_p, s.hkv, 1, s, s.ng, problem->prompt_cu_d, pl.mq.prompt_pad,
                       s.p_pad, st));
  FwdLaunch f;
  f.waves = fs.waves;
  f.o_part = nullptr;
  f.lse_part = nullptr;
  f.q = q_p;
  f.o = o_p;
  f.lse = lse_p;
  f.k_a = k_p;
  f.vt_a = pl.vt_p;
  f.k_b = k_p;
  f.vt_b = pl.vt_p;
  f.items = pl.mq.items;
  f.n_items = (int)fs.items;
  f.hq = s.hq;
  f.hkv = s.hkv;
  f.hp = s.hp;
  f.d = s.d;
  f.dtype = s.dtype;
  f.lse_stride = (int)s.p_tokens;
  f.vt_a_stride = (int)s.p_pad;
  f.vt_b_stride = (int)s.p_pad;
  f.scale = problem->softmax_scale;
  TA_TRY(launch_fwd(f, st));
  return TREE_ATTN_OK;
}

int tree_attn_replay_fwd(const tree_attn_problem* problem, const void* k_p, const void* v_p,
                         const void* q_r, const void* k_r, const void* v_r, void* o_r,
                         float* lse_r, void* ws, size_t ws_bytes, tree_attn_stream_t stream) {
  Shape s;
  int rc = check_replay_fwd(problem, k_p, v_p, q_r, k_r, v_r, o_r, lse_r, s);
  if (rc != TREE_ATTN_OK) return rc;
  Plan pl;
  rc = check_ws(s, TREE_ATTN_OP_REPLAY_FWD, ws, ws_bytes, pl);
  if (rc != TREE_ATTN_OK) return rc;
  return run_replay_fwd(problem, s, pl, k_p, v_p, q_r, k_r, v_r, o_r, lse_r,
                        static_cast<hipStream_t>(stream));
}

int tree_attn_replay_fwd_noalloc(const tree_attn_problem* problem, const void* k_p,
                                 const void* v_p, const void* q_r, const void* k_r,
                                 const void* v_r, void* o_r, float* lse_r,
                                 tree_attn_stream_t stream) {
  Shape s;
  int rc = check_replay_fwd(problem, k_p, v_p, q_r, k_r, v_r, o_r, lse_r, s);
  if (rc != TREE_ATTN_OK) return rc;
  if (make_plan(s, TREE_ATTN_OP_REPLAY_FWD, nullptr).bytes > kStaticScratchBytes)
    return TREE_ATTN_ERR_SCRATCH;  // rejected before any HIP call
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* base = nullptr;
  rc = static_scratch(st, &base);
  if (rc != TREE_ATTN_OK) return rc;
  const Plan pl = make_plan(s, TREE_ATTN_OP_REPLAY_FWD, base);
  return run_replay_fwd(problem, s, pl, k_p, v_p, q_r, k_r, v_r, o_r, lse_r, st);
}

int tree_attn_replay_bwd(const tree_attn_problem* problem, const void* k_p, const void* v_p,
                         const void* q_r, const void* k_r, const void* v_r, const void* o_r,
                         const float* lse_r, const void* do_r, void* dq_r, void* dk_r,
                         void* dv_r, float* dk_p_seed, float* dv_p_seed, void* ws,
                         size_t ws_bytes, tree_attn_stream_t stream) {
  Shape s;
  int rc = validate_problem(problem, true, s);
  if (rc != TREE_ATTN_OK) return rc;
  if ((dk_p_seed == nullptr) != (dv_p_seed == nullptr)) return TREE_ATTN_ERR_INVALID;
  const bool seeds = dk_p_seed != nullptr;
  if (!tensor_ok(k_p, s.p_tokens) || !tensor_ok(v_p, s.p_tokens)) return TREE_ATTN_ERR_INVALID;
  if (seeds && (!tensor_ok(dk_p_seed, s.p_tokens) || !tensor_ok(dv_p_seed, s.p_tokens)))
    return TREE_ATTN_ERR_INVALID;
  for (const void* t : {q_r, k_r, v_r, o_r, static_cast<const void*>(lse_r), do_r,
                        static_cast<const void*>(dq_r), static_cast<const void*>(dk_r),
                        static_cast<const void*>(dv_r)})
    if (!tensor_ok(t, s.r_tokens)) return TREE_ATTN_ERR_INVALID;
  Plan pl;
  rc = check_ws(s, TREE_ATTN_OP_REPLAY_BWD, ws, ws_bytes, pl);
  if (rc != TREE_ATTN_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  // K-stationary list first: it also writes both padded offset arrays.
  TA_TRY(run_meta(problem, s, pl.mk, kMetaKReplay, s.k_items_replay, st));
  const bool fused = s.fused_replay && s.r_tokens > 0;
  if (fused) {
    // dQ from the dK/dV kernel: only the transposed Q and dO copies and the
    // zeroed float32 accumulator are needed
    TA_TRY(run_transpose(q_r, pl.qt, s.hq, s.hp, s, s.nb, problem->resp_cu_d, pl.mk.resp_pad,
                         s.r_pad, st));
    TA_TRY(run_transpose(do_r, pl.dot, s.hq, s.hp, s, s.nb, problem->resp_cu_d, pl.mk.resp_pad,
                         s.r_pad, st, o_r, pl.delta, s.r_tokens));
    TA_TRY(launch_zero(pl.dq_acc, s.r_tokens * s.hq * s.d, st));
  } else if (!s.fused_replay) {  // (fused with no response row: nothing to do for dQ)
    TA_TRY(run_meta(problem, s, pl.mq, kMetaQReplay, s.q_items_replay * s.col_splits_bwd, st, 0,
                    s.col_splits_bwd));
  }
  if (s.r_tokens > 0 && !fused) {
    TA_TRY(run_transpose(k_p, pl.kt_p, s.hkv, 1, s, s.ng, problem->prompt_cu_d,
                         pl.mq.prompt_pad, s.p_pad, st));
    TA_TRY(run_transpose(k_r, pl.kt_r, s.hkv, 1, s, s.nb, problem->resp_cu_d, pl.mq.resp_pad,
                         s.r_pad, st));
    TA_TRY(run_transpose(q_r, pl.qt, s.hq, s.hp, s, s.nb, problem->resp_cu_d, pl.mq.resp_pad,
                         s.r_pad, st));
    TA_TRY(run_transpose(do_r, pl.dot, s.hq, s.hp, s, s.nb, problem->resp_cu_d, pl.mq.resp_pad,
                         s.r_pad, st, o_r, pl.delta, s.r_tokens));
    DqLaunch q;
    q.q = q_r;
    q.dout = do_r;
    q.lse = lse_r;
    q.delta = pl.delta;
    q.dq = dq_r;
    q.k_a = k_p;
    q.v_a = v_p;
    q.kt_a = pl.kt_p;
    q.k_b = k_r;
    q.v_b = v_r;
    q.kt_b = pl.kt_r;
    q.items = pl.mq.items;
    q.n_items = (int)(s.q_items_replay * s.col_splits_bwd);
    q.dq_part = pl.dq_part;
    q.hq = s.hq;
    q.hkv = s.hkv;
    q.hp = s.hp;
    q.d = s.d;
    q.dtype = s.dtype;
    q.lse_stride = (int)s.r_tokens;
    q.kt_a_stride = (int)s.p_pad;
    q.kt_b_stride = (int)s.r_pad;
    q.scale = problem->softmax_scale;
    TA_TRY(launch_dq(q, st));
    if (pl.dq_part)
      TA_TRY(launch_sum_parts(pl.dq_part, s.col_splits_bwd, s.r_tokens * s.hq * s.d, dq_r, s.dtype,
                              st));
  }
  if (s.r_tokens > 0 || (seeds && s.p_tokens > 0)) {
    DkvLaunch k;
    k.k = k_r;
    k.v = v_r;
    k.k_prompt = k_p;
    k.v_prompt = v_p;
    k.q = q_r;
    k.dout = do_r;
    k.qt = pl.qt;
    k.dot = pl.dot;
    k.lse = lse_r;
    k.delta = pl.delta;
    k.seg_cu = problem->resp_cu_d;
    k.seg_pad = pl.mk.resp_pad;
    k.dk = dk_r;
    k.dv = dv_r;
    k.dk_seed = dk_p_seed;
    k.dv_seed = dv_p_seed;
    k.part_k = pl.part_k;
    k.part_v = pl.part_v;
    k.items = pl.mk.items;
    k.n_items = (int)s.k_items_replay;
    k.hq = s.hq;
    k.hkv = s.hkv;
    k.hp = s.hp;
    k.d = s.d;
    k.dtype = s.dtype;
    k.lse_stride = (int)s.r_tokens;
    k.qt_stride = (int)(s.r_pad * s.hp);
    k.scale = problem->softmax_scale;
    k.dq_acc = fused ? pl.dq_acc : nullptr;
    TA_TRY(launch_dkv(k, st));
    if (fused)
      TA_TRY(launch_sum_parts(pl.dq_acc, 1, s.r_tokens * s.hq * s.d, dq_r, s.dtype, st,
                              problem->softmax_scale));
    if (seeds && s.part_rows > 0) {
      SeedReduceArgs r;
      r.part_k = pl.part_k;
      r.part_v = pl.part_v;
      r.dk_seed = dk_p_seed;
      r.dv_seed = dv_p_seed;
      r.prompt_cu = problem->prompt_cu_d;
      r.split_cu = pl.mk.split_cu;
      r.part_row = pl.mk.part_row;
      r.n_groups = s.ng;
      r.tokens = (int)s.p_tokens;
      r.width = s.hkv * s.d;
      TA_TRY(launch_seed_reduce(r, st));
    }
  }
  return TREE_ATTN_OK;
}

int tree_attn_prefill_bwd(const tree_attn_problem* problem, const void* q_p, const void* k_p,
                          const void* v_p, const void* o_p, const float* lse_p,
                          const void* do_p, const float* dk_p_seed, const float* dv_p_seed,
                          void* dq_p, void* dk_p, void* dv_p, void* ws, size_t ws_bytes,
                          tree_attn_stream_t stream) {
  Shape s;
  int rc = validate_problem(problem, true, s);
  if (rc != TREE_ATTN_OK) return rc;
  if ((dk_p_seed == nullptr) != (dv_p_seed == nullptr)) return TREE_ATTN_ERR_INVALID;
  for (const void* t : {q_p, k_p, v_p, o_p, static_cast<const void*>(lse_p), do_p,
                        static_cast<const void*>(dq_p), static_cast<const void*>(dk_p),
                        static_cast<const void*>(dv_p)})
    if (!tensor_ok(t, s.p_tokens)) return TREE_ATTN_ERR_INVALID;
  if (dk_p_seed && (!tensor_ok(dk_p_seed, s.p_tokens) || !tensor_ok(dv_p_seed, s.p_tokens)))
    return TREE_ATTN_ERR_INVALID;
  Plan pl;
  rc = check_ws(s, TREE_ATTN_OP_PREFILL_BWD, ws, ws_bytes, pl);
  if (rc != TREE_ATTN_OK) return rc;
  if (s.p_tokens == 0) return TREE_ATTN_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  TA_TRY(run_meta(problem, s, pl.mk, kMetaKPrefill, s.k_items_prefill, st));
  const bool fused = s.fused_prefill;
  if (!fused) TA_TRY(run_meta(problem, s, pl.mq, kMetaQPrefill, s.q_items_prefill, st));
  if (!fused)
    TA_TRY(run_transpose(k_p, pl.kt_p, s.hkv, 1, s, s.ng, problem->prompt_cu_d, pl.mk.prompt_pad,
                         s.p_pad, st));
  TA_TRY(run_transpose(q_p, pl.qt, s.hq, s.hp, s, s.ng, problem->prompt_cu_d, pl.mk.prompt_pad,
                       s.p_pad, st));
  TA_TRY(run_transpose(do_p, pl.dot, s.hq, s.hp, s, s.ng, problem->prompt_cu_d,
                       pl.mk.prompt_pad, s.p_pad, st, o_p, pl.delta, s.p_tokens));
  if (fused) TA_TRY(launch_zero(pl.dq_acc, s.p_tokens * s.hq * s.d, st));
  DqLaunch q;
  q.q = q_p;
  q.dout = do_p;
  q.lse = lse_p;
  q.delta = pl.delta;
  q.dq = dq_p;
  q.k_a = k_p;
  q.v_a = v_p;
  q.kt_a = pl.kt_p;
  q.k_b = k_p;
  q.v_b = v_p;
  q.kt_b = pl.kt_p;
  q.items = pl.mq.items;
  q.n_items = (int)s.q_items_prefill;
  q.dq_part = nullptr;
  q.hq = s.hq;
  q.hkv = s.hkv;
  q.hp = s.hp;
  q.d = s.d;
  q.dtype = s.dtype;
  q.lse_stride = (int)s.p_tokens;
  q.kt_a_stride = (int)s.p_pad;
  q.kt_b_stride = (int)s.p_pad;
  q.scale = problem->softmax_scale;
  if (!fused) TA_TRY(launch_dq(q, st));
  DkvLaunch k;
  k.k = k_p;
  k.v = v_p;
  k.k_prompt = k_p;
  k.v_prompt = v_p;
  k.q = q_p;
  k.dout = do_p;
  k.qt = pl.qt;
  k.dot = pl.dot;
  k.lse = lse_p;
  k.delta = pl.delta;
  k.seg_cu = problem->prompt_cu_d;
  k.seg_pad = pl.mk.prompt_pad;
  k.dk = dk_p;
  k.dv = dv_p;
  k.dk_seed = const_cast<float*>(dk_p_seed);
  k.part_k = nullptr;
  k.part_v = nullptr;
  k.dv_seed = const_cast<float*>(dv_p_seed);
  k.items = pl.mk.items;
  k.n_items = (int)s.k_items_prefill;
  k.hq = s.hq;
  k.hkv = s.hkv;
  k.hp = s.hp;
  k.d = s.d;
  k.dtype = s.dtype;
  k.lse_stride = (int)s.p_tokens;
  k.qt_stride = (int)(s.p_pad * s.hp);
  k.scale = problem->softmax_scale;
  k.dq_acc = fused ? pl.dq_acc : nullptr;
  TA_TRY(launch_dkv(k, st));
  if (fused)
    TA_TRY(launch_sum_parts(pl.dq_acc, 1, s.p_tokens * s.hq * s.d, dq_p, s.dtype, st,
                            problem->softmax_scale));
  return TREE_ATTN_OK;
}

int lse_merge(int32_t num_splits, int32_t rows, int32_t heads, int32_t head_dim,
              int32_t out_dtype, const float* o_parts, const float* lse_parts, void* o_out,
              float* lse_out, tree_attn_stream_t stream) {
  if (out_dtype != TREE_ATTN_F32 && out_dtype != TREE_ATTN_BF16) return TREE_ATTN_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return TREE_ATTN_ERR_UNSUPPORTED;
  if (num_splits < 1 || rows < 0 || heads < 1) return TREE_ATTN_ERR_INVALID;
  if ((long long)num_splits * rows * heads * head_dim > (1LL << 40)) return TREE_ATTN_ERR_INVALID;
  if (rows > 0 && (!o_parts || !lse_parts || !o_out || !lse_out)) return TREE_ATTN_ERR_INVALID;
  if (rows == 0) return TREE_ATTN_OK;
  (void)hipGetLastError();
  TA_TRY(launch_lse_merge(num_splits, rows, heads, head_dim, out_dtype, o_parts, lse_parts, o_out,
                          lse_out, static_cast<hipStream_t>(stream)));
  return TREE_ATTN_OK;
}

int tree_attn_prompt_col_splits_of(const tree_attn_problem* problem, int op, int* splits) {
  if (!splits) return TREE_ATTN_ERR_INVALID;
  if (op != TREE_ATTN_OP_REPLAY_FWD && op != TREE_ATTN_OP_REPLAY_BWD) return TREE_ATTN_ERR_INVALID;
  Shape s;
  const int rc = validate_problem(problem, false, s);
  if (rc != TREE_ATTN_OK) return rc;
  *splits = op == TREE_ATTN_OP_REPLAY_FWD ? s.col_splits_fwd
            : s.fused_replay                ? 1  // no query-stationary dQ launch
                                            : s.col_splits_bwd;
  return TREE_ATTN_OK;
}

int tree_attn_prompt_tile_splits_of(const tree_attn_problem* problem, int* splits) {
  if (!splits) return TREE_ATTN_ERR_INVALID;
  Shape s;
  const int rc = validate_problem(problem, false, s);
  if (rc != TREE_ATTN_OK) return rc;
  *splits = (int)s.n_splits;
  return TREE_ATTN_OK;
}

int tree_attn_dq_strategy_of(const tree_attn_problem* problem, int op, int* strategy) {
  if (!strategy) return TREE_ATTN_ERR_INVALID;
  if (op != TREE_ATTN_OP_REPLAY_BWD && op != TREE_ATTN_OP_PREFILL_BWD) return TREE_ATTN_ERR_INVALID;
  Shape s;
  const int rc = validate_problem(problem, false, s);
  if (rc != TREE_ATTN_OK) return rc;
  const bool fused = op == TREE_ATTN_OP_REPLAY_BWD ? s.fused_replay : s.fused_prefill;
  *strategy = fused ? TREE_ATTN_DQ_FUSED : TREE_ATTN_DQ_SEPARATE;
  return TREE_ATTN_OK;
}

int tree_attn_set_kernel_events(int kind, void* start_event, void* stop_event) {
  if (kind < 0 || kind > 2) return TREE_ATTN_ERR_INVALID;
  if ((start_event == nullptr) != (stop_event == nullptr)) return TREE_ATTN_ERR_INVALID;
  g_events[kind][0] = static_cast<hipEvent_t>(start_event);
  g_events[kind][1] = static_cast<hipEvent_t>(stop_event);
  return TREE_ATTN_OK;
}

int tree_attn_last_hip_error(void) { return static_cast<int>(g_last_hip); }

const char* tree_attn_error_string(int code) {
  switch (code) {
    case TREE_ATTN_OK: return "ok";
    case TREE_ATTN_ERR_INVALID: return "invalid argument";
    case TREE_ATTN_ERR_UNSUPPORTED: return "unsupported dtype or head_dim";
    case TREE_ATTN_ERR_WORKSPACE: return "workspace too small";
    case TREE_ATTN_ERR_HIP: return "HIP launch or runtime error";
    case TREE_ATTN_ERR_SCRATCH:
      return "problem needs more scratch than the static scratch of "
             "tree_attn_replay_fwd_noalloc (TREE_ATTN_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
