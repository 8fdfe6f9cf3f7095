// Internal launch interface between the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace treeattn {

// Timing hook: events to record around the next launches of a main kernel
// (0 forward, 1 dQ, 2 dK/dV) on this host thread; both null when unset.
enum KernelKind { kKernelFwd = 0, kKernelDq = 1, kKernelDkv = 2 };
void kernel_events(int kind, hipEvent_t* start, hipEvent_t* stop);

struct QItem;
struct KItem;

// Which work list the metadata kernel builds.
enum MetaMode { kMetaQPrefill = 0, kMetaQReplay = 1, kMetaKPrefill = 2, kMetaKReplay = 3 };

struct MetaArgs {
  int mode;
  int n_groups, n_branches;
  const int32_t* prompt_cu;
  const int32_t* group_branch_cu;
  const int32_t* resp_cu;
  int32_t* prompt_pad;    // [n_groups + 1] out: padded token offsets
  int32_t* resp_pad;      // [n_branches + 1] out
  int32_t* branch_group;  // [n_branches] out
  int32_t* src_cu;        // [n_sources + 1] scratch: tile offsets in rank order
  int32_t* src_order;     // [n_sources + 1] scratch: source of each rank
  void* items;            // [cap] out, segment-major
  int cap;                // number of items the host computed
  int tile_q;             // query tokens per query-stationary tile
  // Replay query-stationary lists only: the prompt column of every query
  // tile is cut into col_splits chunks of whole 64-key tiles (1: not split);
  // the last chunk also holds the row's own branch.
  int col_splits;
  // Replay key-stationary lists only: the prompt tiles of a group are split
  // into prompt_splits(...) ranges of its branches.
  long long split_target; // rows one split should read at most (0: no split)
  int32_t* split_cu;      // [n_groups + 1] out: prefix of splits per group
  int32_t* split_first;   // [sum of splits] out: first branch of each split
  int32_t* part_row;      // [n_groups + 1] out: first partial-seed row of a group
};
hipError_t launch_meta(const MetaArgs& a, hipStream_t s);

// Splits of the prompt key tiles of a group with `branches` branches that
// hold `rows` response tokens: enough that one split reads at most `target`
// rows, at most one per branch, at least one.  Host and device use this same
// rule.
__host__ __device__ inline int prompt_splits(int branches, long long rows, long long target) {
  if (branches <= 1 || target <= 0) return 1;
  const long long s = (rows + target - 1) / target;
  return (int)(s < 1 ? 1 : (s > branches ? branches : s));
}

// Sum of the partial prompt seeds of split groups:
// seed[t] = sum_k part[part_row[g] + k * P_g + (t - prompt_cu[g])].
struct SeedReduceArgs {
  const float* part_k;
  const float* part_v;
  float* dk_seed;
  float* dv_seed;
  const int32_t* prompt_cu;
  const int32_t* split_cu;
  const int32_t* part_row;
  int n_groups;
  int tokens;  // prompt tokens
  int width;   // hkv * d floats per token
};
hipError_t launch_seed_reduce(const SeedReduceArgs& a, hipStream_t s);

// Transposed, padded copy: out[hg][d][perm(col)] with col = pad[s]*hp +
// u*hp + j for token u of segment s and head hg*hp + j; padding columns are
// zero.  `in` is [tokens][heads][d].
struct TransposeArgs {
  const void* in;
  void* out;
  int heads, hp, d;
  int n_seg;
  const int32_t* seg_cu;
  const int32_t* seg_pad;
  int pad_tokens;  // seg_pad[n_seg], from the host
  // Optional (both null: off): while copying `in` (dO), also the backward's
  // row dot delta[h][t] = sum_c in[t][h][c] * dot_with[t][h][c] in float32,
  // delta row stride dot_tokens (the tensor's tokens).
  const void* dot_with = nullptr;
  float* dot_out = nullptr;
  int dot_tokens = 0;
};
hipError_t launch_transpose(const TransposeArgs& a, int dtype, hipStream_t s);


hipError_t launch_lse_merge(int splits, int rows, int heads, int d, int out_dtype,
                            const float* o_parts, const float* lse_parts, void* o_out,
                            float* lse_out, hipStream_t s);

struct FwdLaunch {
  const void* q;
  void* o;
  float* lse;
  const void* k_a;
  const void* vt_a;
  const void* k_b;
  const void* vt_b;
  const void* items;
  int n_items;
  int hq, hkv, hp, d, dtype;
  int lse_stride;
  int vt_a_stride, vt_b_stride;
  float scale;
  int waves;  // 8 (256 query rows per item) or 12 (384, bf16 only)
  // Split prompt column: each item writes its chunk's normalised O (float32,
  // [chunks][tokens][hq][d]) and LSE ([chunks][hq][tokens]) instead of o/lse.
  float* o_part;   // null: not split
  float* lse_part;
};
hipError_t launch_fwd(const FwdLaunch& a, hipStream_t s);

struct DqLaunch {
  const void* q;
  const void* dout;
  const float* lse;
  const float* delta;
  void* dq;
  const void* k_a;
  const void* v_a;
  const void* kt_a;
  const void* k_b;
  const void* v_b;
  const void* kt_b;
  const void* items;
  int n_items;
  int hq, hkv, hp, d, dtype;
  int lse_stride;
  int kt_a_stride, kt_b_stride;
  float scale;
  // Split prompt column: each item writes its chunk's dQ share (float32,
  // [chunks][tokens][hq][d]) instead of dq.
  float* dq_part;  // null: not split
};
hipError_t launch_dq(const DqLaunch& a, hipStream_t s);

// out[i] = scale * sum over k < parts of in[k * n + i], in the output dtype
// (0 float32, 1 bf16); the chunk partial sums of a split dQ, or (one part)
// the scaled float32 dQ accumulator of the fused backward.
hipError_t launch_sum_parts(const float* in, int parts, long long n, void* out, int dtype,
                            hipStream_t s, float scale = 1.f);

struct DkvLaunch {
  const void* k;       // own-branch keys (kind 0 tiles) [tokens][hkv][d]
  const void* v;
  const void* k_prompt;  // prompt keys (kind 1 and 2 tiles)
  const void* v_prompt;
  const void* q;       // query tensor [tokens][hq][d]
  const void* dout;
  const void* qt;      // transposed query copy [hq/hp][d][pad*hp]
  const void* dot;     // transposed dO copy
  const float* lse;    // [hq][lse_stride]
  const float* delta;  // [hq][lse_stride]
  const int32_t* seg_cu;   // query segments (token offsets)
  const int32_t* seg_pad;  // query segments (padded offsets)
  void* dk;            // kind 0/2 output [tokens][hkv][d] (I/O dtype)
  void* dv;
  float* dk_seed;      // kind 1 output / kind 2 input [tokens][hkv][d] float32
  float* dv_seed;
  float* part_k;       // kind 3 output: partial seeds [partial rows][hkv][d] float32
  float* part_v;
  const void* items;
  int n_items;
  int hq, hkv, hp, d, dtype;
  int lse_stride;
  int qt_stride;       // columns per d row of the transposed copies
  float scale;
  // Fused variant (bf16, head_dim 128): also adds dQ / scale of the query
  // rows to this float32 accumulator [tokens][hq][d] (zeroed beforehand),
  // with atomics.  Null: dK/dV only.
  float* dq_acc;
};
hipError_t launch_dkv(const DkvLaunch& a, hipStream_t s);

// Fill n floats with zero (a kernel, so that captured graphs hold no memset
// node).
hipError_t launch_zero(float* p, long long n, hipStream_t s);

}  // namespace treeattn
