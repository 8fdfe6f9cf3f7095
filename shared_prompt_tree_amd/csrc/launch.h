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
};
hipError_t launch_meta(const MetaArgs& a, hipStream_t s);

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
};
hipError_t launch_transpose(const TransposeArgs& a, int dtype, hipStream_t s);

// delta[h][t] = sum_c dout[t][h][c] * out[t][h][c] in float32.
hipError_t launch_row_dot(const void* dout, const void* out, float* delta, int tokens, int heads,
                          int d, int dtype, hipStream_t s);

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
};
hipError_t launch_dq(const DqLaunch& a, hipStream_t s);

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
  const void* items;
  int n_items;
  int hq, hkv, hp, d, dtype;
  int lse_stride;
  int qt_stride;       // columns per d row of the transposed copies
  float scale;
};
hipError_t launch_dkv(const DkvLaunch& a, hipStream_t s);

}  // namespace treeattn
