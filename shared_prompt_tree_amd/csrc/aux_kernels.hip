// Auxiliary kernels: the device-side work lists, transposed copies, the
// backward row dot product, and the standalone partial-state merge.
#include "device_common.h"
#include "grid_math.h"
#include "launch.h"

namespace treeattn {

// ------------------------------------------------------------ work lists
//
// One workgroup derives every tile of a launch from the device offset arrays.
// Tiles are ordered segment by segment, longest segment first (in the
// spirit of the largest-first unit assignment of the AugTree planner,
// section 3.4), and within a segment longest tile first.  Workgroups are
// dealt to the XCDs in this order, so the tiles of one segment run at the
// same time on the same XCD and share its keys / queries in that XCD's L2.

constexpr int kMetaThreads = 1024;
constexpr int kRankMax = 4096;  // segments ranked by length up to this count

__device__ int block_exclusive_scan(int v, int* sh) {
  // sh: kMetaThreads ints.  Returns the exclusive prefix; sh[last] holds the
  // inclusive total afterwards (read it after a barrier).
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int off = 1; off < kMetaThreads; off <<= 1) {
    const int x = t >= off ? sh[t - off] : 0;
    __syncthreads();
    sh[t] += x;
    __syncthreads();
  }
  return sh[t] - v;
}

// Writes out[i] = sum_{k<i} f(k) for i in [0, n] and returns the total.
template <typename F>
__device__ int scan_into(int n, F f, int32_t* out, int* sh) {
  int carry = 0;
  for (int base = 0; base < n; base += kMetaThreads) {
    const int i = base + threadIdx.x;
    const int v = i < n ? f(i) : 0;
    const int ex = block_exclusive_scan(v, sh);
    if (i < n) out[i] = carry + ex;
    const int tot = sh[kMetaThreads - 1];
    __syncthreads();
    carry += tot;
  }
  if (threadIdx.x == 0) out[n] = carry;
  __syncthreads();
  return carry;
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }
__device__ __forceinline__ int pad_len(int n) { return ceil_div(n, kPad) * kPad; }

__global__ __launch_bounds__(kMetaThreads) void meta_kernel(MetaArgs a) {
  __shared__ int sh[kMetaThreads];
  const int t = threadIdx.x;
  const int ng = a.n_groups, nbr = a.n_branches;
  const int32_t* pcu = a.prompt_cu;
  const int32_t* gcu = a.group_branch_cu;
  const int32_t* rcu = a.resp_cu;

  // padded offsets of every segment in the transposed copies
  scan_into(ng, [&](int g) { return pad_len(pcu[g + 1] - pcu[g]); }, a.prompt_pad, sh);
  if (a.mode == kMetaQReplay || a.mode == kMetaKReplay) {
    scan_into(nbr, [&](int i) { return pad_len(rcu[i + 1] - rcu[i]); }, a.resp_pad, sh);
    for (int g = t; g < ng; g += kMetaThreads)
      for (int i = gcu[g]; i < gcu[g + 1]; ++i) a.branch_group[i] = g;
  }
  __syncthreads();

  // Replay key-stationary lists: the prompt tiles of a group read every
  // response row of the group.  Where that is far more than a fair share of
  // the launch, the group's branches are cut into splits (contiguous branch
  // ranges with balanced row counts, at least one branch each); each split
  // of each prompt tile is its own work item writing float32 partial seeds,
  // summed afterwards in a fixed order.
  const bool ksplit = a.mode == kMetaKReplay;
  auto splits_of = [&](int g) {
    return prompt_splits(gcu[g + 1] - gcu[g], (long long)rcu[gcu[g + 1]] - rcu[gcu[g]],
                         a.split_target);
  };
  if (ksplit) {
    scan_into(ng, splits_of, a.split_cu, sh);
    scan_into(
        ng,
        [&](int g) {
          const int sg = splits_of(g);
          return sg > 1 ? sg * (pcu[g + 1] - pcu[g]) : 0;
        },
        a.part_row, sh);
    for (int g = t; g < ng; g += kMetaThreads) {
      const int sg = a.split_cu[g + 1] - a.split_cu[g];
      const int b0 = gcu[g];
      const long long rows = (long long)rcu[gcu[g + 1]] - rcu[b0];
      int i = b0;
      for (int k = 0; k < sg; ++k) {
        // first branch at or after i whose preceding rows reach k/sg of the
        // group's rows, leaving one branch for every later split
        const long long want = (rows * k + sg - 1) / sg;
        const int last = gcu[g + 1] - (sg - k);
        while (i < last && (long long)rcu[i] - rcu[b0] < want) ++i;
        a.split_first[a.split_cu[g] + k] = i;
        ++i;
      }
    }
    __syncthreads();
  }

  // Sources (segments that own tiles), their tile counts and ranking keys.
  // Replay key-stationary launches hold the prompt tiles of every group
  // (ranked first) followed by the own-branch tiles.
  const int tq = a.tile_q;
  int nsrc;
  if (a.mode == kMetaQPrefill || a.mode == kMetaKPrefill) nsrc = ng;
  else if (a.mode == kMetaQReplay) nsrc = nbr;
  else nsrc = ng + nbr;
  auto seg_len = [&](int s) -> int {
    switch (a.mode) {
      case kMetaQPrefill:
      case kMetaKPrefill: return pcu[s + 1] - pcu[s];
      case kMetaQReplay: return rcu[s + 1] - rcu[s];
      default: return s < ng ? pcu[s + 1] - pcu[s] : rcu[s - ng + 1] - rcu[s - ng];
    }
  };
  auto tiles_of = [&](int s) -> int {
    const int len = seg_len(s);
    if (a.mode == kMetaQPrefill) return ceil_div(len, tq);
    if (a.mode == kMetaQReplay) return ceil_div(len, tq) * a.col_splits;
    const int n = ceil_div(len, kTileKV);
    return (ksplit && s < ng) ? n * (a.split_cu[s + 1] - a.split_cu[s]) : n;
  };
  auto key_of = [&](int s) -> int {
    if (a.mode == kMetaKReplay && s < ng) return (1 << 30) + (ng - s);
    return seg_len(s);
  };
  // rank by decreasing key, ties by index; order[rank] = source
  for (int s = t; s < nsrc; s += kMetaThreads) {
    int rank = s;
    if (nsrc <= kRankMax) {
      const int ks = key_of(s);
      rank = 0;
      for (int u = 0; u < nsrc; ++u) {
        const int ku = key_of(u);
        rank += (ku > ks) || (ku == ks && u < s);
      }
    }
    a.src_order[rank] = s;
  }
  __syncthreads();
  int n = scan_into(nsrc, [&](int k) { return tiles_of(a.src_order[k]); }, a.src_cu, sh);
  if (n > a.cap) n = a.cap;
  const bool qmode = a.mode == kMetaQPrefill || a.mode == kMetaQReplay;
  QItem* qout = static_cast<QItem*>(a.items);
  KItem* kout = static_cast<KItem*>(a.items);
  for (int i = n + t; i < a.cap; i += kMetaThreads) {  // never leave a stale slot
    if (qmode) qout[i] = QItem{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};  // nq = 0: no work
    else kout[i] = KItem{0, 0, 0, 0, 0, 0, 0, 0, 0};
  }

  for (int i = t; i < n; i += kMetaThreads) {
    int lo = 0, hi = nsrc - 1;  // last rank with src_cu[k] <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.src_cu[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    const int s = a.src_order[lo];
    const int u = i - a.src_cu[lo];
    if (qmode) {
      // query tiles: the last tile of a causal segment reads the most keys;
      // a split replay list holds the col_splits chunks of a tile in a row
      const int nsplit = a.mode == kMetaQReplay ? a.col_splits : 1;
      const int chunk = u % nsplit;
      const int tile = tiles_of(s) / nsplit - 1 - u / nsplit;
      QItem q;
      q.chunk = chunk;
      q.pad_ = 0;
      if (a.mode == kMetaQPrefill) {
        const int plen = pcu[s + 1] - pcu[s];
        q.qpos = tile * tq;
        q.nq = min(tq, plen - q.qpos);
        q.q0 = pcu[s] + q.qpos;
        q.a0 = 0;
        q.alen = 0;
        q.apad = 0;
        q.b0 = pcu[s];
        q.blen = q.qpos + q.nq;
        q.bpad = a.prompt_pad[s];
      } else {
        const int g = a.branch_group[s];
        const int rlen = rcu[s + 1] - rcu[s];
        q.qpos = tile * tq;
        q.nq = min(tq, rlen - q.qpos);
        q.q0 = rcu[s] + q.qpos;
        // prompt chunk [k0, k1) in whole 64-key tiles
        const int plen = pcu[g + 1] - pcu[g];
        const int ptiles = ceil_div(plen, kTileK);
        const int k0 = min(plen, (int)((long long)ptiles * chunk / nsplit) * kTileK);
        const int k1 = min(plen, (int)((long long)ptiles * (chunk + 1) / nsplit) * kTileK);
        q.a0 = pcu[g] + k0;
        q.alen = k1 - k0;
        q.apad = a.prompt_pad[g] + k0;
        q.b0 = rcu[s];
        q.blen = chunk == nsplit - 1 ? q.qpos + q.nq : 0;
        q.bpad = a.resp_pad[s];
      }
      q.cost = ceil_div(q.alen, kTileK) + ceil_div(q.blen, kTileK);
      qout[i] = q;
    } else {
      // key tiles: the first tile of a causal segment is read by the most rows
      int tile = u;
      KItem k;
      k.prow = 0;
      if (a.mode == kMetaKPrefill) {
        const int plen = pcu[s + 1] - pcu[s];
        k.kpos = tile * kTileKV;
        k.nk = min(kTileKV, plen - k.kpos);
        k.k0 = pcu[s] + k.kpos;
        k.kind = 2;
        k.seg_lo = s;
        k.seg_hi = s + 1;
        k.causal = 1;
        k.cost = plen - k.kpos;
      } else if (s < ng) {  // prompt tile in replay: the branches of one split
        const int plen = pcu[s + 1] - pcu[s];
        const int ntile = ceil_div(plen, kTileKV);
        const int sg = a.split_cu[s + 1] - a.split_cu[s];
        const int split = tile / ntile;
        tile -= split * ntile;
        k.kpos = tile * kTileKV;
        k.nk = min(kTileKV, plen - k.kpos);
        k.k0 = pcu[s] + k.kpos;
        k.kind = sg > 1 ? 3 : 1;
        k.seg_lo = sg > 1 ? a.split_first[a.split_cu[s] + split] : gcu[s];
        k.seg_hi = split + 1 < sg ? a.split_first[a.split_cu[s] + split + 1] : gcu[s + 1];
        k.causal = 0;
        k.cost = rcu[k.seg_hi] - rcu[k.seg_lo];
        k.prow = a.part_row[s] + split * plen + k.kpos;
      } else {  // own-branch tile
        const int b = s - ng;
        const int rlen = rcu[b + 1] - rcu[b];
        k.kpos = tile * kTileKV;
        k.nk = min(kTileKV, rlen - k.kpos);
        k.k0 = rcu[b] + k.kpos;
        k.kind = 0;
        k.seg_lo = b;
        k.seg_hi = b + 1;
        k.causal = 1;
        k.cost = rlen - k.kpos;
      }
      kout[i] = k;
    }
  }
}

hipError_t launch_meta(const MetaArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(meta_kernel, dim3(1), dim3(kMetaThreads), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ seed reduce
//
// Prompt seeds of split groups: the splits' partial sums added in split
// order (deterministic).  One thread per 4 floats of a prompt token.
__global__ __launch_bounds__(kAuxThreads) void seed_reduce_kernel(SeedReduceArgs a) {
  const int per_tok = a.width / 4;
  const long long n = (long long)a.tokens * per_tok;
  for (long long idx = aux_first(blockIdx.x, threadIdx.x); idx < n; idx += aux_stride(gridDim.x)) {
    const int t = (int)(idx / per_tok), c = (int)(idx % per_tok) * 4;
    int lo = 0, hi = a.n_groups - 1;  // group of token t: last g with prompt_cu[g] <= t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.prompt_cu[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    const int g = lo;
    const int sg = a.split_cu[g + 1] - a.split_cu[g];
    if (sg <= 1) continue;
    const int plen = a.prompt_cu[g + 1] - a.prompt_cu[g];
    const size_t r0 = (size_t)a.part_row[g] + (t - a.prompt_cu[g]);
    f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < sg; ++k) {
      const size_t o = (r0 + (size_t)k * plen) * a.width + c;
      sk += *reinterpret_cast<const f32x4*>(a.part_k + o);
      sv += *reinterpret_cast<const f32x4*>(a.part_v + o);
    }
    const size_t o = (size_t)t * a.width + c;
    *reinterpret_cast<f32x4*>(a.dk_seed + o) = sk;
    *reinterpret_cast<f32x4*>(a.dv_seed + o) = sv;
  }
}

// ------------------------------------------------------------ chunk sums
//
// dQ of a split replay launch: the chunks' float32 shares added in chunk
// order (deterministic), written in the output dtype.  One thread per 4
// elements.
template <typename T>
__global__ __launch_bounds__(kAuxThreads) void sum_parts_kernel(const float* in, int parts,
                                                                long long n, T* out, float scale) {
  for (long long q = aux_first(blockIdx.x, threadIdx.x); q < n / 4; q += aux_stride(gridDim.x)) {
    const long long i = q * 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < parts; ++k) acc += *reinterpret_cast<const f32x4*>(in + k * n + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) out[i + e] = static_cast<T>(acc[e] * scale);
  }
}

hipError_t launch_sum_parts(const float* in, int parts, long long n, void* out, int dtype,
                            hipStream_t s, float scale) {
  if (n == 0) return hipSuccess;
  const int grid = (int)aux_blocks(n / 4);
  if (dtype == 1)
    hipLaunchKernelGGL(sum_parts_kernel<bf16>, dim3(grid), dim3(kAuxThreads), 0, s, in, parts, n,
                       static_cast<bf16*>(out), scale);
  else
    hipLaunchKernelGGL(sum_parts_kernel<float>, dim3(grid), dim3(kAuxThreads), 0, s, in, parts, n,
                       static_cast<float*>(out), scale);
  return hipGetLastError();
}

// ------------------------------------------------------------ zero fill

__global__ __launch_bounds__(kAuxThreads) void zero_kernel(float* p, long long n4) {
  for (long long q = aux_first(blockIdx.x, threadIdx.x); q < n4; q += aux_stride(gridDim.x))
    *reinterpret_cast<f32x4*>(p + 4 * q) = f32x4{0.f, 0.f, 0.f, 0.f};
}

hipError_t launch_zero(float* p, long long n, hipStream_t s) {
  // n is a multiple of 4 (whole rows of head_dim floats)
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3((int)aux_blocks(n / 4)), dim3(kAuxThreads), 0, s, p, n / 4);
  return hipGetLastError();
}

hipError_t launch_seed_reduce(const SeedReduceArgs& a, hipStream_t s) {
  const long long n = (long long)a.tokens * (a.width / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(seed_reduce_kernel, dim3((int)aux_blocks(n)), dim3(kAuxThreads), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ transpose
//
// out[hg][d][perm(col)] for 64 columns per workgroup.  Column col of head
// group hg is token u = (col - pad[s]*hp) / hp of segment s and head
// hg*hp + col % hp; padding columns are written as zeros.  Optionally (the
// dO copy of the backward) the same pass forms the row dot
// delta[h][t] = sum_c dO[t][h][c] O[t][h][c] in float32: each thread also
// loads the O chunk of its dO chunk, and the nch lanes that hold one column
// (a power of two, consecutive within a wave) add their partial sums by
// shuffles.

template <typename T>
__global__ __launch_bounds__(kAuxThreads) void transpose_kernel(TransposeArgs a) {
  constexpr int C = 64;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* tile = reinterpret_cast<T*>(smem_raw);  // [C][d + 8]
  const int ld = a.d + 8;
  const int hg = blockIdx.y;
  const int hp = a.hp;
  const T* in = static_cast<const T*>(a.in);
  const T* with = static_cast<const T*>(a.dot_with);
  T* out = static_cast<T*>(a.out);
  constexpr int CH = 16 / sizeof(T);
  const int nch = a.d / CH;
  const size_t stride = (size_t)a.pad_tokens * hp;
  const long long n_cb = stride / C;
  // column blocks, grid-stride (the whole workgroup takes the same blocks)
  for (long long cb = blockIdx.x; cb < n_cb; cb += gridDim.x) {
    const long long col0 = cb * C;
    // segment containing col0 (segments are kPad-token aligned in columns)
    int lo = 0, hi = a.n_seg - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((long long)a.seg_pad[mid] * hp <= col0) lo = mid;
      else hi = mid - 1;
    }
    const int s = lo;
    const int seg_len = a.seg_cu[s + 1] - a.seg_cu[s];
    const int u0 = (int)((col0 - (long long)a.seg_pad[s] * hp) / hp);
    // C * nch is a multiple of kAuxThreads, so every thread runs every
    // iteration (the shuffles below need all lanes)
    for (int q = threadIdx.x; q < C * nch; q += kAuxThreads) {
      const int c = q / nch, ch = q % nch;
      const int u = u0 + c / hp;
      const size_t off =
          ((size_t)(a.seg_cu[s] + (u < seg_len ? u : 0)) * a.heads + hg * hp + c % hp) * a.d +
          ch * CH;
      u32x4 v = u32x4{0, 0, 0, 0};
      if (u < seg_len) v = *reinterpret_cast<const u32x4*>(in + off);
      *reinterpret_cast<u32x4*>(tile + c * ld + ch * CH) = v;
      if (with != nullptr) {
        u32x4 wv = u32x4{0, 0, 0, 0};
        if (u < seg_len) wv = *reinterpret_cast<const u32x4*>(with + off);
        const T* x = reinterpret_cast<const T*>(&v);
        const T* y = reinterpret_cast<const T*>(&wv);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < CH; ++e) acc += to_f32(x[e]) * to_f32(y[e]);
        for (int o = nch >> 1; o > 0; o >>= 1) acc += __shfl_xor(acc, o, nch);
        if (ch == 0 && u < seg_len)
          a.dot_out[(size_t)(hg * hp + c % hp) * a.dot_tokens + a.seg_cu[s] + u] = acc;
      }
    }
    __syncthreads();
    for (int q = threadIdx.x; q < a.d * (C / CH); q += kAuxThreads) {
      const int dd = q / (C / CH), ch = q % (C / CH);
      T vals[CH];
#pragma unroll
      for (int e = 0; e < CH; ++e) {
        const int pos = ch * CH + e;                     // stored position in the 64 columns
        const int src = (pos & ~15) | perm16(pos & 15);  // column held there
        vals[e] = tile[src * ld + dd];
      }
      *reinterpret_cast<u32x4*>(out + ((size_t)hg * a.d + dd) * stride + col0 + ch * CH) =
          *reinterpret_cast<const u32x4*>(vals);
    }
    __syncthreads();  // the tile is refilled by the next column block
  }
}

hipError_t launch_transpose(const TransposeArgs& a, int dtype, hipStream_t s) {
  const int cols = a.pad_tokens * a.hp;
  if (cols == 0) return hipSuccess;
  // one workgroup per 64 columns, up to the cap of a dispatch
  const long long blocks = (long long)cols / 64;
  dim3 grid((unsigned)(blocks < kAuxMaxBlocks ? blocks : kAuxMaxBlocks), a.heads / a.hp);
  const size_t esz = dtype == 1 ? 2 : 4;
  const size_t smem = 64 * (size_t)(a.d + 8) * esz;
  if (dtype == 1) hipLaunchKernelGGL(transpose_kernel<bf16>, grid, dim3(kAuxThreads), smem, s, a);
  else hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(kAuxThreads), smem, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ lse_merge
// Partial states (O_k normalised, LSE_k): LSE = ln sum_k exp(LSE_k),
// O = sum_k exp(LSE_k - LSE) O_k (AugTree paper, section 3.3 and Fig. 8).
// 16 lanes per (row, head), 8 (d = 128) or 4 (d = 64) elements per lane.

template <typename T>
__global__ __launch_bounds__(kAuxThreads) void lse_merge_kernel(int splits, int rows, int heads,
                                                                int d, const float* o_parts,
                                                                const float* lse_parts, T* o_out,
                                                                float* lse_out) {
  const long long n = (long long)rows * heads * 16;
  for (long long gid = aux_first(blockIdx.x, threadIdx.x); gid < n; gid += aux_stride(gridDim.x)) {
    const long long item = gid / 16;
    const int part = (int)(gid % 16);
    const long long r = item / heads, h = item % heads;
    const size_t lstride = (size_t)heads * rows;
    const size_t li = (size_t)h * rows + r;
    float mx = -INFINITY;
    for (int k = 0; k < splits; ++k) mx = fmaxf(mx, lse_parts[k * lstride + li]);
    const int per = d / 16;  // elements per lane
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float wsum = 0.f;
    if (mx != -INFINITY) {
      const size_t ostride = (size_t)rows * heads * d;
      const size_t ob = ((size_t)r * heads + h) * d + part * per;
      for (int k = 0; k < splits; ++k) {
        const float lk = lse_parts[k * lstride + li];
        const float wk = lk == -INFINITY ? 0.f : fast_exp2((lk - mx) * kLog2e);
        wsum += wk;
        if (wk != 0.f) {
          const float* src = o_parts + k * ostride + ob;
          for (int e = 0; e < per; ++e) acc[e] += wk * src[e];
        }
      }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    T* dst = o_out + ((size_t)r * heads + h) * d + part * per;
    for (int e = 0; e < per; ++e) dst[e] = from_f32<T>(acc[e] * inv);
    if (part == 0) lse_out[li] = mx == -INFINITY ? -INFINITY : mx + fast_log2(wsum) * kLn2;
  }
}

hipError_t launch_lse_merge(int splits, int rows, int heads, int d, int out_dtype,
                            const float* o_parts, const float* lse_parts, void* o_out,
                            float* lse_out, hipStream_t s) {
  const long long n = (long long)rows * heads * 16;
  if (n == 0) return hipSuccess;
  const int grid = (int)aux_blocks(n);
  if (out_dtype == 1)
    hipLaunchKernelGGL(lse_merge_kernel<bf16>, dim3(grid), dim3(kAuxThreads), 0, s, splits, rows, heads,
                       d, o_parts, lse_parts, static_cast<bf16*>(o_out), lse_out);
  else
    hipLaunchKernelGGL(lse_merge_kernel<float>, dim3(grid), dim3(kAuxThreads), 0, s, splits, rows, heads,
                       d, o_parts, lse_parts, static_cast<float*>(o_out), lse_out);
  return hipGetLastError();
}

}  // namespace treeattn
