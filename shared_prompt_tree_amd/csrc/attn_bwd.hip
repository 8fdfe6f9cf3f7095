// Attention backward for gfx950 (AugTree paper, section 3.2, "Exact
// many-to-one backward", Eq. 2).
//
// With P = exp(scale * Q K^T - LSE), D = rowsum(dO * O), dP = dO V^T and
// dS = P * (dP - D):  dQ = scale * dS K,  dK = scale * dS^T Q,  dV = P^T dO.
//
// dkv_kernel is key-stationary.  A workgroup (8 waves x 32 keys) owns 256 keys
// of one kv head, keeps them on chip, and loops over every
// query row that reads them, for all query heads of that kv head.  For a
// prompt tile in replay that is every response row of every branch of the
// group, so the sum over branches of Eq. 2 happens in the accumulators and
// the float32 seeds are written once, without atomics.  (Where one group's
// response rows are far more than a fair share of the launch, its branches
// are cut into a few ranges, each writing a partial sum that a small kernel
// adds in a fixed order.)  Query rows stream
// through LDS in blocks of 32, double buffered; Q^T and dO^T come from
// pre-transposed copies so that every operand is read with 16-byte LDS
// loads.
//
// dq_kernel is query-stationary, tiled like the forward kernel: 8 waves x 32
// query rows, keys streamed in tiles of 64 from segment A (no mask) and then
// segment B (causal).  It recomputes P and dP per tile and accumulates
// dQ^T += K^T dS^T with K^T read from a pre-transposed copy.
#include <hip/hip_ext.h>

#include "device_common.h"
#include "launch.h"

namespace treeattn {

// ------------------------------------------------------------------ dQ

template <typename T, int D>
struct DqArgs {
  const T* q;
  const T* dout;
  const float* lse;
  const float* delta;
  T* dq;
  const T* k_a;
  const T* v_a;
  const T* kt_a;
  const T* k_b;
  const T* v_b;
  const T* kt_b;
  const QItem* items;
  int n_items;
  int hq, hkv, hp, n_hg;
  int lse_stride;
  int kt_a_stride, kt_b_stride;
  float scale_log2, scale;
  float* dq_part;  // split prompt column: [chunks][tokens][hq][D] float32, or null
};

// KB 32-key blocks per step: 2 (64 keys), or 1 where two double-buffered
// stages of K, V and K^T would not fit in LDS (float32 at head_dim 128).
template <typename T, int D, int KB>
__global__ __launch_bounds__(512) void dq_kernel(DqArgs<T, D> a) {
  constexpr int NT = 512, KT = 32 * KB, CH = ChunkOf<T>::kElems;
  constexpr int NCHK = D / CH, NCHT = KT / CH;
  constexpr int KROW = tile_row_elems<T, NCHK>(), TROW = tile_row_elems<T, NCHT>();
  constexpr int KTILE = tile_elems<T, KT, NCHK>();  // K or V tile (with slack)
  constexpr int STAGE = 2 * KTILE + tile_elems<T, D, NCHT>();
  constexpr int NKK = D / 16, NDB = D / 32;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* smem = reinterpret_cast<T*>(smem_raw);

  int item_idx, hg;
  if (!xcd_map(blockIdx.x, a.n_items, a.n_hg, item_idx, hg)) return;
  const QItem it = a.items[item_idx];
  if (it.nq <= 0) return;
  const int kv = (hg * a.hp) / (a.hq / a.hkv);

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int lr = l & 31, lh = l >> 5;
  const int row = 32 * w + lr;
  const int tok = row / a.hp;
  const int head = hg * a.hp + (row % a.hp);
  const bool qvalid = tok < it.nq;

  Frag<T> qf[NKK], gf[NKK];
  float lse2 = INFINITY, dl = 0.f;
  {
    const size_t off = ((size_t)(it.q0 + (qvalid ? tok : 0)) * a.hq + head) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (qvalid) {
        load_frag(qf[kk], a.q + off + 16 * kk + 8 * lh);
        load_frag(gf[kk], a.dout + off + 16 * kk + 8 * lh);
      } else {
        qf[kk].v = {};
        gf[kk].v = {};
      }
    }
    if (qvalid) {
      const size_t li = (size_t)head * a.lse_stride + it.q0 + tok;
      lse2 = a.lse[li] * kLog2e;
      dl = a.delta[li];
    }
  }

  const int na = (it.alen + KT - 1) / KT;
  const int nb = (it.blen + KT - 1) / KT;
  const int total = na + nb;
  const size_t kv_stride = (size_t)a.hkv * D;

  // Tile j into LDS stage j % 2: K and V rows (keys past the segment are
  // clamped to its last key and masked later) and K^T rows (padded copy).
  auto gload = [&](int j) {
    const bool inA = j < na;
    const int ks = (inA ? j : j - na) * KT;
    const size_t base = (size_t)((inA ? it.a0 : it.b0) + ks) * kv_stride + kv * D;
    const T* kb = (inA ? a.k_a : a.k_b) + base;
    const T* vb = (inA ? a.v_a : a.v_b) + base;
    const int klast = (inA ? it.alen : it.blen) - 1 - ks;
    const int tstride = inA ? a.kt_a_stride : a.kt_b_stride;
    const T* tb = (inA ? a.kt_a + (size_t)kv * D * a.kt_a_stride + it.apad
                       : a.kt_b + (size_t)kv * D * a.kt_b_stride + it.bpad) + ks;
    T* ks_ = smem + (j & 1) * STAGE;
    auto krow = [&](int r) { return min(r, klast) * (int)kv_stride; };
    g2l_tile<T, KT, NCHK, NT>(ks_, kb, krow);
    g2l_tile<T, KT, NCHK, NT>(ks_ + KTILE, vb, krow);
    g2l_tile<T, D, NCHT, NT>(ks_ + 2 * KTILE, tb, [&](int r) { return r * tstride; });
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  // The dP accumulators start at -D of this lane's row, so the products give
  // dP - D directly.  (float32 at head_dim 128 has no 16 registers to spare
  // for the starting block and subtracts D afterwards.)
  constexpr bool kNegD = !(sizeof(T) == 4 && D == 128);
  f32x16 negd;
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) negd[jj] = kNegD ? -dl : 0.f;
  const float c2 = a.scale_log2;
  const int wave_tok0 = (32 * w) / a.hp;

  if (total > 0) gload(0);
  wait_vmem();
  __syncthreads();
  for (int j = 0; j < total; ++j) {
    if (j + 1 < total) gload(j + 1);
    const T* ks_ = smem + (j & 1) * STAGE;
    const T* vs_ = ks_ + KTILE;
    const T* ts_ = vs_ + KTILE;

    f32x16 s[KB], dp[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = negd;
      const int kr = 32 * kb + lr;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        Frag<T> kf, vf;
        lds_frag(kf, ks_, kr, KROW, 16 * kk + 8 * lh);
        lds_frag(vf, vs_, kr, KROW, 16 * kk + 8 * lh);
        mma(s[kb], kf, qf[kk]);
        mma(dp[kb], vf, gf[kk]);
      }
    }
    const bool inA = j < na;
    const int kst0 = (inA ? j : j - na) * KT;
    const bool need_mask = inA ? (kst0 + KT > it.alen) : (kst0 + KT - 1 > it.qpos + wave_tok0);
    // Causal mask, only on tiles that cross it: hidden scores become -inf,
    // so their P is exactly 0 below.
    if (need_mask) {
      const int lim = inA ? it.alen - 1 : it.qpos + tok;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const int key = kst0 + 32 * kb + 8 * (jj >> 2) + 4 * lh + (jj & 3);
          if (key > lim) s[kb][jj] = -INFINITY;
        }
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const float p = fast_exp2(s[kb][jj] * c2 - lse2);
        s[kb][jj] = p * (kNegD ? dp[kb][jj] : dp[kb][jj] - dl);
      }
    Frag<T> sf[KB][2];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) to_frag(sf[kb][hf], s[kb], 8 * hf);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int tr = 32 * db + lr;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          Frag<T> tf;
          lds_frag(tf, ts_, tr, TROW, 16 * (2 * kb + hf) + 8 * lh);
          mma(acc[db], tf, sf[kb][hf]);
        }
    }
    wait_vmem();
    __syncthreads();
  }

  if (!qvalid) return;
  if (a.dq_part != nullptr) {
    // one chunk of a split prompt column: its float32 share of dQ
    float* prow = a.dq_part +
                  (((size_t)it.chunk * a.lse_stride + it.q0 + tok) * a.hq + head) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[db][4 * g4 + e] * a.scale;
        *reinterpret_cast<f32x4*>(prow + 32 * db + 8 * g4 + 4 * lh) = v;
      }
    return;
  }
  T* drow = a.dq + ((size_t)(it.q0 + tok) * a.hq + head) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * db + 8 * g4 + 4 * lh;
      if constexpr (sizeof(T) == 2) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = static_cast<bf16>(acc[db][4 * g4 + e] * a.scale);
        *reinterpret_cast<bf16x4*>(drow + d0) = v;
      } else {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[db][4 * g4 + e] * a.scale;
        *reinterpret_cast<f32x4*>(drow + d0) = v;
      }
    }
}

// ------------------------------------------------------------------ dK dV

template <typename T, int D>
struct DkvArgs {
  const T* k;
  const T* v;
  const T* k_prompt;
  const T* v_prompt;
  const T* q;
  const T* dout;
  const T* qt;
  const T* dot;
  const float* lse;
  const float* delta;
  const int32_t* seg_cu;
  const int32_t* seg_pad;
  T* dk;
  T* dv;
  float* dk_seed;
  float* dv_seed;
  float* part_k;
  float* part_v;
  float* dq_acc;  // fused variant: float32 dQ / scale accumulated by atomics [tokens][hq][D]
  const KItem* items;
  int n_items;
  int hq, hkv, hp, nsub;
  int lse_stride, qt_stride;
  float scale_log2, scale;
};

// Fused variant: the resident K tile is stored without padding, 16 chunks
// per key, chunk c of key r at position c ^ kswz(r).  Sixteen consecutive
// keys read at one chunk (the score phase) land on sixteen different chunk
// positions, and so do the 4 keys x 2 chunks of one transposing read group
// (the dQ phase): no bank conflicts, and the 4 KB of padding are free for
// the dS exchange buffer.
__device__ __forceinline__ int kswz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

// Copy ROWS keys x 16 chunks into the swizzled layout (global_load_lds, as
// g2l_tile; LDS chunk p holds chunk (p % 16) ^ kswz(p / 16) of key p / 16).
template <typename T, int ROWS, int NT, typename RowOff>
__device__ __forceinline__ void g2l_tile_swz(T* tile, const T* base, RowOff row_off) {
  constexpr int CH = 16 / sizeof(T), NCH = 16, NCHUNK = ROWS * NCH;
  static_assert(NCHUNK % NT == 0, "whole wave copies");
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t tile_lds = (uint32_t)(uintptr_t)tile;
#pragma unroll
  for (int i = 0; i < NCHUNK / NT; ++i) {
    const int p0 = i * NT + 64 * w;
    const int p = p0 + lane;
    const int q = p / NCH;
    const int c = (p % NCH) ^ kswz(q);
    const uint32_t off = ((uint32_t)row_off(q) + (uint32_t)(c * CH)) * (uint32_t)sizeof(T);
    dma_16(base, off, tile_lds + (uint32_t)p0 * 16u);
  }
}

// Key-stationary dK/dV.  A workgroup of NW = 8 waves owns 32 * NW keys of one
// kv head; wave w owns keys [32w, 32w + 32).  Inside a wave the VALU work
// of a query block (exponentials, dS) is issued between MFMAs that do not
// depend on it; the second wave on each SIMD fills the remaining gaps.  V of the
// wave's keys stays in registers; for bf16 the K tile stays in LDS for the
// whole loop (registers would not fit two waves per SIMD), for float32 K
// stays in registers.  Query blocks of 32 rows (Q, dO, Q^T, dO^T, LSE, D)
// stream through LDS, double buffered.
//
// FUSED (bf16, head_dim 128): the same kernel also forms dQ from the dS it
// already holds, so S and dP are computed once per pair (five products
// instead of seven).  Each wave writes its dS^T block to an LDS buffer; after
// a barrier, four waves (one per SIMD, alternating halves of the workgroup
// from block to block) each multiply dS [32 rows x 256 keys] by K [256 keys
// x 32 columns of d], reading K^T fragments with transposing LDS reads from
// the resident K tile, and add the result to a float32 dQ accumulator with
// atomics (summed over key tiles in no fixed order: dQ is not bit-identical
// from run to run).
template <typename T, int D, bool FUSED = false>
__global__ __launch_bounds__(512) void dkv_kernel(DkvArgs<T, D> a) {
  constexpr int NW = 8, NT = 64 * NW, QB = 32, CH = ChunkOf<T>::kElems;
  static_assert(!FUSED || (sizeof(T) == 2 && D == 128), "fused variant: bf16, head_dim 128");
  constexpr bool KLDS = sizeof(T) == 2;
  constexpr int NCHQ = D / CH, NCHT = QB / CH;
  constexpr int QROW = tile_row_elems<T, NCHQ>(), TROW = tile_row_elems<T, NCHT>();
  constexpr int QTILE = tile_elems<T, QB, NCHQ>();  // Q or dO block
  constexpr int TTILE = tile_elems<T, D, NCHT>();   // Q^T or dO^T block
  constexpr int STAGE = 2 * QTILE + 2 * TTILE;      // Q, dO, Q^T, dO^T
  // resident K tile (padded rows; the fused variant swizzled, unpadded)
  constexpr int KTILE = !KLDS ? 0 : FUSED ? 32 * NW * D : tile_elems<T, 32 * NW, NCHQ>();
  constexpr int NKK = D / 16, NDB = D / 32;
  constexpr int DSROW = 32 * NW + CH;  // fused: dS buffer row, 256 keys + one padding chunk
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* smem = reinterpret_cast<T*>(smem_raw);
  T* ktile = smem + 2 * STAGE;
  float* fsm = reinterpret_cast<float*>(ktile + KTILE);  // [2][2][QB] lse2, delta
  T* dsb = reinterpret_cast<T*>(fsm + 4 * QB);           // fused: dS [QB rows][DSROW]

  int item_idx, kv;
  if (!xcd_map(blockIdx.x, a.n_items, a.hkv, item_idx, kv)) return;
  const KItem it = a.items[item_idx];
  if (it.nk <= 0) return;
  // Detached prompt: no seeds to form.  (The fused variant still walks the
  // prompt tiles: their dS feeds dQ of the response rows.)
  const bool no_seeds = (it.kind == 1 || it.kind == 3) && a.dk_seed == nullptr;
  if (!FUSED && no_seeds) return;
  const T* ksrc = it.kind == 0 ? a.k : a.k_prompt;
  const T* vsrc = it.kind == 0 ? a.v : a.v_prompt;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int lr = l & 31, lh = l >> 5;
  const int hp = a.hp;
  const int tpb = QB / hp;  // query tokens per block
  const size_t kv_stride = (size_t)a.hkv * D;

  // V (and for float32 also K) of this lane's key, kept for the whole loop.
  Frag<T> vf[NKK];
  Frag<T> kf[KLDS ? 1 : NKK];
  {
    const int key = 32 * w + lr;
    const bool ok = key < it.nk;
    const size_t off = (size_t)(it.k0 + (ok ? key : 0)) * kv_stride + kv * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (ok) load_frag(vf[kk], vsrc + off + 16 * kk + 8 * lh);
      else vf[kk].v = {};
      if constexpr (!KLDS) {
        if (ok) load_frag(kf[kk], ksrc + off + 16 * kk + 8 * lh);
        else kf[kk].v = {};
      }
    }
  }
  if constexpr (KLDS) {
    // resident K tile [32*NW keys][D]; keys past the tile end are clamped
    const T* kb = ksrc + (size_t)it.k0 * kv_stride + kv * D;
    auto kro = [&](int r) { return min(r, it.nk - 1) * (int)kv_stride; };
    if constexpr (FUSED) g2l_tile_swz<T, 32 * NW, NT>(ktile, kb, kro);
    else g2l_tile<T, 32 * NW, NCHQ, NT>(ktile, kb, kro);
  }

  // Query block cursor: head sub-group hs, segment seg, block blk.  Blocks
  // are visited from the last one backwards, so the key tiles of a segment
  // that run at the same time (they start together, see the work-list
  // order) read the same query blocks at the same time and share them in
  // L2.  A causal tile stops at the block holding its first key.
  struct Cur {
    int hs, seg, blk, blk_lo, q0, nq, qpad;
  };
  // The offsets are read into scalar registers at once, so waiting for
  // them never waits for global-to-LDS copies issued later.
  auto seg_init = [&](Cur& c) {
    c.q0 = __builtin_amdgcn_readfirstlane(a.seg_cu[c.seg]);
    c.nq = __builtin_amdgcn_readfirstlane(a.seg_cu[c.seg + 1]) - c.q0;
    c.qpad = __builtin_amdgcn_readfirstlane(a.seg_pad[c.seg]);
    c.blk = (c.nq + tpb - 1) / tpb - 1;
    c.blk_lo = it.causal ? (it.kpos / tpb) : 0;
  };
  auto settle = [&](Cur& c) -> bool {  // move to the next non-empty block
    while (true) {
      if (c.hs < 0) return false;
      if (c.seg >= it.seg_lo && c.blk >= c.blk_lo) return true;
      if (c.seg >= it.seg_lo) --c.seg;
      if (c.seg < it.seg_lo) {
        c.seg = it.seg_hi - 1;
        --c.hs;
        if (c.hs < 0 || it.seg_lo >= it.seg_hi) return false;
      }
      seg_init(c);
    }
  };

  // Query block -> LDS stage: Q and dO rows (tokens past the segment are
  // clamped to its last token; their LSE is +inf so they add nothing), Q^T
  // and dO^T rows (padded copies), and LSE*log2(e) and D through registers.
  float lst = 0.f;
  bool lvalid = false;
  auto gload = [&](const Cur& c, int stage) {
    const int hg = kv * a.nsub + c.hs;
    const int tok0 = c.blk * tpb;
    const int last = c.nq - 1;
    T* qs = smem + stage * STAGE;
    const size_t qoff = ((size_t)(c.q0 + tok0) * a.hq + (size_t)hg * hp) * D;
    const int rows_left = last - tok0;
    auto qrow = [&](int r) { return min(r / hp, rows_left) * a.hq * D + (r % hp) * D; };
    g2l_tile<T, QB, NCHQ, NT>(qs, a.q + qoff, qrow);
    g2l_tile<T, QB, NCHQ, NT>(qs + QTILE, a.dout + qoff, qrow);
    const size_t tb = (size_t)hg * D * a.qt_stride + (size_t)c.qpad * hp + (size_t)c.blk * QB;
    auto trow = [&](int r) { return r * a.qt_stride; };
    g2l_tile<T, D, NCHT, NT>(qs + 2 * QTILE, a.qt + tb, trow);
    g2l_tile<T, D, NCHT, NT>(qs + 2 * QTILE + TTILE, a.dot + tb, trow);
    // The raw value is only used in lstore at the end of the block, so the
    // wait for this load does not hold up the block's LDS reads.
    if (tid < 2 * QB) {
      const int r = tid & (QB - 1);
      const int tok = tok0 + r / hp;
      lvalid = tok < c.nq;
      const size_t li =
          (size_t)(hg * hp + (r % hp)) * a.lse_stride + c.q0 + (lvalid ? tok : c.nq - 1);
      lst = tid < QB ? a.lse[li] : a.delta[li];
    }
  };
  // LSE is kept as LSE * log2(e) and D as -D (the starting value of the
  // dP accumulator, so the products give dP - D); rows past the segment get
  // LSE = +inf (P = 0) and D = 0.
  auto lstore = [&](int stage) {
    if (tid < 2 * QB)
      fsm[stage * 2 * QB + tid] =
          tid < QB ? (lvalid ? lst * kLog2e : INFINITY) : (lvalid ? -lst : 0.f);
  };

  f32x16 dka[NDB], dva[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dka[db] = f32x16{};
    dva[db] = f32x16{};
  }
  const float c2 = a.scale_log2;
  const int key_loc = it.kpos + 32 * w + lr;  // this lane's key, segment position
  const int wave_kmin = it.kpos + 32 * w;     // smallest key position of the wave
  const int wave_kmax = wave_kmin + 31;
  const bool wave_has_keys = 32 * w < it.nk;
  const int krow = 32 * w + lr;               // this lane's row of the K tile
  const bool key_ok = krow < it.nk;
  int bpar = 0;  // fused: which half of the workgroup forms dQ for this block

  Cur cur{a.nsub - 1, it.seg_hi - 1, 0, 0, 0, 0, 0};
  bool have = false;
  if (it.seg_lo < it.seg_hi) {
    seg_init(cur);
    have = settle(cur);
  }
  if (have) {
    gload(cur, 0);
    lstore(0);
  }
  wait_vmem();
  __syncthreads();
  int stage = 0;
  while (have) {
    Cur nxt = cur;
    --nxt.blk;
    const bool more = settle(nxt);
    if (more) gload(nxt, stage ^ 1);
    const T* qs = smem + stage * STAGE;
    const T* gs = qs + QTILE;
    const T* tqs = gs + QTILE;
    const T* tgs = tqs + TTILE;
    const float* lse_s = fsm + stage * 2 * QB;
    const float* del_s = lse_s + QB;
    const int tok0 = cur.blk * tpb;
    // A causal block whose last row precedes every key of this wave adds
    // nothing to it.
    const bool skip = !wave_has_keys || (it.causal && tok0 + tpb - 1 < wave_kmin);
    if (!skip) {
      // Four MFMA phases; each VALU step runs beside MFMAs that do not
      // depend on it:  S = Q K^T;  dP = dO V^T beside P = exp(S - LSE);
      // dV += P^T dO beside dS = P (dP - D);  dK += dS^T Q.
      // s: lane l, register jj -> query row 8*(jj/4) + 4*lh + jj%4, key lr.
      f32x16 s = f32x16{}, dp = f32x16{};
      Frag<T> fa[2], fb[2];
      // S = Q K^T (operand loads one step ahead)
      auto sload = [&](int kk, int slot) {
        lds_frag(fa[slot], qs, lr, QROW, 16 * kk + 8 * lh);
        if constexpr (FUSED) {
          int ko = krow;  // recomputed per read, not kept across the loop
          asm volatile("" : "+v"(ko));
          load_frag(fb[slot], ktile + ko * D + (((2 * kk + lh) ^ kswz(ko)) << 3));
        }
        else if constexpr (KLDS)
          lds_frag(fb[slot], ktile, krow, QROW, 16 * kk + 8 * lh);
      };
      sload(0, 0);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        if (kk + 1 < NKK) sload(kk + 1, (kk + 1) & 1);
        if constexpr (KLDS) mma(s, fa[kk & 1], fb[kk & 1]);
        else mma(s, fa[kk & 1], kf[kk]);
      }
      // Causal mask, only on blocks that cross it: row r (token tok0 + r/hp)
      // is hidden from this lane's key iff r < (key - tok0) * hp, i.e.
      // 8*(jj/4) + jj%4 < row_lim; hidden scores become -inf, so their P
      // (and dS) is exactly 0 below.
      if (it.causal && tok0 < wave_kmax) {
        const int row_lim = (key_loc - tok0) * hp - 4 * lh;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
          if (8 * (jj >> 2) + (jj & 3) < row_lim) s[jj] = -INFINITY;
      }
      {
        f32x4 lv;
        // dp starts at -D of its query rows (row 8*g4 + 4*lh + e in
        // register 4*g4 + e)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 nd = *reinterpret_cast<const f32x4*>(del_s + 8 * g4 + 4 * lh);
#pragma unroll
          for (int e = 0; e < 4; ++e) dp[4 * g4 + e] = nd[e];
        }
        // Phases 2-4 read one operand fragment per MFMA, from a stream of
        // NKK dO, 2*NDB dO^T and 2*NDB Q^T fragments, loaded two steps ahead.
        constexpr int NS = NKK + 4 * NDB;
        Frag<T> fr[3];
        auto oload = [&](int n) {
          if (n >= NS) return;
          Frag<T>& f = fr[n % 3];
          if (n < NKK) lds_frag(f, gs, lr, QROW, 16 * n + 8 * lh);
          else if (n < NKK + 2 * NDB) {
            const int st = n - NKK;
            lds_frag(f, tgs, 32 * (st >> 1) + lr, TROW, 16 * (st & 1) + 8 * lh);
          } else {
            const int st = n - NKK - 2 * NDB;
            lds_frag(f, tqs, 32 * (st >> 1) + lr, TROW, 16 * (st & 1) + 8 * lh);
          }
        };
        oload(0);
        oload(1);
        // dP = dO V^T beside P = exp(S * scale - LSE), two elements a step
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          oload(kk + 2);
          mma(dp, fr[kk % 3], vf[kk]);
#pragma unroll
          for (int u = 0; u < 16 / NKK; ++u) {
            const int jj = kk * (16 / NKK) + u, g4 = jj >> 2, e = jj & 3;
            if (e == 0) lv = *reinterpret_cast<const f32x4*>(lse_s + 8 * g4 + 4 * lh);
            s[jj] = fast_exp2(s[jj] * c2 - lv[e]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        Frag<T> pf[2], sf[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) to_frag(pf[hf], s, 8 * hf);
        // dV += P^T dO beside dS = P (dP - D), dp holding dP - D
#pragma unroll
        for (int st = 0; st < 2 * NDB; ++st) {  // st = 2*db + hf
          const int n = NKK + st;
          oload(n + 2);
          mma(dva[st >> 1], pf[st & 1], fr[n % 3]);
#pragma unroll
          for (int u = 0; u < 16 / (2 * NDB); ++u) {
            const int jj = st * (16 / (2 * NDB)) + u;
            dp[jj] = s[jj] * dp[jj];
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) to_frag(sf[hf], dp, 8 * hf);
        // dK += dS^T Q
#pragma unroll
        for (int st = 0; st < 2 * NDB; ++st) {
          const int n = NKK + 2 * NDB + st;
          oload(n + 2);
          mma(dka[st >> 1], sf[st & 1], fr[n % 3]);
        }
        if constexpr (FUSED) {
          // dS of this wave's keys into the exchange buffer [row][key]
          // (keys past the tile end are 0: their clamped K rows must add
          // nothing to dQ)
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) {
            const int r = 8 * (jj >> 2) + 4 * lh + (jj & 3);
            dsb[r * DSROW + krow] = key_ok ? sf[jj >> 3].v[jj & 7] : static_cast<T>(0.f);
          }
        }
      }
    }
    if constexpr (FUSED) {
      if (skip) {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
          dsb[(8 * (jj >> 2) + 4 * lh + (jj & 3)) * DSROW + krow] = static_cast<T>(0.f);
      }
      // The next stage's LSE / D row is stored before the atomics below, so
      // the wait for its global load cannot also wait for them.
      if (more) lstore(stage ^ 1);
      // every wave's dS is in LDS before the dQ products read it
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if ((w >> 2) == bpar) {
        // dQ[32 rows][32 db .. 32 db + 31] += dS[32 rows][256 keys] K[256 keys][...]
        // A: dS row lr, keys 16 ks + 8 lh .. +7 (16-byte read);
        // B: K^T, two transposing reads of keys 16 ks + 8 lh + 4 t .. +3 for
        //    column 32 db + (l % 32) (lane l of a 16-lane group reads key
        //    key0 + l16 / 4, columns 4 (l16 % 4) .. +3 of its half of the block)
        // Lane-derived addresses are recomputed here from an opaque copy of
        // the lane index rather than kept across the block loop (registers
        // are full there).
        int lo = l;
        asm volatile("" : "+v"(lo));
        const int lro = lo & 31, lho = lo >> 5;
        const int db = w & 3, l16 = lo & 15, g1 = (lo >> 4) & 1;
        const int kr0 = 8 * lho + (l16 >> 2);
        const int dcol = 32 * db + 16 * g1 + 4 * (l16 & 3);
        const int off0 = kr0 * D + ((((dcol >> 3) ^ kswz(kr0)) << 3) | (dcol & 7));
        const int off1 = (kr0 + 4) * D + ((((dcol >> 3) ^ kswz(kr0 + 4)) << 3) | (dcol & 7));
        const T* arow = dsb + lro * DSROW + 8 * lho;
        f32x16 qacc = f32x16{};
        Frag<T> qa[2], qb[2];
        auto dqload = [&](int ks, int slot) {
          load_frag(qa[slot], arow + 16 * ks);
          const bf16x4 b0 = lds_read_tr(ktile + 16 * ks * D + off0);
          const bf16x4 b1 = lds_read_tr(ktile + 16 * ks * D + off1);
          qb[slot].v = bf16x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        };
        // two key steps per iteration, the next pair's operands loaded while
        // this pair multiplies (a rolled loop keeps the operands in flight
        // to two pairs: the dK/dV accumulators leave no more registers)
        constexpr int NKS = (32 * NW) / 16;
        dqload(0, 0);
        dqload(1, 1);
#pragma unroll 1
        for (int ks = 0; ks < NKS; ks += 2) {
          mma(qacc, qa[0], qb[0]);
          if (ks + 2 < NKS) dqload(ks + 2, 0);
          mma(qacc, qa[1], qb[1]);
          if (ks + 3 < NKS) dqload(ks + 3, 1);
        }
        // qacc: lane l, register jj -> row 8 (jj / 4) + 4 lh + jj % 4, column
        // 32 db + lr.  Exactly 16 atomics per lane (rows past the segment add
        // 0 to its last row), so the wait below can leave them in flight.
        // Row r of the block is token tok0 + r / hp, head hg * hp + r % hp (hp
        // a power of two); the block's rows span at most 32 tokens of one
        // segment, so offsets from the block's first row fit in 32 bits.
        const int tok0 = cur.blk * tpb;
        const int hg = kv * a.nsub + cur.hs;
        const int lg = 31 - __builtin_clz(hp);
        const int tlast = cur.nq - 1 - tok0;  // last token of the segment, block-relative
        float* qb0 = a.dq_acc + ((size_t)(cur.q0 + tok0) * a.hq + (size_t)hg * hp) * D + 32 * db;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          int la = l;
          asm volatile("" : "+v"(la));
          const int r = 8 * (jj >> 2) + 4 * (la >> 5) + (jj & 3);
          const int tk = r >> lg;
          const bool ok = tk <= tlast;
          const uint32_t o = (uint32_t)(((ok ? tk : tlast) * a.hq + (r & (hp - 1))) * D + (la & 31));
          __hip_atomic_fetch_add(qb0 + o, ok ? qacc[jj] : 0.f, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    if (!FUSED && more) lstore(stage ^ 1);
    if constexpr (FUSED) {
      // Vector memory operations complete in issue order: vmcnt(16) leaves
      // only the 16 atomics just issued in flight, after the tile copies.
      if ((w >> 2) == bpar)
        asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      bpar ^= 1;
    } else {
      wait_vmem();
      __syncthreads();
    }
    cur = nxt;
    stage ^= 1;
    have = more;
  }

  if (no_seeds) return;
  // dka/dva: lane l, register jj -> key 8*(jj/4) + 4*lh + jj%4 of this wave,
  // column 32*db + lr.
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const int key = 32 * w + 8 * (jj >> 2) + 4 * lh + (jj & 3);
    if (key >= it.nk) continue;
    const size_t base = (size_t)(it.k0 + key) * kv_stride + kv * D;
    const size_t pbase = (size_t)(it.prow + key) * kv_stride + kv * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const size_t o = base + 32 * db + lr;
      float gk = dka[db][jj] * a.scale;
      float gv = dva[db][jj];
      if (it.kind == 1) {
        a.dk_seed[o] = gk;
        a.dv_seed[o] = gv;
      } else if (it.kind == 3) {
        a.part_k[pbase + 32 * db + lr] = gk;
        a.part_v[pbase + 32 * db + lr] = gv;
      } else {
        if (it.kind == 2 && a.dk_seed != nullptr) {
          gk += a.dk_seed[o];
          gv += a.dv_seed[o];
        }
        a.dk[o] = from_f32<T>(gk);
        a.dv[o] = from_f32<T>(gv);
      }
    }
  }
}

template <typename T, int D>
static hipError_t launch_dq_t(const DqLaunch& l, hipStream_t s) {
  constexpr int KB = (sizeof(T) == 4 && D == 128) ? 1 : 2;
  DqArgs<T, D> a;
  a.q = static_cast<const T*>(l.q);
  a.dout = static_cast<const T*>(l.dout);
  a.lse = l.lse;
  a.delta = l.delta;
  a.dq = static_cast<T*>(l.dq);
  a.k_a = static_cast<const T*>(l.k_a);
  a.v_a = static_cast<const T*>(l.v_a);
  a.kt_a = static_cast<const T*>(l.kt_a);
  a.k_b = static_cast<const T*>(l.k_b);
  a.v_b = static_cast<const T*>(l.v_b);
  a.kt_b = static_cast<const T*>(l.kt_b);
  a.items = static_cast<const QItem*>(l.items);
  a.n_items = l.n_items;
  a.hq = l.hq;
  a.hkv = l.hkv;
  a.hp = l.hp;
  a.n_hg = l.hq / l.hp;
  a.lse_stride = l.lse_stride;
  a.kt_a_stride = l.kt_a_stride;
  a.kt_b_stride = l.kt_b_stride;
  a.scale_log2 = l.scale * kLog2e;
  a.scale = l.scale;
  a.dq_part = l.dq_part;
  constexpr int CH = 16 / sizeof(T);
  const size_t smem = 2 * sizeof(T) *
                      (size_t)(2 * tile_elems<T, 32 * KB, D / CH>() + tile_elems<T, D, 32 * KB / CH>());
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(dq_kernel<T, D, KB>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  const int grid = xcd_grid(l.n_items, a.n_hg);
  if (grid <= 0) return hipSuccess;
  hipEvent_t e0, e1;
  kernel_events(kKernelDq, &e0, &e1);
  if (e0) hipExtLaunchKernelGGL(dq_kernel<T, D, KB>, dim3(grid), dim3(512), smem, s, e0, e1, 0, a);
  else dq_kernel<T, D, KB><<<dim3(grid), dim3(512), smem, s>>>(a);
  return hipGetLastError();
}

template <typename T, int D, bool FUSED = false>
static hipError_t launch_dkv_t(const DkvLaunch& l, hipStream_t s) {
  DkvArgs<T, D> a;
  a.k = static_cast<const T*>(l.k);
  a.v = static_cast<const T*>(l.v);
  a.k_prompt = static_cast<const T*>(l.k_prompt);
  a.v_prompt = static_cast<const T*>(l.v_prompt);
  a.q = static_cast<const T*>(l.q);
  a.dout = static_cast<const T*>(l.dout);
  a.qt = static_cast<const T*>(l.qt);
  a.dot = static_cast<const T*>(l.dot);
  a.lse = l.lse;
  a.delta = l.delta;
  a.seg_cu = l.seg_cu;
  a.seg_pad = l.seg_pad;
  a.dk = static_cast<T*>(l.dk);
  a.dv = static_cast<T*>(l.dv);
  a.dk_seed = l.dk_seed;
  a.dv_seed = l.dv_seed;
  a.part_k = l.part_k;
  a.part_v = l.part_v;
  a.items = static_cast<const KItem*>(l.items);
  a.n_items = l.n_items;
  a.hq = l.hq;
  a.hkv = l.hkv;
  a.hp = l.hp;
  a.nsub = (l.hq / l.hkv) / l.hp;
  a.lse_stride = l.lse_stride;
  a.qt_stride = l.qt_stride;
  a.scale_log2 = l.scale * kLog2e;
  a.scale = l.scale;
  a.dq_acc = l.dq_acc;
  constexpr int CH = 16 / sizeof(T);
  const size_t ktile = sizeof(T) != 2 ? 0
                       : FUSED    ? (size_t)kTileKV * D * sizeof(T)
                                  : (size_t)tile_elems<T, kTileKV, D / CH>() * sizeof(T);
  const size_t dsbuf = FUSED ? (size_t)32 * (kTileKV + CH) * sizeof(T) : 0;
  const size_t smem =
      2 * sizeof(T) * (size_t)(2 * tile_elems<T, 32, D / CH>() + 2 * tile_elems<T, D, 32 / CH>()) +
      ktile + 2 * 2 * 32 * sizeof(float) + dsbuf;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(dkv_kernel<T, D, FUSED>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  const int grid = xcd_grid(l.n_items, l.hkv);
  if (grid <= 0) return hipSuccess;
  hipEvent_t e0, e1;
  kernel_events(kKernelDkv, &e0, &e1);
  if (e0)
    hipExtLaunchKernelGGL(dkv_kernel<T, D, FUSED>, dim3(grid), dim3(512), smem, s, e0, e1, 0, a);
  else dkv_kernel<T, D, FUSED><<<dim3(grid), dim3(512), smem, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_dq(const DqLaunch& l, hipStream_t s) {
  if (l.dtype == 1) return l.d == 128 ? launch_dq_t<bf16, 128>(l, s) : launch_dq_t<bf16, 64>(l, s);
  return l.d == 128 ? launch_dq_t<float, 128>(l, s) : launch_dq_t<float, 64>(l, s);
}

hipError_t launch_dkv(const DkvLaunch& l, hipStream_t s) {
  if (l.dq_acc != nullptr) {  // fused dK/dV/dQ: bf16, head_dim 128 only (host checked)
    if (l.dtype != 1 || l.d != 128) return hipErrorInvalidValue;
    return launch_dkv_t<bf16, 128, true>(l, s);
  }
  if (l.dtype == 1) return l.d == 128 ? launch_dkv_t<bf16, 128>(l, s) : launch_dkv_t<bf16, 64>(l, s);
  return l.d == 128 ? launch_dkv_t<float, 128>(l, s) : launch_dkv_t<float, 64>(l, s);
}

}  // namespace treeattn
