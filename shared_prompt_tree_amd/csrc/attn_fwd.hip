// Query-stationary attention forward for gfx950: prompt prefill and response
// replay (AugTree paper, section 3.2, "Shared prompt prefill pass" and
// "Response replay"; tile semantics of section 2.2 / Fig. 3).
//
// One workgroup = 8 waves = 256 query rows of one head group (or, bf16 with
// enough work, 12 waves = 384 rows, three waves per SIMD).  A row is a
// (token, head) pair: the hp query heads of a token that share one kv head
// are packed next to each other, so every K/V tile staged in LDS feeds all of
// them (GQA reuse).  Each wave owns 32 rows and keeps their Q in registers.
// Keys stream through LDS in tiles of 64 (bf16: triple buffered, the tile
// loop software-pipelined in 32-key halves; float32: double buffered): first
// segment A (no mask: a replay row sees the whole prompt), then segment B
// (causal with diagonal: prefill over the prompt, or the row's own branch in
// replay).  One
// online-softmax state per row runs across both segments, so the prompt
// column and the own-branch part are merged in registers (section 3.3: the
// partial states along a query row are merged associatively).
//
// Scores are computed transposed, S^T = K Q^T, so each lane owns one query
// row and 16 keys per 32-key block: the row maximum and sum are lane-local up
// to one exchange with the other half of the wave.  The output is kept
// transposed too, O^T += V^T P^T, with V^T read from a pre-transposed copy.
#include <hip/hip_ext.h>

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace treeattn {

constexpr float kRescale = 8.0f;  // log2 units
// bf16 launches use the software-pipelined tile loop.
constexpr bool kFwdPipe = true;

template <typename T, int D>
struct FwdArgs {
  const T* q;
  T* o;
  float* lse;
  const T* k_a;
  const T* vt_a;
  const T* k_b;
  const T* vt_b;
  const QItem* items;
  int n_items;
  int hq, hkv, hp, n_hg;
  int lse_stride;
  int vt_a_stride, vt_b_stride;
  float scale_log2;
  float* o_part;    // split prompt column: [chunks][tokens][hq][D] float32, or null
  float* lse_part;  // [chunks][hq][tokens]
};

// PIPE (bf16): the tile loop runs software-pipelined in 32-key halves, with
// three LDS stages (see the PIPE branch below).
template <typename T, int D, int NW, bool PIPE = false>
__global__ __launch_bounds__(64 * NW) void fwd_kernel(FwdArgs<T, D> a) {
  constexpr int NT = 64 * NW, KT = kTileK, CH = ChunkOf<T>::kElems;
  constexpr int NSTAGE = PIPE ? 3 : 2;
  constexpr int NCHK = D / CH;        // 16-byte chunks per K row
  constexpr int NCHV = KT / CH;       // chunks per V^T row
  constexpr int KROW = tile_row_elems<T, NCHK>();  // padded row lengths
  constexpr int VROW = tile_row_elems<T, NCHV>();
  constexpr int KTILE = tile_elems<T, KT, NCHK>();  // K tile (with slack)
  constexpr int STAGE = KTILE + tile_elems<T, D, NCHV>();
  constexpr int NKK = D / 16;         // contraction steps over d
  constexpr int NDB = D / 32;         // 32-wide blocks of d
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* smem = reinterpret_cast<T*>(smem_raw);

  int item_idx, hg;
  if (!xcd_map(blockIdx.x, a.n_items, a.n_hg, item_idx, hg)) return;
  const QItem it = a.items[item_idx];
  if (it.nq <= 0) return;
  const int grp = a.hq / a.hkv;
  const int kv = (hg * a.hp) / grp;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int lr = l & 31, lh = l >> 5;
  const int row = 32 * w + lr;
  const int tok = row / a.hp;
  const int head = hg * a.hp + (row % a.hp);
  const bool qvalid = tok < it.nq;

  Frag<T> qf[NKK];
  {
    const T* qrow = a.q + ((size_t)(it.q0 + (qvalid ? tok : 0)) * a.hq + head) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (qvalid) load_frag(qf[kk], qrow + 16 * kk + 8 * lh);
      else qf[kk].v = {};
    }
  }

  const int na = (it.alen + KT - 1) / KT;
  const int nb = (it.blen + KT - 1) / KT;
  const int total = na + nb;
  const size_t kv_stride = (size_t)a.hkv * D;

  // Tiles are copied in order (j = 0, 1, ...), segment A's then B's; a
  // copy cursor holds the next tile's K and V^T bases, its segment's last
  // key counted from the tile's first (K rows past it are clamped to it) and
  // the V^T row stride, and advances by one tile per copy.
  const T* kcur;
  const T* vcur;
  int klast, vstride;
  auto cursor_to_b = [&]() {
    kcur = a.k_b + (size_t)it.b0 * kv_stride + kv * D;
    vcur = a.vt_b + (size_t)kv * D * a.vt_b_stride + it.bpad;
    klast = it.blen - 1;
    vstride = a.vt_b_stride;
  };
  if (na > 0) {
    kcur = a.k_a + (size_t)it.a0 * kv_stride + kv * D;
    vcur = a.vt_a + (size_t)kv * D * a.vt_a_stride + it.apad;
    klast = it.alen - 1;
    vstride = a.vt_a_stride;
  } else {
    cursor_to_b();
  }
  int copied = 0;
  // The next tile into LDS stage `stage`: K rows (keys past the segment are
  // clamped to its last key and masked later) and V^T rows (padded copy,
  // always in range).
  auto gload_next = [&](int stage) {
    T* kt = smem + stage * STAGE;
    const int kl = klast;
    g2l_tile<T, KT, NCHK, NT>(kt, kcur, [&](int r) { return min(r, kl) * (int)kv_stride; });
    const int vs = vstride;
    g2l_tile<T, D, NCHV, NT>(kt + KTILE, vcur, [&](int r) { return r * vs; });
    if (++copied == na) {
      cursor_to_b();
    } else {
      kcur += (size_t)KT * kv_stride;
      vcur += KT;
      klast -= KT;
    }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY;  // running max of scaled scores, log2 units
  // This lane's share of the running normaliser.  It sums the probabilities
  // as rounded for the P.V product (exact for float32 I/O), so the output
  // is a weighted mean of V rows with weights that sum to one.
  float lsum = 0.f;
  const float c2 = a.scale_log2;
  const int wave_tok0 = (32 * w) / a.hp;  // smallest token index of this wave

  if constexpr (PIPE) {
    // Half h = 2 j + e covers keys 32 e .. 32 e + 31 of tile j.  Per half:
    //   phase A  the scores of half h + 1 (8 products, K fragments loaded
    //            one step ahead) with the softmax of half h issued between
    //            them: mask, row maximum, lazy rescale, P = exp2(S - m),
    //            bf16 conversion and the normaliser sum;
    //   phase B  O^T += V^T P^T for half h (8 products).
    // Tile j + 1's K is read in the second half of tile j, so tiles are
    // triple buffered.  After the first half of tile j every wave waits for
    // its copies of tile j + 1 and meets the others at one barrier; by then
    // tile j - 1 is no longer read, and tile j + 2 is copied into its stage.
    // Tiles rotate through the stages (tile j in stage j % NSTAGE, kept as
    // a counter), and the two halves of a tile are separate instances of
    // the loop body, so that the half index and everything derived from it
    // are compile-time constants.
    if (total > 0) gload_next(0);
    if (total > 1) gload_next(1);
    wait_vmem();
    __syncthreads();
    f32x16 s_cur = f32x16{}, s_nxt = f32x16{};
    Frag<T> kf[2];
    auto kload = [&](const T* kt, int row0, int kk, int slot) {
      lds_frag(kf[slot], kt, row0 + lr, KROW, 16 * kk + 8 * lh);
    };
    if (total > 0) {
      kload(smem, 0, 0, 0);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        if (kk + 1 < NKK) kload(smem, 0, kk + 1, (kk + 1) & 1);
        mma(s_cur, kf[kk & 1], qf[kk]);
      }
    }
    int stage = 0;  // tile j's stage
    for (int j = 0; j < total; ++j) {
      const int stage1 = stage == NSTAGE - 1 ? 0 : stage + 1;  // tile j + 1's
      const T* kt = smem + stage * STAGE;
      const bool inA = j < na;
      const int key0 = (inA ? j : j - na) * KT;  // first key of the tile
      const int lim = inA ? it.alen - 1 : it.qpos + tok;
      // The next half's scores are formed unconditionally so that phase A
      // stays straight-line code; after the item's last half they come from
      // a stage that is in bounds but stale (this tile's second half), and
      // are discarded.
      const bool more = j + 1 < total;
      const T* kt_next = more ? smem + stage1 * STAGE : kt;
      const int row_next = more ? 0 : 32;
      auto half = [&](auto e_const) {
        constexpr int e = decltype(e_const)::value;
        const int kb0 = key0 + 32 * e;  // first key of the half
        const bool need_mask = inA ? (kb0 + 32 > it.alen) : (kb0 + 31 > it.qpos + wave_tok0);
        const T* ktn = e == 0 ? kt : kt_next;  // the next half's K
        const int rown = e == 0 ? 32 : row_next;
        s_nxt = f32x16{};
        kload(ktn, rown, 0, 0);
        Frag<T> pf[2];
        float mx = -INFINITY, m_use = 0.f;
        // phase A: scores of half h + 1 beside the softmax of half h
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          if (kk + 1 < NKK) kload(ktn, rown, kk + 1, (kk + 1) & 1);
          mma(s_nxt, kf[kk & 1], qf[kk]);
          if (kk == 0) {
            if (need_mask) {
#pragma unroll
              for (int jj = 0; jj < 16; ++jj) {
                const int key = kb0 + 8 * (jj >> 2) + 4 * lh + (jj & 3);
                if (key > lim) s_cur[jj] = -INFINITY;
              }
            }
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) mx = fmaxf(mx, s_cur[jj]);
            mx = max_with_other_half(mx) * c2;
          } else if (kk == 1) {
            // lazy rescale (as in the tile loop below)
            if (__any(mx > m_run + kRescale)) {
              const float m_new = fmaxf(m_run, mx);
              const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
              lsum *= alpha;
#pragma unroll
              for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
              m_run = m_new;
            }
          } else {
            m_use = (m_run == -INFINITY) ? 0.f : m_run;
            constexpr int PER = 16 / (NKK - 2);  // exponentials per remaining step
            const int base = (kk - 2) * PER;
#pragma unroll
            for (int u = 0; u < PER; ++u)
              if (base + u < 16) s_cur[base + u] = fast_exp2(s_cur[base + u] * c2 - m_use);
            if (kk == NKK - 1) {
#pragma unroll
              for (int jj = (NKK - 2) * PER; jj < 16; ++jj)
                s_cur[jj] = fast_exp2(s_cur[jj] * c2 - m_use);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        float ps = 0.f;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          to_frag(pf[hf], s_cur, 8 * hf);
          ps = frag_sum(pf[hf], ps);
        }
        lsum += ps;
        // phase B: O^T += V^T P^T for half h
        {
          const T* vt = kt + KTILE;
          Frag<T> vf[2];
          auto vload = [&](int st, int slot) {  // st = 2*db + hf
            lds_frag(vf[slot], vt, 32 * (st >> 1) + lr, VROW, 16 * (2 * e + (st & 1)) + 8 * lh);
          };
          vload(0, 0);
#pragma unroll
          for (int st = 0; st < 2 * NDB; ++st) {
            if (st + 1 < 2 * NDB) vload(st + 1, (st + 1) & 1);
            mma(oacc[st >> 1], vf[st & 1], pf[st & 1]);
          }
        }
        s_cur = s_nxt;
        if constexpr (e == 0) {
          // tile j + 1 complete everywhere, tile j - 1 no longer read
          wait_vmem();
          __syncthreads();
          if (j + 2 < total) gload_next(stage1 == NSTAGE - 1 ? 0 : stage1 + 1);
        }
      };
      half(std::integral_constant<int, 0>{});
      half(std::integral_constant<int, 1>{});
      stage = stage1;
    }
  } else {
  if (total > 0) gload_next(0);
  wait_vmem();
  __syncthreads();
  for (int j = 0; j < total; ++j) {
    if (j + 1 < total) gload_next((j + 1) & 1);
    const T* kt = smem + (j & 1) * STAGE;
    const T* vt = kt + KTILE;

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const int kr = 32 * kb + lr;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        Frag<T> kf;
        lds_frag(kf, kt, kr, KROW, 16 * kk + 8 * lh);
        mma(s[kb], kf, qf[kk]);
      }
    }

    const bool inA = j < na;
    const int ks = (inA ? j : j - na) * KT;
    const bool need_mask = inA ? (ks + KT > it.alen) : (ks + KT - 1 > it.qpos + wave_tok0);
    if (need_mask) {
      const int lim = inA ? it.alen - 1 : it.qpos + tok;  // last visible key
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const int key = ks + 32 * kb + 8 * (jj >> 2) + 4 * lh + (jj & 3);
          if (key > lim) s[kb][jj] = -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) mx = fmaxf(mx, s[kb][jj]);
    mx = max_with_other_half(mx) * c2;
    // Lazy rescale: the running maximum only has to bound the exponents, so
    // it is raised (and O and the normaliser rescaled) only when some row of
    // the wave grew by more than kRescale; otherwise P stays below
    // 2^kRescale.  The result is the same softmax.
    if (__any(mx > m_run + kRescale)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    if constexpr (NW == 12) {
      // Three waves per SIMD: P of keys 0-31, then its products with V, the
      // exponentials of keys 32-63 issued between those products (they do
      // not depend on them), then the products of keys 32-63.  (With two
      // waves per SIMD the plain order below is faster.)
      float ps = 0.f;
      auto expo = [&](int kb, int jj) { s[kb][jj] = fast_exp2(s[kb][jj] * c2 - m_use); };
      Frag<T> pf[2][2];
      Frag<T> vf[2];
      auto vload = [&](int kb, int step, int slot) {  // step = 2*db + hf
        const int db = step >> 1, hf = step & 1;
        lds_frag(vf[slot], vt, 32 * db + lr, VROW, 16 * (2 * kb + hf) + 8 * lh);
      };
      vload(0, 0, 0);
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) expo(0, jj);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        to_frag(pf[0][hf], s[0], 8 * hf);
        ps = frag_sum(pf[0][hf], ps);
      }
#pragma unroll
      for (int step = 0; step < 2 * NDB; ++step) {
        if (step + 1 < 2 * NDB) vload(0, step + 1, (step + 1) & 1);
        else vload(1, 0, (step + 1) & 1);
        mma(oacc[step >> 1], vf[step & 1], pf[0][step & 1]);
#pragma unroll
        for (int u = 0; u < 16 / (2 * NDB); ++u) expo(1, step * (16 / (2 * NDB)) + u);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        to_frag(pf[1][hf], s[1], 8 * hf);
        ps = frag_sum(pf[1][hf], ps);
      }
#pragma unroll
      for (int step = 0; step < 2 * NDB; ++step) {
        const int slot = (2 * NDB + step) & 1;
        if (step + 1 < 2 * NDB) vload(1, step + 1, slot ^ 1);
        mma(oacc[step >> 1], vf[slot], pf[1][step & 1]);
      }
      lsum += ps;
    } else {
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) s[kb][jj] = fast_exp2(s[kb][jj] * c2 - m_use);

      Frag<T> pf[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          to_frag(pf[kb][hf], s[kb], 8 * hf);
          ps = frag_sum(pf[kb][hf], ps);
        }
      lsum += ps;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int vr = 32 * db + lr;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            Frag<T> vf;
            lds_frag(vf, vt, vr, VROW, 16 * (2 * kb + hf) + 8 * lh);
            mma(oacc[db], vf, pf[kb][hf]);
          }
      }
    }

    wait_vmem();
    __syncthreads();
  }
  }

  const float lt = sum_with_other_half(lsum);
  if (!qvalid) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse = lt > 0.f ? (m_run + fast_log2(lt)) * kLn2 : -INFINITY;
  if (a.o_part != nullptr) {
    // one chunk of a split prompt column: float32 partial state (O, LSE),
    // merged afterwards
    const size_t tokens = a.lse_stride;
    float* orow = a.o_part + (((size_t)it.chunk * tokens + it.q0 + tok) * a.hq + head) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = oacc[db][4 * g4 + e] * inv;
        *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * g4 + 4 * lh) = v;
      }
    if (lh == 0) a.lse_part[((size_t)it.chunk * a.hq + head) * tokens + it.q0 + tok] = lse;
    return;
  }
  T* orow = a.o + ((size_t)(it.q0 + tok) * a.hq + head) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * db + 8 * g4 + 4 * lh;
      if constexpr (sizeof(T) == 2) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = static_cast<bf16>(oacc[db][4 * g4 + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + d0) = v;
      } else {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = oacc[db][4 * g4 + e] * inv;
        *reinterpret_cast<f32x4*>(orow + d0) = v;
      }
    }
  if (lh == 0) a.lse[(size_t)head * a.lse_stride + it.q0 + tok] = lse;
}

template <typename T, int D, int NW, bool PIPE = false>
static hipError_t launch_fwd_t(const FwdLaunch& l, hipStream_t s) {
  FwdArgs<T, D> a;
  a.q = static_cast<const T*>(l.q);
  a.o = static_cast<T*>(l.o);
  a.lse = l.lse;
  a.k_a = static_cast<const T*>(l.k_a);
  a.vt_a = static_cast<const T*>(l.vt_a);
  a.k_b = static_cast<const T*>(l.k_b);
  a.vt_b = static_cast<const T*>(l.vt_b);
  a.items = static_cast<const QItem*>(l.items);
  a.n_items = l.n_items;
  a.hq = l.hq;
  a.hkv = l.hkv;
  a.hp = l.hp;
  a.n_hg = l.hq / l.hp;
  a.lse_stride = l.lse_stride;
  a.vt_a_stride = l.vt_a_stride;
  a.vt_b_stride = l.vt_b_stride;
  a.scale_log2 = l.scale * kLog2e;
  a.o_part = l.o_part;
  a.lse_part = l.lse_part;
  constexpr int CH = 16 / sizeof(T);
  const size_t smem = (PIPE ? 3 : 2) * sizeof(T) *
                      (size_t)(tile_elems<T, kTileK, D / CH>() + tile_elems<T, D, kTileK / CH>());
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fwd_kernel<T, D, NW, PIPE>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  const int grid = xcd_grid(l.n_items, a.n_hg);
  if (grid <= 0) return hipSuccess;
  hipEvent_t e0, e1;
  kernel_events(kKernelFwd, &e0, &e1);
  if (e0)
    hipExtLaunchKernelGGL(fwd_kernel<T, D, NW, PIPE>, dim3(grid), dim3(64 * NW), smem, s, e0, e1,
                          0, a);
  else fwd_kernel<T, D, NW, PIPE><<<dim3(grid), dim3(64 * NW), smem, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdLaunch& l, hipStream_t s) {
  if (l.dtype == 1) {
    if (l.waves == 12)
      return l.d == 128 ? launch_fwd_t<bf16, 128, 12, kFwdPipe>(l, s)
                        : launch_fwd_t<bf16, 64, 12, kFwdPipe>(l, s);
    return l.d == 128 ? launch_fwd_t<bf16, 128, 8, kFwdPipe>(l, s)
                      : launch_fwd_t<bf16, 64, 8, kFwdPipe>(l, s);
  }
  return l.d == 128 ? launch_fwd_t<float, 128, 8>(l, s) : launch_fwd_t<float, 64, 8>(l, s);
}

}  // namespace treeattn
