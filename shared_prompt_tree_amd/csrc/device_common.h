// Device helpers shared by the gfx950 attention kernels.
//
// Matrix products use the 32x32 MFMA output block.  For the bf16 path one
// v_mfma_f32_32x32x16_bf16 covers a 16-deep slice of the contraction; for the
// float32 path eight v_mfma_f32_32x32x2_f32 cover the same slice.  Operand
// fragments are 8 elements per lane along the contraction axis: lane l holds
// row (l % 32) of its operand and contraction slots 8*(l/32) .. 8*(l/32)+7.
// Which hardware k index a slot lands on does not matter as long as both
// operands use the same (l/32, element) -> contraction-index assignment,
// which every product here does.
//
// Output block layout (32x32, 16 float32 per lane): lane l, register j holds
// row 8*(j/4) + 4*(l/32) + (j%4) and column l % 32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace treeattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Eight contraction elements of one operand row, per lane.
template <typename T>
struct Frag;
template <>
struct Frag<bf16> {
  bf16x8 v;
};
template <>
struct Frag<float> {
  f32x8 v;
};

__device__ __forceinline__ void mma(f32x16& c, const Frag<bf16>& a, const Frag<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, c, 0, 0, 0);
}

__device__ __forceinline__ void mma(f32x16& c, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[s], b.v[s], c, 0, 0, 0);
}

// Bytes per 16-byte chunk and elements per chunk.
template <typename T>
struct ChunkOf {
  static constexpr int kElems = 16 / sizeof(T);
};

// Load 8 contiguous elements (16-byte aligned for bf16, 32-byte for float).
__device__ __forceinline__ void load_frag(Frag<bf16>& f, const bf16* p) {
  f.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void load_frag(Frag<float>& f, const float* p) {
  f.v = *reinterpret_cast<const f32x8*>(p);
}

// LDS tiles store each row as NCH 16-byte chunks followed by one chunk of
// padding.  The row stride is then an odd number of chunks, so 16
// consecutive rows read at the same column fall into 16 different 16-byte
// bank groups (no bank conflicts), and a fragment address is a per-lane base
// plus a compile-time offset.
template <typename T, int NCH>
__host__ __device__ constexpr int tile_row_elems() {
  return (NCH + 1) * (16 / (int)sizeof(T));
}

// Fragment read: 8 elements of row `row` starting at element elem0.
template <typename T>
__device__ __forceinline__ void lds_frag(Frag<T>& f, const T* tile, int row, int row_elems,
                                         int elem0) {
  const T* p = tile + row * row_elems + elem0;
  if constexpr (sizeof(T) == 2) {
    f.v = *reinterpret_cast<const bf16x8*>(p);
  } else {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
    f.v = f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

// One global_load_lds_dwordx4: every lane copies the 16 bytes at
// base + byte_off (base wave-uniform in scalar registers, byte_off a 32-bit
// per-lane offset) to LDS byte (lds_wave_dst + 16 * lane), lds_wave_dst being
// a 32-bit LDS byte address uniform across the wave (it goes through M0).  The instruction is issued
// from inline assembly so the compiler does not treat it as a pending LDS
// write and stall later LDS reads of other buffers on it; the caller waits
// for completion (wait_vmem) before the barrier that publishes the data.
// Memory reads return in issue order, so any wait the compiler places for
// its own loads stays correct.
__device__ __forceinline__ void dma_16(const void* base, uint32_t byte_off, uint32_t lds_wave_dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_wave_dst);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(byte_off), "s"(base), "s"(lds)
               : "m0");
}

// Elements an LDS tile of ROWS padded rows occupies, rounded up to whole
// 64-chunk wave copies (the slack receives harmless duplicate chunks).
template <typename T, int ROWS, int NCH>
__host__ __device__ constexpr int tile_elems() {
  return ((ROWS * (NCH + 1) + 63) / 64) * 64 * (16 / (int)sizeof(T));
}

// Copy a tile of ROWS rows x NCH 16-byte chunks from global memory straight
// into its padded LDS layout (global_load_lds_dwordx4: no registers
// involved).  One wave instruction fills 64 consecutive LDS chunks, lane l
// writing chunk l of them.  Lanes that land on a padding chunk or in the
// slack load a duplicate of a real chunk, so no lane is switched off.
// Global addresses are the wave-uniform `base` plus row_off(r) + chunk
// offset in elements; the byte offset must fit in 32 bits (the host checks
// the largest one) and the caller clamps rows past the end to a valid row.  Completion is awaited with wait_vmem() before the barrier
// that publishes the tile.
template <typename T, int ROWS, int NCH, int NT, typename RowOff>
__device__ __forceinline__ void g2l_tile(T* tile, const T* base, RowOff row_off) {
  constexpr int CH = 16 / sizeof(T);
  constexpr int STRIDE = NCH + 1;
  constexpr int NCHUNK = tile_elems<T, ROWS, NCH>() / CH;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // The low 32 bits of a generic pointer into LDS are the LDS address;
  // taking them directly keeps the destination arithmetic 32-bit.
  const uint32_t tile_lds = (uint32_t)(uintptr_t)tile;
#pragma unroll
  for (int i = 0; i < (NCHUNK + NT - 1) / NT; ++i) {
    const int p0 = i * NT + 64 * w;  // first chunk of this wave instruction
    if (NCHUNK % NT == 0 || p0 < NCHUNK) {
      const int p = p0 + lane;
      const int q = p / STRIDE;
      const int r = q < ROWS ? q : ROWS - 1;
      const int s = min(p - q * STRIDE, NCH - 1);
      const uint32_t off = ((uint32_t)row_off(r) + (uint32_t)(s * CH)) * (uint32_t)sizeof(T);
      dma_16(base, off, tile_lds + (uint32_t)p0 * 16u);
    }
  }
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane j passes the address of 4 consecutive 16-bit elements; lane i
// receives element i % 4 of the 4-element runs addressed by lanes
// 4e + i / 4, for e = 0..3.  When lane j addresses row r0 + j / 4, columns
// c0 + 4 (j % 4) .. +3 of a row-major matrix, lane i therefore receives
// column c0 + i of rows r0 .. r0 + 3: a 4 x 16 block read column-wise, the
// layout of an MFMA operand whose contraction runs down the rows.  The
// address must be 8-byte aligned.
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  lds_v4i16* q = (lds_v4i16*)(const_cast<bf16*>(p));
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(q);
  return __builtin_bit_cast(bf16x4, r);
}

// Wait until this wave's outstanding memory operations (including the
// global-to-LDS copies above) have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0); }

// Convert 8 float32 (registers j0..j0+7 of an output block) to an operand
// fragment.  bf16 rounds to nearest even.
__device__ __forceinline__ void to_frag(Frag<bf16>& f, const f32x16& c, int j0) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = static_cast<bf16>(c[j0 + e]);
}
__device__ __forceinline__ void to_frag(Frag<float>& f, const f32x16& c, int j0) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = c[j0 + e];
}

// acc plus the sum of a fragment's 8 values.  For bf16, v_dot2 with a (1, 1)
// operand adds two values per instruction (the sum then matches the
// rounded probabilities that the P.V product uses).
__device__ __forceinline__ float frag_sum(const Frag<bf16>& f, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {static_cast<bf16>(1.f), static_cast<bf16>(1.f)};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{f.v[2 * e], f.v[2 * e + 1]}, one, acc, false);
  return acc;
}
__device__ __forceinline__ float frag_sum(const Frag<float>& f, float acc) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc += f.v[e];
  return acc;
}

__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename T>
__device__ __forceinline__ T from_f32(float x) {
  return static_cast<T>(x);
}

// Values of lane l and lane l ^ 32 (the other half of the wave).
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second; called with the same value twice it returns the
// pair (own, other) in some order on every lane.
__device__ __forceinline__ float max_with_other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Position of row/key index k inside its 16-aligned group in the transposed
// copies: bits 2 and 3 are exchanged.  The output block holds rows
// {4*(l/32) + (j%4)} + 8*(j/4); with the exchange, the 8 slots one lane
// feeds to a 16-deep product (registers 8h .. 8h+7) become 8 consecutive
// positions 8*(l/32) .. 8*(l/32)+7 of the 16-group.
__host__ __device__ __forceinline__ int perm16(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// Workgroup -> (work item, head group) with all head groups of a kv head on
// one XCD.  Workgroups are dealt to the 8 XCDs round-robin (block b runs on
// XCD b % 8), and each XCD has its own L2.
__device__ __forceinline__ bool xcd_map(int b, int n_items, int n_hg, int& item, int& hg) {
  const int x = b & 7, j = b >> 3;
  if (n_hg % 8 == 0) {
    const int per = n_hg / 8;
    hg = x * per + (j % per);
    item = j / per;
  } else if (8 % n_hg == 0) {
    const int per = 8 / n_hg;
    hg = x % n_hg;
    item = j * per + x / n_hg;
  } else {
    hg = b % n_hg;
    item = b / n_hg;
  }
  return item < n_items;
}

__host__ __device__ inline int xcd_grid(int n_items, int n_hg) {
  if (n_hg % 8 == 0 || 8 % n_hg != 0) return n_items * n_hg;
  const int per = 8 / n_hg;
  return ((n_items + per - 1) / per) * 8;
}

// Work items built on the device from the offset arrays.
// Query-stationary item: a tile of query tokens and the two key segments it
// reads: segment A without mask (the prompt, for replay) and segment B with
// the causal mask (the prompt for prefill, the own branch for replay).
struct QItem {
  int q0, nq, qpos;      // first query token (global), tokens in tile, position in B
  int a0, alen, apad;    // segment A: first key token, keys, padded offset
  int b0, blen, bpad;    // segment B: first key token, keys read, padded offset
  int cost;
  int chunk;             // prompt-column chunk of a split replay launch (else 0)
  int pad_;
};

// Key-stationary item: a tile of key tokens and the query segments
// [seg_lo, seg_hi) that read it.
struct KItem {
  int k0, nk, kpos;      // first key token (global), keys, position in its segment
  int kind;              // 0: write I/O dtype; 1: write float32 seeds; 2: I/O dtype + seeds;
                         // 3: write float32 partial seeds at row prow
  int seg_lo, seg_hi, causal, cost;
  int prow;              // kind 3: partial-seed row of key 0
};

constexpr int kTileQ = 256;  // query rows per workgroup (query-stationary)
// The bf16 forward kernel also runs as 12 waves (384 query rows, three waves
// per SIMD) where that tiling still gives every CU several workgroups.
constexpr int kTileQWide = 384;
constexpr int kWideMinWorkgroups = 4 * 256;
constexpr int kTileK = 64;   // keys per step (query-stationary)
constexpr int kTileKV = 256; // keys per workgroup (key-stationary)
constexpr int kBlockQ = 64;  // query rows per step (key-stationary)
constexpr int kPad = 64;     // token padding of every segment in transposed copies

}  // namespace treeattn
