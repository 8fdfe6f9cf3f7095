// Sustained dense bf16 matrix-core rate of the GPU: a measurement aid for the
// roofline of the attention kernels, built as its own small library
// (libmfmaceiling.so) and used only by bench.py --mfma-ceiling.
//
// A loop of v_mfma_f32_32x32x16_bf16 on register operands (no memory traffic,
// no other instructions in the loop), four independent accumulators, one
// 8-wave workgroup per CU (two waves per SIMD, as in the dQ and dK/dV
// kernels; an unused 96 KB LDS reservation keeps a second one off the CU),
// launched back to back for a given time.  Two operand kinds:
//   constant  the same few nonzero bf16 values in every product, which
//             shows the instruction rate;
//   random    16 fragments of uniform(-1.7, 1.7) bf16 values (variance
//             near 1, like normalised Q, K, V, dO) with a different pair in
//             every product of an iteration, which shows the rate the
//             chip's power limit lets the matrix units sustain on real data.
// The attention kernels multiply such data, so the second figure is the
// ceiling their matrix work runs against.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;  // 8 waves per workgroup
constexpr int kIters = 20000;  // 8 products per iteration
constexpr int kGroupsPerCu = 4;   // workgroups per CU over the launch
constexpr int kLdsBytes = 96 * 1024;  // reserved, unused: one workgroup per CU

__device__ __forceinline__ unsigned mix(unsigned x) {  // integer hash
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

template <bool RANDOM>
__device__ __forceinline__ bf16x8 operand(unsigned id, int lane) {
  bf16x8 f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float u = (float)(mix(id * 8u + i) & 0xffffu) * (1.f / 65536.f) - 0.5f;
    f[i] = static_cast<__bf16>(RANDOM ? 3.4f * u : 1e-3f * (float)(lane + i));
  }
  return f;
}

template <bool RANDOM>
__device__ __forceinline__ void mfma_loop(float* out) {
  const unsigned t = blockIdx.x * kThreads + threadIdx.x;
  const int lane = threadIdx.x & 63;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    a[f] = operand<RANDOM>(16 * t + f, lane);
    b[f] = operand<RANDOM>(16 * t + 8 + f, lane);
  }
  f32x16 c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = f32x16{};
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      c[k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[(k + 3) & 7], c[k & 3], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += c[i][j];
  out[t] = s;  // out holds gridDim.x * kThreads floats
}

__global__ __launch_bounds__(kThreads) void mfma_loop_constant(float* out) {
  mfma_loop<false>(out);
}
__global__ __launch_bounds__(kThreads) void mfma_loop_random(float* out) {
  mfma_loop<true>(out);
}

}  // namespace

// Runs launches of the loop back to back on the current device's default
// stream until `seconds` have elapsed (at least 4 launches).  Writes the
// median rate (dense bf16 TFLOP/s) over the second half of the launches,
// after the clock has settled, to *tflops, the first launch's rate to
// *first_tflops and the launch count to *launches.  random_operands selects
// the operand kind (see above).  Allocates and frees one output buffer.
// Returns 0, -1 for a bad argument, or -4 if a HIP call failed.
extern "C" int mfma_ceiling_run(int random_operands, double seconds, double* tflops,
                                double* first_tflops, int* launches) {
  if (!(seconds > 0) || tflops == nullptr || first_tflops == nullptr || launches == nullptr)
    return -1;
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return -4;
  const int grid = kGroupsPerCu * prop.multiProcessorCount;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(mfma_loop_constant),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes) != hipSuccess ||
      hipFuncSetAttribute(reinterpret_cast<const void*>(mfma_loop_random),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes) != hipSuccess)
    return -4;
  float* out = nullptr;
  if (hipMalloc(&out, (size_t)grid * kThreads * sizeof(float)) != hipSuccess) return -4;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  bool ok = hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess;
  const double flops = (double)grid * (kThreads / 64) * kIters * 8 * 32768.0;
  std::vector<double> rates;
  double elapsed_ms = 0;
  while (ok && (elapsed_ms < seconds * 1e3 || rates.size() < 4)) {
    ok = hipEventRecord(e0, 0) == hipSuccess;
    if (random_operands)
      hipLaunchKernelGGL(mfma_loop_random, dim3(grid), dim3(kThreads), kLdsBytes, 0, out);
    else
      hipLaunchKernelGGL(mfma_loop_constant, dim3(grid), dim3(kThreads), kLdsBytes, 0, out);
    ok = ok && hipGetLastError() == hipSuccess && hipEventRecord(e1, 0) == hipSuccess &&
         hipEventSynchronize(e1) == hipSuccess;
    float ms = 0;
    ok = ok && hipEventElapsedTime(&ms, e0, e1) == hipSuccess && ms > 0;
    if (ok) {
      elapsed_ms += ms;
      rates.push_back(flops / (ms * 1e-3) / 1e12);
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipFree(out);
  if (!ok) return -4;
  *first_tflops = rates.front();
  std::vector<double> tail(rates.begin() + rates.size() / 2, rates.end());
  std::sort(tail.begin(), tail.end());
  *tflops = tail[tail.size() / 2];
  *launches = (int)rates.size();
  return 0;
}
