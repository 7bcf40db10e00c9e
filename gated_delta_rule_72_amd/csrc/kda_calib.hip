// kda_calib.hip — device ceilings for the roofline figures: a dense fp16 MFMA
// loop and a streaming 16-byte copy (include/kda_calib.h).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/kda_calib.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Eight independent accumulators per wavefront keep the MFMA pipeline full;
// the operands change every iteration so the loop cannot be folded.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int32_t iters, float* out) {
  const int lane = threadIdx.x % 64;
  f16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (_Float16)(0.001f * (lane + e));
    b[e] = (_Float16)(0.002f * (lane - e));
  }
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
    a = a + (_Float16)0.0001f;
  }
  f32x4 s = acc[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) s += acc[j];
  reinterpret_cast<f32x4*>(out)[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Each thread moves four 16-byte vectors per step (all loads issued before
// the stores), nontemporal, over a grid-stride loop.
__global__ __launch_bounds__(256) void copy_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst,
                                                   int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 1024;
  for (int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x; base < n; base += stride) {
    f32x4 x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t i = base + 256 * j;
      x[j] = i < n ? __builtin_nontemporal_load(src + i) : f32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t i = base + 256 * j;
      if (i < n) __builtin_nontemporal_store(x[j], dst + i);
    }
  }
}

}  // namespace

extern "C" {

int kda_calib_mfma_f16(int32_t blocks, int32_t iters, float* out, void* hip_stream) {
  if (blocks <= 0 || iters <= 0 || !out || (reinterpret_cast<uintptr_t>(out) & 15)) return -1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(hip_stream), iters,
                     out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int kda_calib_copy(const void* src, void* dst, int64_t n_vec, int32_t blocks, void* hip_stream) {
  if (n_vec < 0 || blocks <= 0 || (n_vec > 0 && (!src || !dst)) ||
      (reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(dst) & 15))
    return -1;
  if (n_vec == 0) return 0;
  hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(hip_stream),
                     static_cast<const f32x4*>(src), static_cast<f32x4*>(dst), n_vec);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
