// Shared device/host helpers of the TTT-E2E gfx950 library.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

#define TTT_DEV __device__ __forceinline__

TTT_DEV float to_f32(float x) { return x; }
TTT_DEV float to_f32(bf16 x) { return (float)x; }
template <typename T> TTT_DEV T from_f32(float x);
template <> TTT_DEV float from_f32<float>(float x) { return x; }
template <> TTT_DEV bf16 from_f32<bf16>(float x) { return (bf16)x; }

// wave64 reductions with DPP-free cross-lane shuffles
TTT_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
TTT_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide sum for blockDim.x a multiple of 64 (<= 1024). `red` has >= 16 floats.
TTT_DEV float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}
TTT_DEV float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = -INFINITY;
  for (int i = 0; i < nw; ++i) s = fmaxf(s, red[i]);
  return s;
}

// Host-side launch error check used by the launchers.
#define TTT_LAUNCH_CHECK() (hipGetLastError())

// Every kernel launch of the library: a plain launch, or, while the timing
// events of launch_events() (kernels.h) are set, one with them attached to
// its own dispatch.
#define TTT_LAUNCH(kernel, grid, block, shmem, stream, ...)                                       \
  do {                                                                                            \
    LaunchEvents& le_ = launch_events();                                                          \
    hipEvent_t start_ = le_.start;                                                                \
    le_.start = nullptr;                                                                          \
    hipExtLaunchKernelGGL(kernel, grid, block, (std::uint32_t)(shmem), stream, start_, le_.stop, 0u, \
                          __VA_ARGS__);                                                           \
  } while (0)
