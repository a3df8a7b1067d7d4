// ceilings.hip -- machine-ceiling kernels for the benchmark (libceilings.so).
//
// The forward's and the merge's rates are reported against the nominal
// MI355X figures and against what this GPU measurably sustains for the same
// kind of work, measured in the same run:
//   * ceil_mfma: only v_mfma_f32_16x16x32_bf16 in a loop, operands in
//     registers (the dense bf16 matrix rate the chip holds under a full load,
//     which sets its clock), with the shader-clock and real-time counters
//     read at the start and end of every workgroup;
//   * ceil_copy: a streaming read + write of a buffer, 16 B per lane;
//   * ceil_read: a streaming read of a buffer, 16 B per lane, nothing written
//     unless an impossible value turns up (so the loads cannot be removed).
// None of these is part of the LoRA path; they share no code with it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ceilings.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;  // independent accumulators per wave

__global__ __launch_bounds__(512) void ceil_mfma_kernel(int iters, float* out, uint64_t* clocks) {
  const int lane = threadIdx.x & 63;
  // Operands derived from the lane index so they are not compile-time values.
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1.0f + 0.001f * (float)((lane + i) & 15));
    b[i] = (__bf16)(0.5f - 0.001f * (float)((lane * 3 + i) & 15));
  }
  f32x4 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint64_t t0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    clocks[blockIdx.x * 4 + 0] = t0;
    clocks[blockIdx.x * 4 + 1] = t1;
    clocks[blockIdx.x * 4 + 2] = r0;
    clocks[blockIdx.x * 4 + 3] = r1;
  }
}

constexpr int kUnroll = 4;  // 16-B loads in flight per lane per iteration (grid stride)
constexpr int kBlockU = 8;  // 16-B loads in flight per lane per step (blocked)

// Variant 0: every lane strides over the whole buffer, kUnroll loads at a time.
// Variant 1: each workgroup streams one contiguous block, its 256 lanes
// reading 4 KiB per load round, kBlockU rounds in flight.  Variant 2: as 1
// with non-temporal loads and stores (streamed data bypasses cache retention).
template <int V>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
  if constexpr (V == 2) return __builtin_nontemporal_load(p);
  return *p;
}
template <int V>
__device__ __forceinline__ void st(u32x4* p, u32x4 v) {
  if constexpr (V == 2) __builtin_nontemporal_store(v, p);
  else *p = v;
}

template <int V>
__global__ __launch_bounds__(256) void ceil_copy_kernel(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, int64_t n16) {
  if constexpr (V == 0) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) dst[i + u * stride] = v[u];
    }
    for (; i < n16; i += stride) dst[i] = src[i];
  } else {
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = (int64_t)blockIdx.x * per;
    const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
    int64_t i = b0 + threadIdx.x;
    for (; i + (kBlockU - 1) * 256 < b1; i += kBlockU * 256) {
      u32x4 v[kBlockU];
#pragma unroll
      for (int u = 0; u < kBlockU; ++u) v[u] = ld<V>(src + i + u * 256);
#pragma unroll
      for (int u = 0; u < kBlockU; ++u) st<V>(dst + i + u * 256, v[u]);
    }
    for (; i < b1; i += 256) st<V>(dst + i, ld<V>(src + i));
  }
}

template <int V>
__global__ __launch_bounds__(256) void ceil_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                        uint32_t* __restrict__ out) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  if constexpr (V == 0) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= src[i];
  } else {
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = (int64_t)blockIdx.x * per;
    const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
    int64_t i = b0 + threadIdx.x;
    for (; i + (kBlockU - 1) * 256 < b1; i += kBlockU * 256) {
      u32x4 v[kBlockU];
#pragma unroll
      for (int u = 0; u < kBlockU; ++u) v[u] = ld<V>(src + i + u * 256);
#pragma unroll
      for (int u = 0; u < kBlockU; ++u) acc ^= v[u];
    }
    for (; i < b1; i += 256) acc ^= ld<V>(src + i);
  }
  // Never true for the benchmark's data (it reads a buffer of zeros): the
  // store keeps the loads alive without writing anything.
  if ((acc[0] & acc[1] & acc[2] & acc[3]) == 0xFFFFFFFFu) out[blockIdx.x] = acc[0];
}

}  // namespace

extern "C" {

int ceil_mfma(int workgroups, int waves, int iters, float* out, uint64_t* clocks, void* stream) {
  if (workgroups < 1 || waves < 1 || waves > 8 || iters < 1 || !out || !clocks) return 1;
  hipLaunchKernelGGL(ceil_mfma_kernel, dim3(workgroups), dim3(waves * 64), 0,
                     static_cast<hipStream_t>(stream), iters, out, clocks);
  return hipGetLastError() == hipSuccess ? 0 : 8;
}

double ceil_mfma_flops(int workgroups, int waves, int iters) {
  return (double)workgroups * waves * iters * kChains * (16.0 * 16.0 * 32.0 * 2.0);
}

int ceil_copy(const void* src, void* dst, int64_t bytes, int workgroups, int variant,
              void* stream) {
  if (!src || !dst || bytes < 0 || (bytes & 15) || workgroups < 1) return 1;
  if (variant < 0 || variant > 2) return 1;
  if (((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return 4;
  if (bytes == 0) return 0;
  auto k = variant == 0 ? ceil_copy_kernel<0> : variant == 1 ? ceil_copy_kernel<1>
                                                              : ceil_copy_kernel<2>;
  hipLaunchKernelGGL(k, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 8;
}

int ceil_read(const void* src, int64_t bytes, void* out, int workgroups, int variant,
              void* stream) {
  if (!src || !out || bytes < 0 || (bytes & 15) || workgroups < 1) return 1;
  if (variant < 0 || variant > 2) return 1;
  if ((uintptr_t)src & 15) return 4;
  if (bytes == 0) return 0;
  auto k = variant == 0 ? ceil_read_kernel<0> : variant == 1 ? ceil_read_kernel<1>
                                                              : ceil_read_kernel<2>;
  hipLaunchKernelGGL(k, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), bytes / 16, static_cast<uint32_t*>(out));
  return hipGetLastError() == hipSuccess ? 0 : 8;
}

}  // extern "C"
