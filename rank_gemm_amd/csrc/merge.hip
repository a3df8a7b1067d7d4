// merge.hip -- merge a LoRA adapter into a pristine weight in one pass:
//   W_inf[n, k] = round(W0[n, k] + scale * sum_j B[n, j] A[j, k])
// (the addmm refresh from the unsloth commit log for
// scripts/benchmarks/qwen3_flex_inference.py: pristine read only, W_inf
// rewritten, fp32 accumulation).
//
// bf16 kernel, per workgroup an output tile of TN rows x 256 columns:
//   1. issue the 16-B loads of the W0 tile (the HBM read stream) into registers;
//   2. stage the A[r x 256] slab in LDS transposed to [k][j], so that the
//      rank is the contiguous (MFMA reduction) axis of both operands;
//   3. P = B A for the tile on MFMA (16x16x32, fp32 accumulate, r padded to
//      a multiple of 32 with zeros);
//   4. P -> LDS (fp32), then every thread combines its W0 chunks with the
//      matching P values, rounds once to bf16 and writes 16-B chunks.
// W0 is never written; nothing is accumulated across workgroups, so repeated
// merges of the same inputs are bitwise identical.
#include "common.h"
#include "kernels.h"

namespace lora {
namespace {

template <int TNB, int RP>
struct Mrg {
  static constexpr int kThreads = 256;
  static constexpr int TN = TNB * 16;
  static constexpr int TK = 256;
  static constexpr int RB32 = RP / 32;
  static constexpr int kAS = RP + 8;   // transposed-A row stride (bf16 elements)
  static constexpr int kPS = TK + 4;   // P row stride (floats)
  static constexpr int kAtB = TK * kAS * 2;
  static constexpr int kPB = TN * kPS * 4;
  static constexpr int kLds = kAtB + kPB;
  static constexpr int kWChunks = TN * TK / 8 / kThreads;
  static constexpr int kAChunks = RP * TK / 8 / kThreads;
  static_assert(kWChunks >= 1 && kAChunks >= 1, "tile too small for the thread count");
};

template <int TNB, int RP>
__global__ __launch_bounds__(256) void merge_bf16_kernel(
    int N, int K, int r, const uint16_t* __restrict__ W0, int64_t ldw0,
    const uint16_t* __restrict__ B, int64_t ldb, const uint16_t* __restrict__ A, int64_t lda,
    float scale, uint16_t* __restrict__ Wi, int64_t ldwi, int tiles_k, int b_vec) {
  using C = Mrg<TNB, RP>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* at = reinterpret_cast<uint16_t*>(smem);
  float* pl = reinterpret_cast<float*>(smem + C::kAtB);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lk = lane >> 4;
  const int n0 = (blockIdx.x / tiles_k) * C::TN;
  const int k0 = (blockIdx.x % tiles_k) * C::TK;
  const u32x4 z = {0, 0, 0, 0};

  // 1. W0 tile -> registers (32 chunks of 16 B per 256-wide row).
  u32x4 w[C::kWChunks];
#pragma unroll
  for (int i = 0; i < C::kWChunks; ++i) {
    const int e = tid + i * C::kThreads;
    const int gn = n0 + (e >> 5), gk = k0 + (e & 31) * 8;
    w[i] = (gn < N && gk < K) ? *reinterpret_cast<const u32x4*>(W0 + (int64_t)gn * ldw0 + gk) : z;
  }

  // 2. A slab -> LDS, transposed to at[k][j].
#pragma unroll
  for (int i = 0; i < C::kAChunks; ++i) {
    const int e = tid + i * C::kThreads;
    const int j = e >> 5, c = e & 31, gk = k0 + c * 8;
    const u32x4 v =
        (j < r && gk < K) ? *reinterpret_cast<const u32x4*>(A + (int64_t)j * lda + gk) : z;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      at[(c * 8 + q) * C::kAS + j] = static_cast<uint16_t>(v[q >> 1] >> ((q & 1) * 16));
  }

  // B rows of this tile as MFMA A-operands (rank along the lane's 8 values).
  u32x4 bfr[TNB][C::RB32];
#pragma unroll
  for (int nb = 0; nb < TNB; ++nb) {
    const int gn = n0 + nb * 16 + lrow;
#pragma unroll
    for (int kk = 0; kk < C::RB32; ++kk) {
      const int j0 = kk * 32 + lk * 8;
      u32x4 v = z;
      if (gn < N) {
        const uint16_t* src = B + (int64_t)gn * ldb + j0;
        if (b_vec && j0 + 8 <= r) {
          v = *reinterpret_cast<const u32x4*>(src);
        } else {
          uint16_t h[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) h[q] = (j0 + q < r) ? src[q] : uint16_t(0);
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = (uint32_t)h[2 * q] | ((uint32_t)h[2 * q + 1] << 16);
        }
      }
      bfr[nb][kk] = v;
    }
  }
  __syncthreads();

  // 3. P = B A on MFMA: wave w owns k-blocks [4w, 4w + 4) of the 16 in the tile.
  f32x4 p[TNB][4];
#pragma unroll
  for (int nb = 0; nb < TNB; ++nb)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) p[nb][kb] = zero4();
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int kcol = (wave * 4 + kb) * 16 + lrow;
#pragma unroll
    for (int kk = 0; kk < C::RB32; ++kk) {
      const u32x4 bv = *reinterpret_cast<const u32x4*>(at + kcol * C::kAS + kk * 32 + lk * 8);
#pragma unroll
      for (int nb = 0; nb < TNB; ++nb) p[nb][kb] = mfma16x16x32(bfr[nb][kk], bv, p[nb][kb]);
    }
  }
  // 4. P -> LDS, then combine with W0 and store.
#pragma unroll
  for (int nb = 0; nb < TNB; ++nb)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        pl[(nb * 16 + lk * 4 + q) * C::kPS + (wave * 4 + kb) * 16 + lrow] = p[nb][kb][q];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < C::kWChunks; ++i) {
    const int e = tid + i * C::kThreads;
    const int row = e >> 5, c = e & 31;
    const int gn = n0 + row, gk = k0 + c * 8;
    if (gn >= N || gk >= K) continue;
    const f32x4 p0 = *reinterpret_cast<const f32x4*>(pl + row * C::kPS + c * 8);
    const f32x4 p1 = *reinterpret_cast<const f32x4*>(pl + row * C::kPS + c * 8 + 4);
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t wv = w[i][q];
      const float pa = q < 2 ? p0[2 * q] : p1[2 * q - 4];
      const float pb = q < 2 ? p0[2 * q + 1] : p1[2 * q - 3];
      const float lo = __builtin_bit_cast(float, wv << 16) + scale * pa;
      const float hi = __builtin_bit_cast(float, wv & 0xFFFF0000u) + scale * pb;
      o[q] = pack_bf2(lo, hi);
    }
    *reinterpret_cast<u32x4*>(Wi + (int64_t)gn * ldwi + gk) = o;
  }
}

template <int TNB, int RP>
hipError_t launch_m(const MergeArgs& a, hipStream_t s) {
  using C = Mrg<TNB, RP>;
  auto kern = merge_bf16_kernel<TNB, RP>;
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int tiles_n = (int)((a.N + C::TN - 1) / C::TN);
  const int tiles_k = (int)((a.K + C::TK - 1) / C::TK);
  const int b_vec = ((reinterpret_cast<uintptr_t>(a.B) & 15) == 0) && (a.ldb % 8 == 0);
  hipLaunchKernelGGL(kern, dim3(tiles_n * tiles_k), dim3(C::kThreads), C::kLds, s, (int)a.N,
                     (int)a.K, (int)a.r, static_cast<const uint16_t*>(a.W0), a.ldw0,
                     static_cast<const uint16_t*>(a.B), a.ldb, static_cast<const uint16_t*>(a.A),
                     a.lda, a.scale, static_cast<uint16_t*>(a.Wi), a.ldwi, tiles_k, b_vec);
  return hipGetLastError();
}

template <int TNB>
hipError_t launch_m_tn(const MergeArgs& a, hipStream_t s) {
  switch (pad_rank(a.r)) {
    case 16:
    case 32: return launch_m<TNB, 32>(a, s);
    case 64: return launch_m<TNB, 64>(a, s);
    case 128: return launch_m<TNB, 128>(a, s);
    default: return launch_m<1, 256>(a, s);
  }
}

// fp32 merge: plain VALU, 4 consecutive columns per thread, fp32 FMA chain
// over the rank.
__global__ __launch_bounds__(256) void merge_f32_kernel(
    int N, int K, int r, const float* __restrict__ W0, int64_t ldw0, const float* __restrict__ B,
    int64_t ldb, const float* __restrict__ A, int64_t lda, float scale, float* __restrict__ Wi,
    int64_t ldwi, int kblocks) {
  const int n = blockIdx.x / kblocks;
  const int k = ((blockIdx.x % kblocks) * 256 + threadIdx.x) * 4;
  if (n >= N || k >= K) return;
  f32x4 acc = zero4();
  for (int j = 0; j < r; ++j) {
    const float b = B[(int64_t)n * ldb + j];
    const f32x4 av = *reinterpret_cast<const f32x4*>(A + (int64_t)j * lda + k);
    acc += b * av;
  }
  const f32x4 w = *reinterpret_cast<const f32x4*>(W0 + (int64_t)n * ldw0 + k);
  *reinterpret_cast<f32x4*>(Wi + (int64_t)n * ldwi + k) = w + scale * acc;
}

}  // namespace

hipError_t launch_merge_bf16(const MergeArgs& a, hipStream_t s) {
  // Small targets get 16-row tiles so that the grid still covers the chip.
  // Rank above 128 keeps 16-row tiles: the transposed A slab alone needs 132 KiB.
  const int64_t tiles32 = ((a.N + 31) / 32) * ((a.K + 255) / 256);
  return (tiles32 >= 1024 && a.r <= 128) ? launch_m_tn<2>(a, s) : launch_m_tn<1>(a, s);
}

hipError_t launch_merge_f32(const MergeArgs& a, hipStream_t s) {
  const int kblocks = (int)((a.K + 1023) / 1024);
  hipLaunchKernelGGL(merge_f32_kernel, dim3((unsigned)(a.N * kblocks)), dim3(256), 0, s, (int)a.N,
                     (int)a.K, (int)a.r, static_cast<const float*>(a.W0), a.ldw0,
                     static_cast<const float*>(a.B), a.ldb, static_cast<const float*>(a.A), a.lda,
                     a.scale, static_cast<float*>(a.Wi), a.ldwi, kblocks);
  return hipGetLastError();
}

}  // namespace lora
