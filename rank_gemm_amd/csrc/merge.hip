// merge.hip -- merge a LoRA adapter into a pristine weight in one pass:
//   W_inf[n, k] = round(W0[n, k] + scale * sum_j B[n, j] A[j, k])
// (the addmm refresh from the unsloth commit log for
// scripts/benchmarks/qwen3_flex_inference.py: pristine read only, W_inf
// rewritten, fp32 accumulation).
//
// The cost is streaming W0 in and W_inf out; the rank-r product is small
// (2r flop per element) and runs on MFMA.
//
// bf16 kernel.  A workgroup (4 waves) owns a 256-column strip of the output
// and a range of 16-row blocks; wave w owns columns [64w, 64w + 64) of the
// strip.  P^T = A^T B^T is computed as 16 x 16 MFMA blocks (rows = k,
// columns = n, v_mfma_f32_16x16x32_bf16, fp32 accumulate).  The four k-blocks
// of a wave use a permuted k order, MFMA row i of block kb <-> column
// 16 (i / 4) + 4 kb + i % 4, so that after the four MFMAs lane l holds, for
// row n = l % 16, the 16 consecutive columns [16 (l / 16), +16) of the
// wave's 64: exactly one 32-byte run of W0 and of W_inf.  Each lane then
// adds its W0 run, rounds once to bf16 and stores the run; no LDS round trip
// for P.  The A strip is staged in LDS once per workgroup, transposed so that
// the rank is contiguous, and its fragments stay in registers for every row
// block.  Several row blocks of W0 loads are kept in flight.
//
// W0 is never written; nothing is accumulated across workgroups, so repeated
// merges of the same inputs are bitwise identical.
#include "common.h"
#include "kernels.h"

namespace lora {
namespace {

constexpr int kMergeThreads = 256;
constexpr int kStrip = 256;  // columns per workgroup (64 per wave)

template <int RP>
struct Mrg {
  static constexpr int RB32 = RP / 32;          // rank chunks of 32
  static constexpr int kAS = RP + 8;            // transposed-A row stride (elements, even)
  static constexpr int kLds = kStrip * kAS * 2;
  static constexpr int kU = RP <= 64 ? 4 : 2;   // row blocks in flight per wave
};

// Column (within the wave's 64) of element e (0..15) of lane group lg's run:
// elements 0..7 are columns 8 lg .. 8 lg + 7, elements 8..15 are columns
// 32 + 8 lg .. +7, so each 16-B load or store of the four lane groups of a
// row covers 64 contiguous bytes.
__device__ __forceinline__ int run_col(int lg, int e) { return (e >> 3) * 32 + 8 * lg + (e & 7); }

template <int RP>
__global__ __launch_bounds__(kMergeThreads) void merge_bf16_kernel(
    int N, int K, int r, const uint16_t* __restrict__ W0, int64_t ldw0,
    const uint16_t* __restrict__ B, int64_t ldb, const uint16_t* __restrict__ A, int64_t lda,
    float scale, uint16_t* __restrict__ Wi, int64_t ldwi, int strips, int nblk_per_wg,
    int b_vec) {
  using C = Mrg<RP>;
  constexpr int RB32 = C::RB32, U = C::kU;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint32_t* at32 = reinterpret_cast<uint32_t*>(smem);  // at[k][j] as j-pairs, k < 256
  const uint16_t* at = reinterpret_cast<const uint16_t*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lg = lane >> 4;
  const int strip = blockIdx.x % strips;
  const int ngrp = blockIdx.x / strips;
  const int k0 = strip * kStrip;
  const int nb_begin = ngrp * nblk_per_wg;
  const int nblocks = (N + 15) / 16;
  const int nb_end = min(nblocks, nb_begin + nblk_per_wg);
  const u32x4 z = {0, 0, 0, 0};

  // 1. A strip -> LDS transposed to at[k][j]: a thread takes two ranks
  //    (2p, 2p + 1) of one 8-column chunk and writes 32-bit words, so
  //    neighbouring threads write neighbouring words (no bank conflicts).
  for (int e = tid; e < (RP / 2) * (kStrip / 8); e += kMergeThreads) {
    const int pj = e % (RP / 2), c = e / (RP / 2), gk = k0 + c * 8;
    const int j = 2 * pj;
    const u32x4 v0 =
        (j < r && gk < K) ? *reinterpret_cast<const u32x4*>(A + (int64_t)j * lda + gk) : z;
    const u32x4 v1 =
        (j + 1 < r && gk < K) ? *reinterpret_cast<const u32x4*>(A + (int64_t)(j + 1) * lda + gk) : z;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t lo = (v0[q >> 1] >> ((q & 1) * 16)) & 0xFFFFu;
      const uint32_t hi = (v1[q >> 1] >> ((q & 1) * 16)) & 0xFFFFu;
      at32[((c * 8 + q) * C::kAS) / 2 + pj] = lo | (hi << 16);
    }
  }
  __syncthreads();

  // 2. This wave's A^T fragments for its 64 columns: block kb, MFMA row i
  //    holds column run_col(i / 4, 4 kb + i % 4).
  const int kw = wave * 64;
  u32x4 af[4][RB32];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int kl = kw + run_col(lrow >> 2, 4 * kb + (lrow & 3));
#pragma unroll
    for (int kk = 0; kk < RB32; ++kk)
      af[kb][kk] = *reinterpret_cast<const u32x4*>(at + kl * C::kAS + kk * 32 + lg * 8);
  }

  // Lane's output: row n, columns g0 .. g0 + 7 and g1 .. g1 + 7.
  const int g0 = k0 + kw + 8 * lg, g1 = g0 + 32;
  const bool c0 = g0 < K, c1 = g1 < K;

  auto load = [&](int nb, u32x4 (&w)[U][2], u32x4 (&bf)[U][RB32]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int n = (nb + u) * 16 + lrow;
      const bool nin = (nb + u) < nb_end && n < N;
      const int64_t row = (int64_t)(nin ? n : 0);
      w[u][0] = (nin && c0) ? *reinterpret_cast<const u32x4*>(W0 + row * ldw0 + g0) : z;
      w[u][1] = (nin && c1) ? *reinterpret_cast<const u32x4*>(W0 + row * ldw0 + g1) : z;
#pragma unroll
      for (int kk = 0; kk < RB32; ++kk) {
        const int j0 = kk * 32 + lg * 8;
        u32x4 v = z;
        if (nin) {
          const uint16_t* src = B + row * ldb + j0;
          if (b_vec && j0 + 8 <= r) {
            v = *reinterpret_cast<const u32x4*>(src);
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t lo = (j0 + 2 * q < r) ? src[2 * q] : 0u;
              const uint32_t hi = (j0 + 2 * q + 1 < r) ? src[2 * q + 1] : 0u;
              v[q] = lo | (hi << 16);
            }
          }
        }
        bf[u][kk] = v;
      }
    }
  };
  auto compute_store = [&](int nb, const u32x4 (&w)[U][2], const u32x4 (&bf)[U][RB32]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // The MFMAs read operands from all 64 lanes, so they run wave-uniform;
      // rows past N only skip their stores.
      if ((nb + u) >= nb_end) continue;
      const int n = (nb + u) * 16 + lrow;
      f32x4 p[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        p[kb] = zero4();
#pragma unroll
        for (int kk = 0; kk < RB32; ++kk) p[kb] = mfma16x16x32(af[kb][kk], bf[u][kk], p[kb]);
      }
      // p[kb][q] is element e = 4 kb + q of the lane's run (row n).
      u32x4 o[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const int e = 8 * h + 2 * q2;
          const uint32_t wv = w[u][h][q2];
          const float lo = __builtin_bit_cast(float, wv << 16) + scale * p[e >> 2][e & 3];
          const float hi =
              __builtin_bit_cast(float, wv & 0xFFFF0000u) + scale * p[(e + 1) >> 2][(e + 1) & 3];
          o[h][q2] = pack_bf2(lo, hi);
        }
      if (n < N) {
        uint16_t* dst = Wi + (int64_t)n * ldwi;
        if (c0) *reinterpret_cast<u32x4*>(dst + g0) = o[0];
        if (c1) *reinterpret_cast<u32x4*>(dst + g1) = o[1];
      }
    }
  };

  // 3. Row blocks, U at a time, the loads of the next group in flight while
  //    the current group is combined and stored.
  u32x4 wa[U][2], ba[U][RB32], wb[U][2], bb[U][RB32];
  int nb = nb_begin;
  if (nb < nb_end) load(nb, wa, ba);
  while (nb < nb_end) {
    if (nb + U < nb_end) load(nb + U, wb, bb);
    compute_store(nb, wa, ba);
    nb += U;
    if (nb >= nb_end) break;
    if (nb + U < nb_end) load(nb + U, wa, ba);
    compute_store(nb, wb, bb);
    nb += U;
  }
}

template <int RP>
hipError_t launch_m(const MergeArgs& a, hipStream_t s) {
  using C = Mrg<RP>;
  auto kern = merge_bf16_kernel<RP>;
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int strips = (int)((a.K + kStrip - 1) / kStrip);
  const int nblocks = (int)((a.N + 15) / 16);
  // About 512 workgroups (2 per CU), each streaming at least 2 U-groups of
  // row blocks so the A-strip staging is amortised.
  int groups = (512 + strips - 1) / strips;
  if (groups > nblocks) groups = nblocks;
  if (groups < 1) groups = 1;
  int per = (nblocks + groups - 1) / groups;
  if (per < 2 * C::kU) per = nblocks < 2 * C::kU ? nblocks : 2 * C::kU;
  groups = (nblocks + per - 1) / per;
  const int b_vec = ((reinterpret_cast<uintptr_t>(a.B) & 15) == 0) && (a.ldb % 8 == 0);
  hipLaunchKernelGGL(kern, dim3(strips * groups), dim3(kMergeThreads), C::kLds, s, (int)a.N,
                     (int)a.K, (int)a.r, static_cast<const uint16_t*>(a.W0), a.ldw0,
                     static_cast<const uint16_t*>(a.B), a.ldb, static_cast<const uint16_t*>(a.A),
                     a.lda, a.scale, static_cast<uint16_t*>(a.Wi), a.ldwi, strips, per, b_vec);
  return hipGetLastError();
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
  switch (pad_rank(a.r)) {
    case 16:
    case 32: return launch_m<32>(a, s);
    case 64: return launch_m<64>(a, s);
    case 128: return launch_m<128>(a, s);
    default: return launch_m<256>(a, s);
  }
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
