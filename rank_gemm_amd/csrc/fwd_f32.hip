// fwd_f32.hip -- fused LoRA linear forward for fp32 operands on gfx950
// (v_mfma_f32_16x16x4_f32: true fp32 products, fp32 accumulate).
//
// Same single-launch structure as the bf16 kernel (layer defined in "fastaf:
// Minimal LoRA fine-tuning with hand-written Triton kernels", section "FWD
// kernel speedup"): per 64 x 64 output tile, one K loop accumulates both
// X W^T and T = X A^T; the epilogue adds scale * T B^T with T kept in fp32 on
// chip.  fp32 workloads here are small and launch-bound, so this kernel is
// single-staged and favours clarity over speed.
#include "common.h"
#include "kernels.h"

namespace lora {
namespace {

constexpr int kF32Threads = 256;
constexpr int kF32BM = 64, kF32BN = 64, kF32BK = 32;
constexpr int kF32Stride = kF32BK + 4;  // floats per staged row (breaks bank aliasing)

template <int RP>
struct F32Cfg {
  static constexpr int RB = RP / 16;
  static constexpr int kStageFloats = (kF32BM + kF32BN + RP) * kF32Stride;
  static constexpr int kES = RP + 4;
  static constexpr int kEpiFloats = (kF32BM + kF32BN) * kES;
  static constexpr int kLds = 4 * (kStageFloats > kEpiFloats ? kStageFloats : kEpiFloats);
  static constexpr int kTTiles = 2 * RB;               // T tiles per wave row (TM = 2)
  static constexpr int kTSlots = (kTTiles + 1) / 2;    // split over the 2 waves of a row
};

template <int RP>
__global__ __launch_bounds__(kF32Threads) void fwd_tiled_f32_kernel(
    int M, int N, int K, int r, const float* __restrict__ X, int64_t ldx,
    const float* __restrict__ W, int64_t ldw, const float* __restrict__ A, int64_t lda,
    const float* __restrict__ B, int64_t ldb, float scale, float* __restrict__ Y, int64_t ldy,
    int tiles_n) {
  using C = F32Cfg<RP>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  float* smem = reinterpret_cast<float*>(smem_raw);
  float* xs = smem;
  float* ws = xs + kF32BM * kF32Stride;
  float* as = ws + kF32BN * kF32Stride;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = lane & 15, lk = lane >> 4;
  const int m0 = (blockIdx.x / tiles_n) * kF32BM;
  const int n0 = (blockIdx.x % tiles_n) * kF32BN;

  f32x4 acc[2][2];
  f32x4 tacc[C::kTSlots];
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j) acc[i][j] = zero4();
  for (int s = 0; s < C::kTSlots; ++s) tacc[s] = zero4();

  // 16-B chunks: 8 per 32-float row.
  for (int k0 = 0; k0 < K; k0 += kF32BK) {
    for (int e = tid; e < (kF32BM + kF32BN + RP) * 8; e += kF32Threads) {
      const int row = e >> 3, c = e & 7;
      const int k = k0 + c * 4;
      f32x4 v = zero4();
      float* dst;
      if (row < kF32BM) {
        const int gm = min(m0 + row, M - 1);
        if (k < K) v = *reinterpret_cast<const f32x4*>(X + (int64_t)gm * ldx + k);
        dst = xs + row * kF32Stride + c * 4;
      } else if (row < kF32BM + kF32BN) {
        const int gn = min(n0 + row - kF32BM, N - 1);
        if (k < K) v = *reinterpret_cast<const f32x4*>(W + (int64_t)gn * ldw + k);
        dst = ws + (row - kF32BM) * kF32Stride + c * 4;
      } else {
        const int j = row - kF32BM - kF32BN;
        if (k < K && j < r) v = *reinterpret_cast<const f32x4*>(A + (int64_t)j * lda + k);
        dst = as + j * kF32Stride + c * 4;
      }
      *reinterpret_cast<f32x4*>(dst) = v;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kF32BK / 4; ++ks) {
      const int kc = ks * 4 + lk;
      float a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = xs[(wm * 32 + i * 16 + lrow) * kF32Stride + kc];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = ws[(wn * 32 + j * 16 + lrow) * kF32Stride + kc];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma16x16x4f32(a[i], b[j], acc[i][j]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int tj = 0; tj < C::RB; ++tj) {
          const int idx = i * C::RB + tj;
          if ((idx & 1) != wn) continue;
          const float bt = as[(tj * 16 + lrow) * kF32Stride + kc];
          tacc[idx >> 1] = mfma16x16x4f32(a[i], bt, tacc[idx >> 1]);
        }
    }
    __syncthreads();
  }

  // Epilogue: scaled fp32 T and the B tile in LDS, then acc += (s T) B^T.
  float* ts = smem;
  float* bs = smem + kF32BM * C::kES;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int tj = 0; tj < C::RB; ++tj) {
      const int idx = i * C::RB + tj;
      if ((idx & 1) != wn) continue;
      const int j = tj * 16 + lrow;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        ts[(wm * 32 + i * 16 + lk * 4 + q) * C::kES + j] = j < r ? scale * tacc[idx >> 1][q] : 0.f;
    }
  for (int e = tid; e < kF32BN * RP; e += kF32Threads) {
    const int n = e / RP, j = e % RP;
    bs[n * C::kES + j] = (j < r && n0 + n < N) ? B[(int64_t)(n0 + n) * ldb + j] : 0.f;
  }
  __syncthreads();
#pragma unroll 4
  for (int js = 0; js < RP / 4; ++js) {
    const int jc = js * 4 + lk;
    float a[2], b[2];
    for (int i = 0; i < 2; ++i) a[i] = ts[(wm * 32 + i * 16 + lrow) * C::kES + jc];
    for (int j = 0; j < 2; ++j) b[j] = bs[(wn * 32 + j * 16 + lrow) * C::kES + jc];
    for (int i = 0; i < 2; ++i)
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma16x16x4f32(a[i], b[j], acc[i][j]);
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int gm = m0 + wm * 32 + i * 16 + lk * 4 + q;
        const int gn = n0 + wn * 32 + j * 16 + lrow;
        if (gm < M && gn < N) Y[(int64_t)gm * ldy + gn] = acc[i][j][q];
      }
}

template <int RP>
hipError_t launch_f32(const FwdArgs& a, hipStream_t s) {
  using C = F32Cfg<RP>;
  const int tiles_m = (int)((a.M + kF32BM - 1) / kF32BM);
  const int tiles_n = (int)((a.N + kF32BN - 1) / kF32BN);
  auto kern = fwd_tiled_f32_kernel<RP>;
  static std::atomic<uint64_t> attr_done{0};
  if (hipError_t e = ensure_lds(kern, C::kLds, attr_done); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(tiles_m * tiles_n), dim3(kF32Threads), C::kLds, s, (int)a.M,
                     (int)a.N, (int)a.K, (int)a.r, static_cast<const float*>(a.X), a.ldx,
                     static_cast<const float*>(a.W), a.ldw, static_cast<const float*>(a.A), a.lda,
                     static_cast<const float*>(a.B), a.ldb, a.scale, static_cast<float*>(a.Y),
                     a.ldy, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_tiled_f32(const FwdArgs& a, hipStream_t s) {
  switch (pad_rank(a.r)) {
    case 16: return launch_f32<16>(a, s);
    case 32: return launch_f32<32>(a, s);
    case 64: return launch_f32<64>(a, s);
    case 128: return launch_f32<128>(a, s);
    default: return launch_f32<256>(a, s);
  }
}

}  // namespace lora
