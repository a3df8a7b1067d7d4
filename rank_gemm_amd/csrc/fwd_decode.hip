// fwd_decode.hip -- fused LoRA linear forward for few tokens (M <= 64), bf16.
//
// Same layer as the tiled kernel (defined in "fastaf: Minimal LoRA fine-tuning
// with hand-written Triton kernels", section "FWD kernel speedup"), shaped for
// decode: the cost is streaming W once from HBM, so the kernel is organised
// around that stream instead of around output tiles.
//
// Per workgroup: 16 output columns (16 rows of W), NW waves.  The K axis is
// cut into 64-wide blocks dealt round-robin to the waves; each lane streams
// 32 contiguous bytes of one W row per block, and the matching X and A
// elements come from L2.  MFMA (16x16x32) accumulates, per wave,
//   Ybase[m, n] += X W^T   and   T[m, j] += X A^T   (T fully on chip).
// The waves' partial sums are added in a fixed order through LDS
// (deterministic), then the epilogue adds scale * T B^T in fp32 on the VALU
// and stores bf16.
#include "common.h"
#include "kernels.h"

namespace lora {
namespace {

template <int MB, int RP, int NW>
struct Dec {
  static constexpr int RB = RP / 16;
  static constexpr int kSlots = MB * (1 + RB);           // f32x4 partials per lane
  static constexpr int kRedB = NW * kSlots * kWave * 16;  // LDS for the reduction
  static constexpr int kTB = MB * 16 * (RP + 1) * 4;      // T rows for the epilogue
  static constexpr int kLds = kRedB + kTB;
  static constexpr int kU = MB >= 4 ? 2 : MB >= 2 ? 4 : 8;  // 64-wide blocks per batch
};

template <int MB, int RP, int NW>
__global__ __launch_bounds__(NW * 64) void fwd_decode_bf16_kernel(
    int M, int N, int K, int r, const uint16_t* __restrict__ X, int64_t ldx,
    const uint16_t* __restrict__ W, int64_t ldw, const uint16_t* __restrict__ A, int64_t lda,
    const uint16_t* __restrict__ B, int64_t ldb, float scale, uint16_t* __restrict__ Y,
    int64_t ldy) {
  using C = Dec<MB, RP, NW>;
  constexpr int RB = C::RB;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, lq = lane >> 4;
  const int n0 = blockIdx.x * 16;

  const uint16_t* wrow = W + (int64_t)min(n0 + lrow, N - 1) * ldw + lq * 16;
  const uint16_t* xrow[MB];
  bool xin[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = mb * 16 + lrow;
    xin[mb] = m < M;
    xrow[mb] = X + (int64_t)min(m, M - 1) * ldx + lq * 16;
  }
  const uint16_t* arow[RB];
  bool ain[RB];
#pragma unroll
  for (int tj = 0; tj < RB; ++tj) {
    const int j = tj * 16 + lrow;
    ain[tj] = j < r;
    arow[tj] = A + (int64_t)min(j, r - 1) * lda + lq * 16;
  }

  f32x4 yacc[MB], tacc[MB][RB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    yacc[mb] = zero4();
#pragma unroll
    for (int tj = 0; tj < RB; ++tj) tacc[mb][tj] = zero4();
  }

  const u32x4 z = {0, 0, 0, 0};
  const int nblk = (K + 63) / 64;
  for (int b0 = wave; b0 < nblk; b0 += NW * C::kU) {
    u32x4 wv[C::kU][2];
    // Issue the whole batch of W loads first: they are the HBM stream.
#pragma unroll
    for (int u = 0; u < C::kU; ++u) {
      const int blk = b0 + u * NW;
      const int k = blk * 64 + lq * 16;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        wv[u][h] = (blk < nblk && k + h * 8 < K)
                       ? *reinterpret_cast<const u32x4*>(wrow + (int64_t)blk * 64 + h * 8)
                       : z;
    }
#pragma unroll
    for (int u = 0; u < C::kU; ++u) {
      const int blk = b0 + u * NW;
      if (blk >= nblk) break;
      const int k = blk * 64 + lq * 16;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bool kin = k + h * 8 < K;
        u32x4 xv[MB], av[RB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          xv[mb] = (kin && xin[mb])
                       ? *reinterpret_cast<const u32x4*>(xrow[mb] + (int64_t)blk * 64 + h * 8)
                       : z;
#pragma unroll
        for (int tj = 0; tj < RB; ++tj)
          av[tj] = (kin && ain[tj])
                       ? *reinterpret_cast<const u32x4*>(arow[tj] + (int64_t)blk * 64 + h * 8)
                       : z;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          yacc[mb] = mfma16x16x32(xv[mb], wv[u][h], yacc[mb]);
#pragma unroll
          for (int tj = 0; tj < RB; ++tj) tacc[mb][tj] = mfma16x16x32(xv[mb], av[tj], tacc[mb][tj]);
        }
      }
    }
  }

  // Cross-wave reduction in a fixed order (wave 0 + wave 1 + ...).
  f32x4* red = reinterpret_cast<f32x4*>(smem);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    red[(wave * C::kSlots + mb * (1 + RB)) * kWave + lane] = yacc[mb];
#pragma unroll
    for (int tj = 0; tj < RB; ++tj) red[(wave * C::kSlots + mb * (1 + RB) + 1 + tj) * kWave + lane] = tacc[mb][tj];
  }
  __syncthreads();
  const bool active = wave < MB;
  const int mb = active ? wave : 0;
  f32x4 y = zero4();
  float* tl = reinterpret_cast<float*>(smem + C::kRedB) + mb * 16 * (RP + 1);
  if (active) {
    f32x4 t[RB];
#pragma unroll
    for (int tj = 0; tj < RB; ++tj) t[tj] = zero4();
    for (int w = 0; w < NW; ++w) {
      y += red[(w * C::kSlots + mb * (1 + RB)) * kWave + lane];
#pragma unroll
      for (int tj = 0; tj < RB; ++tj)
        t[tj] += red[(w * C::kSlots + mb * (1 + RB) + 1 + tj) * kWave + lane];
    }
    // T rows of this M block to LDS (fp32) for the up-projection below.
#pragma unroll
    for (int tj = 0; tj < RB; ++tj)
#pragma unroll
      for (int q = 0; q < 4; ++q) tl[(lq * 4 + q) * (RP + 1) + tj * 16 + lrow] = t[tj][q];
  }
  __syncthreads();
  if (!active) return;
  // L[m, n] = sum_j T[m, j] B[n, j]; Y = Ybase + scale * L, rounded once.
  const int n = n0 + lrow;
  if (n >= N) return;
  float bn[RP];
#pragma unroll
  for (int j = 0; j < RP; ++j) bn[j] = j < r ? bf2f(B[(int64_t)n * ldb + j]) : 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int m = mb * 16 + lq * 4 + q;
    if (m >= M) break;
    float l = 0.f;
#pragma unroll
    for (int j = 0; j < RP; ++j) l += tl[(lq * 4 + q) * (RP + 1) + j] * bn[j];
    Y[(int64_t)m * ldy + n] = f2bf(y[q] + scale * l);
  }
}

template <int MB, int RP>
hipError_t launch_dec(const FwdArgs& a, hipStream_t s) {
  constexpr int NW = 8;
  using C = Dec<MB, RP, NW>;
  auto kern = fwd_decode_bf16_kernel<MB, RP, NW>;
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int blocks = (int)((a.N + 15) / 16);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(NW * 64), C::kLds, s, (int)a.M, (int)a.N, (int)a.K,
                     (int)a.r, static_cast<const uint16_t*>(a.X), a.ldx,
                     static_cast<const uint16_t*>(a.W), a.ldw, static_cast<const uint16_t*>(a.A),
                     a.lda, static_cast<const uint16_t*>(a.B), a.ldb, a.scale,
                     static_cast<uint16_t*>(a.Y), a.ldy);
  return hipGetLastError();
}

template <int RP>
hipError_t launch_dec_rp(const FwdArgs& a, hipStream_t s) {
  switch ((a.M + 15) / 16) {
    case 1: return launch_dec<1, RP>(a, s);
    case 2: return launch_dec<2, RP>(a, s);
    case 3: return launch_dec<3, RP>(a, s);
    default: return launch_dec<4, RP>(a, s);
  }
}

}  // namespace

hipError_t launch_fwd_decode_bf16(const FwdArgs& a, hipStream_t s) {
  return a.r <= 16 ? launch_dec_rp<16>(a, s) : launch_dec_rp<32>(a, s);
}

}  // namespace lora
