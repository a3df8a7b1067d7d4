// fwd_tiled.hip -- fused LoRA linear forward, bf16 operands, fp32 accumulate,
// on gfx950 MFMA (v_mfma_f32_16x16x32_bf16).
//
// Computes Y = X W^T + scale * (X A^T) B^T (the layer defined in "fastaf:
// Minimal LoRA fine-tuning with hand-written Triton kernels", section "FWD
// kernel speedup") in ONE launch: the base product, the rank-r
// down-projection, the up-projection, the scale and the add all happen in one
// workgroup per output tile, and the [tokens, r] intermediate never leaves the
// chip (registers, then LDS for the operand re-layout).
//
// Per workgroup (BM x BN output tile, WM x WN waves, each wave TM x TN blocks
// of 16 x 16):
//   K loop (BK = 64, two LDS stages, register prefetch of the next stage):
//     X[BM x 64], W[BN x 64], A[RP x 64] staged in LDS, rows of 128 B with the
//     16-B chunks XOR-swizzled by (row & 7) so MFMA operand reads are free of
//     bank conflicts;
//     acc[BM x BN] += X W^T          (MFMA)
//     T[BM x RP]   += X A^T          (MFMA, reusing the X operand registers)
//   epilogue:
//     T -> scale * T -> bf16 -> LDS; B[BN x RP] -> LDS (zero padded)
//     acc += (s T) B^T               (MFMA over the rank)
//     acc -> bf16 -> LDS -> coalesced 16-B stores of Y.
#include "common.h"
#include "kernels.h"

namespace lora {
namespace {

template <int WM_, int WN_, int TM_, int TN_, int RP_>
struct Tiled {
  static constexpr int WM = WM_, WN = WN_, TM = TM_, TN = TN_, RP = RP_;
  static constexpr int kThreads = WM * WN * kWave;
  static constexpr int BM = WM * TM * 16;
  static constexpr int BN = WN * TN * 16;
  static constexpr int BK = 64;
  static constexpr int RB = RP / 16;                 // 16-wide rank blocks
  static constexpr int kRowB = BK * 2;               // bytes per staged row
  static constexpr int kStageB = (BM + BN + RP) * kRowB;
  static constexpr int kTS = RP + 8;                 // epilogue row stride (elements)
  static constexpr int kEpiB = (BM + BN) * kTS * 2;
  static constexpr int kYS = BN + 8;                 // output staging row stride
  static constexpr int kYB = BM * kYS * 2;
  static constexpr int kLds = (2 * kStageB > kEpiB ? (2 * kStageB > kYB ? 2 * kStageB : kYB)
                                                   : (kEpiB > kYB ? kEpiB : kYB));
  static constexpr int kRowsPerPass = kThreads / 8;  // rows covered by one chunk pass
  static constexpr int kXPass = BM / kRowsPerPass;
  static constexpr int kWPass = BN / kRowsPerPass;
  static constexpr int kAPass = (RP + kRowsPerPass - 1) / kRowsPerPass;
  static constexpr int kTTiles = TM * RB;            // T tiles per wave row group
  static constexpr int kTSlots = (kTTiles + WN - 1) / WN;
  static_assert(BM % kRowsPerPass == 0 && BN % kRowsPerPass == 0, "tile rows per pass");
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

template <class C>
__global__ __launch_bounds__(C::kThreads) void fwd_tiled_bf16_kernel(
    int M, int N, int K, int r, const uint16_t* __restrict__ X, int64_t ldx,
    const uint16_t* __restrict__ W, int64_t ldw, const uint16_t* __restrict__ A, int64_t lda,
    const uint16_t* __restrict__ B, int64_t ldb, float scale, uint16_t* __restrict__ Y,
    int64_t ldy, int tiles_m, int tiles_n, int y_vec) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int BM = C::BM, BN = C::BN, RP = C::RP, RB = C::RB, TM = C::TM, TN = C::TN;
  constexpr int WN = C::WN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;

  // ---- tile id: XCD-contiguous, then grouped along M for L2 reuse of W.
  const int total = tiles_m * tiles_n;
  int pid = xcd_contiguous_id(blockIdx.x, total);
  constexpr int kGroup = 8;
  const int group = pid / (kGroup * tiles_n);
  const int first_m = group * kGroup;
  const int gsize = min(tiles_m - first_m, kGroup);
  const int tile_m = first_m + (pid % (kGroup * tiles_n)) % gsize;
  const int tile_n = (pid % (kGroup * tiles_n)) / gsize;
  const int m0 = tile_m * BM;
  const int n0 = tile_n * BN;

  // ---- per-thread global chunk sources (row clamped; K tail zero-filled).
  const int crow = tid >> 3;  // row within a pass
  const int cchk = tid & 7;   // 16-B chunk within the 64-wide k slab
  const uint16_t* xsrc[C::kXPass];
  const uint16_t* wsrc[C::kWPass];
  const uint16_t* asrc[C::kAPass];
#pragma unroll
  for (int p = 0; p < C::kXPass; ++p) {
    const int row = min(m0 + crow + p * C::kRowsPerPass, M - 1);
    xsrc[p] = X + (int64_t)row * ldx + cchk * 8;
  }
#pragma unroll
  for (int p = 0; p < C::kWPass; ++p) {
    const int row = min(n0 + crow + p * C::kRowsPerPass, N - 1);
    wsrc[p] = W + (int64_t)row * ldw + cchk * 8;
  }
#pragma unroll
  for (int p = 0; p < C::kAPass; ++p) {
    const int row = min(crow + p * C::kRowsPerPass, r - 1);
    asrc[p] = A + (int64_t)row * lda + cchk * 8;
  }

  u32x4 px[C::kXPass], pw[C::kWPass], pa[C::kAPass];
  auto load_stage = [&](int k0) {
    const bool kin = k0 + cchk * 8 < K;
#pragma unroll
    for (int p = 0; p < C::kXPass; ++p)
      px[p] = kin ? *reinterpret_cast<const u32x4*>(xsrc[p] + k0) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < C::kWPass; ++p)
      pw[p] = kin ? *reinterpret_cast<const u32x4*>(wsrc[p] + k0) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < C::kAPass; ++p) {
      const bool in = kin && (crow + p * C::kRowsPerPass < RP);
      pa[p] = in ? *reinterpret_cast<const u32x4*>(asrc[p] + k0) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_stage = [&](int buf) {
    unsigned char* base = smem + buf * C::kStageB;
#pragma unroll
    for (int p = 0; p < C::kXPass; ++p)
      *reinterpret_cast<u32x4*>(base + swz(crow + p * C::kRowsPerPass, cchk)) = px[p];
#pragma unroll
    for (int p = 0; p < C::kWPass; ++p)
      *reinterpret_cast<u32x4*>(base + BM * 128 + swz(crow + p * C::kRowsPerPass, cchk)) = pw[p];
#pragma unroll
    for (int p = 0; p < C::kAPass; ++p) {
      const int row = crow + p * C::kRowsPerPass;
      if (row < RP) *reinterpret_cast<u32x4*>(base + (BM + BN) * 128 + swz(row, cchk)) = pa[p];
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = zero4();
  f32x4 tacc[C::kTSlots];
#pragma unroll
  for (int s = 0; s < C::kTSlots; ++s) tacc[s] = zero4();

  // Which rank blocks this wave works on (T tile (i, tj) belongs to wave
  // (i * RB + tj) % WN of its wave row).
  bool uses_tj[RB];
#pragma unroll
  for (int tj = 0; tj < RB; ++tj) {
    bool u = false;
#pragma unroll
    for (int i = 0; i < TM; ++i) u |= ((i * RB + tj) % WN) == wn;
    uses_tj[tj] = u;
  }

  const int nk = (K + C::BK - 1) / C::BK;
  if (nk > 0) {
    load_stage(0);
    store_stage(0);
  }
  __syncthreads();

  const int lrow = lane & 15;
  const int lk = lane >> 4;
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) load_stage((kt + 1) * C::BK);
    const unsigned char* xs = smem + (kt & 1) * C::kStageB;
    const unsigned char* ws = xs + BM * 128;
    const unsigned char* as = ws + BN * 128;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int cc = kk * 4 + lk;
      u32x4 a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *reinterpret_cast<const u32x4*>(xs + swz(wm * TM * 16 + i * 16 + lrow, cc));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = *reinterpret_cast<const u32x4*>(ws + swz(wn * TN * 16 + j * 16 + lrow, cc));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
#pragma unroll
      for (int tj = 0; tj < RB; ++tj) {
        if (!uses_tj[tj]) continue;
        const u32x4 bt = *reinterpret_cast<const u32x4*>(as + swz(tj * 16 + lrow, cc));
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int idx = i * RB + tj;
          if (idx % WN == wn) tacc[idx / WN] = mfma16x16x32(a[i], bt, tacc[idx / WN]);
        }
      }
    }
    if (more) store_stage((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue 1: scaled T (bf16) and the B tile into LDS.
  uint16_t* ts = reinterpret_cast<uint16_t*>(smem);
  uint16_t* bs = ts + BM * C::kTS;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int tj = 0; tj < RB; ++tj) {
      const int idx = i * RB + tj;
      if (idx % WN != wn) continue;
      const int j = tj * 16 + lrow;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = wm * TM * 16 + i * 16 + lk * 4 + q;
        ts[row * C::kTS + j] = j < r ? f2bf(scale * tacc[idx / WN][q]) : uint16_t(0);
      }
    }
  for (int e = tid; e < BN * RP; e += C::kThreads) {
    const int n = e / RP, j = e % RP;
    uint16_t v = 0;
    if (j < r && n0 + n < N) v = B[(int64_t)(n0 + n) * ldb + j];
    bs[n * C::kTS + j] = v;
  }
  __syncthreads();

  // ---- epilogue 2: acc += (s T) B^T on MFMA, contraction over the rank.
  if constexpr (RP >= 32) {
#pragma unroll
    for (int kk = 0; kk < RP / 32; ++kk) {
      u32x4 a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *reinterpret_cast<const u32x4*>(ts + (wm * TM * 16 + i * 16 + lrow) * C::kTS +
                                               kk * 32 + lk * 8);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = *reinterpret_cast<const u32x4*>(bs + (wn * TN * 16 + j * 16 + lrow) * C::kTS +
                                               kk * 32 + lk * 8);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
    }
  } else {
    u32x2 a[TM], b[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
      a[i] = *reinterpret_cast<const u32x2*>(ts + (wm * TM * 16 + i * 16 + lrow) * C::kTS + lk * 4);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      b[j] = *reinterpret_cast<const u32x2*>(bs + (wn * TN * 16 + j * 16 + lrow) * C::kTS + lk * 4);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma16x16x16(a[i], b[j], acc[i][j]);
  }
  __syncthreads();

  // ---- epilogue 3: round once to bf16, stage, store coalesced.
  uint16_t* ys = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = wm * TM * 16 + i * 16 + lk * 4 + q;
        ys[row * C::kYS + wn * TN * 16 + j * 16 + lrow] = f2bf(acc[i][j][q]);
      }
  __syncthreads();
  constexpr int kCPR = BN / 8;  // 16-B chunks per output row
  for (int e = tid; e < BM * kCPR; e += C::kThreads) {
    const int row = e / kCPR, c = e % kCPR;
    const int gm = m0 + row, gn = n0 + c * 8;
    if (gm >= M || gn >= N) continue;
    const uint16_t* src = ys + row * C::kYS + c * 8;
    uint16_t* dst = Y + (int64_t)gm * ldy + gn;
    if (y_vec && gn + 8 <= N) {
      *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
    } else {
      for (int q = 0; q < 8 && gn + q < N; ++q) dst[q] = src[q];
    }
  }
}

template <class C>
hipError_t launch(const FwdArgs& a, hipStream_t s) {
  const int tiles_m = (int)((a.M + C::BM - 1) / C::BM);
  const int tiles_n = (int)((a.N + C::BN - 1) / C::BN);
  const int y_vec = ((reinterpret_cast<uintptr_t>(a.Y) & 15) == 0) && (a.ldy % 8 == 0);
  auto kern = fwd_tiled_bf16_kernel<C>;
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  hipLaunchKernelGGL(kern, dim3(tiles_m * tiles_n), dim3(C::kThreads), C::kLds, s, (int)a.M,
                     (int)a.N, (int)a.K, (int)a.r, static_cast<const uint16_t*>(a.X), a.ldx,
                     static_cast<const uint16_t*>(a.W), a.ldw, static_cast<const uint16_t*>(a.A),
                     a.lda, static_cast<const uint16_t*>(a.B), a.ldb, a.scale,
                     static_cast<uint16_t*>(a.Y), a.ldy, tiles_m, tiles_n, y_vec);
  return hipGetLastError();
}

template <int RP>
hipError_t launch_rp(const FwdArgs& a, hipStream_t s) {
  return launch<Tiled<2, 2, 4, 4, RP>>(a, s);
}

}  // namespace

hipError_t launch_fwd_tiled_bf16(const FwdArgs& a, hipStream_t s) {
  switch (pad_rank(a.r)) {
    case 16: return launch_rp<16>(a, s);
    case 32: return launch_rp<32>(a, s);
    case 64: return launch_rp<64>(a, s);
    case 128: return launch_rp<128>(a, s);
    default: return launch_rp<256>(a, s);
  }
}

}  // namespace lora
