// fwd_f32.hip -- fused LoRA linear forward for fp32 operands on gfx950
// (v_mfma_f32_16x16x4_f32: true fp32 products, fp32 accumulate).
//
// Same single-launch structure as the bf16 kernel (layer defined in "fastaf:
// Minimal LoRA fine-tuning with hand-written Triton kernels", section "FWD
// kernel speedup"): per 64 x 64 output tile, one K loop accumulates both
// X W^T and T = X A^T; the epilogue adds scale * T B^T with T kept in fp32 on
// chip.  fp32 workloads here are small and bound by memory latency (a few
// workgroups, one stage after another), so the K loop keeps a ring of
// 32-deep stages in flight: X, W and A rows reach LDS by 16-B-per-lane direct
// loads (buffer_load ... lds: 8 rows x 128 B per instruction, rows and K
// past the operands read as zeros), 16-B chunks XOR-swizzled by row, and a
// stage is waited for only when it is about to be read.
#include "common.h"
#include "kernels.h"

namespace lora {
namespace {

constexpr int kF32Threads = 256;  // 4 waves, 2 x 2 over the output tile
constexpr int kF32BK = 32;        // 32 floats: 128-B staged rows

// BT x BT output tile (64 or 32; each wave owns a BT/2 x BT/2 quarter of
// 16 x 16 MFMA blocks).
template <int RP, int BT>
struct F32Cfg {
  static constexpr int RB = RP / 16;
  static constexpr int TW = BT / 32;  // 16-row blocks per wave in each direction
  // A rows staged per stage: at least 32, so that the staged rows (X, W, A)
  // are a whole number of 1-KiB loads (8 rows) for each of the 4 waves.
  static constexpr int kAR = RP < 32 ? 32 : RP;
  static constexpr int kRows = BT + BT + kAR;
  static constexpr int kLoads = kRows / 8 / 4;          // 1-KiB loads per wave per stage
  static_assert(kRows % 32 == 0, "whole loads per wave");
  static constexpr int kStageB = kRows * kF32BK * 4;
  // As many stages in flight as the LDS holds, up to 8.
  static constexpr int kFit = 160 * 1024 / kStageB;
  static constexpr int STAGES = kFit > 8 ? 8 : kFit;
  static_assert(STAGES >= 2 && (STAGES - 2) * kLoads < 64, "ring depth");
  static constexpr int kES = RP + 4;
  static constexpr int kEpiB = (BT + BT) * kES * 4;
  static constexpr int kLds = STAGES * kStageB > kEpiB ? STAGES * kStageB : kEpiB;
  static_assert(kLds <= 160 * 1024, "LDS budget");
  static constexpr int kTTiles = TW * RB;              // T tiles per wave row
  static constexpr int kTSlots = (kTTiles + 1) / 2;    // split over the 2 waves of a row
  // T tile ownership within a wave row: with an even number of rank blocks,
  // wave wn takes rank blocks [wn RB / 2, (wn + 1) RB / 2) of every row
  // block (slot i RB / 2 + t), so its A fragments are the same for all row
  // blocks; with one rank block, row block i goes to wave i % 2 (slot i / 2).
  static constexpr bool kTHalf = RB % 2 == 0;
  static constexpr int kTB = kTHalf ? RB / 2 : 1;      // A fragments per wave and k step
};

// Byte offset of float k of staged row `row`: 16-B chunk k / 4 sits at
// chunk ^ (row % 8).
__device__ __forceinline__ int f32_off(int row, int k) {
  return row * (kF32BK * 4) + ((((k >> 2) ^ (row & 7)) << 4) | ((k & 3) << 2));
}

template <int RP, int BT>
__global__ __launch_bounds__(kF32Threads) void fwd_tiled_f32_kernel(
    int M, int N, int K, int r, const float* __restrict__ X, int64_t ldx,
    const float* __restrict__ W, int64_t ldw, const float* __restrict__ A, int64_t lda,
    const float* __restrict__ B, int64_t ldb, float scale, float* __restrict__ Y, int64_t ldy,
    int tiles_n) {
  using C = F32Cfg<RP, BT>;
  constexpr int TW = C::TW, HB = BT / 2;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];
  float* smem = reinterpret_cast<float*>(smem_raw);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = lane & 15, lk = lane >> 4;
  const int m0 = (blockIdx.x / tiles_n) * BT;
  const int n0 = (blockIdx.x % tiles_n) * BT;

  f32x4 acc[TW][TW];
  f32x4 tacc[C::kTSlots];
  for (int i = 0; i < TW; ++i)
    for (int j = 0; j < TW; ++j) acc[i][j] = zero4();
  for (int s = 0; s < C::kTSlots; ++s) tacc[s] = zero4();

  // Buffer resources from each operand tile's first row to its last valid
  // row: rows past M, N or r read as zeros.
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(X + (int64_t)m0 * ldx), 0, (int)(min(BT, M - m0) * ldx * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + (int64_t)n0 * ldw), 0, (int)(min(BT, N - n0) * ldw * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)A, 0, (int)(r * lda * 4), 0x00020000);
  // Load q of a stage (q = wave + 4 i) covers staged rows [8 q, 8 q + 8); lane
  // l writes row 8 q + l / 8, physical chunk l % 8, i.e. logical chunk
  // (l % 8) ^ (row % 8) (row % 8 = l / 8).
  const int lr = lane >> 3;
  const int lc = (lane & 7) ^ lr;
  auto issue = [&](int slot, int k0) {
    unsigned char* base = smem_raw + slot * C::kStageB;
    const bool kin = k0 + lc * 4 < K;
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int q = wave + 4 * i;
      const int row = q * 8 + lr;  // staged row (q wave-uniform)
      __amdgpu_buffer_rsrc_t rs;
      uint32_t off;
      if (q * 8 < BT) {
        rs = rx;
        off = (uint32_t)row * (uint32_t)ldx * 4;
      } else if (q * 8 < 2 * BT) {
        rs = rw;
        off = (uint32_t)(row - BT) * (uint32_t)ldw * 4;
      } else {
        rs = ra;
        off = (uint32_t)(row - 2 * BT) * (uint32_t)lda * 4;
      }
      off += (uint32_t)(k0 + lc * 4) * 4;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(base + q * 1024), 16,
                                               kin ? off : 0x80000000u, 0, 0, 0);
    }
  };

  constexpr int S = C::STAGES;
  const int nk = (K + kF32BK - 1) / kF32BK;
#pragma unroll
  for (int st = 0; st < S - 1; ++st) issue(st, st * kF32BK);
  for (int kt = 0; kt < nk; ++kt) {
    // Stage kt has landed (S - 2 newer stages may still be in flight) for
    // every wave after the barrier; the barrier also ends every read of the
    // slot the next issue refills (stage kt - 1's).
    wait_vmcnt<(S - 2) * C::kLoads>();
    __builtin_amdgcn_s_barrier();
    issue((kt + S - 1) % S, (kt + S - 1) * kF32BK);
    const unsigned char* xs = smem_raw + (kt % S) * C::kStageB;
    const unsigned char* ws = xs + BT * kF32BK * 4;
    const unsigned char* as = ws + BT * kF32BK * 4;
    // The stage's fragments first (X, W and this wave's A ones), then the
    // MFMAs: read and multiplied in turn, each 4-deep k step waited for its
    // own LDS reads.
    constexpr int KS = kF32BK / 4;
    float a[KS][TW], b[KS][TW], bt[KS][C::kTB];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int kc = ks * 4 + lk;
#pragma unroll
      for (int i = 0; i < TW; ++i)
        a[ks][i] = *reinterpret_cast<const float*>(xs + f32_off(wm * HB + i * 16 + lrow, kc));
#pragma unroll
      for (int j = 0; j < TW; ++j)
        b[ks][j] = *reinterpret_cast<const float*>(ws + f32_off(wn * HB + j * 16 + lrow, kc));
#pragma unroll
      for (int t = 0; t < C::kTB; ++t) {
        const int tj = C::kTHalf ? wn * C::kTB + t : 0;
        bt[ks][t] = *reinterpret_cast<const float*>(as + f32_off(tj * 16 + lrow, kc));
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every read of the stage ahead of the MFMAs
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int kc = ks * 4 + lk;
#pragma unroll
      for (int i = 0; i < TW; ++i)
#pragma unroll
        for (int j = 0; j < TW; ++j) acc[i][j] = mfma16x16x4f32(a[ks][i], b[ks][j], acc[i][j]);
      if constexpr (C::kTHalf) {
#pragma unroll
        for (int i = 0; i < TW; ++i)
#pragma unroll
          for (int t = 0; t < C::kTB; ++t)
            tacc[i * C::kTB + t] = mfma16x16x4f32(a[ks][i], bt[ks][t], tacc[i * C::kTB + t]);
      } else {
#pragma unroll
        for (int i = 0; i < TW; ++i) {
          if ((i & 1) != wn) continue;
          tacc[i >> 1] = mfma16x16x4f32(a[ks][i], bt[ks][0], tacc[i >> 1]);
        }
      }
    }
    // This wave's reads of stage kt are done before the next barrier.
    wait_lgkm0();
  }
  // Loads of the stages past K (zeros) land before the epilogue reuses LDS.
  wait_vmcnt<0>();
  __syncthreads();

  // Epilogue: scaled fp32 T and the B tile in LDS, then acc += (s T) B^T.
  float* ts = smem;
  float* bs = smem + BT * C::kES;
#pragma unroll
  for (int i = 0; i < TW; ++i)
#pragma unroll
    for (int t = 0; t < C::kTB; ++t) {
      if (!C::kTHalf && (i & 1) != wn) continue;
      const int sl = C::kTHalf ? i * C::kTB + t : i >> 1;
      const int j = (C::kTHalf ? wn * C::kTB + t : 0) * 16 + lrow;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        ts[(wm * HB + i * 16 + lk * 4 + q) * C::kES + j] = j < r ? scale * tacc[sl][q] : 0.f;
    }
  for (int e = tid; e < BT * RP; e += kF32Threads) {
    const int n = e / RP, j = e % RP;
    bs[n * C::kES + j] = (j < r && n0 + n < N) ? B[(int64_t)(n0 + n) * ldb + j] : 0.f;
  }
  __syncthreads();
#pragma unroll 4
  for (int js = 0; js < RP / 4; ++js) {
    const int jc = js * 4 + lk;
    float a[TW], b[TW];
    for (int i = 0; i < TW; ++i) a[i] = ts[(wm * HB + i * 16 + lrow) * C::kES + jc];
    for (int j = 0; j < TW; ++j) b[j] = bs[(wn * HB + j * 16 + lrow) * C::kES + jc];
    for (int i = 0; i < TW; ++i)
      for (int j = 0; j < TW; ++j) acc[i][j] = mfma16x16x4f32(a[i], b[j], acc[i][j]);
  }

#pragma unroll
  for (int i = 0; i < TW; ++i)
#pragma unroll
    for (int j = 0; j < TW; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int gm = m0 + wm * HB + i * 16 + lk * 4 + q;
        const int gn = n0 + wn * HB + j * 16 + lrow;
        if (gm < M && gn < N) Y[(int64_t)gm * ldy + gn] = acc[i][j][q];
      }
}

template <int RP, int BT>
hipError_t launch_f32_bt(const FwdArgs& a, hipStream_t s) {
  using C = F32Cfg<RP, BT>;
  const int tiles_m = (int)((a.M + BT - 1) / BT);
  const int tiles_n = (int)((a.N + BT - 1) / BT);
  auto kern = fwd_tiled_f32_kernel<RP, BT>;
  static std::atomic<uint64_t> attr_done{0};
  if (hipError_t e = ensure_lds(kern, C::kLds, attr_done); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(tiles_m * tiles_n), dim3(kF32Threads), C::kLds, s, (int)a.M,
                     (int)a.N, (int)a.K, (int)a.r, static_cast<const float*>(a.X), a.ldx,
                     static_cast<const float*>(a.W), a.ldw, static_cast<const float*>(a.A), a.lda,
                     static_cast<const float*>(a.B), a.ldb, a.scale, static_cast<float*>(a.Y),
                     a.ldy, tiles_n);
  return hipGetLastError();
}

// 32 x 32 tiles when 64 x 64 ones would leave most CUs idle (fewer than 128
// workgroups): four times the workgroups, each with a quarter of the work
// per stage.
template <int RP>
hipError_t launch_f32(const FwdArgs& a, hipStream_t s) {
  const int64_t t64 = ((a.M + 63) / 64) * ((a.N + 63) / 64);
  if (t64 < 128) return launch_f32_bt<RP, 32>(a, s);
  return launch_f32_bt<RP, 64>(a, s);
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
