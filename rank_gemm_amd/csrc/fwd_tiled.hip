// fwd_tiled.hip -- fused LoRA linear forward, bf16 operands, fp32 accumulate,
// on gfx950 MFMA (v_mfma_f32_16x16x32_bf16).
//
// Computes Y = X W^T + scale * (X A^T) B^T (the layer defined in "fastaf:
// Minimal LoRA fine-tuning with hand-written Triton kernels", section "FWD
// kernel speedup") in ONE launch: the base product, the rank-r
// down-projection, the up-projection, the scale and the add all happen in one
// workgroup per output tile, and the [tokens, r] intermediate never leaves the
// chip (accumulator registers, then LDS for the operand re-layout).
//
// Per workgroup (BM x BN output tile, WM x WN waves, each wave a grid of
// 16 x 16 MFMA blocks):
//   K loop, BK = 32 per stage, STAGES-deep ring of LDS stages:
//     X[BM x 32], W[BN x 32] and A[RP x 32] go straight from global memory to
//     LDS (buffer_load ... lds, 16 B per lane, no register staging).  Each
//     buffer resource starts at the tile's first row and ends at the last
//     valid row, so rows past M, N or r and the K tail read as zeros.
//     Rows are 64 B; 16-B chunks are XOR-swizzled so that MFMA operand reads
//     (16 rows x one chunk per instruction) hit distinct banks.
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

typedef __attribute__((address_space(3))) void lds_void;

constexpr int BK = 32;          // k per LDS stage
constexpr int kRowB = BK * 2;   // bytes per staged row
// Buffer offset for a lane that must read zeros: past every valid range.
__device__ __forceinline__ uint32_t off_or_oob(bool in, uint32_t off) { return in ? off : 0x80000000u; }

// 16-B chunk swizzle within a 64-B row.  For the 16 rows one operand read
// touches, (row * 4 + chunk) takes 16 distinct values mod 16 and 8 distinct
// values mod 8 within each half, so it is conflict-free whether the LDS
// serves 8 lanes per 128 B or 16 lanes per 256 B.
// Depends on row & 15 only, so a 1-KiB load (16 rows) can apply it from the
// lane index alone.
__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ ((row >> 3) & 1)) & 3; }
__device__ __forceinline__ int stage_off(int row, int chunk) {
  return row * kRowB + ((chunk ^ swz(row)) << 4);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <int BM_, int BN_, int WM_, int WN_, int RP_, int ST_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, RP = RP_, STAGES = ST_;
  static constexpr int NW = WM * WN;
  static constexpr int NT = NW * kWave;
  static constexpr int TM = BM / WM / 16;
  static constexpr int TN = BN / WN / 16;
  static constexpr int RB = RP / 16;
  static constexpr int ROWS = BM + BN + RP;         // staged rows per stage
  static constexpr int kStageB = ROWS * kRowB;
  static constexpr int kXL = BM / 16 / NW;           // X loads (1 KiB each) per wave per stage
  static constexpr int kWL = BN / 16 / NW;           // W loads per wave per stage
  static constexpr int kAL = (RP / 16 + NW - 1) / NW;  // A load slots per wave per stage
  static constexpr int kLoadsMin = kXL + kWL + (RP / 16) / NW;  // fewest any wave issues
  static constexpr int kTS = RP + 8;                // epilogue T / B row stride (elements)
  static constexpr int kEpiB = (BM + BN) * kTS * 2;
  static constexpr int kYS = BN + 8;                // output staging row stride (elements)
  static constexpr int kYB = BM * kYS * 2;
  static constexpr int kLds = cmax(STAGES * kStageB, cmax(kEpiB, kYB));
  static constexpr int kTSlots = (TM * RB + WN - 1) / WN;
  static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "wave tiling");
  static_assert(BM % (16 * NW) == 0 && BN % (16 * NW) == 0, "X/W loads split evenly over waves");
  static_assert(kLds <= 160 * 1024, "LDS budget");
  static_assert(STAGES >= 2, "ring depth");
};

// Issue one stage of direct-to-LDS loads for this wave: its X slots, its W
// slots and (waves below RP / 16) its A slot.  Lanes whose 16-B chunk lies
// past K read zeros.
template <class C>
__device__ __forceinline__ void issue_stage(unsigned char* smem, int buf, int k0, int K, int wave,
                                            int lchunk, __amdgpu_buffer_rsrc_t rx,
                                            __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t ra,
                                            const uint32_t (&voffx)[C::kXL],
                                            const uint32_t (&voffw)[C::kWL],
                                            const uint32_t (&voffa)[C::kAL]) {
  const bool kin = k0 + lchunk * 8 < K;
  const uint32_t kb = (uint32_t)k0 * 2;
  unsigned char* base = smem + buf * C::kStageB;
#pragma unroll
  for (int s = 0; s < C::kXL; ++s)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(base + (wave + s * C::NW) * 1024), 16,
                                             off_or_oob(kin, voffx[s] + kb), 0, 0, 0);
#pragma unroll
  for (int s = 0; s < C::kWL; ++s)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rw, (lds_void*)(base + C::BM * kRowB + (wave + s * C::NW) * 1024), 16,
        off_or_oob(kin, voffw[s] + kb), 0, 0, 0);
#pragma unroll
  for (int s = 0; s < C::kAL; ++s)
    if (wave + s * C::NW < C::RP / 16)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (lds_void*)(base + (C::BM + C::BN) * kRowB + (wave + s * C::NW) * 1024), 16,
          off_or_oob(kin, voffa[s] + kb), 0, 0, 0);
}

template <class C>
__global__ __launch_bounds__(C::NT) void fwd_tiled_bf16_kernel(
    int M, int N, int K, int r, const uint16_t* __restrict__ X, int64_t ldx,
    const uint16_t* __restrict__ W, int64_t ldw, const uint16_t* __restrict__ A, int64_t lda,
    const uint16_t* __restrict__ B, int64_t ldb, float scale, uint16_t* __restrict__ Y,
    int64_t ldy, int tiles_m, int tiles_n, int y_vec) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  constexpr int BM = C::BM, BN = C::BN, RP = C::RP, RB = C::RB, TM = C::TM, TN = C::TN;
  constexpr int WN = C::WN, NW = C::NW, STAGES = C::STAGES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int lrow = lane & 15;
  const int lk = lane >> 4;

  // ---- tile id: XCD-contiguous, then grouped along M for L2 reuse of W.
  const int total = tiles_m * tiles_n;
  const int pid = xcd_contiguous_id(blockIdx.x, total);
  constexpr int kGroup = 8;
  const int group = pid / (kGroup * tiles_n);
  const int first_m = group * kGroup;
  const int gsize = min(tiles_m - first_m, kGroup);
  const int local = pid % (kGroup * tiles_n);
  const int m0 = (first_m + local % gsize) * BM;
  const int n0 = (local / gsize) * BN;

  // ---- buffer resources from the tile's first row to its last valid row.
  const int xrows = min(BM, M - m0);
  const int wrows = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(X + (int64_t)m0 * ldx), 0, (int)(xrows * ldx * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + (int64_t)n0 * ldw), 0, (int)(wrows * ldw * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)A, 0, (int)(r * lda * 2), 0x00020000);

  // Lane i of a 1-KiB load writes staged row (16q + i/4), physical chunk
  // i%4, so it fetches logical chunk (i%4) ^ swz(row).  Wave w issues X loads
  // q = w, w + NW, ..., the same for W, and A load q = w when w < RP / 16.
  const int lrow_in_load = lane >> 2;
  const int lchunk = (lane & 3) ^ swz(lrow_in_load);
  uint32_t voffx[C::kXL], voffw[C::kWL], voffa[C::kAL];
#pragma unroll
  for (int s = 0; s < C::kXL; ++s)
    voffx[s] = (uint32_t)(((wave + s * NW) * 16 + lrow_in_load) * ldx * 2 + lchunk * 16);
#pragma unroll
  for (int s = 0; s < C::kWL; ++s)
    voffw[s] = (uint32_t)(((wave + s * NW) * 16 + lrow_in_load) * ldw * 2 + lchunk * 16);
#pragma unroll
  for (int s = 0; s < C::kAL; ++s)
    voffa[s] = (uint32_t)(((wave + s * NW) * 16 + lrow_in_load) * lda * 2 + lchunk * 16);

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = zero4();
  f32x4 tacc[C::kTSlots];
#pragma unroll
  for (int s = 0; s < C::kTSlots; ++s) tacc[s] = zero4();

  // T tile (i, tj) belongs to wave (i * RB + tj) % WN of its wave row.
  bool uses_tj[RB];
#pragma unroll
  for (int tj = 0; tj < RB; ++tj) {
    bool u = false;
#pragma unroll
    for (int i = 0; i < TM; ++i) u |= ((i * RB + tj) % WN) == wn;
    uses_tj[tj] = u;
  }

  const int nk = (K + BK - 1) / BK;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue_stage<C>(smem, s, s * BK, K, wave, lchunk, rx, rw, ra, voffx, voffw, voffa);

  int buf = 0;
  for (int kt = 0; kt < nk; ++kt) {
    // Stage kt has landed once at most (STAGES - 2) later stages are in flight.
    // A bare s_barrier: each wave has waited for its own loads of stage kt,
    // and the operand reads of stage kt-1 completed before the MFMAs that
    // consumed them, so no fence (which would drain every in-flight stage)
    // is needed here.
    if (kt + STAGES - 2 < nk)
      wait_vmcnt<(STAGES - 2) * C::kLoadsMin>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    {
      const int nxt = kt + STAGES - 1;
      if (nxt < nk) {
        int nb = buf + STAGES - 1;
        if (nb >= STAGES) nb -= STAGES;
        issue_stage<C>(smem, nb, nxt * BK, K, wave, lchunk, rx, rw, ra, voffx, voffw, voffa);
      }
    }
    const unsigned char* xs = smem + buf * C::kStageB;
    const unsigned char* ws = xs + BM * kRowB;
    const unsigned char* as = ws + BN * kRowB;
    u32x4 a[TM], b[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
      a[i] = *reinterpret_cast<const u32x4*>(xs + stage_off(wm * TM * 16 + i * 16 + lrow, lk));
#pragma unroll
    for (int j = 0; j < TN; ++j)
      b[j] = *reinterpret_cast<const u32x4*>(ws + stage_off(wn * TN * 16 + j * 16 + lrow, lk));
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
#pragma unroll
    for (int tj = 0; tj < RB; ++tj) {
      if (!uses_tj[tj]) continue;
      const u32x4 bt = *reinterpret_cast<const u32x4*>(as + stage_off(tj * 16 + lrow, lk));
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int idx = i * RB + tj;
        if (idx % WN == wn) tacc[idx / WN] = mfma16x16x32(a[i], bt, tacc[idx / WN]);
      }
    }
    buf = buf + 1 == STAGES ? 0 : buf + 1;
  }
  __syncthreads();

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
  for (int e = tid; e < BN * RP; e += C::NT) {
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
  for (int e = tid; e < BM * kCPR; e += C::NT) {
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
  hipLaunchKernelGGL(kern, dim3(tiles_m * tiles_n), dim3(C::NT), C::kLds, s, (int)a.M, (int)a.N,
                     (int)a.K, (int)a.r, static_cast<const uint16_t*>(a.X), a.ldx,
                     static_cast<const uint16_t*>(a.W), a.ldw, static_cast<const uint16_t*>(a.A),
                     a.lda, static_cast<const uint16_t*>(a.B), a.ldb, a.scale,
                     static_cast<uint16_t*>(a.Y), a.ldy, tiles_m, tiles_n, y_vec);
  return hipGetLastError();
}

// Tile shapes.  Large: 256 x 256, 8 waves (2 x 4), wave tile 128 x 64.
// Medium: 128 x 128, 4 waves (2 x 2), wave tile 64 x 64.
template <int RP>
using Big = Cfg<256, 256, 2, 4, RP, 4>;
template <int RP>
using Mid = Cfg<128, 128, 2, 2, RP, 4>;

template <int RP>
hipError_t launch_rp(const FwdArgs& a, hipStream_t s) {
  const int64_t big_tiles = ((a.M + 255) / 256) * ((a.N + 255) / 256);
  if constexpr (RP <= 64) {
    if (big_tiles >= 256) return launch<Big<RP>>(a, s);
  }
  return launch<Mid<RP>>(a, s);
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
