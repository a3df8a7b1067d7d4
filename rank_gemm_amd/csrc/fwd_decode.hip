// fwd_decode.hip -- fused LoRA linear forward for few tokens (M <= 64), bf16.
//
// Same layer as the tiled kernel (defined in "fastaf: Minimal LoRA fine-tuning
// with hand-written Triton kernels", section "FWD kernel speedup"), shaped for
// decode: the cost is streaming W once from HBM, so the kernel is organised
// around that stream instead of around output tiles.
//
// Per workgroup: 16 output columns (16 rows of W), NW waves.  K is cut into
// 128-deep blocks dealt round-robin to the waves.  Substep q of a block is
// one 16-B load per lane: lane l reads row l % 16 at k = 128 b + 32 q +
// 8 (l / 16), so the four lanes of a row read 64 contiguous bytes and one
// load instruction touches 16 row segments.  That is the operand layout of
// v_mfma_f32_16x16x32_bf16 for the k range [128 b + 32 q, +32), the same for
// the X, W and A operands, so the MFMA accumulates
//   Ybase[m, n] += X W^T   and   T[m, j] += X A^T   (T stays on chip)
// straight from the loaded registers.  All loads of a round (U blocks) are
// issued before its MFMAs, W first: U * 4 KiB of W per wave in flight.  X and
// A are small and come from L2; rows past M, N or r and k past K read as zero
// (buffer loads outside the resource's range return 0).
//
// The waves' partial sums are added in a fixed order through LDS
// (deterministic), then the epilogue adds scale * T B^T in fp32 on the VALU
// and stores bf16 (one rounding).
#include <algorithm>
#include <atomic>

#include "common.h"
#include "kernels.h"

namespace lora {
namespace {

constexpr uint32_t kDecOob = 0x80000000u;  // offset past any resource's range


// AL: A reaches the waves through LDS: each
// wave stages the rows of its own K range with 16-B-per-lane DMA loads
// (buffer_load ... lds), whole 128-B lines per instruction, instead of
// 16-row x 64-B register loads; the MFMA fragments are then read from LDS.
template <int MB, int RB, int U, int NW, bool AL, bool TP = false>
struct Dec {
  static constexpr int RP = RB * 16;
  static constexpr int kRowB = U * 256;                   // bytes of a staged row per round
  static constexpr int kChunks = U * 16;                  // 16-B chunks per staged row
  static constexpr int kAB = AL && !TP ? NW * RP * kRowB : 0;  // per-wave A regions
  static constexpr int kSlots = MB * (1 + RB);            // f32x4 partials per lane
  static constexpr int kRedB = NW * kSlots * kWave * 16;  // LDS for the reduction
  static constexpr int kTS = RP + 1;                      // T row stride (floats)
  static constexpr int kTB = MB * 16 * kTS * 4;           // T rows for the epilogue
  static constexpr int kRedOff = kAB;
  static constexpr int kLds = kRedOff + kRedB + kTB;
  static_assert(kLds <= 160 * 1024, "LDS budget");
  static_assert(!AL || (MB == 1 && (kRowB == 512 || kRowB == 1024)), "LDS staging shape");
};

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// One workgroup's work: output columns [n0, n0 + 16) of one forward.
// TP: T = X A^T was computed beforehand (tp: the NW per-wave partial sums,
// as dec_t_kernel writes them); A is neither loaded nor multiplied here.
template <int MB, int RB, int U, int NW, bool AL, bool TP = false>
__device__ __forceinline__ void dec_body(
    int M, int N, int K, int r, const uint16_t* __restrict__ X, int64_t ldx,
    const uint16_t* __restrict__ W, int64_t ldw, const uint16_t* __restrict__ A, int64_t lda,
    const uint16_t* __restrict__ B, int64_t ldb, float scale, uint16_t* __restrict__ Y,
    int64_t ldy, int b_vec, int n0, unsigned char* smem, const f32x4* __restrict__ tp = nullptr) {
  static_assert(!TP || MB == 1, "precomputed T: one 16-row block of tokens");
  using C = Dec<MB, RB, U, NW, AL, TP>;
  constexpr int RP = C::RP;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 15, lg = lane >> 4;

  // Lanes of rows past N (or M) read row N - 1 (M - 1) again: those MFMA
  // rows and columns are never stored, and the repeated addresses cost no
  // extra memory traffic.  Rank rows past r read as zero (the epilogue sums
  // only j < r, but zero rows keep T finite there).
  const int wrows = min(16, N - n0);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + (int64_t)n0 * ldw), 0, (int)(wrows * ldw * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)X, 0, (int)(M * ldx * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)A, 0, (int)(r * lda * 2), 0x00020000);
  const uint32_t lane_k = lg * 16;  // byte offset of the lane's 16-B piece in a substep
  const uint32_t wbase = min(lrow, wrows - 1) * (uint32_t)ldw * 2 + lane_k;
  uint32_t xbase[MB], abase[RB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
    xbase[mb] = min(mb * 16 + lrow, M - 1) * (uint32_t)ldx * 2 + lane_k;
#pragma unroll
  for (int jb = 0; jb < RB; ++jb) abase[jb] = (jb * 16 + lrow) * (uint32_t)lda * 2 + lane_k;

  // The epilogue's B row (lane: row n0 + l % 16), loaded now by the waves
  // that run the epilogue, so its latency hides behind the W stream; masking
  // past r waits for the epilogue, so nothing here waits on these loads.
  // b_vec holds only when r % 8 == 0 (and rows are 16-B aligned), so every
  // chunk min(8 c, r - 8) lies inside the row's r elements; otherwise the
  // epilogue reads B element by element.
  u32x4 bv[RP / 8];
  const int64_t brow = min(n0 + lrow, N - 1);
  if (b_vec && wave < MB) {
#pragma unroll
    for (int c = 0; c < RP / 8; ++c)
      bv[c] = *reinterpret_cast<const u32x4*>(B + brow * ldb + min(c * 8, (r - 1) & ~7));
  }

  f32x4 yacc[MB], tacc[MB][RB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    yacc[mb] = zero4();
#pragma unroll
    for (int jb = 0; jb < RB; ++jb) tacc[mb][jb] = zero4();
  }

  // Wave w takes U consecutive 128-deep blocks per round: K range
  // [128 kbw, 128 (kbw + U)) with kbw = (round NW + w) U.
  const int nkb = (K + 127) >> 7;
  unsigned char* as = smem + wave * (RP * C::kRowB);            // AL: this wave's A rows
  for (int kbw = wave * U; kbw < nkb; kbw += NW * U) {
    // Byte offset of each (block, substep) chunk within a row, or past the
    // range when the 8-element chunk lies beyond K.
    uint32_t off[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = kbw + u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = kb * 128 + q * 32 + lg * 8;
        off[u][q] = k < K ? (uint32_t)(kb * 256 + q * 64) : kDecOob;
      }
    }
    // X and A first: they come from L2 and leave the L1's miss queue
    // quickly, and the T MFMAs run on them while W streams in behind.
    u32x4 w[U][4], a[U][RB][4], x[U][MB][4];
    if constexpr (AL) {
      // Staged row j holds chunk c of the round's K range in slot c ^ (j % 16)
      // (conflict-free 16-row fragment reads); a 1-KiB DMA covers
      // 1024 / kRowB rows, lane i writing slot i % kChunks.
      constexpr int kRowsPerDma = 1024 / C::kRowB;
#pragma unroll
      for (int d = 0; d < (TP ? 0 : RP / kRowsPerDma); ++d) {
        const int j = d * kRowsPerDma + lane / C::kChunks;
        const int c = (lane % C::kChunks) ^ (j & 15);
        const int k = kbw * 128 + c * 8;
        const uint32_t vo = k < K ? (uint32_t)j * (uint32_t)lda * 2 + (uint32_t)k * 2 : kDecOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(as + d * 1024), 16, vo, 0, 0, 0);
      }
      // Nothing below may be scheduled before the DMAs: the wait further
      // down counts on them being the oldest loads of the round.
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) x[u][0][q] = bload(rx, xbase[0] + off[u][q]);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) x[u][mb][q] = bload(rx, xbase[mb] + off[u][q]);
          if constexpr (!TP) {
#pragma unroll
            for (int jb = 0; jb < RB; ++jb) a[u][jb][q] = bload(ra, abase[jb] + off[u][q]);
          }
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) w[u][q] = bload(rw, wbase + off[u][q]);
    // Keep the whole round's loads in flight: no MFMA (and no wait) is
    // scheduled before the last load is issued.
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (AL) {
      // The DMAs were issued first: waiting until only the later register
      // loads (X and W) are outstanding completes them.
      wait_vmcnt<U * 4 * 2>();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = u * 16 + q * 4 + lg;
#pragma unroll
          for (int jb = 0; jb < (TP ? 0 : RB); ++jb) {
            const int j = jb * 16 + lrow;
            a[u][jb][q] = *reinterpret_cast<const u32x4*>(as + j * C::kRowB + ((c ^ lrow) << 4));
          }
        }
    }
    if constexpr (!TP) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int jb = 0; jb < RB; ++jb)
              tacc[mb][jb] = mfma16x16x32(x[u][mb][q], a[u][jb][q], tacc[mb][jb]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) yacc[mb] = mfma16x16x32(x[u][mb][q], w[u][q], yacc[mb]);
  }

  // Cross-wave reduction in a fixed order (wave 0 + wave 1 + ...).
  f32x4* red = reinterpret_cast<f32x4*>(smem + C::kRedOff);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    red[(wave * C::kSlots + mb * (1 + RB)) * kWave + lane] = yacc[mb];
#pragma unroll
    for (int jb = 0; jb < RB; ++jb)
      red[(wave * C::kSlots + mb * (1 + RB) + 1 + jb) * kWave + lane] = tacc[mb][jb];
  }
  __syncthreads();
  const bool active = wave < MB;
  const int mb = active ? wave : 0;
  f32x4 y = zero4();
  float* tl = reinterpret_cast<float*>(smem + C::kRedOff + C::kRedB) + mb * 16 * C::kTS;
  if (active) {
    f32x4 t[RB];
#pragma unroll
    for (int jb = 0; jb < RB; ++jb) t[jb] = zero4();
    for (int w = 0; w < NW; ++w) {
      y += red[(w * C::kSlots + mb * (1 + RB)) * kWave + lane];
#pragma unroll
      for (int jb = 0; jb < RB; ++jb) {
        if constexpr (TP) {
          t[jb] += tp[(w * RB + jb) * kWave + lane];  // the same order as below
        } else {
          t[jb] += red[(w * C::kSlots + mb * (1 + RB) + 1 + jb) * kWave + lane];
        }
      }
    }
    // T rows of this M block to LDS (accumulator layout: lane holds column
    // j = 16 jb + l % 16 of rows 4 (l / 16) + q).
#pragma unroll
    for (int jb = 0; jb < RB; ++jb)
#pragma unroll
      for (int q = 0; q < 4; ++q) tl[(lg * 4 + q) * C::kTS + jb * 16 + lrow] = t[jb][q];
  }
  __syncthreads();
  if (!active) return;
  // L[m, n] = sum_j T[m, j] B[n, j]; Y = Ybase + scale * L, rounded once.
  const int n = n0 + lrow;
  if (n >= N) return;
  // Branch-free: every load below is issued before any is waited on (a
  // branch per rank element serialised one memory round trip each).  B is
  // read at indices clamped into the row and zeroed past r; T's columns past
  // r are zero (A rows past r read as zeros), so all RP terms can be summed.
  float bn[RP];
  if (b_vec) {
#pragma unroll
    for (int j = 0; j < RP; ++j) {
      const uint32_t h = (bv[j >> 3][(j >> 1) & 3] >> ((j & 1) * 16)) & 0xFFFFu;
      bn[j] = j < r ? bf2f((uint16_t)h) : 0.f;
    }
  } else {
    uint16_t bh[RP];
#pragma unroll
    for (int j = 0; j < RP; ++j) bh[j] = B[brow * ldb + min(j, r - 1)];
#pragma unroll
    for (int j = 0; j < RP; ++j) bn[j] = j < r ? bf2f(bh[j]) : 0.f;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int m = mb * 16 + lg * 4 + q;
    const float* trow = tl + (lg * 4 + q) * C::kTS;
    float l = 0.f;
#pragma unroll
    for (int j = 0; j < RP; ++j) l += trow[j] * bn[j];
    if (m < M) Y[(int64_t)m * ldy + n] = f2bf(y[q] + scale * l);
  }
}

template <int MB, int RB, int U, int NW, bool AL>
__global__ __launch_bounds__(NW * 64) void fwd_decode_bf16_kernel(
    int M, int N, int K, int r, const uint16_t* __restrict__ X, int64_t ldx,
    const uint16_t* __restrict__ W, int64_t ldw, const uint16_t* __restrict__ A, int64_t lda,
    const uint16_t* __restrict__ B, int64_t ldb, float scale, uint16_t* __restrict__ Y,
    int64_t ldy, int b_vec) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  dec_body<MB, RB, U, NW, AL>(M, N, K, r, X, ldx, W, ldw, A, lda, B, ldb, scale, Y, ldy, b_vec,
                                  blockIdx.x * 16, smem);
}

// One token (M = 1): the same workgroup partition (16 rows of W per
// workgroup, 8 waves splitting K), but every operand is loaded as whole 128-B
// lines -- lane l reads row 8 h + l / 8 of a 16-row block at k = 64 s +
// 8 (l % 8), so one 16-B-per-lane load covers 8 rows x 128 B -- and the dot
// products run on the VALU (v_dot2_f32_bf16): with one token the MFMA's 16
// token rows would be 15/16 idle anyway, and its operand layout needs 16 rows
// x 64 B per load.  A load's cost in the load pipe follows the cache lines it
// touches, and each workgroup re-reads all of A next to its share of W, so
// whole-line loads of both cut the lines per byte in half (measured with a
// W-and-A stream alone: 7.9 against 10.1 us per launch for 32 MiB of W).
// Each lane accumulates its 8-element pieces of rows (8 h + l / 8) of Ybase
// and of T; the 8 lanes of a row are added by a fixed butterfly, the waves
// in wave order through LDS, and the epilogue is the decode kernel's.
//
// acc + the 8 products of p and q, in element-pair order.  (The pairs are
// taken as swizzles of the 8-wide vector: a dynamically indexed dword
// bit-cast to a pair miscompiled here to the first dword every time.)
__device__ __forceinline__ float dot8(const u32x4& p, const u32x4& q, float acc) {
  const bf16x8 pv = __builtin_bit_cast(bf16x8, p), qv = __builtin_bit_cast(bf16x8, q);
  acc = __builtin_amdgcn_fdot2_f32_bf16(pv.s01, qv.s01, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(pv.s23, qv.s23, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(pv.s45, qv.s45, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(pv.s67, qv.s67, acc, false);
  return acc;
}

// Device-scope (agent) accesses of the words one workgroup hands another
// within a launch: each is coherent across the XCDs' L2s by itself, so the
// hand-over needs no L2 write-back or invalidation, only completion order
// (the writer waits for its stores before it sets the flag; the reader
// issues its loads after the flag's value came back).
__device__ __forceinline__ void dev_store(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float dev_load(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(p),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Wait (the calling wave) until *flag holds tok, then clear it.  The wait is
// bounded (about 0.1 s): false if the value never came.
__device__ __forceinline__ bool dec_wait_flag(uint64_t* flag, uint64_t tok) {
  uint64_t v = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int it = 0; v != tok && it < (1 << 20); ++it) {
    __builtin_amdgcn_s_sleep(2);
    v = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __hip_atomic_store(flag, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v == tok;
}

// The 16 rows [n0, n0 + 16) of one forward.  TP: the T partial sums of the
// NW waves come from `tp` (RP floats per wave, as dec_row_t_wave writes
// them) and A is neither loaded nor multiplied.  flag (TP only, may be
// null): the partial sums are written by another workgroup of the same
// launch, which then stores `tok` into *flag; wave 0 waits for that value
// before it reads them, and sets the flag back to zero.
template <int RB, int R, bool TP>
__device__ __forceinline__ void dec_row_body(int N, int K, int r, const uint16_t* __restrict__ X,
                                             const uint16_t* __restrict__ W, int64_t ldw,
                                             const uint16_t* __restrict__ A, int64_t lda,
                                             const uint16_t* __restrict__ B, int64_t ldb,
                                             float scale, uint16_t* __restrict__ Y, int b_vec,
                                             int n0, const float* tp,
                                             uint64_t* flag = nullptr, uint64_t tok = 0) {
  constexpr int NW = 8, RP = RB * 16;
  static_assert(R <= 8 && 2 * RB * R + 2 * R < 64, "one 1-KiB X piece per wave and round");
  __shared__ float red[NW][16 + (TP ? 0 : RP)];
  __shared__ __attribute__((aligned(16))) unsigned char xsh[NW][1024];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 3, c = lane & 7;
  const int wrows = min(16, N - n0);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + (int64_t)n0 * ldw), 0, (int)(wrows * ldw * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)X, 0, K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)A, 0, (int)(r * lda * 2), 0x00020000);
  // Rows 8 h + g of the 16-row W block and of the rank blocks.
  const uint32_t wrow[2] = {(uint32_t)g * (uint32_t)ldw * 2, (uint32_t)(8 + g) * (uint32_t)ldw * 2};
  uint32_t arow[2 * RB];
#pragma unroll
  for (int q = 0; q < 2 * RB; ++q) arow[q] = (uint32_t)(8 * q + g) * (uint32_t)lda * 2;

  // The epilogue's B row (lane < 16: row n0 + lane), as in the decode kernel.
  u32x4 bv[RP / 8];
  const int64_t brow = min(n0 + (lane & 15), N - 1);
  if (b_vec && wave == 0 && lane < 16) {
#pragma unroll
    for (int q = 0; q < RP / 8; ++q)
      bv[q] = *reinterpret_cast<const u32x4*>(B + brow * ldb + min(q * 8, (r - 1) & ~7));
  }

  float yacc[2] = {0.f, 0.f};
  float tacc[2 * RB];
#pragma unroll
  for (int q = 0; q < 2 * RB; ++q) tacc[q] = 0.f;
  // Wave w takes R consecutive 64-deep segments per round.
  const int nseg = (K + 63) >> 6;
  for (int s0 = wave * R; s0 < nseg; s0 += NW * R) {
    u32x4 x[R], w[R][2], a[R][2 * RB];
    // The round's X piece (R segments of 128 B) by one DMA into this wave's
    // LDS slot, lane i chunk i; lanes past the round read zeros.
    {
      const int k = (s0 + (lane >> 3)) * 64 + c * 8;
      const uint32_t ko = (lane >> 3) < R && k < K ? (uint32_t)k * 2 : kDecOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)xsh[wave], 16, ko, 0, 0, 0);
    }
    // The DMA must stay the oldest load of the round (the wait below counts
    // on it).
    __builtin_amdgcn_sched_barrier(0);
    // Rank 16: W (from HBM) and A (from L2) segment by segment, W first
    // (1 x 4096 x 4096: 9.2 us against 10.0 with all A loads first).  Rank
    // 32, where A is twice W: all A loads first (1 x 9728 x 2560: 19.3
    // against 20.7 us interleaved).
    auto wload = [&](int u) {
      const int k = (s0 + u) * 64 + c * 8;
      const uint32_t ko = k < K ? (uint32_t)k * 2 : kDecOob;
#pragma unroll
      for (int h = 0; h < 2; ++h) w[u][h] = bload(rw, k < K ? wrow[h] + ko : kDecOob);
    };
    auto aload = [&](int u) {
      const int k = (s0 + u) * 64 + c * 8;
      const uint32_t ko = k < K ? (uint32_t)k * 2 : kDecOob;
#pragma unroll
      for (int q = 0; q < 2 * RB; ++q) a[u][q] = bload(ra, k < K ? arow[q] + ko : kDecOob);
    };
    if constexpr (TP) {
#pragma unroll
      for (int u = 0; u < R; ++u) wload(u);
    } else if constexpr (RB == 1) {
#pragma unroll
      for (int u = 0; u < R; ++u) {
        wload(u);
        aload(u);
      }
    } else {
#pragma unroll
      for (int u = 0; u < R; ++u) aload(u);
#pragma unroll
      for (int u = 0; u < R; ++u) wload(u);
    }
    // Every load of the round in flight before the first product; then the
    // X piece (all later loads may still be in flight) from LDS.
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<(TP ? 0 : 2 * RB * R) + 2 * R>();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < R; ++u) x[u] = *reinterpret_cast<const u32x4*>(&xsh[wave][u * 128 + c * 16]);
#pragma unroll
    for (int u = 0; u < R; ++u) {
      if constexpr (!TP) {
#pragma unroll
        for (int q = 0; q < 2 * RB; ++q) tacc[q] = dot8(a[u][q], x[u], tacc[q]);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) yacc[h] = dot8(w[u][h], x[u], yacc[h]);
    }
  }
  // The 8 lanes of a row: a fixed butterfly (every lane ends with the same
  // sum), then lane c == 0 of each row group publishes the wave's partials.
#pragma unroll
  for (int m = 1; m < 8; m <<= 1) {
#pragma unroll
    for (int h = 0; h < 2; ++h) yacc[h] += __shfl_xor(yacc[h], m);
    if constexpr (!TP) {
#pragma unroll
      for (int q = 0; q < 2 * RB; ++q) tacc[q] += __shfl_xor(tacc[q], m);
    }
  }
  if (c == 0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) red[wave][8 * h + g] = yacc[h];
    if constexpr (!TP) {
#pragma unroll
      for (int q = 0; q < 2 * RB; ++q) red[wave][16 + 8 * q + g] = tacc[q];
    }
  }
  __syncthreads();
  if (wave != 0) return;
  bool ready = true;
  if constexpr (TP) {
    if (flag != nullptr) ready = dec_wait_flag(flag, tok);
  }
  // Wave 0, lane l < 16 + RP: partial l summed over the waves in wave order
  // (l < 16: Ybase of row n0 + l; else T[l - 16]), each sum once; the row
  // lanes then take T by shuffles and add the rank sum in j order.  T's
  // columns past r are zero (A rows past r read as zeros) and B is zeroed
  // past r, so the rank loop needs no branch.
  float sl = 0.f;
  if (lane < 16) {
    for (int v = 0; v < NW; ++v) sl += red[v][lane];
  } else if (lane < 16 + RP) {
    for (int v = 0; v < NW; ++v) {
      if constexpr (TP) sl += dev_load(&tp[v * RP + lane - 16]);
      else sl += red[v][lane];
    }
  }
  float tv[RP];
#pragma unroll
  for (int j = 0; j < RP; ++j) tv[j] = __shfl(sl, 16 + j);
  if (lane >= 16) return;
  const int n = n0 + lane;
  if (n >= N) return;
  float l = 0.f;
  if (b_vec) {
#pragma unroll
    for (int j = 0; j < RP; ++j) {
      const uint32_t hw = (bv[j >> 3][(j >> 1) & 3] >> ((j & 1) * 16)) & 0xFFFFu;
      l += tv[j] * (j < r ? bf2f((uint16_t)hw) : 0.f);
    }
  } else {
    uint16_t bh[RP];
#pragma unroll
    for (int j = 0; j < RP; ++j) bh[j] = B[brow * ldb + min(j, r - 1)];
#pragma unroll
    for (int j = 0; j < RP; ++j) l += tv[j] * (j < r ? bf2f(bh[j]) : 0.f);
  }
  // A partial sum that never arrived (a wait past its bound) shows as NaN.
  Y[n] = ready ? f2bf(sl + scale * l) : (uint16_t)0x7FC0u;
}

template <int RB, int R>
__global__ __launch_bounds__(512) void fwd_decode_row_kernel(
    int N, int K, int r, const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
    int64_t ldw, const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B,
    int64_t ldb, float scale, uint16_t* __restrict__ Y, int b_vec) {
  dec_row_body<RB, R, false>(N, K, r, X, W, ldw, A, lda, B, ldb, scale, Y, b_vec,
                             blockIdx.x * 16, nullptr);
}

// Batched decode: up to kDecBatch forwards with the same M and rank class per
// launch, their descriptors in the kernel arguments (no device memory).
// Workgroups [first[t], first[t + 1]) belong to forward t; a workgroup finds
// its forward by a uniform binary search.
constexpr int kDecBatch = 24;
struct DecDesc {
  const uint16_t* X;
  const uint16_t* W;
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* Y;
  f32x4* tp;  // with a workspace: this forward's T partial sums (kDecTpBytes)
  int64_t ldx, ldw, lda, ldb, ldy;
  int N, K, r, b_vec;
  float scale;
};
struct DecBatch {
  int count, M;
  int first[kDecBatch + 1];
  DecDesc d[kDecBatch];
};

// T = X A^T of every forward of a batch, as the NW waves of dec_body with
// the same U would accumulate it: workgroup (t, w) is one wave doing exactly
// wave w's part (its 128-deep K blocks kbw = (round NW + w) U + u, the same
// X and A operands, the same MFMA order) and stores its accumulators; the
// batch kernel adds the NW partials in wave order, as its LDS reduction
// does.  A is read once per forward instead of once per 16 rows of W.
template <int RB, int U>
__global__ __launch_bounds__(64) void dec_t_kernel(const DecBatch args) {
  constexpr int NW = 8;
  const int t = blockIdx.x / NW, w = blockIdx.x % NW;
  const DecDesc& d = args.d[t];
  const int lane = threadIdx.x, lrow = lane & 15, lg = lane >> 4;
  const int M = args.M, K = d.K, r = d.r;
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)d.X, 0, (int)(M * d.ldx * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)d.A, 0, (int)(r * d.lda * 2), 0x00020000);
  const uint32_t lane_k = lg * 16;
  const uint32_t xbase = min(lrow, M - 1) * (uint32_t)d.ldx * 2 + lane_k;
  uint32_t abase[RB];
#pragma unroll
  for (int jb = 0; jb < RB; ++jb) abase[jb] = (jb * 16 + lrow) * (uint32_t)d.lda * 2 + lane_k;
  f32x4 tacc[RB];
#pragma unroll
  for (int jb = 0; jb < RB; ++jb) tacc[jb] = zero4();
  const int nkb = (K + 127) >> 7;
  for (int kbw = w * U; kbw < nkb; kbw += NW * U) {
    u32x4 x[U][4], a[U][RB][4];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kb = kbw + u, k = kb * 128 + q * 32 + lg * 8;
        const uint32_t off = k < K ? (uint32_t)(kb * 256 + q * 64) : kDecOob;
        x[u][q] = bload(rx, xbase + off);
#pragma unroll
        for (int jb = 0; jb < RB; ++jb) a[u][jb][q] = bload(ra, abase[jb] + off);
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int jb = 0; jb < RB; ++jb) tacc[jb] = mfma16x16x32(x[u][q], a[u][jb][q], tacc[jb]);
  }
#pragma unroll
  for (int jb = 0; jb < RB; ++jb) d.tp[(w * RB + jb) * kWave + lane] = tacc[jb];
}

template <int MB, int RB, int U, int NW, bool AL, bool TP>
__global__ __launch_bounds__(NW * 64) void fwd_decode_bf16_batch_kernel(const DecBatch args) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int b = blockIdx.x;
  int lo = 0, hi = args.count - 1;  // last t with first[t] <= b
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (args.first[mid] <= b) lo = mid; else hi = mid - 1;
  }
  const DecDesc& d = args.d[lo];
  dec_body<MB, RB, U, NW, AL, TP>(args.M, d.N, d.K, d.r, d.X, d.ldx, d.W, d.ldw, d.A, d.lda,
                                      d.B, d.ldb, d.scale, d.Y, d.ldy, d.b_vec,
                                      (b - args.first[lo]) * 16, smem, d.tp);
}

// 16-B loads of B rows: aligned rows whose rank is a multiple of 8 (no chunk
// reaches past a row's last element).
inline int dec_b_vec(const FwdArgs& a) {
  return ((reinterpret_cast<uintptr_t>(a.B) & 15) == 0) && (a.ldb % 8 == 0) && (a.r % 8 == 0);
}

// The descriptors of forwards a[i0, i1) (one workgroup per 16 rows of W);
// tws (may be null): kDecTpBytes of T partial sums per forward.  Returns
// the workgroup count.
inline int dec_batch_fill(DecBatch& bt, const FwdArgs* a, int i0, int i1, unsigned char* tws) {
  bt.count = i1 - i0;
  bt.M = (int)a[i0].M;
  int blocks = 0;
  for (int t = 0; t < bt.count; ++t) {
    const FwdArgs& f = a[i0 + t];
    bt.first[t] = blocks;
    f32x4* tp = tws ? reinterpret_cast<f32x4*>(tws + (size_t)t * kDecTpBytes) : nullptr;
    bt.d[t] = DecDesc{static_cast<const uint16_t*>(f.X), static_cast<const uint16_t*>(f.W),
                      static_cast<const uint16_t*>(f.A), static_cast<const uint16_t*>(f.B),
                      static_cast<uint16_t*>(f.Y), tp, f.ldx, f.ldw, f.lda, f.ldb, f.ldy,
                      (int)f.N, (int)f.K, (int)f.r, dec_b_vec(f), f.scale};
    blocks += (int)((f.N + 15) / 16);
  }
  bt.first[bt.count] = blocks;
  return blocks;
}

// One-token forwards of a batch: dec_row_body per forward, so each output
// is bitwise the one lora_fwd gives for it.  TP: T from the workspace.
template <int RB, int R, bool TP>
__global__ __launch_bounds__(512) void fwd_decode_row_batch_kernel(const DecBatch args) {
  const int b = blockIdx.x;
  int lo = 0, hi = args.count - 1;  // last t with first[t] <= b
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (args.first[mid] <= b) lo = mid; else hi = mid - 1;
  }
  const DecDesc& d = args.d[lo];
  dec_row_body<RB, R, TP>(d.N, d.K, d.r, d.X, d.W, d.ldw, d.A, d.lda, d.B, d.ldb, d.scale, d.Y,
                          d.b_vec, (b - args.first[lo]) * 16, reinterpret_cast<const float*>(d.tp));
}

// T of one one-token forward, one wave's share: exactly what wave `wave`
// of dec_row_body does for T -- the same segments, X piece (through this
// wave's 1 KiB of LDS, xsh), A loads, dot8 chains and butterfly -- stored
// as its RP partial sums (tp[wave * RP + j]).  The weight stream adds the
// eight in wave order, as dec_row_body's LDS reduction does, so T and Y are
// bitwise those of the single forward; A is read once per forward instead
// of once per 16 rows of W.
template <int RB, int R>
__device__ __forceinline__ void dec_row_t_wave(const DecDesc& d, int wave, int lane,
                                               unsigned char* xsh) {
  constexpr int NW = 8, RP = RB * 16;
  const int g = lane >> 3, c = lane & 7;
  const int K = d.K, r = d.r;
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)d.X, 0, K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)d.A, 0, (int)(r * d.lda * 2), 0x00020000);
  uint32_t arow[2 * RB];
#pragma unroll
  for (int q = 0; q < 2 * RB; ++q) arow[q] = (uint32_t)(8 * q + g) * (uint32_t)d.lda * 2;
  float tacc[2 * RB];
#pragma unroll
  for (int q = 0; q < 2 * RB; ++q) tacc[q] = 0.f;
  const int nseg = (K + 63) >> 6;
  for (int s0 = wave * R; s0 < nseg; s0 += NW * R) {
    u32x4 x[R], a[R][2 * RB];
    {
      const int k = (s0 + (lane >> 3)) * 64 + c * 8;
      const uint32_t ko = (lane >> 3) < R && k < K ? (uint32_t)k * 2 : kDecOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)xsh, 16, ko, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);  // the DMA stays the oldest load
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int k = (s0 + u) * 64 + c * 8;
      const uint32_t ko = k < K ? (uint32_t)k * 2 : kDecOob;
#pragma unroll
      for (int q = 0; q < 2 * RB; ++q) a[u][q] = bload(ra, k < K ? arow[q] + ko : kDecOob);
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<2 * RB * R>();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < R; ++u) x[u] = *reinterpret_cast<const u32x4*>(&xsh[u * 128 + c * 16]);
#pragma unroll
    for (int u = 0; u < R; ++u)
#pragma unroll
      for (int q = 0; q < 2 * RB; ++q) tacc[q] = dot8(a[u][q], x[u], tacc[q]);
  }
#pragma unroll
  for (int m = 1; m < 8; m <<= 1)
#pragma unroll
    for (int q = 0; q < 2 * RB; ++q) tacc[q] += __shfl_xor(tacc[q], m);
  float* tp = reinterpret_cast<float*>(d.tp);
  if (c == 0) {
#pragma unroll
    for (int q = 0; q < 2 * RB; ++q) dev_store(&tp[wave * RP + 8 * q + g], tacc[q]);
  }
}

// T of every one-token forward of a batch in a launch of its own: workgroup
// (t, w) is one wave doing wave w's share of forward t.
template <int RB, int R>
__global__ __launch_bounds__(64) void dec_row_t_kernel(const DecBatch args) {
  __shared__ __attribute__((aligned(16))) unsigned char xsh[1024];
  dec_row_t_wave<RB, R>(args.d[blockIdx.x / 8], blockIdx.x % 8, threadIdx.x, xsh);
}

// The T partial sums and the weight stream of one-token forwards in one
// launch.  Workgroups [0, count) compute T, one per forward (wave w doing
// wave w's share), then store `tok` into the flag of every weight
// workgroup of that forward (kDecFlagOff bytes into the forward's workspace
// slot, one 8-byte flag per 16 rows of W).  The weight workgroups follow;
// they stream W as in the two-launch form and wait for their flag only
// before the epilogue reads T.  Workgroups are dispatched in id order, so
// every T workgroup is running before any weight workgroup can wait on it.
// Each weight workgroup clears its flag after the wait, which leaves every
// flag zero at the end of a launch: a replayed graph reusing tok finds no
// stale value.
constexpr int kDecFlagOff = 1024;  // after the 8 x RP <= 256 partial sums
constexpr int kDecMaxFlags = (kDecTpBytes - kDecFlagOff) / 8;
constexpr int kDecFusedMinBlocks = 256;
template <int RB, int R>
__global__ __launch_bounds__(512) void fwd_decode_row_fused_kernel(const DecBatch args,
                                                                   uint64_t tok) {
  static_assert(8 * RB * 16 * 4 <= kDecFlagOff, "T partial sums below the flags");
  const int b = blockIdx.x;
  if (b < args.count) {
    __shared__ __attribute__((aligned(16))) unsigned char xsh[8][1024];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const DecDesc& d = args.d[b];
    dec_row_t_wave<RB, R>(d, wave, lane, xsh[wave]);
    // Every wave's partial sums (device-scope stores) complete before any
    // flag is set.
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    uint64_t* flags = reinterpret_cast<uint64_t*>(reinterpret_cast<unsigned char*>(d.tp) +
                                                  kDecFlagOff);
    const int nf = args.first[b + 1] - args.first[b];
    for (int i = threadIdx.x; i < nf; i += 512)
      __hip_atomic_store(&flags[i], tok, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int bw = b - args.count;
  int lo = 0, hi = args.count - 1;  // last t with first[t] <= bw
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (args.first[mid] <= bw) lo = mid; else hi = mid - 1;
  }
  const DecDesc& d = args.d[lo];
  uint64_t* flags =
      reinterpret_cast<uint64_t*>(reinterpret_cast<unsigned char*>(d.tp) + kDecFlagOff);
  const int wb = bw - args.first[lo];
  dec_row_body<RB, R, true>(d.N, d.K, d.r, d.X, d.W, d.ldw, d.A, d.lda, d.B, d.ldb, d.scale, d.Y,
                            d.b_vec, wb * 16, reinterpret_cast<const float*>(d.tp), flags + wb,
                            tok);
}

// The forwards a[i0, i1) (same M, same rank class) in one launch; with a
// workspace (tws: kDecTpBytes per forward) T first, in a launch of its own.
template <int MB, int RB, int U, bool AL>
hipError_t launch_dec_batch(const FwdArgs* a, int i0, int i1, unsigned char* tws, hipStream_t s) {
  constexpr int NW = 8;
  using C = Dec<MB, RB, U, NW, AL>;
  DecBatch bt{};
  const int blocks = dec_batch_fill(bt, a, i0, i1, tws);
  if constexpr (MB == 1) {
    if (tws != nullptr) {
      // Without A the W stream has the registers of rank 16 at any rank:
      // four 128-deep blocks per wave per round, A-less LDS staging of X.
      // (With rank 16 this is the single-forward kernel's own partition, so
      // the outputs stay bitwise; above it Y differs from it by rounding.)
      constexpr int UT = 4;
      using CT = Dec<1, RB, UT, NW, true, true>;
      static_assert(NW * RB * kWave * 16 <= kDecTpBytes, "T partials fit the workspace slot");
      hipLaunchKernelGGL((dec_t_kernel<RB, UT>), dim3(bt.count * NW), dim3(64), 0, s, bt);
      if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
      auto kern = fwd_decode_bf16_batch_kernel<1, RB, UT, NW, true, true>;
      static std::atomic<uint64_t> attr_done{0};
      if (hipError_t e = ensure_lds(kern, CT::kLds, attr_done); e != hipSuccess) return e;
      hipLaunchKernelGGL(kern, dim3(blocks), dim3(NW * 64), CT::kLds, s, bt);
      return hipGetLastError();
    }
  }
  auto kern = fwd_decode_bf16_batch_kernel<MB, RB, U, NW, AL, false>;
  static std::atomic<uint64_t> attr_done{0};
  if (hipError_t e = ensure_lds(kern, C::kLds, attr_done); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(NW * 64), C::kLds, s, bt);
  return hipGetLastError();
}

template <int MB, int RB, int U, bool AL = false>
hipError_t launch_dec(const FwdArgs& a, hipStream_t s) {
  constexpr int NW = 8;
  using C = Dec<MB, RB, U, NW, AL>;
  auto kern = fwd_decode_bf16_kernel<MB, RB, U, NW, AL>;
  static std::atomic<uint64_t> attr_done{0};
  if (hipError_t e = ensure_lds(kern, C::kLds, attr_done); e != hipSuccess) return e;
  const int blocks = (int)((a.N + 15) / 16);
  const int b_vec = dec_b_vec(a);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(NW * 64), C::kLds, s, (int)a.M, (int)a.N, (int)a.K,
                     (int)a.r, static_cast<const uint16_t*>(a.X), a.ldx,
                     static_cast<const uint16_t*>(a.W), a.ldw, static_cast<const uint16_t*>(a.A),
                     a.lda, static_cast<const uint16_t*>(a.B), a.ldb, a.scale,
                     static_cast<uint16_t*>(a.Y), a.ldy, b_vec);
  return hipGetLastError();
}

// Blocks per round: the loads of a round (16 U (1 + RB + MB) VGPRs) stay
// within about 200 registers.
// (One template choice for a single forward and for a batch of forwards
// with the same M and rank class: batch = nullptr launches a alone.)
template <int RB>
hipError_t launch_dec_rb(const FwdArgs& a, const FwdArgs* batch, int i0, int i1,
                         unsigned char* tws, hipStream_t s) {
#define LORA_DEC(MB, U, AL)                                                        \
  return batch ? launch_dec_batch<MB, RB, U, AL>(batch, i0, i1, tws, s)            \
               : launch_dec<MB, RB, U, AL>(a, s)
  switch ((a.M + 15) / 16) {
    case 1:
      LORA_DEC(1, (RB == 1 ? 4 : 2), true);
    case 2: LORA_DEC(2, 2, false);
    case 3: LORA_DEC(3, (RB == 1 ? 2 : 1), false);
    default: LORA_DEC(4, (RB == 1 ? 2 : 1), false);
  }
#undef LORA_DEC
}

}  // namespace

// One token: whole-line loads and VALU dot products (fwd_decode_row_kernel).
template <int RB, int R>
hipError_t launch_dec_row(const FwdArgs& a, hipStream_t s) {
  const int blocks = (int)((a.N + 15) / 16);
  hipLaunchKernelGGL((fwd_decode_row_kernel<RB, R>), dim3(blocks), dim3(512), 0, s, (int)a.N,
                     (int)a.K, (int)a.r, static_cast<const uint16_t*>(a.X),
                     static_cast<const uint16_t*>(a.W), a.ldw, static_cast<const uint16_t*>(a.A),
                     a.lda, static_cast<const uint16_t*>(a.B), a.ldb, a.scale,
                     static_cast<uint16_t*>(a.Y), dec_b_vec(a));
  return hipGetLastError();
}

// One-token forwards a[i0, i1) (same rank class) in one launch; with a
// workspace (tws: kDecTpBytes per forward) T is computed once per forward,
// by the first workgroups of the same launch (by a launch of its own when a
// forward has more 16-row blocks than its slot has flags).
template <int RB, int R>
hipError_t launch_dec_row_batch(const FwdArgs* a, int i0, int i1, unsigned char* tws,
                                hipStream_t s) {
  static_assert(8 * RB * 16 * 4 <= kDecTpBytes, "T partial sums fit the workspace slot");
  DecBatch bt{};
  const int blocks = dec_batch_fill(bt, a, i0, i1, tws);
  int most = 0;  // weight workgroups of the largest forward
  for (int t = 0; t < bt.count; ++t) most = std::max(most, bt.first[t + 1] - bt.first[t]);
  // With at most one weight workgroup per CU (256 on this chip) the stream
  // ends about when T does, and T's latency adds to it (1 x 4096 x 4096:
  // 11.1 us against 9.2 us recomputing T per workgroup); with more, T is
  // ready before the stream's last workgroups start (1 x 9728 x 2560 r16:
  // 13.4 against 15.9 us; q/k/v r16: 9.9 against 11.7 us).  Both ways give
  // the same bits.
  if (blocks <= kDecFusedMinBlocks) tws = nullptr;
  if (tws != nullptr && most <= kDecMaxFlags) {
    // A token per launch with the bit pattern of a signalling NaN (never a
    // partial sum's bits) and a nonzero count below it.
    static std::atomic<uint64_t> launches{0};
    const uint64_t tok = 0x7FF4000000000000ull | ((launches.fetch_add(1) + 1) & 0xFFFFFFFFFFFull);
    hipLaunchKernelGGL((fwd_decode_row_fused_kernel<RB, R>), dim3(bt.count + blocks), dim3(512),
                       0, s, bt, tok);
  } else if (tws != nullptr) {
    hipLaunchKernelGGL((dec_row_t_kernel<RB, R>), dim3(bt.count * 8), dim3(64), 0, s, bt);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL((fwd_decode_row_batch_kernel<RB, R, true>), dim3(blocks), dim3(512), 0, s,
                       bt);
  } else {
    hipLaunchKernelGGL((fwd_decode_row_batch_kernel<RB, R, false>), dim3(blocks), dim3(512), 0,
                       s, bt);
  }
  return hipGetLastError();
}

// 64-deep segments per wave and round of the one-token kernel: eight at
// rank 16; at rank 32, where the A rows take twice the registers, five when
// that covers K in one round of the 8 waves (K <= 2560: a second round for
// some waves would wait on the first one's products), else four.  The
// single forward and the batched forms take the same choice, so their
// partitions -- and outputs -- stay the same.
inline int row_segments(const FwdArgs& a) { return a.r <= 16 ? 8 : (a.K <= 2560 ? 5 : 4); }

hipError_t launch_fwd_decode_bf16(const FwdArgs& a, hipStream_t s) {
  if (a.M == 1) {
    switch (row_segments(a)) {
      case 8: return launch_dec_row<1, 8>(a, s);
      case 5: return launch_dec_row<2, 5>(a, s);
      default: return launch_dec_row<2, 4>(a, s);
    }
  }
  return a.r <= 16 ? launch_dec_rb<1>(a, nullptr, 0, 0, nullptr, s)
                   : launch_dec_rb<2>(a, nullptr, 0, 0, nullptr, s);
}

// ---- Scratch of the no-allocation batch entry point: the T partial sums of
// up to kNoAllocForwards forwards (kDecTpBytes each), one copy of the array
// per GPU, held until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: the device address is taken with
// hipGetSymbolAddress once per device and only that address is used.
static __device__ __align__(256) unsigned char scratch[kNoAllocForwards * kDecTpBytes];

hipError_t decode_scratch(void** out) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  static std::atomic<void*> ptrs[kMaxDevices];
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // With device `dev` current: the address of this device's copy.
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    ptrs[dev].store(p, std::memory_order_release);  // concurrent first calls store the same value
  }
  *out = p;
  return hipSuccess;
}

// Forwards a[0, count): same M (<= LORA_DECODE_MAX_M) and the same rank class
// (r <= 16, or 16 < r <= 32); kDecBatch at a time.
hipError_t launch_fwd_decode_bf16_batch(const FwdArgs* a, int count, void* tws, hipStream_t s) {
  unsigned char* w = static_cast<unsigned char*>(tws);
  for (int i = 0; i < count; i += kDecBatch) {
    const int j = i + kDecBatch < count ? i + kDecBatch : count;
    unsigned char* wi = w ? w + (size_t)i * kDecTpBytes : nullptr;
    hipError_t e = hipSuccess;
    if (a[i].M == 1) {
      // the one-token kernel of lora_fwd, per forward: one launch per run of
      // forwards with the same segment count
      for (int k = i; k < j && e == hipSuccess;) {
        int l = k + 1;
        while (l < j && row_segments(a[l]) == row_segments(a[k])) ++l;
        unsigned char* wk = w ? w + (size_t)k * kDecTpBytes : nullptr;
        switch (row_segments(a[k])) {
          case 8: e = launch_dec_row_batch<1, 8>(a, k, l, wk, s); break;
          case 5: e = launch_dec_row_batch<2, 5>(a, k, l, wk, s); break;
          default: e = launch_dec_row_batch<2, 4>(a, k, l, wk, s); break;
        }
        k = l;
      }
    } else
      e = a[i].r <= 16 ? launch_dec_rb<1>(a[i], a, i, j, wi, s)
                       : launch_dec_rb<2>(a[i], a, i, j, wi, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lora
