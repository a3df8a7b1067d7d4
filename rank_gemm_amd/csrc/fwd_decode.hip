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
#include "common.h"
#include "kernels.h"

namespace lora {
namespace {

constexpr uint32_t kDecOob = 0x80000000u;  // offset past any resource's range


// AL: A (and, with XL, the single X row) reach the waves through LDS: each
// wave stages the rows of its own K range with 16-B-per-lane DMA loads
// (buffer_load ... lds), whole 128-B lines per instruction, instead of
// 16-row x 64-B register loads; the MFMA fragments are then read from LDS.
template <int MB, int RB, int U, int NW, bool AL, bool XL, bool TP = false>
struct Dec {
  static constexpr int RP = RB * 16;
  static constexpr int kRowB = U * 256;                   // bytes of a staged row per round
  static constexpr int kChunks = U * 16;                  // 16-B chunks per staged row
  static constexpr int kAB = AL && !TP ? NW * RP * kRowB : 0;  // per-wave A regions
  static constexpr int kXB = XL ? NW * kRowB : 0;         // per-wave X row
  static constexpr int kSlots = MB * (1 + RB);            // f32x4 partials per lane
  static constexpr int kRedB = NW * kSlots * kWave * 16;  // LDS for the reduction
  static constexpr int kTS = RP + 1;                      // T row stride (floats)
  static constexpr int kTB = MB * 16 * kTS * 4;           // T rows for the epilogue
  static constexpr int kRedOff = kAB + kXB;
  static constexpr int kLds = kRedOff + kRedB + kTB;
  static_assert(kLds <= 160 * 1024, "LDS budget");
  static_assert(!AL || (MB == 1 && (kRowB == 512 || kRowB == 1024)), "LDS staging shape");
  static_assert(!XL || (AL && kRowB == 1024), "X staging: one full 1-KiB DMA per round");
};

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// One workgroup's work: output columns [n0, n0 + 16) of one forward.
// TP: T = X A^T was computed beforehand (tp: the NW per-wave partial sums,
// as dec_t_kernel writes them); A is neither loaded nor multiplied here.
template <int MB, int RB, int U, int NW, bool AL, bool XL, bool TP = false>
__device__ __forceinline__ void dec_body(
    int M, int N, int K, int r, const uint16_t* __restrict__ X, int64_t ldx,
    const uint16_t* __restrict__ W, int64_t ldw, const uint16_t* __restrict__ A, int64_t lda,
    const uint16_t* __restrict__ B, int64_t ldb, float scale, uint16_t* __restrict__ Y,
    int64_t ldy, int b_vec, int n0, unsigned char* smem, const f32x4* __restrict__ tp = nullptr) {
  static_assert(!TP || MB == 1, "precomputed T: one 16-row block of tokens");
  using C = Dec<MB, RB, U, NW, AL, XL, TP>;
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
  // Positions past r load a valid chunk of the row.  Rows that are not
  // 16-B aligned (ldb % 8 != 0) are read in the epilogue instead.
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
  unsigned char* xs = smem + C::kAB + wave * C::kRowB;          // XL: this wave's X row
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
      if constexpr (XL) {
        // The X row (M == 1): one 1-KiB DMA, lane i chunk i, unswizzled (all
        // sixteen row lanes read the same chunk: a broadcast).
        const int k = kbw * 128 + lane * 8;
        const uint32_t vo = k < K ? (uint32_t)k * 2 : kDecOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)xs, 16, vo, 0, 0, 0);
      }
      // Nothing below may be scheduled before the DMAs: the wait further
      // down counts on them being the oldest loads of the round.
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!XL) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int q = 0; q < 4; ++q) x[u][0][q] = bload(rx, xbase[0] + off[u][q]);
      }
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
      // loads (W, and X unless staged) are outstanding completes them.
      wait_vmcnt<U * 4 * (XL ? 1 : 2)>();
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
          if constexpr (XL) x[u][0][q] = *reinterpret_cast<const u32x4*>(xs + (c << 4));
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
  float bn[RP];
  if (b_vec) {
#pragma unroll
    for (int j = 0; j < RP; ++j) {
      const uint32_t h = (bv[j >> 3][(j >> 1) & 3] >> ((j & 1) * 16)) & 0xFFFFu;
      bn[j] = j < r ? bf2f((uint16_t)h) : 0.f;
    }
  } else {
#pragma unroll
    for (int j = 0; j < RP; ++j) bn[j] = j < r ? bf2f(B[brow * ldb + j]) : 0.f;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int m = mb * 16 + lg * 4 + q;
    if (m >= M) break;
    float l = 0.f;
#pragma unroll
    for (int j = 0; j < RP; ++j)
      if (j < r) l += tl[(lg * 4 + q) * C::kTS + j] * bn[j];
    Y[(int64_t)m * ldy + n] = f2bf(y[q] + scale * l);
  }
}

template <int MB, int RB, int U, int NW, bool AL, bool XL>
__global__ __launch_bounds__(NW * 64) void fwd_decode_bf16_kernel(
    int M, int N, int K, int r, const uint16_t* __restrict__ X, int64_t ldx,
    const uint16_t* __restrict__ W, int64_t ldw, const uint16_t* __restrict__ A, int64_t lda,
    const uint16_t* __restrict__ B, int64_t ldb, float scale, uint16_t* __restrict__ Y,
    int64_t ldy, int b_vec) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  dec_body<MB, RB, U, NW, AL, XL>(M, N, K, r, X, ldx, W, ldw, A, lda, B, ldb, scale, Y, ldy, b_vec,
                                  blockIdx.x * 16, smem);
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

template <int MB, int RB, int U, int NW, bool AL, bool XL, bool TP>
__global__ __launch_bounds__(NW * 64) void fwd_decode_bf16_batch_kernel(const DecBatch args) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int b = blockIdx.x;
  int lo = 0, hi = args.count - 1;  // last t with first[t] <= b
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (args.first[mid] <= b) lo = mid; else hi = mid - 1;
  }
  const DecDesc& d = args.d[lo];
  dec_body<MB, RB, U, NW, AL, XL, TP>(args.M, d.N, d.K, d.r, d.X, d.ldx, d.W, d.ldw, d.A, d.lda,
                                      d.B, d.ldb, d.scale, d.Y, d.ldy, d.b_vec,
                                      (b - args.first[lo]) * 16, smem, d.tp);
}

inline int dec_b_vec(const FwdArgs& a) {
  return ((reinterpret_cast<uintptr_t>(a.B) & 15) == 0) && (a.ldb % 8 == 0);
}

// The forwards a[i0, i1) (same M, same rank class) in one launch; with a
// workspace (tws: kDecTpBytes per forward) T first, in a launch of its own.
template <int MB, int RB, int U, bool AL, bool XL>
hipError_t launch_dec_batch(const FwdArgs* a, int i0, int i1, unsigned char* tws, hipStream_t s) {
  constexpr int NW = 8;
  using C = Dec<MB, RB, U, NW, AL, XL>;
  DecBatch bt{};
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
  if constexpr (MB == 1) {
    if (tws != nullptr) {
      // Without A the W stream has the registers of rank 16 at any rank:
      // four 128-deep blocks per wave per round, A-less LDS staging of X.
      // (With rank 16 this is the single-forward kernel's own partition, so
      // the outputs stay bitwise; above it Y differs from it by rounding.)
      constexpr int UT = 4;
      using CT = Dec<1, RB, UT, NW, true, XL, true>;
      static_assert(NW * RB * kWave * 16 <= kDecTpBytes, "T partials fit the workspace slot");
      hipLaunchKernelGGL((dec_t_kernel<RB, UT>), dim3(bt.count * NW), dim3(64), 0, s, bt);
      if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
      auto kern = fwd_decode_bf16_batch_kernel<1, RB, UT, NW, true, XL, true>;
      static std::atomic<uint64_t> attr_done{0};
      if (hipError_t e = ensure_lds(kern, CT::kLds, attr_done); e != hipSuccess) return e;
      hipLaunchKernelGGL(kern, dim3(blocks), dim3(NW * 64), CT::kLds, s, bt);
      return hipGetLastError();
    }
  }
  auto kern = fwd_decode_bf16_batch_kernel<MB, RB, U, NW, AL, XL, false>;
  static std::atomic<uint64_t> attr_done{0};
  if (hipError_t e = ensure_lds(kern, C::kLds, attr_done); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(NW * 64), C::kLds, s, bt);
  return hipGetLastError();
}

template <int MB, int RB, int U, bool AL = false, bool XL = false>
hipError_t launch_dec(const FwdArgs& a, hipStream_t s) {
  constexpr int NW = 8;
  using C = Dec<MB, RB, U, NW, AL, XL>;
  auto kern = fwd_decode_bf16_kernel<MB, RB, U, NW, AL, XL>;
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
#define LORA_DEC(MB, U, AL, XL)                                                    \
  return batch ? launch_dec_batch<MB, RB, U, AL, XL>(batch, i0, i1, tws, s)        \
               : launch_dec<MB, RB, U, AL, XL>(a, s)
  switch ((a.M + 15) / 16) {
    case 1:
      if constexpr (RB == 1) {
        if (a.M == 1) LORA_DEC(1, 4, true, true);
      }
      LORA_DEC(1, (RB == 1 ? 4 : 2), true, false);
    case 2: LORA_DEC(2, 2, false, false);
    case 3: LORA_DEC(3, (RB == 1 ? 2 : 1), false, false);
    default: LORA_DEC(4, (RB == 1 ? 2 : 1), false, false);
  }
#undef LORA_DEC
}

}  // namespace

hipError_t launch_fwd_decode_bf16(const FwdArgs& a, hipStream_t s) {
  return a.r <= 16 ? launch_dec_rb<1>(a, nullptr, 0, 0, nullptr, s)
                   : launch_dec_rb<2>(a, nullptr, 0, 0, nullptr, s);
}

// Forwards a[0, count): same M (<= LORA_DECODE_MAX_M) and the same rank class
// (r <= 16, or 16 < r <= 32); kDecBatch at a time.
hipError_t launch_fwd_decode_bf16_batch(const FwdArgs* a, int count, void* tws, hipStream_t s) {
  unsigned char* w = static_cast<unsigned char*>(tws);
  for (int i = 0; i < count; i += kDecBatch) {
    const int j = i + kDecBatch < count ? i + kDecBatch : count;
    unsigned char* wi = w ? w + (size_t)i * kDecTpBytes : nullptr;
    const hipError_t e = a[i].r <= 16 ? launch_dec_rb<1>(a[i], a, i, j, wi, s)
                                      : launch_dec_rb<2>(a[i], a, i, j, wi, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lora
