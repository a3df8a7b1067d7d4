// bwd.hip -- backward of the fused LoRA linear layer, bf16 operands, fp32
// accumulation, on gfx950 MFMA.
//
// With the base weight frozen, the backward of Y = X W^T + s (X A^T) B^T (the
// gradients dA, dB and dX of "fastaf: Minimal LoRA fine-tuning with
// hand-written Triton kernels", section "BWD kernel speedup") is
//   T  = X A^T   [M, r]           G  = dY B    [M, r]
//   dX = dY W + s G A             the forward of dY with W' = W^T, A' = B^T,
//                                 B' = A^T, on the tiled forward kernel
//   dA = s G^T X  [r, K]          dB = s dY^T T  [N, r]
// dA and dB contract over the tokens.  That page found a loop over the whole
// sequence inside one program per output block starves the GPU, and moved dA
// to a token-parallel split with atomic adds.  Here both are split over S
// token ranges, each range writing fp32 partial sums that a second kernel
// adds in a fixed order: every CU has work and the result is deterministic.
//
// Launches, in stream order, all through the caller's workspace.  With dX:
//   1. proj_kernel   (s T)^T = s A X^T, [r, Mp] bf16, and in the same grid
//                    the preparation: W^T [K, N], B^T [r, N], A^T [K, r]
//   2. dX: the tiled forward kernel on (dY, W^T, B^T, A^T); its rank
//      intermediate is s dY B = s G, which it also stores as (s G)^T
//   3. tc_kernel     dA and dB partial sums per token range, fp32
//   4. red_kernel    dA, dB = round(ordered sum of the partials)
// Without dX: prep_kernel (B^T), proj_kernel (s G and s T), tc_kernel,
// red_kernel.  With no tokens, red_kernel alone writes dA = 0 and dB = 0.
// (Folding the reduction into the token contraction, the last workgroup of
// a column tile adding the others' partials: with an agent-scope release
// fence per workgroup, which on gfx950 writes back the XCD's L2, the
// contraction ran 8x slower than the separate reduce launch; with the
// partials written and read by device-scope atomic stores and loads and a
// per-tile counter instead, the pass took 29.9 against 27.6 us on
// X[4096,1024] W[1024,1024] r16 and 206 against 196-202 us on
// X[8192,2560] W[4096,2560] r32, graph replays.)
// W^T is rewritten on every call (2 |W| bytes of traffic): the forward
// kernel's contiguous-contraction operand reads run faster than reading W
// as stored through transposing LDS reads, by more than the copy costs
// (measured on X[4096,1024] W[1024,1024] and on X[8192,2560] W[4096,2560]).
#include "common.h"
#include "kernels.h"

namespace lora {
namespace {

constexpr int cmaxi(int a, int b) { return a > b ? a : b; }
constexpr int cmini(int a, int b) { return a < b ? a : b; }
constexpr int clampi(int v, int lo, int hi) { return v < lo ? lo : v > hi ? hi : v; }

// 128-B staged rows of 64 bf16 with 16-B chunks swizzled by row & 7: the MFMA
// operand read pattern (16 rows at one chunk) is free of bank conflicts.
__device__ __forceinline__ int row_off(int row, int chunk) {
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}

// 128-B staged rows read with transposing reads (rows 8g + 0..3 of lane group
// g at one 32-B segment): segments XOR-swizzled by bits 1 and 3 of the row put
// each half wave's 8 rows in 8 distinct 32-B bank windows.
__device__ __forceinline__ int tr_swz(int row) { return ((row >> 1) & 1) | ((row >> 2) & 2); }
__device__ __forceinline__ int tr_off(int row, int col) {
  return row * 128 + (((col >> 4) ^ tr_swz(row)) << 5) + ((col & 15) << 1);
}

// ---------------------------------------------------------------- transposes
// Preparation work, in blocks of nt threads (nt / 64 waves): the first
// blocks write W^T, one 64 x 64 tile per wave; the following blocks write B^T
// and A^T, one element per thread.
struct PrepArgs {
  int N, K, r, wtiles_k, wtiles;
  const uint16_t* W; int64_t ldw; uint16_t* Wt; int64_t ldwt;
  const uint16_t* B; int64_t ldb; uint16_t* Bt; int64_t ldbt;
  const uint16_t* A; int64_t lda; uint16_t* At; int64_t ldat;
};

// Blocks the preparation needs with nt threads per block.
inline int64_t prep_blocks(const PrepArgs& a, int nt) {
  const int wpb = nt / kWave;
  const int64_t small = (int64_t)a.r * a.N + (int64_t)a.K * a.r;
  return (a.wtiles + wpb - 1) / wpb + (small + nt - 1) / nt;
}

// W^T tile t through registers: lane l owns the 8 x 8 block at W rows
// n0 + 8 (l / 8) + 0..7 and columns k0 + 8 (l % 8) + 0..7, read as eight
// 16-B row loads and written as eight 16-B rows of W^T; each instruction
// moves whole 128-B segments (8 lanes per row), with no LDS and no barrier.
// N and K are multiples of 8, so a block is wholly inside or outside.
__device__ __forceinline__ void prep_wt_tile(const PrepArgs& a, int t, int lane) {
  const int n = (t / a.wtiles_k) * 64 + 8 * (lane >> 3);
  const int k = (t % a.wtiles_k) * 64 + 8 * (lane & 7);
  if (n >= a.N || k >= a.K) return;
  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const u32x4*>(a.W + (int64_t)(n + i) * a.ldw + k);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    // W^T row k + j: element j of each of the eight W rows, two per word.
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t x0 = v[2 * q][j >> 1], x1 = v[2 * q + 1][j >> 1];
      w[q] = (j & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
    }
    *reinterpret_cast<u32x4*>(a.Wt + (int64_t)(k + j) * a.ldwt + n) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

__device__ __forceinline__ void prep_block(const PrepArgs& a, int b, int tid, int nt) {
  const int wpb = nt / kWave;
  const int wblocks = (a.wtiles + wpb - 1) / wpb;
  if (b < wblocks) {
    const int t = b * wpb + (tid >> 6);
    if (t < a.wtiles) prep_wt_tile(a, t, tid & 63);
    return;
  }
  int64_t e = (int64_t)(b - wblocks) * nt + tid;
  const int64_t nb = (int64_t)a.r * a.N;
  if (e < nb) {
    const int j = (int)(e / a.N), n = (int)(e % a.N);
    a.Bt[(int64_t)j * a.ldbt + n] = a.B[(int64_t)n * a.ldb + j];
    return;
  }
  e -= nb;
  if (e < (int64_t)a.K * a.r) {
    const int k = (int)(e / a.r), j = (int)(e % a.r);
    a.At[(int64_t)k * a.ldat + j] = a.A[(int64_t)j * a.lda + k];
  }
}

__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
  prep_block(a, blockIdx.x, threadIdx.x, 256);
}

// ---------------------------------------------------------------- projection
// P^T[j, m] = round(scale * sum_c Z[m, c] U[j, c]) for a tile of 16 tokens,
// both operands contraction-contiguous: s T (Z = X, U = A), and s G (Z = dY,
// U = B^T) when dX is not computed (otherwise the dX kernel provides it).
// The contraction is split over the KW waves of a workgroup: wave w takes the
// 64-wide stages w, w + KW, ... through a ring of its own (no barriers inside
// the loop), and wave 0 adds the KW partial sums in wave order.  One wave
// walking the whole contraction of its 16 tokens keeps too few loads in
// flight and runs at latency, not bandwidth.  s G summed this way is rounded
// differently from the dX kernel's, so dA with and without dX agree to
// rounding, not bitwise; each is deterministic.
struct ProjJob {
  const uint16_t* Z;
  int64_t ldz;
  int C;
  const uint16_t* U;
  int64_t ldu;
  uint16_t* Pt;
};

template <int RP, int KW_>
struct PrjK {
  static constexpr int KW = KW_, NT = KW * kWave, RB = RP / 16;
  static constexpr int kStageB = (16 + RP) * 128;  // 16 token rows, then RP rank rows
  static constexpr int kLoads = (16 + RP) / 8;     // 1-KiB loads per stage, all one wave's
  // Ring depth per wave: up to 4 stages within the LDS and the vmcnt of
  // STAGES - 2 stages in flight within its 6-bit field; at least 2.
  static constexpr int STAGES = cmini(cmini(4, 160 * 1024 / (KW * kStageB)), 2 + 63 / kLoads);
  static constexpr int kRing = STAGES * kStageB;
  static constexpr int kRed = KW * RB * kWave * 16;  // partial sums, after the loop
  static constexpr int kLds = cmaxi(KW * kRing, kRed);
  static_assert(STAGES >= 2, "LDS budget");
  static_assert((STAGES - 2) * kLoads <= 63, "vmcnt range");
  static_assert(kLds <= 160 * 1024, "LDS budget");
};

// Wait until this wave's loads of all but its Newer most recent stages have
// landed.  Load q of a stage is issued by wave q % NW.
template <int Lo, int Hi, int Loads, int NW, int Newer>
__device__ __forceinline__ void wait_own(int wave) {
  if constexpr (Hi != Lo) {
    if (wave < Loads % NW) {
      wait_vmcnt<Newer * Hi>();
      return;
    }
  }
  wait_vmcnt<Newer * Lo>();
}

template <int RP, int KW>
__device__ __forceinline__ void proj_split(int M, int r, float scale, const ProjJob& jb,
                                           int64_t ldp, int tile, unsigned char* smem) {
  using P = PrjK<RP, KW>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 15, lk = lane >> 4;
  const int m0 = tile * 16;
  const int C = jb.C;

  // Z rows of the tile (rows past M read zeros); U rows past r read zeros.
  const int zrows = max(0, min(16, M - m0));
  const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(jb.Z + (int64_t)m0 * jb.ldz), 0, (int)(zrows * jb.ldz * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t ru =
      __builtin_amdgcn_make_buffer_rsrc((void*)jb.U, 0, (int)(r * jb.ldu * 2), 0x00020000);
  // Lane i of 1-KiB load q writes row 8 q + i / 8, physical chunk i % 8:
  // loads 0-1 the 16 token rows, loads 2.. the rank rows.
  const int lrl = lane >> 3;
  const int lch = (lane & 7) ^ lrl;
  const uint32_t vz = (uint32_t)(lrl * jb.ldz * 2 + lch * 16);
  const uint32_t vu = (uint32_t)(lrl * jb.ldu * 2 + lch * 16);
  unsigned char* ring = smem + wave * P::kRing;

  auto issue = [&](int st, int slot) {
    unsigned char* base = ring + slot * P::kStageB;
    const int c0 = st * 64;
    const bool kin = c0 + lch * 8 < C;
    const uint32_t cb = (uint32_t)c0 * 2;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rz, (lds_void*)(base + q * 1024), 16,
          off_or_oob(kin, vz + sgpr((uint32_t)(8 * q * jb.ldz * 2) + cb)), 0, 0, 0);
#pragma unroll
    for (int q = 0; q < RP / 8; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ru, (lds_void*)(base + (2 + q) * 1024), 16,
          off_or_oob(kin, vu + sgpr((uint32_t)(8 * q * jb.ldu * 2) + cb)), 0, 0, 0);
  };

  f32x4 acc[P::RB];
#pragma unroll
  for (int i = 0; i < P::RB; ++i) acc[i] = zero4();

  // This wave's stages: wave + KW i for i < mine; the prefetches past them
  // read zeros.
  const int nk = (C + 63) / 64;
  const int mine = nk > wave ? (nk - wave + KW - 1) / KW : 0;
#pragma unroll
  for (int i = 0; i < P::STAGES - 1; ++i) issue(wave + KW * i, i);
  int slot = 0;
  for (int i = 0; i < mine; ++i) {
    wait_vmcnt<(P::STAGES - 2) * P::kLoads>();
    wait_lgkm0();
    issue(wave + KW * (i + P::STAGES - 1), slot == 0 ? P::STAGES - 1 : slot - 1);
    const unsigned char* sb = ring + slot * P::kStageB;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const u32x4 z = *reinterpret_cast<const u32x4*>(sb + row_off(lrow, 4 * u + lk));
#pragma unroll
      for (int j = 0; j < P::RB; ++j) {
        const u32x4 w =
            *reinterpret_cast<const u32x4*>(sb + row_off(16 + 16 * j + lrow, 4 * u + lk));
        acc[j] = mfma16x16x32(z, w, acc[j]);
      }
    }
    slot = slot + 1 == P::STAGES ? 0 : slot + 1;
  }
  // Loads of the stages past the end (zeros) may still be landing in the ring.
  wait_vmcnt<0>();
  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(smem);
#pragma unroll
  for (int j = 0; j < P::RB; ++j) red[(wave * P::RB + j) * kWave + lane] = acc[j];
  __syncthreads();
  if (wave != 0) return;

  // acc[j] lane: rank 16 j + lrow, tokens m0 + 4 lk + 0..3 (< ldp: the grid
  // covers ldp / 16 tiles).
  const int64_t m = m0 + 4 * lk;
#pragma unroll
  for (int j = 0; j < P::RB; ++j) {
    f32x4 sum = red[j * kWave + lane];
#pragma unroll
    for (int w = 1; w < KW; ++w) sum += red[(w * P::RB + j) * kWave + lane];
    const int jr = 16 * j + lrow;
    if (jr < r) {
      uint32_t* o = reinterpret_cast<uint32_t*>(jb.Pt + (int64_t)jr * ldp + m);
      o[0] = pack_bf2(scale * sum[0], scale * sum[1]);
      o[1] = pack_bf2(scale * sum[2], scale * sum[3]);
    }
  }
}

// Blocks [0, gtiles): s G (without dX); [gtiles, gtiles + tiles): s T; the
// rest: the preparation (with dX).
template <int RP, int KW>
__global__ __launch_bounds__(KW * kWave) void proj_kernel(int M, int r, float scale, ProjJob jt,
                                                          ProjJob jg, int64_t ldp, PrepArgs pa,
                                                          int gtiles, int tiles) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int b = blockIdx.x;
  if (b < gtiles)
    proj_split<RP, KW>(M, r, scale, jg, ldp, b, smem);
  else if (b < gtiles + tiles)
    proj_split<RP, KW>(M, r, scale, jt, ldp, b - gtiles, smem);
  else
    prep_block(pa, b - gtiles - tiles, threadIdx.x, KW * kWave);
}

// Sum of S float4 partials p[0], p[stride], ... added in index order; the
// loads are issued eight at a time so their latencies overlap.
__device__ __forceinline__ f32x4 ordered_sum(const float* __restrict__ p, int64_t stride, int S) {
  f32x4 s4 = zero4();
  int sp = 0;
  for (; sp + 8 <= S; sp += 8) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const f32x4*>(p + (sp + u) * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) s4 += v[u];
  }
  for (; sp < S; ++sp) s4 += *reinterpret_cast<const f32x4*>(p + sp * stride);
  return s4;
}

// ---------------------------------------------------------------- token contraction
// Partial sums over one token range of out[j, c] = sum_m P^T[j, m] Q[m, c]
// for a 64-column tile of Q.  Job 0: Q = X, P^T = G^T (dA, partials stored
// [S][RP][K]); job 1: Q = dY, P^T = T^T (dB, partials stored [S][N][RP]).
struct TcJob {
  const uint16_t* Q;
  int64_t ldq;
  int C;
  const uint16_t* Pt;
  float* part;
};

template <int RP>
struct Tc {
  static constexpr int BC = 64, BMT = 64, NW = 4, NT = NW * kWave, RB = RP / 16;
  static constexpr int kQB = BMT * BC * 2;       // Q stage: 64 token rows of 64 columns
  static constexpr int kPB = RP * BMT * 2;       // P stage: RP rank rows of 64 tokens
  static constexpr int kStageB = kQB + kPB;
  static constexpr int kLoads = 8 + RP / 8;      // 1-KiB loads per stage; the first 8 are Q
  static constexpr int kPL = (RP / 8 + NW - 1) / NW;  // P load slots per wave
  static constexpr int kLo = kLoads / NW, kHi = kLo + (kLoads % NW != 0 ? 1 : 0);
  static constexpr int STAGES = clampi(96 * 1024 / kStageB, 2, 4);
  static constexpr int kLds = STAGES * kStageB;
  static_assert(kLds <= 160 * 1024, "LDS budget");
};

template <int RP>
__global__ __launch_bounds__(Tc<RP>::NT) void tc_kernel(int M, int r, TcJob j0, TcJob j1,
                                                        int64_t ldp, int tiles0, int tiles1,
                                                        int tps) {
  using T = Tc<RP>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 15, lk = lane >> 4;
  const int per = tiles0 + tiles1;
  const int split = blockIdx.x / per, rem = blockIdx.x % per;
  const int job = rem < tiles0 ? 0 : 1;
  const TcJob jb = job == 0 ? j0 : j1;
  const int c0 = (job == 0 ? rem : rem - tiles0) * T::BC;
  const int t0 = split * tps, t1 = min(M, t0 + tps);
  const int C = jb.C;

  // Q load q < 8 covers token rows 8q .. 8q + 7 of the stage (lane i: row
  // 8q + i / 8, physical chunk i % 8, fetching the chunk the segment swizzle
  // puts there); P load p covers rank rows 8p .. 8p + 7.
  const int lrl = lane >> 3, pc = lane & 7;
  const int qrow = 8 * wave + lrl;  // + 32 for the second Q slot: same swizzle
  const int qch = 2 * ((pc >> 1) ^ tr_swz(qrow)) + (pc & 1);
  const uint32_t vq = (uint32_t)(qrow * jb.ldq * 2 + qch * 16);
  const uint32_t sq = (uint32_t)(32 * jb.ldq * 2);
  const int pch = pc ^ lrl;
  const uint32_t vp = (uint32_t)((8 * wave + lrl) * ldp * 2 + pch * 16);
  const uint32_t sp = (uint32_t)(8 * T::NW * ldp * 2);

  auto issue = [&](int st) {
    unsigned char* base = smem + (st % T::STAGES) * T::kStageB;
    const int t = t0 + st * T::BMT;
    const bool live = t < t1;  // wave-uniform; stages past the range read zeros
    const int qrows = live ? min(T::BMT, M - t) : 0;
    // From column c0 of row t to the last valid element of row t + qrows - 1:
    // rows past M read zeros and no read leaves Q.  Columns past C on earlier
    // rows read the next row; they only reach columns that are never stored.
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(jb.Q + (int64_t)(live ? t : 0) * jb.ldq + c0), 0,
        qrows > 0 ? (int)(((qrows - 1) * jb.ldq + (C - c0)) * 2) : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(jb.Pt + (live ? t : 0)), 0, live ? (int)((r * ldp - t) * 2) : 0, 0x00020000);
#pragma unroll
    for (int s = 0; s < 2; ++s)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void*)(base + (wave + s * T::NW) * 1024),
                                               16, vq + sgpr(s * sq), 0, 0, 0);
#pragma unroll
    for (int s = 0; s < T::kPL; ++s) {
      const int p = wave + s * T::NW;  // stage load 8 + p
      if (p < RP / 8)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rp, (lds_void*)(base + T::kQB + p * 1024), 16, vp + sgpr(s * sp), 0, 0, 0);
    }
  };

  f32x4 acc[T::RB];
#pragma unroll
  for (int i = 0; i < T::RB; ++i) acc[i] = zero4();

  const int nst = t1 > t0 ? (t1 - t0 + T::BMT - 1) / T::BMT : 0;
#pragma unroll
  for (int s = 0; s < T::STAGES - 1; ++s) issue(s);
  const int qcol = 16 * wave + 4 * (lrow & 3);  // wave w owns columns 16w .. 16w + 15
  for (int kt = 0; kt < nst; ++kt) {
    wait_own<T::kLo, T::kHi, T::kLoads, T::NW, T::STAGES - 2>(wave);
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    issue(kt + T::STAGES - 1);
    const unsigned char* sb = smem + (kt % T::STAGES) * T::kStageB;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int row = 32 * u + 8 * lk + (lrow >> 2);
      const u32x2 lo = lds_read_tr16(sb + tr_off(row, qcol));
      const u32x2 hi = lds_read_tr16(sb + tr_off(row + 4, qcol));
      const u32x4 q = u32x4{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
      for (int i = 0; i < T::RB; ++i) {
        const u32x4 p =
            *reinterpret_cast<const u32x4*>(sb + T::kQB + row_off(16 * i + lrow, 4 * u + lk));
        acc[i] = mfma16x16x32(p, q, acc[i]);
      }
    }
  }
  wait_vmcnt<0>();

  // acc[i] lane: column c0 + 16 w + lrow, ranks 16 i + 4 lk + 0..3.
  const int c = c0 + 16 * wave + lrow;
  if (c < C) {
    if (job == 0) {
      float* part = jb.part + (int64_t)split * RP * C;
#pragma unroll
      for (int i = 0; i < T::RB; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) part[(int64_t)(16 * i + 4 * lk + q) * C + c] = acc[i][q];
    } else {
      float* part = jb.part + ((int64_t)split * C + c) * RP;
#pragma unroll
      for (int i = 0; i < T::RB; ++i) *reinterpret_cast<f32x4*>(part + 16 * i + 4 * lk) = acc[i];
    }
  }

}

// ---------------------------------------------------------------- reduce
// dA[j, k] = round(sum_split partA[split][j][k]) and
// dB[n, j] = round(sum_split partB[split][n][j]), splits added in order (the
// scale is already in s G and s T).  One thread per 4 consecutive outputs.
__global__ __launch_bounds__(64) void red_kernel(int S, int r, int RP, int K, int N,
                                                  const float* __restrict__ pa,
                                                  const float* __restrict__ pb,
                                                  uint16_t* __restrict__ dA, int64_t ldda,
                                                  uint16_t* __restrict__ dB, int64_t lddb,
                                                  int64_t na) {
  const int64_t e = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (e < na) {
    const int k4 = K / 4;
    const int j = (int)(e / k4), k = (int)(e % k4) * 4;
    const f32x4 s4 = ordered_sum(pa + (int64_t)j * K + k, (int64_t)RP * K, S);
    uint32_t* out = reinterpret_cast<uint32_t*>(dA + (int64_t)j * ldda + k);
    out[0] = pack_bf2(s4[0], s4[1]);
    out[1] = pack_bf2(s4[2], s4[3]);
    return;
  }
  const int64_t f = e - na;
  const int r4 = (r + 3) / 4;
  if (f >= (int64_t)N * r4) return;
  const int n = (int)(f / r4), j = (int)(f % r4) * 4;
  const f32x4 s4 = ordered_sum(pb + (int64_t)n * RP + j, (int64_t)N * RP, S);
  uint16_t* out = dB + (int64_t)n * lddb + j;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (j + q < r) out[q] = f2bf(s4[q]);
}

// The projection: s T, and either s G (want_g) or the preparation blocks.
template <int RP, int KW>
hipError_t launch_proj(const BwdArgs& a, const BwdPlan& p, const ProjJob& jt, const ProjJob& jg,
                       bool want_g, const PrepArgs* pre, hipStream_t s) {
  auto kern = proj_kernel<RP, KW>;
  constexpr int lds = PrjK<RP, KW>::kLds;
  static std::atomic<uint64_t> done{0};
  if (hipError_t e = ensure_lds(kern, lds, done); e != hipSuccess) return e;
  const int tiles = (int)(p.ldp / 16);
  const int gtiles = want_g ? tiles : 0;
  const int64_t extra = pre != nullptr ? prep_blocks(*pre, KW * kWave) : 0;
  const PrepArgs none{};
  hipLaunchKernelGGL(kern, dim3((unsigned)(gtiles + tiles + extra)), dim3(KW * kWave), lds, s,
                     (int)a.M, (int)a.r, a.scale, jt, jg, p.ldp, extra > 0 ? *pre : none, gtiles,
                     tiles);
  return hipGetLastError();
}

// Waves per workgroup (KW): about 1024 waves over the 16-token tiles, at
// most 4 (2 for the 256 ranks, whose rings take the LDS).  The choice
// depends on the tokens alone, so s T, hence dB, is bitwise the same with
// and without dX.
template <int RP>
hipError_t launch_proj_kw(const BwdArgs& a, const BwdPlan& p, const ProjJob& jt,
                          const ProjJob& jg, bool want_g, const PrepArgs* pre, hipStream_t s) {
  const int64_t tiles = p.ldp / 16;
  if (tiles <= 256) return launch_proj<RP, RP < 256 ? 4 : 2>(a, p, jt, jg, want_g, pre, s);
  if (tiles <= 512) return launch_proj<RP, 2>(a, p, jt, jg, want_g, pre, s);
  return launch_proj<RP, 1>(a, p, jt, jg, want_g, pre, s);
}

// Launches 1-3 for M > 0 (see the top of the file).
template <int RP>
hipError_t launch_rank(const BwdArgs& a, const BwdPlan& p, unsigned char* ws, bool want_dx,
                       const PrepArgs& pre, hipStream_t s) {
  const int M = (int)a.M, N = (int)a.N, K = (int)a.K, r = (int)a.r;
  const uint16_t* Bt = reinterpret_cast<const uint16_t*>(ws + p.off_bt);
  uint16_t* Tt = reinterpret_cast<uint16_t*>(ws + p.off_tt);
  uint16_t* Gt = reinterpret_cast<uint16_t*>(ws + p.off_gt);
  const ProjJob jt{static_cast<const uint16_t*>(a.X), a.ldx, K,
                   static_cast<const uint16_t*>(a.A), a.lda, Tt};
  const ProjJob jg{static_cast<const uint16_t*>(a.dY), a.lddy, N, Bt, p.ldbt, Gt};
  if (want_dx) {
    // 1. s T with the transposes; 2. dX, whose rank intermediate is s G.
    if (hipError_t e = launch_proj_kw<RP>(a, p, jt, jg, false, &pre, s); e != hipSuccess) return e;
    const uint16_t* Wt = reinterpret_cast<const uint16_t*>(ws + p.off_wt);
    const uint16_t* At = reinterpret_cast<const uint16_t*>(ws + p.off_at);
    const FwdArgs f{a.M, a.K, a.N, a.r, a.dY, a.lddy, Wt, p.ldwt, Bt, p.ldbt, At, p.ldat,
                    a.scale, a.dX, a.lddx, Gt, p.ldp};
    if (hipError_t e = launch_fwd_tiled_bf16(f, s); e != hipSuccess) return e;
  } else {
    // 1. B^T (nothing when N == 0); 2. s T and s G.
    if (const int64_t blocks = prep_blocks(pre, 256); blocks > 0) {
      hipLaunchKernelGGL(prep_kernel, dim3((unsigned)blocks), dim3(256), 0, s, pre);
      if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    if (hipError_t e = launch_proj_kw<RP>(a, p, jt, jg, true, nullptr, s); e != hipSuccess) return e;
  }
  // 3. Token contraction, reduction included.
  const int tiles0 = (K + 63) / 64, tiles1 = (N + 63) / 64;
  const int64_t grid = (int64_t)(tiles0 + tiles1) * p.S;
  if (grid == 0) return hipSuccess;
  const TcJob ja{static_cast<const uint16_t*>(a.X), a.ldx, K, Gt,
                 reinterpret_cast<float*>(ws + p.off_pa)};
  const TcJob jb{static_cast<const uint16_t*>(a.dY), a.lddy, N, Tt,
                 reinterpret_cast<float*>(ws + p.off_pb)};
  auto kern = tc_kernel<RP>;
  static std::atomic<uint64_t> done{0};
  if (hipError_t e = ensure_lds(kern, Tc<RP>::kLds, done); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Tc<RP>::NT), Tc<RP>::kLds, s, M, r, ja, jb,
                     p.ldp, tiles0, tiles1, (int)p.tps);
  return hipGetLastError();
}

// 4. dA = round(sum of partials), dB likewise; with S = 0 (no tokens) zeros.
hipError_t launch_red(const BwdArgs& a, const BwdPlan& p, unsigned char* ws, hipStream_t s) {
  const int N = (int)a.N, K = (int)a.K, r = (int)a.r;
  const int64_t na = (int64_t)r * (K / 4);
  const int64_t total = na + (int64_t)N * ((r + 3) / 4);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(red_kernel, dim3((unsigned)((total + 63) / 64)), dim3(64), 0, s, p.S, r,
                     pad_rank(a.r), K, N, reinterpret_cast<const float*>(ws + p.off_pa),
                     reinterpret_cast<const float*>(ws + p.off_pb), static_cast<uint16_t*>(a.dA),
                     a.ldda, static_cast<uint16_t*>(a.dB), a.lddb, na);
  return hipGetLastError();
}

int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }

}  // namespace

BwdPlan bwd_plan(int64_t M, int64_t N, int64_t K, int64_t r) {
  BwdPlan p{};
  const int64_t RP = pad_rank(r);
  p.ldbt = (N + 7) / 8 * 8;
  p.ldp = (M + 63) / 64 * 64;
  // Token ranges: aim at ~512 workgroups for the token contraction, keep the
  // fp32 partials (S * RP * (K + N) * 4 bytes) within 1/8 of the bytes of X
  // and dY that it streams (M * (K + N) * 2), and never split below one
  // 64-token stage.
  const int64_t stages = p.ldp / 64;
  const int64_t tiles = (K + 63) / 64 + (N + 63) / 64;
  int64_t S = tiles > 0 ? (512 + tiles - 1) / tiles : 1;
  S = std::min<int64_t>(S, std::max<int64_t>(1, M / (16 * RP)));
  S = std::max<int64_t>(1, std::min<int64_t>(S, stages));
  const int64_t per = stages > 0 ? (stages + S - 1) / S : 1;  // stages per range
  p.tps = per * 64;
  p.S = M > 0 ? (int)((M + p.tps - 1) / p.tps) : 0;
  p.ldwt = N;   // N % 8 == 0
  p.ldat = r;
  int64_t off = 0;
  p.off_wt = off; off = align256(off + K * N * 2);
  p.off_at = off; off = align256(off + K * r * 2);
  p.off_bt = off; off = align256(off + r * p.ldbt * 2);
  p.off_tt = off; off = align256(off + r * p.ldp * 2);
  p.off_gt = off; off = align256(off + r * p.ldp * 2);
  p.off_pa = off; off = align256(off + (int64_t)p.S * RP * K * 4);
  p.off_pb = off; off = align256(off + (int64_t)p.S * N * RP * 4);
  p.bytes = off;
  return p;
}

hipError_t launch_bwd_bf16(const BwdArgs& a, void* workspace, hipStream_t s) {
  const BwdPlan p = bwd_plan(a.M, a.N, a.K, a.r);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  const int N = (int)a.N, K = (int)a.K, r = (int)a.r;
  if (a.M == 0) return launch_red(a, p, ws, s);  // no tokens: p.S = 0, zeros
  const bool want_dx = a.dX != nullptr && a.K > 0;
  PrepArgs pre{N, want_dx ? K : 0, r, (K + 63) / 64, 0,
               static_cast<const uint16_t*>(a.W), a.ldw, reinterpret_cast<uint16_t*>(ws + p.off_wt),
               p.ldwt, static_cast<const uint16_t*>(a.B), a.ldb,
               reinterpret_cast<uint16_t*>(ws + p.off_bt), p.ldbt,
               static_cast<const uint16_t*>(a.A), a.lda, reinterpret_cast<uint16_t*>(ws + p.off_at),
               p.ldat};
  if (want_dx) pre.wtiles = ((N + 63) / 64) * pre.wtiles_k;
  hipError_t e;
  switch (pad_rank(a.r)) {
    case 16: e = launch_rank<16>(a, p, ws, want_dx, pre, s); break;
    case 32: e = launch_rank<32>(a, p, ws, want_dx, pre, s); break;
    case 64: e = launch_rank<64>(a, p, ws, want_dx, pre, s); break;
    case 128: e = launch_rank<128>(a, p, ws, want_dx, pre, s); break;
    default: e = launch_rank<256>(a, p, ws, want_dx, pre, s); break;
  }
  if (e != hipSuccess) return e;
  return launch_red(a, p, ws, s);
}

}  // namespace lora
