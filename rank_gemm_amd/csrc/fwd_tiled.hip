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
// Per workgroup (BM x BN output tile; WM x WN multiplying waves, each a grid
// of 16 x 16 MFMA blocks, twice that with the k split; PW loader waves or
// none, see Cfg):
//   K loop, BK (32 or 64) per stage, STAGES-deep ring of LDS stages:
//     X[BM x BK], W[BN x BK] and A[RP x BK] go straight from global memory to
//     LDS (buffer_load ... lds, 16 B per lane, no register staging), issued
//     by the loader waves, or by the multiplying waves when there are none.  Each
//     buffer resource starts at the tile's first row and ends at the last
//     valid row, so rows past M, N or r and the K tail read as zeros.
//     16-B chunks are XOR-swizzled per row so that MFMA operand reads
//     (16 rows x one chunk per instruction) hit distinct banks.
//     acc[BM x BN] += X W^T          (MFMA with W as the first operand: each
//                                     lane accumulates 4 consecutive output
//                                     columns of one row)
//     T[BM x RP]   += X A^T          (MFMA, reusing the X operand registers)
//   epilogue:
//     T -> scale * T -> bf16 -> LDS; B[BN x RP] -> LDS (zero padded)
//     acc += (s T) B^T               (MFMA over the rank)
//     acc -> bf16 -> LDS (8 B per lane and block) -> coalesced 16-B stores of Y.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace lora {
namespace {

// LDS stage rows hold BK k-values (BK = 32: 64-B rows, 4 chunks of 16 B;
// BK = 64: 128-B rows, 8 chunks).  The 16-B chunks are XOR-swizzled per row.
// With the MFMA operand read pattern (16 consecutive rows at one logical chunk
// per ds_read_b128) both layouts below measured free of LDS bank conflicts on
// gfx950 (SQ_LDS_BANK_CONFLICT = 0), where e.g. chunk ^ (row & 3) on 64-B rows
// is 2-way conflicted.  Both depend on row & 7 only, so a 1-KiB direct load
// (16 or 8 rows) can apply them from the lane index alone.
template <int BK>
__device__ __forceinline__ int swz(int row) {
  if constexpr (BK == 32) return (row >> 1) & 3;
  return row & 7;
}
template <int BK>
__device__ __forceinline__ int stage_off(int row, int chunk) {
  return row * (BK * 2) + ((chunk ^ swz<BK>(row)) << 4);
}

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// KS = 2 splits every stage's k range between two groups of WM x WN waves
// that compute the same BM x BN tile: group g multiplies k32 half g of each
// stage, and the epilogue adds the two partial sums through LDS.  It doubles
// the waves per tile (more latency hiding) without more LDS reads per stage,
// or, with half as many waves per group, gives each wave a tile twice as
// large for the same number of waves.
//
// PW > 0 adds PW loader waves that issue every stage's loads while the
// WM x WN x KS multiplying waves only read LDS and run MFMAs.  A wave stalls
// at a load issue when the memory pipeline is backed up, and a multiplying
// wave stalled there cannot issue its MFMAs either: with separate loaders the
// loads and the MFMAs overlap.
//
// TS = 1 stores the epilogue's T tile unpadded (rows of RP elements) with its
// 16-B chunks XOR-swizzled by row, so that a tile keeping T across several N
// tiles fits T after a ring that fills all but RP x BM x 2 bytes of the LDS.
//
// LD > 0 (without loader waves): only multiplying waves [0, LD) issue the
// stage loads, each LD-th load of every stage.  In the 256 x 256 tile the
// first four waves reach each stage's barrier well ahead of the other four
// (they win the SIMD's issue arbitration); giving them the loads evens the
// two out.
//
// PP = 1 runs the K loop as a ping-pong between two groups of four waves
// (see the kernel): the first group multiplies while the second reads its
// next fragments from LDS and issues stage loads, then the roles swap.
//
// TP = 1 (with a group of N tiles, TS = 1) computes the group's s T in a
// prologue of its own before the first tile (t_prologue) and keeps it in LDS
// past the ring; the stages then hold only X and W rows, and no tile of the
// group runs the down-projection in its K loop.
template <int BM_, int BN_, int WM_, int WN_, int RP_, int ST_, int BK_, int KS_ = 1, int PW_ = 0,
          int TS_ = 0, int PP_ = 0, int LD_ = 0, int TP_ = 0>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, RP = RP_, STAGES = ST_, BK = BK_;
  static constexpr int KS = KS_, PW = PW_;
  static constexpr bool kPP = PP_ >= 1;
  static constexpr bool kTP = TP_ == 1;
  static constexpr bool kPPSpread = PP_ == 2;  // X/W loads among the MFMAs of M
  static constexpr int kRowB = BK * 2;                // bytes per staged row
  static constexpr int kRowsPerLoad = 1024 / kRowB;   // rows one 1-KiB wave load covers
  static constexpr int kChunks = BK / 8;              // 16-B chunks per row
  static constexpr int NWC = WM * WN * KS;          // multiplying waves
  static constexpr int NW = NWC + PW;               // all waves
  static constexpr int LW = PW > 0 ? PW : (LD_ > 0 ? LD_ : NWC);  // waves that issue the stage loads
  static constexpr int NT = NW * kWave;
  static constexpr int TM = BM / WM / 16;
  static constexpr int TN = BN / WN / 16;
  static constexpr int RB = RP / 16;
  static constexpr int ROWS = BM + BN + (kTP ? 0 : RP);  // staged rows per stage
  static constexpr int kStageB = ROWS * kRowB;
  static_assert(BK == 32 || BK == 64, "stage depth");
  static constexpr int kXL = BM / kRowsPerLoad / LW;  // X loads (1 KiB each) per loader per stage
  static constexpr int kWL = BN / kRowsPerLoad / LW;  // W loads per loader per stage
  static constexpr int kAN = (RP + kRowsPerLoad - 1) / kRowsPerLoad;  // A loads per stage
  static constexpr int kAL = (kAN + LW - 1) / LW;     // A load slots per loader per stage
  // Loads per stage: loaders below kAN % LW issue one A load more than the rest.
  static constexpr int kLoadsLo = kXL + kWL + kAN / LW;
  static constexpr int kLoadsHi = kLoadsLo + (kAN % LW != 0 ? 1 : 0);
  static constexpr int kTS = RP + 8;                // epilogue T / B row stride (elements)
  static constexpr bool kTSw = TS_ == 1;
  static constexpr int kTRow = kTSw ? RP : kTS;     // T row stride (elements)
  // Element index of T[row][col] in the epilogue's T tile.  Swizzled: chunk
  // c = col / 8 of a row sits at c ^ (row mod RP / 8), so 16 rows read at one
  // logical chunk (an MFMA operand fragment) hit distinct banks (RP = 128).
  __device__ static __forceinline__ int t_idx(int row, int col) {
    if constexpr (kTSw)
      return row * RP + ((((col >> 3) ^ (row & (RP / 8 - 1))) << 3) | (col & 7));
    return row * kTS + col;
  }
  static constexpr int kEpiB = (BM * kTRow + BN * kTS) * 2;
  static constexpr int kYS = BN + 8;                // output staging row stride (elements)
  static constexpr int kYB = BM * kYS * 2;
  // K split: after the loop each wave sends the half of its accumulators that
  // its partner in the other group keeps (1 KiB per fragment), and group 1
  // sends its partial T; the area starts after the epilogue's T and B tiles.
  static constexpr int kXOff = kEpiB;
  static constexpr int kXchB = KS == 2 ? WM * WN * (TM * TN + (TM * RB + WN - 1) / WN) * 1024 : 0;
  static constexpr int kLds0 = cmax(cmax(STAGES * kStageB, kXOff + kXchB), cmax(kEpiB, kYB));
  // With T kept across the N tiles of a group: T after the ring, the B tile
  // and the output staging inside it.
  static constexpr int kTOffG = STAGES * kStageB;
  static constexpr int kLdsG = kTOffG + BM * kTRow * 2;
  // A group tile's output staging that does not fit in the ring also covers
  // s T, which the threads then hold in registers meanwhile (see the kernel).
  static constexpr bool kYSplit = kYB > kTOffG;
  // (only then can a workgroup take several N tiles: see the kernel)
  static constexpr bool kGroupFits = BN * kTS * 2 <= kTOffG && kYB <= kLdsG;
  // T prologue: its own ring in the stage ring's LDS, 64-deep stages of BM X
  // rows then RP A rows, 8 rows per 1-KiB load, every wave an equal share.
  static constexpr int kPRows = BM + RP;
  static constexpr int kPStageB = kPRows * 128;
  static constexpr int kPStages = kTP ? (STAGES * kStageB / kPStageB < 4 ? STAGES * kStageB / kPStageB : 4) : 2;
  static constexpr int kPLoads = kPRows / 8 / (WM * WN);
  // B tile elements per thread, fetched into registers at kernel start when
  // few enough (the epilogue's gather would otherwise put a memory round trip
  // after the K loop).  Not for 256 x 256 tiles: their main loop already
  // holds nearly every register, and the early loads slowed it down; nor for
  // 64 x 32 tiles past rank 16, where the live values push the kernel past
  // 64 VGPRs and cost a wave of occupancy per SIMD.
  // (held by the multiplying waves' threads)
  static constexpr int kBPre = BN * RP / (NWC * kWave);
  static constexpr bool kBEarly = BN * RP % (NWC * kWave) == 0 && kBPre <= 8 &&
                                  BM * BN <= 128 * 128 && (BM * BN > 64 * 32 || RP <= 16);
  // Otherwise, where it fits after the ring and the output staging without
  // costing a workgroup per CU, the B tile is fetched at kernel start by
  // direct loads into LDS (unpadded rows of RP elements), landing with the
  // first stage; in tiles with loader waves the loaders fetch it into
  // registers instead (see the kernel), and the k split keeps the gather
  // after the K loop.
  static constexpr int kBDmaOff = cmax(STAGES * kStageB, kYB);
  static constexpr int kBDmaB = BN * RP * 2;
  static constexpr bool kBDma = !kBEarly && PW == 0 && KS == 1 && kBDmaB % 1024 == 0 &&
                                kBDmaOff + kBDmaB <= 160 * 1024 &&
                                (160 * 1024) / (kBDmaOff + kBDmaB) >= (160 * 1024) / kLds0;
  static constexpr int kLds = kBDma ? cmax(kLds0, kBDmaOff + kBDmaB) : kLds0;
  static constexpr int kTSlots = (TM * RB + WN - 1) / WN;  // T accumulators per wave
  static constexpr int kGroup = 4;         // M tiles per group (XCD-contiguous ids)
  static constexpr int kGroupShared = 8;   // M tiles swept together by all XCDs (measured best)
  // T tile (i, tj) of a wave row belongs to wave (i * RB + tj) % WN.  With RB a
  // multiple of WN a wave owns rank blocks tj = wn + u * WN for every i and keeps
  // RB / WN A fragments; with WN a multiple of RB it owns rows
  // i = wn / RB + s * (WN / RB) of rank block wn % RB and keeps one.
  static constexpr bool kTByRank = RB % WN == 0;
  static_assert(kTByRank || (WN % RB == 0 && TM % (WN / RB) == 0), "T tile ownership");
  static_assert((TM & (TM - 1)) == 0, "ring rotation needs a power-of-two row-block count");
  static constexpr int kTF = kTByRank ? RB / WN : 1;       // A fragments per wave
  static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "wave tiling");
  static_assert(BM % (kRowsPerLoad * LW) == 0 && BN % (kRowsPerLoad * LW) == 0,
                "X/W loads split evenly over the loaders");
  static_assert(kLds <= 160 * 1024, "LDS budget");
  static_assert(!kTSw || (RP >= 64 && RP % 8 == 0), "swizzled T: at least 8 chunks per row");
  static_assert(STAGES >= 2, "ring: one stage being read, at least one in flight");
  static_assert(KS == 1 || (KS == 2 && BK == 64 && TM % 2 == 0), "k split: one k32 half per group");
  static_assert(LD_ == 0 || (PW == 0 && KS == 1 && PP_ == 0 && LD_ <= NWC), "load subset");
  static_assert(!kPP || (WM * WN == 8 && KS == 1 && PW == 0 && BK == 32 && STAGES >= 3 &&
                         (STAGES & (STAGES - 1)) == 0),
                "ping-pong: two groups of four waves, one k32 step per stage, a power-of-two ring");
  static_assert(BK == 32 || BK == 64, "one or two k32 substeps per stage");
  static_assert(!kTP || (kTSw && PW == 0 && KS == 1 && !kPP && BM == 256 && WM * WN == 8 &&
                         RP % 32 == 0 && kPRows % 64 == 0 && kPStages >= 2),
                "T prologue: 4 x 2 waves over T, equal load shares, two stages at least");
};


// Operand fragments of one k32 stage for one wave: X rows (a), W rows (b) and
// the A rows (t) of the rank block(s) this wave owns.
template <class C>
struct Frags {
  u32x4 a[C::TM];
  u32x4 b[C::TN];
  u32x4 t[C::kTF];
};

// T tile ownership.  T tiles of a wave row are (row block i, rank block tj),
// i < TM, tj < RB, shared by the WN waves of the row.
//  * RB a multiple of WN: wave wn owns rank blocks tj = wn + u * WN for all
//    i; it keeps RB / WN A fragments.
//  * WN a multiple of RB (G = WN / RB waves per rank block): wave wn owns
//    rank block wn % RB for row blocks [q * TM / G, (q + 1) * TM / G),
//    q = wn / RB; it keeps one A fragment.
// Each wave keeps its X fragments in a ring rotated by rot(wn), so that the
// row blocks it owns T tiles for sit in ring slots 0, 1, ... : every index
// below is compile-time and the T MFMAs need no branches.
template <class C>
__device__ __forceinline__ int ring_rot(int wn) {
  if constexpr (C::kTByRank) return 0;
  return (wn / C::RB) * (C::TM / (C::WN / C::RB));
}

// Row block held in ring slot k.
template <class C>
__device__ __forceinline__ int ring_row_block(int k, int rot) { return (k + rot) & (C::TM - 1); }

// Rank block held in A fragment f of wave wn.
template <class C>
__device__ __forceinline__ int t_block(int wn, int f) {
  if constexpr (C::kTByRank) return wn + f * C::WN;
  return wn % C::RB;
}

// T slot sl: ring slot of its X fragment and index of its A fragment.
template <class C>
__device__ __forceinline__ constexpr int t_ring_slot(int sl) {
  if constexpr (C::kTByRank) return sl / (C::RB / C::WN);
  return sl;
}
template <class C>
__device__ __forceinline__ constexpr int t_frag(int sl) {
  if constexpr (C::kTByRank) return sl % (C::RB / C::WN);
  return 0;
}

template <class C>
__device__ __forceinline__ void t_update_ab(const u32x4 (&a)[C::TM], const u32x4 (&t)[C::kTF],
                                            f32x4 (&tacc)[C::kTSlots]) {
#pragma unroll
  for (int sl = 0; sl < C::kTSlots; ++sl)
    tacc[sl] = mfma16x16x32(a[t_ring_slot<C>(sl)], t[t_frag<C>(sl)], tacc[sl]);
}

// Wait until the loads of loader `wave` (its index among the waves that issue
// stage loads) of all but its `Newer` most recent stages have landed.  Loads
// complete in issue order, so the count must be this loader's own per-stage
// load count: loaders that also load an A row issue one more.
template <class C, int Newer, bool WT = true>
__device__ __forceinline__ void wait_stages(int wave) {
  if constexpr (!WT) {
    wait_vmcnt<Newer * (C::kXL + C::kWL)>();  // stages without A loads
    return;
  }
  if constexpr (C::kLoadsHi != C::kLoadsLo) {
    if (wave < C::kAN % C::LW) {
      wait_vmcnt<Newer * C::kLoadsHi>();
      return;
    }
  }
  wait_vmcnt<Newer * C::kLoadsLo>();
}

// Issue one stage of direct-to-LDS loads for loader `wave`: its X slots, its
// W slots and (loaders below kAN) its A slot.  Slot s of a matrix is the
// loader's slot 0 plus s * LW 1-KiB loads, i.e. a wave-uniform byte stride.
// Lanes whose 16-B chunk lies past K read zeros.
template <class C, bool WT = true>
__device__ __forceinline__ void issue_stage(unsigned char* smem, int buf, int k0, int K, int wave,
                                            int lchunk, __amdgpu_buffer_rsrc_t rx,
                                            __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t ra,
                                            uint32_t vx, uint32_t vw, uint32_t va, uint32_t sx,
                                            uint32_t sw, uint32_t sa) {
  const bool kin = k0 + lchunk * 8 < K;
  const uint32_t kb = (uint32_t)k0 * 2;
  unsigned char* base = smem + buf * C::kStageB;
  constexpr int kRowB = C::kRowB;
#pragma unroll
  for (int s = 0; s < C::kXL; ++s)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(base + (wave + s * C::LW) * 1024), 16,
                                             off_or_oob(kin, vx + sgpr(s * sx + kb)), 0, 0, 0);
#pragma unroll
  for (int s = 0; s < C::kWL; ++s)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rw, (lds_void*)(base + C::BM * kRowB + (wave + s * C::LW) * 1024), 16,
        off_or_oob(kin, vw + sgpr(s * sw + kb)), 0, 0, 0);
  if constexpr (!WT) return;  // T already known: no A rows
#pragma unroll
  for (int s = 0; s < C::kAL; ++s)
    if (wave + s * C::LW < C::kAN)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (lds_void*)(base + (C::BM + C::BN) * kRowB + (wave + s * C::LW) * 1024), 16,
          off_or_oob(kin, va + sgpr(s * sa + kb)), 0, 0, 0);
}

// The A loads of one stage alone (loaders below kAN).
template <class C>
__device__ __forceinline__ void issue_stage_a(unsigned char* smem, int buf, int k0, int K, int wave,
                                              int lchunk, __amdgpu_buffer_rsrc_t ra, uint32_t va,
                                              uint32_t sa) {
  const bool kin = k0 + lchunk * 8 < K;
  const uint32_t kb = (uint32_t)k0 * 2;
  unsigned char* base = smem + buf * C::kStageB + (C::BM + C::BN) * C::kRowB;
#pragma unroll
  for (int s = 0; s < C::kAL; ++s)
    if (wave + s * C::LW < C::kAN)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(base + (wave + s * C::LW) * 1024), 16,
                                               off_or_oob(kin, va + sgpr(s * sa + kb)), 0, 0, 0);
}

// The group's down-projection ahead of its first tile (TP = 1): s T =
// s X_tile A^T, BM x RP, rounded once to bf16 into the LDS region `ts` past
// the stage ring, where every N tile of the group reads it.  A ring of
// kPStages 64-deep stages (BM X rows, then RP A rows) in the stage ring's
// LDS; every wave issues kPLoads 1-KiB loads per stage and owns a
// (BM / 4) x (RP / 2) block of T (4 x 2 waves).  The accumulation runs over
// k32 steps in ascending k on the same MFMA as the fused K loop, so T is the
// one that loop would produce.  Loads past K or past the last row read
// zeros; all of them have landed and every wave is past its reads when this
// returns.
template <class C>
__device__ __forceinline__ void t_prologue(unsigned char* smem, uint16_t* ts, int K, int r,
                                           float scale, __amdgpu_buffer_rsrc_t rx,
                                           __amdgpu_buffer_rsrc_t ra, int64_t ldx, int64_t lda,
                                           int wave, int lane) {
  constexpr int BM = C::BM, RP = C::RP, S = C::kPStages, NWP = C::WM * C::WN;
  constexpr int kPL = C::kPLoads;
  constexpr int kXQ = BM / 8;           // X loads per stage
  constexpr int PTM = BM / 4 / 16;      // row blocks per wave
  constexpr int PTN = RP / 2 / 16;      // rank blocks per wave
  static_assert(kXQ % NWP == 0, "X loads: the same count for every wave");
  const int lrow = lane & 15, lk = lane >> 4;
  const int pm = wave >> 1, pn = wave & 1;
  // Lane l of a load writes staged row 8 q + l / 8 at physical chunk l % 8,
  // so it fetches logical chunk (l % 8) ^ (row & 7) (the 64-deep swizzle).
  const int lr = lane >> 3;
  const int lc = (lane & 7) ^ lr;
  const uint32_t vx = (uint32_t)((wave * 8 + lr) * ldx * 2 + lc * 16);
  const uint32_t va = (uint32_t)((wave * 8 + lr) * lda * 2 + lc * 16);  // A load s - kXQ / NWP
  const uint32_t sx = (uint32_t)(NWP * 8 * ldx * 2);
  const uint32_t sa = (uint32_t)(NWP * 8 * lda * 2);
  auto issue = [&](int slot, int kt) {
    const uint32_t kb = (uint32_t)kt * 128;
    const bool kin = kt * 64 + lc * 8 < K;
    unsigned char* base = smem + slot * C::kPStageB;
#pragma unroll
    for (int s = 0; s < kPL; ++s) {
      const int q = wave + s * NWP;  // load index in the stage (wave-uniform)
      if (s < kXQ / NWP)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(base + q * 1024), 16,
                                                 off_or_oob(kin, vx + sgpr(s * sx + kb)), 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (lds_void*)(base + q * 1024), 16,
            off_or_oob(kin, va + sgpr((s - kXQ / NWP) * sa + kb)), 0, 0, 0);
    }
  };
  f32x4 tacc[PTM][PTN];
#pragma unroll
  for (int i = 0; i < PTM; ++i)
#pragma unroll
    for (int j = 0; j < PTN; ++j) tacc[i][j] = zero4();
  const int nk = (K + 63) / 64;
#pragma unroll
  for (int st = 0; st < S; ++st) issue(st, st);
  int slot = 0;
  for (int kt = 0; kt < nk; ++kt) {
    // Stage kt has landed once at most S - 1 newer stages are in flight.
    wait_vmcnt<(S - 1) * kPL>();
    __builtin_amdgcn_s_barrier();
    const unsigned char* xs = smem + slot * C::kPStageB;
    const unsigned char* as = xs + BM * 128;
    u32x4 xa[2][PTM], ta[2][PTN];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < PTM; ++i)
        xa[h][i] = *reinterpret_cast<const u32x4*>(
            xs + stage_off<64>(pm * PTM * 16 + i * 16 + lrow, h * 4 + lk));
#pragma unroll
      for (int j = 0; j < PTN; ++j)
        ta[h][j] = *reinterpret_cast<const u32x4*>(
            as + stage_off<64>(pn * PTN * 16 + j * 16 + lrow, h * 4 + lk));
    }
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();  // every wave's reads of this slot are done
    issue(slot, kt + S);
    slot = slot + 1 == S ? 0 : slot + 1;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < PTM; ++i)
#pragma unroll
        for (int j = 0; j < PTN; ++j) tacc[i][j] = mfma16x16x32(xa[h][i], ta[h][j], tacc[i][j]);
  }
  wait_vmcnt<0>();
  // Lane: T rows lk * 4 + q of its row block, rank column lrow of its block.
#pragma unroll
  for (int i = 0; i < PTM; ++i)
#pragma unroll
    for (int j = 0; j < PTN; ++j) {
      const int col = pn * PTN * 16 + j * 16 + lrow;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = pm * PTM * 16 + i * 16 + lk * 4 + q;
        ts[C::t_idx(row, col)] = col < r ? f2bf(scale * tacc[i][j][q]) : uint16_t(0);
      }
    }
  __syncthreads();  // T complete; the ring is free for the first tile's stages
}

// G > 1: a workgroup computes G consecutive N tiles of one M tile.  The first
// tile runs the fused K loop (base and T = X A^T); its epilogue keeps s T
// (bf16) in an LDS region outside the stage ring, and the later tiles run
// the K loop without A loads or T MFMAs and reuse it.  For large ranks this
// removes the per-tile recomputation of T (2 M K r flop per N tile, as much
// as the base contraction when r = BN).  tiles_n then counts groups of G.
template <class C, int G>
__global__ __launch_bounds__(C::NT) void fwd_tiled_bf16_kernel(
    int M, int N, int K, int r, const uint16_t* __restrict__ X, int64_t ldx,
    const uint16_t* __restrict__ W, int64_t ldw, const uint16_t* __restrict__ A, int64_t lda,
    const uint16_t* __restrict__ B, int64_t ldb, float scale, uint16_t* __restrict__ Y,
    int64_t ldy, int tiles_m, int tiles_n, int y_vec, int map_mode, uint16_t* __restrict__ tout,
    int64_t ldt) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  constexpr int BM = C::BM, BN = C::BN, RP = C::RP, TM = C::TM, TN = C::TN;
  constexpr int WN = C::WN, STAGES = C::STAGES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  static_assert(C::KS == 1 || G == 1, "k split: one tile per workgroup");
  static_assert(G == 1 || C::kGroupFits, "group epilogue fits in the ring");
  static_assert(!C::kPP || G == 1, "ping-pong: one tile per workgroup");
  // With loader waves: waves [0, NWC) multiply, waves [NWC, NW) load.
  const bool mul = C::PW == 0 || wave < C::NWC;
  const int lw = C::PW == 0 ? wave : wave - C::NWC;  // loader index (loaders only)
  // Without loader waves: does this wave issue stage loads (all do unless LD)?
  const bool ldr = C::PW > 0 || C::LW == C::NWC || wave < C::LW;
  const int cw = C::PW == 0 ? wave : (mul ? wave : 0);
  const int wgi = C::KS == 1 ? cw : cw % (C::WM * WN);  // wave within its k group
  const int kg = C::KS == 1 ? 0 : cw / (C::WM * WN);     // k group (KS = 2: its k32 half)
  const int wm = wgi / WN;
  const int wn = wgi % WN;
  const int lrow = lane & 15;
  const int lk = lane >> 4;

  // ---- tile id.  Workgroups reach the 8 XCDs round-robin (id % 8), and each
  // XCD has its own L2.  Mode 1: XCD x takes N tiles [x * tn/8, (x+1) * tn/8)
  // and all XCDs sweep the same group of G M tiles at the same time, so the X
  // rows of the group are shared by all XCDs through the last-level cache and
  // each L2 serves G M tiles x its N tiles.  Mode 2, the transpose: XCD x
  // takes M tiles [x * tm/8, (x+1) * tm/8) and sweeps the N tiles with all of
  // them at once (W shared through the last-level cache).  The host picks the
  // mode with fewer L2 fills.  Mode 0: tiles grouped along M (G at a time)
  // within XCD-contiguous id ranges.
  int m0, ng0;  // ng0: first N column of the group, in units of BN
  {
    const int total = tiles_m * tiles_n;
    if (map_mode == 1) {
      constexpr int GS = C::kGroupShared;
      const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, nper = tiles_n >> 3;
      const int sg = slot / (GS * nper), within = slot % (GS * nper);
      m0 = (sg * GS + within % GS) * BM;
      ng0 = (xcd * nper + within / GS) * G;
    } else if (map_mode == 2) {
      const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, mper = tiles_m >> 3;
      m0 = (xcd * mper + slot % mper) * BM;
      ng0 = (slot / mper) * G;
    } else {
      constexpr int GS = C::kGroup;
      const int pid = xcd_contiguous_id(blockIdx.x, total);
      const int group = pid / (GS * tiles_n);
      const int first_m = group * GS;
      const int gsize = min(tiles_m - first_m, GS);
      const int local = pid % (GS * tiles_n);
      m0 = (first_m + local % gsize) * BM;
      ng0 = (local / gsize) * G;
    }
  }

  // ---- buffer resources from the tile's first row to its last valid row.
  const int xrows = min(BM, M - m0);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(X + (int64_t)m0 * ldx), 0, (int)(xrows * ldx * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)A, 0, (int)(r * lda * 2), 0x00020000);

  // Lane i of a 1-KiB load writes staged row (q * rows_per_load + i / chunks),
  // physical chunk i % chunks, so it fetches logical chunk (i % chunks) ^
  // swz(row).  Loader w (a loader wave, or every wave of a tile without
  // loaders) issues X loads q = w, w + LW, ..., the same for W, and A load
  // q = w when w < kAN.
  constexpr int BK = C::BK, kRowB = C::kRowB, kRPL = C::kRowsPerLoad;
  const int lrow_in_load = lane / C::kChunks;
  const int lchunk = (lane % C::kChunks) ^ swz<BK>(lrow_in_load);
  const uint32_t vx = (uint32_t)((lw * kRPL + lrow_in_load) * ldx * 2 + lchunk * 16);
  const uint32_t vw = (uint32_t)((lw * kRPL + lrow_in_load) * ldw * 2 + lchunk * 16);
  const uint32_t va = (uint32_t)((lw * kRPL + lrow_in_load) * lda * 2 + lchunk * 16);
  const uint32_t sx = (uint32_t)(C::LW * kRPL * ldx * 2);  // byte stride between a loader's slots
  const uint32_t sw = (uint32_t)(C::LW * kRPL * ldw * 2);
  const uint32_t sa = (uint32_t)(C::LW * kRPL * lda * 2);

  const int rot = ring_rot<C>(wn);
  f32x4 acc[TM][TN];
  f32x4 tacc[C::kTSlots];
#pragma unroll
  for (int s = 0; s < C::kTSlots; ++s) tacc[s] = zero4();

  // G == 1: the B tile's elements of this thread, loaded before the K loop.
  constexpr bool kBEarly = C::kBEarly && G == 1;
  uint16_t bpre[kBEarly ? C::kBPre : 1];
  if constexpr (kBEarly) {
    const int n0 = ng0 * BN;
#pragma unroll
    for (int i = 0; i < C::kBPre; ++i) {
      const int e = tid + i * C::NWC * kWave;
      const int n = e / RP, j = e % RP;
      bpre[i] = (j < r && n0 + n < N) ? B[(int64_t)(n0 + n) * ldb + j] : uint16_t(0);
    }
  }

  // G == 1, no early B: the B tile by direct loads into LDS past the ring,
  // when every 16-B chunk of a B row is aligned and wholly inside or wholly
  // past the rank (else the gather after the K loop).  These loads are older
  // than every stage load, so the K loop's waits cover them.
  constexpr bool kBDma = C::kBDma && G == 1;
  const bool bdma = kBDma && mul && r % 8 == 0 && ldb % 8 == 0 &&
                    (reinterpret_cast<uintptr_t>(B) & 15) == 0;
  if constexpr (kBDma) {
    if (bdma) {
      const int n0 = ng0 * BN;
      const int brows = max(0, min(BN, N - n0));
      const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(B + (int64_t)n0 * ldb), 0, (int)(brows * ldb * 2), 0x00020000);
      constexpr int kBL = C::kBDmaB / 1024;  // 1-KiB loads
      for (int p = cw; p < kBL; p += C::NWC) {
        const int byte = p * 1024 + lane * 16;
        const int row = byte / (RP * 2), j0 = (byte % (RP * 2)) / 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (lds_void*)(smem + C::kBDmaOff + p * 1024), 16,
            off_or_oob(j0 < r, (uint32_t)(row * ldb * 2 + j0 * 2)), 0, 0, 0);
      }
    }
  }

  // Tiles with loader waves: the loaders fetch the B tile into registers
  // (16 B per load, before any stage load, so the stage waits' counts still
  // hold: loads complete in order) and write it to LDS after the K loop,
  // when every 16-B chunk of a B row is aligned and wholly inside or wholly
  // past the rank (else the gather after the K loop).  Assigned only on the
  // loaders' path, so the multiplying waves' loop does not hold it.  (Not
  // for 256 x 160: its multiplying waves then spill.)
  constexpr bool kBPf = C::PW > 0 && G == 1 && C::KS == 1 && C::BM * C::BN <= 128 * 256;
  constexpr int kBChunks = C::BN * RP / 8;                        // 16-B chunks of the tile
  constexpr int kBCh = kBPf ? (kBChunks + C::PW * kWave - 1) / (C::PW * kWave) : 1;
  const bool bpf = kBPf && r % 8 == 0 && ldb % 8 == 0 && (reinterpret_cast<uintptr_t>(B) & 15) == 0;
  u32x4 bpre16[kBCh];
  auto fetch_b = [&](int nb0) {
#pragma unroll
    for (int i = 0; i < kBCh; ++i) {
      const int cidx = lw * kWave + lane + i * C::PW * kWave;
      const int n = cidx / (RP / 8), j0 = (cidx % (RP / 8)) * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (cidx < kBChunks && nb0 + n < N && j0 < r)
        v = *reinterpret_cast<const u32x4*>(B + (int64_t)(nb0 + n) * ldb + j0);
      bpre16[i] = v;
    }
  };

  if constexpr (C::kTP) {
    static_assert(G > 1, "T prologue: a group of N tiles");
    t_prologue<C>(smem, reinterpret_cast<uint16_t*>(smem + C::kTOffG), K, r, scale, rx, ra, ldx,
                  lda, wave, lane);
  }

  for (int g = 0; g < G; ++g) {
  const int n0 = (ng0 + g) * BN;
  if (n0 >= N) break;  // uniform: the group's last tiles may lie past N
  const int wrows = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + (int64_t)n0 * ldw), 0, (int)(wrows * ldw * 2), 0x00020000);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = zero4();

  // The K loop, with (WT) or without the down-projection.
  auto kloop = [&](auto wt) {
  constexpr bool WT = decltype(wt)::value;

  // K loop, software-pipelined three ways.  A stage holds BK = 32 * NSUB
  // k-values; the MFMAs consume it in NSUB substeps of k32.  Substep u of
  // stage kt multiplies from registers while the fragments of the next
  // substep are read from LDS into a register ring (row i lands in a[i] as
  // soon as the MFMAs of row i have consumed it).  Before the last substep of
  // stage kt the waves synchronise once: stage kt+1 has landed, and the slot
  // of stage kt, all of whose fragments have now been read, is refilled with
  // stage kt+STAGES from global memory.  Loads of stages past K read zeros, so
  // the substeps have no branches and the scheduler can interleave their
  // streams.
  constexpr int NSUB = BK / 32;
  const int nk = (K + BK - 1) / BK;
  if constexpr (C::kPP) {
    // Ping-pong.  Waves 0-3 (group 0) and 4-7 (group 1) sit in pairs on the
    // four SIMDs (a wave's SIMD is its index mod 4).  Each k32 stage q is a
    // read phase R(q) -- this wave's X, W and A fragments of stage q from
    // LDS into registers, then its share of the loads of stage q + STAGES -
    // 1 into the ring slot that stage q - 1 has left -- and a multiply
    // phase M(q) on those registers.  Group 1 runs one phase behind group 0
    // and every phase ends at a barrier of all eight waves, so on each SIMD
    // one wave issues MFMAs while the other reads: the matrix pipe is fed
    // by one wave at a time without the two competing for it, and one
    // register set per wave suffices.  Order of the phases (barrier b_k
    // between phases k - 1 and k of the sequence R(0) M(0) R(1) M(1) ...):
    // group 0 runs phase k, group 1 phase k - 1, after b_k.
    //  * Slot reuse: stage q - 1's slot is refilled in R(q) of either group,
    //    after both groups' R(q - 1) have waited for their reads (lgkmcnt)
    //    and passed a barrier.
    //  * Arrival: stage q + 1 is read from R(q + 1) of group 0 on; every
    //    wave waits for its own loads of that stage (vmcnt, two newer stages
    //    in flight) before the barrier that precedes it: group 0 at the end
    //    of M(q), group 1 at the end of R(q).
    // Loads of stages past K read zeros; all of them have landed (vmcnt 0)
    // before the epilogue reuses the LDS.
    constexpr int S = STAGES;
    const int grp = wave >> 2;
    const int px0 = wm * TM * 16 + lrow;
    const int pw0 = wn * TN * 16 + lrow;
    Frags<C> f;
    auto bar = [] {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int st = 0; st < S - 1; ++st)
      issue_stage<C, WT>(smem, st, st * BK, K, wave, lchunk, rx, rw, ra, vx, vw, va, sx, sw, sa);
    wait_stages<C, S - 2, WT>(wave);
    bar();
    if (grp == 1) bar();
    for (int q = 0; q < nk; ++q) {
      const unsigned char* xs = smem + (q & (S - 1)) * C::kStageB;
      const unsigned char* ws = xs + BM * kRowB;
      const unsigned char* as = ws + BN * kRowB;
#pragma unroll
      for (int i = 0; i < TM; ++i)
        f.a[i] = *reinterpret_cast<const u32x4*>(
            xs + stage_off<BK>(px0 + ring_row_block<C>(i, rot) * 16, lk));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        f.b[j] = *reinterpret_cast<const u32x4*>(ws + stage_off<BK>(pw0 + j * 16, lk));
#pragma unroll
      for (int u = 0; u < C::kTF; ++u)
        f.t[u] = *reinterpret_cast<const u32x4*>(as + stage_off<BK>(t_block<C>(wn, u) * 16 + lrow, lk));
      wait_lgkm0();
      __builtin_amdgcn_sched_barrier(0);
      const int ls = (q + S - 1) & (S - 1);
      const int lk0 = (q + S - 1) * BK;
      if constexpr (C::kPPSpread) {
        issue_stage_a<C>(smem, ls, lk0, K, wave, lchunk, ra, va, sa);
        // Newer than stage q + 1: stage q + 2 and the A load of q + 3.
        if (grp == 1) {
          if (wave < C::kAN) wait_vmcnt<C::kLoadsHi + 1>();
          else wait_vmcnt<C::kLoadsLo>();
        }
      } else {
        issue_stage<C, WT>(smem, ls, lk0, K, wave, lchunk, rx, rw, ra, vx, vw, va, sx, sw, sa);
        if (grp == 1) wait_stages<C, S - 2, WT>(wave);
      }
      bar();
      t_update_ab<C>(f.a, f.t, tacc);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16x16x32(f.b[j], f.a[i], acc[i][j]);
      if constexpr (C::kPPSpread) {
        issue_stage<C, false>(smem, ls, lk0, K, wave, lchunk, rx, rw, ra, vx, vw, va, sx, sw, sa);
        // One X or W load after every eighth MFMA.
        constexpr int kXW = C::kXL + C::kWL;
        constexpr int kM = C::kTSlots + TM * TN;
        constexpr int kEvery = kM / (kXW + 1);
#pragma unroll
        for (int d = 0; d < kXW; ++d) {
          __builtin_amdgcn_sched_group_barrier(0x008, kEvery, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);       // VMEM (DMA) issue
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kM - kXW * kEvery, 0);
      }
      if (grp == 0) wait_stages<C, S - 2, WT>(wave);
      bar();
    }
    if (grp == 0) bar();
    wait_vmcnt<0>();
    return;
  } else {
  if constexpr (C::PW > 0) {
    if (!mul) {
      if constexpr (kBPf) {
        if (bpf) fetch_b(n0);
      }
      // Loader: the same barriers as the multiplying waves (one after stage
      // 0 has landed, one per stage), each preceded by the wait for the
      // stage the multipliers read next; after the barrier of stage kt every
      // read of stage kt is done and its slot is refilled.
#pragma unroll
      for (int s = 0; s < STAGES; ++s)
        issue_stage<C, WT>(smem, s, s * BK, K, lw, lchunk, rx, rw, ra, vx, vw, va, sx, sw, sa);
      wait_stages<C, STAGES - 1, WT>(lw);
      __builtin_amdgcn_s_barrier();
      int slot = 0;
      for (int kt = 0; kt < nk; ++kt) {
        wait_stages<C, STAGES - 2, WT>(lw);
        __builtin_amdgcn_s_barrier();
        issue_stage<C, WT>(smem, slot, (kt + STAGES) * BK, K, lw, lchunk, rx, rw, ra, vx, vw, va,
                           sx, sw, sa);
        slot = slot + 1 == STAGES ? 0 : slot + 1;
      }
      return;
    }
  } else {
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
      if (ldr) issue_stage<C, WT>(smem, s, s * BK, K, wave, lchunk, rx, rw, ra, vx, vw, va, sx, sw, sa);
  }

  const int xrow0 = wm * TM * 16 + lrow;  // + 16 * ring_row_block(k) for ring slot k
  const int wrow0 = wn * TN * 16 + lrow;
  Frags<C> cur;
  const int lk0 = C::KS == 2 ? kg * 4 + lk : lk;  // logical chunk of this wave's first k32
  if constexpr (C::PW == 0) {
    if (ldr) wait_stages<C, STAGES - 1, WT>(wave);
  }
  __builtin_amdgcn_s_barrier();
  {
    const unsigned char* xs = smem;
    const unsigned char* ws = xs + BM * kRowB;
    const unsigned char* as = ws + BN * kRowB;
#pragma unroll
    for (int i = 0; i < TM; ++i)
      cur.a[i] = *reinterpret_cast<const u32x4*>(
          xs + stage_off<BK>(xrow0 + ring_row_block<C>(i, rot) * 16, lk0));
#pragma unroll
    for (int j = 0; j < TN; ++j)
      cur.b[j] = *reinterpret_cast<const u32x4*>(ws + stage_off<BK>(wrow0 + j * 16, lk0));
    if constexpr (WT) {
#pragma unroll
      for (int u = 0; u < C::kTF; ++u)
        cur.t[u] = *reinterpret_cast<const u32x4*>(as + stage_off<BK>(t_block<C>(wn, u) * 16 + lrow, lk0));
    }
  }

  // One substep: MFMAs from (a ring, bc, tc); the next substep's W and A
  // fragments go to (bx, tx) and its X fragments refill the ring row by row.
  // The two B/T register sets alternate between substeps, so no copies.
  auto substep = [&](bool sync, int rslot, int nslot, int kt, int u, u32x4 (&bc)[TN],
                     u32x4 (&tc)[C::kTF], u32x4 (&bx)[TN], u32x4 (&tx)[C::kTF]) {
    // T MFMAs first: they keep the MFMA pipe busy across the barrier.
    if constexpr (WT) t_update_ab<C>(cur.a, tc, tacc);
    if (sync) {
      // Stage kt+1 has landed once at most STAGES-2 later stages are in
      // flight; this wave's reads of stage kt are complete.  After the
      // barrier every wave is past both.  A bare s_barrier: a fence would
      // drain every stage in flight.
      if constexpr (C::PW == 0) {
        if (ldr) wait_stages<C, STAGES - 2, WT>(wave);
      }
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      if constexpr (C::PW == 0) {
        if (ldr)
          issue_stage<C, WT>(smem, rslot, (kt + STAGES) * BK, K, wave, lchunk, rx, rw, ra, vx, vw,
                             va, sx, sw, sa);
      }
    }
    const unsigned char* xs = smem + (sync ? nslot : rslot) * C::kStageB;
    const unsigned char* ws = xs + BM * kRowB;
    const unsigned char* as = ws + BN * kRowB;
    // logical 16-B chunk of the next substep
    const int cc = (sync ? (C::KS == 2 ? kg * 4 : 0) : (u + 1) * 4) + lk;
    // After the final substep the reads fetch a zero stage (never used).
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bx[j] = *reinterpret_cast<const u32x4*>(ws + stage_off<BK>(wrow0 + j * 16, cc));
    if constexpr (WT) {
#pragma unroll
      for (int f = 0; f < C::kTF; ++f)
        tx[f] = *reinterpret_cast<const u32x4*>(as + stage_off<BK>(t_block<C>(wn, f) * 16 + lrow, cc));
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma16x16x32(bc[j], cur.a[i], acc[i][j]);
      cur.a[i] = *reinterpret_cast<const u32x4*>(
          xs + stage_off<BK>(xrow0 + ring_row_block<C>(i, rot) * 16, cc));
    }
    // Interleave DMA issues and LDS reads between the MFMAs.
    constexpr int kDma = C::PW > 0 ? 0 : C::kXL + C::kWL;
    constexpr int kReads = TN + (WT ? C::kTF : 0) + TM;
    constexpr int kMfma = TM * TN;
    if (sync) {
#pragma unroll
      for (int d = 0; d < kDma; ++d) {
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM (DMA) issue
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      }
#pragma unroll
      for (int q = 0; q < kReads; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      }
      __builtin_amdgcn_sched_group_barrier(
          0x008, kMfma - kDma - kReads > 0 ? kMfma - kDma - kReads : 0, 0);
    } else {
#pragma unroll
      for (int q = 0; q < kReads; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kReads > 0 ? kMfma - kReads : 0, 0);
    }
  };

  u32x4 b2[TN], t2[C::kTF];
  int rslot = 0;  // ring slot of stage kt
  if constexpr (C::KS == 2) {
    // One substep per stage (this group's k32 half), ending in the stage's
    // barrier; two stages per iteration so the register sets alternate.
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      int nslot = rslot + 1 == STAGES ? 0 : rslot + 1;
      substep(true, rslot, nslot, kt, 0, cur.b, cur.t, b2, t2);
      rslot = nslot;
      nslot = rslot + 1 == STAGES ? 0 : rslot + 1;
      substep(true, rslot, nslot, kt + 1, 0, b2, t2, cur.b, cur.t);
      rslot = nslot;
    }
    if (kt < nk) substep(true, rslot, rslot + 1 == STAGES ? 0 : rslot + 1, kt, 0, cur.b, cur.t, b2, t2);
  } else {
  for (int kt = 0; kt < nk; ++kt) {
    const int nslot = rslot + 1 == STAGES ? 0 : rslot + 1;  // slot of stage kt+1
    if constexpr (NSUB == 2) {
      substep(false, rslot, nslot, kt, 0, cur.b, cur.t, b2, t2);
      substep(true, rslot, nslot, kt, 1, b2, t2, cur.b, cur.t);
    } else {
      substep(true, rslot, nslot, kt, 0, cur.b, cur.t, b2, t2);
#pragma unroll
      for (int j = 0; j < TN; ++j) cur.b[j] = b2[j];
#pragma unroll
      for (int f = 0; f < C::kTF; ++f) cur.t[f] = t2[f];
    }
    rslot = nslot;
  }
  }
  }  // not ping-pong
  };  // kloop
  if constexpr (C::kTP) {
    kloop(std::false_type{});  // T from the prologue
  } else {
    if (g == 0) kloop(std::true_type{});
    else kloop(std::false_type{});
  }
  __syncthreads();

  // ---- k split: add the two groups' partial sums.  Group g keeps ring slots
  // [g TM/2, (g+1) TM/2) of its accumulators and receives the partner's
  // values for them; group 0 receives group 1's partial T.  Addition is
  // commutative, so every kept value is (group 0's sum) + (group 1's sum).
  constexpr int TH = TM / C::KS;  // ring slots a wave keeps
  if constexpr (C::KS == 2) {
    float* xch = reinterpret_cast<float*>(smem + C::kXOff);
    constexpr int kTOff = C::WM * WN * TM * TN;  // fragment index of the T area
    auto frag = [&](int f) { return reinterpret_cast<f32x4*>(xch + (f * kWave + lane) * 4); };
    auto put = [&](auto s0c) {
      constexpr int S0 = decltype(s0c)::value;
#pragma unroll
      for (int i = 0; i < TH; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) *frag(((wgi * 2 + kg) * TH + i) * TN + j) = acc[S0 + i][j];
    };
    auto take = [&](auto s0c) {
      constexpr int S0 = decltype(s0c)::value;
#pragma unroll
      for (int i = 0; i < TH; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const f32x4 v = *frag(((wgi * 2 + 1 - kg) * TH + i) * TN + j);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[S0 + i][j][q] += v[q];
        }
    };
    if (mul) {
      if (kg == 0) {
        put(std::integral_constant<int, TH>{});
      } else {
        put(std::integral_constant<int, 0>{});
#pragma unroll
        for (int sl = 0; sl < C::kTSlots; ++sl) *frag(kTOff + wgi * C::kTSlots + sl) = tacc[sl];
      }
    }
    __syncthreads();
    if (mul) {
      if (kg == 0) {
        take(std::integral_constant<int, 0>{});
#pragma unroll
        for (int sl = 0; sl < C::kTSlots; ++sl) {
          const f32x4 v = *frag(kTOff + wgi * C::kTSlots + sl);
#pragma unroll
          for (int q = 0; q < 4; ++q) tacc[sl][q] += v[q];
        }
      } else {
        take(std::integral_constant<int, TH>{});
      }
    }
  }

  // ---- epilogue 1: scaled T (bf16) and the B tile into LDS.  With G > 1,
  // T lives past the stage ring and is written by the first tile only.
  uint16_t* ts = reinterpret_cast<uint16_t*>(smem + (G > 1 ? C::kTOffG : 0));
  uint16_t* bs = G > 1 ? reinterpret_cast<uint16_t*>(smem) : ts + BM * C::kTRow;
  int bst = C::kTS;  // B tile row stride (elements)
  // A group tile with the swizzled T keeps its B tile in the same layout
  // (unpadded rows of RP, 16-B chunks XOR-swizzled by row), filled by direct
  // 16-B loads where every chunk of a B row is aligned and wholly inside or
  // wholly past the rank, else gathered element by element.
  constexpr bool kBSw = G > 1 && C::kTSw;
  auto bidx = [&](int n, int col) { return kBSw ? C::t_idx(n, col) : n * bst + col; };
  if constexpr (kBDma) {
    if (bdma) {
      bs = reinterpret_cast<uint16_t*>(smem + C::kBDmaOff);
      bst = RP;
    }
  }
  if (!C::kTP && g == 0 && kg == 0 && mul) {
#pragma unroll
  for (int sl = 0; sl < C::kTSlots; ++sl) {
    const int i = ring_row_block<C>(t_ring_slot<C>(sl), rot);
    const int j = t_block<C>(wn, t_frag<C>(sl)) * 16 + lrow;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = wm * TM * 16 + i * 16 + lk * 4 + q;
      ts[C::t_idx(row, j)] = j < r ? f2bf(scale * tacc[sl][q]) : uint16_t(0);
    }
  }
  }
  if constexpr (kBEarly) {
    if (mul) {
#pragma unroll
      for (int i = 0; i < C::kBPre; ++i) {
        const int e = tid + i * C::NWC * kWave;
        bs[(e / RP) * C::kTS + e % RP] = bpre[i];
      }
    }
  } else if constexpr (kBSw) {
    if (r % 8 == 0 && ldb % 8 == 0 && (reinterpret_cast<uintptr_t>(B) & 15) == 0) {
      const int brows = max(0, min(BN, N - n0));
      const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(B + (int64_t)n0 * ldb), 0, (int)(brows * ldb * 2), 0x00020000);
      constexpr int kBL = BN * RP * 2 / 1024;  // 1-KiB loads
      static_assert(kBL % C::NW == 0, "B tile loads: the same count for every wave");
      for (int p = wave; p < kBL; p += C::NW) {
        // lane: row n, physical chunk pc; it fetches logical chunk pc ^ (n mod RP / 8)
        const int byte = p * 1024 + lane * 16;
        const int n = byte / (RP * 2), pc = (byte % (RP * 2)) / 16;
        const int j0 = (pc ^ (n & (RP / 8 - 1))) * 8;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (lds_void*)(smem + p * 1024), 16,
            off_or_oob(j0 < r, (uint32_t)(n * ldb * 2 + j0 * 2)), 0, 0, 0);
      }
      wait_vmcnt<0>();
    } else {
      for (int e = tid; e < BN * RP; e += C::NT) {
        const int n = e / RP, j = e % RP;
        uint16_t v = 0;
        if (j < r && n0 + n < N) v = B[(int64_t)(n0 + n) * ldb + j];
        bs[C::t_idx(n, j)] = v;
      }
    }
  } else {
    if (kBPf && bpf) {
      if (!mul) {
#pragma unroll
        for (int i = 0; i < kBCh; ++i) {
          const int cidx = lw * kWave + lane + i * C::PW * kWave;
          if (cidx < kBChunks) {
            const int n = cidx / (RP / 8), j0 = (cidx % (RP / 8)) * 8;
            *reinterpret_cast<u32x4*>(bs + n * C::kTS + j0) = bpre16[i];
          }
        }
      }
    } else if (!bdma) {
      for (int e = tid; e < BN * RP; e += C::NT) {
        const int n = e / RP, j = e % RP;
        uint16_t v = 0;
        if (j < r && n0 + n < N) v = B[(int64_t)(n0 + n) * ldb + j];
        bs[n * C::kTS + j] = v;
      }
    }
  }
  __syncthreads();

  // Optional side output: the scaled down-projection s T of this M tile, as
  // the epilogue rounded it, stored transposed ([r, ldt], tokens contiguous)
  // by the workgroup of the first N tile.  Rows past M hold zeros (X rows
  // past M read as zeros); the last M tile also writes the zero rows from its
  // end up to ldt, which can lie past it when BM is smaller than ldt's
  // padding.  The backward takes s dY B from here.
  if (tout != nullptr && ng0 == 0 && g == 0) {
    const int rend = m0 + BM >= M ? (int)ldt : min(m0 + BM, (int)ldt);  // rows [m0, rend)
    const int nrow = rend - m0;
    for (int e = tid; e < nrow * r; e += C::NT) {
      const int row = e % nrow, j = e / nrow;
      tout[(int64_t)j * ldt + m0 + row] = row < BM ? ts[C::t_idx(row, j)] : uint16_t(0);
    }
  }

  uint16_t* ys = reinterpret_cast<uint16_t*>(smem);
  // A group tile whose output staging does not fit in the ring stages it
  // over the start of s T as well: from the up-projection until the stores
  // have read the staging area each thread holds 16-B chunks tid, tid + NT,
  // ... of the covered part of s T in registers (which the K loop's
  // operands have left free), then writes them back for the next tile.
  constexpr bool kTPark = G > 1 && C::kYSplit;
  constexpr int kTParkN = kTPark ? (C::kYB - C::kTOffG + 16 * C::NT - 1) / (16 * C::NT) : 1;
  static_assert(!kTPark || kTParkN * 16 * C::NT <= BM * C::kTRow * 2, "parked chunks lie in s T");
  u32x4 tpark[kTParkN];
  if constexpr (C::KS == 1) {
  // ---- epilogue 2: acc += (s T) B^T on MFMA, contraction over the rank.
  if (!mul) {
  } else if constexpr (RP >= 32) {
#pragma unroll
    for (int kk = 0; kk < RP / 32; ++kk) {
      u32x4 a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *reinterpret_cast<const u32x4*>(
            ts + C::t_idx(wm * TM * 16 + ring_row_block<C>(i, rot) * 16 + lrow, kk * 32 + lk * 8));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = *reinterpret_cast<const u32x4*>(
            bs + bidx(wn * TN * 16 + j * 16 + lrow, kk * 32 + lk * 8));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16x16x32(b[j], a[i], acc[i][j]);
    }
  } else {
    u32x2 a[TM], b[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
      a[i] = *reinterpret_cast<const u32x2*>(
          ts + C::t_idx(wm * TM * 16 + ring_row_block<C>(i, rot) * 16 + lrow, lk * 4));
#pragma unroll
    for (int j = 0; j < TN; ++j)
      b[j] = *reinterpret_cast<const u32x2*>(bs + (wn * TN * 16 + j * 16 + lrow) * bst + lk * 4);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma16x16x16(b[j], a[i], acc[i][j]);
  }
  if constexpr (kTPark) {
#pragma unroll
    for (int i = 0; i < kTParkN; ++i)
      tpark[i] = reinterpret_cast<const u32x4*>(ts)[i * C::NT + tid];
  }
  __syncthreads();

  // ---- epilogue 3: round once to bf16, stage, store coalesced.
  if (mul) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int row = wm * TM * 16 + ring_row_block<C>(i, rot) * 16 + lrow;
      *reinterpret_cast<u32x2*>(ys + row * C::kYS + wn * TN * 16 + j * 16 + lk * 4) =
          u32x2{pack_bf2(acc[i][j][0], acc[i][j][1]), pack_bf2(acc[i][j][2], acc[i][j][3])};
    }
  }
  __syncthreads();
  } else {
  // ---- epilogue 2: acc += (s T) B^T on MFMA, contraction over the rank, for
  // the ring slots [S0, S0 + TH) this wave keeps.
  auto epi2 = [&](auto s0c) {
    constexpr int S0 = decltype(s0c)::value;
    if constexpr (RP >= 32) {
#pragma unroll
      for (int kk = 0; kk < RP / 32; ++kk) {
        u32x4 a[TH], b[TN];
#pragma unroll
        for (int i = 0; i < TH; ++i)
          a[i] = *reinterpret_cast<const u32x4*>(
              ts + C::t_idx(wm * TM * 16 + ring_row_block<C>(S0 + i, rot) * 16 + lrow,
                            kk * 32 + lk * 8));
#pragma unroll
        for (int j = 0; j < TN; ++j)
          b[j] = *reinterpret_cast<const u32x4*>(
              bs + bidx(wn * TN * 16 + j * 16 + lrow, kk * 32 + lk * 8));
#pragma unroll
        for (int i = 0; i < TH; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[S0 + i][j] = mfma16x16x32(b[j], a[i], acc[S0 + i][j]);
      }
    } else {
      u32x2 a[TH], b[TN];
#pragma unroll
      for (int i = 0; i < TH; ++i)
        a[i] = *reinterpret_cast<const u32x2*>(
            ts + C::t_idx(wm * TM * 16 + ring_row_block<C>(S0 + i, rot) * 16 + lrow, lk * 4));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = *reinterpret_cast<const u32x2*>(bs + (wn * TN * 16 + j * 16 + lrow) * bst + lk * 4);
#pragma unroll
      for (int i = 0; i < TH; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[S0 + i][j] = mfma16x16x16(b[j], a[i], acc[S0 + i][j]);
    }
  };
  if (mul) {
    if (kg == 0) epi2(std::integral_constant<int, 0>{});
    else epi2(std::integral_constant<int, TH>{});
  }
  __syncthreads();

  // ---- epilogue 3: round once to bf16, stage, store coalesced.
  auto epi3 = [&](auto s0c) {
    constexpr int S0 = decltype(s0c)::value;
#pragma unroll
    for (int i = S0; i < S0 + TH; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = wm * TM * 16 + ring_row_block<C>(i, rot) * 16 + lrow;
        *reinterpret_cast<u32x2*>(ys + row * C::kYS + wn * TN * 16 + j * 16 + lk * 4) =
            u32x2{pack_bf2(acc[i][j][0], acc[i][j][1]), pack_bf2(acc[i][j][2], acc[i][j][3])};
      }
  };
  if (mul) {
    if (kg == 0) epi3(std::integral_constant<int, 0>{});
    else epi3(std::integral_constant<int, TH>{});
  }
  __syncthreads();
  }
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
  if (G > 1) __syncthreads();  // the next tile's loads reuse the staging area
  if constexpr (kTPark) {
#pragma unroll
    for (int i = 0; i < kTParkN; ++i) reinterpret_cast<u32x4*>(ts)[i * C::NT + tid] = tpark[i];
  }
  }  // tiles of the group
}

template <class C, int G = 1>
hipError_t launch(const FwdArgs& a, hipStream_t s) {
  const int tiles_m = (int)((a.M + C::BM - 1) / C::BM);
  const int tiles_n = (int)((a.N + C::BN * G - 1) / (C::BN * G));  // groups of G N tiles
  const int y_vec = ((reinterpret_cast<uintptr_t>(a.Y) & 15) == 0) && (a.ldy % 8 == 0);
  // L2 fills (in K-rows of X or W) of the two XCD-split mappings: mode 1
  // reads all of X on every XCD and W once per group of G M tiles; mode 2
  // reads all of W on every XCD and X once per N sweep step (32 resident
  // tiles per XCD).
  int map_mode = 0;
  {
    const bool ok1 = (tiles_n % 8 == 0) && (tiles_m % C::kGroupShared == 0);
    const bool ok2 = (tiles_m % 8 == 0);
    const double f1 = 8.0 * a.M + (double)(tiles_m / C::kGroupShared) * a.N;
    const int per_sweep = 32 / (tiles_m / 8 > 0 ? tiles_m / 8 : 1);
    const double f2 = 8.0 * a.N + (double)((tiles_n + per_sweep - 1) / (per_sweep > 0 ? per_sweep : 1)) * a.M;
    if (ok1 && (!ok2 || f1 <= f2)) map_mode = 1;
    else if (ok2) map_mode = 2;
  }
  auto kern = fwd_tiled_bf16_kernel<C, G>;
  constexpr int lds = G > 1 ? C::kLdsG : C::kLds;
  static_assert(lds <= 160 * 1024, "LDS budget");
  static std::atomic<uint64_t> attr_done{0};
  if (hipError_t e = ensure_lds(kern, lds, attr_done); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(tiles_m * tiles_n), dim3(C::NT), lds, s, (int)a.M, (int)a.N,
                     (int)a.K, (int)a.r, static_cast<const uint16_t*>(a.X), a.ldx,
                     static_cast<const uint16_t*>(a.W), a.ldw, static_cast<const uint16_t*>(a.A),
                     a.lda, static_cast<const uint16_t*>(a.B), a.ldb, a.scale,
                     static_cast<uint16_t*>(a.Y), a.ldy, tiles_m, tiles_n, y_vec, map_mode,
                     static_cast<uint16_t*>(a.tout), a.ldt);
  return hipGetLastError();
}

// Tile shapes.  Large: 256 x 256, 8 waves (2 x 4), wave tile 128 x 64.
// Medium: 128 x 128, 8 waves (4 x 2), wave tile 32 x 64; two waves per SIMD
// hide more of the L2 latency than one 64 x 64 wave per SIMD (measured:
// 17.2 -> 14.0 us on X[4096,1024] W[1024,1024]), and 64-deep stages move
// whole 128-B lines per row.
template <int RP>
using Big = Cfg<256, 256, 2, 4, RP, 2, 64>;
// The same tile with the ping-pong K loop: 32-deep stages, four in flight.
template <int RP>
using BigPP = Cfg<256, 256, 2, 4, RP, 4, 32, 1, 0, 0, 1>;
template <int RP>
using BigPP2 = Cfg<256, 256, 2, 4, RP, 4, 32, 1, 0, 0, 2>;
// The two-stage 256 x 256 tile with the stage loads issued by waves 0-3 only
// (see LD): 16384 x 8192 x 8192 r16 1.57-1.60 ms against 1.64-1.69, r64
// 1.84 against 2.01 (and 1.96 on the ping-pong tile), q_proj 145-150 against
// 158-163 us; with waves 0-1 only 1.66 ms.  A single round of tiles (4096^3)
// runs 5 % slower: four waves fill the first two stages alone.
template <int RP>
using BigL4 = Cfg<256, 256, 2, 4, RP, 2, 64, 1, 0, 0, 0, 4>;
// (Measured and dropped: the same tile as 4 waves of 128 x 128, one per
// SIMD with the accumulators in AGPRs, reads a third fewer LDS bytes per
// MFMA but ran 1.48x slower on 16384 x 8192 x 8192 r16 (2621 vs 1768 us) and
// 1.55x on 8192 x 4096 x 2560: one wave per SIMD cannot hide its own loads.)
// Tall: 64 x 32, 4 waves (4 x 1), eight 64-deep stages in flight, for few
// tokens (M <= 64): the cost is streaming W and re-reading X from L2, so the
// tile is narrow and the ring deep.
template <int RP>
using Tall = Cfg<64, 32, 4, 1, RP, 8, 64>;
template <int RP>
using Mid = Cfg<128, 128, 4, 2, RP, 2, 64>;
// The same tile with three stages: one workgroup per CU with two stages in
// flight (2048 x 2048 x 2048 r16: 24.5 vs 27.1 us; slower on the projection
// shapes).  Measured and dropped: 32-deep stages four deep (64-B rows; 10-25 %
// slower: half-line loads and twice the barriers) and 4 waves of 64 x 64 with
// four stages (10-30 % slower).
template <int RP>
using Mid3 = Cfg<128, 128, 4, 2, RP, 3, 64>;
// 128 x 128 with the k split: 4 x 2 waves of 32 x 64 per k group, two
// groups (16 waves, four per SIMD), three stages.
template <int RP>
using MidK2 = Cfg<128, 128, 4, 2, RP, 3, 64, 2>;
// The three-stage 128 x 128 tile with four loader waves (12 waves).
// Measured on X[4096,1024] W[1024,1024] r16: 13.0 us against 14.6 us for
// the same tile without loaders; two loaders 13.2 us, eight 12.9 us but
// slower elsewhere; with two stages 13.1 us but slower at larger K.
template <int RP>
using Mid3L = Cfg<128, 128, 4, 2, RP, 3, 64, 1, 4>;
// 128 x 256 with wave tiles of 64 x 64 (fewer LDS bytes per MFMA than 32 x
// 64) and four loaders, three stages: 8192 x 1024 x 2560 r32 44.4 us against
// 50.5 on 128 x 128 (two workgroups per CU); 256 x 128 measured slower.
template <int RP>
using WideL = Cfg<128, 256, 2, 4, RP, 3, 64, 1, 4>;
// 256 x 160 with four loaders, two stages (8 waves of 64 x 80: 0.45 LDS
// fragment reads per MFMA), for grids whose 128 x 256 tiles leave the last
// round of 256 CUs part-empty: 8192 x 2560 outputs, K 4096, r32 (the q_proj
// backward's dX product) take 512 such tiles, two full rounds, 162 us
// against 183.5 us on 640 tiles of 128 x 256 (2.5 rounds).
template <int RP>
using BigNL = Cfg<256, 160, 4, 2, RP, 2, 64, 1, 4>;
// Ranks 33-128 on large grids: 128 x 256 tiles (8 waves of 64 x 64, two
// stages) where a workgroup walks 8 consecutive N tiles of one row block and
// computes T = X A^T with the first only; s T (bf16) stays in the last
// BM x RP x 2 bytes of the LDS (unpadded, swizzled), after the ring.
template <int RP>
using WideT = Cfg<128, 256, 2, 4, RP, 2, 64, 1, 0, 1>;
constexpr int kWideTGroup = 8;
// 256 x 256 keeping T over 8 N tiles, T from a prologue (ranks 33-128): s T
// (BM x RP bf16) stays in LDS past the ring, so rank 128 leaves 96 KiB for
// three 32-deep stages and rank 64 128 KiB for two 64-deep ones; stage loads
// from waves 0-3.
template <int RP>
using BigT = std::conditional_t<(RP <= 64), Cfg<256, 256, 2, 4, RP, 2, 64, 1, 0, 1, 0, 4, 1>,
                                Cfg<256, 256, 2, 4, RP, 3, 32, 1, 0, 1, 0, 4, 1>>;
// Small tiles with four loaders and four stages, for grids that the 128 x
// 128 tile would leave under-filled: the smaller the tile, the more
// workgroups share the streaming of W (tall-skinny and decode-like shapes).
// Measured with W streamed from HBM (16 rotating operand sets):
// 1024 x 1024 x 2048 r16 on 64 x 64: 10.3 us (128 x 128: 16.4); 512 x 1024 x
// 1024 r32 on 64 x 32: 6.7 us (64 x 32 without loaders, eight stages: 8.8);
// 64 x 4096 x 4096 r16 on 32 x 32: 18.0 us (19.9).
template <int RP>
using SqL = Cfg<64, 64, 4, 1, RP, 4, 64, 1, 4>;
template <int RP>
using TallL = Cfg<64, 32, 4, 1, RP, 4, 64, 1, 4>;
template <int RP>
using SmallL = Cfg<32, 32, 2, 1, RP, 4, 64, 1, 4>;
// The same two tiles with eight stages in flight, for grids of at most one
// workgroup per CU, where the LDS that a second workgroup would have used
// holds more of the W stream in flight instead (64 x 4096 x 4096 r16 on
// 32 x 32: 15.1-15.3 against 17.6-17.8 us; 128 x 4096 x 4096 on 64 x 32:
// 19.1 against 20.1 us; twelve stages no better than eight).
template <int RP>
using TallL8 = Cfg<64, 32, 4, 1, RP, 8, 64, 1, 4>;
template <int RP>
using SmallL8 = Cfg<32, 32, 2, 1, RP, 8, 64, 1, 4>;

// The built-in choice (lora_fwd's default), from the tile tuner's
// measurements on the benchmark shapes and on rotating operand sets:
//  * ranks 33-128: 256 x 256 keeping T over 8 N tiles (T from a prologue)
//    when its grid has >= 256 workgroups and its rounds are at least 80 %
//    filled with whole tiles (the 16384 x 8192 x 8192 square: r128 1.90 ms
//    against 2.26 on 128 x 256 keeping T; r64 1.70 against 1.81 on 256 x 256
//    recomputing T);
//  * 256 x 256 (r <= 64; its stage loads from four of the eight waves when
//    there is more than one round) when there are >= 256 such tiles and the
//    last round of them is at least 80 % full
//    (q_proj, 512 tiles: 160 vs 202 us; the q_proj backward's dX product,
//    320 tiles: 211 us vs 191 us on 128 x 128);
//  * rank 128 with >= 512 128 x 128 tiles: 128 x 256 tiles keeping T over 8
//    N tiles when that grid has >= 256 workgroups (the 16384 x 8192 x 8192
//    square: 2.73 ms), else 128 x 128 tiles sharing T over 2 N tiles (square:
//    3.27-3.53 ms; over 4 tiles 3.73 ms; unshared 3.87 ms);
//  * at most 256 tiles of 128 x 128: the largest loader tile (128 x 128,
//    64 x 64, 64 x 32, 32 x 32) whose grid has at least 160 workgroups, else
//    32 x 32; 64 x 32 and 32 x 32 with eight stages when their grid is at
//    most 256 workgroups.  128 x 128 keeps the work at 192 tiles (3072 x 1024 x 1024:
//    12.6 vs 16.7 us on 64 x 64) and gives it up at 128 (2048 x 1024 x 4096:
//    40.1 vs 38.4 us);
//  * rank <= 32 past that: 128 x 256 with loaders (8192 x 1024 x 2560 r32:
//    44.4 vs 50.5 us), or 256 x 160 with loaders when its grid fills the
//    rounds of 256 workgroups at least 10 % better (the q_proj backward's dX
//    product: 162 us, against 183.5 on 128 x 256 and 188 on 128 x 128);
//  * else 128 x 128, two stages (two workgroups per CU).
template <int RP>
hipError_t launch_rp(const FwdArgs& a, hipStream_t s) {
  auto grid = [&](int bm, int bn) { return ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
  const int64_t mid_tiles = grid(128, 128);
  if constexpr (RP == 64 || RP == 128) {
    const int64_t tm = (a.M + 255) / 256, tn = (a.N + 255) / 256;
    const int64_t wgs = tm * ((tn + kWideTGroup - 1) / kWideTGroup);
    const int64_t rounds = (wgs + 255) / 256;
    if (wgs >= 256 && tm * tn * 5 >= rounds * 256 * kWideTGroup * 4)
      return launch<BigT<RP>, kWideTGroup>(a, s);
  }
  if constexpr (RP <= 64) {
    const int64_t big_tiles = grid(256, 256);
    const int64_t rounds = (big_tiles + 255) / 256;
    if (big_tiles >= 256 && big_tiles * 5 >= rounds * 256 * 4) {
      // two or more rounds: stage loads from waves 0-3 only
      if (big_tiles > 256) return launch<BigL4<RP>>(a, s);
      return launch<Big<RP>>(a, s);
    }
  }
  if constexpr (RP == 128) {
    if (a.N > 128 && mid_tiles >= 512) {
      // T kept over 8 N tiles of 128 x 256 when that grid still fills a round
      // of 256 workgroups (16384 x 8192 x 8192: 2.73 ms against 3.53 ms on
      // 128 x 128 tiles sharing T over 2; on 8192 x 4096 x 2560, 128
      // workgroups, 442 against 368 us)
      if (grid(128, 256 * kWideTGroup) >= 256) return launch<WideT<RP>, kWideTGroup>(a, s);
      return launch<Mid<RP>, 2>(a, s);
    }
  }
  if constexpr (RP <= 128) {
    if (mid_tiles <= 256) {
      constexpr int64_t kFill = 160;
      if (mid_tiles >= kFill) return launch<Mid3L<RP>>(a, s);
      if constexpr (RP <= 64) {
        if (grid(64, 64) >= kFill) return launch<SqL<RP>>(a, s);
        if (grid(64, 32) >= kFill) {
          if (grid(64, 32) <= 256) return launch<TallL8<RP>>(a, s);
          return launch<TallL<RP>>(a, s);
        }
        if (grid(32, 32) <= 256) return launch<SmallL8<RP>>(a, s);
        return launch<SmallL<RP>>(a, s);
      }
      return launch<Mid3L<RP>>(a, s);
    }
  }
  if constexpr (RP <= 32) {
    // Output elements per workgroup slot of the grid rounded up to whole
    // rounds of 256: 256 x 160 when it fills the rounds clearly better.
    auto fill = [&](int bm, int bn) {
      const int64_t t = grid(bm, bn);
      return (double)a.M * (double)a.N / ((double)((t + 255) / 256) * 256.0 * bm * bn);
    };
    if (fill(256, 160) >= 1.1 * fill(128, 256)) return launch<BigNL<RP>>(a, s);
    return launch<WideL<RP>>(a, s);
  } else {
    return launch<Mid<RP>>(a, s);
  }
}

// ---- selectable tile configurations (the tile tuner's search space).  The
// ids are part of the C ABI (lora_fwd_tile); an id exists only for the ranks
// whose instantiation fits the LDS and the register file.
template <class C, int G>
void tile_fill(TileProps* t) {
  t->bm = C::BM;
  t->bn = C::BN;
  t->waves = C::NW;
  t->stages = C::STAGES;
  t->bk = C::BK;
  t->group = G;
  t->rank_pad = C::RP;
  t->lds_bytes = G > 1 ? C::kLdsG : C::kLds;
  t->k_split = C::KS;
  t->kernel = reinterpret_cast<const void*>(fwd_tiled_bf16_kernel<C, G>);
}

// One dispatch for both uses: with props, describe tile `id`; else launch it.
template <int RP>
hipError_t tile_rp(int id, TileProps* props, const FwdArgs* a, hipStream_t s) {
  switch (id) {
    case kTileTall:
      if constexpr (RP <= 32) {
        if (props) return tile_fill<Tall<RP>, 1>(props), hipSuccess;
        return launch<Tall<RP>>(*a, s);
      }
      break;
    case kTileMid:
      if (props) return tile_fill<Mid<RP>, 1>(props), hipSuccess;
      return launch<Mid<RP>>(*a, s);
    case kTileMidG2:
      if constexpr (RP <= 128) {
        if (props) return tile_fill<Mid<RP>, 2>(props), hipSuccess;
        return launch<Mid<RP>, 2>(*a, s);
      }
      break;
    case kTileMidG4:
      if constexpr (RP <= 128) {
        if (props) return tile_fill<Mid<RP>, 4>(props), hipSuccess;
        return launch<Mid<RP>, 4>(*a, s);
      }
      break;
    case kTileBig:
      if constexpr (RP <= 64) {
        if (props) return tile_fill<Big<RP>, 1>(props), hipSuccess;
        return launch<Big<RP>>(*a, s);
      }
      break;
    case kTileBigG2:
      // Retired: 256 x 256 with T shared over 2 N tiles spilled registers
      // at every rank; the id stays reserved and is never instantiated.
      break;
    case kTileMid3:
      if constexpr (RP <= 128) {
        if (props) return tile_fill<Mid3<RP>, 1>(props), hipSuccess;
        return launch<Mid3<RP>>(*a, s);
      }
      break;
    case kTileMidK2:
      if constexpr (RP <= 64) {
        if (props) return tile_fill<MidK2<RP>, 1>(props), hipSuccess;
        return launch<MidK2<RP>>(*a, s);
      }
      break;
    case kTileMid3L:
      if constexpr (RP <= 128) {
        if (props) return tile_fill<Mid3L<RP>, 1>(props), hipSuccess;
        return launch<Mid3L<RP>>(*a, s);
      }
      break;
    case kTileWideL:
      if constexpr (RP <= 32) {
        if (props) return tile_fill<WideL<RP>, 1>(props), hipSuccess;
        return launch<WideL<RP>>(*a, s);
      }
      break;
    case kTileWideT:
      if constexpr (RP >= 64 && RP <= 128) {
        if (props) return tile_fill<WideT<RP>, kWideTGroup>(props), hipSuccess;
        return launch<WideT<RP>, kWideTGroup>(*a, s);
      }
      break;
    case kTileBigNL:
      if constexpr (RP <= 32) {
        if (props) return tile_fill<BigNL<RP>, 1>(props), hipSuccess;
        return launch<BigNL<RP>>(*a, s);
      }
      break;
    case kTileBigPP:
      if constexpr (RP <= 64) {
        if (props) return tile_fill<BigPP<RP>, 1>(props), hipSuccess;
        return launch<BigPP<RP>>(*a, s);
      }
      break;
    case kTileBigL4:
      if constexpr (RP <= 64) {
        if (props) return tile_fill<BigL4<RP>, 1>(props), hipSuccess;
        return launch<BigL4<RP>>(*a, s);
      }
      break;
    case kTileBigT:
      if constexpr (RP >= 64 && RP <= 128) {
        if (props) return tile_fill<BigT<RP>, kWideTGroup>(props), hipSuccess;
        return launch<BigT<RP>, kWideTGroup>(*a, s);
      }
      break;
    case kTileSqL:
      if constexpr (RP <= 64) {
        if (props) return tile_fill<SqL<RP>, 1>(props), hipSuccess;
        return launch<SqL<RP>>(*a, s);
      }
      break;
    case kTileTallL:
      if constexpr (RP <= 64) {
        if (props) return tile_fill<TallL<RP>, 1>(props), hipSuccess;
        return launch<TallL<RP>>(*a, s);
      }
      break;
    case kTileTallL8:
      if constexpr (RP <= 64) {
        if (props) return tile_fill<TallL8<RP>, 1>(props), hipSuccess;
        return launch<TallL8<RP>>(*a, s);
      }
      break;
    case kTileSmallL8:
      if constexpr (RP <= 64) {
        if (props) return tile_fill<SmallL8<RP>, 1>(props), hipSuccess;
        return launch<SmallL8<RP>>(*a, s);
      }
      break;
    case kTileSmallL:
      if constexpr (RP <= 64) {
        if (props) return tile_fill<SmallL<RP>, 1>(props), hipSuccess;
        return launch<SmallL<RP>>(*a, s);
      }
      break;
    default:
      break;
  }
  return hipErrorInvalidValue;
}

hipError_t tile_dispatch(int id, int64_t r, TileProps* props, const FwdArgs* a, hipStream_t s) {
  switch (pad_rank(r)) {
    case 16: return tile_rp<16>(id, props, a, s);
    case 32: return tile_rp<32>(id, props, a, s);
    case 64: return tile_rp<64>(id, props, a, s);
    case 128: return tile_rp<128>(id, props, a, s);
    default: return tile_rp<256>(id, props, a, s);
  }
}

}  // namespace

hipError_t fwd_tile_props(int id, int64_t r, TileProps* out) {
  return tile_dispatch(id, r, out, nullptr, nullptr);
}

hipError_t launch_fwd_tile_bf16(int id, const FwdArgs& a, hipStream_t s) {
  return tile_dispatch(id, a.r, nullptr, &a, s);
}

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
