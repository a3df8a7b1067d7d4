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
// columns = n, v_mfma_f32_16x16x32_bf16, fp32 accumulate); with a permuted k
// order (run_col below) each of the four accumulators of a lane holds four
// consecutive columns of one row.  The wave writes them to its own fp32 P
// tile in LDS and reads them back line-wise: lane l takes 8 columns of row
// l / 8 (and l / 8 + 8), so W0 is loaded and W_inf stored as whole 128-B
// lines (8 rows x 128 B per instruction), which a half-line layout (16 rows
// x 64 B) streams measurably slower.  Each lane adds its W0 values in fp32,
// rounds once to bf16 and stores.  The A strip is staged in LDS once per
// workgroup, transposed so that the rank is contiguous, and its fragments
// stay in registers for every row block; the first row blocks' loads are
// issued before it, and later row blocks are double-buffered.
//
// W0 is never written; nothing is accumulated across workgroups, so repeated
// merges of the same inputs are bitwise identical.  Every element of W0 is
// read once and its W_inf element written afterwards by the same lane, so
// the same code also merges in place (W_inf == W0), which lora_merge_inplace
// offers as the merge/unmerge path that the pristine merge replaces.
#include "common.h"
#include "kernels.h"

namespace lora {
namespace {

constexpr int kMergeThreads = 256;
constexpr int kStrip = 256;  // columns per workgroup (64 per wave)
constexpr int kPS = 64 + 4;  // row stride (floats) of a wave's P tile in LDS
constexpr int kMergeBatch = 24;  // targets per batched launch (kernel-argument space)

template <int RP>
struct Mrg {
  static constexpr int RB32 = RP / 32;          // rank chunks of 32
  static constexpr int kAS = RP + 8;            // transposed-A row stride (elements, even)
  static constexpr int kLdsA = kStrip * kAS * 2;  // transposed A strip
  static constexpr int kLds = kLdsA + 4 * 16 * kPS * 4;  // + one fp32 P tile per wave
  static constexpr int kU = 2;                  // row blocks per load group (two groups in flight)
};

// Column (within the wave's 64) of element e (0..15) of lane group lg's run:
// elements 0..7 are columns 8 lg .. 8 lg + 7, elements 8..15 are columns
// 32 + 8 lg .. +7, so each 16-B load or store of the four lane groups of a
// row covers 64 contiguous bytes.
__device__ __forceinline__ int run_col(int lg, int e) { return (e >> 3) * 32 + 8 * lg + (e & 7); }

// One workgroup's work: strip (wg % strips) of the output, row blocks
// [(wg / strips) * nblk_per_wg, +nblk_per_wg).  Shared by the one-target and
// the batched kernels.
template <int RP>
__device__ __forceinline__ void merge_bf16_tile(
    unsigned char* smem, int wg, int N, int K, int r, const uint16_t* W0,
    int64_t ldw0, const uint16_t* __restrict__ B, int64_t ldb, const uint16_t* __restrict__ A,
    int64_t lda, float scale, uint16_t* Wi, int64_t ldwi, int strips,
    int nblk_per_wg, int b_vec) {
  using C = Mrg<RP>;
  constexpr int RB32 = C::RB32, U = C::kU;
  uint32_t* at32 = reinterpret_cast<uint32_t*>(smem);  // at[k][j] as j-pairs, k < 256
  const uint16_t* at = reinterpret_cast<const uint16_t*>(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 15, lg = lane >> 4;
  const int strip = wg % strips;
  const int ngrp = wg / strips;
  const int k0 = strip * kStrip;
  const int nb_begin = ngrp * nblk_per_wg;
  const int nblocks = (N + 15) / 16;
  const int nb_end = min(nblocks, nb_begin + nblk_per_wg);
  const u32x4 z = {0, 0, 0, 0};
  const int kw = wave * 64;
  // This wave's P tile in LDS (fp32, 16 rows x 64 columns, padded rows).
  float* pl = reinterpret_cast<float*>(smem + C::kLdsA) + wave * 16 * kPS;

  // W0 and W_inf move in whole 128-B lines: lane l takes row l / 8 (+ 8 for
  // the second half) of the row block and columns 8 (l % 8) .. + 7 of the
  // wave's 64, so one load or store instruction covers 8 rows x 128 B.
  const int srow = lane >> 3;
  const int gcol = k0 + kw + 8 * (lane & 7);
  const bool cin = gcol < K;

  auto load = [&](int nb, u32x4 (&w)[U][2], u32x4 (&bf)[U][RB32]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool bin = (nb + u) < nb_end;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int n = (nb + u) * 16 + srow + 8 * h;
        // Streamed once: non-temporal, so the lines do not displace B and
        // the A strip in the caches (3.02 -> 2.92 ms for the 36 x 7 pass).
        w[u][h] = (bin && n < N && cin)
                      ? __builtin_nontemporal_load(
                            reinterpret_cast<const u32x4*>(W0 + (int64_t)n * ldw0 + gcol))
                      : z;
      }
      // B fragment (MFMA operand): row (nb + u) * 16 + l % 16.
      const int n = (nb + u) * 16 + lrow;
      const bool nin = bin && n < N;
      const int64_t row = (int64_t)(nin ? n : 0);
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

  // The first row blocks' loads go out before the A strip is staged, so the
  // two latencies overlap.
  u32x4 wa[U][2], ba[U][RB32], wb[U][2], bb[U][RB32];
  int nb = nb_begin;
  if (nb < nb_end) load(nb, wa, ba);

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
  u32x4 af[4][RB32];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int kl = kw + run_col(lrow >> 2, 4 * kb + (lrow & 3));
#pragma unroll
    for (int kk = 0; kk < RB32; ++kk)
      af[kb][kk] = *reinterpret_cast<const u32x4*>(at + kl * C::kAS + kk * 32 + lg * 8);
  }

  auto compute_store = [&](int nb, const u32x4 (&w)[U][2], const u32x4 (&bf)[U][RB32]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // The MFMAs read operands from all 64 lanes, so they run wave-uniform;
      // rows past N only skip their stores.
      if ((nb + u) >= nb_end) continue;
      f32x4 p[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        p[kb] = zero4();
#pragma unroll
        for (int kk = 0; kk < RB32; ++kk) p[kb] = mfma16x16x32(af[kb][kk], bf[u][kk], p[kb]);
      }
      // p[kb] holds row l % 16, columns run_col(l / 16, 4 kb .. 4 kb + 3):
      // four consecutive columns.  Through LDS to the line-wise layout.
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        *reinterpret_cast<f32x4*>(pl + lrow * kPS + run_col(lg, 4 * kb)) = p[kb];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float* src = pl + (srow + 8 * h) * kPS + 8 * (lane & 7);
        const f32x4 q0 = *reinterpret_cast<const f32x4*>(src);
        const f32x4 q1 = *reinterpret_cast<const f32x4*>(src + 4);
        const float pv[8] = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
        u32x4 o;
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const uint32_t wv = w[u][h][q2];
          const float lo = __builtin_bit_cast(float, wv << 16) + scale * pv[2 * q2];
          const float hi = __builtin_bit_cast(float, wv & 0xFFFF0000u) + scale * pv[2 * q2 + 1];
          o[q2] = pack_bf2(lo, hi);
        }
        const int n = (nb + u) * 16 + srow + 8 * h;
        if (n < N && cin)
          __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(Wi + (int64_t)n * ldwi + gcol));
      }
    }
  };

  // 3. Row blocks, U at a time, the loads of the next group in flight while
  //    the current group is combined and stored.
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
__global__ __launch_bounds__(kMergeThreads) void merge_bf16_kernel(
    int N, int K, int r, const uint16_t* W0, int64_t ldw0,
    const uint16_t* __restrict__ B, int64_t ldb, const uint16_t* __restrict__ A, int64_t lda,
    float scale, uint16_t* Wi, int64_t ldwi, int strips, int nblk_per_wg,
    int b_vec) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  merge_bf16_tile<RP>(smem, blockIdx.x, N, K, r, W0, ldw0, B, ldb, A, lda, scale, Wi, ldwi,
                      strips, nblk_per_wg, b_vec);
}

// Batched merge: up to kMergeBatch targets per launch, their descriptors in
// the kernel arguments (no device memory).  Workgroups [first[t], first[t+1])
// belong to target t; a workgroup finds its target by a uniform binary search.
struct MergeDesc {
  const uint16_t* W0;
  const uint16_t* B;
  const uint16_t* A;
  uint16_t* Wi;
  int64_t ldw0, ldb, lda, ldwi;
  int N, K, r, strips, per, b_vec;
  float scale;
};

struct MergeBatch {
  int count;
  int first[kMergeBatch + 1];
  MergeDesc d[kMergeBatch];
};

template <int RP>
__global__ __launch_bounds__(kMergeThreads) void merge_bf16_batch_kernel(const MergeBatch args) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int b = blockIdx.x;
  int lo = 0, hi = args.count - 1;  // last t with first[t] <= b
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (args.first[mid] <= b) lo = mid; else hi = mid - 1;
  }
  const MergeDesc& d = args.d[lo];
  merge_bf16_tile<RP>(smem, b - args.first[lo], d.N, d.K, d.r, d.W0, d.ldw0, d.B, d.ldb, d.A,
                      d.lda, d.scale, d.Wi, d.ldwi, d.strips, d.per, d.b_vec);
}

// Grid of one target: 256-column strips x groups of row blocks.  About 512
// workgroups (2 per CU) for a lone target, each streaming at least two load
// groups of row blocks so the A-strip staging is amortised.
struct MergeGrid {
  int strips, per, groups;
};

template <int RP>
MergeGrid merge_grid(int64_t N, int64_t K, int target_wgs) {
  using C = Mrg<RP>;
  MergeGrid g;
  g.strips = (int)((K + kStrip - 1) / kStrip);
  const int nblocks = (int)((N + 15) / 16);
  int groups = (target_wgs + g.strips - 1) / g.strips;
  if (groups > nblocks) groups = nblocks;
  if (groups < 1) groups = 1;
  int per = (nblocks + groups - 1) / groups;
  if (per < 2 * C::kU) per = nblocks < 2 * C::kU ? nblocks : 2 * C::kU;
  g.per = per;
  g.groups = (nblocks + per - 1) / per;
  return g;
}

int b_vec_of(const void* B, int64_t ldb) {
  return ((reinterpret_cast<uintptr_t>(B) & 15) == 0) && (ldb % 8 == 0);
}

template <int RP>
hipError_t launch_m(const MergeArgs& a, hipStream_t s) {
  using C = Mrg<RP>;
  auto kern = merge_bf16_kernel<RP>;
  static std::atomic<uint64_t> attr_done{0};
  if (hipError_t e = ensure_lds(kern, C::kLds, attr_done); e != hipSuccess) return e;
  const MergeGrid g = merge_grid<RP>(a.N, a.K, 512);
  hipLaunchKernelGGL(kern, dim3(g.strips * g.groups), dim3(kMergeThreads), C::kLds, s, (int)a.N,
                     (int)a.K, (int)a.r, static_cast<const uint16_t*>(a.W0), a.ldw0,
                     static_cast<const uint16_t*>(a.B), a.ldb, static_cast<const uint16_t*>(a.A),
                     a.lda, a.scale, static_cast<uint16_t*>(a.Wi), a.ldwi, g.strips, g.per,
                     b_vec_of(a.B, a.ldb));
  return hipGetLastError();
}

// Targets [i0, i1) of a batch, all padded to rank RP, in one launch.  Each
// target gets row-block groups of 4 load groups (128 rows), so small and
// large targets share the launch in proportion to their size.
template <int RP>
hipError_t launch_mb(const MergeArgs* a, int i0, int i1, hipStream_t s) {
  using C = Mrg<RP>;
  auto kern = merge_bf16_batch_kernel<RP>;
  static std::atomic<uint64_t> attr_done{0};
  if (hipError_t e = ensure_lds(kern, C::kLds, attr_done); e != hipSuccess) return e;
  MergeBatch mb{};
  mb.count = i1 - i0;
  int wgs = 0;
  for (int i = i0; i < i1; ++i) {
    const MergeArgs& t = a[i];
    const int strips = (int)((t.K + kStrip - 1) / kStrip);
    const int nblocks = (int)((t.N + 15) / 16);
    const int per = 8 * C::kU;
    const int groups = (nblocks + per - 1) / per;
    MergeDesc& d = mb.d[i - i0];
    d.W0 = static_cast<const uint16_t*>(t.W0);
    d.B = static_cast<const uint16_t*>(t.B);
    d.A = static_cast<const uint16_t*>(t.A);
    d.Wi = static_cast<uint16_t*>(t.Wi);
    d.ldw0 = t.ldw0; d.ldb = t.ldb; d.lda = t.lda; d.ldwi = t.ldwi;
    d.N = (int)t.N; d.K = (int)t.K; d.r = (int)t.r;
    d.strips = strips; d.per = per; d.b_vec = b_vec_of(t.B, t.ldb);
    d.scale = t.scale;
    mb.first[i - i0] = wgs;
    wgs += strips * groups;
  }
  mb.first[i1 - i0] = wgs;
  if (wgs == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(wgs), dim3(kMergeThreads), C::kLds, s, mb);
  return hipGetLastError();
}

// fp32 merge: plain VALU, 4 consecutive columns per thread, fp32 FMA chain
// over the rank.
__global__ __launch_bounds__(256) void merge_f32_kernel(
    int N, int K, int r, const float* W0, int64_t ldw0, const float* __restrict__ B,
    int64_t ldb, const float* __restrict__ A, int64_t lda, float scale, float* Wi,
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

// Batch: runs of consecutive targets with the same padded rank, at most
// kMergeBatch per launch.
hipError_t launch_merge_bf16_batch(const MergeArgs* a, int count, hipStream_t s) {
  int i = 0;
  while (i < count) {
    const int rp = pad_rank(a[i].r) < 32 ? 32 : pad_rank(a[i].r);
    int j = i + 1;
    while (j < count && j - i < kMergeBatch &&
           (pad_rank(a[j].r) < 32 ? 32 : pad_rank(a[j].r)) == rp)
      ++j;
    hipError_t e;
    switch (rp) {
      case 32: e = launch_mb<32>(a, i, j, s); break;
      case 64: e = launch_mb<64>(a, i, j, s); break;
      case 128: e = launch_mb<128>(a, i, j, s); break;
      default: e = launch_mb<256>(a, i, j, s); break;
    }
    if (e != hipSuccess) return e;
    i = j;
  }
  return hipSuccess;
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
