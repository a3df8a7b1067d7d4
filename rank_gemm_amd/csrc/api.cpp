// api.cpp -- the C ABI of liblora.so (declared in include/lora.h).
//
// Every entry point validates all of its arguments on the host and returns an
// error before touching the HIP runtime; only then does it choose a kernel and
// launch it on the caller's stream.  The library holds no device memory and no
// state besides per-kernel launch attributes.
#include "lora.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "kernels.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Byte range [lo, hi) touched by a row-major matrix of `rows` rows of `cols`
// elements with leading dimension ld.
struct Range {
  uintptr_t lo, hi;
};

Range span(const void* p, int64_t rows, int64_t cols, int64_t ld, int64_t esz) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  if (rows <= 0 || cols <= 0) return {lo, lo};
  return {lo, lo + static_cast<uintptr_t>(((rows - 1) * ld + cols) * esz)};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

int esize(int dtype) { return dtype == LORA_BF16 ? 2 : 4; }

// Checks shared by lora_fwd / lora_fwd_variant.
int check_fwd(int dtype, int64_t M, int64_t N, int64_t K, int64_t r, const void* X, int64_t ldx,
              const void* W, int64_t ldw, const void* A, int64_t lda, const void* B, int64_t ldb,
              void* Y, int64_t ldy) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0 || r < 1) return LORA_ERR_SHAPE;
  if (r > LORA_MAX_RANK) return LORA_ERR_UNSUPPORTED;
  // Kernel index arithmetic is 32-bit per dimension.
  if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return LORA_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return LORA_OK;
  if (Y == nullptr || B == nullptr) return LORA_ERR_NULL;
  if (K > 0 && (X == nullptr || W == nullptr || A == nullptr)) return LORA_ERR_NULL;
  if (ldx < K || ldw < K || lda < K || ldb < r || ldy < N) return LORA_ERR_STRIDE;
  if (ldx > LORA_MAX_LD || ldw > LORA_MAX_LD || lda > LORA_MAX_LD) return LORA_ERR_UNSUPPORTED;
  const int64_t e = esize(dtype);
  // A is addressed as one signed 32-bit byte range of r rows (fp32 above
  // rank 128 can exceed it at the largest lda).
  if (r * lda * e > INT32_MAX) return LORA_ERR_UNSUPPORTED;
  const int64_t kal = dtype == LORA_BF16 ? 8 : 4;
  if (K > 0) {
    if (!aligned16(X) || !aligned16(W) || !aligned16(A)) return LORA_ERR_ALIGN;
    if (K % kal || ldx % kal || ldw % kal || lda % kal) return LORA_ERR_ALIGN;
  }
  if ((reinterpret_cast<uintptr_t>(B) % e) || (reinterpret_cast<uintptr_t>(Y) % e))
    return LORA_ERR_ALIGN;
  const Range y = span(Y, M, N, ldy, e);
  if (overlap(y, span(X, M, K, ldx, e)) || overlap(y, span(W, N, K, ldw, e)) ||
      overlap(y, span(A, r, K, lda, e)) || overlap(y, span(B, N, r, ldb, e)))
    return LORA_ERR_ALIAS;
  return LORA_OK;
}

int pick(int dtype, int64_t M, int64_t r) {
  if (dtype == LORA_BF16 && M <= LORA_DECODE_AUTO_M && r <= lora::kDecodeMaxRank)
    return LORA_VARIANT_DECODE;
  return LORA_VARIANT_TILED;
}

// Host validation shared by lora_merge and lora_merge_batch.
int check_merge(int dtype, int64_t N, int64_t K, int64_t r, const void* W0, int64_t ldw0,
                const void* B, int64_t ldb, const void* A, int64_t lda, void* W_inf,
                int64_t ldwi) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_DTYPE;
  if (N < 0 || K < 0 || r < 1) return LORA_ERR_SHAPE;
  if (r > LORA_MAX_RANK) return LORA_ERR_UNSUPPORTED;
  if (N > INT32_MAX / 2 || K > INT32_MAX / 2) return LORA_ERR_UNSUPPORTED;
  if (N == 0 || K == 0) return LORA_OK;
  if (W0 == nullptr || B == nullptr || A == nullptr || W_inf == nullptr) return LORA_ERR_NULL;
  if (ldw0 < K || ldwi < K || lda < K || ldb < r) return LORA_ERR_STRIDE;
  const int64_t e = esize(dtype);
  const int64_t kal = dtype == LORA_BF16 ? 8 : 4;
  if (!aligned16(W0) || !aligned16(A) || !aligned16(W_inf)) return LORA_ERR_ALIGN;
  if (K % kal || ldw0 % kal || ldwi % kal || lda % kal) return LORA_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(B) % e) return LORA_ERR_ALIGN;
  const Range wi = span(W_inf, N, K, ldwi, e);
  if (overlap(wi, span(W0, N, K, ldw0, e)) || overlap(wi, span(A, r, K, lda, e)) ||
      overlap(wi, span(B, N, r, ldb, e)))
    return LORA_ERR_ALIAS;
  return LORA_OK;
}

// Workspace bytes of the backward, or -1 when the sizes are out of range.
int64_t bwd_ws_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
  if (M < 0 || N < 0 || K < 0 || r < 1 || r > LORA_MAX_RANK) return -1;
  if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return -1;
  // T^T and G^T ([rank padded, M rounded to 64] bf16) are addressed with
  // signed 32-bit byte ranges (r x ldp x 2 < 2^31).
  if ((int64_t)lora::pad_rank(r) * ((M + 63) / 64 * 64) > (int64_t(1) << 30) - 64) return -1;
  return lora::bwd_plan(M, N, K, r).bytes;
}

int check_bwd(int dtype, int64_t M, int64_t N, int64_t K, int64_t r, const void* X, int64_t ldx,
              const void* W, int64_t ldw, const void* A, int64_t lda, const void* B, int64_t ldb,
              const void* dY, int64_t lddy, void* dX, int64_t lddx, void* dA, int64_t ldda,
              void* dB, int64_t lddb, void* ws, int64_t ws_bytes) {
  if (dtype == LORA_F32) return LORA_ERR_UNSUPPORTED;
  if (dtype != LORA_BF16) return LORA_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0 || r < 1) return LORA_ERR_SHAPE;
  const int64_t need = bwd_ws_bytes(M, N, K, r);
  if (need < 0) return LORA_ERR_UNSUPPORTED;
  const bool tok = M > 0, wantx = dX != nullptr && M > 0 && K > 0;
  if ((K > 0 && (dA == nullptr || A == nullptr)) || (N > 0 && (dB == nullptr || B == nullptr)) ||
      (tok && K > 0 && X == nullptr) || (tok && N > 0 && dY == nullptr) ||
      (wantx && N > 0 && W == nullptr))
    return LORA_ERR_NULL;
  // X and dY are only read when there are tokens.
  if ((tok && (ldx < K || lddy < N)) || lda < K || ldda < K || ldb < r || lddb < r ||
      (wantx && (ldw < K || lddx < K)))
    return LORA_ERR_STRIDE;
  if ((tok && (ldx > LORA_MAX_LD || lddy > LORA_MAX_LD)) || lda > LORA_MAX_LD ||
      N > LORA_MAX_LD || (wantx && ldw > LORA_MAX_LD))
    return LORA_ERR_UNSUPPORTED;
  // Leading-dimension alignment matters only for operands with elements.
  if (K % 8 || N % 8 || (tok && K > 0 && ldx % 8) || (tok && N > 0 && lddy % 8) ||
      (K > 0 && (lda % 8 || ldda % 8)) || (wantx && N > 0 && ldw % 8))
    return LORA_ERR_ALIGN;
  if ((K > 0 && (!aligned16(A) || !aligned16(dA) || (tok && !aligned16(X)))) ||
      (tok && N > 0 && !aligned16(dY)) || (wantx && N > 0 && !aligned16(W)) ||
      (N > 0 && ((reinterpret_cast<uintptr_t>(B) & 1) || (reinterpret_cast<uintptr_t>(dB) & 1))) ||
      (wantx && (reinterpret_cast<uintptr_t>(dX) & 1)))
    return LORA_ERR_ALIGN;
  if (need > 0 && (ws == nullptr || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255)))
    return LORA_ERR_WORKSPACE;
  // Outputs and workspace against every input and against each other.
  const Range in[5] = {span(X, M, K, ldx, 2), span(W, wantx ? N : 0, K, ldw, 2),
                       span(A, r, K, lda, 2), span(B, N, r, ldb, 2), span(dY, M, N, lddy, 2)};
  const Range out[4] = {span(dX, wantx ? M : 0, K, lddx, 2), span(dA, r, K, ldda, 2),
                        span(dB, N, r, lddb, 2),
                        {reinterpret_cast<uintptr_t>(ws), reinterpret_cast<uintptr_t>(ws) +
                                                              static_cast<uintptr_t>(need)}};
  for (int i = 0; i < 4; ++i) {
    for (const Range& x : in)
      if (overlap(out[i], x)) return LORA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(out[i], out[j])) return LORA_ERR_ALIAS;
  }
  return LORA_OK;
}

}  // namespace

extern "C" {

int lora_abi_version(void) { return LORA_ABI_VERSION; }

const char* lora_status_str(int s) {
  switch (s) {
    case LORA_OK: return "LORA_OK: validated and launched";
    case LORA_ERR_NULL: return "LORA_ERR_NULL: a required pointer is NULL";
    case LORA_ERR_SHAPE: return "LORA_ERR_SHAPE: negative size or rank < 1";
    case LORA_ERR_STRIDE: return "LORA_ERR_STRIDE: leading dimension smaller than the row";
    case LORA_ERR_ALIGN: return "LORA_ERR_ALIGN: pointer, K or leading-dimension alignment";
    case LORA_ERR_DTYPE: return "LORA_ERR_DTYPE: unknown element type";
    case LORA_ERR_ALIAS: return "LORA_ERR_ALIAS: output overlaps an input";
    case LORA_ERR_UNSUPPORTED: return "LORA_ERR_UNSUPPORTED: rank or variant not supported";
    case LORA_ERR_HIP: return "LORA_ERR_HIP: HIP launch error";
    case LORA_ERR_WORKSPACE: return "LORA_ERR_WORKSPACE: workspace missing, too small or misaligned";
    case LORA_ERR_SCRATCH:
      return "LORA_ERR_SCRATCH: more forwards than the no-allocation scratch holds (64)";
    default: return "unknown lora_status";
  }
}

int lora_fwd_pick(int dtype, int64_t M, int64_t N, int64_t K, int64_t r) {
  (void)N;
  (void)K;
  return pick(dtype, M, r);
}

int lora_fwd_variant(int variant, int dtype, int64_t M, int64_t N, int64_t K, int64_t r,
                     const void* X, int64_t ldx, const void* W, int64_t ldw, const void* A,
                     int64_t lda, const void* B, int64_t ldb, float scale, void* Y, int64_t ldy,
                     void* stream) {
  if (variant != LORA_VARIANT_AUTO && variant != LORA_VARIANT_TILED &&
      variant != LORA_VARIANT_DECODE)
    return LORA_ERR_UNSUPPORTED;
  const int st = check_fwd(dtype, M, N, K, r, X, ldx, W, ldw, A, lda, B, ldb, Y, ldy);
  if (st != LORA_OK) return st;
  if (variant == LORA_VARIANT_DECODE &&
      (dtype != LORA_BF16 || M > LORA_DECODE_MAX_M || r > lora::kDecodeMaxRank))
    return LORA_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return LORA_OK;
  if (variant == LORA_VARIANT_AUTO) variant = pick(dtype, M, r);
  const lora::FwdArgs a{M, N, K, r, X, ldx, W, ldw, A, lda, B, ldb, scale, Y, ldy};
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == LORA_F32)
    e = lora::launch_fwd_tiled_f32(a, s);
  else if (variant == LORA_VARIANT_DECODE)
    e = lora::launch_fwd_decode_bf16(a, s);
  else
    e = lora::launch_fwd_tiled_bf16(a, s);
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

int lora_fwd(int dtype, int64_t M, int64_t N, int64_t K, int64_t r, const void* X, int64_t ldx,
             const void* W, int64_t ldw, const void* A, int64_t lda, const void* B, int64_t ldb,
             float scale, void* Y, int64_t ldy, void* stream) {
  return lora_fwd_variant(LORA_VARIANT_AUTO, dtype, M, N, K, r, X, ldx, W, ldw, A, lda, B, ldb,
                          scale, Y, ldy, stream);
}

int lora_merge(int dtype, int64_t N, int64_t K, int64_t r, const void* W0, int64_t ldw0,
               const void* B, int64_t ldb, const void* A, int64_t lda, float scale, void* W_inf,
               int64_t ldwi, void* stream) {
  const int st = check_merge(dtype, N, K, r, W0, ldw0, B, ldb, A, lda, W_inf, ldwi);
  if (st != LORA_OK || N == 0 || K == 0) return st;
  const lora::MergeArgs a{N, K, r, W0, ldw0, B, ldb, A, lda, scale, W_inf, ldwi};
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t err =
      dtype == LORA_BF16 ? lora::launch_merge_bf16(a, s) : lora::launch_merge_f32(a, s);
  return err == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

int lora_merge_inplace(int dtype, int64_t N, int64_t K, int64_t r, void* W, int64_t ldw,
                       const void* B, int64_t ldb, const void* A, int64_t lda, float scale,
                       void* stream) {
  // lora_merge's checks with W as both the input and the output.
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_DTYPE;
  if (N < 0 || K < 0 || r < 1) return LORA_ERR_SHAPE;
  if (r > LORA_MAX_RANK) return LORA_ERR_UNSUPPORTED;
  if (N > INT32_MAX / 2 || K > INT32_MAX / 2) return LORA_ERR_UNSUPPORTED;
  if (N == 0 || K == 0) return LORA_OK;
  if (W == nullptr || B == nullptr || A == nullptr) return LORA_ERR_NULL;
  if (ldw < K || lda < K || ldb < r) return LORA_ERR_STRIDE;
  const int64_t e = esize(dtype);
  const int64_t kal = dtype == LORA_BF16 ? 8 : 4;
  if (!aligned16(W) || !aligned16(A)) return LORA_ERR_ALIGN;
  if (K % kal || ldw % kal || lda % kal) return LORA_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(B) % e) return LORA_ERR_ALIGN;
  const Range w = span(W, N, K, ldw, e);
  if (overlap(w, span(A, r, K, lda, e)) || overlap(w, span(B, N, r, ldb, e)))
    return LORA_ERR_ALIAS;
  const lora::MergeArgs a{N, K, r, W, ldw, B, ldb, A, lda, scale, W, ldw};
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t err =
      dtype == LORA_BF16 ? lora::launch_merge_bf16(a, s) : lora::launch_merge_f32(a, s);
  return err == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

int lora_merge_batch(int dtype, int count, const lora_merge_desc* descs, void* stream) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_DTYPE;
  if (count < 0) return LORA_ERR_SHAPE;
  if (count == 0) return LORA_OK;
  if (descs == nullptr) return LORA_ERR_NULL;
  const int64_t e = esize(dtype);
  std::vector<lora::MergeArgs> work;
  work.reserve(count);
  for (int i = 0; i < count; ++i) {
    const lora_merge_desc& d = descs[i];
    const int st = check_merge(dtype, d.N, d.K, d.r, d.W0, d.ldw0, d.B, d.ldb, d.A, d.lda,
                               d.W_inf, d.ldwi);
    if (st != LORA_OK) return st;
    if (d.N == 0 || d.K == 0) continue;
    work.push_back({d.N, d.K, d.r, d.W0, d.ldw0, d.B, d.ldb, d.A, d.lda, d.scale, d.W_inf,
                    d.ldwi});
  }
  // Every output against every other target's inputs and output.
  for (size_t i = 0; i < work.size(); ++i) {
    const lora::MergeArgs& a = work[i];
    const Range wi = span(a.Wi, a.N, a.K, a.ldwi, e);
    for (size_t j = 0; j < work.size(); ++j) {
      if (j == i) continue;
      const lora::MergeArgs& b = work[j];
      if (overlap(wi, span(b.W0, b.N, b.K, b.ldw0, e)) ||
          overlap(wi, span(b.A, b.r, b.K, b.lda, e)) ||
          overlap(wi, span(b.B, b.N, b.r, b.ldb, e)) ||
          overlap(wi, span(b.Wi, b.N, b.K, b.ldwi, e)))
        return LORA_ERR_ALIAS;
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = hipSuccess;
  if (dtype == LORA_BF16) {
    err = lora::launch_merge_bf16_batch(work.data(), (int)work.size(), s);
  } else {
    for (const lora::MergeArgs& a : work)
      if ((err = lora::launch_merge_f32(a, s)) != hipSuccess) break;
  }
  return err == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

int64_t lora_bwd_workspace_size(int dtype, int64_t M, int64_t N, int64_t K, int64_t r) {
  if (dtype != LORA_BF16) return -1;
  return bwd_ws_bytes(M, N, K, r);
}

int lora_bwd(int dtype, int64_t M, int64_t N, int64_t K, int64_t r, const void* X, int64_t ldx,
             const void* W, int64_t ldw, const void* A, int64_t lda, const void* B, int64_t ldb,
             const void* dY, int64_t lddy, float scale, void* dX, int64_t lddx, void* dA,
             int64_t ldda, void* dB, int64_t lddb, void* workspace, int64_t workspace_bytes,
             void* stream) {
  const int st = check_bwd(dtype, M, N, K, r, X, ldx, W, ldw, A, lda, B, ldb, dY, lddy, dX, lddx,
                           dA, ldda, dB, lddb, workspace, workspace_bytes);
  if (st != LORA_OK) return st;
  const lora::BwdArgs a{M, N, K, r, X, ldx, W, ldw, A, lda, B, ldb, dY, lddy, scale,
                        (M > 0 && K > 0) ? dX : nullptr, lddx, dA, ldda, dB, lddb};
  const hipError_t e = lora::launch_bwd_bf16(a, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

int lora_tile_get_info(int tile, int64_t r, lora_tile_info* out) {
  if (out == nullptr) return LORA_ERR_NULL;
  if (r < 1) return LORA_ERR_SHAPE;
  if (r > LORA_MAX_RANK || tile < 0 || tile >= LORA_TILE_COUNT) return LORA_ERR_UNSUPPORTED;
  lora::TileProps t{};
  if (lora::fwd_tile_props(tile, r, &t) != hipSuccess) return LORA_ERR_UNSUPPORTED;
  *out = lora_tile_info{tile, t.bm, t.bn, t.waves, t.stages, t.bk, t.group, t.rank_pad,
                        t.lds_bytes, t.k_split};
  return LORA_OK;
}

int lora_tile_get_usage(int tile, int64_t r, lora_tile_usage* out) {
  if (out == nullptr) return LORA_ERR_NULL;
  if (r < 1) return LORA_ERR_SHAPE;
  if (r > LORA_MAX_RANK || tile < 0 || tile >= LORA_TILE_COUNT) return LORA_ERR_UNSUPPORTED;
  lora::TileProps t{};
  if (lora::fwd_tile_props(tile, r, &t) != hipSuccess) return LORA_ERR_UNSUPPORTED;
  hipFuncAttributes attr{};
  if (hipFuncGetAttributes(&attr, t.kernel) != hipSuccess) return LORA_ERR_HIP;
  // Occupancy at the kernel's LDS needs the raised dynamic-LDS limit.
  if (hipFuncSetAttribute(t.kernel, hipFuncAttributeMaxDynamicSharedMemorySize, t.lds_bytes) !=
      hipSuccess)
    return LORA_ERR_HIP;
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, t.kernel, t.waves * 64,
                                                   t.lds_bytes) != hipSuccess)
    return LORA_ERR_HIP;
  *out = lora_tile_usage{attr.numRegs, (int32_t)attr.localSizeBytes, blocks};
  return LORA_OK;
}

int lora_get_device_limits(lora_device_limits* out) {
  if (out == nullptr) return LORA_ERR_NULL;
  int dev = 0;
  hipDeviceProp_t p{};
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&p, dev) != hipSuccess)
    return LORA_ERR_HIP;
  *out = lora_device_limits{p.multiProcessorCount, (int32_t)p.sharedMemPerBlock,
                            (int32_t)p.maxSharedMemoryPerMultiProcessor, p.regsPerBlock,
                            p.maxThreadsPerBlock, p.warpSize};
  return LORA_OK;
}

int lora_fwd_tile(int tile, int dtype, int64_t M, int64_t N, int64_t K, int64_t r,
                  const void* X, int64_t ldx, const void* W, int64_t ldw, const void* A,
                  int64_t lda, const void* B, int64_t ldb, float scale, void* Y, int64_t ldy,
                  void* stream) {
  const int st = check_fwd(dtype, M, N, K, r, X, ldx, W, ldw, A, lda, B, ldb, Y, ldy);
  if (st != LORA_OK) return st;
  lora::TileProps t{};
  if (dtype != LORA_BF16 || tile < 0 || tile >= LORA_TILE_COUNT ||
      lora::fwd_tile_props(tile, r, &t) != hipSuccess)
    return LORA_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return LORA_OK;
  const lora::FwdArgs a{M, N, K, r, X, ldx, W, ldw, A, lda, B, ldb, scale, Y, ldy};
  const hipError_t e = lora::launch_fwd_tile_bf16(tile, a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

int64_t lora_fwd_batch_workspace_size(int count) {
  return count < 0 ? -1 : (int64_t)count * lora::kDecTpBytes;
}

}  // extern "C"

namespace {

// Validation of a batch of forward descriptors (into work, which holds at
// least count entries; returns the number of non-empty forwards through n).
int check_fwd_batch(int dtype, int count, const lora_fwd_desc* descs, const void* workspace,
                    int64_t ws_bytes, lora::FwdArgs* work, size_t* n) {
  const int64_t e = esize(dtype);
  size_t k = 0;
  for (int i = 0; i < count; ++i) {
    const lora_fwd_desc& d = descs[i];
    const int st = check_fwd(dtype, d.M, d.N, d.K, d.r, d.X, d.ldx, d.W, d.ldw, d.A, d.lda, d.B,
                             d.ldb, d.Y, d.ldy);
    if (st != LORA_OK) return st;
    if (d.M == 0 || d.N == 0) continue;
    work[k++] = lora::FwdArgs{d.M, d.N, d.K, d.r, d.X, d.ldx, d.W, d.ldw, d.A, d.lda, d.B, d.ldb,
                              d.scale, d.Y, d.ldy};
  }
  // Every output against every other forward's inputs and output, and the
  // workspace against every operand.
  const Range wsr{reinterpret_cast<uintptr_t>(workspace),
                  reinterpret_cast<uintptr_t>(workspace) + (workspace ? (uintptr_t)ws_bytes : 0)};
  for (size_t i = 0; i < k; ++i) {
    const lora::FwdArgs& a = work[i];
    const Range y = span(a.Y, a.M, a.N, a.ldy, e);
    if (overlap(wsr, y) || overlap(wsr, span(a.X, a.M, a.K, a.ldx, e)) ||
        overlap(wsr, span(a.W, a.N, a.K, a.ldw, e)) || overlap(wsr, span(a.A, a.r, a.K, a.lda, e)) ||
        overlap(wsr, span(a.B, a.N, a.r, a.ldb, e)))
      return LORA_ERR_ALIAS;
    for (size_t j = 0; j < k; ++j) {
      if (j == i) continue;
      const lora::FwdArgs& b = work[j];
      if (overlap(y, span(b.X, b.M, b.K, b.ldx, e)) || overlap(y, span(b.W, b.N, b.K, b.ldw, e)) ||
          overlap(y, span(b.A, b.r, b.K, b.lda, e)) || overlap(y, span(b.B, b.N, b.r, b.ldb, e)) ||
          overlap(y, span(b.Y, b.M, b.N, b.ldy, e)))
        return LORA_ERR_ALIAS;
    }
  }
  *n = k;
  return LORA_OK;
}

// Launches of a validated batch (work[0, n)); workspace as lora_fwd_batch's.
int run_fwd_batch(int dtype, const lora::FwdArgs* work, size_t n, void* workspace,
                  hipStream_t s) {
  hipError_t err = hipSuccess;
  size_t i = 0;
  while (i < n && err == hipSuccess) {
    const lora::FwdArgs& a = work[i];
    if (pick(dtype, a.M, a.r) == LORA_VARIANT_DECODE) {
      size_t j = i + 1;
      while (j < n && pick(dtype, work[j].M, work[j].r) == LORA_VARIANT_DECODE &&
             work[j].M == a.M && (work[j].r <= 16) == (a.r <= 16))
        ++j;
      unsigned char* tws =
          workspace ? static_cast<unsigned char*>(workspace) + i * lora::kDecTpBytes : nullptr;
      err = lora::launch_fwd_decode_bf16_batch(&work[i], (int)(j - i), tws, s);
      i = j;
    } else {
      err = dtype == LORA_F32 ? lora::launch_fwd_tiled_f32(a, s) : lora::launch_fwd_tiled_bf16(a, s);
      ++i;
    }
  }
  return err == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

}  // namespace

extern "C" {

int lora_fwd_batch(int dtype, int count, const lora_fwd_desc* descs, void* workspace,
                   int64_t workspace_bytes, void* stream) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_DTYPE;
  if (count < 0) return LORA_ERR_SHAPE;
  if (count == 0) return LORA_OK;
  if (descs == nullptr) return LORA_ERR_NULL;
  if (workspace != nullptr && (workspace_bytes < (int64_t)count * lora::kDecTpBytes ||
                               (reinterpret_cast<uintptr_t>(workspace) & 255)))
    return LORA_ERR_WORKSPACE;
  std::vector<lora::FwdArgs> work(count);
  size_t n = 0;
  const int st = check_fwd_batch(dtype, count, descs, workspace,
                                 workspace ? (int64_t)count * lora::kDecTpBytes : 0, work.data(),
                                 &n);
  if (st != LORA_OK) return st;
  return run_fwd_batch(dtype, work.data(), n, workspace, static_cast<hipStream_t>(stream));
}

int lora_fwd_batch_noalloc(int dtype, int count, const lora_fwd_desc* descs, void* stream) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_DTYPE;
  if (count < 0) return LORA_ERR_SHAPE;
  if (count == 0) return LORA_OK;
  if (count > LORA_NOALLOC_MAX_FORWARDS) return LORA_ERR_SCRATCH;
  if (descs == nullptr) return LORA_ERR_NULL;
  static_assert(LORA_NOALLOC_MAX_FORWARDS == lora::kNoAllocForwards, "scratch size");
  lora::FwdArgs work[LORA_NOALLOC_MAX_FORWARDS];  // host stack: nothing is allocated
  size_t n = 0;
  const int st = check_fwd_batch(dtype, count, descs, nullptr, 0, work, &n);
  if (st != LORA_OK) return st;
  if (n == 0) return LORA_OK;
  void* scratch = nullptr;
  if (lora::decode_scratch(&scratch) != hipSuccess) return LORA_ERR_HIP;
  return run_fwd_batch(dtype, work, n, scratch, static_cast<hipStream_t>(stream));
}

}  // extern "C"
