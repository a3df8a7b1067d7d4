// kernels.h -- host-side launchers of the gfx950 kernels (C++ linkage, internal
// to liblora.so).  Arguments are validated by the C ABI layer before any of
// these is called; the launchers only pick a tile configuration and launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace lora {

// Raise a kernel's dynamic-LDS limit once per device: the first launch on a
// device sets the attribute, later launches (from any thread) skip the call.
template <class F>
hipError_t ensure_lds(F kern, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = uint64_t(1) << (dev & 63);
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

struct FwdArgs {
  int64_t M, N, K, r;
  const void* X; int64_t ldx;
  const void* W; int64_t ldw;
  const void* A; int64_t lda;
  const void* B; int64_t ldb;
  float scale;
  void* Y; int64_t ldy;
  // Optional (tiled bf16 kernel only): when non-null, s T = s X A^T as
  // rounded to bf16 is also written transposed, tout[j * ldt + m] for j < r
  // and m < ldt (ldt >= M; rows past M are zeros).
  void* tout = nullptr; int64_t ldt = 0;
};

struct MergeArgs {
  int64_t N, K, r;
  const void* W0; int64_t ldw0;
  const void* B; int64_t ldb;
  const void* A; int64_t lda;
  float scale;
  void* Wi; int64_t ldwi;
};

struct BwdArgs {
  int64_t M, N, K, r;
  const void* X; int64_t ldx;
  const void* W; int64_t ldw;
  const void* A; int64_t lda;
  const void* B; int64_t ldb;
  const void* dY; int64_t lddy;
  float scale;
  void* dX; int64_t lddx;   // may be null: no input gradient
  void* dA; int64_t ldda;
  void* dB; int64_t lddb;
};

// Workspace layout of the backward (byte offsets from a 256-B aligned base):
// W^T [K, ldwt], A^T [K, ldat], B^T [r, ldbt], T^T and G^T [r, ldp], all
// bf16, the fp32 partial sums of dA [S][RP][K] and of dB [S][N][RP] over S
// token ranges of tps tokens.
struct BwdPlan {
  int S;
  int64_t tps, ldwt, ldat, ldbt, ldp;
  int64_t off_wt, off_at, off_bt, off_tt, off_gt, off_pa, off_pb, bytes;
};

// Rank padded to the MFMA-friendly size the kernels are instantiated for.
inline int pad_rank(int64_t r) {
  return r <= 16 ? 16 : r <= 32 ? 32 : r <= 64 ? 64 : r <= 128 ? 128 : 256;
}

hipError_t launch_fwd_tiled_bf16(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_tiled_f32(const FwdArgs& a, hipStream_t s);

// Selectable tiled configurations (ids of the C ABI's lora_fwd_tile).
enum TileId { kTileTall = 0, kTileMid = 1, kTileMidG2 = 2, kTileMidG4 = 3, kTileBig = 4,
              kTileBigG2 = 5, kTileMid3 = 6, kTileMidK2 = 7,
              kTileMid3L = 8, kTileWideL = 9,
              kTileSqL = 10, kTileTallL = 11, kTileSmallL = 12, kTileBigNL = 13,
              kTileWideT = 14, kTileBigPP = 15, kTileTallL8 = 16, kTileSmallL8 = 17,
              kTileBigL4 = 18, kTileBigT = 19, kTileCount = 20 };
struct TileProps {
  int bm, bn, waves, stages, bk, group, rank_pad, lds_bytes, k_split;
  const void* kernel;
};
// hipErrorInvalidValue when tile `id` has no instantiation for rank r.
hipError_t fwd_tile_props(int id, int64_t r, TileProps* out);
hipError_t launch_fwd_tile_bf16(int id, const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_decode_bf16(const FwdArgs& a, hipStream_t s);
// Decode forwards with the same M (<= 16) and rank class (r <= 16 or
// 16 < r <= 32), several per launch; each result is bitwise
// launch_fwd_decode_bf16's.  tws (may be null): kDecTpBytes of device memory
// per forward, 16-B aligned; with it T = X A^T is computed once per forward
// in a launch of its own instead of by every workgroup.
constexpr int kDecTpBytes = 8 * 2 * 64 * 16;  // NW waves x rank blocks (<= 2) x 64 lanes x f32x4
hipError_t launch_fwd_decode_bf16_batch(const FwdArgs* a, int count, void* tws, hipStream_t s);
// The library's static scratch for lora_fwd_batch_noalloc: kNoAllocForwards
// workspace slots of kDecTpBytes, one array per device (up to kMaxDevices),
// its device address looked up once per device.
constexpr int kNoAllocForwards = 64;
constexpr int kMaxDevices = 64;
hipError_t decode_scratch(void** out);
hipError_t launch_merge_bf16(const MergeArgs& a, hipStream_t s);
hipError_t launch_merge_f32(const MergeArgs& a, hipStream_t s);
hipError_t launch_merge_bf16_batch(const MergeArgs* a, int count, hipStream_t s);
BwdPlan bwd_plan(int64_t M, int64_t N, int64_t K, int64_t r);
hipError_t launch_bwd_bf16(const BwdArgs& a, void* workspace, hipStream_t s);

// Largest rank the decode kernel is instantiated for.
constexpr int kDecodeMaxRank = 32;

}  // namespace lora
