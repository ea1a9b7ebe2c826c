// Host-side launchers of the gfx950 kernels (no argument checking here:
// the C-ABI layer validates every argument before calling these).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace grn {

// Rows per dw chunk.  The backward adds the dw contributions of chunk c, a
// fixed set of R rows (chunk_blocks() in kernels.hip says which), into one
// FP32 partial, one workgroup per chunk.  R depends only on the row size;
// the bits of dw depend only on rows, D and the type.  R = 128 rows
// serves every row count (smaller chunks for small problems, 32 or 64 rows,
// measured slower on MI355X: the extra partials and hand-offs cost more
// than the added parallelism gains).  Rows of 128 bytes (D = 64 in a 16-bit
// type) take 256-row chunks, so that a chunk's fixed cost is spread over as
// many bytes (measured at 7684x48: 54 -> 48 us; 256-byte FP32 rows of
// D = 64 were faster with 128-row chunks).
#ifndef GRN_CHUNK_ROWS
#define GRN_CHUNK_ROWS 128
#endif
constexpr int kChunkRows = GRN_CHUNK_ROWS;

constexpr int chunk_rows_for(int32_t row_bytes) {
  return row_bytes <= 128 ? 2 * kChunkRows : kChunkRows;
}

// Workspace of the backward, in this order:
//   counters  uint32[kCounterWords]  arrival counters (zero between calls)
//   partial   float[nchunks][D]       one dw partial per chunk
//   gpart     float[ngroups][D]       one dw partial per group of chunks
// The counter region holds:
//   words [0, kGroupCounterWords)  one arrival counter per group, group g
//                                  at word g * counter_stride (ngroups is at
//                                  most 4096: ceil(sqrt(nchunks)) <= 4096
//                                  for nchunks <= 2^24, i.e. rows < 2^31)
//   bytes [kNondetAccumByte, +nondet_slots(D)*8*D)
//                                  the FP64 accumulators of the
//                                  non-deterministic dw
//   word  kClaimCounter            the tail-claim counter of the
//                                  deterministic backward (claim_chunks)
//   word  kOverallCounter          the overall counter (the last word)
#ifndef GRN_COUNTER_WORDS
#define GRN_COUNTER_WORDS 8192
#endif
#ifndef GRN_MAX_COUNTER_STRIDE
#define GRN_MAX_COUNTER_STRIDE 64
#endif
constexpr int kCounterWords = GRN_COUNTER_WORDS;
constexpr int kOverallCounter = kCounterWords - 1;
constexpr int kGroupCounterWords = kCounterWords / 2;
constexpr int kMaxCounterStride = GRN_MAX_COUNTER_STRIDE;  // 64: counters 256 B apart
static_assert(kGroupCounterWords >= 4096, "one counter word per group at least");
#ifndef GRN_NONDET_SLOTS
#define GRN_NONDET_SLOTS 16
#endif
constexpr int kNondetAccumByte = kGroupCounterWords * 4;
// Accumulators of D doubles each that fit below the overall counter (16 for
// D = 64, 15 for D = 128, 7 for D = 256).
constexpr int nondet_slots(int D) {
  return (kOverallCounter * 4 - kNondetAccumByte) / (8 * D) < GRN_NONDET_SLOTS
             ? (kOverallCounter * 4 - kNondetAccumByte) / (8 * D)
             : GRN_NONDET_SLOTS;
}
static_assert(nondet_slots(256) >= 1, "the non-deterministic accumulators fit");
constexpr size_t kCounterBytes = (size_t)kCounterWords * sizeof(uint32_t);
constexpr int kClaimCounter = kOverallCounter - 1;
static_assert(kNondetAccumByte + nondet_slots(64) * 8 * 64 <= kClaimCounter * 4 &&
                  kNondetAccumByte + nondet_slots(128) * 8 * 128 <= kClaimCounter * 4 &&
                  kNondetAccumByte + nondet_slots(256) * 8 * 256 <= kClaimCounter * 4,
              "the claim counter lies past the non-deterministic accumulators");

// Chunks the deterministic backward hands out at run time (0: none).  The
// grid's first nchunks - K items take chunk = item index; then come 2K
// claim items, each taking the next of the last K chunks from an atomic
// counter, or nothing once they are gone.  Workgroups are dealt to the 8
// XCDs in index order, and the XCDs stream at rates a few per cent apart
// (which one is slowest varies from run to run), so with static chunks
// they finished 4-5 us apart at 7684x48 and 8-14 us at 32768x48; claim
// items on an XCD that is ahead start sooner and take more of the tail.
// Which workgroup runs a chunk does not change dw's bits.  Measured
// (backward alone, BF16 D = 128, same process, alternating; static vs
// K = 512): 7684x48 81.9 vs 81.0 us, 12296x48 126.8 vs 125.7, 16384x32
// 112.8 vs 111.8, 32768x48 331.0 vs 327.6, 65536x48 669.4 vs 664.0,
// 262144x48 2,746 vs 2,731; K = 256 gained less and K = 1024 lost up to
// 2.7 %.  Grids of 1,024 to 2,047 chunks claim 256 (3534x48 43.6 vs 43.2
// us, 5000x48 56.7 vs 56.3, BF16 D = 64 at 7684x48 rows 45.2 vs 44.9);
// smaller grids, which run as about one round of workgroups, claim none.
#ifndef GRN_BWD_CLAIM
#define GRN_BWD_CLAIM 512
#endif
__host__ __device__ constexpr int64_t claim_chunks(bool det, int64_t nchunks) {
  return (!det || GRN_BWD_CLAIM <= 0)                  ? 0
         : nchunks >= 4 * (int64_t)GRN_BWD_CLAIM      ? GRN_BWD_CLAIM
         : nchunks >= 2 * (int64_t)GRN_BWD_CLAIM      ? GRN_BWD_CLAIM / 2
                                                      : 0;
}

struct BwdLayout {
  int64_t chunk_rows = 0;
  int64_t nchunks = 0;
  int64_t group_size = 1;
  int64_t ngroups = 0;
  int64_t counter_stride = 1;  // words between group counters (a power of 2)
  size_t partial_off = 0;
  size_t gpart_off = 0;
  size_t bytes = 0;
};

// Exact layout for rows of D values of `esize` bytes.  esize = 0 gives the
// largest layout over the element types (the size to allocate when the type
// is not known).
BwdLayout bwd_layout(int64_t rows, int32_t D, int32_t esize);

// Row strides of the activations, in elements (each keeps rows 16-byte
// aligned: a multiple of 8 for 16-bit types, of 4 for FP32; at most
// kMaxStride).  Packed rows have stride D.
struct RowStrides {
  int64_t x = 0, g = 0, y = 0, dy = 0, dx = 0, dg = 0;
};
constexpr int64_t kMaxStride = int64_t{1} << 24;

// dtype: 0 BF16, 1 FP16, 2 FP32 (GRN_DTYPE_*); D: 64, 128 or 256.
hipError_t launch_fwd(const void* x, const void* g, const void* w, void* y,
                      const RowStrides& st, int64_t rows, int32_t D, int32_t dtype,
                      float eps, int max_wg, hipStream_t s);

hipError_t launch_bwd(const void* x, const void* g, const void* w,
                      const void* dy, void* dx, void* dg, void* dw,
                      int dw_fp32, int deterministic, void* workspace,
                      const RowStrides& st, int64_t rows, int32_t D, int32_t dtype,
                      float eps, int max_wg, hipStream_t s, void* fused_y = nullptr);

// Whether the checkpointed step runs its recomputed forward inside the
// backward's launch (launch_bwd with fused_y = y): for the deterministic dw
// and tensors below 32 MiB, whose backward runs as one round of workgroups.
// Measured (checkpointed step, same process, alternating; separate vs
// fused): 1031x48 32.0 vs 27.9 us, 1500x48 42.8 vs 37.0, 2000x48 48.9 vs
// 47.6, 2600x48 63.1 vs 59.7; from 41 MiB up the forward's tiles, run at the
// backward's occupancy, made the step slower (3534x48 83.6 vs 84.9,
// 7684x48 160.3 vs 175.0).  Every output bit is the same either way.
bool ckpt_fuses_forward(int64_t rows, int32_t D, int32_t dtype, int deterministic);

hipError_t launch_counters_zero(void* workspace, hipStream_t s);

}  // namespace grn
