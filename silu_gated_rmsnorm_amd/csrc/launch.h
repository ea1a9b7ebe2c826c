// Host-side launchers of the gfx950 kernels (no argument checking here:
// the C-ABI layer validates every argument before calling these).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace grn {

// Rows per dw chunk.  The backward adds the dw contributions of chunk
// [c*R, (c+1)*R) into one FP32 partial, one workgroup per chunk; R, and
// therefore the bits of dw, depend only on the number of rows.  One size
// serves all row counts: smaller chunks for small problems (32 or 64 rows
// below 196,608 rows) measured slower on MI355X, because the extra partials
// and hand-offs cost more than the added parallelism gains.
#ifndef GRN_CHUNK_ROWS
#define GRN_CHUNK_ROWS 128
#endif
constexpr int kChunkRows = GRN_CHUNK_ROWS;

constexpr int chunk_rows_for(int64_t /*rows*/) { return kChunkRows; }

// Workspace of the backward, in this order:
//   counters  uint32[kCounterWords]  arrival counters (zero between calls)
//   partial   float[nchunks][128]     one dw partial per chunk
//   gpart     float[ngroups][128]     one dw partial per group of chunks
// The counter region holds, as 32-bit words:
//   [0, ngroups)                 one arrival counter per group (ngroups is at
//                                most 4096: ceil(sqrt(nchunks)) <= 4096 for
//                                nchunks <= 2^24, i.e. rows < 2^31)
//   [kNondetAccum, +slots*128)   the FP32 accumulators of the
//                                non-deterministic dw, kNondetSlots of them
//   [kMaxGroups]                 the overall counter
constexpr int kMaxGroups = 8191;
constexpr int kCounterWords = kMaxGroups + 1;
#ifndef GRN_NONDET_SLOTS
#define GRN_NONDET_SLOTS 16
#endif
constexpr int kNondetSlots = GRN_NONDET_SLOTS;
constexpr int kNondetAccum = 4096;
static_assert(kNondetSlots >= 1 && kNondetAccum + kNondetSlots * 128 <= kMaxGroups,
              "the non-deterministic accumulators must fit the counter region");
constexpr size_t kCounterBytes = (size_t)kCounterWords * sizeof(uint32_t);

struct BwdLayout {
  int64_t chunk_rows = 0;
  int64_t nchunks = 0;
  int64_t group_size = 1;
  int64_t ngroups = 0;
  size_t partial_off = 0;
  size_t gpart_off = 0;
  size_t bytes = 0;
};

BwdLayout bwd_layout(int64_t rows);

// Row strides of the activations, in elements (each a multiple of 8, i.e.
// 16-byte rows, and at most kMaxStride).  Packed rows have stride 128.
struct RowStrides {
  int64_t x = 128, g = 128, y = 128, dy = 128, dx = 128, dg = 128;
};
constexpr int64_t kMaxStride = int64_t{1} << 24;

hipError_t launch_fwd(const void* x, const void* g, const void* w, void* y,
                      const RowStrides& st, int64_t rows, float eps, int max_wg,
                      hipStream_t s);

hipError_t launch_bwd(const void* x, const void* g, const void* w,
                      const void* dy, void* dx, void* dg, void* dw,
                      int dw_fp32, int deterministic, void* workspace,
                      const RowStrides& st, int64_t rows, float eps, int max_wg,
                      hipStream_t s);

hipError_t launch_counters_zero(void* workspace, hipStream_t s);

}  // namespace grn
