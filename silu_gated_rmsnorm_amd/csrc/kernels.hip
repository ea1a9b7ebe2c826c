// gfx950 kernels of the SiLU-gated RMSNorm training forward and backward.
//
// Operator (flashinfer PR #8701, "perf(cake_rmsnorm_silu_gate_train):
// L2-prefetching extra-long forward on SM107": PR description and commit
// 10c6017 message), per row i of D = 128 values, with w shared by all rows:
//   r = 1/sqrt(mean(x^2) + eps),  n = x r,  s = silu(g) = g sigmoid(g)
//   y = n w s
//   dn = dy w s,  c = mean(dn n),  dx = r (dn - n c)
//   dg = dy w n silu'(g),  silu'(g) = sigmoid(g) + s (1 - sigmoid(g))
//   dw = sum over rows of dy n s
//
// All three kernels stream HBM and do a few FP32 operations per byte, below
// the ridge point of the vector ALUs, so they are written for memory
// throughput: 16-byte coalesced accesses, several independent row groups in
// flight per wave before any arithmetic, row sums in DPP, no LDS on the
// per-row path, no MFMA (there is no contraction to feed it).  The
// backward's per-element arithmetic (two transcendentals and ~20 other
// operations) is not negligible next to its memory time, so it is kept
// lean: shared products, wave-uniform (scalar) addressing, and no per-lane
// predicates except in the one tile that holds the ragged end of the rows.
#include "common.h"
#include "launch.h"

#include <mutex>

// Tiling knobs (compile-time; results other than dw do not depend on them,
// and dw depends only on GRN_CHUNK_ROWS, fixed in launch.h).
#ifndef GRN_FWD_U
#define GRN_FWD_U 2          // row groups of 4 per wave tile in the forward
#endif
#ifndef GRN_BWD_U
#define GRN_BWD_U 4          // row groups of 4 per wave step in the backward
#endif
#ifndef GRN_FWD_WG_PER_CU
#define GRN_FWD_WG_PER_CU -1 // forward grid cap per CU; 0 = occupancy limit,
                             // -1 = one workgroup per 4 tiles (no cap)
#endif
#ifndef GRN_BWD_WAVES
#define GRN_BWD_WAVES 4      // waves per backward workgroup
#endif
#ifndef GRN_BWD_MIN_WAVES
#define GRN_BWD_MIN_WAVES 0  // >0: ask for at least this many waves per SIMD
#endif
#ifndef GRN_BWD_PREFETCH
#define GRN_BWD_PREFETCH 1   // steps of loads kept in flight ahead of the one
#endif                       // being computed (0 = none), deterministic dw
#ifndef GRN_BWD_ND_PREFETCH
#define GRN_BWD_ND_PREFETCH 0  // the same for the non-deterministic dw kernel
#endif
#ifndef GRN_SUM_BATCH
#define GRN_SUM_BATCH 8      // partial rows per thread per round trip in the dw tree
#endif
#ifndef GRN_BWD_WG_PER_CU
#define GRN_BWD_WG_PER_CU -1 // backward grid cap per CU; 0 = occupancy limit,
#endif                       // -1 = one workgroup per chunk (no cap)
// Cache policy of the streamed accesses: bit masks selecting non-temporal
// loads/stores per tensor (forward loads: x=1, g=2; forward stores: y=1;
// backward loads: x=1, g=2, dy=4; backward stores: dx=1, dg=2).
#ifndef GRN_FWD_NTL
#define GRN_FWD_NTL 1
#endif
#ifndef GRN_FWD_NTS
#define GRN_FWD_NTS 1
#endif
#ifndef GRN_BWD_NTL
#define GRN_BWD_NTL 7
#endif
#ifndef GRN_BWD_NTS
#define GRN_BWD_NTS 3
#endif

namespace grn {

template <bool kNT, typename T>
__device__ __forceinline__ T ld_stream(const T* p) {
  if constexpr (kNT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool kNT, typename T>
__device__ __forceinline__ void st_stream(T* p, T v) {
  if constexpr (kNT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// Wave index as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

// Row pitch of a tensor in 16-byte units (a packed row of 128 BF16 is 16).
// Lane l of a wave touches row 4u + l/16 of its tile, bytes
// [16(l%16), 16(l%16)+16) of that row: offset (4u + l/16) * pitch + l%16.
__device__ __forceinline__ uint32_t lane_offset(int lane, int u, uint32_t pitch) {
  return (uint32_t)(kRowsPerAccess * u + lane / kLanesPerRow) * pitch +
         (uint32_t)(lane & (kLanesPerRow - 1));
}

// --------------------------------------------------------------------------
// Forward.  A wave tile is U groups of 4 consecutive rows (4U rows).  Lane l
// owns columns [8(l%16), 8(l%16)+8) of tile row 4u + l/16.  With packed rows
// (pitch 16) a tile is U contiguous KiB per tensor and lane l reads offset
// l + 64u.  Waves walk the tiles with a grid stride.

struct FwdPitch {
  uint32_t x, g, y;  // row pitches in 16-byte units
};

template <int U, bool kFull>
__device__ __forceinline__ void fwd_tile(const u32x4* __restrict__ xb,
                                         const u32x4* __restrict__ gb,
                                         u32x4* __restrict__ yb, FwdPitch pt,
                                         const float (&wf)[kVec], float eps,
                                         int lane, int nvalid) {
  const int sub = lane / kLanesPerRow;
  u32x4 xv[U], gv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (kFull || kRowsPerAccess * u + sub < nvalid) {
      xv[u] = ld_stream<(GRN_FWD_NTL & 1) != 0>(xb + lane_offset(lane, u, pt.x));
      gv[u] = ld_stream<(GRN_FWD_NTL & 2) != 0>(gb + lane_offset(lane, u, pt.g));
    } else {
      xv[u] = u32x4{0, 0, 0, 0};
      gv[u] = u32x4{0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float xf[kVec], gf[kVec];
    unpack_bf16x8(xv[u], xf);
    unpack_bf16x8(gv[u], gf);
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < kVec; ++e) ss = fmaf(xf[e], xf[e], ss);
    ss = row16_sum(ss);
    const float r = rsqrt_fast(ss * (1.0f / kD) + eps);
    float yf[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      const float s = gf[e] * sigmoid_fast(gf[e]);
      yf[e] = (xf[e] * r) * wf[e] * s;
    }
    if (kFull || kRowsPerAccess * u + sub < nvalid)
      st_stream<(GRN_FWD_NTS & 1) != 0>(yb + lane_offset(lane, u, pt.y),
                                         pack_bf16x8(yf));
  }
}

template <int U>
__global__ void __launch_bounds__(kBlock)
fwd_kernel(const u32x4* __restrict__ x, const u32x4* __restrict__ g,
           const u32x4* __restrict__ w, u32x4* __restrict__ y, FwdPitch pt,
           int64_t rows, float eps, int64_t ntiles) {
  constexpr int kTileRows = kRowsPerAccess * U;
  const int lane = threadIdx.x & (kWave - 1);
  float wf[kVec];
  unpack_bf16x8(w[lane & (kLanesPerRow - 1)], wf);

  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  for (int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + wave_index();
       t < ntiles; t += nwaves) {
    const int64_t row0 = t * kTileRows;
    const u32x4* xb = x + row0 * pt.x;
    const u32x4* gb = g + row0 * pt.g;
    u32x4* yb = y + row0 * pt.y;
    if (row0 + kTileRows <= rows) {
      fwd_tile<U, true>(xb, gb, yb, pt, wf, eps, lane, kTileRows);
    } else {
      fwd_tile<U, false>(xb, gb, yb, pt, wf, eps, lane, (int)(rows - row0));
    }
  }
}

// --------------------------------------------------------------------------
// Backward, dx/dg and one partial dw per chunk of R rows (R depends only on
// the number of rows: chunk_rows_for()).
//
// The dw order is fixed by the chunk alone: within chunk c, wave v of the
// workgroup takes step `it` on rows c*R + (it*4 + v)*4U + 4u + l/16, and
// lane l adds its 8 columns' contributions in (it, u) order into FP32
// registers.  At the end of the chunk the 16 (wave, row-in-group)
// accumulators of each column are added in index order through LDS and
// written as partial[c].  Which workgroup runs a chunk, and when, changes
// nothing, so dw does not depend on the grid or on timing.

// Raw BF16 registers of one wave step (U groups of 4 rows, three inputs).
template <int U>
struct BwdRaw {
  u32x4 x[U], g[U], dy[U];
};

struct BwdPitch {
  uint32_t x, g, dy, dx, dg;  // row pitches in 16-byte units
};

template <int U, bool kFull>
__device__ __forceinline__ void bwd_load(BwdRaw<U>& r,
                                         const u32x4* __restrict__ xb,
                                         const u32x4* __restrict__ gb,
                                         const u32x4* __restrict__ dyb,
                                         BwdPitch pt, int lane, int nvalid) {
  const int sub = lane / kLanesPerRow;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (kFull || kRowsPerAccess * u + sub < nvalid) {
      r.x[u] = ld_stream<(GRN_BWD_NTL & 1) != 0>(xb + lane_offset(lane, u, pt.x));
      r.g[u] = ld_stream<(GRN_BWD_NTL & 2) != 0>(gb + lane_offset(lane, u, pt.g));
      r.dy[u] = ld_stream<(GRN_BWD_NTL & 4) != 0>(dyb + lane_offset(lane, u, pt.dy));
    } else {
      r.x[u] = u32x4{0, 0, 0, 0};
      r.g[u] = u32x4{0, 0, 0, 0};
      r.dy[u] = u32x4{0, 0, 0, 0};
    }
  }
}

template <int U, bool kFull>
__device__ __forceinline__ void bwd_compute(const BwdRaw<U>& r,
                                            u32x4* __restrict__ dxb,
                                            u32x4* __restrict__ dgb, BwdPitch pt,
                                            const float (&wf)[kVec], float eps,
                                            int lane, int nvalid,
                                            float (&acc)[kVec]) {
  const int sub = lane / kLanesPerRow;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float xf[kVec], gf[kVec], dyf[kVec];
    unpack_bf16x8(r.x[u], xf);
    unpack_bf16x8(r.g[u], gf);
    unpack_bf16x8(r.dy[u], dyf);
    // Before the row sums: dn = dy w s, t = dy w silu'(g), q = dy s.  Only
    // x, dn, t and q stay live across the two row reductions.
    float dn[kVec], tg[kVec], q[kVec];
    float ss = 0.0f, sd = 0.0f;
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      const float sig = sigmoid_fast(gf[e]);
      const float s = gf[e] * sig;
      const float ds = fmaf(s, 1.0f - sig, sig);  // silu'(g) = sig + s (1 - sig)
      const float dyw = dyf[e] * wf[e];
      dn[e] = dyw * s;
      tg[e] = dyw * ds;
      q[e] = dyf[e] * s;
      ss = fmaf(xf[e], xf[e], ss);
      sd = fmaf(dn[e], xf[e], sd);
    }
    ss = row16_sum(ss);
    sd = row16_sum(sd);
    const float rs = rsqrt_fast(ss * (1.0f / kD) + eps);
    const float cr = rs * sd * (1.0f / kD);  // c = mean(dn n) = r mean(dn x)
    float dxf[kVec], dgf[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      const float n = xf[e] * rs;
      dxf[e] = rs * fmaf(-n, cr, dn[e]);
      dgf[e] = tg[e] * n;
      q[e] *= n;  // dw contribution dy n s
    }
    if (kFull || kRowsPerAccess * u + sub < nvalid) {
      st_stream<(GRN_BWD_NTS & 1) != 0>(dxb + lane_offset(lane, u, pt.dx),
                                         pack_bf16x8(dxf));
      st_stream<(GRN_BWD_NTS & 2) != 0>(dgb + lane_offset(lane, u, pt.dg),
                                         pack_bf16x8(dgf));
#pragma unroll
      for (int e = 0; e < kVec; ++e) acc[e] += q[e];
    }
  }
}

// One chunk for one workgroup: wave `wave` takes steps it = 0..kIters-1 on
// rows row0(it) = chunk0 + (it*4 + wave)*4U.  The loads of step it+1 are
// issued before the arithmetic of step it, so every wave keeps a step of
// reads in flight while it computes.
template <int U, int kWaves, int R, int kPrefetch, bool kFull>
__device__ __forceinline__ void bwd_chunk(const u32x4* __restrict__ x,
                                          const u32x4* __restrict__ g,
                                          const u32x4* __restrict__ dy,
                                          u32x4* __restrict__ dx,
                                          u32x4* __restrict__ dg, BwdPitch pt,
                                          const float (&wf)[kVec], float eps,
                                          int64_t chunk0, int64_t rows,
                                          int wave, int lane,
                                          float (&acc)[kVec]) {
  constexpr int kStepRows = kRowsPerAccess * U;
  constexpr int kIters = R / (kWaves * kStepRows);
  auto row_of = [&](int it) {
    return chunk0 + (int64_t)(it * kWaves + wave) * kStepRows;
  };
  auto nvalid_of = [&](int it) {
    const int64_t left = rows - row_of(it);
    return (int)(left < 0 ? 0 : (left > kStepRows ? kStepRows : left));
  };
  // A ring of kDepth register buffers: step it+kDepth-1 is loaded while
  // step it is computed.
  constexpr int kDepth = kPrefetch + 1;
  BwdRaw<U> buf[kDepth];
  auto load = [&](BwdRaw<U>& b, int it) {
    const int64_t row0 = row_of(it);
    bwd_load<U, kFull>(b, x + row0 * pt.x, g + row0 * pt.g, dy + row0 * pt.dy, pt,
                       lane, nvalid_of(it));
  };
#pragma unroll
  for (int k = 0; k < kDepth - 1; ++k) {
    if (k < kIters) load(buf[k], k);
  }
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int ahead = it + kDepth - 1;
    if (ahead < kIters) load(buf[ahead % kDepth], ahead);
    const int64_t row0 = row_of(it);
    bwd_compute<U, kFull>(buf[it % kDepth], dx + row0 * pt.dx, dg + row0 * pt.dg, pt,
                          wf, eps, lane, nvalid_of(it), acc);
  }
}

// Cross-workgroup hand-off of the dw partials.  A partial is written with
// device-scope (write-through) stores, each wave waits until its stores are
// complete, and only then does one thread bump the arrival counter; the
// workgroup that sees itself last reads the partials with device-scope loads
// (which do not hit stale lines in the per-XCD L2).  No cache-wide write-back
// or invalidation is needed, so the streaming of dx and dg is not disturbed.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A raw buffer over `count` rows of 128 FP32 values; loads past the end of
// the buffer return zero (hardware range check).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const float* p,
                                                            int64_t count) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), 0,
                                           (int)(count * kD * sizeof(float)),
                                           0x00020000);
}

// 16-byte device-scope load (cache policy sc1: served coherently for the
// whole device, not from a stale line of this XCD's L2).
constexpr int kCpolDevice = 16;

__device__ __forceinline__ float4 load_coherent4(__amdgpu_buffer_rsrc_t rsrc,
                                                 int byte_off) {
  return __builtin_bit_cast(
      float4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, byte_off, 0, kCpolDevice));
}

// Wait until every memory access this wave issued is complete.
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Column sums of a [count, 128] FP32 array, in a fixed order.  Thread t of
// the workgroup owns columns 4*(t%32) .. 4*(t%32)+3 and row slot t/32: it
// adds rows slot, slot+S, slot+2S, ... (S = threads/32 slots) in increasing
// order (16-byte loads issued GRN_SUM_BATCH rows at a time, so one round
// trip covers up to 8 * GRN_SUM_BATCH rows; rows past the end read as zero).
// The S slots of each column are then added in slot order.  The result is
// valid in threads 0..127 (one column each).
template <int kThreads>
__device__ __forceinline__ float column_sum_fixed(const float* __restrict__ src,
                                                  int64_t count,
                                                  float* __restrict__ lds) {
  constexpr int kSlots = kThreads / 32;
  constexpr int kBatch = GRN_SUM_BATCH;
  const int t = threadIdx.x;
  const int quad = t & 31;
  const int slot = t / 32;
  const __amdgpu_buffer_rsrc_t rsrc = rows_rsrc(src, count);
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t r0 = slot; r0 < count; r0 += kSlots * kBatch) {
    float4 v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int64_t r = r0 + (int64_t)kSlots * k;  // past the end: reads zero
      v[k] = load_coherent4(rsrc, (int)((r * kD + 4 * quad) * sizeof(float)));
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      a.x += v[k].x; a.y += v[k].y; a.z += v[k].z; a.w += v[k].w;
    }
  }
  // lds[slot][column]
  lds[slot * kD + 4 * quad + 0] = a.x;
  lds[slot * kD + 4 * quad + 1] = a.y;
  lds[slot * kD + 4 * quad + 2] = a.z;
  lds[slot * kD + 4 * quad + 3] = a.w;
  __syncthreads();
  float res = 0.0f;
  if (t < kD) {
#pragma unroll
    for (int k = 0; k < kSlots; ++k) res += lds[k * kD + t];
  }
  __syncthreads();
  return res;
}

__device__ __forceinline__ void store_dw(void* dw, int dw_fp32, int col, float v) {
  if (dw_fp32) {
    static_cast<float*>(dw)[col] = v;
  } else {
    static_cast<uint16_t*>(dw)[col] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu);
  }
}

// The backward: dx and dg row by row, and dw through a fixed-order tree.
//
// dw tree (every level in a fixed order, so the bits depend only on rows):
//  1. chunk c (R rows, one workgroup): each lane adds its rows in
//     step order, then the 16 lane/wave accumulators of a column are added
//     in index order -> partial[c];
//  2. group g (chunks [g*G, g*G + G), G = ceil(sqrt(nchunks))): the
//     workgroup that finishes last among the group's chunks (an arrival
//     counter tells it) adds their partials in chunk order -> gpart[g];
//  3. the workgroup that completes the last group adds gpart in group order
//     -> dw, rounded once to BF16 unless dw_fp32.
// Arrival counters live at the front of the workspace; each is returned to
// zero by the workgroup that consumes it, so a zero-filled workspace stays
// ready for the next call.
#ifndef GRN_BWD_REDUCERS
#define GRN_BWD_REDUCERS 1
#endif
constexpr bool kReducers = GRN_BWD_REDUCERS != 0;

#if GRN_BWD_MIN_WAVES > 0
#define GRN_BWD_OCCUPANCY __attribute__((amdgpu_waves_per_eu(GRN_BWD_MIN_WAVES)))
#else
#define GRN_BWD_OCCUPANCY
#endif

template <int U, int kWaves, int R, int kPrefetch, bool kDet>
__global__ void __launch_bounds__(kWaves * kWave) GRN_BWD_OCCUPANCY
bwd_kernel(const u32x4* __restrict__ x, const u32x4* __restrict__ g,
           const u32x4* __restrict__ w, const u32x4* __restrict__ dy,
           u32x4* __restrict__ dx, u32x4* __restrict__ dg, BwdPitch pt,
           float* __restrict__ partial, float* __restrict__ gpart,
           uint32_t* __restrict__ counters, void* __restrict__ dw,
           int dw_fp32, int64_t rows, float eps, int64_t nchunks,
           int64_t group_size, int64_t ngroups) {
  constexpr int kThreads = kWaves * kWave;
  constexpr int kStepRows = kRowsPerAccess * U;                 // per wave
  static_assert(R % (kWaves * kStepRows) == 0,
                "a chunk must be a whole number of workgroup steps");
  constexpr int kContrib = kWaves * kRowsPerAccess;
  __shared__ float red[kContrib][kD];
  __shared__ int last_in_group, last_overall;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_index();
  const int col = lane & (kLanesPerRow - 1);
  const int sub = lane / kLanesPerRow;
  const int t = threadIdx.x;
  float wf[kVec];
  unpack_bf16x8(w[col], wf);

  // Level 1 for chunk c: dx and dg of its rows, and the column sums of its
  // dw terms (each lane's rows in step order, then the 16 lane/wave
  // accumulators of a column in index order); valid in threads 0..127.
  auto chunk_partial = [&](int64_t c) {
    float acc[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) acc[e] = 0.0f;
    const int64_t chunk0 = c * R;
    if (chunk0 + R <= rows) {
      bwd_chunk<U, kWaves, R, kPrefetch, true>(x, g, dy, dx, dg, pt, wf, eps, chunk0, rows,
                                               wave, lane, acc);
    } else {
      bwd_chunk<U, kWaves, R, kPrefetch, false>(x, g, dy, dx, dg, pt, wf, eps, chunk0, rows,
                                                wave, lane, acc);
    }
    const int contrib = wave * kRowsPerAccess + sub;
#pragma unroll
    for (int e = 0; e < kVec; ++e) red[contrib][col * kVec + e] = acc[e];
    __syncthreads();
    float v = 0.0f;
    if (t < kD) {
#pragma unroll
      for (int k = 0; k < kContrib; ++k) v += red[k][t];
    }
    return v;
  };

  // Work items: chunks [0, nchunks), then (deterministic dw) one reducer
  // item per group, which arrives at its group's counter like a chunk but
  // carries no partial.  Being last in the grid, reducers usually arrive
  // after all of their group's chunks, so most group sums run once the
  // streaming is done instead of amid it.
  const int64_t nwork = nchunks + (kDet && kReducers ? ngroups : 0);
  for (int64_t item = blockIdx.x; item < nwork; item += gridDim.x) {
    int64_t grp = item - nchunks;  // for a reducer item
    if (item < nchunks) {
      const int64_t c = item;
      const float v = chunk_partial(c);
      if constexpr (!kDet) {
        // Non-deterministic dw: the chunk sum is added with float atomics
        // into one of kNondetSlots FP32 accumulators (chunk c uses slot
        // c mod slots, so concurrent chunks hit different addresses); the
        // last chunk to arrive adds the slots and returns them to zero.  The
        // order of the atomic adds, and so the bits of dw, vary per run.
        float* accum = reinterpret_cast<float*>(counters) + kNondetAccum;
        if (t < kD) {
          __hip_atomic_fetch_add(accum + (c % kNondetSlots) * kD + t, v, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
          wait_memory();
        }
        __syncthreads();
        if (t == 0)
          last_overall = __hip_atomic_fetch_add(&counters[kMaxGroups], 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT) ==
                         (uint32_t)(nchunks - 1);
        __syncthreads();
        if (last_overall) {
          if (t < kD) {
            float slot[kNondetSlots];
#pragma unroll
            for (int k = 0; k < kNondetSlots; ++k)
              slot[k] = __hip_atomic_load(accum + k * kD + t, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
            float total = 0.0f;
#pragma unroll
            for (int k = 0; k < kNondetSlots; ++k) total += slot[k];
            store_dw(dw, dw_fp32, t, total);
#pragma unroll
            for (int k = 0; k < kNondetSlots; ++k)
              __hip_atomic_store(accum + k * kD + t, 0.0f, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
          }
          if (t == 0)
            __hip_atomic_store(&counters[kMaxGroups], 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        continue;
      }
      if (t < kD) {
        store_coherent(partial + c * kD + t, v);
        wait_memory();  // the partial is complete before anyone arrives
      }
      __syncthreads();
      grp = c / group_size;
    }

    // Level 2: the last arrival at group grp's counter (its chunks, plus its
    // reducer item) sums the group.
    const int64_t gbeg = grp * group_size;
    const int64_t gcnt = (nchunks - gbeg) < group_size ? (nchunks - gbeg) : group_size;
    const uint32_t arrivals = (uint32_t)gcnt + (kReducers ? 1u : 0u);
    if (t == 0)
      last_in_group = __hip_atomic_fetch_add(&counters[grp], 1u, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT) == arrivals - 1u;
    __syncthreads();
    if (last_in_group) {
      float* lds = &red[0][0];
      const float gsum = column_sum_fixed<kThreads>(partial + gbeg * kD, gcnt, lds);
      if (t < kD) store_coherent(gpart + grp * kD + t, gsum);
      if (t == 0)
        __hip_atomic_store(&counters[grp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      wait_memory();
      __syncthreads();
      // Level 3: the workgroup that completes the last group sums them all.
      if (t == 0)
        last_overall = __hip_atomic_fetch_add(&counters[kMaxGroups], 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT) ==
                       (uint32_t)(ngroups - 1);
      __syncthreads();
      if (last_overall) {
        const float total = column_sum_fixed<kThreads>(gpart, ngroups, lds);
        if (t < kD) store_dw(dw, dw_fp32, t, total);
        if (t == 0)
          __hip_atomic_store(&counters[kMaxGroups], 0u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
  }
}

// rows = 0: dw is an empty sum.
__global__ void __launch_bounds__(kD)
dw_zero_kernel(void* __restrict__ dw, int dw_fp32) {
  store_dw(dw, dw_fp32, threadIdx.x, 0.0f);
}

// Zero the arrival counters at the front of a workspace.
__global__ void __launch_bounds__(kBlock)
counters_zero_kernel(uint32_t* __restrict__ counters) {
  for (int k = threadIdx.x; k < kCounterWords; k += kBlock) counters[k] = 0u;
}

// --------------------------------------------------------------------------
// Launchers.


namespace {

constexpr int kFwdU = GRN_FWD_U;
// The two backward kernels.  Each has its own prefetch depth: the one that
// measured fastest for it (the register budgets of the two differ).
constexpr auto kBwdDet = bwd_kernel<GRN_BWD_U, GRN_BWD_WAVES, kChunkRows, GRN_BWD_PREFETCH, true>;
constexpr auto kBwdNondet =
    bwd_kernel<GRN_BWD_U, GRN_BWD_WAVES, kChunkRows, GRN_BWD_ND_PREFETCH, false>;
constexpr int kBwdWaves = GRN_BWD_WAVES;

struct DeviceInfo {
  int cus = 0;
  int fwd_blocks_per_cu = 0;
  int bwd_blocks_per_cu = 0;
};

// Per-device launch facts, filled once per device (immutable afterwards).
DeviceInfo device_info() {
  static DeviceInfo cache[64];
  static bool ready[64] = {};
  static std::mutex fill_mutex;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!__atomic_load_n(&ready[dev], __ATOMIC_ACQUIRE)) {
    std::lock_guard<std::mutex> lock(fill_mutex);
    if (__atomic_load_n(&ready[dev], __ATOMIC_ACQUIRE)) return cache[dev];
    DeviceInfo info;
    if (hipDeviceGetAttribute(&info.cus, hipDeviceAttributeMultiprocessorCount,
                              dev) != hipSuccess || info.cus <= 0)
      info.cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &info.fwd_blocks_per_cu, fwd_kernel<kFwdU>, kBlock, 0) !=
            hipSuccess || info.fwd_blocks_per_cu <= 0)
      info.fwd_blocks_per_cu = 4;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &info.bwd_blocks_per_cu, kBwdDet,
            kBwdWaves * kWave, 0) !=
            hipSuccess || info.bwd_blocks_per_cu <= 0)
      info.bwd_blocks_per_cu = 4;
    if (GRN_FWD_WG_PER_CU > 0 && GRN_FWD_WG_PER_CU < info.fwd_blocks_per_cu)
      info.fwd_blocks_per_cu = GRN_FWD_WG_PER_CU;
    if (GRN_BWD_WG_PER_CU > 0 && GRN_BWD_WG_PER_CU < info.bwd_blocks_per_cu)
      info.bwd_blocks_per_cu = GRN_BWD_WG_PER_CU;
    cache[dev] = info;
    __atomic_store_n(&ready[dev], true, __ATOMIC_RELEASE);
  }
  return cache[dev];
}

// A dispatch counts work-items in 32 bits, so a grid of 256-thread
// workgroups stays below 2^24 of them; the kernels' grid-stride loops cover
// any remaining work.
constexpr int64_t kMaxGrid = (int64_t{1} << 24) - 1;

int64_t cap_grid(int64_t want, int64_t resident, int max_wg) {
  int64_t grid = (resident > 0 && want > resident) ? resident : want;
  if (max_wg > 0 && grid > max_wg) grid = max_wg;
  if (grid > kMaxGrid) grid = kMaxGrid;
  return grid < 1 ? 1 : grid;
}

}  // namespace

BwdLayout bwd_layout(int64_t rows) {
  BwdLayout L;
  if (rows <= 0) {
    L.bytes = kCounterBytes;
    return L;
  }
  L.chunk_rows = chunk_rows_for(rows);
  L.nchunks = (rows + L.chunk_rows - 1) / L.chunk_rows;
  int64_t gs = 1;
  while (gs * gs < L.nchunks) ++gs;  // ceil(sqrt(nchunks)), at most 4096
  L.group_size = gs;
  L.ngroups = (L.nchunks + gs - 1) / gs;
  L.partial_off = kCounterBytes;
  L.gpart_off = L.partial_off + (size_t)L.nchunks * kD * sizeof(float);
  L.bytes = L.gpart_off + (size_t)L.ngroups * kD * sizeof(float);
  return L;
}

hipError_t launch_fwd(const void* x, const void* g, const void* w, void* y,
                      const RowStrides& st, int64_t rows, float eps, int max_wg,
                      hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const FwdPitch pt{(uint32_t)(st.x / kVec), (uint32_t)(st.g / kVec),
                    (uint32_t)(st.y / kVec)};
  const DeviceInfo info = device_info();
  const int64_t ntiles = (rows + kRowsPerAccess * kFwdU - 1) /
                         (kRowsPerAccess * kFwdU);
  const int64_t want = (ntiles + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t resident =
      GRN_FWD_WG_PER_CU < 0 ? 0 : (int64_t)info.cus * info.fwd_blocks_per_cu;
  const int64_t grid = cap_grid(want, resident, max_wg);
  hipLaunchKernelGGL(fwd_kernel<kFwdU>, dim3((unsigned)grid), dim3(kBlock), 0,
                     s, static_cast<const u32x4*>(x),
                     static_cast<const u32x4*>(g),
                     static_cast<const u32x4*>(w), static_cast<u32x4*>(y), pt,
                     rows, eps, ntiles);
  return hipGetLastError();
}

hipError_t launch_bwd(const void* x, const void* g, const void* w,
                      const void* dy, void* dx, void* dg, void* dw,
                      int dw_fp32, int deterministic, void* workspace,
                      const RowStrides& st, int64_t rows, float eps, int max_wg,
                      hipStream_t s) {
  const BwdLayout L = bwd_layout(rows);
  const BwdPitch pt{(uint32_t)(st.x / kVec), (uint32_t)(st.g / kVec),
                    (uint32_t)(st.dy / kVec), (uint32_t)(st.dx / kVec),
                    (uint32_t)(st.dg / kVec)};
  if (L.nchunks == 0) {
    hipLaunchKernelGGL(dw_zero_kernel, dim3(1), dim3(kD), 0, s, dw, dw_fp32);
    return hipGetLastError();
  }
  char* ws = static_cast<char*>(workspace);
  const DeviceInfo info = device_info();
  const int64_t resident =
      GRN_BWD_WG_PER_CU < 0 ? 0 : (int64_t)info.cus * info.bwd_blocks_per_cu;
  const int64_t nwork = L.nchunks + (deterministic && kReducers ? L.ngroups : 0);
  const int64_t grid = cap_grid(nwork, resident, max_wg);
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kBwdWaves * kWave), 0, s,
                       static_cast<const u32x4*>(x), static_cast<const u32x4*>(g),
                       static_cast<const u32x4*>(w), static_cast<const u32x4*>(dy),
                       static_cast<u32x4*>(dx), static_cast<u32x4*>(dg), pt,
                       reinterpret_cast<float*>(ws + L.partial_off),
                       reinterpret_cast<float*>(ws + L.gpart_off),
                       reinterpret_cast<uint32_t*>(ws), dw, dw_fp32, rows, eps,
                       L.nchunks, L.group_size, L.ngroups);
  };
  if (deterministic) {
    launch(kBwdDet);
  } else {
    launch(kBwdNondet);
  }
  return hipGetLastError();
}

hipError_t launch_counters_zero(void* workspace, hipStream_t s) {
  hipLaunchKernelGGL(counters_zero_kernel, dim3(1), dim3(kBlock), 0, s,
                     static_cast<uint32_t*>(workspace));
  return hipGetLastError();
}

}  // namespace grn
