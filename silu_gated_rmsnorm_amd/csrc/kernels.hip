// gfx950 kernels of the SiLU-gated RMSNorm training forward and backward.
//
// Operator (flashinfer PR #8701, "perf(cake_rmsnorm_silu_gate_train):
// L2-prefetching extra-long forward on SM107": PR description and commit
// 10c6017 message), per row i of D values, with w shared by all rows:
//   r = 1/sqrt(mean(x^2) + eps),  n = x r,  s = silu(g) = g sigmoid(g)
//   y = n w s
//   dn = dy w s,  c = mean(dn n),  dx = r (dn - n c)
//   dg = dy w n silu'(g),  silu'(g) = sigmoid(g) + s (1 - sigmoid(g))
//   dw = sum over rows of dy n s
// The pages time D = 128 in BF16; the same kernels are instantiated for
// D = 64, 128, 256 and BF16, FP16 or FP32 storage (arithmetic is FP32).
//
// All three kernels stream HBM and do a few FP32 operations per byte, below
// the ridge point of the vector ALUs, so they are written for memory
// throughput: 16-byte coalesced accesses, several independent row groups in
// flight per wave before any arithmetic, row sums in registers, no LDS on
// the per-row path, no MFMA (there is no contraction to feed it).  The
// backward's per-element arithmetic (two transcendentals and ~20 other
// operations) is not negligible next to its memory time, so it is kept
// lean: shared products, wave-uniform (scalar) addressing, and no per-lane
// predicates except in the one tile that holds the ragged end of the rows.
// Rows whose sum of squares overflows FP32 are marked (r becomes NaN) at
// the cost of two instructions and redone by a cold fix-up pass that the
// wave enters only when it saw such a row (fwd_tile, bwd_chunk_fixup).
#include "common.h"
#include "launch.h"

#include <type_traits>

// Tiling knobs (compile-time; results other than dw do not depend on them,
// and dw depends only on the chunk size, chunk_rows_for() in launch.h).
#ifndef GRN_FWD_U
#define GRN_FWD_U 2          // row groups per wave tile in the forward ...
#endif
#ifndef GRN_FWD_U_LARGE
#define GRN_FWD_U_LARGE 4    // ... and for tensors of at least GRN_FWD_LARGE_BYTES
#endif
#ifndef GRN_FWD_LARGE_BYTES
#define GRN_FWD_LARGE_BYTES (128ll << 20)
#endif
// ... up to tensors of this size, from which the 8-row tiles in two-wave
// workgroups are faster again (forward alone, eager, same process: 16-row /
// 8-row tiles 131072x48 797 / 786 us, 262144x48 1,619 / 1,572; 65536x48
// 381 / 388; the step fwd + bwd 2,143 / 2,129, 4,347 / 4,301 and 1,024 /
// 1,028 us).
#ifndef GRN_FWD_HUGE_BYTES
#define GRN_FWD_HUGE_BYTES (1ll << 30)
#endif
// Waves per forward workgroup, below and from GRN_FWD_LARGE_BYTES.
// Measured (forward alone, graph-batched, same process, alternating; 4 vs 2
// waves): 1031x48 9.02 vs 8.74 us, 2000x48 14.21 vs 13.99, 3534x48 22.81 vs
// 22.45, 7684x48 46.36 vs 45.68, 10600x48 63.05 vs 62.05; with the 16-row
// tiles 12296x48 71.8 vs 73.3 and 32768x48 186.9 vs 195.3.  One wave was no
// better than two; eight and sixteen were slower.
#ifndef GRN_FWD_WAVES
#define GRN_FWD_WAVES 2
#endif
#ifndef GRN_FWD_WAVES_LARGE
#define GRN_FWD_WAVES_LARGE 4
#endif
// Backward shape by tensor size (bytes of one [rows, D] activation):
// row groups per wave step (U) and steps of loads prefetched ahead (PF).
// From GRN_BWD_LARGE_BYTES up only some types and widths take the LARGE
// shape (prefetch_large()); the others keep the MID one.  U and the chunk
// layout change the order in which a chunk's rows are added into dw, so
// dw's bits depend on the tier, which depends only on rows, D and the type.
#ifndef GRN_BWD_SMALL_BYTES
#define GRN_BWD_SMALL_BYTES (32ll << 20)
#endif
#ifndef GRN_BWD_LARGE_BYTES
#define GRN_BWD_LARGE_BYTES (256ll << 20)
#endif
#ifndef GRN_BWD_U_SMALL
#define GRN_BWD_U_SMALL 2
#endif
#ifndef GRN_BWD_PF_SMALL
#define GRN_BWD_PF_SMALL 1
#endif
#ifndef GRN_BWD_U_MID
#define GRN_BWD_U_MID 4
#endif
#ifndef GRN_BWD_PF_MID
#define GRN_BWD_PF_MID 0
#endif
#ifndef GRN_BWD_U_LARGE
#define GRN_BWD_U_LARGE 4
#endif
#ifndef GRN_BWD_PF_LARGE
#define GRN_BWD_PF_LARGE 1
#endif
// Large tensors: hold the dx/dg stores of a chunk's last step until after
// the wait for the chunk's dw partial (see bwd_kernel; hold_large()).
#ifndef GRN_BWD_HOLD_LARGE
#define GRN_BWD_HOLD_LARGE 1
#endif
// Steps without prefetch (the middle tier): issue the next step's loads
// before this step's stores (see bwd_chunk).
#ifndef GRN_BWD_LBS
#define GRN_BWD_LBS 1
#endif
#ifndef GRN_BWD_U_ND
#define GRN_BWD_U_ND 4       // the non-deterministic dw kernel, all sizes
#endif
#ifndef GRN_BWD_WAVES
#define GRN_BWD_WAVES 4      // waves per backward workgroup
#endif
#ifndef GRN_BWD_MIN_WAVES
#define GRN_BWD_MIN_WAVES 0  // >0: ask for at least this many waves per SIMD
#endif
#ifndef GRN_BWD_ND_PREFETCH
#define GRN_BWD_ND_PREFETCH 0  // steps prefetched by the non-deterministic kernel
#endif
#ifndef GRN_SUM_BATCH
#define GRN_SUM_BATCH 8      // partial rows per thread per round trip in the dw tree
#endif
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

// The forward loads w once per workgroup, before its streamed loads, but
// keeps it raw until the first tile's data is needed: this opaque copy stops
// the compiler from hoisting w's unpacking (and so the wait for its load)
// ahead of the streamed loads, which made every workgroup wait a full
// memory round trip before issuing anything (measured: 46.5 -> 45.7 us at
// 7684x48).  The backward keeps w unpacked from the start: the same change
// there altered its register allocation and measured slower.
__device__ __forceinline__ u32x4 use_when_needed(u32x4 v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Wave index as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

// Row pitch of a tensor in 16-byte units (a packed row of 128 BF16 is 16).
// Lane l of a wave touches row kRows*u + l/kLanes of its tile, 16 bytes at
// (l % kLanes) * 16 within that row.
template <class S>
__device__ __forceinline__ uint32_t lane_offset(int lane, int u, uint32_t pitch) {
  return (uint32_t)(S::kRows * u + lane / S::kLanes) * pitch +
         (uint32_t)(lane & (S::kLanes - 1));
}

// The same offset as a signed 64-bit value, for the backward's fix-up pass
// (bwd_chunk): had the fix-up used lane_offset's unsigned 32-bit form, which
// the main pass needs for its scalar-base addressing, the compiler would have
// shared that form between the two and given the whole kernel 256 VGPRs.
template <class S>
__device__ __forceinline__ int64_t lane_offset_cold(int lane, int u, uint32_t pitch) {
  return (int64_t)(S::kRows * u + lane / S::kLanes) * (int64_t)pitch +
         (int64_t)(lane & (S::kLanes - 1));
}

// --------------------------------------------------------------------------
// Forward.  A wave tile is U groups of kRows consecutive rows.  Lane l owns
// values [kVec(l%kLanes), kVec(l%kLanes)+kVec) of tile row kRows*u +
// l/kLanes.  With packed rows a tile is U contiguous KiB per tensor.  Waves
// walk the tiles with a grid stride.

struct FwdPitch {
  uint32_t x, g, y;  // row pitches in 16-byte units
};

// Whether a row's sum of squares can exceed FP32's range: not for FP16
// storage (its largest square, 65504^2, times 256 entries is about 1.1e12).
template <Dt T, int D>
constexpr bool can_overflow() {
  return T != Dt::f16;
}

// y for one row group of a forward tile (lane l: row kRows*u + l/kLanes).
// The main pass (kFix = false) marks a row whose sum of squares overflowed
// FP32 by making its r NaN (r times fma(ss, 0, 1): exactly 1 for a finite
// sum), so its y comes out NaN and so does `mark`.  The fix-up pass (kFix =
// true) takes the sum again over x scaled by kOverflowScale and stores y of
// those rows only.
template <Dt T, int D, bool kFix>
__device__ __forceinline__ void fwd_rows(u32x4 xv, u32x4 gv, u32x4* __restrict__ dst,
                                         const float (&wf)[Shape<T, D>::kVec], float eps,
                                         bool valid, float& mark) {
  using S = Shape<T, D>;
  using C = typename S::C;
  constexpr int kVec = S::kVec;
  float xf[kVec], gf[kVec];
  C::unpack(xv, xf);
  C::unpack(gv, gf);
  float ss = 0.0f;
#pragma unroll
  for (int e = 0; e < kVec; ++e) ss = fmaf(xf[e], xf[e], ss);
  ss = row_sum<S::kLanes>(ss);
  float r = rsqrt_fast(ss * (1.0f / D) + eps);
  bool fix_row = false;
  if constexpr (!kFix) {
    if constexpr (can_overflow<T, D>()) {
      r *= fmaf(ss, 0.0f, 1.0f);
      mark += r;
    }
  } else {
    float ss2 = 0.0f;
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      const float xs = xf[e] * kOverflowScale;
      ss2 = fmaf(xs, xs, ss2);
    }
    ss2 = row_sum<S::kLanes>(ss2);
    fix_row = overflowed(ss);
    r = rsqrt_fast(ss2 * (1.0f / D) + eps * kOverflowScale2) * kOverflowScale;
  }
  float yf[kVec];
#pragma unroll
  for (int e = 0; e < kVec; ++e) {
    const float s = gf[e] * sigmoid_fast(gf[e]);
    yf[e] = (xf[e] * r) * wf[e] * s;
  }
  if (valid && (!kFix || fix_row)) st_stream<(GRN_FWD_NTS & 1) != 0>(dst, C::pack(yf));
}

template <Dt T, int D, int U, bool kFull>
__device__ __forceinline__ void fwd_tile(const u32x4* __restrict__ xb,
                                         const u32x4* __restrict__ gb,
                                         u32x4* __restrict__ yb, FwdPitch pt,
                                         u32x4 w_raw, float eps, int lane, int nvalid) {
  using S = Shape<T, D>;
  using C = typename S::C;
  constexpr int kVec = S::kVec;
  const int sub = lane / S::kLanes;
  u32x4 xv[U], gv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (kFull || S::kRows * u + sub < nvalid) {
      xv[u] = ld_stream<(GRN_FWD_NTL & 1) != 0>(xb + lane_offset<S>(lane, u, pt.x));
      gv[u] = ld_stream<(GRN_FWD_NTL & 2) != 0>(gb + lane_offset<S>(lane, u, pt.g));
    } else {
      xv[u] = u32x4{0, 0, 0, 0};
      gv[u] = u32x4{0, 0, 0, 0};
    }
  }
  float wf[kVec];
  C::unpack(use_when_needed(w_raw), wf);
  float mark = 0.0f;
#pragma unroll
  for (int u = 0; u < U; ++u)
    fwd_rows<T, D, false>(xv[u], gv[u], yb + lane_offset<S>(lane, u, pt.y), wf, eps,
                          kFull || S::kRows * u + sub < nvalid, mark);
  // A row whose sum of squares overflowed FP32 (entries beyond ~1.8e19 at
  // D = 128): its y went out NaN; store it again from the scaled sum (the
  // same address, later in the same lane's program order).  Taken by no
  // wave on data within FP32's range.
  if (can_overflow<T, D>() && wave_any_nan(mark)) {
    // Opaque copies (as in the backward's fix-up): nothing here is hoisted
    // into, or shared with, the main pass.
    int cl = lane;
    FwdPitch cp = pt;
    asm volatile("" : "+v"(cl), "+s"(cp.x), "+s"(cp.g), "+s"(cp.y));
    const int csub = cl / S::kLanes;
#pragma unroll 1
    for (int u = 0; u < U; ++u) {
      const bool valid = kFull || S::kRows * u + csub < nvalid;
      u32x4 xr = u32x4{0, 0, 0, 0}, gr = u32x4{0, 0, 0, 0};
      if (valid) {
        xr = xb[lane_offset_cold<S>(cl, u, cp.x)];
        gr = gb[lane_offset_cold<S>(cl, u, cp.g)];
      }
      fwd_rows<T, D, true>(xr, gr, yb + lane_offset_cold<S>(cl, u, cp.y), wf, eps, valid, mark);
    }
  }
}

template <Dt T, int D, int U, int kWaves>
__global__ void __launch_bounds__(kWaves * kWave)
fwd_kernel(const u32x4* __restrict__ x, const u32x4* __restrict__ g,
           const u32x4* __restrict__ w, u32x4* __restrict__ y, FwdPitch pt,
           int64_t rows, float eps, int64_t ntiles) {
  using S = Shape<T, D>;
  constexpr int kTileRows = S::kRows * U;
  const int lane = threadIdx.x & (kWave - 1);
  const u32x4 w_raw = w[lane & (S::kLanes - 1)];  // this lane's kVec values of w

  const int64_t nwaves = (int64_t)gridDim.x * kWaves;
  for (int64_t t = (int64_t)blockIdx.x * kWaves + wave_index(); t < ntiles; t += nwaves) {
    const int64_t row0 = t * kTileRows;
    const u32x4* xb = x + row0 * pt.x;
    const u32x4* gb = g + row0 * pt.g;
    u32x4* yb = y + row0 * pt.y;
    if (row0 + kTileRows <= rows) {
      fwd_tile<T, D, U, true>(xb, gb, yb, pt, w_raw, eps, lane, kTileRows);
    } else {
      fwd_tile<T, D, U, false>(xb, gb, yb, pt, w_raw, eps, lane, (int)(rows - row0));
    }
  }
}

// --------------------------------------------------------------------------
// Backward, dx/dg and one partial dw per chunk of R rows (R depends only on
// the row size: chunk_rows_for()).
//
// The dw order is fixed by the chunk alone: within chunk c, wave v of the
// workgroup takes step `it` on rows row0(c) + it*stride(c) + v*kRows*U +
// kRows*u + l/kLanes (chunk_blocks(): contiguous chunks have row0 = c*R and
// stride = kWaves*kRows*U), and lane l adds its kVec columns' contributions
// in (it, u) order into FP32 registers.  At the end of the chunk the kWaves*kRows
// (wave, row-in-group) accumulators of each column are added in index order
// through LDS.  Which workgroup runs a chunk, and when, changes nothing, so
// dw does not depend on the grid or on timing.

// Raw registers of one wave step (U row groups, three inputs).
template <int U>
struct BwdRaw {
  u32x4 x[U], g[U], dy[U];
};

// Packed dx and dg of one wave step whose stores are held back (the last
// step of a chunk: see bwd_kernel), with the step's first row and count of
// valid rows.
template <int U>
struct BwdOut {
  u32x4 dx[U], dg[U];
  int64_t row0;
  int nvalid;
};

struct BwdPitch {
  uint32_t x, g, dy, dx, dg;  // row pitches in 16-byte units
};

template <class S, int U, bool kFull>
__device__ __forceinline__ void bwd_load(BwdRaw<U>& r,
                                         const u32x4* __restrict__ xb,
                                         const u32x4* __restrict__ gb,
                                         const u32x4* __restrict__ dyb,
                                         BwdPitch pt, int lane, int nvalid) {
  const int sub = lane / S::kLanes;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (kFull || S::kRows * u + sub < nvalid) {
      r.x[u] = ld_stream<(GRN_BWD_NTL & 1) != 0>(xb + lane_offset<S>(lane, u, pt.x));
      r.g[u] = ld_stream<(GRN_BWD_NTL & 2) != 0>(gb + lane_offset<S>(lane, u, pt.g));
      r.dy[u] = ld_stream<(GRN_BWD_NTL & 4) != 0>(dyb + lane_offset<S>(lane, u, pt.dy));
    } else {
      r.x[u] = u32x4{0, 0, 0, 0};
      r.g[u] = u32x4{0, 0, 0, 0};
      r.dy[u] = u32x4{0, 0, 0, 0};
    }
  }
}

// One wave step of the backward.
//
// Rows whose sum of squares overflows FP32 (entries beyond about 1.8e19 at
// D = 128) need the sums taken over scaled x (kOverflowScale).  A branch
// inside the unrolled step, however rarely taken, made the compiler keep
// every row group's values live across it (256 VGPRs: one wave per SIMD
// instead of two or three), and so did any per-row flag carried through
// the steps.  So the main pass (kFix = false) marks such a row by making
// its r NaN instead (r times fma(ss, 0, 1), which is exactly 1 for a finite
// sum and NaN for an infinite one: two instructions, no live state); the
// NaN reaches the lane's dw accumulator, which bwd_chunk tests once per
// chunk.  The fix-up pass (kFix = true) recomputes a wave's steps: every
// row's dw term again, in the main pass's order (the same bits for the
// other rows), and for the overflowed rows the scaled sums, whose dx and dg
// it writes over the main pass's NaN.
template <Dt T, int D, int U, bool kFull, bool kDefer, bool kFix = false>
__device__ __forceinline__ void bwd_compute(const BwdRaw<U>& r,
                                            u32x4* __restrict__ dxb,
                                            u32x4* __restrict__ dgb, BwdPitch pt,
                                            const float (&wf)[Shape<T, D>::kVec],
                                            float eps, int lane, int nvalid,
                                            float (&acc)[Shape<T, D>::kVec],
                                            BwdOut<U>& held) {
  using S = Shape<T, D>;
  using C = typename S::C;
  constexpr int kVec = S::kVec;
  const int sub = lane / S::kLanes;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float xf[kVec], gf[kVec], dyf[kVec];
    C::unpack(r.x[u], xf);
    C::unpack(r.g[u], gf);
    C::unpack(r.dy[u], dyf);
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
    ss = row_sum<S::kLanes>(ss);
    sd = row_sum<S::kLanes>(sd);
    float rs = rsqrt_fast(ss * (1.0f / D) + eps);
    float cr;
    bool fix_row = false;
    if constexpr (!kFix) {
      if constexpr (can_overflow<T, D>())
        rs *= fmaf(ss, 0.0f, 1.0f);  // NaN marks a row beyond FP32's range
      cr = rs * sd * (1.0f / D);   // c = mean(dn n) = r mean(dn x)
    } else {
      cr = rs * sd * (1.0f / D);
      // Both sums again over x scaled by 2^-70 (exact), which also keeps
      // sum(dn x) of such rows in range; used for overflowed rows only.
      float ss2 = 0.0f, sd2 = 0.0f;
#pragma unroll
      for (int e = 0; e < kVec; ++e) {
        const float xs = xf[e] * kOverflowScale;
        ss2 = fmaf(xs, xs, ss2);
        sd2 = fmaf(dn[e], xs, sd2);
      }
      ss2 = row_sum<S::kLanes>(ss2);
      sd2 = row_sum<S::kLanes>(sd2);
      const float rs2 = rsqrt_fast(ss2 * (1.0f / D) + eps * kOverflowScale2);
      fix_row = overflowed(ss);
      rs = fix_row ? rs2 * kOverflowScale : rs;
      cr = fix_row ? rs2 * sd2 * (1.0f / D) : cr;
    }
    float dxf[kVec], dgf[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      const float n = xf[e] * rs;
      dxf[e] = rs * fmaf(-n, cr, dn[e]);
      dgf[e] = tg[e] * n;
      q[e] *= n;  // dw contribution dy n s
    }
    const bool valid = kFull || S::kRows * u + sub < nvalid;
    if (valid) {
      if (!kFix || fix_row) {
        if constexpr (kDefer) {
          // Packed here, not where they are stored: the opaque copies keep
          // the compiler from carrying the FP32 values to the stores.
          held.dx[u] = use_when_needed(C::pack(dxf));
          held.dg[u] = use_when_needed(C::pack(dgf));
        } else if constexpr (kFix) {
          st_stream<(GRN_BWD_NTS & 1) != 0>(dxb + lane_offset_cold<S>(lane, u, pt.dx),
                                            C::pack(dxf));
          st_stream<(GRN_BWD_NTS & 2) != 0>(dgb + lane_offset_cold<S>(lane, u, pt.dg),
                                            C::pack(dgf));
        } else {
          st_stream<(GRN_BWD_NTS & 1) != 0>(dxb + lane_offset<S>(lane, u, pt.dx), C::pack(dxf));
          st_stream<(GRN_BWD_NTS & 2) != 0>(dgb + lane_offset<S>(lane, u, pt.dg), C::pack(dgf));
        }
      }
#pragma unroll
      for (int e = 0; e < kVec; ++e) acc[e] += q[e];
    }
  }
}

// The stores bwd_compute held back (kFull: every row of the step is valid).
template <class S, int U, bool kFull = false>
__device__ __forceinline__ void bwd_store_held(const BwdOut<U>& held,
                                               u32x4* __restrict__ dx,
                                               u32x4* __restrict__ dg, BwdPitch pt,
                                               int lane) {
  const int sub = lane / S::kLanes;
  u32x4* dxb = dx + held.row0 * pt.dx;
  u32x4* dgb = dg + held.row0 * pt.dg;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (kFull || S::kRows * u + sub < held.nvalid) {
      st_stream<(GRN_BWD_NTS & 1) != 0>(dxb + lane_offset<S>(lane, u, pt.dx), held.dx[u]);
      st_stream<(GRN_BWD_NTS & 2) != 0>(dgb + lane_offset<S>(lane, u, pt.dg), held.dg[u]);
    }
  }
}

// The backward's fix-up of one wave's share of a chunk, for a wave whose
// dw accumulator came out NaN: some row's sum of squares overflowed FP32 (or
// the inputs hold a NaN or an infinity).  The wave reads its steps again,
// one row group at a time, and redoes them in the main pass's order
// (bwd_compute, kFix): dw's bits are those of a pass that had summed those
// rows right the first time.  Its stores go to the same addresses as the main
// pass's, later in the same lane's program order.  Kept out of line: inlined,
// its address arithmetic changed how the compiler allocated the main pass's
// registers (256 VGPRs, one wave per SIMD).
template <Dt T, int D, int U, int kWaves, int R, bool kHold, bool kFull>
__device__ __forceinline__ void bwd_chunk_fixup(
    const u32x4* __restrict__ x, const u32x4* __restrict__ g, const u32x4* __restrict__ dy,
    u32x4* __restrict__ dx, u32x4* __restrict__ dg, BwdPitch pt,
    const float (&wf)[Shape<T, D>::kVec], float eps, int64_t chunk0, int64_t it_stride,
    int64_t rows, int wave, int lane, float (&acc)[Shape<T, D>::kVec], BwdOut<U>& held) {
  using S = Shape<T, D>;
  constexpr int kRows = S::kRows;
  constexpr int kStepRows = kRows * U;
  constexpr int kIters = R / (kWaves * kStepRows);
  asm volatile("" : "+v"(lane), "+s"(pt.x), "+s"(pt.g), "+s"(pt.dy), "+s"(pt.dx), "+s"(pt.dg));
#pragma unroll
  for (int e = 0; e < S::kVec; ++e) acc[e] = 0.0f;
#pragma unroll 1
  for (int it = 0; it < kIters; ++it) {
    const int64_t row0 = chunk0 + it * it_stride + (int64_t)wave * kStepRows;
    const int64_t left = rows - row0;
    const int nvalid = (int)(left < 0 ? 0 : (left > kStepRows ? kStepRows : left));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t r0 = row0 + kRows * u;
      const int nv = nvalid - kRows * u;
      BwdRaw<1> b;
      BwdOut<1> h;
      bwd_load<S, 1, kFull>(b, x + r0 * pt.x, g + r0 * pt.g, dy + r0 * pt.dy, pt, lane, nv);
      if (kHold && it + 1 == kIters) {
        // this step's stores are still held: patch the held values
        h.dx[0] = held.dx[u];
        h.dg[0] = held.dg[u];
        bwd_compute<T, D, 1, kFull, true, true>(b, dx + r0 * pt.dx, dg + r0 * pt.dg, pt, wf,
                                                eps, lane, nv, acc, h);
        held.dx[u] = h.dx[0];
        held.dg[u] = h.dg[0];
      } else {
        bwd_compute<T, D, 1, kFull, false, true>(b, dx + r0 * pt.dx, dg + r0 * pt.dg, pt, wf,
                                                 eps, lane, nv, acc, h);
      }
    }
  }
}

// One chunk for one workgroup: wave `wave` takes steps it = 0..kIters-1 on
// rows row0(it) = chunk0 + it*it_stride + wave*kRows*U (it_stride is
// kWaves*kRows*U for a contiguous chunk: chunk_blocks()).  The loads of the
// next kPrefetch steps are issued before the arithmetic of step it, so
// every wave keeps reads in flight while it computes.
template <Dt T, int D, int U, int kWaves, int R, int kPrefetch, bool kHold, bool kLbs,
          bool kFull>
__device__ __forceinline__ void bwd_chunk(const u32x4* __restrict__ x,
                                          const u32x4* __restrict__ g,
                                          const u32x4* __restrict__ dy,
                                          u32x4* __restrict__ dx,
                                          u32x4* __restrict__ dg, BwdPitch pt,
                                          const float (&wf)[Shape<T, D>::kVec],
                                          float eps, int64_t chunk0, int64_t it_stride,
                                          int64_t rows,
                                          int wave, int lane,
                                          float (&acc)[Shape<T, D>::kVec],
                                          BwdOut<U>& held) {
  using S = Shape<T, D>;
  constexpr int kStepRows = S::kRows * U;
  constexpr int kIters = R / (kWaves * kStepRows);
  auto row_of = [&](int it) {
    return chunk0 + it * it_stride + (int64_t)wave * kStepRows;
  };
  auto nvalid_of = [&](int it) {
    const int64_t left = rows - row_of(it);
    return (int)(left < 0 ? 0 : (left > kStepRows ? kStepRows : left));
  };
  if constexpr (kLbs) {
    // Without prefetch, the next step's loads go out after this step's
    // arithmetic but before its stores.  A wave's memory counter retires
    // loads and stores in issue order, so loads issued after the stores
    // would also wait for the stores to complete; this order keeps the
    // next loads independent of them, at the cost of this step's packed
    // outputs waiting in registers (lbs_mid() says where it pays).
    static_assert(kPrefetch == 0, "the step order without prefetch");
    BwdRaw<U> b;
    auto load1 = [&](int it) {
      const int64_t row0 = row_of(it);
      bwd_load<S, U, kFull>(b, x + row0 * pt.x, g + row0 * pt.g, dy + row0 * pt.dy, pt,
                            lane, nvalid_of(it));
    };
    load1(0);
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      BwdOut<U> out;
      out.row0 = row_of(it);
      out.nvalid = nvalid_of(it);
      bwd_compute<T, D, U, kFull, true>(b, dx + out.row0 * pt.dx, dg + out.row0 * pt.dg, pt,
                                        wf, eps, lane, out.nvalid, acc, out);
      if (it + 1 < kIters) {
        asm volatile("" ::: "memory");  // keep the loads after this step's arithmetic
        load1(it + 1);
      }
      if (kHold && it + 1 == kIters) {
        held = out;
      } else {
        bwd_store_held<S, U, kFull>(out, dx, dg, pt, lane);
        asm volatile("" ::: "memory");  // and the stores before the next step
      }
    }
  } else {
    // A ring of kDepth register buffers: step it+kDepth-1 is loaded while
    // step it is computed.
    constexpr int kDepth = kPrefetch + 1;
    BwdRaw<U> buf[kDepth];
    auto load = [&](BwdRaw<U>& b, int it) {
      const int64_t row0 = row_of(it);
      bwd_load<S, U, kFull>(b, x + row0 * pt.x, g + row0 * pt.g, dy + row0 * pt.dy, pt,
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
      if (!kHold || it + 1 < kIters) {
        bwd_compute<T, D, U, kFull, false>(buf[it % kDepth], dx + row0 * pt.dx,
                                           dg + row0 * pt.dg, pt, wf, eps, lane,
                                           nvalid_of(it), acc, held);
      } else {
        held.row0 = row0;
        held.nvalid = nvalid_of(it);
        bwd_compute<T, D, U, kFull, true>(buf[it % kDepth], dx + row0 * pt.dx,
                                          dg + row0 * pt.dg, pt, wf, eps, lane,
                                          held.nvalid, acc, held);
      }
    }
  }
}

// Cross-workgroup hand-off of the dw partials, and why its order holds.
//
// Producer (the workgroup of chunk c):
//   1. each of threads 0..D-1 writes its column of partial[c] with a relaxed
//      agent-scope atomic store (store_coherent: global_store_dword sc1 on
//      gfx950, written through this XCD's L2 to the point where every XCD's
//      accesses meet);
//   2. s_waitcnt vmcnt(0) (wait_memory): the wave waits until those stores
//      are acknowledged, which for an sc1 store means the value is visible
//      to agent-scope accesses from any XCD;
//   3. __syncthreads(), so every storing wave has passed step 2;
//   4. thread 0 increments the group's counter (relaxed agent-scope atomic
//      add that returns the old value: global_atomic_add sc0).
// Consumer (the workgroup whose increment was the group's last):
//   5. it has waited for the atomic's returned value (s_waitcnt) and branched
//      on it through LDS and a barrier before it issues any load of the
//      partials; GPUs issue no load ahead of such a branch;
//   6. it reads the partials with agent-scope loads (buffer_load sc1), which
//      are served at the same point of coherence, never from a stale line of
//      its own XCD's L2 (a line left, e.g., by an earlier call that used
//      the same workspace).
// Every producer's increment is ordered after its partial is visible (2-4),
// and the last increment follows all others in the counter's modification
// order, so the consumer's loads (5-6) see every partial of the group.  The
// same holds one level up (group sums -> overall counter -> final sum).
// This is the sequence the compiler's own agent-scope release/acquire
// lowering for gfx950 produces (release: s_waitcnt vmcnt(0) before the
// atomic; acquire: wait for the atomic, then coherent loads), minus the
// cache-wide L2 write-back (buffer_wbl2) and invalidate (buffer_inv) that
// such a fence adds for plain stores and loads elsewhere in the wave: the
// partials are themselves agent-scope atomic accesses and need neither.  A
// version with __threadfence() (both cache-wide operations per workgroup)
// ran 5x slower.  What it relies on: sc1 stores and loads and the vmcnt
// wait behave as above (gfx942/gfx950 memory model); the compiler does not
// move the stores past wait_memory (an s_waitcnt builtin, a barrier to it)
// nor the loads above the branch on the atomic's result.  The 200-run soak
// (tests/test_handoff_soak.py) and the 10-run bitwise tests check it on the
// device.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A raw buffer over `count` rows of D FP32 values; loads past the end of
// the buffer return zero (hardware range check).
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const float* p,
                                                            int64_t count) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), 0,
                                           (int)(count * D * sizeof(float)),
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

// Column sums of a [count, D] FP32 array, in a fixed order.  Thread t of the
// workgroup owns columns 4q .. 4q+3 (q = t % (D/4)) and row slot
// t / (D/4): it adds rows slot, slot+S, slot+2S, ... (S = 4*threads/D
// slots) in increasing order (16-byte loads issued GRN_SUM_BATCH rows at a
// time; rows past the end read as zero).  The S slots of each column are
// then added in slot order.  The result is valid in threads 0..D-1 (one
// column each).  `lds` holds at least 4*threads floats.
template <int kThreads, int D>
__device__ __forceinline__ float column_sum_fixed(const float* __restrict__ src,
                                                  int64_t count,
                                                  float* __restrict__ lds) {
  constexpr int kQuads = D / 4;
  constexpr int kSlots = kThreads / kQuads;
  static_assert(kSlots >= 1 && kThreads % kQuads == 0, "threads cover the columns");
  constexpr int kBatch = GRN_SUM_BATCH;
  const int t = threadIdx.x;
  const int quad = t % kQuads;
  const int slot = t / kQuads;
  const __amdgpu_buffer_rsrc_t rsrc = rows_rsrc<D>(src, count);
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t r0 = slot; r0 < count; r0 += kSlots * kBatch) {
    float4 v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int64_t r = r0 + (int64_t)kSlots * k;  // past the end: reads zero
      v[k] = load_coherent4(rsrc, (int)((r * D + 4 * quad) * sizeof(float)));
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      a.x += v[k].x; a.y += v[k].y; a.z += v[k].z; a.w += v[k].w;
    }
  }
  // lds[slot][column]
  lds[slot * D + 4 * quad + 0] = a.x;
  lds[slot * D + 4 * quad + 1] = a.y;
  lds[slot * D + 4 * quad + 2] = a.z;
  lds[slot * D + 4 * quad + 3] = a.w;
  __syncthreads();
  float res = 0.0f;
  if (t < D) {
#pragma unroll
    for (int k = 0; k < kSlots; ++k) res += lds[k * D + t];
  }
  __syncthreads();
  return res;
}

// Which rows make up chunk c.  A chunk is R/B blocks of B rows (B: the rows
// a workgroup step covers), block it starting at row0 + it*stride.
//  * W = 0: the chunk is rows [c*R, c*R + R) (stride B).
//  * W > 0: chunks are taken in windows of W; within the
//    window of chunks [s*W, s*W + Ws), block it of its j-th chunk is block
//    s*W*(R/B) + it*Ws + j of the tensor.  The windows tile the rows in
//    order, so the mapping is a bijection onto blocks (the last window has
//    Ws = nchunks - s*W <= W chunks); blocks at or past the end of the rows
//    are empty.  Chunks resident at the same time then read neighbouring
//    blocks at each step, instead of one block of each of W separate chunks.
// `end` is one past the chunk's last row (for its last, highest block).
// The mapping depends on c, nchunks and the shape only, never on the grid.
//
// Measured (backward alone, BF16 D = 128, same process, alternating): with
// W = 256 chunks (a chunk's two blocks 4 MiB apart per tensor) 1031x48
// 17.48 -> 17.18 us, 3534x48 44.3 -> 43.4, 7684x48 82.8 -> 81.9, 12296x48
// 128.3 -> 127.0, 16384x32 115.2 -> 113.4; W = 64 and 128 were slower than
// contiguous chunks at most of these sizes.  The shape that loads both of a
// wave's steps at once (prefetch_large()) was 1-2 % slower with every W
// tried (256, 512, 1024) and keeps contiguous chunks.
#ifndef GRN_BWD_SWZ
#define GRN_BWD_SWZ 256   // window of the shapes without prefetch
#endif
struct ChunkBlocks {
  int64_t row0, stride, end;
};

template <int R, int B, int kW>
__device__ __forceinline__ ChunkBlocks chunk_blocks(int64_t c, int64_t nchunks) {
  constexpr int kBlocks = R / B;
  ChunkBlocks cb;
  if constexpr (kW == 0) {
    cb.row0 = c * R;
    cb.stride = B;
  } else {
    constexpr int64_t W = kW;
    const int64_t s = c / W;
    const int64_t j = c - s * W;
    const int64_t ws = (nchunks - s * W) < W ? (nchunks - s * W) : W;
    cb.row0 = (s * W * kBlocks + j) * B;
    cb.stride = ws * B;
  }
  cb.end = cb.row0 + (kBlocks - 1) * cb.stride + B;
  return cb;
}

// dw[col] = v in FP32, or rounded once to the input type.
template <Dt T>
__device__ __forceinline__ void store_dw(void* dw, int dw_fp32, int col, float v) {
  if (dw_fp32) {
    static_cast<float*>(dw)[col] = v;
  } else {
    Codec<T>::store1(dw, col, v);
  }
}

// The backward: dx and dg row by row, and dw through a fixed-order tree.
//
// dw tree (every level in a fixed order, so for given D, type and tier the
// bits depend only on rows):
//  1. chunk c (R rows, one workgroup): each lane adds its rows in
//     step order, then the lane/wave accumulators of a column are added
//     in index order -> partial[c];
//  2. group g (chunks [g*G, g*G + G), G = ceil(sqrt(nchunks))): the last
//     arrival at the group's counter adds the group's partials in chunk
//     order -> gpart[g];
//  3. the workgroup that completes the last group adds gpart in group order
//     -> dw, rounded once to the input type unless dw_fp32.
// Arrival counters live at the front of the workspace; each is returned to
// zero by the workgroup that consumes it, so a zero-filled workspace stays
// ready for the next call.
#ifndef GRN_BWD_REDUCERS
#define GRN_BWD_REDUCERS 1
#endif
constexpr bool kReducers = GRN_BWD_REDUCERS != 0;

// Whether the deterministic middle-tier backward (no prefetch) issues the
// next step's loads before this step's stores (bwd_chunk).  Measured on the
// backward alone at 7684x48 rows: FP32 D = 64 / 128 / 256 84.3 -> 82.8,
// 178 -> 173, 362 -> 359 us and BF16 D = 256 179 -> 175 us, but BF16 D = 128
// 82.6 -> 83.1 us and D = 64 45.8 -> 46.2 us (fwd + bwd back to back gains
// there, from the rows the forward leaves in the caches); FP16 would drop to
// one wave per SIMD.  Only the timing of the accesses changes.
template <Dt T, int D>
constexpr bool lbs_mid() {
  return GRN_BWD_LBS != 0 && (T == Dt::f32 || (T == Dt::bf16 && D == 256));
}

// Whether the large-tensor (prefetching) backward holds back its last
// step's stores.  Measured 1-2 % faster from 65536x48 up with BF16 at
// D = 128 (which has since moved to the middle shape), no change at 32768x48
// and slower at smaller sizes, hence large tensors only; of the types and
// widths that take the prefetching shape, BF16 at D = 64 holds.  The held
// registers cost occupancy where the kernel is already near 256 VGPRs: FP16
// at every width would drop to one wave per SIMD, so it does not hold.
// Where it holds, only the timing of the stores changes: every output bit
// is the same.
template <Dt T, int D>
constexpr bool hold_large() {
  return GRN_BWD_HOLD_LARGE != 0 && (T == Dt::f32 || (T == Dt::bf16 && D <= 128));
}

// Whether tensors of GRN_BWD_LARGE_BYTES and more take the shape that loads
// both of a wave's steps at once (otherwise the middle tier's shape, with
// interleaved chunk blocks, serves them too).  Measured per type and width
// (backward alone, same process, alternating; us, prefetching shape vs
// middle shape): FP16 D = 128 at 32768x48 / 65536x48 327 vs 329 / 658 vs
// 683, FP16 D = 64 at 65536x48 325 vs 330, BF16 D = 64 at 65536x48 332 vs
// 334; but BF16 D = 128 at 32768x48 / 65536x48 / 262144x48 335 vs 329 /
// 665 vs 665 / 2,823 vs 2,756, BF16 D = 256 at 32768x48 737 vs 684, FP16
// D = 256 748 vs 680, FP32 D = 64 / 128 at 32768x48 342 vs 338 / 751 vs
// 689, FP32 D = 256 at 7684x48 rows 362 vs 337.
template <Dt T, int D>
constexpr bool prefetch_large() {
  return (T == Dt::f16 && D <= 128) || (T == Dt::bf16 && D == 64);
}

#if GRN_BWD_MIN_WAVES > 0
#define GRN_BWD_OCCUPANCY __attribute__((amdgpu_waves_per_eu(GRN_BWD_MIN_WAVES)))
#else
#define GRN_BWD_OCCUPANCY
#endif

template <Dt T, int D, int U, int kWaves, int R, int kPrefetch, bool kDet, bool kHold,
          bool kItemFence, int kSwz, bool kFuseFwd>
__global__ void __launch_bounds__(kWaves * kWave) GRN_BWD_OCCUPANCY
bwd_kernel(const u32x4* __restrict__ x, const u32x4* __restrict__ g,
           const u32x4* __restrict__ w, const u32x4* __restrict__ dy,
           u32x4* __restrict__ dx, u32x4* __restrict__ dg, BwdPitch pt,
           float* __restrict__ partial, float* __restrict__ gpart,
           uint32_t* __restrict__ counters, void* __restrict__ dw,
           int dw_fp32, int64_t rows, float eps, int64_t nchunks,
           int64_t group_size, int64_t ngroups, int64_t cstride,
           u32x4* __restrict__ y, uint32_t ypitch, int64_t fwd_ntiles) {
  using S = Shape<T, D>;
  constexpr int kVec = S::kVec;
  constexpr int kThreads = kWaves * kWave;
  constexpr int kStepRows = S::kRows * U;                 // per wave
  static_assert(R % (kWaves * kStepRows) == 0,
                "a chunk must be a whole number of workgroup steps");
  static_assert(D <= kThreads, "one thread per column in the dw sums");
  constexpr int kContrib = kWaves * S::kRows;
  static_assert(kContrib * D >= 4 * kThreads, "LDS of level 1 serves the column sums");
  constexpr int kSlotsNd = nondet_slots(D);
  constexpr bool kLbs = kDet && kPrefetch == 0 && lbs_mid<T, D>();
  __shared__ float red[kContrib][D];
  __shared__ int last_in_group, last_overall;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_index();
  const int col = lane & (S::kLanes - 1);
  const int sub = lane / S::kLanes;
  const int t = threadIdx.x;
  float wf[kVec];
  S::C::unpack(w[col], wf);

  // Level 1 for chunk c: dx and dg of its rows, and the column sums of its
  // dw terms (each lane's rows in step order, then the kContrib lane/wave
  // accumulators of a column in index order); valid in threads 0..D-1.
  auto chunk_partial = [&](int64_t c, BwdOut<U>& held) {
    float acc[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) acc[e] = 0.0f;
    const ChunkBlocks cb = chunk_blocks<R, kWaves * kStepRows, kSwz>(c, nchunks);
    if (cb.end <= rows) {
      bwd_chunk<T, D, U, kWaves, R, kPrefetch, kHold, kLbs, true>(
          x, g, dy, dx, dg, pt, wf, eps, cb.row0, cb.stride, rows, wave, lane, acc, held);
    } else {
      bwd_chunk<T, D, U, kWaves, R, kPrefetch, kHold, kLbs, false>(
          x, g, dy, dx, dg, pt, wf, eps, cb.row0, cb.stride, rows, wave, lane, acc, held);
    }
    if (can_overflow<T, D>() && wave_any_nan(acc[0])) {
      bwd_chunk_fixup<T, D, U, kWaves, R, kHold, false>(x, g, dy, dx, dg, pt, wf, eps, cb.row0,
                                                        cb.stride, rows, wave, lane, acc, held);
    }
    const int contrib = wave * S::kRows + sub;
#pragma unroll
    for (int e = 0; e < kVec; ++e) red[contrib][col * kVec + e] = acc[e];
    __syncthreads();
    float v = 0.0f;
    if (t < D) {
#pragma unroll
      for (int k = 0; k < kContrib; ++k) v += red[k][t];
    }
    return v;
  };

  // Work items: chunks [0, nchunks - K), then 2K claim items that take the
  // last K chunks at run time (claim_chunks(); K = 0 for the
  // non-deterministic dw and for small grids), then (deterministic dw) one
  // reducer item per group, which arrives at its group's counter like a
  // chunk but carries no partial.  Being last in the grid, reducers usually
  // arrive after all of their group's chunks, so most group sums run once
  // the streaming is done instead of amid it.
  const int64_t K = claim_chunks(kDet, nchunks);
  const int64_t nstatic = nchunks - K;
  const int64_t nwork = nchunks + K + (kDet && kReducers ? ngroups : 0);
  __shared__ uint32_t claimed;
  // kFuseFwd: after every backward item come the forward's tiles (the
  // recomputed forward of the checkpointed step, which the backward does not
  // read: it recomputes r from x), one tile of two row groups per wave (the
  // forward's tile below 128 MiB), so that they fill the slots the
  // backward's last workgroups leave idle.
  const int64_t nall = nwork + (kFuseFwd ? (fwd_ntiles + kWaves - 1) / kWaves : 0);
  for (int64_t item = blockIdx.x; item < nall; item += gridDim.x) {
    if constexpr (kFuseFwd) {
      if (item >= nwork) {
        constexpr int kFwdTileRows = S::kRows * 2;
        const int64_t tile = (item - nwork) * kWaves + wave;
        if (tile < fwd_ntiles) {
          const FwdPitch fp{pt.x, pt.g, ypitch};
          const int64_t row0 = tile * kFwdTileRows;
          const u32x4 w_raw = w[col];
          if (row0 + kFwdTileRows <= rows) {
            fwd_tile<T, D, 2, true>(x + row0 * fp.x, g + row0 * fp.g, y + row0 * fp.y, fp,
                                    w_raw, eps, lane, kFwdTileRows);
          } else {
            fwd_tile<T, D, 2, false>(x + row0 * fp.x, g + row0 * fp.g, y + row0 * fp.y, fp,
                                     w_raw, eps, lane, (int)(rows - row0));
          }
        }
        continue;
      }
    }
    // A compiler-only fence at the top of each work item (kItemFence): the
    // non-deterministic kernel then needs 184-205 VGPRs instead of 224-256
    // (two waves per SIMD instead of one at D = 256 and for FP32 at D =
    // 128), and runs faster below 256 MiB tensors but 1.5-3.5 % slower above
    // (measured), where it goes without.  The deterministic kernel is
    // unchanged by it.
    if constexpr (kItemFence) asm volatile("" ::: "memory");
    int64_t grp = item - nchunks - K;  // for a reducer item
    int64_t c = -1;                    // the chunk of this item, if any
    if (item < nstatic) {
      c = item;
    } else if (item < nstatic + 2 * K) {
      // A claim item: each of the 2K increments the counter once, so
      // values 0 .. K-1 go to K distinct items and every tail chunk is
      // taken exactly once; the item that makes the last increment returns
      // the counter to zero, after which nothing in this launch touches it.
      if (t == 0) {
        const uint32_t v = __hip_atomic_fetch_add(&counters[kClaimCounter], 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        if (v == (uint32_t)(2 * K - 1))
          __hip_atomic_store(&counters[kClaimCounter], 0u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        claimed = v;
      }
      __syncthreads();
      const uint32_t v = claimed;
      __syncthreads();  // read by all before a later item writes it again
      if (v >= (uint32_t)K) continue;  // the tail is gone
      c = nstatic + v;
    }
    if (c >= 0) {
      // With kHold, the dx and dg stores of the chunk's last step are held
      // back until this wave's wait for its partial's store (below) is over:
      // that wait covers every store the wave has issued, and the freshest
      // ones would take longest.
      BwdOut<U> held;
      const float v = chunk_partial(c, held);
      if constexpr (!kDet) {
        // Non-deterministic dw: the chunk sum is added with FP64 atomics
        // into one of kSlotsNd accumulators (chunk c uses slot c mod slots,
        // so concurrent chunks hit different addresses); the last chunk to
        // arrive adds the slots, rounds once to FP32 and returns them to
        // zero.  The order of the atomic adds varies from run to run; FP64
        // keeps its effect far below FP32 rounding, but the bits of dw are
        // not guaranteed to repeat.
        double* accum = reinterpret_cast<double*>(reinterpret_cast<char*>(counters) +
                                                  kNondetAccumByte);
        if (t < D) {
          __hip_atomic_fetch_add(accum + (c % kSlotsNd) * D + t, (double)v, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
          wait_memory();
        }
        if constexpr (kHold) bwd_store_held<S, U>(held, dx, dg, pt, lane);
        __syncthreads();
        if (t == 0)
          last_overall = __hip_atomic_fetch_add(&counters[kOverallCounter], 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT) ==
                         (uint32_t)(nchunks - 1);
        __syncthreads();
        if (last_overall) {
          if (t < D) {
            double slot[kSlotsNd];
#pragma unroll
            for (int k = 0; k < kSlotsNd; ++k)
              slot[k] = __hip_atomic_load(accum + k * D + t, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
            double total = 0.0;
#pragma unroll
            for (int k = 0; k < kSlotsNd; ++k) total += slot[k];
            store_dw<T>(dw, dw_fp32, t, (float)total);
#pragma unroll
            for (int k = 0; k < kSlotsNd; ++k)
              __hip_atomic_store(accum + k * D + t, 0.0, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
          }
          if (t == 0)
            __hip_atomic_store(&counters[kOverallCounter], 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        continue;
      }
      if (t < D) {
        store_coherent(partial + c * D + t, v);
        wait_memory();  // the partial is complete before anyone arrives
      }
      if constexpr (kHold) bwd_store_held<S, U>(held, dx, dg, pt, lane);
      __syncthreads();
      grp = c / group_size;
    }

    // Level 2: the last arrival at group grp's counter (its chunks, plus its
    // reducer item) sums the group.
    const int64_t gbeg = grp * group_size;
    const int64_t gcnt = (nchunks - gbeg) < group_size ? (nchunks - gbeg) : group_size;
    const uint32_t arrivals = (uint32_t)gcnt + (kReducers ? 1u : 0u);
    if (t == 0)
      last_in_group = __hip_atomic_fetch_add(&counters[grp * cstride], 1u, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT) == arrivals - 1u;
    __syncthreads();
    if (last_in_group) {
      float* lds = &red[0][0];
      const float gsum = column_sum_fixed<kThreads, D>(partial + gbeg * D, gcnt, lds);
      if (t < D) store_coherent(gpart + grp * D + t, gsum);
      if (t == 0)
        __hip_atomic_store(&counters[grp * cstride], 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      wait_memory();
      __syncthreads();
      // Level 3: the workgroup that completes the last group sums them all.
      if (t == 0)
        last_overall = __hip_atomic_fetch_add(&counters[kOverallCounter], 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT) ==
                       (uint32_t)(ngroups - 1);
      __syncthreads();
      if (last_overall) {
        const float total = column_sum_fixed<kThreads, D>(gpart, ngroups, lds);
        if (t < D) store_dw<T>(dw, dw_fp32, t, total);
        if (t == 0)
          __hip_atomic_store(&counters[kOverallCounter], 0u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
  }
}

// rows = 0: dw is an empty sum.
template <Dt T>
__global__ void __launch_bounds__(kMaxD)
dw_zero_kernel(void* __restrict__ dw, int dw_fp32) {
  store_dw<T>(dw, dw_fp32, threadIdx.x, 0.0f);
}

// Zero the arrival counters at the front of a workspace.
__global__ void __launch_bounds__(kBlock)
counters_zero_kernel(uint32_t* __restrict__ counters) {
  for (int k = threadIdx.x; k < kCounterWords; k += kBlock) counters[k] = 0u;
}

// --------------------------------------------------------------------------
// Launchers.

namespace {

// Tile size of the forward by tensor size (results do not depend on it):
// 4 row groups per tile stream tensors of 128 MiB to 1 GiB faster (65536x48:
// 393 -> 378 us), 2 keep more waves in flight on small ones (1031x48: 9.4
// -> 8.7 us) and suit the largest (GRN_FWD_HUGE_BYTES).
constexpr int kFwdU = GRN_FWD_U;
constexpr int kFwdULarge = GRN_FWD_U_LARGE;
constexpr int kBwdWaves = GRN_BWD_WAVES;

// A dispatch counts work-items in 32 bits, so a grid of workgroups of at
// most 256 threads stays below 2^24 of them; the kernels' grid-stride loops
// cover any remaining work.
constexpr int64_t kMaxGrid = (int64_t{1} << 24) - 1;

int64_t cap_grid(int64_t want, int max_wg) {
  int64_t grid = want;
  if (max_wg > 0 && grid > max_wg) grid = max_wg;
  if (grid > kMaxGrid) grid = kMaxGrid;
  return grid < 1 ? 1 : grid;
}

template <Dt T>
using DtTag = std::integral_constant<Dt, T>;
template <int D>
using DTag = std::integral_constant<int, D>;

// Calls f(DtTag, DTag) for the element type and row width of a call (the
// C-ABI layer has checked both).
template <class F>
hipError_t with_shape(int dtype, int D, F&& f) {
  auto by_width = [&](auto t) -> hipError_t {
    switch (D) {
      case 64: return f(t, DTag<64>{});
      case 128: return f(t, DTag<128>{});
      case 256: return f(t, DTag<256>{});
      default: return hipErrorInvalidValue;
    }
  };
  switch (dtype) {
    case (int)Dt::bf16: return by_width(DtTag<Dt::bf16>{});
    case (int)Dt::f16: return by_width(DtTag<Dt::f16>{});
    case (int)Dt::f32: return by_width(DtTag<Dt::f32>{});
    default: return hipErrorInvalidValue;
  }
}

constexpr int vec_of(int dtype) { return dtype == (int)Dt::f32 ? 4 : 8; }

}  // namespace

BwdLayout bwd_layout(int64_t rows, int32_t D, int32_t esize) {
  BwdLayout L;
  if (rows <= 0) {
    L.bytes = kCounterBytes;
    return L;
  }
  // The largest layout has the smallest chunks: those of the widest rows.
  L.chunk_rows = chunk_rows_for(D * (esize > 0 ? esize : 4));
  L.nchunks = (rows + L.chunk_rows - 1) / L.chunk_rows;
  int64_t gs = 1;
  while (gs * gs < L.nchunks) ++gs;  // ceil(sqrt(nchunks)), at most 4096
  L.group_size = gs;
  L.ngroups = (L.nchunks + gs - 1) / gs;
  // Spread the group counters over separate cache lines where they fit:
  // every chunk's arrival is an atomic on its group's counter, and packed
  // counters made the atomics of neighbouring groups queue behind each
  // other (7684x48 backward: 86 -> 84 us).
  L.counter_stride = kMaxCounterStride;
  while (L.counter_stride > 1 && L.counter_stride * L.ngroups > kGroupCounterWords)
    L.counter_stride /= 2;
  L.partial_off = kCounterBytes;
  L.gpart_off = L.partial_off + (size_t)L.nchunks * D * sizeof(float);
  L.bytes = L.gpart_off + (size_t)L.ngroups * D * sizeof(float);
  return L;
}

hipError_t launch_fwd(const void* x, const void* g, const void* w, void* y,
                      const RowStrides& st, int64_t rows, int32_t D, int32_t dtype,
                      float eps, int max_wg, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int vec = vec_of(dtype);
  const FwdPitch pt{(uint32_t)(st.x / vec), (uint32_t)(st.g / vec), (uint32_t)(st.y / vec)};
  const int64_t tensor_bytes = rows * (int64_t)D * (16 / vec);
  const bool large = tensor_bytes >= (int64_t)GRN_FWD_LARGE_BYTES &&
                     tensor_bytes < (int64_t)GRN_FWD_HUGE_BYTES;
  return with_shape(dtype, D, [&](auto tt, auto dd) {
    constexpr Dt T = decltype(tt)::value;
    constexpr int DD = decltype(dd)::value;
    auto launch = [&](auto u, auto waves) {
      constexpr int kU = decltype(u)::value;
      constexpr int kW = decltype(waves)::value;
      constexpr int kTileRows = Shape<T, DD>::kRows * kU;
      const int64_t ntiles = (rows + kTileRows - 1) / kTileRows;
      const int64_t want = (ntiles + kW - 1) / kW;
      const int64_t grid = cap_grid(want, max_wg);
      hipLaunchKernelGGL((fwd_kernel<T, DD, kU, kW>), dim3((unsigned)grid), dim3(kW * kWave), 0,
                         s, static_cast<const u32x4*>(x), static_cast<const u32x4*>(g),
                         static_cast<const u32x4*>(w), static_cast<u32x4*>(y), pt, rows, eps,
                         ntiles);
    };
    if (large) {
      launch(std::integral_constant<int, kFwdULarge>{},
             std::integral_constant<int, GRN_FWD_WAVES_LARGE>{});
    } else {
      launch(std::integral_constant<int, kFwdU>{}, std::integral_constant<int, GRN_FWD_WAVES>{});
    }
    return hipGetLastError();
  });
}

bool ckpt_fuses_forward(int64_t rows, int32_t D, int32_t dtype, int deterministic) {
  const int64_t tensor_bytes = rows * (int64_t)D * (16 / vec_of(dtype));
  return deterministic != 0 && rows > 0 && tensor_bytes < GRN_BWD_SMALL_BYTES;
}

hipError_t launch_bwd(const void* x, const void* g, const void* w,
                      const void* dy, void* dx, void* dg, void* dw,
                      int dw_fp32, int deterministic, void* workspace,
                      const RowStrides& st, int64_t rows, int32_t D, int32_t dtype,
                      float eps, int max_wg, hipStream_t s, void* fused_y) {
  if (fused_y != nullptr && !ckpt_fuses_forward(rows, D, dtype, deterministic))
    return hipErrorInvalidValue;
  const int vec = vec_of(dtype);
  const BwdLayout L = bwd_layout(rows, D, 16 / vec);
  const BwdPitch pt{(uint32_t)(st.x / vec), (uint32_t)(st.g / vec),
                    (uint32_t)(st.dy / vec), (uint32_t)(st.dx / vec),
                    (uint32_t)(st.dg / vec)};
  char* ws = static_cast<char*>(workspace);
  const int64_t tensor_bytes = rows * (int64_t)D * (16 / vec);
  const int64_t nwork = L.nchunks + claim_chunks(deterministic != 0, L.nchunks) +
                       (deterministic && kReducers ? L.ngroups : 0);
  return with_shape(dtype, D, [&](auto tt, auto dd) {
    constexpr Dt T = decltype(tt)::value;
    constexpr int DD = decltype(dd)::value;
    constexpr int kR = chunk_rows_for(DD * 16 / Shape<T, DD>::kVec);
    constexpr int kFwdTileRows = Shape<T, DD>::kRows * 2;
    const int64_t fwd_ntiles = fused_y ? (rows + kFwdTileRows - 1) / kFwdTileRows : 0;
    const int64_t grid = cap_grid(nwork + (fwd_ntiles + kBwdWaves - 1) / kBwdWaves, max_wg);
    if (L.nchunks == 0) {
      hipLaunchKernelGGL(dw_zero_kernel<T>, dim3(1), dim3(DD), 0, s, dw, dw_fp32);
      return hipGetLastError();
    }
    auto launch = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kBwdWaves * kWave), 0, s,
                         static_cast<const u32x4*>(x), static_cast<const u32x4*>(g),
                         static_cast<const u32x4*>(w), static_cast<const u32x4*>(dy),
                         static_cast<u32x4*>(dx), static_cast<u32x4*>(dg), pt,
                         reinterpret_cast<float*>(ws + L.partial_off),
                         reinterpret_cast<float*>(ws + L.gpart_off),
                         reinterpret_cast<uint32_t*>(ws), dw, dw_fp32, rows, eps,
                         L.nchunks, L.group_size, L.ngroups, L.counter_stride,
                         static_cast<u32x4*>(fused_y), (uint32_t)(st.y / vec), fwd_ntiles);
    };
    // Shapes measured fastest per size (1031x48 is "small", 7684x48 and up
    // "mid"; tensors of 256 MiB and more take the prefetching shape only
    // where prefetch_large() says so); the non-deterministic kernel has one
    // shape, with the item fence below 256 MiB tensors.
    if (!deterministic) {
      if (tensor_bytes < GRN_BWD_LARGE_BYTES) {
        launch(bwd_kernel<T, DD, GRN_BWD_U_ND, kBwdWaves, kR, GRN_BWD_ND_PREFETCH, false, false,
                          true, GRN_BWD_SWZ, false>);
      } else {
        launch(bwd_kernel<T, DD, GRN_BWD_U_ND, kBwdWaves, kR, GRN_BWD_ND_PREFETCH, false, false,
                          false, GRN_BWD_SWZ, false>);
      }
    } else if (tensor_bytes < GRN_BWD_SMALL_BYTES) {
      if (fused_y != nullptr) {
        launch(bwd_kernel<T, DD, GRN_BWD_U_SMALL, kBwdWaves, kR, GRN_BWD_PF_SMALL, true, false,
                          false, GRN_BWD_SWZ, true>);
      } else {
        launch(bwd_kernel<T, DD, GRN_BWD_U_SMALL, kBwdWaves, kR, GRN_BWD_PF_SMALL, true, false,
                          false, GRN_BWD_SWZ, false>);
      }
    } else if (tensor_bytes < GRN_BWD_LARGE_BYTES || !prefetch_large<T, DD>()) {
      launch(bwd_kernel<T, DD, GRN_BWD_U_MID, kBwdWaves, kR, GRN_BWD_PF_MID, true, false,
                        false, GRN_BWD_SWZ, false>);
    } else {
      launch(bwd_kernel<T, DD, GRN_BWD_U_LARGE, kBwdWaves, kR, GRN_BWD_PF_LARGE, true,
                        hold_large<T, DD>(), false, 0, false>);
    }
    return hipGetLastError();
  });
}

hipError_t launch_counters_zero(void* workspace, hipStream_t s) {
  hipLaunchKernelGGL(counters_zero_kernel, dim3(1), dim3(kBlock), 0, s,
                     static_cast<uint32_t*>(workspace));
  return hipGetLastError();
}

}  // namespace grn
