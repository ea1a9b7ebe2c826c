// Device helpers shared by the gfx950 kernels of the SiLU-gated RMSNorm.
//
// Data layout the kernels rely on: one row of D = 128 BF16 values is 256
// bytes, i.e. 16 lanes x one 16-byte access of 8 values.  A wave of 64
// lanes therefore touches 4 consecutive rows (1 KiB, fully coalesced) per
// load instruction, and the 16 lanes of one row are exactly one DPP "row"
// of the wave, so a row sum is four DPP steps with no LDS and no barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace grn {

constexpr int kD = 128;                              // row width (values)
constexpr int kVec = 8;                              // BF16 values per lane access
constexpr int kLanesPerRow = kD / kVec;              // 16
constexpr int kWave = 64;                            // CDNA wavefront
constexpr int kRowsPerAccess = kWave / kLanesPerRow; // 4 rows per wave access
constexpr int kBlock = 256;                          // threads per workgroup
constexpr int kWavesPerBlock = kBlock / kWave;       // 4

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 8 BF16 values (packed in 4 dwords, element 2k in the low half of dword k)
// to FP32.  BF16 is the top half of binary32, so this is exact.
__device__ __forceinline__ void unpack_bf16x8(u32x4 p, float (&f)[kVec]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = __uint_as_float(p[k] << 16);
    f[2 * k + 1] = __uint_as_float(p[k] & 0xffff0000u);
  }
}

// Two FP32 values to a BF16 pair, round to nearest even (gfx950 has a
// native packed conversion, v_cvt_pk_bf16_f32, which this lowers to).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ u32x4 pack_bf16x8(const float (&f)[kVec]) {
  u32x4 p;
#pragma unroll
  for (int k = 0; k < 4; ++k) p[k] = pack_bf16x2(f[2 * k], f[2 * k + 1]);
  return p;
}

template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(
      __builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row, the result in all 16 lanes.  Steps:
// swap neighbours, swap pairs (quad_perm), then mirror within 8 and within
// 16 lanes.  Every step adds two values that the partner lane adds in the
// other order, and FP32 addition is commutative, so all 16 lanes end with
// the same bits.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  v += dpp_mov<0x140>(v);  // row_mirror
  return v;
}

// Logistic sigmoid from the hardware exp2 and reciprocal.  For g -> -inf,
// exp overflows to +inf and the reciprocal gives 0; for g -> +inf it gives
// 1: no NaN for any finite g.
__device__ __forceinline__ float sigmoid_fast(float g) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

__device__ __forceinline__ float rsqrt_fast(float v) {
  return __builtin_amdgcn_rsqf(v);
}

}  // namespace grn
