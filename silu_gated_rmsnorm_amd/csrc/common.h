// Device helpers shared by the gfx950 kernels of the SiLU-gated RMSNorm.
//
// Data layout the kernels rely on: a row of D values is cut into 16-byte
// lane accesses (8 BF16 or FP16 values, or 4 FP32 values), so a row spans
// kLanes = D / values-per-access consecutive lanes and one wave access
// covers 64 / kLanes consecutive rows (1 KiB, fully coalesced).  For the
// main case, D = 128 BF16, that is 16 lanes per row and 4 rows per access,
// and the 16 lanes of a row are exactly one DPP row of the wave.  Row sums
// stay in registers: DPP within 16 lanes, a lane swap beyond.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace grn {

constexpr int kWave = 64;                            // CDNA wavefront
constexpr int kBlock = 256;                          // threads of the counter-zeroing kernel
constexpr int kMaxD = 256;                           // widest supported row

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Element types of the activations and the weight (the numeric values are
// those of GRN_DTYPE_* in the C header).
enum class Dt : int { bf16 = 0, f16 = 1, f32 = 2 };

// Conversions between one 16-byte access and FP32 registers.  Values are
// packed little-endian: element 2k in the low half of dword k for 16-bit
// types.  Narrowing rounds to nearest, ties to even.
template <Dt T>
struct Codec;

template <>
struct Codec<Dt::bf16> {
  static constexpr int kPer = 8;  // values per 16 bytes
  // BF16 is the top half of binary32: widening is exact.
  static __device__ __forceinline__ void unpack(u32x4 p, float (&f)[kPer]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[2 * k] = __uint_as_float(p[k] << 16);
      f[2 * k + 1] = __uint_as_float(p[k] & 0xffff0000u);
    }
  }
  // gfx950 has a native packed conversion, v_cvt_pk_bf16_f32, which this
  // lowers to.
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ u32x4 pack(const float (&f)[kPer]) {
    u32x4 p;
#pragma unroll
    for (int k = 0; k < 4; ++k) p[k] = pack2(f[2 * k], f[2 * k + 1]);
    return p;
  }
  static __device__ __forceinline__ void store1(void* dst, int i, float v) {
    static_cast<uint16_t*>(dst)[i] = (uint16_t)(pack2(v, 0.0f) & 0xffffu);
  }
};

template <>
struct Codec<Dt::f16> {
  static constexpr int kPer = 8;
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ void unpack(u32x4 p, float (&f)[kPer]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // The element goes through a scalar first: a bit_cast applied to the
      // vector element expression itself was compiled as a read of element
      // 0 for every k.
      const uint32_t d = p[k];
      const f16x2 h = __builtin_bit_cast(f16x2, d);
      f[2 * k] = (float)h.x;
      f[2 * k + 1] = (float)h.y;
    }
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    const f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ u32x4 pack(const float (&f)[kPer]) {
    u32x4 p;
#pragma unroll
    for (int k = 0; k < 4; ++k) p[k] = pack2(f[2 * k], f[2 * k + 1]);
    return p;
  }
  static __device__ __forceinline__ void store1(void* dst, int i, float v) {
    static_cast<_Float16*>(dst)[i] = (_Float16)v;
  }
};

template <>
struct Codec<Dt::f32> {
  static constexpr int kPer = 4;
  static __device__ __forceinline__ void unpack(u32x4 p, float (&f)[kPer]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) f[k] = __uint_as_float(p[k]);
  }
  static __device__ __forceinline__ u32x4 pack(const float (&f)[kPer]) {
    u32x4 p;
#pragma unroll
    for (int k = 0; k < 4; ++k) p[k] = __float_as_uint(f[k]);
    return p;
  }
  static __device__ __forceinline__ void store1(void* dst, int i, float v) {
    static_cast<float*>(dst)[i] = v;
  }
};

// How a row of D values of type T sits on the lanes of a wave.
template <Dt T, int D>
struct Shape {
  using C = Codec<T>;
  static constexpr int kVec = C::kPer;              // values per lane access
  static constexpr int kLanes = D / kVec;           // lanes per row
  static constexpr int kRows = kWave / kLanes;      // rows per wave access
  static_assert(D % kVec == 0, "a row is a whole number of 16-byte accesses");
  static_assert(kLanes == 8 || kLanes == 16 || kLanes == 32 || kLanes == 64,
                "a row spans 8, 16, 32 or 64 lanes");
};

template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(
      __builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// v[l] + v[l ^ 16] in every lane l, from gfx950's v_permlane16_swap_b32
// (a VALU lane swap between neighbouring 16-lane rows; no LDS).  Called
// with both operands equal to v, it returns the lower row's value and the
// upper row's value of each pair in every lane of the pair, and they are
// added in that order, so both lanes get the same bits.
__device__ __forceinline__ float add_across16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// v[l] + v[l ^ 32], from v_permlane32_swap_b32 (swaps the wave's halves).
__device__ __forceinline__ float add_across32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over the kLanes lanes of a row, the result in all of them.  Steps:
// swap neighbours, swap pairs (quad_perm), mirror within 8 lanes, mirror
// within 16 lanes (DPP), then adds across 16-lane rows and wave halves
// (lane swaps).  Every step adds two values that the partner lane adds in
// the other order or in the same order, and FP32 addition is commutative,
// so all lanes of a row end with the same bits.  Every lane of the wave
// must be active.
template <int kLanes>
__device__ __forceinline__ float row_sum(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  if constexpr (kLanes >= 16) v += dpp_mov<0x140>(v);  // row_mirror
  if constexpr (kLanes >= 32) v = add_across16(v);
  if constexpr (kLanes >= 64) v = add_across32(v);
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

// Rows whose sum of squares exceeds the FP32 range (entries beyond about
// 1.8e19 at D = 128; BF16 and FP32 storage hold values up to 3.4e38, while
// FP16's largest, 65504, squares to far less) are summed again with every x
// scaled by kOverflowScale = 2^-70, an exact power of two: the scaled
// squares of up to 256 entries of at most 3.4e38 stay below 2^124, and the
// largest entry of such a row (at least 2^60) keeps its scaled square far
// above FP32's underflow.  With x' = 2^-70 x:
//   mean(x^2) + eps = 2^140 (mean(x'^2) + 2^-140 eps)
//   r = 2^-70 r',  r' = rsqrt(mean(x'^2) + 2^-140 eps)
//   mean(dn n) = r' mean(dn x')
constexpr float kOverflowScale = 0x1p-70f;
constexpr float kOverflowScale2 = 0x1p-140f;

// Whether a row sum of squares is not a finite FP32 number (+inf, or NaN
// from a NaN or infinite input).
__device__ __forceinline__ bool overflowed(float ss) { return !(ss <= 0x1.fffffep127f); }

// Whether some lane of the wave holds a NaN in v (wave-uniform).
__device__ __forceinline__ bool wave_any_nan(float v) {
  return __builtin_amdgcn_ballot_w64(v != v) != 0;
}

}  // namespace grn
