// Matrix-core building blocks shared by the decode and prefill kernels
// (gfx950 MFMA, 16-bit inputs, fp32 accumulation).
#pragma once

#include "common.h"

namespace pkv {

template <typename E>
struct MfmaOps;

template <>
struct MfmaOps<F16> {
  static constexpr bool kSplit = false;
  __device__ static inline f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline f32x4 pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float x, float y) {
    f16x2 h = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, h);
  }
  __device__ static inline float widen_lo(uint32_t v) {
    return (float)__builtin_bit_cast(f16x2, v)[0];
  }
  __device__ static inline float widen_hi(uint32_t v) {
    return (float)__builtin_bit_cast(f16x2, v)[1];
  }
  // acc + both halves of a packed pair (a dot2 against ones)
  __device__ static inline float sum2(uint32_t v, float acc) {
    return __builtin_amdgcn_fdot2(lane_as<f16x2>(v), lane_as<f16x2>(0x3C003C00u), acc, false);
  }
};

template <>
struct MfmaOps<BF16> {
  static constexpr bool kSplit = true;
  __device__ static inline f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static inline f32x4 pv(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a),
                                                     __builtin_bit_cast(bf16x4, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float x, float y) {
    bf16x2 h = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, h);
  }
  __device__ static inline float widen_lo(uint32_t v) { return __uint_as_float(v << 16); }
  __device__ static inline float widen_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
  __device__ static inline float sum2(uint32_t v, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(lane_as<bf16x2>(v), lane_as<bf16x2>(0x3F803F80u), acc,
                                          false);
  }
};

// Two E4M3 codes (bytes 2*kHi, 2*kHi + 1 of w) as a pair of E's 16-bit
// values, element 0 from the lower byte (exact: every code is a 16-bit value)
template <typename E, bool kHi>
__device__ inline uint32_t codes_to_pair(uint32_t w) {
  if constexpr (__is_same(E, F16))
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, kHi));
  else
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, kHi));
}

// {lo16 = 16-bit element e of x, hi16 = element e of y}; e is a constant
// after unrolling
__device__ inline uint32_t pair_of(int e, const uint32_t* x, const uint32_t* y) {
  // v_perm_b32 selector: bytes 0-3 come from the second source, 4-7 from the first
  const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
  return __builtin_amdgcn_perm(y[e >> 1], x[e >> 1], sel);
}

// Head dim of element i < 8 of k-step kk in lane group g4, for the A
// operand (K) and the B operand (Q^T) alike.  16-bit caches: dims 32*kk +
// 8*g4 + i.  8-bit caches: a lane reads 16 contiguous codes at 64*(kk/2) +
// 16*g4 and feeds the first 8 to k-step 2*(kk/2), the next 8 to the step
// after.  Both orders cover every dim once, and a dot product does not
// depend on the order of its terms.
template <typename C>
__device__ constexpr int mfma_dim0(int kk, int g4) {
  return sizeof(typename C::storage) == 1 ? 64 * (kk / 2) + 16 * g4 + 8 * (kk % 2)
                                          : 32 * kk + 8 * g4;
}

}  // namespace pkv
