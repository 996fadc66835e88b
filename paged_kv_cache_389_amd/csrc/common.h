// Device-side building blocks shared by the paged decode kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// Reinterpret one 32-bit lane of a vector.  The element is copied into a
// scalar first: bit-casting a vector element expression directly picks the
// wrong element with this compiler.
template <typename To>
__device__ inline To lane_as(uint32_t x) {
  return __builtin_bit_cast(To, x);
}

// 16-byte global load / store.
__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Element types.  Each describes how a 16-byte vector of the type is read
// into fp32 and how an fp32 result is rounded back (nearest even).
struct F32 {
  using storage = float;
  static constexpr int kVec = 4;  // elements per 16 bytes
  __device__ static inline float dot16(u32x4 a, u32x4 b, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(__uint_as_float(a[i]), __uint_as_float(b[i]), acc);
    return acc;
  }
  __device__ static inline void unpack16(u32x4 a, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(a[i]);
  }
  __device__ static inline storage round(float x) { return x; }
};

struct F16 {
  using storage = _Float16;
  static constexpr int kVec = 8;
  __device__ static inline float dot16(u32x4 a, u32x4 b, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2(lane_as<f16x2>(a[i]), lane_as<f16x2>(b[i]), acc, false);
    return acc;
  }
  __device__ static inline void unpack16(u32x4 a, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x2 h = lane_as<f16x2>(a[i]);
      out[2 * i] = (float)h[0];
      out[2 * i + 1] = (float)h[1];
    }
  }
  __device__ static inline storage round(float x) { return (_Float16)x; }
  // round two floats and pack them into one 32-bit word, x in the low half
  __device__ static inline uint32_t pack2(float x, float y) {
    const f16x2 h = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, h);
  }
};

struct BF16 {
  using storage = __bf16;
  static constexpr int kVec = 8;
  __device__ static inline float dot16(u32x4 a, u32x4 b, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(lane_as<bf16x2>(a[i]), lane_as<bf16x2>(b[i]), acc,
                                            false);
    return acc;
  }
  __device__ static inline void unpack16(u32x4 a, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(a[i] << 16);
      out[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
    }
  }
  __device__ static inline storage round(float x) { return (__bf16)x; }
  __device__ static inline uint32_t pack2(float x, float y) {
    const bf16x2 h = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, h);
  }
};

// 8-bit cache codes in the OCP E4M3 format (sign, 4-bit exponent with bias
// 7, 3-bit fraction; largest finite 448, no infinity), which gfx950 converts
// natively.  Every code is exact in f16, bf16 and f32.  A cache of codes
// carries one float scale per K or V cache, applied outside the dot products.
struct E4M3 {
  using storage = uint8_t;
  static constexpr int kVec = 16;  // codes per 16 bytes
  // the 16 codes as floats, byte i of the vector first
  __device__ static inline void unpack16(u32x4 a, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(a[i], false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(a[i], true);
      out[4 * i] = lo[0];
      out[4 * i + 1] = lo[1];
      out[4 * i + 2] = hi[0];
      out[4 * i + 3] = hi[1];
    }
  }
  // the code of x / scale: float32 quotient, saturated to +-448, nearest
  // even; NaN gives 0x7F
  __device__ static inline uint32_t encode4(float x0, float x1, float x2, float x3, float scale) {
    const float xs[4] = {x0 / scale, x1 / scale, x2 / scale, x3 / scale};
    float c[4];
    uint32_t nan_mask = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = fminf(fmaxf(xs[i], -448.f), 448.f);
      if (xs[i] != xs[i]) nan_mask |= 0xFFu << (8 * i);
    }
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w, true);
    return ((uint32_t)w & ~nan_mask) | (0x7F7F7F7Fu & nan_mask);
  }
};

// Dot product of one lane's 16 bytes of a cache row (type C) with the
// matching query elements (type E, QW 16-byte words).
template <typename E, typename C>
struct KvDot {
  static constexpr int QW = C::kVec * (int)sizeof(typename E::storage) / 16;
  __device__ static inline float dot(u32x4 k, const u32x4* q) {
    if constexpr (__is_same(E, C)) {
      return E::dot16(k, q[0], 0.f);
    } else if constexpr (__is_same(E, F16)) {
      // codes -> f16 pairs (scale 1: exact), then v_dot2 with the query
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k[w], 1.f, false);
        const f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k[w], 1.f, true);
        acc = __builtin_amdgcn_fdot2(lo, lane_as<f16x2>(q[w / 2][2 * (w % 2)]), acc, false);
        acc = __builtin_amdgcn_fdot2(hi, lane_as<f16x2>(q[w / 2][2 * (w % 2) + 1]), acc, false);
      }
      return acc;
    } else if constexpr (__is_same(E, BF16)) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k[w], 1.f, false);
        const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k[w], 1.f, true);
        acc = __builtin_amdgcn_fdot2_f32_bf16(lo, lane_as<bf16x2>(q[w / 2][2 * (w % 2)]), acc,
                                              false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(hi, lane_as<bf16x2>(q[w / 2][2 * (w % 2) + 1]),
                                              acc, false);
      }
      return acc;
    } else {
      // f32 query: codes -> f32, fused multiply-adds
      float kf[16];
      C::unpack16(k, kf);
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc = __builtin_fmaf(kf[i], __uint_as_float(q[i / 4][i % 4]), acc);
      return acc;
    }
  }
};

// Round n floats (n a multiple of 4) to E's storage type and store them at
// p with the widest aligned vector stores (16 bytes for 8 half-width or 4
// single-width elements).
template <typename E, int N>
__device__ inline void store_rounded(typename E::storage* p, const float* x) {
  static_assert(N % 4 == 0, "store_rounded needs a multiple of 4 elements");
  if constexpr (sizeof(typename E::storage) == 4) {
#pragma unroll
    for (int i = 0; i < N; i += 4)
      *reinterpret_cast<f32x4*>(p + i) = f32x4{x[i], x[i + 1], x[i + 2], x[i + 3]};
  } else if constexpr (N % 8 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 8)
      st16(p + i, u32x4{E::pack2(x[i], x[i + 1]), E::pack2(x[i + 2], x[i + 3]),
                        E::pack2(x[i + 4], x[i + 5]), E::pack2(x[i + 6], x[i + 7])});
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 4)
      *reinterpret_cast<u32x2*>(p + i) = u32x2{E::pack2(x[i], x[i + 1]), E::pack2(x[i + 2], x[i + 3])};
  }
}


// Cross-lane moves inside a 16-lane DPP row.
template <int CTRL>
__device__ inline float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Row-pair exchanges of gfx950 (v_permlane16_swap / v_permlane32_swap with
// the same register as both operands).  swap16 returns, in every lane, the
// value of its own 16-lane row and of the partner row (rows 0<->1, 2<->3);
// swap32 the same for the two 32-lane halves.  op(first, second) therefore
// combines each lane with lane ^ 16 (resp. lane ^ 32), with the operands in
// the same order in both partners, so both get bit-identical results.
struct Pair {
  float lo, hi;
};
__device__ inline Pair swap16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ inline Pair swap32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Max / sum over the four 16-lane rows (lanes with equal lane % 16).
__device__ inline float rows_max(float v) {
  Pair p = swap16(v);
  v = fmaxf(p.lo, p.hi);
  p = swap32(v);
  return fmaxf(p.lo, p.hi);
}
__device__ inline float rows_sum(float v) {
  Pair p = swap16(v);
  v = p.lo + p.hi;
  p = swap32(v);
  return p.lo + p.hi;
}

// Sum over aligned groups of N lanes (N a power of two, 1..64); every lane
// of a group receives the group's sum.  Steps inside a 16-lane row use DPP;
// the 32- and 64-lane steps use the row-pair exchanges.
template <int N>
__device__ inline float group_sum(float v) {
  if constexpr (N >= 2) v += dpp<kDppXor1>(v);
  if constexpr (N >= 4) v += dpp<kDppXor2>(v);
  if constexpr (N >= 8) v += dpp<kDppRowHalfMirror>(v);   // quads uniform: mirror == xor 4
  if constexpr (N >= 16) v += dpp<kDppRowMirror>(v);      // halves uniform: mirror == xor 8
  if constexpr (N >= 32) {
    const Pair p = swap16(v);
    v = p.lo + p.hi;
  }
  if constexpr (N >= 64) {
    const Pair p = swap32(v);
    v = p.lo + p.hi;
  }
  return v;
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum / sum over all 64 lanes of a wave; every lane receives it.
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Raw buffer descriptor over `bytes` bytes at a wave-uniform base (four
// scalar registers; word 3 is the GFX9-family raw-buffer format).  Loads
// through it take one VGPR of per-lane byte offset, do their address
// arithmetic in scalar registers, and return zero past `bytes`.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
//
// POL is the load's cache policy: 0 for ordinary loads, kStream for the
// nontemporal bit (lines marked for early eviction).  A plain random gather
// of 4 KiB chunks measured 6.3-6.5 TB/s with it against 5.7-5.9 TB/s
// without, and the decode kernels gain as much: they stream their K/V loads
// unless a batch's sequences share blocks, where a block read by several
// workgroups in one call should stay in the cache.
constexpr int kStream = 2;
template <int POL = 0>
__device__ inline u32x4 bld16(rsrc_t r, uint32_t lane_off, uint32_t const_off) {
  return __builtin_bit_cast(u32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, const_off, POL));
}
template <int POL = 0>
__device__ inline u32x2 bld8(rsrc_t r, uint32_t lane_off, uint32_t const_off) {
  return __builtin_bit_cast(u32x2,
                            __builtin_amdgcn_raw_buffer_load_b64(r, lane_off, const_off, POL));
}
template <int POL = 0>
__device__ inline uint32_t bld4(rsrc_t r, uint32_t lane_off, uint32_t const_off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, lane_off, const_off, POL);
}

// Value of a wave-uniform lane's register (v_readlane with an SGPR index).
__device__ inline int lane_value(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

// Scalar (wave-uniform) copy of a value.
__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Read of an int at a wave-uniform address that nothing writes during the
// kernel, through the constant address space so that it is issued as a
// scalar-memory read: its wait is counted apart from the vector loads
// issued after it, which therefore need not wait for it.
__device__ inline int load_uniform(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}
// Four ints at a 16-byte aligned uniform address, the same way.
__device__ inline i32x4 load_uniform4(const int32_t* p) {
  return *(const __attribute__((address_space(4))) i32x4*)p;
}

}  // namespace pkv
