// Device-side helpers shared by the gfx950 kernels: 16-bit element types,
// MFMA operand vectors, conversions and the per-token sequence geometry.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfag {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// Element traits: storage is uint16_t; MFMA operands are 8 elements per lane.
struct BF16 {
  typedef bf16x8 vec8;
  static __device__ __forceinline__ float to_f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }
  static __device__ __forceinline__ uint16_t from_f(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
  static __device__ __forceinline__ f32x4 mfma(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // 16x16x16: 4 elements per lane (k = 4 * (lane / 16) .. + 3)
  typedef s16x4 vec4;
  static __device__ __forceinline__ f32x4 mfma16(vec4 a, vec4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
};

struct FP16 {
  typedef f16x8 vec8;
  static __device__ __forceinline__ float to_f(uint16_t u) { return (float)__builtin_bit_cast(_Float16, u); }
  static __device__ __forceinline__ uint16_t from_f(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
  static __device__ __forceinline__ f32x4 mfma(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  typedef f16x4 vec4;
  static __device__ __forceinline__ f32x4 mfma16(vec4 a, vec4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
};

template <typename V>
__device__ __forceinline__ V as_vec8(uint4 u) { return __builtin_bit_cast(V, u); }

template <typename V>
__device__ __forceinline__ V zero_vec8() { return __builtin_bit_cast(V, make_uint4(0, 0, 0, 0)); }

// Index of the calling wave in its workgroup as a wave-uniform value: through
// readfirstlane the compiler keeps it, and what is derived from it, in scalar
// registers and branches on it with scalar instructions.
__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Transposing LDS read of gfx950 (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane L supplies the address of 4 consecutive 16-bit elements; calling
// that 16x4 block M[L][e], lane j of the group receives M[4i + j/4][j%4] for
// i = 0..3.  With lane L addressing row (r0 + L/4), columns c0 + 4*(L%4) .. +3
// of a row-major matrix X, lane j receives X[r0 + i][c0 + j], i = 0..3: four
// consecutive rows of one column, the shape an MFMA operand needs when the
// contraction runs along X's rows.
__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

template <typename V>
__device__ __forceinline__ V join_tr(s16x4 a, s16x4 b) {
  s16x8 r = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(V, r);
}

// Geometry of one query token (BSND: fixed S1/S2; TND: per-sequence offsets
// produced by the offsets kernel, B+1 entries each).
struct TokenGeo {
  int64_t kv_base;  // first global key row of the token's sequence
  int32_t Lk;       // key length of the sequence
  int32_t bound;    // largest valid position under sparseMode 3 (t_loc + Lk - Lq)
  bool ok;          // false for tokens past the declared sequence lengths
};

__device__ __forceinline__ TokenGeo token_geo(int64_t t, int32_t layout, int64_t S1, int64_t S2,
                                              const int32_t* q_off, const int32_t* kv_off, int32_t B) {
  TokenGeo g;
  if (layout == 0) {
    const int64_t b = t / S1;
    const int64_t tl = t - b * S1;
    g.kv_base = b * S2;
    g.Lk = (int32_t)S2;
    g.bound = (int32_t)(tl + S2 - S1);
    g.ok = true;
    return g;
  }
  // binary search: largest b with q_off[b] <= t
  int lo = 0, hi = B;  // q_off[0] = 0 <= t
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (q_off[mid] <= t) lo = mid;
    else hi = mid;
  }
  const int64_t qs = q_off[lo], qe = q_off[lo + 1];
  g.ok = t < qe;
  g.kv_base = kv_off[lo];
  g.Lk = kv_off[lo + 1] - kv_off[lo];
  g.bound = (int32_t)((t - qs) + g.Lk - (qe - qs));
  return g;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace sfag
