// Device-side building blocks shared by the PISA kernels (gfx950 / CDNA4).
//
// Matrix products run on the 32x32 MFMA shapes of CDNA4: for bf16 operands
// v_mfma_f32_32x32x16_bf16 (8 bf16 per lane per operand), for fp32 operands
// four v_mfma_f32_32x32x2_f32 per 16-byte chunk. For both, with lane l of a
// 64-wide wavefront and lane half h = l / 32:
//   A operand  : row l % 32,   KW contraction elements of half h
//   B operand  : column l % 32, the same KW contraction elements
//   accumulator: 16 fp32 registers r, row 8*(r/4) + 4*h + r%4, column l % 32
// Every operand is moved as one 16-byte chunk per lane ("chunk"): KW = 8 bf16
// or 4 fp32 values. Because the order of a contraction is free, each chunk
// covers contraction indices chosen so that both operands can be read with
// plain 16-byte loads:
//   contraction over the head dimension d (Sᵀ = K Qᵀ, Uᵀ = H̄ᵀ Qᵀ):
//     chunk c, half h, element e  <->  d = 2*KW*c + KW*h + e
//   contraction over keys (Oᵀ = Vᵀ Pᵀ, G = Kᵀ V), per 32 keys:
//     chunk c, half h, element e  <->  key vkey(KW*c + e, h)
// The second rule makes the key order of a chunk equal to the row order of the
// accumulator registers KW*c .. KW*c+KW-1, so the softmax weights P computed in
// Sᵀ's accumulator layout are already a B operand for the Vᵀ Pᵀ product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pisa_internal.h"

namespace pisa {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;   // wavefront width
constexpr int kSub = 64;    // keys per packed sub-tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Key (0..31) held in accumulator register r by lane half h.
__host__ __device__ constexpr int vkey(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

template <typename T>
struct Op;

template <>
struct Op<bf16> {
  static constexpr int KW = 8;
  __device__ static inline void mma(f32x16& c, const uint4& a, const uint4& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // Round KW fp32 values to the element type (round to nearest even).
  __device__ static inline uint4 pack(const float* x) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)x[e];
    return __builtin_bit_cast(uint4, v);
  }
  // The KW values of a packed chunk, widened exactly to fp32 (element 2i in
  // the low half of word i).
  __device__ static inline void unpack(const uint4& c, float* x) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static inline float to_f32(bf16 x) { return (float)x; }
  __device__ static inline bf16 from_f32(float x) { return (bf16)x; }
  // acc + the sum of the KW rounded values held in one packed chunk
  __device__ static inline float rowsum(const uint4& c, float acc) {
    typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, c.x), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, c.y), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, c.z), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, c.w), one, acc, false);
    return acc;
  }
  // acc + the dot product of two packed chunks (fp32 products and sums)
  __device__ static inline float dot(const uint4& x, const uint4& y, float acc) {
    typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x.x), __builtin_bit_cast(bf16x2, y.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x.y), __builtin_bit_cast(bf16x2, y.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x.z), __builtin_bit_cast(bf16x2, y.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x.w), __builtin_bit_cast(bf16x2, y.w), acc, false);
    return acc;
  }
};

template <>
struct Op<float> {
  static constexpr int KW = 4;
  __device__ static inline void mma(f32x16& c, const uint4& a, const uint4& b) {
    const f32x4 av = __builtin_bit_cast(f32x4, a);
    const f32x4 bv = __builtin_bit_cast(f32x4, b);
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[e], bv[e], c, 0, 0, 0);
  }
  __device__ static inline uint4 pack(const float* x) {
    f32x4 v = {x[0], x[1], x[2], x[3]};
    return __builtin_bit_cast(uint4, v);
  }
  __device__ static inline void unpack(const uint4& c, float* x) {
    const f32x4 v = __builtin_bit_cast(f32x4, c);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = v[e];
  }
  __device__ static inline float to_f32(float x) { return x; }
  __device__ static inline float from_f32(float x) { return x; }
  __device__ static inline float rowsum(const uint4& c, float acc) {
    const f32x4 v = __builtin_bit_cast(f32x4, c);
    return acc + ((v[0] + v[1]) + (v[2] + v[3]));
  }
  __device__ static inline float dot(const uint4& x, const uint4& y, float acc) {
    const f32x4 a = __builtin_bit_cast(f32x4, x), b = __builtin_bit_cast(f32x4, y);
    return fmaf(a[3], b[3], fmaf(a[2], b[2], fmaf(a[1], b[1], fmaf(a[0], b[0], acc))));
  }
};

// Geometry of the packed, operand-ordered copies of one (batch, head).
//  K-format sub-tile (64 keys x D): chunk (w, c) of lane l at byte
//      ((w*NC + c)*64 + l)*16, key 32*w + l%32, d = 2*KW*c + KW*(l/32) + e.
//  V-format sub-tile (Vᵀ of 64 keys x D): chunk (w, dt, c) of lane l at byte
//      (((w*DT + dt)*CPK + c)*64 + l)*16, d = 32*dt + l%32,
//      key 32*w + vkey(KW*c + e, l/32).
//  H̄ᵀ (D x D): chunk (et, c) of lane l at byte ((et*NC + c)*64 + l)*16,
//      element e' = H̄[d = 2*KW*c + KW*(l/32) + e'][32*et + l%32].
template <typename T, int D>
struct Geo {
  static constexpr int KW = Op<T>::KW;
  static constexpr int ESZ = (int)sizeof(T);
  static constexpr int NC = D / (2 * KW);     // chunks per contraction over D
  static constexpr int DT = D / 32;           // 32-wide tiles over D
  static constexpr int CPK = 32 / (2 * KW);   // chunks per 32-key contraction
  static constexpr int SUB_BYTES = kSub * D * ESZ;
  static constexpr int ROW_BYTES = D * ESZ;
  static constexpr int CPR = ROW_BYTES / 16;  // 16-byte chunks per row
};

// Byte offset, inside a K-format sub-tile, of element (key kk in 0..63, d).
template <typename T, int D>
__host__ __device__ constexpr int kfmt_offset(int kk, int d) {
  using G = Geo<T, D>;
  const int w = kk >> 5, lane = ((d % (2 * G::KW)) / G::KW) * 32 + (kk & 31);
  const int c = d / (2 * G::KW), e = d % G::KW;
  return (((w * G::NC + c) * kWave + lane) * G::KW + e) * G::ESZ;
}

// Byte offset, inside a V-format sub-tile, of element (key kk in 0..63, d).
template <typename T, int D>
__host__ __device__ constexpr int vfmt_offset(int kk, int d) {
  using G = Geo<T, D>;
  const int w = kk >> 5, k32 = kk & 31;
  const int g = k32 >> 3, h = (k32 >> 2) & 1, rr = k32 & 3;
  const int r = 4 * g + rr;  // accumulator register holding this key
  const int c = r / G::KW, e = r % G::KW;
  const int dt = d >> 5, lane = h * 32 + (d & 31);
  return ((((w * G::DT + dt) * G::CPK + c) * kWave + lane) * G::KW + e) * G::ESZ;
}

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

}  // namespace pisa
