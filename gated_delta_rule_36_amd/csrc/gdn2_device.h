// Device-side helpers shared by the GDN-2 HIP kernels (gfx950 / CDNA4 only).
//
//   * element types: __bf16 (hardware RNE conversion, v_cvt_pk_bf16_f32) and float;
//   * 16-byte global / LDS vector access;
//   * MFMA traits for the two tile instructions the kernels use:
//       bf16: v_mfma_f32_16x16x32_bf16  (8 K-values per lane, K step 32)
//       fp32: v_mfma_f32_16x16x4_f32    (1 K-value per lane,  K step 4)
//     plus a K=16 "small" product used inside the 64x64 triangular inverse:
//       bf16: v_mfma_f32_16x16x16_bf16, fp32: four 16x16x4 steps.
//
// Lane layout of a 16x16 tile product D = A * B on a 64-lane wave (lane l, g = l / 16):
//   A fragment: row (l % 16) of A, K-values [g*KPL, g*KPL + KPL) of the K step;
//   B fragment: column (l % 16) of B, the same K-values;
//   D (and C): column (l % 16), rows 4g .. 4g+3 (4 floats per lane).
// Because D holds 4 consecutive rows per lane, a D tile can be fed back as the B
// operand of a later product provided the A operand reads its K-values in the same
// (permuted) order; `kperm_*` below give that order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn2 {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return static_cast<bf16>(x); }

// Eight consecutive elements of type T, loaded / stored as 16-byte vectors.
template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
  uint4 r;
  __device__ __forceinline__ void load(const bf16* p) { r = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void zero() { r = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void to_float(float* f) const {
    bf16x8 v = __builtin_bit_cast(bf16x8, r);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = static_cast<float>(v[i]);
  }
};
template <> struct Vec8<float> {
  uint4 r0, r1;
  __device__ __forceinline__ void load(const float* p) {
    r0 = reinterpret_cast<const uint4*>(p)[0];
    r1 = reinterpret_cast<const uint4*>(p)[1];
  }
  __device__ __forceinline__ void zero() { r0 = r1 = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void to_float(float* f) const {
    f4 a = __builtin_bit_cast(f4, r0), b = __builtin_bit_cast(f4, r1);
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[i] = a[i]; f[4 + i] = b[i]; }
  }
};

// Store 8 floats as 8 consecutive T values (16 or 32 bytes; destination aligned).
__device__ __forceinline__ void store8(bf16* p, const float* f) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = static_cast<bf16>(f[i]);
  *reinterpret_cast<bf16x8*>(p) = v;
}
__device__ __forceinline__ void store8(float* p, const float* f) {
  reinterpret_cast<f4*>(p)[0] = f4{f[0], f[1], f[2], f[3]};
  reinterpret_cast<f4*>(p)[1] = f4{f[4], f[5], f[6], f[7]};
}

// ---------------------------------------------------------------- MFMA traits
template <typename T> struct Mma;

template <> struct Mma<bf16> {
  static constexpr int KS = 32;   // K per instruction
  static constexpr int KPL = 8;   // K-values per lane
  typedef bf16x8 frag;
  // Fragment from a row-major [row][k] array: KPL contiguous values.
  static __device__ __forceinline__ frag load(const bf16* base, int ld, int row, int k) {
    return *reinterpret_cast<const bf16x8*>(base + row * ld + k);
  }
  // Same, each value multiplied by a per-k factor (8 floats).
  static __device__ __forceinline__ frag load_scaled(const bf16* base, int ld, int row, int k,
                                                      const float* s) {
    bf16x8 v = *reinterpret_cast<const bf16x8*>(base + row * ld + k);
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = static_cast<bf16>(static_cast<float>(v[i]) * s[i]);
    return o;
  }
  // Permuted fragment matching a B operand built from two D tiles (see kperm):
  // K-values {32s + 4g + i, 32s + 16 + 4g + i}, i = 0..3.
  static __device__ __forceinline__ frag load_perm(const bf16* base, int ld, int row, int s,
                                                    int g) {
    const bf16* p = base + row * ld + 32 * s + 4 * g;
    bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
    bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  // Channel index of permuted slot i (for per-k scaling of a permuted fragment).
  static __device__ __forceinline__ int perm_k(int s, int g, int i) {
    return 32 * s + 4 * g + (i & 3) + ((i >> 2) << 4);
  }
  // B fragment for K step s from D tiles (2s, 2s+1).
  static __device__ __forceinline__ frag from_acc(const f4* tiles, int s) {
    const f4 a = tiles[2 * s], b = tiles[2 * s + 1];
    return bf16x8{static_cast<bf16>(a[0]), static_cast<bf16>(a[1]), static_cast<bf16>(a[2]),
                  static_cast<bf16>(a[3]), static_cast<bf16>(b[0]), static_cast<bf16>(b[1]),
                  static_cast<bf16>(b[2]), static_cast<bf16>(b[3])};
  }
  static __device__ __forceinline__ f4 mma(frag a, frag b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // K = 16 product; a and b hold 4 K-values per lane (A row-fragment, B col-fragment).
  typedef bf16x4 frag16;
  static __device__ __forceinline__ f4 mma16(frag16 a, frag16 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4v, a),
                                                     __builtin_bit_cast(short4v, b), c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  static constexpr int KS = 4;
  static constexpr int KPL = 1;
  typedef float frag;
  static __device__ __forceinline__ frag load(const float* base, int ld, int row, int k) {
    return base[row * ld + k];
  }
  static __device__ __forceinline__ frag load_scaled(const float* base, int ld, int row, int k,
                                                      const float* s) {
    return base[row * ld + k] * s[0];
  }
  // K step s covers D tile s/4, slot s%4: K-value 16*(s/4) + 4g + (s%4).
  static __device__ __forceinline__ frag load_perm(const float* base, int ld, int row, int s,
                                                    int g) {
    return base[row * ld + 16 * (s >> 2) + 4 * g + (s & 3)];
  }
  static __device__ __forceinline__ int perm_k(int s, int g, int) {
    return 16 * (s >> 2) + 4 * g + (s & 3);
  }
  static __device__ __forceinline__ frag from_acc(const f4* tiles, int s) {
    return tiles[s >> 2][s & 3];
  }
  static __device__ __forceinline__ f4 mma(frag a, frag b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace gdn2
