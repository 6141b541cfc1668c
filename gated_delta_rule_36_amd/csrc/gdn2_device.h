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
typedef float f2v __attribute__((ext_vector_type(2)));

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
  // A gate shared by every channel: load_one fetches the one value (nothing waits on it
  // there, so a prefetch stays in flight); splat broadcasts it to all 8 lanes when the
  // vector is consumed.
  __device__ __forceinline__ void load_one(const bf16* p) {
    r.x = *reinterpret_cast<const unsigned short*>(p);
  }
  __device__ __forceinline__ void splat() {
    const uint32_t h = r.x & 0xffffu;
    const uint32_t x = h | (h << 16);
    r = make_uint4(x, x, x, x);
  }
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
  __device__ __forceinline__ void load_one(const float* p) {
    r0.x = *reinterpret_cast<const uint32_t*>(p);
  }
  __device__ __forceinline__ void splat() {
    const uint32_t x = r0.x;
    r0 = r1 = make_uint4(x, x, x, x);
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

// Store 8 consecutive logical K-values k0..k0+7 (k0 % 8 == 0) into a phi-ordered row:
// bf16 rows are phi-permuted (two 8-byte pieces), fp32 rows are in logical order.
__device__ __forceinline__ void store8_phi(bf16* row, int k0, const float* f) {
  const int p0 = (k0 & ~31) | (((k0 >> 2) & 3) << 3) | (((k0 >> 4) & 1) << 2);
  *reinterpret_cast<bf16x4*>(row + p0) = bf16x4{static_cast<bf16>(f[0]), static_cast<bf16>(f[1]),
                                                static_cast<bf16>(f[2]), static_cast<bf16>(f[3])};
  *reinterpret_cast<bf16x4*>(row + p0 + 8) = bf16x4{static_cast<bf16>(f[4]), static_cast<bf16>(f[5]),
                                                    static_cast<bf16>(f[6]), static_cast<bf16>(f[7])};
}
__device__ __forceinline__ void store8_phi(float* row, int k0, const float* f) { store8(row + k0, f); }

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
  // Storage permutation of a K axis inside each 32-wide block: logical
  // k = 32s + 16h + 4g + i is stored at 32s + 8g + 4h + i, so the 8 K-values of a permuted
  // fragment (K step s, lane group g) are 8 contiguous elements: one 16-byte LDS read.
  static __device__ __forceinline__ int phi(int k) {
    return (k & ~31) | (((k >> 2) & 3) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
  }
  static __device__ __forceinline__ int phi_inv(int p) {
    return (p & ~31) | (((p >> 2) & 1) << 4) | (((p >> 3) & 3) << 2) | (p & 3);
  }
  // Permuted fragment from a phi-stored [row][k] array.
  static __device__ __forceinline__ frag load_phi(const bf16* base, int ld, int row, int s, int g) {
    return *reinterpret_cast<const bf16x8*>(base + row * ld + 32 * s + 8 * g);
  }
  // Same from a token-transposed (swizzled) array stored in phi order along the tokens.
  static __device__ __forceinline__ frag load_phi_t(const bf16* base, int ld, int c, int s, int g);
  // load_perm from a token-transposed (swizzled) array; `c` is the logical row.
  static __device__ __forceinline__ frag load_perm_t(const bf16* base, int ld, int c, int s,
                                                      int g);
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
  static __device__ __forceinline__ frag load_perm_t(const float* base, int ld, int c, int s,
                                                      int g);
  static __device__ __forceinline__ int phi(int k) { return k; }
  static __device__ __forceinline__ int phi_inv(int p) { return p; }
  static __device__ __forceinline__ frag load_phi(const float* base, int ld, int row, int s, int g) {
    return load_perm(base, ld, row, s, g);
  }
  static __device__ __forceinline__ frag load_phi_t(const float* base, int ld, int c, int s, int g) {
    return load_perm_t(base, ld, c, s, g);
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

// K = 16 product with B taken from a D tile (4 consecutive rows per lane = the B
// fragment of a 16-deep product) and A row `arow` (16 values of row l%16 of A, in LDS).
__device__ __forceinline__ f4 mma16_acc(const bf16* arow, int g, f4 bacc, f4 c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(arow + 4 * g);
  const bf16x2 b01 = __builtin_convertvector((f2v{bacc[0], bacc[1]}), bf16x2);
  const bf16x2 b23 = __builtin_convertvector((f2v{bacc[2], bacc[3]}), bf16x2);
  const bf16x4 b = __builtin_shufflevector(b01, b23, 0, 1, 2, 3);
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4v, a),
                                                   __builtin_bit_cast(short4v, b), c, 0, 0, 0);
}
__device__ __forceinline__ f4 mma16_acc(const float* arow, int g, f4 bacc, f4 c) {
#pragma unroll
  for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(arow[4 * g + s], bacc[s], c, 0, 0, 0);
  return c;
}

// Two floats -> packed bf16 pair (RNE), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v{a, b}), bf16x2));
}

// The value held by the neighbouring lane (lane ^ 1), by a DPP quad permutation [1,0,3,2]
// (a register operation, no LDS round trip).
__device__ __forceinline__ float lane_swap1(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xf, 0xf, false));
}

// Store a 16x16 D tile (lane: column l%16, rows 4g..4g+3) into a row-major [row][col]
// array with 2-element stores: neighbouring lanes swap two rows so that each lane writes
// (row, cols 2j..2j+1) pairs; no two lanes share an LDS dword. `colmap` maps the tile's
// pair-aligned logical column to its stored column (identity or a permutation that keeps
// pairs (2j, 2j+1) adjacent and in order).
template <typename T, typename F>
__device__ __forceinline__ void store_tile_pairs(T* base, int ld, int lane, f4 v, F colmap) {
  const int n = lane & 15, g = lane >> 4;
  const bool odd = n & 1;
  // even lane keeps rows 4g, 4g+1 and receives them from the odd neighbour;
  // odd lane keeps rows 4g+2, 4g+3 and receives them from the even neighbour
  const float s0 = odd ? v[0] : v[2], s1 = odd ? v[1] : v[3];
  const float r0 = lane_swap1(s0), r1 = lane_swap1(s1);
  const int c0 = colmap(n & ~1);
  const int ra = 4 * g + (odd ? 2 : 0);
  float a0, a1, b0, b1;  // (row ra: col c0, c0+1), (row ra+1: col c0, c0+1)
  if (!odd) { a0 = v[0]; a1 = r0; b0 = v[1]; b1 = r1; }
  else      { a0 = r0; a1 = v[2]; b0 = r1; b1 = v[3]; }
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<uint32_t*>(base + ra * ld + c0) = pack_bf16(a0, a1);
    *reinterpret_cast<uint32_t*>(base + (ra + 1) * ld + c0) = pack_bf16(b0, b1);
  } else {
    typedef float f2 __attribute__((ext_vector_type(2)));
    *reinterpret_cast<f2*>(base + ra * ld + c0) = f2{a0, a1};
    *reinterpret_cast<f2*>(base + (ra + 1) * ld + c0) = f2{b0, b1};
  }
}

// K = 16 product with a preloaded A fragment (row l%16 of A, K-values 4g..4g+3) and B from
// a D tile, converted here (fp32 path: the 4 K-values as 4 fp32 16x16x4 steps).
__device__ __forceinline__ f4 mma16_frag(bf16x4 a, bf16x4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4v, a),
                                                   __builtin_bit_cast(short4v, b), c, 0, 0, 0);
}
__device__ __forceinline__ f4 mma16_frag(f4 a, f4 b, f4 c) {
#pragma unroll
  for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
  return c;
}
template <typename T> struct Frag16;
template <> struct Frag16<bf16> {
  typedef bf16x4 type;
  static __device__ __forceinline__ type load(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
  static __device__ __forceinline__ type from_acc(f4 v) {
    return __builtin_bit_cast(bf16x4, make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])));
  }
};
template <> struct Frag16<float> {
  typedef f4 type;
  static __device__ __forceinline__ type load(const float* p) { return *reinterpret_cast<const f4*>(p); }
  static __device__ __forceinline__ type from_acc(f4 v) { return v; }
};

// Four consecutive elements (a D-tile row group) from LDS, as floats.
__device__ __forceinline__ f4 load4f(const bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f4{static_cast<float>(v[0]), static_cast<float>(v[1]), static_cast<float>(v[2]),
            static_cast<float>(v[3])};
}
__device__ __forceinline__ f4 load4f(const float* p) { return *reinterpret_cast<const f4*>(p); }

// Store N consecutive values (N in {1, 2, 4, 8, 16}) from floats.
template <int N>
__device__ __forceinline__ void store_run(bf16* p, const float* v) {
  if constexpr (N == 1) {
    *p = static_cast<bf16>(v[0]);
  } else if constexpr (N == 2) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    *reinterpret_cast<bf16x2*>(p) = bf16x2{static_cast<bf16>(v[0]), static_cast<bf16>(v[1])};
  } else if constexpr (N == 4) {
    *reinterpret_cast<bf16x4*>(p) = bf16x4{static_cast<bf16>(v[0]), static_cast<bf16>(v[1]),
                                           static_cast<bf16>(v[2]), static_cast<bf16>(v[3])};
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 8) store8(p + i, v + i);
  }
}
template <int N>
__device__ __forceinline__ void store_run(float* p, const float* v) {
  if constexpr (N == 1) {
    *p = v[0];
  } else if constexpr (N == 2) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    *reinterpret_cast<f2*>(p) = f2{v[0], v[1]};
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 4) *reinterpret_cast<f4*>(p + i) = f4{v[i], v[i + 1], v[i + 2], v[i + 3]};
  }
}

// Token-transposed LDS arrays ([channel][64 tokens]) store 4-token groups XOR-swizzled by
// the channel: group' = group ^ ((c >> 3) & 14). Writers (8 consecutive channels per lane,
// lanes 8 channels apart) and MFMA readers (16 consecutive channels, one group) are then
// both free of LDS bank conflicts.
__device__ __forceinline__ int tswz(int c) { return (c >> 3) & 14; }
__device__ __forceinline__ int tcol(int c, int r) { return ((((r >> 2) ^ tswz(c))) << 2) | (r & 3); }

// Store a run of N tokens (N in {1, 2, 4, 8, 16}, aligned to N) of channel row `c`.
template <int N, typename T>
__device__ __forceinline__ void store_run_t(T* row, int c, int r0, const float* v) {
  if constexpr (N <= 4) {
    store_run<N>(row + tcol(c, r0), v);
  } else {
#pragma unroll
    for (int j = 0; j < N; j += 4) store_run<4>(row + tcol(c, r0 + j), v + j);
  }
}

// Workgroup barrier that orders LDS only: outstanding global loads (prefetches into
// registers) stay in flight across it, unlike __syncthreads().
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Returns x unchanged but opaque to the optimiser, so values derived from it (per-lane LDS
// addresses) are recomputed where used instead of being hoisted out of the chunk loop and
// kept live (or spilled) across it. An empty asm statement: no instruction is emitted.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ Mma<bf16>::frag Mma<bf16>::load_perm_t(const bf16* base, int ld, int c,
                                                                  int s, int g) {
  const bf16* row = base + c * ld;
  const int sw = tswz(c);
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + (((8 * s + g) ^ sw) << 2));
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + (((8 * s + 4 + g) ^ sw) << 2));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ Mma<bf16>::frag Mma<bf16>::load_phi_t(const bf16* base, int ld, int c,
                                                                 int s, int g) {
  // groups (8s + 2g, 8s + 2g + 1) stay adjacent under the even XOR swizzle
  return *reinterpret_cast<const bf16x8*>(base + c * ld + (((8 * s + 2 * g) ^ tswz(c)) << 2));
}
__device__ __forceinline__ float Mma<float>::load_perm_t(const float* base, int ld, int c, int s,
                                                         int g) {
  return base[c * ld + ((((4 * (s >> 2) + g) ^ tswz(c))) << 2) + (s & 3)];
}

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace gdn2
