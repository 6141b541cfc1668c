// Chunk-stage building blocks shared by the fused chunk kernel (gdn2_chunk.hip) and the
// two-phase path (gdn2_split.hip): causal tile pairs, the A / P tile products, the per-
// channel decay scan and factors, the 16x16 diagonal inverses, and packed LDS runs.
//
// Notation (one 64-token chunk, local tokens r, i; 16-token blocks R, I; log2 units):
//   G[r]   cumulative log2-decay of the chunk up to and including token r (per channel)
//   Gs(R)  G just before block R starts, Ge(R) = Gs(R + 1), Glast = G[63]
//   A      strictly lower, sum_c E[r,c] K[i,c] 2^(G[r,c]-G[i,c])  (stored negated)
//   P      lower incl. diagonal, the same with Q in place of E
#pragma once

#include "gdn2_device.h"

namespace gdn2 {

// Rows of the per-channel factor table (fp32 [Fac::N][d_k]); the block rows are used only
// by the block-referenced path.
struct Fac {
  static constexpr int ES = 0;    // 2^Gs(R)                R = 0..3
  static constexpr int KE = 4;    // 2^(Glast - Ge(R))      R = 0..3
  static constexpr int GAM = 8;   // 2^Glast: the chunk's decay of the state
  static constexpr int OFF = 9;   // 2^(Gs(R) - Ge(I)) for (R, I) = (2,0), (3,0), (3,1)
  static constexpr int GS = 12;   // Gs(R)                  R = 0..3
  static constexpr int GL = 16;   // Glast (= Ge(3): row GS + R + 1 holds Ge(R) for every R)
  static constexpr int N = 17;
};
static_assert(Fac::GL == Fac::GS + 4, "Ge(R) is read as row GS + R + 1");

// Threshold on a chunk's total log2-decay above which the block-referenced path runs:
// 120 log2 units = 83 nats, so exp(-G) <= 1.3e36 stays finite in fp32 and bf16.
constexpr float kFastPathMaxDecay2 = 120.f;

// Number of K steps of a product whose K range is the causal prefix [0, 16(R+1)).
template <int KS>
__device__ __forceinline__ constexpr int causal_steps(int R) {
  return (16 * (R + 1) + KS - 1) / KS;
}

// Causal 16x16 tile pairs (R, I), I <= R, in the order of the bits of a pair mask.
__device__ __forceinline__ constexpr int pair_R(int p) { return p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3; }
__device__ __forceinline__ constexpr int pair_I(int p) { return p - (pair_R(p) * (pair_R(p) + 1)) / 2; }

// A (stored negated; strictly lower) and P (lower incl. diagonal) tiles for the pairs in
// MASK_A / MASK_P, with the chunk-referenced operands: every tile is a plain product of
// (E exp(G) | Q exp(G)) rows and K exp(-G) rows, K = d_k.
template <typename T, int DK, int LDK, int LDT, int MASK_A, int MASK_P>
__device__ __forceinline__ void ap_tiles(const T* sE, const T* sQ, const T* sK, T* sAm, T* sP,
                                         float* sAd, int m16, int g4) {
  const int lane = 16 * g4 + m16;
  using M = Mma<T>;
  constexpr int MASK = MASK_A | MASK_P;
  f4 accA[10], accP[10];
#pragma unroll
  for (int p = 0; p < 10; ++p) accA[p] = accP[p] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < DK / M::KS; ++s) {
    const int kk = s * M::KS + M::KPL * g4;
    typename M::frag kf[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      bool need = false;
#pragma unroll
      for (int p = 0; p < 10; ++p) need |= ((MASK >> p) & 1) && pair_I(p) == I;
      if (need) kf[I] = M::load(sK, LDK, 16 * I + m16, kk);
    }
#pragma unroll
    for (int p = 0; p < 10; ++p) {
      const int R = pair_R(p), I = pair_I(p);
      if ((MASK_A >> p) & 1) accA[p] = M::mma(M::load(sE, LDK, 16 * R + m16, kk), kf[I], accA[p]);
      if ((MASK_P >> p) & 1) accP[p] = M::mma(M::load(sQ, LDK, 16 * R + m16, kk), kf[I], accP[p]);
    }
  }
#pragma unroll
  for (int p = 0; p < 10; ++p) {
    const int R = pair_R(p), I = pair_I(p);
    if ((MASK_A >> p) & 1) {
      f4 val;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g4 + i, c = m16;
        val[i] = (I < R || c < r) ? -accA[p][i] : 0.f;
        if (sizeof(T) == 2 && I == R) sAd[R * 16 * 20 + r * 20 + c] = val[i];
      }
      store_tile_pairs(sAm + (16 * R) * LDT + 16 * I, LDT, lane, val, [](int c) { return c; });
    }
    if ((MASK_P >> p) & 1) {
      f4 val;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g4 + i, c = m16;
        val[i] = (I < R || c <= r) ? accP[p][i] : 0.f;
      }
      store_tile_pairs(sP + (16 * R) * LDT, LDT, lane, val,
                       [&](int c) { return Mma<T>::phi(16 * I + c); });
    }
  }
}

// A run of N consecutive tokens of one channel row of a token-transposed array, built one
// token at a time (j is a compile-time index after unrolling). bf16 runs are kept packed
// two per register.
template <typename T, int N> struct RunBuf {
  float v[N];
  __device__ __forceinline__ void put(int j, float x) { v[j] = x; }
  template <bool PHI = false>
  __device__ __forceinline__ void store(T* row, int c, int r0) const { store_run_t<N>(row, c, r0, v); }
  template <bool PHI = false>
  __device__ __forceinline__ void store_sw(T* row, int sw, int r0) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int r = PHI ? Mma<T>::phi(r0 + j) : r0 + j;
      row[((((r >> 2) ^ sw)) << 2) | (r & 3)] = v[j];
    }
  }
};
template <int N> struct RunBuf<bf16, N> {
  static_assert(N == 1 || N % 2 == 0, "run length");
  uint32_t w[N / 2 > 0 ? N / 2 : 1];
  float pend;
  __device__ __forceinline__ void put(int j, float x) {
    if (N == 1) {
      pend = x;
    } else if (j & 1) {
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      w[j >> 1] = __builtin_bit_cast(uint32_t, bf16x2{static_cast<bf16>(pend), static_cast<bf16>(x)});
    } else {
      pend = x;
    }
  }
  // PHI: tokens stored in the phi order of Mma<bf16> (runs of 2 and aligned runs of 4 stay
  // contiguous under it).
  template <bool PHI = false>
  __device__ __forceinline__ void store(bf16* row, int c, int r0) const { store_sw<PHI>(row, tswz(c), r0); }
  // sw: the token-group swizzle of the row (shared by the 8 channels of a thread)
  template <bool PHI = false>
  __device__ __forceinline__ void store_sw(bf16* row, int sw, int r0) const {
    auto pos = [&](int r) {
      const int rr = PHI ? Mma<bf16>::phi(r) : r;
      return ((((rr >> 2) ^ sw)) << 2) | (rr & 3);
    };
    if constexpr (N == 1) {
      row[pos(r0)] = static_cast<bf16>(pend);
    } else if constexpr (N == 2) {
      *reinterpret_cast<uint32_t*>(row + pos(r0)) = w[0];
    } else {
#pragma unroll
      for (int q = 0; q < N / 4; ++q)
        *reinterpret_cast<uint2*>(row + pos(r0 + 4 * q)) = make_uint2(w[2 * q], w[2 * q + 1]);
    }
  }
};

// Per-channel scan of a chunk's log2-decay. On entry sTot ([TG][DK], fp32) holds each
// token group's total; on exit it holds the chunk-relative exclusive prefix of each group,
// sFac the factor rows (Fac), and *sFlag is set when some channel's total decay exceeds
// kFastPathMaxDecay2 (the caller clears it beforehand).
template <int DK, int TG, int GPB, int NT>
__device__ __forceinline__ void channel_scan(float* sTot, float* sFac, int* sFlag, int tid) {
  for (int ch = tid; ch < DK; ch += NT) {
    float tot[TG];
#pragma unroll
    for (int x = 0; x < TG; ++x) tot[x] = sTot[x * DK + ch];
    float run = 0.f, gs[4];
#pragma unroll
    for (int x = 0; x < TG; ++x) {
      if (x % GPB == 0) gs[x / GPB] = run;
      sTot[x * DK + ch] = run;
      run += tot[x];
    }
    const float gn = run;
    const float ge[4] = {gs[1], gs[2], gs[3], gn};
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      sFac[(Fac::ES + R) * DK + ch] = fast_exp2(gs[R]);
      sFac[(Fac::KE + R) * DK + ch] = fast_exp2(gn - ge[R]);
      sFac[(Fac::GS + R) * DK + ch] = gs[R];
    }
    sFac[Fac::GAM * DK + ch] = fast_exp2(gn);
    sFac[Fac::GL * DK + ch] = gn;
    sFac[(Fac::OFF + 0) * DK + ch] = fast_exp2(gs[2] - ge[0]);
    sFac[(Fac::OFF + 1) * DK + ch] = fast_exp2(gs[3] - ge[0]);
    sFac[(Fac::OFF + 2) * DK + ch] = fast_exp2(gs[3] - ge[1]);
    if (-gn > kFastPathMaxDecay2) *sFlag = 1;
  }
}

// One 16x16 diagonal block jb of (I + A)^{-1} by fp32 forward substitution, column c per lane,
// from the fp32 copy of the diagonal blocks of -A (block jb, row r, column i at
// sAd[jb * ADB + r * ADP + i]); written to block jb of sT ([64][LDT]) when `write`.
template <typename T, int LDT, int ADB, int ADP>
__device__ __forceinline__ void diag_inverse_block(const float* sAd, T* sT, int jb, int c,
                                                   bool write) {
  const float* Ab = sAd + jb * ADB;
  float am[16][16];
#pragma unroll
  for (int r = 1; r < 16; ++r) {
#pragma unroll
    for (int i4 = 0; i4 < r; i4 += 4) {
      const f4 v = *reinterpret_cast<const f4*>(Ab + r * ADP + i4);
#pragma unroll
      for (int j = 0; j < 4; ++j) am[r][i4 + j] = v[j];
    }
  }
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = (r == c) ? 1.f : 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
#pragma unroll
    for (int r = i + 1; r < 16; ++r) x[r] += am[r][i] * x[i];  // am holds -A
  }
  if (write) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sT[(16 * jb + r) * LDT + 16 * jb + c] = from_f<T>(x[r]);
  }
}

// All four diagonal blocks, one per 16-lane group.
template <typename T, int LDT, int ADB, int ADP>
__device__ __forceinline__ void diag_inverse(const float* sAd, T* sT, int m16, int g4) {
  diag_inverse_block<T, LDT, ADB, ADP>(sAd, sT, g4, m16, true);
}

// Two of them, jb0 and jb0 + 1, on lane groups 0 and 1 (groups 2 and 3 repeat them and do
// not write).
template <typename T, int LDT, int ADB, int ADP>
__device__ __forceinline__ void diag_inverse_pair(const float* sAd, T* sT, int m16, int g4, int jb0) {
  diag_inverse_block<T, LDT, ADB, ADP>(sAd, sT, jb0 + (g4 & 1), m16, g4 < 2);
}

// Block-referenced off-diagonal A and P tiles (chunks whose total decay is too large for
// the chunk-referenced factors): rows of block R (E or Q times 2^(G - Gs(R)), each factor
// <= 1) against the rows of block I (K times 2^(Ge(I) - G), <= 1); two or more blocks apart
// the left operand is also scaled by 2^(Gs(R) - Ge(I)) <= 1, so no factor can overflow. The
// 12 tiles are dealt round-robin to the NW waves; the diagonal tiles come from
// diag_tiles_pairwise.
template <typename T, int DK, int LDK, int LDT, int NW>
__device__ __forceinline__ void ap_tiles_block(const T* sE, const T* sQ, const T* sK, T* sAm,
                                               T* sP, const float* sFac, int wave, int lane) {
  using M = Mma<T>;
  constexpr int KS = M::KS, KPL = M::KPL;
  constexpr int kOffPairs[6] = {1, 3, 4, 6, 7, 8};  // (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
  const int m16 = lane & 15, g4 = lane >> 4;
  for (int job = wave; job < 12; job += NW) {
    const int pair = kOffPairs[job >> 1];
    const bool isP = job & 1;
    const int R = pair_R(pair), I = pair_I(pair);
    const T* lhs = isP ? sQ : sE;
    const int off = (R - I >= 2) ? (R == 2 ? 0 : (I == 0 ? 1 : 2)) : -1;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < DK / KS; ++s) {
      const int kk = s * KS + KPL * g4;  // physical (phi-ordered) K position
      typename M::frag a;
      if (off >= 0) {
        float fa[KPL];
#pragma unroll
        for (int i = 0; i < KPL; ++i) fa[i] = sFac[(Fac::OFF + off) * DK + M::phi_inv(kk + i)];
        a = M::load_scaled(lhs, LDK, 16 * R + m16, kk, fa);
      } else {
        a = M::load(lhs, LDK, 16 * R + m16, kk);
      }
      acc = M::mma(a, M::load(sK, LDK, 16 * I + m16, kk), acc);
    }
    if (isP)
      store_tile_pairs(sP + (16 * R) * LDT, LDT, lane, acc, [&](int c) { return M::phi(16 * I + c); });
    else
      store_tile_pairs(sAm + (16 * R) * LDT + 16 * I, LDT, lane, -acc, [](int c) { return c; });
  }
}

// The diagonal 16x16 tiles of A (negated, fp32: block R, row r, column i at
// sAd[R * ADB + r * ADP + i], zero for i >= r) and of P (sP, phi-ordered columns, zero above
// the diagonal), computed from the raw inputs of the chunk with the exact pairwise decay
// 2^(G[r] - G[i]) = prod_{i < j <= r} alpha_j (a running product, each factor <= 1), so any
// decay in (0, 1] is represented. Rows (R, r) x 8-channel groups are dealt to the NT
// threads; the NCG = d_k / 8 lanes of one row are adjacent and reduce by lane exchange.
// qb, kb, gb, bb: the chunk's first token of this head ([tokens][kstride] rows); bsb the
// scalar b of that token (BS: one b per token and head, H apart).
template <typename T, int DK, int LDT, int ADB, int ADP, int NT, bool BS>
__device__ __forceinline__ void diag_tiles_pairwise(const T* qb, const T* kb, const T* gb,
                                                    const T* bb, const T* bsb, long kstride,
                                                    int H, int nvalid, int tid, float* sAd,
                                                    T* sP) {
  constexpr int NCG = DK / 8;
  static_assert(64 % NCG == 0 && NT % 64 == 0, "a row's channel groups share one wave");
  for (int idx = tid; idx < 64 * NCG; idx += NT) {
    const int cq = idx % NCG, item = idx / NCG;
    const int R = item >> 4, r = item & 15, tr = 16 * R + r;
    float er[8], qr[8], f[8];
    {
      Vec8<T> vq, vk, vb;
      if (tr < nvalid) {
        const long off = (long)tr * kstride + cq * 8;
        vq.load(qb + off);
        vk.load(kb + off);
        if constexpr (BS) { vb.load_one(bsb + (long)tr * H); vb.splat(); }
        else vb.load(bb + off);
      } else {
        vq.zero(); vk.zero(); vb.zero();
      }
      float fk[8], fb[8];
      vq.to_float(qr); vk.to_float(fk); vb.to_float(fb);
#pragma unroll
      for (int c = 0; c < 8; ++c) { er[c] = fb[c] * fk[c]; f[c] = 1.f; }
    }
    float* arow = sAd + R * ADB + r * ADP;
    T* prow = sP + tr * LDT;
    for (int i = r; i >= 0; --i) {
      const int ti = 16 * R + i;
      float ki[8], gi[8];
      {
        Vec8<T> vk, vg;
        if (ti < nvalid) {
          const long off = (long)ti * kstride + cq * 8;
          vk.load(kb + off);
          vg.load(gb + off);
        } else {
          vk.zero(); vg.zero();
        }
        vk.to_float(ki);
        vg.to_float(gi);
      }
      float a = 0.f, p = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float kf = ki[c] * f[c];
        a += er[c] * kf;
        p += qr[c] * kf;
        f[c] *= fast_exp2(gi[c] * kLog2e);  // alpha_i: the product now spans tokens i..r
      }
#pragma unroll
      for (int m = 1; m < NCG; m <<= 1) {
        a += __shfl_xor(a, m, 64);
        p += __shfl_xor(p, m, 64);
      }
      if (cq == 0) {
        arow[i] = i < r ? -a : 0.f;
        prow[Mma<T>::phi(16 * R + i)] = from_f<T>(p);
      }
    }
    if (cq == 0) {
      for (int i = r + 1; i < 16; ++i) {
        arow[i] = 0.f;
        prow[Mma<T>::phi(16 * R + i)] = from_f<T>(0.f);
      }
    }
  }
}

// The upper tiles (0,1) and (2,3) of P (phi-ordered columns) are read as zeros by the
// 32-wide K steps of products with P.
template <typename T, int LDT, int NT>
__device__ __forceinline__ void zero_p_upper(T* sP, int tid) {
  for (int idx = tid; idx < 2 * 256; idx += NT) {
    const int t = idx >> 8, e = idx & 255;
    sP[((t ? 32 : 0) + (e >> 4)) * LDT + Mma<T>::phi((t ? 48 : 16) + (e & 15))] = from_f<T>(0.f);
  }
}

// Where a (chunk slot, head) unit's tokens are: first row of the packed token axis and
// the number of valid tokens (0: an unused slot).
struct ChunkUnit {
  long row;
  int nvalid;
  int h;
};

// Maps unit u = slot * H + h to its tokens. Without cu_seqlens the slots of sequence n are
// n * nch + c. With cu_seqlens, sequence n's slots start at floor(a_n / 64) + n (a_n its
// clamped first token); the owner of a slot is found by a 64-way ballot search over the
// table (wave-uniform result).
__device__ __forceinline__ ChunkUnit map_unit(long u, int H, const int* cu_seqlens, int N,
                                              int T_len, int lane) {
  constexpr int C = 64;
  ChunkUnit r;
  const long slot = u / H;
  r.h = (int)(u - slot * H);
  if (cu_seqlens == nullptr) {
    const int nch = (T_len + C - 1) / C;
    const long n = slot / nch;
    const int c = (int)(slot - n * nch);
    r.row = n * T_len + (long)c * C;
    r.nvalid = min(C, T_len - c * C);
    return r;
  }
  auto clamp_cu = [&](int i) { const int x = cu_seqlens[i]; return x < 0 ? 0 : (x > T_len ? T_len : x); };
  // largest n in [0, N) with start slot s_n = floor(a_n / 64) + n <= slot
  int lo = 0, hi = N;
  if ((long)(clamp_cu(0) / C) > slot) {
    r.row = 0; r.nvalid = 0;
    return r;
  }
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) / 64;
    const int cand = lo + lane * step;
    const bool ok = cand < hi && (long)(clamp_cu(cand) / C + cand) <= slot;
    const unsigned long long m = __ballot(ok);
    const int kk = __popcll(m) - 1;  // lane 0 (cand = lo) always passes
    lo = lo + kk * step;
    hi = min(lo + step, hi);
  }
  const int n = __builtin_amdgcn_readfirstlane(lo);
  const int a = clamp_cu(n);
  int b = clamp_cu(n + 1);
  b = b < a ? a : b;
  const long c = slot - (long)(a / C + n);
  const int len = b - a;
  if (c < 0 || c * C >= len) {
    r.row = 0; r.nvalid = 0;
    return r;
  }
  r.row = a + c * C;
  r.nvalid = len - c * C < C ? (int)(len - c * C) : C;
  return r;
}

}  // namespace gdn2
