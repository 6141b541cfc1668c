// Two-phase chunkwise forward of Gated Delta Rule-2 on gfx950 (bf16 inputs).
//
// The chunk form (GDN-2 reading note, §3 chunkwise-training paragraph; UT transform of the
// Gated DeltaNet visual reading, chunkwise section) splits into work that depends only on
// the chunk's own tokens and a short recurrence over the state:
//   chunk-local:  A, P, T = (I + A)^{-1}, W = T (E 2^G), U~ = T Z, Qbar = Q 2^G,
//                 Kt = (K 2^(Glast - G))^T, gamma = 2^Glast
//   recurrence:   U = U~ - W S,  O = Qbar S + P U,  S <- Diag(gamma) S + Kt U
// Phase 1 (gdn2_prep_kernel) computes the chunk-local factors of every (chunk, head) in
// parallel and stores them in MFMA fragment order (SplitLayout). Phase 2
// (gdn2_state_kernel) walks each (sequence, head, value slice)'s chunks in order with the
// state in accumulator registers; its per-chunk operands do not depend on the state, so
// they are staged into LDS one chunk ahead and its critical path is three MFMA products.
//
// Compared with the fused kernel (gdn2_chunk.hip) this moves the triangular inverse and
// the A / P products off the sequential path and computes them once per head instead of
// once per value slice, at the cost of writing and reading back the factors.

#include <atomic>

#include "gdn2_chunk_common.h"
#include "gdn2_launch.h"

namespace gdn2 {
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ phase 1: factors
template <int DK, int DV>
struct PrepShape {
  typedef bf16 T;
  static constexpr int C = 64;
  static constexpr int NW = 8;            // waves
  static constexpr int NT = 64 * NW;
  static constexpr int CG = DK / 8;       // key-side prep: 8 channels per thread
  static constexpr int TG = NT / CG;      // token groups
  static constexpr int TPT = C / TG;      // tokens per thread (inside one 16-token block)
  static constexpr int GPB = 16 / TPT;    // token groups per 16-token block
  static constexpr int VCG = DV / 8;      // value-side prep: 8 columns per thread
  static constexpr int VTG = NT / VCG;
  static constexpr int VTPT = C / VTG;
  static constexpr int PAD = 16;          // row padding (odd multiple of 8 words: LDS banks)
  static constexpr int LDK = DK + PAD;
  static constexpr int LDT = C + PAD;
  static constexpr int NCT = DK / 16;     // key-channel tiles
  static constexpr int NVT = DV / 16;     // value-column tiles
  static constexpr int NTT = NCT + NVT;   // forward-substitution column tiles
  static constexpr int NTW = (NTT + NW - 1) / NW;  // ... per wave (max)

  static constexpr int SZ_K = C * LDK * 2;
  static constexpr int OFF_E = 0;                  // E 2^G (or Ea); later -W
  static constexpr int OFF_Q = OFF_E + SZ_K;       // Q 2^G (or Qa, rescaled)
  static constexpr int OFF_K = OFF_Q + SZ_K;       // K 2^-G (or K 2^(Ge(block) - G))
  static constexpr int SZ_T = DK * LDT * 2;
  static constexpr int OFF_ET = OFF_K + SZ_K;      // (E 2^G)^T          [DK][64]
  static constexpr int OFF_KT = OFF_ET + SZ_T;     // (K 2^(Gl - G))^T   [DK][64]
  static constexpr int SZ_Z = DV * LDT * 2;
  static constexpr int OFF_ZT = OFF_KT + SZ_T;     // Z^T                [DV][64]
  static constexpr int SZ_P = C * LDT * 2;
  static constexpr int OFF_P = OFF_ZT + SZ_Z;      // P
  static constexpr int OFF_A = OFF_P + SZ_P;       // -A
  static constexpr int OFF_TB = OFF_A + SZ_P;      // diagonal blocks of (I + A)^{-1}
  static constexpr int OFF_FAC = OFF_TB + SZ_P;
  static constexpr int SZ_FAC = Fac::N * DK * 4;
  static constexpr int LDD = 20;                   // fp32 diagonal blocks of -A
  static constexpr int OFF_AD = OFF_FAC + SZ_FAC;
  static constexpr int OFF_FLAG = OFF_AD + 4 * 16 * LDD * 4;
  // U~ tiles in workspace order, written in (f): into the K buffer (dead since (d)) when it
  // is large enough, else into a buffer of their own
  static constexpr int SZ_U = NVT * 4 * 512;
  static constexpr int OFF_U = SZ_U <= SZ_K ? OFF_K : OFF_FLAG + 16;
  static constexpr int LDS_BYTES = (SZ_U <= SZ_K ? OFF_FLAG + 16 : OFF_U + SZ_U);
  static constexpr int OFF_TOT = OFF_P;            // cumsum scratch [TG][DK] in P and -A

  static_assert(TPT >= 1 && TPT <= 16 && 16 % TPT == 0, "token groups must tile 16-blocks");
  static_assert(VTPT >= 1 && C % VTG == 0, "value prep mapping");
  static_assert(TG * DK * 4 <= 2 * SZ_P, "cumsum scratch fits in P and -A");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// 16-byte pieces of one unit's factors held per thread between (g) and the stores: counts
// per workspace region (-W, Qbar, Kt, U~ each a whole number of pieces per thread; P one;
// gamma one on the first d_k / 4 threads) and their index in the thread's register array.
template <int DK, int DV>
struct PrepPieces {
  static constexpr int NT = PrepShape<DK, DV>::NT;
  static constexpr int NW_ = 4 * (DK / 32) * 64 / NT;
  static constexpr int NK_ = (DK / 16) * 2 * 64 / NT;
  static constexpr int NU_ = (DV / 16) * 4 * 32 / NT;
  static constexpr int J_W = 0, J_Q = NW_, J_K = 2 * NW_, J_P = J_K + NK_, J_U = J_P + 1,
                       J_G = J_U + NU_, N = J_G + 1;
  static_assert(4 * (DK / 32) * 64 % NT == 0 && (DK / 16) * 2 * 64 % NT == 0 &&
                (DV / 16) * 4 * 32 % NT == 0 && 8 * 64 == NT && DK / 4 <= NT,
                "factor pieces tile the workgroup");
};

// BWD: also write the reverse chain's operands (BwdLayout) after the forward factors, and
// use the backward unit stride. out_factors = 0 leaves out Qbar and P, which only the output
// o needs (the backward's own forward pass writes none).
template <int DK, int DV, bool BWD, int GL>
__global__ void __launch_bounds__(512)
gdn2_prep_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                 const bf16* __restrict__ v, const bf16* __restrict__ g,
                 const bf16* __restrict__ bg, const bf16* __restrict__ wg,
                 char* __restrict__ ws, const int* __restrict__ cu_seqlens, int N, int T_len,
                 int H, long nunits, int out_factors) {
  typedef bf16 T;
  using Sh = PrepShape<DK, DV>;
  using M = Mma<T>;
  constexpr SplitLayout L(DK, DV);
  constexpr BwdLayout LB(DK, DV);
  constexpr long UNIT = BWD ? LB.bytes : L.bytes;
  constexpr int C = Sh::C, NW = Sh::NW, NT = Sh::NT;
  constexpr int LDK = Sh::LDK, LDT = Sh::LDT, NCT = Sh::NCT;
  constexpr int ADB = 16 * Sh::LDD, ADP = Sh::LDD;
  __shared__ __attribute__((aligned(16))) char smem[Sh::LDS_BYTES];
  T* sE = reinterpret_cast<T*>(smem + Sh::OFF_E);
  T* sWm = sE;  // -W reuses the E buffer once A and P are formed
  T* sQ = reinterpret_cast<T*>(smem + Sh::OFF_Q);
  T* sK = reinterpret_cast<T*>(smem + Sh::OFF_K);
  T* sEt = reinterpret_cast<T*>(smem + Sh::OFF_ET);
  T* sKt = reinterpret_cast<T*>(smem + Sh::OFF_KT);
  T* sZt = reinterpret_cast<T*>(smem + Sh::OFF_ZT);
  T* sP = reinterpret_cast<T*>(smem + Sh::OFF_P);
  T* sAm = reinterpret_cast<T*>(smem + Sh::OFF_A);
  T* sT = reinterpret_cast<T*>(smem + Sh::OFF_TB);
  float* sFac = reinterpret_cast<float*>(smem + Sh::OFF_FAC);
  float* sTot = reinterpret_cast<float*>(smem + Sh::OFF_TOT);
  float* sAd = reinterpret_cast<float*>(smem + Sh::OFF_AD);
  int* sFlag = reinterpret_cast<int*>(smem + Sh::OFF_FLAG);

  int tid = threadIdx.x;
  int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int m16 = lane & 15, g4 = lane >> 4;
  int cg = tid % Sh::CG, tg = tid / Sh::CG, blk = tg / Sh::GPB;
  int vcg = tid % Sh::VCG, vtg = tid / Sh::VCG;
  auto fresh = [&]() {  // re-derive lane indices at each stage (see opaque())
    tid = opaque(tid);
    lane = tid & 63;
    m16 = lane & 15;
    g4 = lane >> 4;
    cg = tid % Sh::CG;
    tg = tid / Sh::CG;
    blk = tg / Sh::GPB;
    vcg = tid % Sh::VCG;
    vtg = tid / Sh::VCG;
  };
  const long kstride = (long)H * DK, vstride = (long)H * DV;

  Vec8<T> rq[Sh::TPT], rk[Sh::TPT], rg[Sh::TPT], rb[Sh::TPT];
  Vec8<T> rv[Sh::VTPT], rw[Sh::VTPT];
  auto load_key = [&](const ChunkUnit& cu) {
    const long kb = cu.row * kstride + (long)cu.h * DK + cg * 8;
#pragma unroll
    for (int j = 0; j < Sh::TPT; ++j) {
      const int r = tg * Sh::TPT + j;
      if (r < cu.nvalid) {
        const long off = kb + (long)r * kstride;
        rq[j].load(q + off);
        rk[j].load(k + off);
        rg[j].load(g + off);
        // a scalar gate: the aligned 8-element block holding it (same load either way; its
        // element is picked out when the unit is consumed)
        if constexpr ((GL & kGateBScalar) != 0) rb[j].load_one(bg + (cu.row + r) * H + cu.h);
        else rb[j].load(bg + off);
      } else {
        rq[j].zero(); rk[j].zero(); rg[j].zero(); rb[j].zero();
      }
    }
  };
  auto load_val = [&](const ChunkUnit& cu) {
    const long vb = cu.row * vstride + (long)cu.h * DV + vcg * 8;
#pragma unroll
    for (int j = 0; j < Sh::VTPT; ++j) {
      const int r = vtg * Sh::VTPT + j;
      if (r < cu.nvalid) {
        const long off = vb + (long)r * vstride;
        rv[j].load(v + off);
        if constexpr ((GL & kGateWScalar) != 0) rw[j].load_one(wg + (cu.row + r) * H + cu.h);
        else rw[j].load(wg + off);
      } else {
        rv[j].zero(); rw[j].zero();
      }
    }
  };
  auto load_raw = [&](const ChunkUnit& cu) {
    load_key(cu);
    load_val(cu);
  };

  // this thread's pieces of the previous unit's factors (see (g)) and their destination
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  constexpr int KSK = DK / 32;
  using Op = PrepPieces<DK, DV>;
  u32x4 ost[Op::N];
  char* prev_out = nullptr;
  auto flush = [&]() {
    if (prev_out == nullptr) return;
#pragma unroll
    for (int q = 0; q < Op::NW_; ++q) {
      *reinterpret_cast<u32x4*>(prev_out + L.w + (tid + q * NT) * 16) = ost[Op::J_W + q];
      if (out_factors) *reinterpret_cast<u32x4*>(prev_out + L.q + (tid + q * NT) * 16) = ost[Op::J_Q + q];
    }
#pragma unroll
    for (int q = 0; q < Op::NK_; ++q)
      *reinterpret_cast<u32x4*>(prev_out + L.kt + (tid + q * NT) * 16) = ost[Op::J_K + q];
    const int pb = tid >> 6;  // P blocks (0,1) and (1,1) are never read
    if (out_factors && pb != 1 && pb != 3) *reinterpret_cast<u32x4*>(prev_out + L.p + tid * 16) = ost[Op::J_P];
#pragma unroll
    for (int q = 0; q < Op::NU_; ++q)
      *reinterpret_cast<u32x4*>(prev_out + L.u + (tid + q * NT) * 16) = ost[Op::J_U + q];
    if (tid < DK / 4) *reinterpret_cast<u32x4*>(prev_out + L.g + tid * 16) = ost[Op::J_G];
  };

  // An unused slot (nvalid = 0) goes through the same steps on zero inputs and fills its
  // own workspace unit, which nothing reads; the loads are unconditional (the prefetch
  // after the last unit re-reads it) so the compiler's waits stay precise.
  long u = blockIdx.x;
  ChunkUnit cur = map_unit(u, H, cu_seqlens, N, T_len, lane);
  load_raw(cur);

  for (; u < nunits; u += gridDim.x) {
    const long un = u + gridDim.x;
    const ChunkUnit nxt = map_unit(un < nunits ? un : u, H, cu_seqlens, N, T_len, lane);
    char* out = ws + u * UNIT;

    lds_barrier();  // the previous unit's readers of every buffer are done
    fresh();
    // ---- (a) per-thread totals of log2-decay
    {
      float tot8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < Sh::TPT; ++j) {
        float f[8];
        rg[j].to_float(f);
#pragma unroll
        for (int i = 0; i < 8; ++i) tot8[i] += f[i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) tot8[i] *= kLog2e;
      store8(sTot + tg * DK + cg * 8, tot8);
    }
    if (tid == 0) *sFlag = 0;
    lds_barrier();
    fresh();

    // ---- (b) per-channel scan and decay factors
    channel_scan<DK, Sh::TG, Sh::GPB, NT>(sTot, sFac, sFlag, tid);
    lds_barrier();
    fresh();
    const bool block_path = __builtin_amdgcn_readfirstlane(*sFlag) != 0;

    // ---- (c) gated, decayed operands
    {
      float run[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) run[i] = sTot[tg * DK + cg * 8 + i];
      RunBuf<T, Sh::TPT> ev[8], kv[8];  // E 2^G and K 2^(Glast - G), per channel
      auto token = [&](int j, const float* sub, const float* subk, const float* fA,
                       const float* fB, bool scaled) {
        const int r = tg * Sh::TPT + j;
        float fg[8], fq[8], fk[8], fb[8], e1[8], q1[8], k1[8];
        rg[j].to_float(fg);
        rq[j].to_float(fq);
        rk[j].to_float(fk);
        if constexpr ((GL & kGateBScalar) != 0) rb[j].splat();
        rb[j].to_float(fb);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          run[i] += fg[i] * kLog2e;
          const float x = scaled ? run[i] - sub[i] : run[i];
          const float xe = fast_exp2(x), xk = fast_exp2(scaled ? subk[i] - run[i] : -run[i]);
          e1[i] = fb[i] * fk[i] * xe;
          q1[i] = fq[i] * xe;
          k1[i] = fk[i] * xk;
          ev[i].put(j, scaled ? e1[i] * fA[i] : e1[i]);
          kv[i].put(j, k1[i] * fB[i]);
        }
        store8_phi(sE + r * LDK, cg * 8, e1);
        store8_phi(sQ + r * LDK, cg * 8, q1);
        store8_phi(sK + r * LDK, cg * 8, k1);
      };
      if (!block_path) {
        float gam[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) gam[i] = sFac[Fac::GAM * DK + cg * 8 + i];
#pragma unroll
        for (int j = 0; j < Sh::TPT; ++j) token(j, nullptr, nullptr, nullptr, gam, false);
      } else {
        // E, Q times 2^(G - Gs(block)); K times 2^(Ge(block) - G); every factor <= 1
        float fA[8], fB[8], sub[8], subk[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          fA[i] = sFac[(Fac::ES + blk) * DK + cg * 8 + i];
          fB[i] = sFac[(Fac::KE + blk) * DK + cg * 8 + i];
          sub[i] = sFac[(Fac::GS + blk) * DK + cg * 8 + i];
          subk[i] = sFac[(Fac::GS + blk + 1) * DK + cg * 8 + i];
        }
#pragma unroll
        for (int j = 0; j < Sh::TPT; ++j) token(j, sub, subk, fA, fB, true);
      }
      const int sw = tswz(cg * 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ev[i].store_sw(sEt + (cg * 8 + i) * LDT, sw, tg * Sh::TPT);
        kv[i].template store_sw<true>(sKt + (cg * 8 + i) * LDT, sw, tg * Sh::TPT);
      }
      RunBuf<T, Sh::VTPT> zv[8];
#pragma unroll
      for (int j = 0; j < Sh::VTPT; ++j) {
        float fv[8], fw[8];
        rv[j].to_float(fv);
        if constexpr ((GL & kGateWScalar) != 0) rw[j].splat();
        rw[j].to_float(fw);
#pragma unroll
        for (int i = 0; i < 8; ++i) zv[i].put(j, fv[i] * fw[i]);
      }
      const int zsw = tswz(vcg * 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) zv[i].store_sw(sZt + (vcg * 8 + i) * LDT, zsw, vtg * Sh::VTPT);
    }
    // the previous unit's factors to the workspace, then the next unit's key-side prefetch:
    // the wait for these loads (next unit's (a)) then covers stores issued before them
    // rather than after (the waits cannot tell late stores from the loads). The value side
    // follows after (d), so the two bursts do not queue together behind the stores.
    flush();
    load_key(nxt);
    lds_barrier();
    fresh();

    // ---- (d) A (negated) and P; the last wave forms the diagonal A tiles and inverts
    // them in the same stage
    constexpr int TDW = NW - 1;
    if (!block_path) {
      switch (wave) {
        case 0: ap_tiles<T, DK, LDK, LDT, 0x0C0, 0>(sE, sQ, sK, sAm, sP, sAd, m16, g4); break;
        case 1: ap_tiles<T, DK, LDK, LDT, 0x118, 0>(sE, sQ, sK, sAm, sP, sAd, m16, g4); break;
        case 2: ap_tiles<T, DK, LDK, LDT, 0x002, 0x001>(sE, sQ, sK, sAm, sP, sAd, m16, g4); break;
        case 3: ap_tiles<T, DK, LDK, LDT, 0, 0x0C0>(sE, sQ, sK, sAm, sP, sAd, m16, g4); break;
        case 4: ap_tiles<T, DK, LDK, LDT, 0, 0x300>(sE, sQ, sK, sAm, sP, sAd, m16, g4); break;
        case 5: ap_tiles<T, DK, LDK, LDT, 0, 0x038>(sE, sQ, sK, sAm, sP, sAd, m16, g4); break;
        case 6: ap_tiles<T, DK, LDK, LDT, 0, 0x006>(sE, sQ, sK, sAm, sP, sAd, m16, g4); break;
        default:
          ap_tiles<T, DK, LDK, LDT, 0x225, 0>(sE, sQ, sK, sAm, sP, sAd, m16, g4);
          diag_inverse<T, LDT, ADB, ADP>(sAd, sT, m16, g4);
          break;
      }
    } else {
      ap_tiles_block<T, DK, LDK, LDT, NW>(sE, sQ, sK, sAm, sP, sFac, wave, lane);
      const long base = cur.row * kstride + (long)cur.h * DK;
      diag_tiles_pairwise<T, DK, LDT, ADB, ADP, NT, (GL & kGateBScalar) != 0>(
          q + base, k + base, g + base, bg + base, bg + cur.row * H + cur.h, kstride, H,
          cur.nvalid, tid, sAd, sP);
    }
    zero_p_upper<T, LDT, NT>(sP, tid);
    lds_barrier();
    fresh();
    if (block_path) {
      // inverse blocks by the last wave; the others rescale Qa to Q 2^G
      if (wave == TDW) diag_inverse<T, LDT, ADB, ADP>(sAd, sT, m16, g4);
      for (int idx = tid; wave != TDW && idx < C * DK; idx += NT - 64) {
        const int r = idx / DK, pc = idx % DK;
        sQ[r * LDK + pc] = from_f<T>(to_f(sQ[r * LDK + pc]) *
                                     sFac[(Fac::ES + r / 16) * DK + M::phi_inv(pc)]);
      }
      lds_barrier();
      fresh();
    }

    load_val(nxt);
    // ---- (f) [W | U~] = (I + A)^{-1} [E 2^G | Z] by block forward substitution:
    //   X_R = T_RR (RHS_R - sum_{J<R} A_RJ X_J)
    // Column tiles (key tiles, then value tiles) are dealt round-robin to the waves.
    {
      using F16 = Frag16<T>;
      typename F16::type fa[4][4];
#pragma unroll
      for (int R = 0; R < 4; ++R) {
#pragma unroll
        for (int J = 0; J < R; ++J) fa[R][J] = F16::load(sAm + (16 * R + m16) * LDT + 16 * J + 4 * g4);
        fa[R][R] = F16::load(sT + (16 * R + m16) * LDT + 16 * R + 4 * g4);
      }
#pragma unroll
      for (int t = 0; t < Sh::NTW; ++t) {
        const int idx = wave + t * NW;
        if (idx >= Sh::NTT) continue;
        const bool isZ = idx >= NCT;
        const int ct = isZ ? idx - NCT : idx;
        const int crow = 16 * ct + m16;
        const T* src = (isZ ? sZt : sEt) + crow * LDT;
        f4 X[4];
        typename F16::type Xb[4];
#pragma unroll
        for (int R = 0; R < 4; ++R) {
          f4 acc = load4f(src + tcol(crow, 16 * R + 4 * g4));
#pragma unroll
          for (int J = 0; J < R; ++J) acc = mma16_frag(fa[R][J], Xb[J], acc);
          X[R] = mma16_frag(fa[R][R], F16::from_acc(acc), f4{0.f, 0.f, 0.f, 0.f});
          Xb[R] = F16::from_acc(X[R]);
        }
        if (!isZ) {
#pragma unroll
          for (int R = 0; R < 4; ++R)
            store_tile_pairs(sWm + (16 * R) * LDK, LDK, lane, -X[R],
                             [&](int c) { return M::phi(16 * ct + c); });
        } else {
          // U~ D tile (ct, R), lane-major with 4 bf16 per lane (its workspace order)
#pragma unroll
          for (int R = 0; R < 4; ++R)
            *reinterpret_cast<uint2*>(smem + Sh::OFF_U + ((ct * 4 + R) * 64 + lane) * 8) =
                make_uint2(pack_bf16(X[R][0], X[R][1]), pack_bf16(X[R][2], X[R][3]));
        }
      }
    }
    lds_barrier();
    fresh();

    // ---- (g) this unit's factors, in workspace order, from LDS into registers; they are
    // stored during the next unit (or after the loop), just before its prefetch loads
    {
#pragma unroll
      for (int q = 0; q < Op::NW_; ++q) {  // -W and Qbar
        const int p = tid + q * NT, bi = p >> 6, l = p & 63;
        const int row = 16 * (bi / KSK) + (l & 15), col = 32 * (bi % KSK) + 8 * (l >> 4);
        ost[Op::J_W + q] = *reinterpret_cast<const u32x4*>(sWm + row * LDK + col);
        ost[Op::J_Q + q] = *reinterpret_cast<const u32x4*>(sQ + row * LDK + col);
      }
#pragma unroll
      for (int q = 0; q < Op::NK_; ++q) {  // Kt: [channel][phi-ordered tokens], swizzled
        const int p = tid + q * NT, bi = p >> 6, l = p & 63;
        const int row = 16 * (bi >> 1) + (l & 15), grp = 8 * (bi & 1) + 2 * (l >> 4);
        ost[Op::J_K + q] = *reinterpret_cast<const u32x4*>(sKt + row * LDT + ((grp ^ tswz(row)) << 2));
      }
      {  // P
        const int p = tid, bi = p >> 6, l = p & 63;
        const int row = 16 * (bi >> 1) + (l & 15), col = 32 * (bi & 1) + 8 * (l >> 4);
        ost[Op::J_P] = *reinterpret_cast<const u32x4*>(sP + row * LDT + col);
      }
#pragma unroll
      for (int q = 0; q < Op::NU_; ++q)  // U~ tiles
        ost[Op::J_U + q] = *reinterpret_cast<const u32x4*>(smem + Sh::OFF_U + (tid + q * NT) * 16);
      if (tid < DK / 4)  // gamma
        ost[Op::J_G] = *reinterpret_cast<const u32x4*>(sFac + Fac::GAM * DK + 4 * tid);
    }
    if constexpr (BWD) {
      // the reverse chain's operands, stored at once (16-byte pieces; transposed reads of
      // the LDS arrays, two bf16 per 4-byte word)
      auto put8 = [&](long off, const float* f) {
        *reinterpret_cast<uint4*>(out + off) =
            make_uint4(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]),
                       pack_bf16(f[6], f[7]));
      };
      constexpr int KSK = DK / 32;
#pragma unroll
      for (int qq = 0; qq < 4 * KSK * 64 / NT; ++qq) {  // Ktil, row-major: rows = tokens
        // from the token-transposed copy (K 2^(Glast - G) on both paths; phi-ordered,
        // swizzled tokens)
        const int p = tid + qq * NT, bi = p >> 6, l = p & 63;
        const int r = 16 * (bi / KSK) + (l & 15), p0 = 32 * (bi % KSK) + 8 * (l >> 4);
        float f[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = M::phi_inv(p0 + j);
          f[j] = to_f(sKt[c * LDT + tcol(c, M::phi(r))]);
        }
        put8(LB.kr + p * 16, f);
      }
      {  // P^T: rows r, K = tokens i (natural); blocks (2,0), (3,0) are zero
        const int p = tid, bi = p >> 6, l = p & 63;
        const int r = 16 * (bi >> 1) + (l & 15), i0 = 32 * (bi & 1) + 8 * (l >> 4);
        if (!(bi == 4 || bi == 6)) {
          float f[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) f[j] = to_f(sP[(i0 + j) * LDT + M::phi(r)]);
          put8(LB.pt + p * 16, f);
        }
      }
#pragma unroll
      for (int qq = 0; qq < NCT * 2 * 64 / NT; ++qq) {  // Qbar^T and -W^T: rows = channels
        const int p = tid + qq * NT, bi = p >> 6, l = p & 63;
        const int c = 16 * (bi >> 1) + (l & 15), t0 = 32 * (bi & 1) + 8 * (l >> 4);
        float fq[8], fw[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          fq[j] = to_f(sQ[(t0 + j) * LDK + M::phi(c)]);            // tokens natural
          fw[j] = to_f(sWm[M::phi_inv(t0 + j) * LDK + M::phi(c)]);  // tokens phi-ordered
        }
        put8(LB.qt + p * 16, fq);
        put8(LB.wt + p * 16, fw);
      }
      {  // back-substitution blocks (R, J), J >= R: 2 lanes x 4 bf16 per 16-byte piece
        const int p = tid, bi = p >> 5, l0 = 2 * (p & 31);
        const int R = bi >> 2, J = bi & 3;
        if (J >= R) {
          float f[8];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int a = (l0 + h2) & 15, gq = (l0 + h2) >> 4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int c = 4 * gq + i;
              f[4 * h2 + i] = J > R ? to_f(sAm[(16 * J + c) * LDT + 16 * R + a])
                                    : to_f(sT[(16 * R + c) * LDT + 16 * R + a]);
            }
          }
          put8(LB.bt + p * 16, f);
        }
      }
    }
    prev_out = out;
    cur = nxt;
  }
  lds_barrier();
  flush();
}

// ------------------------------------------------------------------ phase 2: recurrence
// OUTBUF: the two output staging buffers (not needed by the transfer pass, MODE 3)
template <int DK, int DV, int NV, bool OUTBUF = true>
struct StateShape {
  static constexpr int C = 64;
  static constexpr int NWV = NV / 16;     // waves: wave w owns state columns [16w, 16w+16)
  static constexpr int NT = 64 * NWV;
  static constexpr int KSK = DK / 32;     // 32-channel K steps
  static constexpr int NMT = DK / 16;     // 16-row state tiles per wave
  static constexpr SplitLayout L = SplitLayout(DK, DV);
  // one staged chunk: [-W | Qbar | Kt | P] (contiguous in the workspace), this slice's U~
  // tiles, gamma
  static constexpr int SZ_A = (int)L.u;
  static constexpr int SZ_U = NWV * 4 * 512;
  static constexpr int OFF_U = SZ_A;
  static constexpr int OFF_G = OFF_U + SZ_U;
  static constexpr int NPIECE = (OFF_G + DK * 4) / 16;  // 16-byte pieces per chunk
  static constexpr int STAGE = NPIECE * 16;
  static constexpr int OP = NV + 8;                   // output staging pitch
  static constexpr int SZ_O = C * OP * 2;
  static constexpr int OFF_O = 2 * STAGE;             // two output staging buffers
  static constexpr int LDS_BYTES = OUTBUF ? OFF_O + 2 * SZ_O : 2 * STAGE;
  static_assert(STAGE % 16 == 0, "stage");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// MODE 0: the forward (output o). MODE 1 (the backward's own forward pass): no output;
// instead the state entering every chunk and that chunk's U are stored into the backward
// workspace (BwdLayout::h, ::ub). MODE 2 (training forward): both, so that a later backward
// can skip its forward pass. MODE 3 (segment transfer pass of a long sequence; MODE 4: the
// same on the backward workspace, whose units start with the same factors): no output;
// the columns are [d_v value columns | d_k identity columns]: the value columns run from a
// zero state, the identity columns from the identity with U~ = 0 (so they carry the
// segment's product of chunk transitions Diag(gamma) - Kt^T W), and the segment's end
// state [N | M] is written to ebuf.
// Segments: a sequence's chunks are cut into nseg runs of seg_chunks (the last may be
// shorter); a unit is (sequence, head, segment), its start state is s0[unit] (MODE 0; the
// combine kernel's output when nseg > 1) and only the last segment writes sN.
template <int DK, int DV, int NV, int MODE>
__global__ void __launch_bounds__((StateShape<DK, DV, NV, (MODE < 3)>::NT))
__attribute__((amdgpu_waves_per_eu(StateShape<DK, DV, NV, (MODE < 3)>::NT / 256,
                                   StateShape<DK, DV, NV, (MODE < 3)>::NT / 256)))
gdn2_state_kernel(const char* __restrict__ ws, const float* s0, bf16* __restrict__ o,
                  float* sN, const int* __restrict__ cu_seqlens, int T_len, int H,
                  int nslices, int nunits, int nseg, int seg_chunks, float* __restrict__ ebuf) {
  typedef bf16 T;
  constexpr bool XFER = MODE == 3 || MODE == 4;
  constexpr bool STORE = MODE == 1 || MODE == 2;  // entering states and U to the backward workspace
  constexpr bool OUT = MODE == 0 || MODE == 2;    // the output o
  using Sh = StateShape<DK, DV, NV, !XFER>;
  using M = Mma<T>;
  constexpr SplitLayout L(DK, DV);
  constexpr BwdLayout LB(DK, DV);
  constexpr long UNIT = (STORE || MODE == 4) ? LB.bytes : L.bytes;
  constexpr int C = Sh::C, NT = Sh::NT, KSK = Sh::KSK, NMT = Sh::NMT, OP = Sh::OP;
  __shared__ __attribute__((aligned(16))) char smem[Sh::LDS_BYTES];

  int tid = threadIdx.x;
  int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int m16 = lane & 15, g4 = lane >> 4;

  // workgroup -> (sequence, head, slice); slices of one head on one XCD (ids congruent
  // mod 8) so the shared factor reads of the second slice hit that XCD's L2
  const int grp = blockIdx.x / (8 * nslices);
  const int gsz = min(8, nunits - grp * 8);
  const int gi = blockIdx.x - grp * 8 * nslices;
  const int slice = gi / gsz;
  const int unit_id = grp * 8 + gi % gsz;  // (sequence * H + head) * nseg + segment
  const int seg = unit_id % nseg;
  const int nh = unit_id / nseg;
  const int h = nh % H;
  const int n = nh / H;
  const int col0 = slice * NV;              // MODE 3: within [d_v value | d_k identity] columns
  const bool ident = XFER && col0 >= DV;    // this slice carries transfer (identity) columns

  long row0, slot0;
  int len;
  if (cu_seqlens != nullptr) {
    int a = cu_seqlens[n], b = cu_seqlens[n + 1];
    a = a < 0 ? 0 : (a > T_len ? T_len : a);
    b = b < a ? a : (b > T_len ? T_len : b);
    row0 = a;
    len = b - a;
    slot0 = a / C + n;
  } else {
    row0 = (long)n * T_len;
    len = T_len;
    slot0 = (long)n * ((T_len + C - 1) / C);
  }
  {  // this unit's segment of the sequence
    const int cbeg = seg * seg_chunks;
    row0 += (long)cbeg * C;
    slot0 += cbeg;
    const int rest = len - cbeg * C;
    len = rest < 0 ? 0 : (nseg > 1 && rest > seg_chunks * C ? seg_chunks * C : rest);
  }
  const int nch = (len + C - 1) / C;
  const long vstride = (long)H * DV;
  T* ob = o + row0 * vstride + (long)h * DV + col0;

  // state: tile mt holds key rows [16mt, 16mt+16), column col0 + 16*wave + m16; lane holds
  // rows 16mt + 4*g4 + i
  f4 S[NMT];
  const long sbase = ((long)n * H + h) * DK * DV + col0 + 16 * wave + m16;       // sN
  const long s0base = (long)unit_id * DK * DV + col0 + 16 * wave + m16;           // s0[unit]
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * mt + 4 * g4 + i;
      if constexpr (XFER)
        S[mt][i] = (ident && row == col0 - DV + 16 * wave + m16) ? 1.f : 0.f;
      else
        S[mt][i] = (s0 != nullptr) ? s0[s0base + (long)row * DV] : 0.f;
    }

  // Staging of the chunk operands: global -> registers -> LDS, one chunk ahead: at the end
  // of chunk c the registers (chunk c+1) go to the LDS buffer that chunk c-1 used and are
  // refilled with chunk c+2. (A plain vector type: an array of HIP's uint4 struct of this
  // length is kept in scratch memory.)
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  // Without an output, Qbar and P are not staged (they feed only o): the staged pieces are
  // [-W | Kt | U~ | gamma], each at its usual place in the stage, whose layout is the
  // workspace's prefix [-W | Qbar | Kt | P], then this slice's U~ tiles, then gamma.
  static_assert(Sh::OFF_U == (int)L.u, "staged prefix matches the workspace prefix");
  constexpr int SKIP_Q = OUT ? 0 : (int)(L.kt - L.q);
  constexpr int SKIP_P = OUT ? 0 : (int)(L.u - L.p);
  constexpr int NPC = Sh::NPIECE - (SKIP_Q + SKIP_P) / 16;  // pieces staged per chunk
  constexpr int PPC = (NPC + NT - 1) / NT;                  // ... per thread
  u32x4 stg[PPC];
  // stage offset of staged piece p (the tail pieces repeat the last one, same data to the
  // same place, so the staging code has no branches); selects only
  auto piece_off = [&](int p) {
    int off = (p < NPC ? p : NPC - 1) * 16;
    off += off >= (int)L.q ? SKIP_Q : 0;
    off += off >= (int)L.p ? SKIP_P : 0;
    return off;
  };
  const int u_shift = (XFER && ident ? 0 : slice) * Sh::SZ_U;  // identity slices: unused
  auto piece_src = [&](int off, long chunk) -> const u32x4* {
    const char* unit = ws + ((slot0 + chunk) * H + h) * UNIT;
    off += (off >= Sh::OFF_U && off < Sh::OFF_G ? u_shift : 0) +
           (off >= Sh::OFF_G ? (int)L.g - Sh::OFF_G : 0);
    return reinterpret_cast<const u32x4*>(unit + off);
  };
  auto stage_load = [&](long chunk) {
#pragma unroll
    for (int j = 0; j < PPC; ++j) stg[j] = *piece_src(piece_off(tid + j * NT), chunk);
  };
  auto stage_store = [&](char* buf) {
#pragma unroll
    for (int j = 0; j < PPC; ++j) *reinterpret_cast<u32x4*>(buf + piece_off(tid + j * NT)) = stg[j];
  };
  // output rows of the previous chunk: staging buffer -> HBM (16-byte pieces, written once:
  // non-temporal)
  constexpr int OPR = NV / 8;  // pieces per row
  static_assert((C * OPR) % NT == 0, "output pieces per thread");
  auto out_store = [&](const T* so, long c0, int nrows) {
#pragma unroll
    for (int j = 0; j < C * OPR / NT; ++j) {
      const int p = tid + j * NT;
      const int r = p / OPR, cc = p % OPR;
      if (r < nrows) {
        typedef uint32_t u4 __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(*reinterpret_cast<const u4*>(so + r * OP + cc * 8),
                                    reinterpret_cast<u4*>(ob + (c0 + r) * vstride + cc * 8));
      }
    }
  };

  if (nch > 0) {
    stage_load(0);
    stage_store(smem);
    stage_load(nch > 1 ? 1 : 0);
  }
  lds_barrier();

  for (int ci = 0; ci < nch; ++ci) {
    tid = opaque(tid);
    lane = tid & 63;
    m16 = lane & 15;
    g4 = lane >> 4;
    const char* B = smem + (ci & 1) * Sh::STAGE;
    T* so = OUT ? reinterpret_cast<T*>(smem + Sh::OFF_O + (ci & 1) * Sh::SZ_O) : nullptr;
    auto frag = [&](int off, int blk) {
      return *reinterpret_cast<const typename M::frag*>(B + off + blk * 1024 + lane * 16);
    };
    typename M::frag sb[KSK];
#pragma unroll
    for (int s = 0; s < KSK; ++s) sb[s] = M::from_acc(S, s);
    char* const bunit = const_cast<char*>(ws) + ((slot0 + ci) * H + h) * UNIT;
    const int ctg = slice * Sh::NWV + wave;  // this wave's column tile within d_v
    if constexpr (STORE) {  // the state entering this chunk (non-temporal, as U below: read
                            // back by other workgroups of a later launch)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
        __builtin_nontemporal_store(
            (u32x2){pack_bf16(S[mt][0], S[mt][1]), pack_bf16(S[mt][2], S[mt][3])},
            reinterpret_cast<u32x2*>(bunit + LB.h + ((ctg * NMT + mt) * 64 + lane) * 8));
    }
    // U = U~ - W S
    f4 U[4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      const bf16x4 ut = *reinterpret_cast<const bf16x4*>(B + Sh::OFF_U + ((wave * 4 + R) * 64 + lane) * 8);
      U[R] = ident ? f4{0.f, 0.f, 0.f, 0.f} : f4{to_f(ut[0]), to_f(ut[1]), to_f(ut[2]), to_f(ut[3])};
    }
    // Fragments are read from LDS in batches ahead of their products, so that many reads
    // are in flight at once (one wave per SIMD: nothing else hides LDS latency).
    typename M::frag fw[4 * KSK];
#pragma unroll
    for (int i = 0; i < 4 * KSK; ++i) fw[i] = frag((int)L.w, i);
    typename M::frag fq[4 * KSK];
    if constexpr (OUT) {
#pragma unroll
      for (int i = 0; i < 4 * KSK; ++i) fq[i] = frag((int)L.q, i);
    }
    __builtin_amdgcn_sched_barrier(0);  // all of the above is issued before any product
    typename M::frag fk[2 * NMT], fp[6];
#pragma unroll
    for (int i = 0; i < 2 * NMT; ++i) fk[i] = frag((int)L.kt, i);
    if constexpr (OUT) {
#pragma unroll
      for (int i = 0; i < 6; ++i) fp[i] = frag((int)L.p, i < 2 ? 2 * i : i + 2);  // blocks 0,2,4,5,6,7
    }
    f4 gam[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) gam[mt] = *reinterpret_cast<const f4*>(B + Sh::OFF_G + (16 * mt + 4 * g4) * 4);
#pragma unroll
    for (int R = 0; R < 4; ++R)
#pragma unroll
      for (int s = 0; s < KSK; ++s) U[R] = M::mma(fw[R * KSK + s], sb[s], U[R]);
    // O = Qbar S + P U
    f4 O[4];
    if constexpr (OUT) {
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        O[R] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSK; ++s) O[R] = M::mma(fq[R * KSK + s], sb[s], O[R]);
      }
    }
    if constexpr (STORE) {
#pragma unroll
      for (int R = 0; R < 4; ++R)
        __builtin_nontemporal_store(
            (u32x2){pack_bf16(U[R][0], U[R][1]), pack_bf16(U[R][2], U[R][3])},
            reinterpret_cast<u32x2*>(bunit + LB.ub + ((ctg * 4 + R) * 64 + lane) * 8));
    }
    typename M::frag ub[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) ub[s] = M::from_acc(U, s);
    // S <- Diag(gamma) S + Kt U
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      f4 acc = S[mt] * gam[mt];
#pragma unroll
      for (int s = 0; s < 2; ++s) acc = M::mma(fk[mt * 2 + s], ub[s], acc);
      S[mt] = acc;
    }
    if constexpr (OUT) {
#pragma unroll
      for (int R = 0; R < 4; ++R) {
#pragma unroll
        for (int s = 0; s < causal_steps<32>(R); ++s) O[R] = M::mma(fp[R < 2 ? R : 2 * R - 2 + s], ub[s], O[R]);
        store_tile_pairs(so + (16 * R) * OP + 16 * wave, OP, lane, O[R], [](int c) { return c; });
      }
    }
    // next chunk's operands into the other buffer (its last readers finished before the
    // previous barrier); the previous chunk's output (staged before the last barrier) to
    // HBM; then the loads for the chunk after (unconditional: past the end they re-read the
    // last chunk). Issuing the stores before the loads matters: the wait for these loads
    // at the end of the next chunk then also covers stores a whole chunk old, instead of
    // stores issued after the loads (which the waits cannot tell apart from them).
    if (ci + 1 < nch) stage_store(smem + ((ci + 1) & 1) * Sh::STAGE);
    if (OUT && ci > 0) {
      const int pv = len - (ci - 1) * C;
      out_store(reinterpret_cast<const T*>(smem + Sh::OFF_O + ((ci - 1) & 1) * Sh::SZ_O),
                (long)(ci - 1) * C, pv < C ? pv : C);
    }
    stage_load(ci + 2 < nch ? ci + 2 : nch - 1);
    lds_barrier();
  }
  if (OUT && nch > 0) {
    const int pv = len - (nch - 1) * C;
    out_store(reinterpret_cast<const T*>(smem + Sh::OFF_O + ((nch - 1) & 1) * Sh::SZ_O),
              (long)(nch - 1) * C, pv < C ? pv : C);
  }
  if constexpr (XFER) {  // the segment's end state [N | M] (rows d_k, d_v + d_k columns)
    constexpr int LE = DV + DK;
    float* E = ebuf + (long)unit_id * DK * LE + col0 + 16 * wave + m16;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) E[(long)(16 * mt + 4 * g4 + i) * LE] = S[mt][i];
  } else if (sN != nullptr && seg == nseg - 1) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sN[sbase + (long)(16 * mt + 4 * g4 + i) * DV] = S[mt][i];
  }
}

// Segment start states of a long sequence: S_0 = the sequence's initial state (or 0) and
// S_{s+1} = M_s S_s + N_s, with [N_s | M_s] the end state of segment s's transfer pass.
// REV (the backward's state gradient, which runs from the last chunk to the first): D at
// the end of the last segment is the final state's gradient (or 0) and D_{s-1} = A_s D_s + b_s
// with b_s from the reverse chain's transfer pass and A_s = M_s^T (the buffer holds
// [b_s | M_s]); sbuf then holds each segment's end value.
// One workgroup per (sequence, head, 16 value columns); one wave per 16-row tile; M_s is
// staged in LDS with 16-byte loads, products in fp32 (16x16x4 MFMA), S exchanged through
// LDS every step.
template <int DK, int DV, bool REV>
__global__ void __launch_bounds__(DK * 4)
gdn2_seg_combine_kernel(const float* __restrict__ ebuf, const float* __restrict__ s0,
                        float* __restrict__ sbuf, int H, int nseg) {
  constexpr int LE = DV + DK, NRT = DK / 16, RPW = 1, NT = 64 * NRT;
  constexpr int LDM = DK + 4;                                 // padded pitch of M in LDS
  __shared__ float sS[DK][16];
  __shared__ __attribute__((aligned(16))) float sM[DK * LDM];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int m16 = lane & 15, g4 = lane >> 4;
  const int ct = blockIdx.x % (DV / 16);
  const int nh = blockIdx.x / (DV / 16);  // sequence * H + head
  const int c = 16 * ct + m16;            // this lane's value column
  f4 S[RPW];
#pragma unroll
  for (int t = 0; t < RPW; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * (wave * RPW + t) + 4 * g4 + i;
      S[t][i] = s0 != nullptr ? s0[((long)nh * DK + row) * DV + c] : 0.f;
    }
  for (int step = 0; step < nseg; ++step) {
    const int s = REV ? nseg - 1 - step : step;
    const long unit = (long)nh * nseg + s;
    float* out = sbuf + unit * DK * DV;
    const float* E = ebuf + unit * DK * LE;
#pragma unroll
    for (int t = 0; t < RPW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * (wave * RPW + t) + 4 * g4 + i;
        out[(long)row * DV + c] = S[t][i];
        sS[row][m16] = S[t][i];
      }
    if (step + 1 < nseg) {
      // M_s (d_k x d_k, the last d_k columns of E's rows) -> LDS
      for (int p = tid; p < DK * DK / 4; p += NT) {
        const int row = p / (DK / 4), c4 = p % (DK / 4);
        *reinterpret_cast<f4*>(sM + row * LDM + 4 * c4) =
            *reinterpret_cast<const f4*>(E + (long)row * LE + DV + 4 * c4);
      }
      f4 acc[RPW];
#pragma unroll
      for (int t = 0; t < RPW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)  // N_s
          acc[t][i] = E[(long)(16 * (wave * RPW + t) + 4 * g4 + i) * LE + c];
      __syncthreads();
#pragma unroll 8
      for (int k0 = 0; k0 < DK; k0 += 4) {
        const float b = sS[k0 + g4][m16];  // S_s[k][col]
#pragma unroll
        for (int t = 0; t < RPW; ++t) {
          const int row = 16 * (wave * RPW + t) + m16, k = k0 + g4;
          const float a = REV ? sM[k * LDM + row] : sM[row * LDM + k];  // A = M^T, or M
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[t], 0, 0, 0);
        }
      }
#pragma unroll
      for (int t = 0; t < RPW; ++t) S[t] = acc[t];
    }
    __syncthreads();  // sS and sM are rewritten next step
  }
}

// ------------------------------------------------------------------ launch
hipError_t launch_seg_combine(const float* ebuf, const float* s_in, float* sbuf, int N, int H,
                              int d_k, int d_v, int nseg, bool reverse, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid((unsigned)((long)N * H * (d_v / 16)));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(d_k * 4), 0, st, ebuf, s_in, sbuf, H, nseg);
    return hipGetLastError();
  };
  if (d_k == 64 && d_v == 64) return reverse ? go(gdn2_seg_combine_kernel<64, 64, true>) : go(gdn2_seg_combine_kernel<64, 64, false>);
  if (d_k == 64 && d_v == 128) return reverse ? go(gdn2_seg_combine_kernel<64, 128, true>) : go(gdn2_seg_combine_kernel<64, 128, false>);
  if (d_k == 128 && d_v == 64) return reverse ? go(gdn2_seg_combine_kernel<128, 64, true>) : go(gdn2_seg_combine_kernel<128, 64, false>);
  if (d_k == 128 && d_v == 128) return reverse ? go(gdn2_seg_combine_kernel<128, 128, true>) : go(gdn2_seg_combine_kernel<128, 128, false>);
  return hipErrorInvalidValue;
}

int cu_count() {
  // per device, filled on first use; concurrent first calls store the same value
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int DK, int DV, int NV>
static hipError_t launch_split(const ChunkArgs& a) {
  const bool varlen = a.cu_seqlens != nullptr;
  const long nunits = split_slots(varlen, a.B, a.T, a.N) * a.H;
  hipStream_t st = (hipStream_t)a.stream;
  if (nunits > 0) {
    const long grid1 = nunits < cu_count() ? nunits : cu_count();
    auto prep = a.gate_flags == 3 ? gdn2_prep_kernel<DK, DV, false, 3>
                : a.gate_flags == 2 ? gdn2_prep_kernel<DK, DV, false, 2>
                : a.gate_flags == 1 ? gdn2_prep_kernel<DK, DV, false, 1>
                                    : gdn2_prep_kernel<DK, DV, false, 0>;
    hipLaunchKernelGGL(prep, dim3((unsigned)grid1), dim3(512), 0, st,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.g,
                       (const bf16*)a.b, (const bf16*)a.w, (char*)a.workspace, a.cu_seqlens,
                       a.N, a.T, a.H, nunits, 1);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int nslices = DV / NV;
  if (a.nseg > 1) {
    // long sequences: transfer pass per segment, start states by a scan, outputs per segment
    const int nseg = a.nseg;
    const long units = (long)a.N * a.H * nseg;
    const size_t base = split_workspace_bytes(false, a.B, a.T, a.H, DK, DV, a.N);
    float* ebuf = reinterpret_cast<float*>((char*)a.workspace + (base + 255) / 256 * 256);
    float* sbuf = ebuf + units * DK * (DV + DK);
    // transfer slices: with d_k = d_v = 128, one of 128 value columns and one of 128
    // identity columns (8 waves, no output buffers: half the workgroups of 64-wide slices)
    constexpr int NVX = (DK == 128 && DV == 128) ? 128 : 64;
    const int xslices = (DV + DK) / NVX;
    hipLaunchKernelGGL((gdn2_state_kernel<DK, DV, NVX, 3>), dim3((unsigned)(units * xslices)),
                       dim3(StateShape<DK, DV, NVX, false>::NT), 0, st, (const char*)a.workspace,
                       nullptr, nullptr, nullptr, nullptr, a.T, a.H, xslices, (int)units, nseg,
                       a.seg_chunks, ebuf);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_seg_combine(ebuf, a.s0, sbuf, a.N, a.H, DK, DV, nseg, false, a.stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gdn2_state_kernel<DK, DV, NV, 0>), dim3((unsigned)(units * nslices)),
                       dim3(StateShape<DK, DV, NV>::NT), 0, st, (const char*)a.workspace, sbuf,
                       (bf16*)a.o, a.sN, nullptr, a.T, a.H, nslices, (int)units, nseg,
                       a.seg_chunks, nullptr);
    return hipGetLastError();
  }
  const long grid2 = (long)a.N * a.H * nslices;
  hipLaunchKernelGGL((gdn2_state_kernel<DK, DV, NV, 0>), dim3((unsigned)grid2),
                     dim3(StateShape<DK, DV, NV>::NT), 0, st, (const char*)a.workspace, a.s0,
                     (bf16*)a.o, a.sN, a.cu_seqlens, a.T, a.H, nslices, a.N * a.H, 1, 0, nullptr);
  return hipGetLastError();
}

// Backward's forward part: the factors in the backward layout, then the forward chain that
// stores every chunk's entering state and U; with a.o set (training forward) the chain
// also writes the output and, with a.sN, the final state.
template <int DK, int DV>
static hipError_t launch_bwd_forward(const ChunkArgs& a) {
  const bool varlen = a.cu_seqlens != nullptr;
  const long nunits = split_slots(varlen, a.B, a.T, a.N) * a.H;
  hipStream_t st = (hipStream_t)a.stream;
  if (nunits > 0) {
    const long grid1 = nunits < cu_count() ? nunits : cu_count();
    auto prep = a.gate_flags == 3 ? gdn2_prep_kernel<DK, DV, true, 3>
                : a.gate_flags == 2 ? gdn2_prep_kernel<DK, DV, true, 2>
                : a.gate_flags == 1 ? gdn2_prep_kernel<DK, DV, true, 1>
                                    : gdn2_prep_kernel<DK, DV, true, 0>;
    hipLaunchKernelGGL(prep, dim3((unsigned)grid1), dim3(512), 0, st,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.g,
                       (const bf16*)a.b, (const bf16*)a.w, (char*)a.workspace, a.cu_seqlens,
                       a.N, a.T, a.H, nunits, a.o != nullptr ? 1 : 0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  constexpr int NV = 64 <= DV ? 64 : DV;
  const int nslices = DV / NV;
  auto chain = a.o != nullptr ? gdn2_state_kernel<DK, DV, NV, 2> : gdn2_state_kernel<DK, DV, NV, 1>;
  if (a.nseg > 1) {
    // long sequences: transfer pass per segment (on this workspace), start states by a scan,
    // then the entering states (and o) per segment, as in the two-phase forward
    const int nseg = a.nseg;
    const long units = (long)a.N * a.H * nseg;
    float* ebuf = reinterpret_cast<float*>(
        (char*)a.workspace + (bwd_workspace_bytes(false, a.B, a.T, a.H, DK, DV, a.N) + 255) / 256 * 256);
    float* sbuf = ebuf + units * DK * (DV + DK);
    constexpr int NVX = (DK == 128 && DV == 128) ? 128 : 64;
    const int xslices = (DV + DK) / NVX;
    hipLaunchKernelGGL((gdn2_state_kernel<DK, DV, NVX, 4>), dim3((unsigned)(units * xslices)),
                       dim3(StateShape<DK, DV, NVX, false>::NT), 0, st, (const char*)a.workspace,
                       nullptr, nullptr, nullptr, nullptr, a.T, a.H, xslices, (int)units, nseg,
                       a.seg_chunks, ebuf);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_seg_combine(ebuf, a.s0, sbuf, a.N, a.H, DK, DV, nseg, false, a.stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(chain, dim3((unsigned)(units * nslices)), dim3(StateShape<DK, DV, NV>::NT), 0,
                       st, (const char*)a.workspace, sbuf, (bf16*)a.o,
                       a.o != nullptr ? a.sN : nullptr, nullptr, a.T, a.H, nslices, (int)units,
                       nseg, a.seg_chunks, nullptr);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(chain, dim3((unsigned)(a.N * a.H * nslices)),
                     dim3(StateShape<DK, DV, NV>::NT), 0, st, (const char*)a.workspace, a.s0,
                     (bf16*)a.o, a.o != nullptr ? a.sN : nullptr, a.cu_seqlens, a.T, a.H, nslices,
                     a.N * a.H, 1, 0, nullptr);
  return hipGetLastError();
}

hipError_t launch_bwd_forward_part(const ChunkArgs& a) {
  if (a.dtype != 0) return hipErrorInvalidValue;
  if (a.d_k == 64 && a.d_v == 64) return launch_bwd_forward<64, 64>(a);
  if (a.d_k == 64 && a.d_v == 128) return launch_bwd_forward<64, 128>(a);
  if (a.d_k == 128 && a.d_v == 64) return launch_bwd_forward<128, 64>(a);
  if (a.d_k == 128 && a.d_v == 128) return launch_bwd_forward<128, 128>(a);
  return hipErrorInvalidValue;
}

template <int DK, int DV>
static hipError_t dispatch_split_nv(const ChunkArgs& a) {
  if (a.nv == 32) return launch_split<DK, DV, 32>(a);
  if (a.nv == 64) return launch_split<DK, DV, 64>(a);
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_fwd_split(const ChunkArgs& a) {
  if (a.dtype != 0) return hipErrorInvalidValue;
  if (a.d_k == 64 && a.d_v == 64) return dispatch_split_nv<64, 64>(a);
  if (a.d_k == 64 && a.d_v == 128) return dispatch_split_nv<64, 128>(a);
  if (a.d_k == 128 && a.d_v == 64) return dispatch_split_nv<128, 64>(a);
  if (a.d_k == 128 && a.d_v == 128) return dispatch_split_nv<128, 128>(a);
  return hipErrorInvalidValue;
}

}  // namespace gdn2
