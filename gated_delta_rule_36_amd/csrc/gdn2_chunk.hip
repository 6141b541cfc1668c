// Chunkwise-parallel forward of Gated Delta Rule-2 on gfx950.
//
// One workgroup owns one (sequence, head, value-slice of NV columns) and walks that
// sequence's 64-token chunks in order, keeping its d_k x NV slice of the fp32 state in
// MFMA accumulator registers (wave w owns columns [16w, 16w+16)). The value columns of
// the state evolve independently (decay, read r = S_bar^T e and erase all act along the
// key axis), so slicing d_v multiplies the number of independent chains; the key-side
// work of a chunk is recomputed per slice.
//
// Per chunk (local tokens r, i in [0, 64), G = cumsum of log-decay, E = b*K, Z = w*V),
// the chunk form of the GDN-2 reading note (§3, chunkwise-training paragraph: the
// cumulative decay normalises the state so the chunk is a pure asymmetric delta
// recurrence) with the UT transform of the Gated DeltaNet visual reading (chunkwise
// section):
//   A = strict_lower( sum_c E[r,c] K[i,c] exp(G[r,c]-G[i,c]) )     (b*k) Gamma k^T
//   P = lower_incl ( sum_c Q[r,c] K[i,c] exp(G[r,c]-G[i,c]) )
//   [W | U~] = (I + A)^{-1} [E exp(G) | Z]      (UT transform, block forward substitution)
//   U = U~ - W S
//   O = (Q exp(G)) S + P U
//   S = Diag(exp(G_last)) S + (K exp(G_last - G))^T U
//
// Stages per chunk (barriers order LDS only; the next chunk's inputs are prefetched into
// registers and stay in flight across them):
//   (a) per-thread cumsum of log2-decay, (b) per-channel scan and decay factors,
//   (c) gated / decayed operands into LDS, (d) A and P on MFMA,
//   (e) 16x16 diagonal blocks of (I + A)^{-1} by forward substitution,
//   (f) block forward substitution of [E exp(G) | Z] on K=16 MFMA (no barrier inside),
//   (g) state-dependent part: U, O, state update, on this wave's 16 state columns.
//
// Range safety. exp(G[r]-G[i]) is formed as exp(G[r]) * exp(-G[i]) with G relative to
// the chunk start when the chunk's total decay is below ~83 nats in every channel (the
// usual case; both factors then fit fp32 / bf16). Otherwise the chunk takes a slower path
// that references every factor to a 16-token block boundary:
//   a_r = G_r - Gs(R)   (Gs(R): cumulative decay at the start of r's block R)
//   Ea = E exp(a), Qa = Q exp(a)  (<= |E|, |Q|)     Kn = K exp(-a)  (grows inside a block)
//   diagonal blocks:      Ea_R . Kn_R
//   off-diagonal (R > I): Ea_R * exp(Gs(R) - Ge(I)) . Kn_I * exp(Ge(I) - Gs(I))
// so no factor exceeds one block's own decay (the API requires > -80 nats per 16 tokens).
// All logs are kept in base 2 (g is scaled by log2(e) on load) so exp is one v_exp_f32.

#include "gdn2_chunk_common.h"
#include "gdn2_launch.h"

namespace gdn2 {

template <typename T, int DK, int NV>
struct ChunkShape {
  static constexpr int C = 64;            // chunk length
  static constexpr int NWC = NV / 16;     // 16-wide state column tiles
  // Row split: with bf16 and d_k = 128, two waves share each column tile, one per half of
  // the key rows (two waves per SIMD for latency hiding); partial sums over the key rows
  // are exchanged through LDS.
  static constexpr int RS = (sizeof(T) == 2 && DK == 128 && NV <= 64) ? 2 : 1;
  static constexpr int NW = NWC * RS;     // waves: wave w owns column tile w % NWC and
                                          // key rows [(w / NWC) * DK / RS, ... + DK / RS)
  static constexpr int NT = 64 * NW;      // threads
  static constexpr int CG = DK / 8;       // key-side prep: 8 channels per thread
  static constexpr int TG = NT / CG;      // token groups
  static constexpr int TPT = C / TG;      // tokens per thread (all inside one 16-block)
  static constexpr int GPB = 16 / TPT;    // token groups per 16-token block
  static constexpr int VCG = NV / 8;      // value-side prep: 8 columns per thread
  static constexpr int VTG = NT / VCG;
  static constexpr int VTPT = C / VTG;
  // Row padding. The LDS has 128 four-byte banks and serves a 16-byte read in two passes of
  // 32 lanes; a fragment read covers 16 rows x 2 slots per pass, which is free of bank
  // conflicts when the row pitch is an odd multiple of 8 words (bf16 rows of DK + 16 and
  // C + 16 elements; with 8 elements of padding every such read took two passes per half).
  static constexpr int PAD = sizeof(T) == 2 ? 16 : 4;
  static constexpr int LDK = DK + PAD;    // pitch of [64][DK] arrays
  static constexpr int LDT = C + PAD;     // pitch of [x][64] arrays
  static constexpr int KS = Mma<T>::KS;
  static constexpr int KPL = Mma<T>::KPL;
  static constexpr int NCT = DK / 16;     // 16-wide key-channel tiles

  static constexpr int NF = Fac::N;  // factor rows (fp32, [NF][DK])

  // LDS layout (bytes)
  static constexpr int SZ_K = C * LDK * (int)sizeof(T);
  static constexpr int OFF_E = 0;                  // E exp(G) (or Ea); later -W
  static constexpr int OFF_Q = OFF_E + SZ_K;       // Q exp(G) (or Qa, rescaled in (e))
  static constexpr int OFF_K = OFF_Q + SZ_K;       // K exp(-G) (or K exp(Ge(block) - G))
  static constexpr int SZ_T = DK * LDT * (int)sizeof(T);
  static constexpr int OFF_ET = OFF_K + SZ_K;      // (E exp(G))^T        [DK][64]
  static constexpr int OFF_KT = OFF_ET + SZ_T;     // (K exp(Gl - G))^T   [DK][64]
  static constexpr int SZ_Z = NV * LDT * (int)sizeof(T);
  static constexpr int OFF_ZT = OFF_KT + SZ_T;     // Z^T                 [NV][64]
  static constexpr int SZ_P = C * LDT * (int)sizeof(T);
  static constexpr int OFF_P = OFF_ZT + SZ_Z;      // P                   [64][64]
  static constexpr int OFF_A = OFF_P + SZ_P;       // -A                  [64][64]
  static constexpr int OFF_TB = OFF_A + SZ_P;      // diagonal blocks of (I+A)^-1
  static constexpr int OFF_FAC = OFF_TB + SZ_P;
  static constexpr int SZ_FAC = NF * DK * 4;
  // fp32 copy of the four diagonal 16x16 blocks of -A for the triangular inverse (the
  // fp32 path reads them from the -A buffer itself)
  static constexpr int LDD = 20;  // pitch (floats)
  static constexpr int SZ_AD = sizeof(T) == 4 ? 0 : 4 * 16 * LDD * 4;
  static constexpr int OFF_AD = OFF_FAC + SZ_FAC;
  static constexpr int OFF_FLAG = OFF_AD + SZ_AD;
  static constexpr int LDS_BYTES = OFF_FLAG + 16;
  // cumsum scratch [TG][DK] fp32 lives in the P and -A buffers (dead until (d))
  static constexpr int OFF_TOT = OFF_P;

  static_assert(NV % 16 == 0 && NV >= 16 && NV <= 128, "value slice");
  static_assert(TPT >= 1 && TPT <= 16 && 16 % TPT == 0, "token groups must tile 16-blocks");
  static_assert(VTPT >= 1 && C % VTG == 0, "value prep mapping");
  static_assert(32 * NT <= 2 * SZ_P, "cumsum scratch fits in P and -A");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  // row-split exchange of partial sums (f4 per lane): U partials (4 tiles) in the K and
  // E^T buffers, O partials (2 tiles) in the -A and T buffers; all dead in (g)
  static_assert(RS == 1 || (NW <= 8 && 4 * 4096 <= SZ_K && 4 * 4096 <= SZ_T &&
                            NW * 2048 <= 2 * SZ_P), "row-split exchange space");
};


// GL: the gate layout this build reads (kGateBScalar | kGateWScalar bits); each layout has
// its own build, so every load is unconditional in the layout's own form.
template <typename T, int DK, int NV, int GL>
__global__ void __launch_bounds__((ChunkShape<T, DK, NV>::NT))
gdn2_chunk_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                  const T* __restrict__ g, const T* __restrict__ bg, const T* __restrict__ wg,
                  const float* s0, T* __restrict__ o, float* sN,
                  const int* __restrict__ cu_seqlens, int T_len, int H, int DV, int nslices,
                  int nunits, int gflags) {
  using Sh = ChunkShape<T, DK, NV>;
  using M = Mma<T>;
  constexpr int C = Sh::C, NW = Sh::NW, NT = Sh::NT, KS = Sh::KS, KPL = Sh::KPL;
  constexpr int LDK = Sh::LDK, LDT = Sh::LDT, NCT = Sh::NCT;
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
  int* sFlag = reinterpret_cast<int*>(smem + Sh::OFF_FLAG);
  // diagonal blocks of -A in fp32: block jb, row r, column i at sAd[jb*ADB + r*ADP + i]
  constexpr int ADB = sizeof(T) == 4 ? 16 * LDT + 16 : 16 * Sh::LDD;
  constexpr int ADP = sizeof(T) == 4 ? LDT : Sh::LDD;
  float* sAd = sizeof(T) == 4 ? reinterpret_cast<float*>(smem + Sh::OFF_A)
                              : reinterpret_cast<float*>(smem + Sh::OFF_AD);

  constexpr int RS = Sh::RS, NWC = Sh::NWC;
  constexpr int NMS = NCT / RS;       // state row tiles per wave
  constexpr int KSH = DK / KS / RS;   // K steps per wave over its key rows
  int tid = threadIdx.x;
  int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wct = wave % NWC;         // this wave's state column tile
  const int whw = wave / NWC;         // this wave's half of the key rows (row split)
  int m16 = lane & 15;  // row (A operand) / column (B, D) inside a 16x16 tile
  int g4 = lane >> 4;   // lane group
  // re-derive the lane indices opaquely at each stage (see opaque())
  auto fresh_lane = [&]() {
    tid = opaque(tid);
    lane = tid & 63;
    m16 = lane & 15;
    g4 = lane >> 4;
  };

  // Workgroup -> (sequence, head, slice). Workgroups are dealt round-robin to the 8 XCDs
  // (each with its own L2), so the slices of one (sequence, head) are given workgroup ids
  // that are congruent mod 8: they run on the same XCD at the same time and the second
  // read of the shared key-side inputs is served by that XCD's L2.
  const int units = nunits;                       // sequences * heads
  const int grp = blockIdx.x / (8 * nslices);     // group of 8 (sequence, head) units
  const int gsz = min(8, units - grp * 8);        // units in this group
  const int gi = blockIdx.x - grp * 8 * nslices;  // index inside the group
  const int slice = gi / gsz;
  const int nh = grp * 8 + gi % gsz;
  const int h = nh % H;
  const int n = nh / H;
  const int col0 = slice * NV;  // first state / value column of this workgroup

  // token range of this sequence, as rows of the [rows, H, d] token arrays
  long row0;
  int len;
  if (cu_seqlens != nullptr) {
    int a = cu_seqlens[n], b = cu_seqlens[n + 1];
    a = a < 0 ? 0 : (a > T_len ? T_len : a);
    b = b < a ? a : (b > T_len ? T_len : b);
    row0 = a;
    len = b - a;
  } else {
    row0 = (long)n * T_len;
    len = T_len;
  }
  const long kstride = (long)H * DK;  // elements between consecutive tokens
  const long vstride = (long)H * DV;
  const T* qb = q + row0 * kstride + (long)h * DK;
  const T* kb = k + row0 * kstride + (long)h * DK;
  const T* gb = g + row0 * kstride + (long)h * DK;
  const T* bb = bg + row0 * kstride + (long)h * DK;
  const T* vb = v + row0 * vstride + (long)h * DV + col0;
  const T* wb = wg + row0 * vstride + (long)h * DV + col0;
  // scalar gates ([rows, H]: one value per token and head, broadcast over the channels)
  constexpr bool b_scalar = (GL & kGateBScalar) != 0;
  constexpr bool w_scalar = (GL & kGateWScalar) != 0;
  (void)gflags;
  const T* bsb = bg + row0 * H + h;  // a scalar gate: one value per (token, head)
  const T* wsb = wg + row0 * H + h;
  T* ob = o + row0 * vstride + (long)h * DV + col0;

  // ---- prep thread mapping
  int cg = tid % Sh::CG;        // channel group: channels [8cg, 8cg+8)
  int tg = tid / Sh::CG;        // token group: tokens [tg*TPT, tg*TPT+TPT)
  int blk = tg / Sh::GPB;       // 16-token block of those tokens
  int vcg = tid % Sh::VCG;      // value columns [8vcg, 8vcg+8)
  int vtg = tid / Sh::VCG;      // tokens [vtg*VTPT, ...)
  auto fresh_prep = [&]() {
    fresh_lane();
    cg = tid % Sh::CG;
    tg = tid / Sh::CG;
    blk = tg / Sh::GPB;
    vcg = tid % Sh::VCG;
    vtg = tid / Sh::VCG;
  };

  Vec8<T> rq[Sh::TPT], rk[Sh::TPT], rg[Sh::TPT], rb[Sh::TPT];
  Vec8<T> rv[Sh::VTPT], rw[Sh::VTPT];

  auto load_raw = [&](int c0, int nvalid) {
#pragma unroll
    for (int j = 0; j < Sh::TPT; ++j) {
      const int r = tg * Sh::TPT + j;
      if (r < nvalid) {
        const long off = (long)(c0 + r) * kstride + cg * 8;
        rq[j].load(qb + off);
        rk[j].load(kb + off);
        rg[j].load(gb + off);
        // a scalar gate is read as the aligned 8-element block that holds it (the same
        // load instruction in both layouts keeps the prefetch's waits precise); its element
        // is picked out when the chunk is consumed
        if constexpr (b_scalar) rb[j].load_one(bsb + (long)(c0 + r) * H);
        else rb[j].load(bb + off);
      } else {
        rq[j].zero(); rk[j].zero(); rg[j].zero(); rb[j].zero();
      }
    }
#pragma unroll
    for (int j = 0; j < Sh::VTPT; ++j) {
      const int r = vtg * Sh::VTPT + j;
      if (r < nvalid) {
        const long off = (long)(c0 + r) * vstride + vcg * 8;
        rv[j].load(vb + off);
        if constexpr (w_scalar) rw[j].load_one(wsb + (long)(c0 + r) * H);
        else rw[j].load(wb + off);
      } else {
        rv[j].zero(); rw[j].zero();
      }
    }
  };

  // ---- state slice in accumulator registers: local tile m holds key rows
  // [16(whw*NMS + m), +16), columns col0 + 16*wct + m16; lane holds rows ... + 4*g4 + i.
  f4 S[NMS];
  const long sbase = ((long)n * H + h) * DK * DV + col0 + 16 * wct + m16;
#pragma unroll
  for (int mt = 0; mt < NMS; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = 16 * (whw * NMS + mt) + 4 * g4 + i;
      S[mt][i] = (s0 != nullptr) ? s0[sbase + (long)ch * DV] : 0.f;
    }
  }

  // Output tiles are staged in LDS (in the Z^T buffer, dead after (f)). The next chunk
  // reads the staging into registers in (a) and issues the 16-byte global stores at the end
  // of (c), just before its prefetch loads: the wait for those loads (vmcnt counts stores
  // too) then comes one full chunk after the stores.
  constexpr int OP = (64 * (NV + Sh::PAD) <= NV * LDT) ? NV + Sh::PAD : NV;  // staging pitch
  constexpr int EPC = 16 / (int)sizeof(T);        // elements per 16-byte chunk
  constexpr int CPT = C * NV / EPC / NT;          // chunks per thread
  static_assert(CPT * NT * EPC == C * NV, "output staging mapping");
  T* const sO = sZt;
  int prev_c0 = 0, prev_n = 0;
  uint4 ostage[CPT];
  auto stage_load = [&]() {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int idx = tid + j * NT;
      const int r = idx / (NV / EPC), cc = idx % (NV / EPC);
      ostage[j] = *reinterpret_cast<const uint4*>(sO + r * OP + cc * EPC);
    }
  };
  auto stage_store = [&](int oc0, int on) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int idx = tid + j * NT;
      const int r = idx / (NV / EPC), cc = idx % (NV / EPC);
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      if (r < on)  // o is written once and not read back here: non-temporal
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, ostage[j]),
                                    reinterpret_cast<u32x4*>(ob + (long)(oc0 + r) * vstride + cc * EPC));
    }
  };

  const int nchunks = (len + C - 1) / C;
  if (nchunks > 0) load_raw(0, len < C ? len : C);

  for (int ci = 0; ci < nchunks; ++ci) {
    const int c0 = ci * C;
    const int nvalid = (len - c0) < C ? (len - c0) : C;
    lds_barrier();  // the previous chunk's readers of every buffer are done
    fresh_prep();

    // ---- (a) previous chunk's output to HBM; per-thread totals of log2-decay
    if (ci > 0) stage_load();
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
    fresh_prep();

    // ---- (b) per-channel scan over token groups: chunk-relative exclusive prefixes
    // and the per-channel decay factors
    channel_scan<DK, Sh::TG, Sh::GPB, NT>(sTot, sFac, sFlag, tid);
    lds_barrier();
    fresh_prep();
    const bool block_path = __builtin_amdgcn_readfirstlane(*sFlag) != 0;

    // ---- (c) gated, decayed operands (token by token, running cumsum of log2-decay)
    {
      float run[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) run[i] = sTot[tg * DK + cg * 8 + i];
      RunBuf<T, Sh::TPT> ev[8], kv[8];  // E exp(G) and K exp(Glast - G), per channel
      // one token of this thread: x = G (chunk path) or G - Gs(block) (block path, where K
      // takes Ge(block) - G)
      auto token = [&](int j, const float* sub, const float* subk, const float* fA,
                       const float* fB, bool scaled) {
        const int r = tg * Sh::TPT + j;
        float fg[8], fq[8], fk[8], fb[8], e1[8], q1[8], k1[8];
        rg[j].to_float(fg);
        rq[j].to_float(fq);
        rk[j].to_float(fk);
        if constexpr (b_scalar) rb[j].splat();
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
      const int sw = tswz(cg * 8);  // same for the thread's 8 channels
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
        if constexpr (w_scalar) rw[j].splat();
        rw[j].to_float(fw);
#pragma unroll
        for (int i = 0; i < 8; ++i) zv[i].put(j, fv[i] * fw[i]);
      }
      const int zsw = tswz(vcg * 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) zv[i].store_sw(sZt + (vcg * 8 + i) * LDT, zsw, vtg * Sh::VTPT);
    }
    if (ci > 0) stage_store(prev_c0, prev_n);
    // prefetch the next chunk; the loads stay in flight until (a) of the next chunk
    if (ci + 1 < nchunks) {
      const int nn = len - c0 - C;
      load_raw(c0 + C, nn < C ? nn : C);
    }
    lds_barrier();
    fresh_prep();

    // ---- (d) A (stored negated) and P, and the diagonal blocks of (I + A)^{-1}.
    // Chunk path: the wave(s) that invert form their diagonal A tiles themselves and go
    // straight on to the inverse blocks (fp32 forward substitution, one block per 16-lane
    // group, one column per lane), with no barrier in between: with 8 waves the last two
    // take two blocks each, otherwise the last wave all four. The other waves form the
    // other tiles and then their partial Q exp(G) S products.
    constexpr int TDW = NW - 1;  // (last) wave that forms diagonal inverse blocks
    typename M::frag sb[KSH];    // this wave's state rows as B operands
#pragma unroll
    for (int s = 0; s < KSH; ++s) sb[s] = M::from_acc(S, s);
    f4 O[4];
    auto o_partial = [&]() {  // O = Q exp(G) S over this wave's key rows
      typename M::frag qf[4][KSH];
#pragma unroll
      for (int R = 0; R < 4; ++R)
#pragma unroll
        for (int s = 0; s < KSH; ++s) qf[R][s] = M::load_phi(sQ, LDK, 16 * R + m16, whw * KSH + s, g4);
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        O[R] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSH; ++s) O[R] = M::mma(qf[R][s], sb[s], O[R]);
      }
    };
    auto tdiag = [&]() { diag_inverse<T, LDT, ADB, ADP>(sAd, sT, m16, g4); };
    // pair bits: (0,0)=0 (1,0)=1 (1,1)=2 (2,0)=3 (2,1)=4 (2,2)=5 (3,0)=6 (3,1)=7 (3,2)=8 (3,3)=9
    constexpr int DIAG = 0x225;     // (0,0) (1,1) (2,2) (3,3)
    constexpr int OFFD = 0x1DA;     // off-diagonal pairs
    if (!block_path) {
      if constexpr (NW >= 8) {
        if (wave >= TDW - 1) {
          if (wave == TDW) ap_tiles<T, DK, LDK, LDT, 0x005, 0>(sE, sQ, sK, sAm, sP, sAd, m16, g4);
          else ap_tiles<T, DK, LDK, LDT, 0x220, 0>(sE, sQ, sK, sAm, sP, sAd, m16, g4);
          // reads only what this wave just wrote: no barrier needed
          diag_inverse_pair<T, LDT, ADB, ADP>(sAd, sT, m16, g4, wave == TDW ? 0 : 2);
        } else {
          switch (wave) {
            case 0: ap_tiles<T, DK, LDK, LDT, 0x0C0, 0>(sE, sQ, sK, sAm, sP, sAd, m16, g4); break;
            case 1: ap_tiles<T, DK, LDK, LDT, 0x118, 0>(sE, sQ, sK, sAm, sP, sAd, m16, g4); break;
            case 2: ap_tiles<T, DK, LDK, LDT, 0x002, 0x003>(sE, sQ, sK, sAm, sP, sAd, m16, g4); break;
            case 3: ap_tiles<T, DK, LDK, LDT, 0, 0x0C0>(sE, sQ, sK, sAm, sP, sAd, m16, g4); break;
            case 4: ap_tiles<T, DK, LDK, LDT, 0, 0x304>(sE, sQ, sK, sAm, sP, sAd, m16, g4); break;
            case 5: ap_tiles<T, DK, LDK, LDT, 0, 0x038>(sE, sQ, sK, sAm, sP, sAd, m16, g4); break;
            default: break;
          }
          o_partial();
        }
      } else if (wave == TDW) {
        if constexpr (NW == 1) {
          ap_tiles<T, DK, LDK, LDT, 0x3FF, 0x3FF>(sE, sQ, sK, sAm, sP, sAd, m16, g4);
        } else if constexpr (NW == 2) {
          ap_tiles<T, DK, LDK, LDT, DIAG, 0x3C1>(sE, sQ, sK, sAm, sP, sAd, m16, g4);
        } else {
          ap_tiles<T, DK, LDK, LDT, DIAG, 0>(sE, sQ, sK, sAm, sP, sAd, m16, g4);
        }
        tdiag();  // reads only what this wave just wrote: no barrier needed
      } else {
        if constexpr (NW >= 4) {
          switch (wave) {
            case 0: ap_tiles<T, DK, LDK, LDT, OFFD, 0>(sE, sQ, sK, sAm, sP, sAd, m16, g4); break;
            case 1: ap_tiles<T, DK, LDK, LDT, 0, 0x3C1>(sE, sQ, sK, sAm, sP, sAd, m16, g4); break;
            case 2: ap_tiles<T, DK, LDK, LDT, 0, 0x03E>(sE, sQ, sK, sAm, sP, sAd, m16, g4); break;
            default: break;
          }
        } else if constexpr (NW == 2) {
          ap_tiles<T, DK, LDK, LDT, OFFD, 0x03E>(sE, sQ, sK, sAm, sP, sAd, m16, g4);
        }
        o_partial();
      }
    } else {
      ap_tiles_block<T, DK, LDK, LDT, NW>(sE, sQ, sK, sAm, sP, sFac, wave, lane);
      diag_tiles_pairwise<T, DK, LDT, ADB, ADP, NT, b_scalar>(
          qb + (long)c0 * kstride, kb + (long)c0 * kstride, gb + (long)c0 * kstride,
          bb + (long)c0 * kstride, bsb + (long)c0 * H, kstride, H, nvalid, tid, sAd, sP);
    }
    zero_p_upper<T, LDT, NT>(sP, tid);
    lds_barrier();
    fresh_prep();
    if (block_path) {
      // block path: inverse blocks by the last wave; the others rescale Qa to Q exp(G)
      if (wave == TDW) tdiag();
      const int nthr = NW > 1 ? NT - 64 : NT;
      const int t0 = (NW == 1 || tid < TDW * 64) ? tid : -1;
      for (int idx = t0; idx >= 0 && idx < C * DK; idx += nthr) {
        const int r = idx / DK, pc = idx % DK;
        sQ[r * LDK + pc] = from_f<T>(to_f(sQ[r * LDK + pc]) *
                                     sFac[(Fac::ES + r / 16) * DK + M::phi_inv(pc)]);
      }
      lds_barrier();
      fresh_prep();
    }

    // ---- (f) [W | U~] = (I + A)^{-1} [E exp(G) | Z] by block forward substitution:
    //   X_R = T_RR (RHS_R - sum_{J<R} A_RJ X_J)
    // Each wave owns whole column tiles, so the rounds need no barrier. Key-channel tiles
    // are dealt round-robin; the wave's own value tile gives U~ in registers.
    f4 U[4];
    {
      constexpr int NE = (NCT + NW - 1) / NW;  // key-channel tiles per wave (max)
      using F16 = Frag16<T>;
      // the A_RJ (J < R) and T_RR fragments are the same for every tile of this wave
      typename F16::type fa[4][4];
#pragma unroll
      for (int R = 0; R < 4; ++R) {
#pragma unroll
        for (int J = 0; J < R; ++J) fa[R][J] = F16::load(sAm + (16 * R + m16) * LDT + 16 * J + 4 * g4);
        fa[R][R] = F16::load(sT + (16 * R + m16) * LDT + 16 * R + 4 * g4);
      }
      f4 X[NE + 1][4];
      typename F16::type Xb[NE + 1][4];  // X as B fragments, converted once
#pragma unroll
      for (int R = 0; R < 4; ++R) {
#pragma unroll
        for (int t = 0; t <= NE; ++t) {
          const int ct = wave + t * NW;
          const bool isZ = (t == NE);
          if constexpr (NCT % NW != 0) {
            if (!isZ && ct >= NCT) continue;
          }
          if constexpr (RS > 1) {
            if (isZ && whw != 0) continue;
          }
          const int crow = isZ ? 16 * wct + m16 : 16 * ct + m16;
          const T* src = (isZ ? sZt : sEt) + crow * LDT;
          f4 acc = load4f(src + tcol(crow, 16 * R + 4 * g4));  // RHS rows 16R+4g4+i, col m16
#pragma unroll
          for (int J = 0; J < R; ++J) acc = mma16_frag(fa[R][J], Xb[t][J], acc);
          X[t][R] = mma16_frag(fa[R][R], F16::from_acc(acc), f4{0.f, 0.f, 0.f, 0.f});
          Xb[t][R] = F16::from_acc(X[t][R]);
        }
      }
#pragma unroll
      for (int t = 0; t < NE; ++t) {
        const int ct = wave + t * NW;
        if constexpr (NCT % NW != 0) {
          if (ct >= NCT) continue;
        }
#pragma unroll
        for (int R = 0; R < 4; ++R)
          store_tile_pairs(sWm + (16 * R) * LDK, LDK, lane, -X[t][R],
                           [&](int c) { return M::phi(16 * ct + c); });
      }
#pragma unroll
      for (int R = 0; R < 4; ++R) U[R] = (RS == 1 || whw == 0) ? X[NE][R] : f4{0.f, 0.f, 0.f, 0.f};
    }
    if ((wave == TDW || (NW >= 8 && wave == TDW - 1)) && !block_path) o_partial();
    lds_barrier();
    fresh_prep();

    // ---- (g) state-dependent part (this wave's 16 columns and key rows)
    if (block_path) o_partial();
    // partial sums over this wave's key rows: U = U~ - W S
    {
      typename M::frag wf[4][KSH];
#pragma unroll
      for (int R = 0; R < 4; ++R)
#pragma unroll
        for (int s = 0; s < KSH; ++s) wf[R][s] = M::load_phi(sWm, LDK, 16 * R + m16, whw * KSH + s, g4);
#pragma unroll
      for (int R = 0; R < 4; ++R) {
#pragma unroll
        for (int s = 0; s < KSH; ++s) U[R] = M::mma(wf[R][s], sb[s], U[R]);
      }
    }
    // output row tiles finished by this wave: all (no split) or {0,3} / {1,2}
    if constexpr (RS > 1) {
      // exchange partial sums with the partner wave (same columns, other key rows)
      f4* xu_mine = reinterpret_cast<f4*>((wave < 4 ? smem + Sh::OFF_K : smem + Sh::OFF_ET)) +
                    (wave & 3) * 256;
      f4* xo_mine = reinterpret_cast<f4*>(smem + Sh::OFF_A) + wave * 128;
      const int pw = wave ^ NWC;  // partner wave (NWC = 4 or 2 divides the wave index)
      const f4* xu_part = reinterpret_cast<const f4*>((pw < 4 ? smem + Sh::OFF_K : smem + Sh::OFF_ET)) +
                          (pw & 3) * 256;
      const f4* xo_part = reinterpret_cast<const f4*>(smem + Sh::OFF_A) + pw * 128;
#pragma unroll
      for (int R = 0; R < 4; ++R) xu_mine[R * 64 + lane] = U[R];
      // the partner finishes the other two output row tiles
      if (whw == 0) {
        xo_mine[lane] = O[1];
        xo_mine[64 + lane] = O[2];
      } else {
        xo_mine[lane] = O[0];
        xo_mine[64 + lane] = O[3];
      }
      lds_barrier();
#pragma unroll
      for (int R = 0; R < 4; ++R) U[R] += xu_part[R * 64 + lane];
      if (whw == 0) {
        O[0] += xo_part[lane];
        O[3] += xo_part[64 + lane];
      } else {
        O[1] += xo_part[lane];
        O[2] += xo_part[64 + lane];
      }
    }
    typename M::frag ub[C / KS];
#pragma unroll
    for (int s = 0; s < C / KS; ++s) ub[s] = M::from_acc(U, s);
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      if (RS > 1 && (whw == 0 ? (R == 1 || R == 2) : (R == 0 || R == 3))) continue;
#pragma unroll
      for (int s = 0; s < causal_steps<KS>(R); ++s)
        O[R] = M::mma(M::load_phi(sP, LDT, 16 * R + m16, s, g4), ub[s], O[R]);
      store_tile_pairs(sO + (16 * R) * OP + 16 * wct, OP, lane, O[R], [](int c) { return c; });
    }
    prev_c0 = c0;
    prev_n = nvalid;
    // S <- Diag(exp(Glast)) S + (K exp(Glast - G))^T U   (this wave's key rows)
#pragma unroll
    for (int mt = 0; mt < NMS; ++mt) {
      const int mg = whw * NMS + mt;
      const f4 gam = *reinterpret_cast<const f4*>(sFac + Fac::GAM * DK + 16 * mg + 4 * g4);
      f4 acc = S[mt] * gam;
#pragma unroll
      for (int s = 0; s < C / KS; ++s)
        acc = M::mma(M::load_phi_t(sKt, LDT, 16 * mg + m16, s, g4), ub[s], acc);
      S[mt] = acc;
    }
  }

  if (nchunks > 0) {
    lds_barrier();
    fresh_lane();
    stage_load();
    stage_store(prev_c0, prev_n);
  }
  if (sN != nullptr) {
#pragma unroll
    for (int mt = 0; mt < NMS; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ch = 16 * (whw * NMS + mt) + 4 * g4 + i;
        sN[sbase + (long)ch * DV] = S[mt][i];
      }
    }
  }
}

template <typename T, int DK, int NV>
static hipError_t launch_chunk(const ChunkArgs& a) {
  const int nslices = a.d_v / NV;
  const long grid = (long)a.N * a.H * nslices;
  auto kern = a.gate_flags == 3 ? gdn2_chunk_kernel<T, DK, NV, 3>
              : a.gate_flags == 2 ? gdn2_chunk_kernel<T, DK, NV, 2>
              : a.gate_flags == 1 ? gdn2_chunk_kernel<T, DK, NV, 1>
                                  : gdn2_chunk_kernel<T, DK, NV, 0>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid),
                     dim3(ChunkShape<T, DK, NV>::NT), 0,
                     (hipStream_t)a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v,
                     (const T*)a.g, (const T*)a.b, (const T*)a.w, a.s0, (T*)a.o, a.sN,
                     a.cu_seqlens, a.T, a.H, a.d_v, nslices, a.N * a.H, a.gate_flags);
  return hipGetLastError();
}

// Value-slice widths built per (dtype, d_k): 16-wide slices only for d_k = 64 (with
// d_k = 128 a 64-thread workgroup would hold 16 tokens of raw inputs per thread), and
// no 128-wide fp32 slice (LDS).
template <typename T, int DK>
static hipError_t dispatch_nv(const ChunkArgs& a) {
  if constexpr (DK == 64) {
    if (a.nv == 16) return launch_chunk<T, DK, 16>(a);
  }
  if (a.nv == 32) return launch_chunk<T, DK, 32>(a);
  if (a.nv == 64) return launch_chunk<T, DK, 64>(a);
  if constexpr (sizeof(T) == 2) {
    if (a.nv == 128) return launch_chunk<T, DK, 128>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_fwd(const ChunkArgs& a) {
  if (a.dtype == 0) {
    if (a.d_k == 64) return dispatch_nv<bf16, 64>(a);
    if (a.d_k == 128) return dispatch_nv<bf16, 128>(a);
  } else {
    if (a.d_k == 64) return dispatch_nv<float, 64>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn2
