// Chunkwise backward of Gated Delta Rule-2 on gfx950 (bf16 inputs).
//
// The gradient of the state flows backwards through the asymmetric factor of every token
// (GDN-2 reading note, §3 gate-aware backward paragraph); in chunk form, with the chunk
// quantities of the forward (gdn2_split.hip) and dSn the gradient of the state leaving
// the chunk:
//   recurrence (sequential over chunks, per value column):
//     dU  = P^T dO + Ktil dSn,   dZ = T^T dU   (T = (I + A)^{-1}, block back-substitution)
//     dS0 = Qbar^T dO + Diag(gamma) dSn - W^T dU           (gradient of the entering state)
//   local (parallel over chunks), with U = U~ - W S0 and S0 the entering state:
//     M1 = lower_incl(dO U^T),   M2 = -strict(dZ U^T)      (M2 is dA)
//     dQbar = dO S0^T + M1 Khat,   dEbar = -dZ S0^T + M2 Khat,
//     dKhat = M2^T Ebar + M1^T Qbar,   dKtil = U dSn^T
//   then the elementwise chain through 2^(+-G), e = b*k, z = w*v and G = cumsum(g).
// The regrouping T^T dW = -dZ S0^T (dW = -dU S0^T) leaves one triangular solve per chunk and
// makes dA = -strict(dZ U^T), so the local part needs neither T nor A.
//
// Pipeline (all per (chunk slot, head) unit of the backward workspace, BwdLayout):
//   1. factor kernel (backward layout) and forward chain storing S0 and U per chunk
//      (gdn2_split.hip);
//   2. gdn2_bwd_chain_kernel: the recurrence, storing dSn and dZ per chunk, and dS0 of the
//      sequence;
//   3. gdn2_bwd_local_kernel: every chunk's gradients of q, k, g, b (and v, w = dZ*w, dZ*v).
// The local kernel references every decay factor to the middle of the chunk's decay
// range, Gm = Glast / 2 per channel: it forms Khat' = K 2^(Gm - G), Qbar' = Q 2^(G - Gm),
// Ebar' = E 2^(G - Gm) and the entering state's rows scaled by 2^Gm, so that the products
// above keep their values up to those per-channel factors (undone in the elementwise
// chain) while no factor exceeds half the chunk's decay. Chunks whose total decay exceeds
// twice the forward's chunk-referenced range (166 nats in some channel) are flagged.

#include "gdn2_chunk_common.h"
#include "gdn2_launch.h"

namespace gdn2 {

// 16 bytes at byte offset `off` from `base` (uniform), non-temporal (the `nt` policy bit):
// for data one workgroup reads once, so that it streams through the caches instead of
// displacing what neighbouring workgroups share in L2.
__device__ __forceinline__ uint4 load16_nt(const void* base, int off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7ffffff0, 0x00020000);
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}

// ------------------------------------------------------------------ the recurrence
template <int DK, int DV, int NV>
struct ChainShape {
  static constexpr int C = 64;
  static constexpr int NWV = NV / 16;  // waves: wave w owns gradient columns [16w, 16w+16)
  static constexpr int NT = 64 * NWV;
  static constexpr int KSK = DK / 32;
  static constexpr int NMT = DK / 16;
  static constexpr BwdLayout LB = BwdLayout(DK, DV);
  // staged per chunk: [Kr | Pt | Qt | Wt | Bt] (contiguous in the unit), gamma, dO^T slice
  static constexpr int OFF_KR = 0;
  static constexpr int OFF_PT = (int)(LB.pt - LB.kr);
  static constexpr int OFF_QT = (int)(LB.qt - LB.kr);
  static constexpr int OFF_WT = (int)(LB.wt - LB.kr);
  static constexpr int OFF_BT = (int)(LB.bt - LB.kr);
  static constexpr int SZ_F = (int)(LB.factors - LB.kr);
  static constexpr int OFF_G = SZ_F;
  static constexpr int NPF = (SZ_F + DK * 4) / 16;      // 16-byte pieces of factors + gamma
  static constexpr int PPF = (NPF + NT - 1) / NT;       // ... per thread (tail re-reads)
  static constexpr int LDO = C + 8;                     // dO^T pitch: [column][token]
  static constexpr int OFF_DO = PPF * NT * 16;
  static constexpr int NPD = C * NV / 8;                // dO pieces: 8 columns of a token
  static constexpr int PPD = NPD / NT;
  static constexpr int STAGE = OFF_DO + NV * LDO * 2;
  static constexpr int LDS_BYTES = 2 * STAGE;
  static_assert(NPD % NT == 0, "dO pieces per thread");
  static_assert(STAGE % 16 == 0 && LDS_BYTES <= 160 * 1024, "LDS budget");
};

// XFER (segment transfer pass of a long sequence): the chain runs from a zero gradient with
// dO and writes the segment's start value b (the affine part of its map of the gradient,
// D_start = A D_end + b) into the value columns of ebuf, nothing being stored per chunk. The
// linear part A is the transpose of the forward transfer pass's M for the same segment (the
// gradient of a linear map is its transpose), which that pass left in the other columns of the
// same buffer. Segments: a unit is (sequence, head, segment); with nseg > 1 the gradient at a
// segment's end comes from dbuf[unit] (the reverse combine), and only segment 0 writes the
// initial state's gradient.
template <int DK, int DV, int NV, bool XFER>
__global__ void __launch_bounds__((ChainShape<DK, DV, NV>::NT)) __attribute__((amdgpu_waves_per_eu(1, 1)))
gdn2_bwd_chain_kernel(char* __restrict__ ws, const bf16* __restrict__ d_o,
                      const float* __restrict__ d_sN, float* __restrict__ d_s0,
                      const int* __restrict__ cu_seqlens, int T_len, int H, int nslices,
                      int nunits, int nseg, int seg_chunks, float* __restrict__ ebuf,
                      const float* __restrict__ dbuf) {
  typedef bf16 T;
  using Sh = ChainShape<DK, DV, NV>;
  using M = Mma<T>;
  constexpr BwdLayout LB(DK, DV);
  constexpr int C = Sh::C, NT = Sh::NT, KSK = Sh::KSK, NMT = Sh::NMT;
  __shared__ __attribute__((aligned(16))) char smem[Sh::LDS_BYTES];

  int tid = threadIdx.x;
  int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int m16 = lane & 15, g4 = lane >> 4;

  // workgroup -> (sequence, head, slice); slices of one head share an XCD (ids congruent
  // mod 8), as in the forward recurrence
  const int grp = blockIdx.x / (8 * nslices);
  const int gsz = min(8, nunits - grp * 8);
  const int gi = blockIdx.x - grp * 8 * nslices;
  const int slice = gi / gsz;
  const int unit_id = grp * 8 + gi % gsz;  // (sequence * H + head) * nseg + segment
  const int seg = unit_id % nseg;
  const int nh = unit_id / nseg;
  const int h = nh % H;
  const int n = nh / H;
  const int col0 = slice * NV;
  const int ctg = slice * Sh::NWV + wave;  // this wave's column tile within d_v

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

  // gradient of the state leaving the current chunk: tile mt holds rows [16mt, +16),
  // column col0 + 16*wave + m16 (lane rows 4*g4 + i)
  f4 D[NMT];
  const long sbase = ((long)n * H + h) * DK * DV + col0 + 16 * wave + m16;
  const long dbase = (long)unit_id * DK * DV + col0 + 16 * wave + m16;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * mt + 4 * g4 + i;
      if constexpr (XFER)
        D[mt][i] = 0.f;
      else if (nseg > 1)
        D[mt][i] = dbuf[dbase + (long)row * DV];
      else
        D[mt][i] = d_sN != nullptr ? d_sN[sbase + (long)row * DV] : 0.f;
    }

  // staging, one chunk ahead (reverse order): the factor pieces go straight from global
  // memory into the stage buffer (direct-to-LDS loads, no registers), this slice of dO
  // through registers (transposed on the way in)
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 std_[Sh::PPD];
  auto unit_of = [&](int ci) { return ws + ((slot0 + ci) * H + h) * LB.bytes; };
  auto stage_factors = [&](int ci, char* buf) {
    const char* unit = unit_of(ci);
#pragma unroll
    for (int j = 0; j < Sh::PPF; ++j) {
      int p = tid + j * NT;
      p = p < Sh::NPF ? p : Sh::NPF - 1;  // the tail re-reads the last piece
      const long off = p < Sh::SZ_F / 16 ? LB.kr + p * 16 : LB.f.g + (p * 16 - Sh::SZ_F);
      // lane l of the wave lands at buf + (64 wave + j NT + l) * 16
      __builtin_amdgcn_global_load_lds(unit + off,
                                       (__attribute__((address_space(3))) void*)(buf + (64 * wave + j * NT) * 16),
                                       16, 0, 0);
    }
  };
  auto load_do = [&](int ci) {
    const int nvalid = min(C, len - ci * C);
#pragma unroll
    for (int j = 0; j < Sh::PPD; ++j) {
      const int p = tid + j * NT, r = p / (NV / 8), cc = p % (NV / 8);
      // this slice's dO columns are read by this workgroup alone: non-temporal
      const T* src0 = d_o + (row0 + (long)ci * C) * vstride + (long)h * DV + col0;
      const u32x4 x = __builtin_bit_cast(
          u32x4, load16_nt(src0, (int)(((r < nvalid ? r : 0) * vstride + cc * 8) * 2)));
      std_[j] = x;  // rows past the end (row 0's values) are zeroed when stored
    }
  };
  auto store_do = [&](char* buf, int ci) {
    const int nvalid = min(C, len - ci * C);
    T* dot = reinterpret_cast<T*>(buf + Sh::OFF_DO);
#pragma unroll
    for (int j = 0; j < Sh::PPD; ++j) {  // transpose: [column][token]
      const int p = tid + j * NT, r = p / (NV / 8), cc = p % (NV / 8);
      const bf16x8 x = __builtin_bit_cast(bf16x8, r < nvalid ? std_[j] : u32x4{0u, 0u, 0u, 0u});
#pragma unroll
      for (int e = 0; e < 8; ++e) dot[(cc * 8 + e) * Sh::LDO + r] = x[e];
    }
  };
  // the direct loads of a stage are complete (s_waitcnt vmcnt(0)); before the barrier that
  // publishes the stage
  auto wait_stage = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };

  if (nch > 0) {
    stage_factors(nch - 1, smem);
    load_do(nch - 1);
    store_do(smem, nch - 1);
    wait_stage();
  }
  lds_barrier();

  for (int k = 0; k < nch; ++k) {
    const int ci = nch - 1 - k;
    tid = opaque(tid);
    lane = tid & 63;
    m16 = lane & 15;
    g4 = lane >> 4;
    const char* B = smem + (k & 1) * Sh::STAGE;
    auto frag = [&](int off, int blk) {
      return *reinterpret_cast<const typename M::frag*>(B + off + blk * 1024 + lane * 16);
    };
    char* unit = unit_of(ci);
    if (ci > 0) {  // the next chunk's operands, arriving while this one is computed
      stage_factors(ci - 1, smem + ((k + 1) & 1) * Sh::STAGE);
      load_do(ci - 1);
    }
    // dSn of this chunk, for the local kernel
    if constexpr (!XFER) {
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
        *reinterpret_cast<uint2*>(unit + LB.db + ((ctg * NMT + mt) * 64 + lane) * 8) =
            make_uint2(pack_bf16(D[mt][0], D[mt][1]), pack_bf16(D[mt][2], D[mt][3]));
    }
    typename M::frag db[KSK], dob[2];
#pragma unroll
    for (int s = 0; s < KSK; ++s) db[s] = M::from_acc(D, s);
#pragma unroll
    for (int s = 0; s < 2; ++s)  // dO^T of this wave's columns, tokens 32s + 8g4 .. + 8
      dob[s] = *reinterpret_cast<const bf16x8*>(B + Sh::OFF_DO +
                                                ((16 * wave + m16) * Sh::LDO + 32 * s + 8 * g4) * 2);
    // dU = P^T dO + Ktil dSn   (P^T is upper: token tiles 2, 3 only see the second K step)
    f4 dU[4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSK; ++s) acc = M::mma(frag(Sh::OFF_KR, R * KSK + s), db[s], acc);
#pragma unroll
      for (int s = R < 2 ? 0 : 1; s < 2; ++s) acc = M::mma(frag(Sh::OFF_PT, R * 2 + s), dob[s], acc);
      dU[R] = acc;
    }
    // dZ = T^T dU:  dZ_R = (T_RR)^T (dU_R + sum_{J > R} (-A_JR)^T dZ_J),  R = 3 .. 0
    f4 dZ[4];
    bf16x4 zb[4];
    auto btf = [&](int R, int J) {
      return *reinterpret_cast<const bf16x4*>(B + Sh::OFF_BT + ((R * 4 + J) * 64 + lane) * 8);
    };
#pragma unroll
    for (int R = 3; R >= 0; --R) {
      f4 acc = dU[R];
#pragma unroll
      for (int J = R + 1; J < 4; ++J) acc = mma16_frag(btf(R, J), zb[J], acc);
      dZ[R] = mma16_frag(btf(R, R), Frag16<T>::from_acc(acc), f4{0.f, 0.f, 0.f, 0.f});
      zb[R] = Frag16<T>::from_acc(dZ[R]);
    }
    if constexpr (!XFER) {
#pragma unroll
      for (int R = 0; R < 4; ++R)
        *reinterpret_cast<uint2*>(unit + LB.zb + ((ctg * 4 + R) * 64 + lane) * 8) =
            make_uint2(pack_bf16(dZ[R][0], dZ[R][1]), pack_bf16(dZ[R][2], dZ[R][3]));
    }
    // dS0 = Diag(gamma) dSn + Qbar^T dO + (-W^T) dU
    typename M::frag ub[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) ub[s] = M::from_acc(dU, s);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const f4 gam = *reinterpret_cast<const f4*>(B + Sh::OFF_G + (16 * mt + 4 * g4) * 4);
      f4 acc = D[mt] * gam;
#pragma unroll
      for (int s = 0; s < 2; ++s) acc = M::mma(frag(Sh::OFF_QT, mt * 2 + s), dob[s], acc);
#pragma unroll
      for (int s = 0; s < 2; ++s) acc = M::mma(frag(Sh::OFF_WT, mt * 2 + s), ub[s], acc);
      D[mt] = acc;
    }
    // the next chunk (ci - 1): its dO slice into the other buffer, whose factor pieces were
    // issued at the start of this chunk
    if (ci > 0) store_do(smem + ((k + 1) & 1) * Sh::STAGE, ci - 1);
    wait_stage();
    lds_barrier();
  }
  if constexpr (XFER) {  // b into the value columns of the segment's [b | M] (rows d_k, d_v + d_k columns)
    constexpr int LE = DV + DK;
    float* E = ebuf + (long)unit_id * DK * LE + col0 + 16 * wave + m16;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) E[(long)(16 * mt + 4 * g4 + i) * LE] = D[mt][i];
  } else if (d_s0 != nullptr && seg == 0) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) d_s0[sbase + (long)(16 * mt + 4 * g4 + i) * DV] = D[mt][i];
  }
}

// ------------------------------------------------------------------ the local gradients
// A value that the code below may use only from this point on: the empty asm reads and
// rewrites the registers, so the wait for a load into them, and the arithmetic on them,
// cannot be scheduled before it (the compiler otherwise pulls such work up to the first use
// of any register loaded with it, ahead of unrelated matrix work). `after` is a value the
// point depends on.
__device__ __forceinline__ void hold(uint4& x, float after) {
  asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w) : "v"(after));
}
__device__ __forceinline__ void hold(bf16x4& x, float after) {
  asm volatile("" : "+v"(x) : "v"(after));
}

// Sums along the 16-lane rows of a wave (lanes 16r .. 16r + 15) with DPP row operations, in
// registers: row_suffix gives lane i the sum over lanes i .. 15 of its row (lanes shifted in
// from past the row's end read 0), row_first the value of its row's lane 0.
template <int N>
__device__ __forceinline__ float row_shl(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x100 + N, 0xf, 0xf, true));
}
__device__ __forceinline__ float row_suffix(float x) {
  x += row_shl<1>(x);
  x += row_shl<2>(x);
  x += row_shl<4>(x);
  x += row_shl<8>(x);
  return x;
}
__device__ __forceinline__ float row_first(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150, 0xf, 0xf, false));
}
template <int DK, int DV>
struct LocalShape {
  static constexpr int C = 64;
  static constexpr int NW = DK / 16;      // wave w owns key channels [16w, 16w+16)
  static constexpr int NT = 64 * NW;
  static constexpr int CG = DK / 8;
  static constexpr int TG = NT / CG;      // 32
  static constexpr int TPT = C / TG;      // 2
  static constexpr int GPB = 16 / TPT;
  static constexpr int VCG = DV / 8;
  static constexpr int VTG = NT / VCG;
  static constexpr int VTPT = C / VTG;
  // [x][64] arrays: rows of 40 words (an odd multiple of 8: conflict-free fragment reads on
  // the 128-bank LDS); [x][d] arrays 16 bytes longer (the LDS budget allows no more)
  static constexpr int LDV = DV + 8, LDK = DK + 8, LDT = C + 16;
  static constexpr int NVT = DV / 16, NCT = DK / 16;
  // LDS regions (bytes)
  static constexpr int SZ_A = DK * LDV * 2;     // dSn, later S0: [DK][DV]
  static constexpr int SZ_R = C * LDV * 2;      // dO, dZ, U: [64][DV]
  static constexpr int SZ_ET = 2 * DK * LDT * 2;  // Ebar^T, Qbar^T
  static constexpr int LDG = DK + 16;  // G rows: 16 words of padding (conflict-free row reads)
  static constexpr int SZ_EL = C * LDG * 4 + 3 * C * LDK * 2;  // G (fp32), q, k, b
  static constexpr int SZ_BIG0 = SZ_A + 3 * SZ_R;
  static constexpr int SZ_BIG = SZ_BIG0 > SZ_EL ? (SZ_BIG0 > SZ_ET ? SZ_BIG0 : SZ_ET)
                                                : (SZ_EL > SZ_ET ? SZ_EL : SZ_ET);
  static constexpr int OFF_A = 0, OFF_O = SZ_A, OFF_Z = OFF_O + SZ_R, OFF_U = OFF_Z + SZ_R;
  static constexpr int OFF_KH = (SZ_BIG + 15) / 16 * 16;  // Khat^T [DK][64], swizzled
  static constexpr int SZ_M = C * LDT * 2;
  static constexpr int OFF_M1 = OFF_KH + DK * LDT * 2;    // M1, M2 row-major; then transposed
  static constexpr int OFF_M2 = OFF_M1 + SZ_M;
  static constexpr int OFF_M1T = OFF_M2 + SZ_M;
  static constexpr int OFF_M2T = OFF_M1T + SZ_M;
  static constexpr int OFF_FAC = OFF_M2T + SZ_M;
  static constexpr int OFF_X = OFF_FAC + Fac::N * DK * 4;  // per-channel constant of dg
  static constexpr int OFF_FLAG = OFF_X + DK * 4;
  static constexpr int LDS_BYTES = OFF_FLAG + 16;
  static constexpr int OFF_TOT = OFF_KH;                   // cumsum scratch in the Khat^T region
  // staging of the elementwise step's row-major outputs (dq, dk, db) in the Khat^T and M
  // regions, dead by then; dg's in the region of the elementwise inputs. Rows padded by 8
  // elements (conflict-free 8-byte writes of 16 rows x 32 bytes)
  static constexpr int LDSG = DK + 8;
  static constexpr int OFF_SG = OFF_KH;
  static_assert(OFF_SG + 3 * C * LDSG * 2 <= OFF_FAC, "staging of dq, dk, db");
  static_assert(C * LDSG * 2 <= SZ_BIG, "staging of dg");
  static_assert(2 * C * LDSG * 2 + (DK / 16) * 64 * 4 <= OFF_FAC - OFF_SG, "scalar-db partials");
  static_assert(TG * DK * 4 <= DK * LDT * 2, "cumsum scratch");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(TPT * TG == C && VTPT * VTG == C, "token mapping");
};

// GL: gate layout (kGateBScalar / kGateWScalar bits); a scalar gate's gradient is the sum
// of its per-channel gradients over the channels it is shared by.
template <int DK, int DV, int GL>
__global__ void __launch_bounds__((LocalShape<DK, DV>::NT))
gdn2_bwd_local_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                      const bf16* __restrict__ v, const bf16* __restrict__ g,
                      const bf16* __restrict__ bg, const bf16* __restrict__ wg,
                      const bf16* __restrict__ d_o, const char* __restrict__ ws,
                      bf16* __restrict__ dq, bf16* __restrict__ dk, bf16* __restrict__ dv,
                      bf16* __restrict__ dg, bf16* __restrict__ db, bf16* __restrict__ dw,
                      int* range_flag, const int* __restrict__ cu_seqlens, int N, int T_len,
                      int H, long nunits) {
  typedef bf16 T;
  using Sh = LocalShape<DK, DV>;
  using M = Mma<T>;
  constexpr bool B_S = (GL & kGateBScalar) != 0, W_S = (GL & kGateWScalar) != 0;
  constexpr bool early_dsn = !(B_S && W_S);  // see the elementwise step
  constexpr BwdLayout LB(DK, DV);
  constexpr int C = Sh::C, NT = Sh::NT, LDV = Sh::LDV, LDK = Sh::LDK, LDT = Sh::LDT;
  constexpr int NVT = Sh::NVT;
  __shared__ __attribute__((aligned(16))) char smem[Sh::LDS_BYTES];
  T* sA = reinterpret_cast<T*>(smem + Sh::OFF_A);
  T* sO = reinterpret_cast<T*>(smem + Sh::OFF_O);
  T* sZ = reinterpret_cast<T*>(smem + Sh::OFF_Z);
  T* sU = reinterpret_cast<T*>(smem + Sh::OFF_U);
  T* sKh = reinterpret_cast<T*>(smem + Sh::OFF_KH);
  T* sM1 = reinterpret_cast<T*>(smem + Sh::OFF_M1);
  T* sM2 = reinterpret_cast<T*>(smem + Sh::OFF_M2);
  T* sM1t = reinterpret_cast<T*>(smem + Sh::OFF_M1T);
  T* sM2t = reinterpret_cast<T*>(smem + Sh::OFF_M2T);
  float* sFac = reinterpret_cast<float*>(smem + Sh::OFF_FAC);
  float* sX = reinterpret_cast<float*>(smem + Sh::OFF_X);
  float* sTot = reinterpret_cast<float*>(smem + Sh::OFF_TOT);
  int* sFlag = reinterpret_cast<int*>(smem + Sh::OFF_FLAG);

  const int lane = threadIdx.x & 63;  // (the unit loop derives its own per-lane indices)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const long kstride = (long)H * DK, vstride = (long)H * DV;
  // The workgroups are persistent (one per compute unit) and walk the units u = blockIdx.x,
  // + gridDim.x, ... Every global read of a unit is issued before it is needed: the workspace
  // tiles dZ, U, dSn (for the matrix work P1, P2) during the previous unit (dSn before its
  // elementwise step, dZ and U after it, ahead of its gradient row stores); dO and S0 at the
  // start of the unit; g, k once dO is in LDS; v, w after P1; q, b
  // after P2. Every compute unit starts its units at about the same time, so what is issued
  // at a unit's start competes for HBM with dO, which P1 waits for: issuing the rest at
  // these later points (each a step ahead of its first use) took the backward from 736 to
  // 700 us on the 1.3B-layer workload, against issuing every late load at the unit's start.
  // Every load is unconditional (a row past the unit's end reads row 0 and is zeroed where
  // it is first used; past the last unit the current one is read again), which keeps the
  // waits on the early groups exact.
  constexpr int NDO = C * DV / 8 / NT;             // 16-byte pieces of dO per thread
  constexpr int NZU = Sh::NVT * 4 / Sh::NW;        // dZ and U tiles per wave
  static_assert(NDO * NT == C * DV / 8 && NZU * Sh::NW == Sh::NVT * 4, "load mapping");
  // accumulator tiles (bf16, lane-major, 8 bytes per lane)
  auto tile_raw = [&](const char* un, long off, int tile) {
    return *reinterpret_cast<const bf16x4*>(un + off + (tile * 64 + lane) * 8);
  };
  auto tof = [](bf16x4 x) { return f4{to_f(x[0]), to_f(x[1]), to_f(x[2]), to_f(x[3])}; };
  bf16x4 rz[NZU], ru[NZU], rds[NVT];
  auto issue_first_a = [&](long uu) {  // dSn
    const char* un = ws + uu * LB.bytes;
#pragma unroll
    for (int ct = 0; ct < NVT; ++ct) rds[ct] = tile_raw(un, LB.db, ct * Sh::NCT + wave);
  };
  auto issue_first_b = [&](long uu) {  // dZ and U
    const char* un = ws + uu * LB.bytes;
#pragma unroll
    for (int i = 0; i < NZU; ++i) {
      rz[i] = tile_raw(un, LB.zb, wave + i * Sh::NW);
      ru[i] = tile_raw(un, LB.ub, wave + i * Sh::NW);
    }
  };
  auto issue_first = [&](long uu) {
    issue_first_b(uu);
    issue_first_a(uu);
  };
  long u = blockIdx.x;
  ChunkUnit cu = map_unit(u, H, cu_seqlens, N, T_len, lane);
  issue_first(u);
  while (u < nunits) {
    const long u_next = u + gridDim.x;
    const long u_pre = u_next < nunits ? u_next : u;  // the unit whose first group is prefetched
    if (cu.nvalid == 0) {  // an unused slot (uniform)
      cu = map_unit(u_pre, H, cu_seqlens, N, T_len, lane);
      issue_first(u_pre);
      u = u_next;
      continue;
    }
    const char* unit = ws + u * LB.bytes;
    const long kb0 = cu.row * kstride + (long)cu.h * DK;
    const long vb0 = cu.row * vstride + (long)cu.h * DV;
    // the per-lane indices, derived again for every unit from an opaque copy of the thread
    // index, so that the offsets computed from them are not hoisted out of the unit loop
    // (where they would hold registers through the whole kernel)
    int tid_u = threadIdx.x;
    asm volatile("" : "+v"(tid_u));
    const int tid = tid_u, lane = tid & 63, m16 = lane & 15, g4 = lane >> 4;
    const int cg = tid % Sh::CG, tg = tid / Sh::CG, vcg = tid % Sh::VCG, vtg = tid / Sh::VCG;
    auto clamp_row = [&](int r) { return r < cu.nvalid ? r : 0; };
    uint4 rdo[NDO];
  #pragma unroll
    for (int i = 0; i < NDO; ++i) {
      const int p = tid + i * NT, r = clamp_row(p / (DV / 8)), cc = p % (DV / 8);
      rdo[i] = *reinterpret_cast<const uint4*>(d_o + vb0 + (long)r * vstride + cc * 8);
    }
    bf16x4 s0t[NVT];
    Vec8<T> rq[Sh::TPT], rk[Sh::TPT], rg[Sh::TPT], rb[Sh::TPT], rv[Sh::VTPT], rw[Sh::VTPT];
    bool kvalid[Sh::TPT];
  #pragma unroll
    for (int ct = 0; ct < NVT; ++ct) s0t[ct] = tile_raw(unit, LB.h, ct * Sh::NCT + wave);

    // ---- dO, dZ and U (tiles (ct, R)) row-major, dSn into LDS. A dO row past the end holds
    // row 0's values: it reaches only M1's row of that token (zeroed in P1) and dQbar's column
    // of that token (not stored).
  #pragma unroll
    for (int i = 0; i < NDO; ++i) {
      const int p = tid + i * NT, r = p / (DV / 8), cc = p % (DV / 8);
      *reinterpret_cast<uint4*>(sO + r * LDV + cc * 8) = rdo[i];
    }
    auto ident = [](int c) { return c; };
  #pragma unroll
    for (int i = 0; i < NZU; ++i) {
      const int t = wave + i * Sh::NW, ct = t / 4, R = t % 4;
      store_tile_pairs(sZ + (16 * R) * LDV + 16 * ct, LDV, lane, tof(rz[i]), ident);
      store_tile_pairs(sU + (16 * R) * LDV + 16 * ct, LDV, lane, tof(ru[i]), ident);
    }
  #pragma unroll
    for (int ct = 0; ct < NVT; ++ct)
      store_tile_pairs(sA + (16 * wave) * LDV + 16 * ct, LDV, lane, tof(rds[ct]), ident);
  #pragma unroll
    for (int j = 0; j < Sh::TPT; ++j) {
      kvalid[j] = tg * Sh::TPT + j < cu.nvalid;
      const long off = kb0 + (long)clamp_row(tg * Sh::TPT + j) * kstride + cg * 8;
      rg[j].load(g + off);
      rk[j].load(k + off);
    }
    if (tid == 0) *sFlag = 0;
    lds_barrier();

    // ---- P1: M1 = lower_incl(dO U^T), M2 = -strict(dZ U^T); stored row-major and transposed
    for (int t = wave; t < 32; t += Sh::NW) {
      const int which = t >> 4, R = (t >> 2) & 3, I = t & 3;
      const T* lhs = which ? sZ : sO;
      f4 acc = {0.f, 0.f, 0.f, 0.f};
      if (I <= R) {
  #pragma unroll
        for (int s = 0; s < DV / 32; ++s)
          acc = M::mma(M::load(lhs, LDV, 16 * R + m16, 32 * s + 8 * g4),
                       M::load(sU, LDV, 16 * I + m16, 32 * s + 8 * g4), acc);
      }
      f4 val;
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g4 + i, c = m16;  // row (token t) within R, column (token i) within I
        const bool keep = (I < R || (which ? c < r : c <= r)) && (which || 16 * R + r < cu.nvalid);
        val[i] = keep ? (which ? -acc[i] : acc[i]) : 0.f;
      }
      T* Mr = which ? sM2 : sM1;
      T* Mt = which ? sM2t : sM1t;
      store_tile_pairs(Mr + (16 * R) * LDT + 16 * I, LDT, lane, val, ident);
      *reinterpret_cast<uint2*>(Mt + (16 * I + m16) * LDT + 16 * R + 4 * g4) =
          make_uint2(pack_bf16(val[0], val[1]), pack_bf16(val[2], val[3]));
    }
  #pragma unroll
    for (int j = 0; j < Sh::VTPT; ++j) {  // rows past the end give outputs that are not stored
      const int r = clamp_row(vtg * Sh::VTPT + j);
      rv[j].load(v + vb0 + (long)r * vstride + vcg * 8);
      if constexpr (W_S) rw[j].load_one(wg + (cu.row + r) * H + cu.h);
      else rw[j].load(wg + vb0 + (long)r * vstride + vcg * 8);
    }
    // ---- P2: dKtil^T = dSn U^T   (rows: this wave's channels; columns: tokens)
    f4 dKt[4];
  #pragma unroll
    for (int Tt = 0; Tt < 4; ++Tt) {
      f4 acc = {0.f, 0.f, 0.f, 0.f};
  #pragma unroll
      for (int s = 0; s < DV / 32; ++s)
        acc = M::mma(M::load(sA, LDV, 16 * wave + m16, 32 * s + 8 * g4),
                     M::load(sU, LDV, 16 * Tt + m16, 32 * s + 8 * g4), acc);
      dKt[Tt] = acc;
    }
  #pragma unroll
    for (int j = 0; j < Sh::TPT; ++j) {
      const int r = clamp_row(tg * Sh::TPT + j);
      rq[j].load(q + kb0 + (long)r * kstride + cg * 8);
      if constexpr (B_S) rb[j].load_one(bg + (cu.row + r) * H + cu.h);
      else rb[j].load(bg + kb0 + (long)r * kstride + cg * 8);
    }
    // ---- (a): per-thread totals of log2-decay (a row past the end decays by nothing) into
    // sTot, which shares the Khat^T region (written only after the scan's prefixes are read)
  #pragma unroll
    for (int j = 0; j < Sh::TPT; ++j) {
      hold(rg[j].r, dKt[3][3]);
      hold(rk[j].r, dKt[3][3]);
      if (!kvalid[j]) { rg[j].zero(); rk[j].zero(); }
    }
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
    lds_barrier();  // M1, M2 written; the totals complete; dSn and U are dead
    // ---- (b): the per-channel scan and the chunk factors
    channel_scan<DK, Sh::TG, Sh::GPB, NT>(sTot, sFac, sFlag, tid);
    lds_barrier();
    (void)sFlag;
    if (tid < DK && range_flag != nullptr && -sFac[Fac::GL * DK + tid] > 2.f * kFastPathMaxDecay2)
      *range_flag = 1;
    // this thread's channels' reference Gm = Glast / 2 (log2)
    float Gm8[8];
  #pragma unroll
    for (int i = 0; i < 8; ++i) Gm8[i] = 0.5f * sFac[Fac::GL * DK + cg * 8 + i];
    // per thread: G (log2) of its tokens; Khat'^T = (K 2^(Gm-G))^T (stored below)
    float G2[Sh::TPT][8];
    RunBuf<T, Sh::TPT> kh[8];
    {
      float run[8];
  #pragma unroll
      for (int i = 0; i < 8; ++i) run[i] = sTot[tg * DK + cg * 8 + i];
  #pragma unroll
      for (int j = 0; j < Sh::TPT; ++j) {
        float fg[8], fk[8];
        rg[j].to_float(fg);
        rk[j].to_float(fk);
  #pragma unroll
        for (int i = 0; i < 8; ++i) {
          run[i] += fg[i] * kLog2e;
          G2[j][i] = run[i];
          kh[i].put(j, fk[i] * fast_exp2(Gm8[i] - run[i]));
        }
      }
    }
    {
      // S0 rows (this lane's channels 16 wave + 4 g4 + i) scaled by 2^Gm into sA (dSn is
      // dead); the dg constant X_c = sum_v dSn[c,v] S0[c,v] (times gamma_c later)
      const f4 gl = *reinterpret_cast<const f4*>(sFac + Fac::GL * DK + 16 * wave + 4 * g4);
  #pragma unroll
      for (int ct = 0; ct < NVT; ++ct) hold(s0t[ct], gl[0]);
      f4 rs, xs = {0.f, 0.f, 0.f, 0.f};
  #pragma unroll
      for (int i = 0; i < 4; ++i) rs[i] = fast_exp2(0.5f * gl[i]);
  #pragma unroll
      for (int ct = 0; ct < NVT; ++ct) {
        const f4 s0 = tof(s0t[ct]);
        store_tile_pairs(sA + (16 * wave) * LDV + 16 * ct, LDV, lane, s0 * rs, ident);
        xs += tof(rds[ct]) * s0;
      }
  #pragma unroll
      for (int i = 0; i < 4; ++i) xs[i] = row_suffix(xs[i]);  // lane 0 of the row: the row's sum
      if (m16 == 0) *reinterpret_cast<f4*>(sX + 16 * wave + 4 * g4) = xs;
    }
    // dv = dZ * w, dw = dZ * v
  #pragma unroll
    for (int j = 0; j < Sh::VTPT; ++j) {
      const int r = vtg * Sh::VTPT + j;
      float fz[8], fv[8], fw[8], o1[8], o2[8];
      Vec8<T> z;
      z.load(sZ + r * LDV + vcg * 8);
      z.to_float(fz);
      hold(rv[j].r, fz[0]);
      hold(rw[j].r, fz[0]);
      rv[j].to_float(fv);
      if constexpr (W_S) rw[j].splat();
      rw[j].to_float(fw);
  #pragma unroll
      for (int i = 0; i < 8; ++i) { o1[i] = fz[i] * fw[i]; o2[i] = fz[i] * fv[i]; }
      if (r < cu.nvalid) {
        // whole rows (VCG lanes of 16 bytes), written once: non-temporal
        const long off = vb0 + (long)r * vstride + vcg * 8;
        bf16x8 pv, pw;
  #pragma unroll
        for (int i = 0; i < 8; ++i) {
          pv[i] = static_cast<bf16>(o1[i]);
          pw[i] = static_cast<bf16>(o2[i]);
        }
        __builtin_nontemporal_store(pv, reinterpret_cast<bf16x8*>(dv + off));
        if constexpr (!W_S) __builtin_nontemporal_store(pw, reinterpret_cast<bf16x8*>(dw + off));
      }
      if constexpr (W_S) {  // sum over the token's d_v channels (VCG adjacent lanes)
        float sw = 0.f;
  #pragma unroll
        for (int i = 0; i < 8; ++i) sw += o2[i];
  #pragma unroll
        for (int m = 1; m < Sh::VCG; m <<= 1) sw += __shfl_xor(sw, m, 64);
        if (vcg == 0 && r < cu.nvalid) dw[(cu.row + r) * H + cu.h] = from_f<T>(sw);
      }
    }
    lds_barrier();  // the prefixes in sTot are read
    {
      const int sw = tswz(cg * 8);
  #pragma unroll
      for (int i = 0; i < 8; ++i) kh[i].store_sw(sKh + (cg * 8 + i) * LDT, sw, tg * Sh::TPT);
    }
    lds_barrier();
    // ---- P3: dQbar^T = S0 dO^T + Khat^T M1^T,  dEbar^T = -S0 dZ^T + Khat^T M2^T
    f4 dQb[4], dEb[4];
  #pragma unroll
    for (int Tt = 0; Tt < 4; ++Tt) {
      f4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
  #pragma unroll
      for (int s = 0; s < DV / 32; ++s) {
        const typename M::frag sf = M::load(sA, LDV, 16 * wave + m16, 32 * s + 8 * g4);
        a1 = M::mma(sf, M::load(sO, LDV, 16 * Tt + m16, 32 * s + 8 * g4), a1);
        a2 = M::mma(sf, M::load(sZ, LDV, 16 * Tt + m16, 32 * s + 8 * g4), a2);
      }
      a2 = -a2;
  #pragma unroll
      for (int s = 0; s < 2; ++s) {
        const typename M::frag kf = M::load_phi_t(sKh, LDT, 16 * wave + m16, s, g4);
        a1 = M::mma(kf, M::load(sM1, LDT, 16 * Tt + m16, 32 * s + 8 * g4), a1);
        a2 = M::mma(kf, M::load(sM2, LDT, 16 * Tt + m16, 32 * s + 8 * g4), a2);
      }
      dQb[Tt] = a1;
      dEb[Tt] = a2;
    }
    lds_barrier();  // S0, dO, dZ are dead
    // Ebar^T = (b k 2^G)^T and Qbar^T = (q 2^G)^T, natural token order, into the big region
    T* sEt = reinterpret_cast<T*>(smem);
    T* sQt = sEt + DK * LDT;
    {
      RunBuf<T, Sh::TPT> ev[8], qv[8];
  #pragma unroll
      for (int j = 0; j < Sh::TPT; ++j) {
        float fq[8], fk[8], fb[8];
        hold(rq[j].r, dQb[3][3]);
        hold(rb[j].r, dQb[3][3]);
        if (!kvalid[j]) { rq[j].zero(); rb[j].zero(); }
        rq[j].to_float(fq);
        rk[j].to_float(fk);
        if constexpr (B_S) rb[j].splat();  // (also what the elementwise step reads back)
        rb[j].to_float(fb);
  #pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float gm = fast_exp2(G2[j][i] - Gm8[i]);
          ev[i].put(j, fb[i] * fk[i] * gm);
          qv[i].put(j, fq[i] * gm);
        }
      }
      const int sw = tswz(cg * 8);
  #pragma unroll
      for (int i = 0; i < 8; ++i) {
        ev[i].store_sw(sEt + (cg * 8 + i) * LDT, sw, tg * Sh::TPT);
        qv[i].store_sw(sQt + (cg * 8 + i) * LDT, sw, tg * Sh::TPT);
      }
    }
    lds_barrier();
    // ---- P4: dKhat^T = Ebar^T M2 + Qbar^T M1
    f4 dKh[4];
  #pragma unroll
    for (int Tt = 0; Tt < 4; ++Tt) {
      f4 acc = {0.f, 0.f, 0.f, 0.f};
  #pragma unroll
      for (int s = 0; s < 2; ++s) {
        acc = M::mma(M::load_phi_t(sEt, LDT, 16 * wave + m16, s, g4),
                     M::load(sM2t, LDT, 16 * Tt + m16, 32 * s + 8 * g4), acc);
        acc = M::mma(M::load_phi_t(sQt, LDT, 16 * wave + m16, s, g4),
                     M::load(sM1t, LDT, 16 * Tt + m16, 32 * s + 8 * g4), acc);
      }
      dKh[Tt] = acc;
    }
    lds_barrier();  // everything but the factors is dead
    // G (log2, fp32) and q, k, b row-major for the elementwise step
    float* sG = reinterpret_cast<float*>(smem);
    T* sq = reinterpret_cast<T*>(smem + C * Sh::LDG * 4);
    T* sk = sq + C * LDK;
    T* sb = sk + C * LDK;
  #pragma unroll
    for (int j = 0; j < Sh::TPT; ++j) {
      const int r = tg * Sh::TPT + j;
      store8(sG + r * Sh::LDG + cg * 8, G2[j]);
      *reinterpret_cast<uint4*>(sq + r * LDK + cg * 8) = rq[j].r;
      *reinterpret_cast<uint4*>(sk + r * LDK + cg * 8) = rk[j].r;
      *reinterpret_cast<uint4*>(sb + r * LDK + cg * 8) = rb[j].r;
    }
    lds_barrier();

    // the next unit's dSn tiles (this unit's are consumed); with both gates scalar the
    // registers are short here, and they are issued with dZ and U after the elementwise step
    if constexpr (early_dsn) issue_first_a(u_pre);
    // ---- elementwise: lane = token 16*Tt + m16, channels c0 .. c0 + 3 of this wave
    const int c0 = 16 * wave + 4 * g4;
    const f4 gam = *reinterpret_cast<const f4*>(sFac + Fac::GAM * DK + c0);
    const f4 gl = *reinterpret_cast<const f4*>(sFac + Fac::GL * DK + c0);
    const f4 xc = *reinterpret_cast<const f4*>(sX + c0);
    // dq, dk and db of a token tile go to row-major staging tiles in LDS as soon as they are
    // formed (the Khat and M regions are dead here), dg once the suffix sums over the chunk are
    // done (into the region of the elementwise inputs, after they are read); the rows are then
    // stored whole, 16 bytes per lane. A wave's own results are 32 bytes of each row: stored
    // directly, each store instruction addressed 16 separate 32-byte row pieces.
    constexpr int LDS_ = Sh::LDSG;
    T* sSq = reinterpret_cast<T*>(smem + Sh::OFF_SG);
    T* sSk = sSq + C * LDS_;
    T* sSb = sSk + C * LDS_;
    T* sSg = reinterpret_cast<T*>(smem);
    auto put4 = [&](T* p, int t, f4 x) {
      *reinterpret_cast<uint2*>(p + t * LDS_ + c0) =
          make_uint2(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]));
    };
    float* sPart = reinterpret_cast<float*>(sSb);  // scalar db: [NW][64] partials
    f4 dgv[4];
    f4 totB = {0.f, 0.f, 0.f, 0.f};
  #pragma unroll
    for (int Tt = 0; Tt < 4; ++Tt) {
      const int t = 16 * Tt + m16;
      const f4 G = *reinterpret_cast<const f4*>(sG + t * Sh::LDG + c0);
      const f4 fq = load4f(sq + t * LDK + c0), fk = load4f(sk + t * LDK + c0);
      const f4 fb = load4f(sb + t * LDK + c0);
      f4 A, Bv, outq, outk, outb;
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        // mid-referenced factors (dQb, dEb, dKh carry the 2^(+-Gm) of their operands)
        const float gmr = 0.5f * gl[i];
        const float gm = fast_exp2(G[i] - gmr), ig = fast_exp2(gmr - G[i]);
        const float kt = fast_exp2(gl[i] - G[i]);  // 2^(Glast - G) <= 1
        const float dE = dEb[Tt][i] * gm;
        outq[i] = dQb[Tt][i] * gm;
        outk[i] = dKh[Tt][i] * ig + dKt[Tt][i] * kt + dE * fb[i];
        outb[i] = dE * fk[i];
        // dG = dEbar Ebar + dQbar Qbar - dKhat Khat - dKtil Ktil, split as A - B
        A[i] = gm * (dEb[Tt][i] * fb[i] * fk[i] + dQb[Tt][i] * fq[i]) - dKh[Tt][i] * fk[i] * ig;
        Bv[i] = dKt[Tt][i] * fk[i] * kt;
      }
      dgv[Tt] = A - Bv;
      totB += Bv;
      put4(sSq, t, outq);
      put4(sSk, t, outk);
      if constexpr (!B_S) {
        put4(sSb, t, outb);
      } else {
        // a scalar b's gradient sums the token's d_k channels: 4 per lane, the 4 lane groups
        // of a wave, then the NW waves through LDS
        float x = outb[0] + outb[1] + outb[2] + outb[3];
        x += __shfl_xor(x, 16, 64);
        x += __shfl_xor(x, 32, 64);
        if (g4 == 0) sPart[wave * 64 + t] = x;
      }
    }
    // the next unit's first load group, in flight from here on
    const ChunkUnit cn = map_unit(u_pre, H, cu_seqlens, N, T_len, lane);
    if constexpr (early_dsn) issue_first_b(u_pre);
    else issue_first(u_pre);
    // dg_t = sum_{t' >= t} (A - B)_{t'} + sum_all B + gamma X   (suffix sums over 64 tokens)
  #pragma unroll
    for (int i = 0; i < 4; ++i) totB[i] = row_first(row_suffix(totB[i]));
    f4 carry = totB + gam * xc;
    lds_barrier();  // every wave is done with G, q, k and b: their region takes dg
  #pragma unroll
    for (int Tt = 3; Tt >= 0; --Tt) {
      f4 x = dgv[Tt];
      f4 tile_tot;
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = row_suffix(x[i]);
        tile_tot[i] = row_first(x[i]);
      }
      put4(sSg, 16 * Tt + m16, x + carry);
      carry += tile_tot;
    }
    lds_barrier();  // the staged rows are complete
    // whole rows, 16-byte pieces (DK / 8 per row), rows past the unit's end not stored
    auto store_rows = [&](T* dst, const T* src) {
  #pragma unroll
      for (int j = 0; j < C * DK / 8 / NT; ++j) {
        const int pc = tid + j * NT, r = pc / (DK / 8), c8 = pc % (DK / 8);
        if (r < cu.nvalid)
          *reinterpret_cast<uint4*>(dst + kb0 + (long)r * kstride + c8 * 8) =
              *reinterpret_cast<const uint4*>(src + r * LDS_ + c8 * 8);
      }
    };
    store_rows(dq, sSq);
    store_rows(dk, sSk);
    if constexpr (!B_S) store_rows(db, sSb);
    store_rows(dg, sSg);
    if constexpr (B_S) {
      if (tid < C) {
        float x = 0.f;
  #pragma unroll
        for (int w = 0; w < Sh::NW; ++w) x += sPart[w * 64 + tid];
        if (tid < cu.nvalid) db[(cu.row + tid) * H + cu.h] = from_f<T>(x);
      }
    }
    cu = cn;
    u = u_next;
    lds_barrier();  // this unit's readers of LDS are done before the next unit's stores
  }
}

// ------------------------------------------------------------------ exact local gradients
// The local kernel references its decay factors to the middle of each chunk's decay, which
// keeps them finite for chunks of up to 2 x kFastPathMaxDecay2 log2 units per channel. This
// kernel recomputes dq, dk, db and dg of the (chunk, head) units past a slightly lower
// bound (every unit the local kernel may have left invalid; dv and dw carry no decay and
// stay as it wrote them), with the pairwise factors 2^(G_r - G_i) <= 1 (r >= i) evaluated
// directly, so any decay in (0, 1] is exact: the same chunk-form formulas as the local
// kernel, term by term, in fp32 and without matrix cores (a rare path).
//   M1 = lower_incl(dO U^T), M2 = -strict(dZ U^T), dOS = dO S0^T, dZS = dZ S0^T,
//   dKt = U dSn^T, X = rowsum(dSn * S0);
//   dq_t = 2^G_t dOS_t + sum_{i<=t} M1[t,i] k_i 2^(G_t-G_i)
//   de_t = -2^G_t dZS_t + sum_{i<t} M2[t,i] k_i 2^(G_t-G_i)
//   dkh_t = sum_{r>=t} (M2[r,t] e_r + M1[r,t] q_r) 2^(G_r-G_t)
//   dk_t = dkh_t + dKt_t 2^(Gl-G_t) + de_t b_t,  db_t = de_t k_t
//   dg_t = sum_{t'>=t} (A - B)_{t'} + sum_t B_t + 2^Gl X,
//   A_t = de_t b_t k_t + dq_t q_t - dkh_t k_t,  B_t = dKt_t k_t 2^(Gl-G_t).
// One 256-thread workgroup per unit (persistent over units); thread = (key channel c, half
// of the chunk's tokens). Launched after the local kernel; with a range flag that the local
// kernel left at 0 (no unit out of its range) every workgroup returns at once.
template <int DK, int DV, int GL>
__global__ void __launch_bounds__(256)
gdn2_bwd_exact_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                      const bf16* __restrict__ g, const bf16* __restrict__ bg,
                      const bf16* __restrict__ d_o, const char* __restrict__ ws,
                      bf16* __restrict__ dq, bf16* __restrict__ dk, bf16* __restrict__ dg,
                      bf16* __restrict__ db, const int* range_flag,
                      const int* __restrict__ cu_seqlens, int N, int T_len, int H, long nunits) {
  static_assert(DK * 2 == 256 || DK * 4 == 256, "thread mapping");
  constexpr int C = 64, NT = 256;
  constexpr int NH = NT / DK;         // token groups per channel (2 for d_k = 128, 4 for 64)
  constexpr int TPH = C / NH;         // tokens per thread
  constexpr int LDV = DV + 8;         // bf16 rows of the value-side arrays
  constexpr int LDM = C + 1;          // fp32 rows of M1, M2
  constexpr bool B_S = (GL & kGateBScalar) != 0;
  constexpr BwdLayout LB(DK, DV);
  // stage 1: S0, dSn [DK][LDV], U, dO, dZ [C][LDV] (bf16); stage 2 reuses the space for
  // G [C][DK] (fp32) and q, k, b [C][DK] (bf16)
  constexpr int SZ1 = (2 * DK + 3 * C) * LDV * 2;
  constexpr int SZ2 = C * DK * 4 + 3 * C * DK * 2;
  constexpr int SZ12 = SZ1 > SZ2 ? SZ1 : SZ2;
  __shared__ __attribute__((aligned(16))) char smem[SZ12 + 2 * C * LDM * 4 + (NH + 2) * DK * 4 + C * 4];
  bf16* sS0 = reinterpret_cast<bf16*>(smem);
  bf16* sdS = sS0 + DK * LDV;
  bf16* sU = sdS + DK * LDV;
  bf16* sO = sU + C * LDV;
  bf16* sZ = sO + C * LDV;
  float* sG = reinterpret_cast<float*>(smem);
  bf16* sq = reinterpret_cast<bf16*>(smem + C * DK * 4);
  bf16* sk = sq + C * DK;
  bf16* sb = sk + C * DK;
  float* sM1 = reinterpret_cast<float*>(smem + SZ12);
  float* sM2 = sM1 + C * LDM;
  float* sPart = sM2 + C * LDM;       // [NH][DK] per-group totals (decay, then dg suffix)
  float* sTB = sPart + NH * DK;       // [DK] sum of B over the chunk
  float* sMx = sTB + DK;              // [DK] largest decay total (range test)
  float* sDb = sMx + DK;              // [C] scalar b: channel sums

  if (range_flag != nullptr && __builtin_amdgcn_readfirstlane(*range_flag) == 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int c = tid % DK, hg = tid / DK, t0 = hg * TPH;
  const long kstride = (long)H * DK, vstride = (long)H * (long)DV;

  for (long u = blockIdx.x; u < nunits; u += gridDim.x) {
    const ChunkUnit cu = map_unit(u, H, cu_seqlens, N, T_len, lane);
    if (cu.nvalid == 0) continue;  // (uniform)
    const long kb0 = cu.row * kstride + (long)cu.h * DK;
    const long vb0 = cu.row * vstride + (long)cu.h * DV;
    // ---- range test: this channel's decay over the chunk (log2), against a bound a little
    // below the local kernel's, so that every unit it may have left invalid is redone
    float tot = 0.f;
    for (int t = t0; t < t0 + TPH; ++t)
      if (t < cu.nvalid) tot += static_cast<float>(g[kb0 + (long)t * kstride + c]) * kLog2e;
    sPart[hg * DK + c] = tot;
    __syncthreads();
    if (tid < DK) {
      float x = 0.f;
      for (int h2 = 0; h2 < NH; ++h2) x += sPart[h2 * DK + tid];
      sMx[tid] = -x;
    }
    __syncthreads();
    float mx = 0.f;
    for (int i = 0; i < DK; ++i) mx = fmaxf(mx, sMx[i]);
    if (!(mx > 2.f * kFastPathMaxDecay2 - 10.f)) {  // (uniform; a NaN total is redone too)
      __syncthreads();
      continue;
    }
    // ---- stage 1: dense products
    const char* un = ws + u * LB.bytes;
    for (int x = tid; x < (DV / 16) * (DK / 16) * 64; x += NT) {  // S0, dSn tiles (ct, channel tile)
      const int tile = x / 64, ln = x % 64, ct = tile / (DK / 16), w = tile % (DK / 16);
      const bf16x4 a = *reinterpret_cast<const bf16x4*>(un + LB.h + (tile * 64 + ln) * 8);
      const bf16x4 d = *reinterpret_cast<const bf16x4*>(un + LB.db + (tile * 64 + ln) * 8);
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * w + 4 * (ln >> 4) + i, col = 16 * ct + (ln & 15);
        sS0[row * LDV + col] = a[i];
        sdS[row * LDV + col] = d[i];
      }
    }
    for (int x = tid; x < (DV / 16) * 4 * 64; x += NT) {  // U, dZ tiles (ct, token block)
      const int tile = x / 64, ln = x % 64, ct = tile / 4, R = tile % 4;
      const bf16x4 a = *reinterpret_cast<const bf16x4*>(un + LB.ub + (tile * 64 + ln) * 8);
      const bf16x4 d = *reinterpret_cast<const bf16x4*>(un + LB.zb + (tile * 64 + ln) * 8);
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * R + 4 * (ln >> 4) + i, col = 16 * ct + (ln & 15);
        const bool ok = row < cu.nvalid;
        sU[row * LDV + col] = ok ? a[i] : static_cast<bf16>(0.f);
        sZ[row * LDV + col] = ok ? d[i] : static_cast<bf16>(0.f);
      }
    }
    for (int x = tid; x < C * DV; x += NT) {
      const int t = x / DV, v = x % DV;
      sO[t * LDV + v] = t < cu.nvalid ? d_o[vb0 + (long)t * vstride + v] : static_cast<bf16>(0.f);
    }
    __syncthreads();
    float dOS[TPH], dZS[TPH], dKt[TPH], X = 0.f;
    for (int j = 0; j < TPH; ++j) dOS[j] = dZS[j] = dKt[j] = 0.f;
    for (int v = 0; v < DV; ++v) {
      const float s0 = static_cast<float>(sS0[c * LDV + v]), ds = static_cast<float>(sdS[c * LDV + v]);
      X += ds * s0;
      for (int j = 0; j < TPH; ++j) {
        const int t = t0 + j;
        dOS[j] += s0 * static_cast<float>(sO[t * LDV + v]);
        dZS[j] += s0 * static_cast<float>(sZ[t * LDV + v]);
        dKt[j] += ds * static_cast<float>(sU[t * LDV + v]);
      }
    }
    for (int e = tid; e < C * C; e += NT) {
      const int r = e / C, i = e % C;
      float m1 = 0.f, m2 = 0.f;
      if (i <= r) {
        for (int v = 0; v < DV; ++v) {
          const float uu = static_cast<float>(sU[i * LDV + v]);
          m1 += static_cast<float>(sO[r * LDV + v]) * uu;
          m2 += static_cast<float>(sZ[r * LDV + v]) * uu;
        }
      }
      sM1[r * LDM + i] = m1;
      sM2[r * LDM + i] = i < r ? -m2 : 0.f;
    }
    __syncthreads();
    // ---- stage 2: q, k, b and the clamped cumulative decay G (log2) of every token
    float gs[TPH];
    float run = 0.f;
    for (int j = 0; j < TPH; ++j) {
      const int t = t0 + j;
      const bool ok = t < cu.nvalid;
      const long off = kb0 + (long)t * kstride + c;
      sq[t * DK + c] = ok ? q[off] : static_cast<bf16>(0.f);
      sk[t * DK + c] = ok ? k[off] : static_cast<bf16>(0.f);
      if constexpr (B_S) sb[t * DK + c] = ok ? bg[(cu.row + t) * H + cu.h] : static_cast<bf16>(0.f);
      else sb[t * DK + c] = ok ? bg[off] : static_cast<bf16>(0.f);
      run += ok ? fmaxf(static_cast<float>(g[off]) * kLog2e, -256.f) : 0.f;
      gs[j] = run;
    }
    sPart[hg * DK + c] = run;
    if (tid < C) sDb[tid] = 0.f;
    __syncthreads();
    float pre = 0.f;
    for (int h2 = 0; h2 < hg; ++h2) pre += sPart[h2 * DK + c];
    for (int j = 0; j < TPH; ++j) sG[(t0 + j) * DK + c] = gs[j] + pre;
    __syncthreads();
    // ---- stage 3: pairwise sums, dq, dk, db and the terms of dg
    const float Gl = sG[(C - 1) * DK + c];
    float amb[TPH], totB = 0.f;
    for (int j = 0; j < TPH; ++j) {
      const int t = t0 + j;
      const float Gt = sG[t * DK + c];
      const float pt = fast_exp2(Gt);
      float dqv = pt * dOS[j], de = -pt * dZS[j];
      for (int i = 0; i <= t; ++i) {
        const float kw = static_cast<float>(sk[i * DK + c]) * fast_exp2(Gt - sG[i * DK + c]);
        dqv += sM1[t * LDM + i] * kw;
        de += sM2[t * LDM + i] * kw;  // (zero at i = t)
      }
      float dkh = 0.f;
      for (int r = t; r < C; ++r) {
        const float w = fast_exp2(sG[r * DK + c] - Gt);
        const float er = static_cast<float>(sb[r * DK + c]) * static_cast<float>(sk[r * DK + c]);
        dkh += (sM2[r * LDM + t] * er + sM1[r * LDM + t] * static_cast<float>(sq[r * DK + c])) * w;
      }
      const float qt = static_cast<float>(sq[t * DK + c]), kt = static_cast<float>(sk[t * DK + c]);
      const float bt = static_cast<float>(sb[t * DK + c]);
      const float sf = fast_exp2(Gl - Gt);
      const float dkv = dkh + dKt[j] * sf + de * bt;
      const float dbv = de * kt;
      amb[j] = de * bt * kt + dqv * qt - dkh * kt - dKt[j] * kt * sf;
      totB += dKt[j] * kt * sf;
      if (t < cu.nvalid) {
        const long off = kb0 + (long)t * kstride + c;
        dq[off] = from_f<bf16>(dqv);
        dk[off] = from_f<bf16>(dkv);
        if constexpr (!B_S) db[off] = from_f<bf16>(dbv);
      }
      if constexpr (B_S) atomicAdd(&sDb[t], dbv);
    }
    // ---- stage 4: dg by suffix sums over the chunk
    float suf = 0.f;
    for (int j = TPH - 1; j >= 0; --j) { suf += amb[j]; amb[j] = suf; }
    __syncthreads();  // (sPart's decay totals are read)
    sPart[hg * DK + c] = suf;
    if (hg == 0) sTB[c] = 0.f;
    __syncthreads();
    atomicAdd(&sTB[c], totB);
    __syncthreads();
    float after = 0.f;
    for (int h2 = hg + 1; h2 < NH; ++h2) after += sPart[h2 * DK + c];
    const float base = sTB[c] + fast_exp2(Gl) * X + after;
    for (int j = 0; j < TPH; ++j) {
      const int t = t0 + j;
      if (t < cu.nvalid) dg[kb0 + (long)t * kstride + c] = from_f<bf16>(amb[j] + base);
    }
    if constexpr (B_S) {
      if (tid < cu.nvalid) db[(cu.row + tid) * H + cu.h] = from_f<bf16>(sDb[tid]);
    }
    __syncthreads();  // this unit's LDS readers are done
  }
}

// ------------------------------------------------------------------ launch
template <int DK, int DV>
static hipError_t launch_bwd(const BwdArgs& a) {
  const ChunkArgs& f = a.fwd;
  hipStream_t st = (hipStream_t)f.stream;
  hipError_t e = hipSuccess;
  if (!a.saved) {
    e = launch_bwd_forward_part(f);
    if (e != hipSuccess) return e;
  }
  constexpr int NV = 64 <= DV ? 64 : DV;
  const int nslices = DV / NV;
  if (f.nseg > 1) {
    // long sequences: transfer pass per segment (b; A = M^T is in the buffer from the forward
    // part's transfer pass, run here or by the training forward), the segments' end
    // gradients by a reverse scan, then the chain per segment
    const int nseg = f.nseg;
    const long units = (long)f.N * f.H * nseg;
    float* ebuf = reinterpret_cast<float*>(
        (char*)f.workspace + (bwd_workspace_bytes(false, f.B, f.T, f.H, DK, DV, f.N) + 255) / 256 * 256);
    float* dbuf = ebuf + units * DK * (DV + DK);
    hipLaunchKernelGGL((gdn2_bwd_chain_kernel<DK, DV, NV, true>), dim3((unsigned)(units * nslices)),
                       dim3(ChainShape<DK, DV, NV>::NT), 0, st, (char*)f.workspace,
                       (const bf16*)a.d_o, nullptr, nullptr, nullptr, f.T, f.H, nslices,
                       (int)units, nseg, f.seg_chunks, ebuf, nullptr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_seg_combine(ebuf, a.d_sN, dbuf, f.N, f.H, DK, DV, nseg, true, f.stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gdn2_bwd_chain_kernel<DK, DV, NV, false>), dim3((unsigned)(units * nslices)),
                       dim3(ChainShape<DK, DV, NV>::NT), 0, st, (char*)f.workspace,
                       (const bf16*)a.d_o, a.d_sN, a.d_s0, nullptr, f.T, f.H, nslices, (int)units,
                       nseg, f.seg_chunks, nullptr, dbuf);
  } else {
    hipLaunchKernelGGL((gdn2_bwd_chain_kernel<DK, DV, NV, false>), dim3((unsigned)(f.N * f.H * nslices)),
                       dim3(ChainShape<DK, DV, NV>::NT), 0, st, (char*)f.workspace,
                       (const bf16*)a.d_o, a.d_sN, a.d_s0, f.cu_seqlens, f.T, f.H, nslices,
                       f.N * f.H, 1, 0, nullptr, nullptr);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long nunits = split_slots(f.cu_seqlens != nullptr, f.B, f.T, f.N) * f.H;
  if (nunits > 0) {
    auto local = f.gate_flags == 3 ? gdn2_bwd_local_kernel<DK, DV, 3>
                 : f.gate_flags == 2 ? gdn2_bwd_local_kernel<DK, DV, 2>
                 : f.gate_flags == 1 ? gdn2_bwd_local_kernel<DK, DV, 1>
                                     : gdn2_bwd_local_kernel<DK, DV, 0>;
    const long grid = nunits < cu_count() ? nunits : cu_count();  // one per compute unit
    hipLaunchKernelGGL(local, dim3((unsigned)grid),
                       dim3(LocalShape<DK, DV>::NT), 0, st, (const bf16*)f.q, (const bf16*)f.k,
                       (const bf16*)f.v, (const bf16*)f.g, (const bf16*)f.b, (const bf16*)f.w,
                       (const bf16*)a.d_o, (const char*)f.workspace, (bf16*)a.dq, (bf16*)a.dk,
                       (bf16*)a.dv, (bf16*)a.dg, (bf16*)a.db, (bf16*)a.dw, a.range_flag,
                       f.cu_seqlens, f.N, f.T, f.H, nunits);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // units past the local kernel's decay range (rare): exact recomputation
    auto exact = f.gate_flags & kGateBScalar ? gdn2_bwd_exact_kernel<DK, DV, kGateBScalar>
                                             : gdn2_bwd_exact_kernel<DK, DV, 0>;
    hipLaunchKernelGGL(exact, dim3((unsigned)grid), dim3(256), 0, st, (const bf16*)f.q,
                       (const bf16*)f.k, (const bf16*)f.g, (const bf16*)f.b, (const bf16*)a.d_o,
                       (const char*)f.workspace, (bf16*)a.dq, (bf16*)a.dk, (bf16*)a.dg,
                       (bf16*)a.db, a.range_flag, f.cu_seqlens, f.N, f.T, f.H, nunits);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_chunk_bwd(const BwdArgs& a) {
  const ChunkArgs& f = a.fwd;
  if (f.dtype != 0) return hipErrorInvalidValue;
  if (f.d_k == 64 && f.d_v == 64) return launch_bwd<64, 64>(a);
  if (f.d_k == 64 && f.d_v == 128) return launch_bwd<64, 128>(a);
  if (f.d_k == 128 && f.d_v == 64) return launch_bwd<128, 64>(a);
  if (f.d_k == 128 && f.d_v == 128) return launch_bwd<128, 128>(a);
  return hipErrorInvalidValue;
}

}  // namespace gdn2
