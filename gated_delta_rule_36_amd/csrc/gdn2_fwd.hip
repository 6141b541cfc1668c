// Pipelined chunkwise forward of Gated Delta Rule-2 on gfx950 (bf16 inputs, fp32 state).
//
// One workgroup (8 waves) owns one (sequence, head, 64-column value slice) and walks the
// sequence's 64-token chunks in order. The chunk form is the one of the GDN-2 reading note
// (§3, chunkwise-training paragraph: inside a chunk the cumulative per-channel decay G
// normalises the state, which turns the chunk into an asymmetric delta recurrence) with the
// UT transform of the Gated DeltaNet visual reading (chunkwise section). With E = b*K,
// Z = w*V, Eg = E 2^G, Qg = Q 2^G, Kg = K 2^-G (log2 units, G relative to the chunk start):
//   A = strict_lower(Eg Kg^T)   P = lower_incl(Qg Kg^T)   T = (I + A)^-1
//   W = T Eg      U~ = T Z      U = U~ - W S
//   O = Qg S + P U              S <- Diag(2^Glast) (S + Kg^T U)
//
// Pipeline. The chunk factors (A, P, T, W, U~) do not depend on the state, so the work for
// chunk c+1's inputs (the decay scan and the gated operands) runs in the same three
// barrier-separated phases as chunk c's factor products and state update:
//   phase 1: chunk c:   A, P tiles on MFMA; 16x16 diagonal inverses (fp32)
//            chunk c+1: per-thread decay totals
//   phase 2: chunk c:   [W | U~] = T [Eg | Z] by block forward substitution
//            chunk c+1: per-channel decay scan and factors
//   phase 3: chunk c:   U, O, state update (waves 0-3, one 16-column state tile each)
//            chunk c+1: gated operands into LDS (all waves), then next loads
// so the VALU-heavy operand preparation of one chunk overlaps the MFMA work of the other.
// The operands of the state update (Qg, Kg) are double-buffered by chunk parity.
//
// Layouts. Every operand is written row-major ([token][channel], channels in the phi order
// of Mma<bf16> so that a state-tile fragment pair is one 16-byte read); products that
// contract over tokens read them with the gfx950 transposing LDS read (ds_read_b64_tr_b16:
// within each 16-lane group, lane i's element j is element i%4 of the 8 bytes addressed by
// lane 4j + i/4), so no operand is ever written twice or transposed through LDS.
// A and P tiles are formed transposed (Kg rows times Eg / Qg rows), which leaves each lane
// holding a row fragment of A / P: they are stored in fragment order, one 8-byte read each.
// The output is formed transposed as well (O^T = S^T Qg^T + U^T P^T), so each lane stores
// 4 consecutive value columns of one token.
//
// Range. The chunk-referenced factors 2^G and 2^-G are used when every channel's decay over
// the chunk stays within kFwdFastDecay2 (100 log2 units, 69 nats). Otherwise the chunk takes
// the general path, exact for any decay (alpha in (0, 1]): operands referenced to 16-token
// block boundaries (E 2^(G - Gs), Q 2^(G - Gs), K 2^(Ge - G), every factor <= 1), the
// off-diagonal A / P tiles scaled by 2^(Gs(R) - Ge(I)) <= 1, and the diagonal 16x16 tiles
// formed in fp32 from the raw inputs with running products of alpha (no cancellation, no
// overflow); the consumers apply the block factors 2^Gs(R) and 2^(Glast - Ge(I)).

#include <type_traits>

#include "gdn2_chunk_common.h"
#include "gdn2_launch.h"

namespace gdn2 {

namespace {

constexpr float kFwdFastDecay2 = 100.f;  // log2 units
// A single token's decay below 2^-256 (alpha < 1e-77) is taken as 2^-256: alpha then
// vanishes at fp32 precision either way, and the bound keeps the chunk's cumulative log2
// decay (at most 64 x 256) resolved to about 1e-3 in fp32, so that differences of it stay
// exact enough for the factors of the tokens after such a reset.
constexpr float kMinTokenDecay2 = -256.f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Buffer resource over `bytes` bytes from p (raw buffer, dword data format): loads at offsets
// at or past the end return zeros, so a chunk's rows past the end of its sequence need
// neither clamped addresses nor masking.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}
// Per-column value loads (v, w) are read by one workgroup only: non-temporal (the `nt`
// policy bit), so they stream through the caches instead of displacing the key-side rows
// that the two value slices of a head share in L2 (measured 154.7 -> 148.5 us per launch on
// the 1.3B-layer workload; the same bit on the key-side loads made it slower).
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}
// Key-side loads (q, k, g, b): both value-slice workgroups of a head read the same rows, one
// through the other's L2 hits, each once. Agent-scope loads (the `sc1` policy bit) skip the
// vector L1, whose pending misses bound this kernel, and stay cached in L2 (measured 145.0
// -> 143.2 us per launch on the 1.3B-layer workload; plain buffer loads 141.9 -> 141.1,
// non-temporal ones slower). `off` is in elements from `base`; the rows are clamped into
// the sequence by the caller.
__device__ __forceinline__ uint4 kload(const bf16* base, unsigned off) {
  return __builtin_bit_cast(
      uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc(base, 0x7ffffff0), (int)(off * 2u), 0, 16));
}
__device__ __forceinline__ uint32_t bload2(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// 4 bf16 from the transposing LDS read (see the file comment for the lane mapping).
__device__ __forceinline__ bf16x4 ds_tr4(const bf16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ bf16x4 to_bf4(f4 v) {
  return __builtin_bit_cast(bf16x4, make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])));
}
__device__ __forceinline__ f4 from_bf4(bf16x4 v) {
  return f4{static_cast<float>(v[0]), static_cast<float>(v[1]), static_cast<float>(v[2]),
            static_cast<float>(v[3])};
}
__device__ __forceinline__ bf16x8 scale8(bf16x8 v, const float* s) {
  bf16x8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = static_cast<bf16>(static_cast<float>(v[i]) * s[i]);
  return o;
}
__device__ __forceinline__ f4 mma32(bf16x8 a, bf16x8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mma16(bf16x4 a, bf16x4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4v, a),
                                                   __builtin_bit_cast(short4v, b), c, 0, 0, 0);
}

// Element offset of (row r, phi-ordered column col) in a [64][DK] operand array. With d_k =
// 128 the rows are 256 bytes (the LDS's 128 four-byte banks hold two of them) and the 16-byte
// chunk index of a column is XORed with f(r) = 4 ((r >> 1) & 3) + 2 ((r >> 3) & 1). Both ways
// the kernel reads these arrays then hit every bank once per 32-lane pass: 16-byte row
// fragments (16 consecutive rows x two chunks; rows of one parity need distinct f >> 1) and
// transposing reads (8 consecutive rows x four chunks of one 64-byte group; rows of one
// parity among eight need distinct f >> 2). The 8-byte pieces and runs of 4 channels the
// kernel addresses never straddle a chunk.
template <int LDK, bool SWZ>
__device__ __forceinline__ int kx(int r, int col) {
  if constexpr (SWZ) return r * LDK + (col ^ ((4 * ((r >> 1) & 3) + 2 * ((r >> 3) & 1)) << 3));
  else return r * LDK + col;
}

// Tile slots of the causal 16x16 pairs (R, I), I <= R: (0,0) (1,0) (1,1) (2,0) (2,1) (2,2)
// (3,0) (3,1) (3,2) (3,3); and of the six strictly-lower pairs of A.
__device__ __forceinline__ constexpr int pair_slot(int R, int I) { return R * (R + 1) / 2 + I; }
__device__ __forceinline__ constexpr int off_slot(int R, int I) { return R * (R - 1) / 2 + I; }

}  // namespace

template <int DK>
struct FwdShape {
  static constexpr int C = 64;          // chunk length
  static constexpr int NV = 64;         // value columns per workgroup
  static constexpr int NW = 8;          // waves: 0-3 hold the state, 4-7 prepare operands
  static constexpr int NT = 64 * NW;
  static constexpr int PT = 256;        // operand-preparation threads (waves 4-7)
  static constexpr int CG = DK / 8;     // key side: 8 channels per thread
  static constexpr int TG = PT / CG;    // token groups
  static constexpr int TPT = C / TG;    // tokens per thread (4 or 2)
  static constexpr int GPB = 16 / TPT;  // token groups per 16-token block
  static constexpr int VTPT = 2;        // value side (waves 0-3): 2 tokens x 8 columns
  static constexpr int NCT = DK / 16;   // key-channel tiles
  static constexpr int KS = DK / 32;    // 32-wide K steps over the channels
  // [64][DK] operand arrays: with d_k = 128, unpadded rows whose 16-byte chunks are
  // XOR-swizzled by the row (see kx); with d_k = 64, rows padded by 8 elements
  static constexpr bool SWZ = DK == 128;
  static constexpr int LDK = SWZ ? DK : DK + 8;  // pitches (elements) of the bf16 arrays
  static constexpr int LDZ = NV + 8;
  static constexpr int LDW = C + 8;
  static constexpr int LDTT = 24;       // column-major 16x16 T blocks
  static constexpr int LDD = 20;        // fp32 diagonal blocks of -A (column-major)
  // factor rows per chunk: Gs(R) (R = 0..3), Glast, 2^Glast, and 2^(Gs(R) - Ge(I)) for the
  // tile pairs (R, I) = (2, 0), (3, 0), (3, 1) two or more blocks apart
  static constexpr int NFAC = 9;
  static constexpr int F_GS = 0, F_GL = 4, F_GAM = 5, F_OFF = 6;

  static constexpr int SZ_K = C * LDK * 2;
  static constexpr int OFF_EG = 0;                      // E 2^G (one buffer)
  static constexpr int OFF_QG = OFF_EG + SZ_K;          // Q 2^G (two, by chunk parity)
  static constexpr int OFF_KG = OFF_QG + 2 * SZ_K;      // K 2^-G (two)
  static constexpr int OFF_Z = OFF_KG + 2 * SZ_K;       // Z [64][NV]
  static constexpr int OFF_W = OFF_Z + C * LDZ * 2;     // -W, column-major [DK][64]
  static constexpr int OFF_A = OFF_W + DK * LDW * 2;    // -A off-diagonal tiles (fragments)
  static constexpr int OFF_P = OFF_A + 6 * 512;         // P tiles (fragments)
  static constexpr int OFF_T = OFF_P + 10 * 512;        // T diagonal blocks, column-major
  static constexpr int OFF_AD = OFF_T + 4 * 16 * LDTT * 2;  // -A diagonal blocks, fp32
  static constexpr int OFF_TOT = OFF_AD + 4 * 16 * LDD * 4; // decay totals / prefixes
  static constexpr int OFF_FAC = OFF_TOT + TG * DK * 4;     // factor rows (two)
  static constexpr int OFF_FLAG = OFF_FAC + 2 * NFAC * DK * 4;
  static constexpr int OFF_ID = OFF_FLAG + 16;              // 16x16 identity, fp32, pitch LDD
  static constexpr int LDS_BYTES = OFF_ID + 16 * LDD * 4;

  static_assert(TPT >= 1 && 16 % TPT == 0, "token groups tile 16-token blocks");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(DK == 64 || DK == 128, "key width");
};

// The diagonal 16x16 blocks of A and P formed exactly for any decay (general path): for
// tokens i <= r of block R, A[r][i] = sum_c e_rc k_ic prod_{j=i+1..r} alpha_jc (i < r) and
// P[r][i] the same with q in place of e, from the raw inputs (global, L2-resident), walking
// i downwards with a running product of alpha (no cancellation, no overflow). Each thread
// takes two (block, row) items, 8 channels each; the 16 channel groups of an item are 16
// adjacent lanes, which reduce the partial sums.
template <int DK, bool BS>
__device__ __forceinline__ void diag_tiles_exact(const bf16* qb, const bf16* kb, const bf16* gb,
                                                 const bf16* bb, const bf16* bsb, long kstride,
                                                 int H, int c0, int nvalid, int tid,
                                                 float* sAd, bf16* sP) {
  constexpr int NCG = DK / 8;          // channel groups of 8
  constexpr int IPT = 64 * NCG / 512;  // items per thread (64 (block, row) items)
  constexpr int LDD = FwdShape<DK>::LDD;
  const int cq = tid % NCG;
  for (int it = 0; it < IPT; ++it) {
    const int item = tid / NCG + it * (512 / NCG);
    const int R = item >> 4, r = item & 15;
    const int tr = 16 * R + r;
    float er[8], qr[8], f[8];
    {
      Vec8<bf16> vq, vk, vb;
      if (tr < nvalid) {
        const long off = (long)(c0 + tr) * kstride + cq * 8;
        vq.load(qb + off);
        vk.load(kb + off);
        if constexpr (BS) { vb.load_one(bsb + (long)(c0 + tr) * H); vb.splat(); }
        else vb.load(bb + off);
      } else {
        vq.zero(); vk.zero(); vb.zero();
      }
      float fk[8], fb[8];
      vq.to_float(qr); vk.to_float(fk); vb.to_float(fb);
#pragma unroll
      for (int c = 0; c < 8; ++c) { er[c] = fb[c] * fk[c]; f[c] = 1.f; }
    }
    bf16* pt = sP + pair_slot(R, R) * 256;
    for (int i = r; i >= 0; --i) {
      const int ti = 16 * R + i;
      float ki[8], gi[8];
      {
        Vec8<bf16> vk, vg;
        if (ti < nvalid) {
          const long off = (long)(c0 + ti) * kstride + cq * 8;
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
        f[c] *= fast_exp2(gi[c] * kLog2e);  // alpha_i: the product now covers tokens i..r
      }
#pragma unroll
      for (int m = 1; m < NCG; m <<= 1) {
        a += __shfl_xor(a, m, 64);
        p += __shfl_xor(p, m, 64);
      }
      if (cq == 0) {
        if (i < r) sAd[R * 16 * LDD + i * LDD + r] = -a;  // column-major
        pt[(16 * (i >> 2) + r) * 4 + (i & 3)] = static_cast<bf16>(p);
      }
    }
    if (cq == 0) {
      for (int i = r + 1; i < 16; ++i) pt[(16 * (i >> 2) + r) * 4 + (i & 3)] = static_cast<bf16>(0.f);
    }
  }
}

// One 16x16 diagonal block of T = (I + A)^-1 by fp32 forward substitution, column c per lane
// (lanes 0..15 write; the other lane groups repeat the work). sAdb: the -A block stored
// column-major (column i at sAdb + i * LDD, rows r > i used), read in full before the
// substitution so that its 15 dependent steps wait on the LDS once; sId: the 16x16 identity
// (row c at sId + c * LDD), which starts column c; sTb: the block of T, column-major.
template <int LDD, int LDTT>
__device__ __forceinline__ void tinv_block(const float* sAdb, const float* sId, bf16* sTb, int lane) {
  const int c = lane & 15;
  float col[15][16];
#pragma unroll
  for (int i = 0; i < 15; ++i) {
#pragma unroll
    for (int r4 = 4 * ((i + 1) / 4); r4 < 16; r4 += 4) {
      const f4 v = *reinterpret_cast<const f4*>(sAdb + i * LDD + r4);
#pragma unroll
      for (int j = 0; j < 4; ++j) col[i][r4 + j] = v[j];
    }
  }
  float x[16];
#pragma unroll
  for (int r4 = 0; r4 < 16; r4 += 4) {
    const f4 v = *reinterpret_cast<const f4*>(sId + c * LDD + r4);
#pragma unroll
    for (int j = 0; j < 4; ++j) x[r4 + j] = v[j];
  }
#pragma unroll
  for (int i = 0; i < 15; ++i) {
#pragma unroll
    for (int r = i + 1; r < 16; ++r) x[r] += col[i][r] * x[i];  // col holds -A[r][i]
  }
  if (lane < 16) {
#pragma unroll
    for (int r4 = 0; r4 < 16; r4 += 4)
      *reinterpret_cast<uint2*>(sTb + c * LDTT + r4) =
          make_uint2(pack_bf16(x[r4], x[r4 + 1]), pack_bf16(x[r4 + 2], x[r4 + 3]));
  }
}

// Packed batches of up to this many sequences are started longest first.
constexpr int kOrderMaxSeqs = 256;

template <int DK, int GL>
__global__ void __launch_bounds__(512)
gdn2_fwd_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                const bf16* __restrict__ v, const bf16* __restrict__ g,
                const bf16* __restrict__ bg, const bf16* __restrict__ wg,
                const float* s0, bf16* __restrict__ o, float* sN,
                const int* __restrict__ cu_seqlens, int T_len, int H, int DV, int nslices,
                int nunits) {
  using Sh = FwdShape<DK>;
  constexpr int C = Sh::C, CG = Sh::CG, TPT = Sh::TPT, NCT = Sh::NCT, KS = Sh::KS;
  constexpr int LDK = Sh::LDK, LDZ = Sh::LDZ, LDW = Sh::LDW, LDTT = Sh::LDTT, LDD = Sh::LDD;
  auto KX = [](int r, int col) __attribute__((always_inline)) { return kx<Sh::LDK, Sh::SWZ>(r, col); };
  constexpr int NFAC = Sh::NFAC;
  constexpr bool b_scalar = (GL & kGateBScalar) != 0;
  constexpr bool w_scalar = (GL & kGateWScalar) != 0;
  __shared__ __attribute__((aligned(16))) char smem[Sh::LDS_BYTES];
  bf16* const sEg = reinterpret_cast<bf16*>(smem + Sh::OFF_EG);
  bf16* const sZ = reinterpret_cast<bf16*>(smem + Sh::OFF_Z);
  bf16* const sW = reinterpret_cast<bf16*>(smem + Sh::OFF_W);
  bf16* const sA = reinterpret_cast<bf16*>(smem + Sh::OFF_A);
  bf16* const sP = reinterpret_cast<bf16*>(smem + Sh::OFF_P);
  bf16* const sT = reinterpret_cast<bf16*>(smem + Sh::OFF_T);
  float* const sAd = reinterpret_cast<float*>(smem + Sh::OFF_AD);
  float* const sId = reinterpret_cast<float*>(smem + Sh::OFF_ID);
  float* const sTot = reinterpret_cast<float*>(smem + Sh::OFF_TOT);
  int* const sFlag = reinterpret_cast<int*>(smem + Sh::OFF_FLAG);
  auto sQg = [&](int p) __attribute__((always_inline)) {
    return reinterpret_cast<bf16*>(smem + Sh::OFF_QG + p * Sh::SZ_K);
  };
  auto sKg = [&](int p) __attribute__((always_inline)) {
    return reinterpret_cast<bf16*>(smem + Sh::OFF_KG + p * Sh::SZ_K);
  };
  auto sFac = [&](int p) __attribute__((always_inline)) {
    return reinterpret_cast<float*>(smem + Sh::OFF_FAC) + p * NFAC * DK;
  };

  int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int lane = tid & 63;
  int m16 = lane & 15, g4 = lane >> 4;
  // Lane-derived indices are re-derived from an opaque copy of the thread id at every phase
  // (see opaque()): otherwise the compiler hoists every per-lane LDS address and constant out
  // of the chunk loop and keeps (or spills) them all across it.
  auto fresh_lane = [&]() __attribute__((always_inline)) {
    tid = opaque(tid);
    lane = tid & 63;
    m16 = lane & 15;
    g4 = lane >> 4;
  };

  // Workgroup -> (sequence, head, slice); the slices of one (sequence, head) get ids that
  // are congruent mod 8, so they run on the same XCD and share its L2 for the key side.
  const int grp = blockIdx.x / (8 * nslices);
  const int gsz = min(8, nunits - grp * 8);
  const int gi = blockIdx.x - grp * 8 * nslices;
  const int slice = gi / gsz;
  const int nh = grp * 8 + gi % gsz;
  const int h = nh % H;
  int n = nh / H;
  if (cu_seqlens != nullptr && nunits / H <= kOrderMaxSeqs) {
    // Packed batch: workgroups start in id order, so ids go to sequences longest first (ties
    // by index) and the longest chains do not wait for a second round of workgroups. Each
    // sequence's rank is counted in LDS (which the chunk loop has not used yet) by two lanes,
    // each over half of the length table (padded with -1, shorter than any sequence).
    static_assert(Sh::LDS_BYTES >= 4 * (kOrderMaxSeqs + 1) && kOrderMaxSeqs * 2 <= 512,
                  "sequence order table");
    const int nseq = nunits / H;
    const int npad = (nseq + 7) & ~7;
    int* const sLen = reinterpret_cast<int*>(smem);
    if (tid < npad) {
      int l = -1;
      if (tid < nseq) {
        int a = cu_seqlens[tid], b = cu_seqlens[tid + 1];
        a = a < 0 ? 0 : (a > T_len ? T_len : a);
        b = b < a ? a : (b > T_len ? T_len : b);
        l = b - a;
      }
      sLen[tid] = l;
    }
    __syncthreads();
    const int i = tid >> 1, part = tid & 1;
    int r = 0;
    if (i < nseq) {
      const int li = sLen[i];
      const int j0 = part * (npad / 2);
      const int4* row = reinterpret_cast<const int4*>(sLen + j0);
      for (int x = 0; x < npad / 8; ++x) {
        const int4 v = row[x];
        const int j = j0 + 4 * x;
        r += (v.x > li || (v.x == li && j < i)) + (v.y > li || (v.y == li && j + 1 < i)) +
             (v.z > li || (v.z == li && j + 2 < i)) + (v.w > li || (v.w == li && j + 3 < i));
      }
    }
    r += __shfl_xor(r, 1, 64);
    if (i < nseq && part == 0 && r == n) sLen[npad] = i;  // ranks are a permutation
    __syncthreads();
    n = __builtin_amdgcn_readfirstlane(sLen[npad]);
    __syncthreads();
  }
  const int col0 = slice * Sh::NV;

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
  const long kstride = (long)H * DK;
  const long vstride = (long)H * DV;
  const bf16* qb = q + row0 * kstride + (long)h * DK;
  const bf16* kb = k + row0 * kstride + (long)h * DK;
  const bf16* gb = g + row0 * kstride + (long)h * DK;
  const bf16* bb = bg + row0 * kstride + (long)h * DK;
  const bf16* vb = v + row0 * vstride + (long)h * DV + col0;
  const bf16* wb = wg + row0 * vstride + (long)h * DV + col0;
  const bf16* bsb = bg + row0 * H + h;  // scalar gates: one value per (token, head)
  const bf16* wsb = wg + row0 * H + h;
  bf16* ob = o + row0 * vstride + (long)h * DV + col0;
  const int nchunks = (len + C - 1) / C;
  auto nvalid_of = [&](int c) __attribute__((always_inline)) { return min(C, len - c * C); };

  // ---------------------------------------------------------------- chunk-c work pieces
  // A / P tile (R, I): D = Kg_I Xg_R^T, so lane (m16, g4) holds X Kg^T [16R + m16][16I + 4g4 + j]
  auto tile = [&](int p, int R, int I, bool isP, bool gen) __attribute__((always_inline)) {
    const bf16* kg = sKg(p);
    const bf16* X = isP ? sQg(p) : sEg;
    const bool scale = gen && R - I >= 2;  // general path: 2^(Gs(R) - Ge(I)) per channel
    const float* fr = sFac(p) + (Sh::F_OFF + (R == 2 ? 0 : I == 0 ? 1 : 2)) * DK;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      bf16x8 a = *reinterpret_cast<const bf16x8*>(kg + KX(16 * I + m16, 32 * s + 8 * g4));
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(X + KX(16 * R + m16, 32 * s + 8 * g4));
      if (scale) {  // the fragment's channels: 32s + 4g4 + (0..3), 32s + 16 + 4g4 + (0..3)
        const f4 lo = *reinterpret_cast<const f4*>(fr + 32 * s + 4 * g4);
        const f4 hi = *reinterpret_cast<const f4*>(fr + 32 * s + 16 + 4 * g4);
        const float sc[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        a = scale8(a, sc);
      }
      acc = mma32(a, b, acc);
    }
    return acc;
  };
  auto put_off_a = [&](int R, int I, f4 acc) __attribute__((always_inline)) {
    *reinterpret_cast<bf16x4*>(sA + off_slot(R, I) * 256 + lane * 4) = to_bf4(-acc);
  };
  auto put_p = [&](int R, int I, f4 acc) __attribute__((always_inline)) {
    if (R == I) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = (4 * g4 + j <= m16) ? acc[j] : 0.f;
    }
    *reinterpret_cast<bf16x4*>(sP + pair_slot(R, I) * 256 + lane * 4) = to_bf4(acc);
  };
  auto put_diag_a = [&](int R, f4 acc) __attribute__((always_inline)) {
    // fp32, column-major: (r, i) at i * LDD + r
#pragma unroll
    for (int j = 0; j < 4; ++j)
      sAd[R * 16 * LDD + (4 * g4 + j) * LDD + m16] = (4 * g4 + j < m16) ? -acc[j] : 0.f;
  };
  // general path, after the tiles and a barrier: turn the block-referenced operands into
  // what phases 2 and 3 read (E 2^G and Q 2^G: times 2^Gs(R) <= 1; K 2^(Glast - G): times
  // 2^(Glast - Ge(R)) <= 1), so that those phases run the same code on both paths. Thread:
  // token r, DK / 8 channels (runs of 4 channels are contiguous in phi order).
  auto rescale = [&](int p) __attribute__((always_inline)) {
    const float* fac = sFac(p);
    bf16* qw = sQg(p);
    bf16* kw = sKg(p);
    constexpr int CPT = DK / 8;
    const int r = tid >> 3, m = tid & 7, R = r >> 4;
    const int geb = R < 3 ? Sh::F_GS + R + 1 : Sh::F_GL;
#pragma unroll
    for (int j = 0; j < CPT / 4; ++j) {
      const int ch = CPT * m + 4 * j;
      const int o = KX(r, Mma<bf16>::phi(ch));
      f4 sx, sy;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sx[e] = fast_exp2(fac[(Sh::F_GS + R) * DK + ch + e]);
        sy[e] = fast_exp2(fac[Sh::F_GL * DK + ch + e] - fac[geb * DK + ch + e]);
      }
      *reinterpret_cast<bf16x4*>(sEg + o) = to_bf4(from_bf4(*reinterpret_cast<const bf16x4*>(sEg + o)) * sx);
      *reinterpret_cast<bf16x4*>(qw + o) = to_bf4(from_bf4(*reinterpret_cast<const bf16x4*>(qw + o)) * sx);
      *reinterpret_cast<bf16x4*>(kw + o) = to_bf4(from_bf4(*reinterpret_cast<const bf16x4*>(kw + o)) * sy);
    }
  };
  // block forward substitution of one column tile: key tile kt (RHS = E 2^G, result -W
  // into sW, column-major) or value tile (RHS = Z, result U~ in X)
  auto column = [&](bool key, int ct, f4* X) __attribute__((always_inline)) {
    bf16x4 fa[6], tf[4], Xb[4];
#pragma unroll
    for (int s = 0; s < 6; ++s) fa[s] = *reinterpret_cast<const bf16x4*>(sA + s * 256 + lane * 4);
#pragma unroll
    for (int R = 0; R < 4; ++R)
      tf[R] = ds_tr4(sT + R * 16 * LDTT + (4 * g4 + (m16 >> 2)) * LDTT + 4 * (m16 & 3));
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      f4 acc;
      if (key) {
        const int pcol = 32 * (ct >> 1) + 8 * (m16 & 3) + 4 * (ct & 1);  // phi of 16ct + 4(m16&3)
        acc = from_bf4(ds_tr4(sEg + KX(16 * R + 4 * g4 + (m16 >> 2), pcol)));
      } else {
        acc = from_bf4(ds_tr4(sZ + (16 * R + 4 * g4 + (m16 >> 2)) * LDZ + 16 * ct + 4 * (m16 & 3)));
      }
#pragma unroll
      for (int J = 0; J < R; ++J) acc = mma16(fa[off_slot(R, J)], Xb[J], acc);
      X[R] = mma16(tf[R], to_bf4(acc), f4{0.f, 0.f, 0.f, 0.f});
      Xb[R] = to_bf4(X[R]);
    }
    if (key) {
#pragma unroll
      for (int R = 0; R < 4; ++R)
        *reinterpret_cast<bf16x4*>(sW + (16 * ct + m16) * LDW + 16 * R + 4 * g4) = to_bf4(-X[R]);
    }
  };
  auto flag = [&](int p) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane(sFlag[p]) != 0;
  };

  if (wave < 4) {
    // ======================================================= state waves (0-3)
    // S[mt]: key rows 16mt + 4g4 + i of value column 16w + m16
    const int w = wave;
    f4 S[NCT];
    const long sbase = ((long)n * H + h) * DK * DV + col0 + 16 * w + m16;
#pragma unroll
    for (int mt = 0; mt < NCT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        S[mt][i] = (s0 != nullptr) ? s0[sbase + (long)(16 * mt + 4 * g4 + i) * DV] : 0.f;
        // consumed here, before the chunk loop: otherwise the compiler, which cannot tell the
        // first iteration from the others, waits for every memory access in flight at the
        // state's first use in every iteration
        asm volatile("" : "+v"(S[mt][i]));
      }
    // value side of the operand preparation: Z = w * v, tokens 2vtk, 2vtk + 1, columns 8vcg..
    int vcg = tid & 7, vtk = tid >> 3;
    auto fresh = [&]() __attribute__((always_inline)) {
      fresh_lane();
      vcg = tid & 7;
      vtk = tid >> 3;
    };
    Vec8<bf16> rv[2], rw[2];
    // Prefetch loads are unconditional (rows clamped into the sequence, chunk index clamped to
    // the last chunk) and tokens past a chunk's end are zeroed where the values are used: the
    // compiler can then count the loads in flight exactly and wait for only the ones it needs.
    auto load_vw = [&](int c) __attribute__((always_inline)) {
      const int cc = min(c, nchunks - 1) * C;
      const int rows = c < nchunks ? nvalid_of(c) : 0;  // past the last chunk: zeros, no traffic
      const auto rv_ = rsrc(vb + (long)cc * vstride, rows * (int)vstride * 2);
      const auto rw_ = rsrc(w_scalar ? wsb + (long)cc * H : wb + (long)cc * vstride,
                            w_scalar ? rows * H * 2 : rows * (int)vstride * 2);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 2 * vtk + j;
        rv[j].r = bload16(rv_, r * (int)vstride * 2 + vcg * 16);
        if constexpr (w_scalar) rw[j].r.x = bload2(rw_, r * H * 2);
        else rw[j].r = bload16(rw_, r * (int)vstride * 2 + vcg * 16);
      }
    };
    auto make_z = [&]() __attribute__((always_inline)) {  // rows past the end load as 0
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float fv[8], fw[8], z[8];
        rv[j].to_float(fv);
        if constexpr (w_scalar) rw[j].splat();
        rw[j].to_float(fw);
#pragma unroll
        for (int i = 0; i < 8; ++i) z[i] = fv[i] * fw[i];
        store8(sZ + (2 * vtk + j) * LDZ + vcg * 8, z);
      }
    };
    f4 Ut[4];  // U~ of this wave's value tile, from phase 2 to phase 3

    if (tid < 256) sId[(tid >> 4) * LDD + (tid & 15)] = (tid >> 4) == (tid & 15) ? 1.f : 0.f;
    if (nchunks > 0) {  // prologue: chunk 0's operands (three barriers, as the other waves)
      load_vw(0);
      lds_barrier();
      fresh();
      lds_barrier();
      fresh();
      make_z();
      lds_barrier();
      fresh();
    }
    for (int c = 0; c < nchunks; ++c) {
      fresh();
      const int p = c & 1;
      const int c0 = c * C;
      const int nvalid = nvalid_of(c);
      const bool more = c + 1 < nchunks;
      const bool gen = flag(p);
      load_vw(c + 1);  // the next chunk's values, for its Z in phase 3
      // ---- phase 1: one A / P tile, diagonal A tile w and its inverse block
      if (!gen) {
        switch (w) {
          case 0: put_p(0, 0, tile(p, 0, 0, true, false)); break;
          case 1: put_p(1, 1, tile(p, 1, 1, true, false)); break;
          case 2: put_p(1, 0, tile(p, 1, 0, true, false)); break;
          default: put_off_a(1, 0, tile(p, 1, 0, false, false)); break;
        }
        put_diag_a(w, tile(p, w, w, false, false));
        // reads only what this wave just wrote: no barrier needed
        tinv_block<LDD, LDTT>(sAd + w * 16 * LDD, sId, sT + w * 16 * LDTT, lane);
      } else {
        switch (w) {
          case 0: put_p(3, 2, tile(p, 3, 2, true, true)); put_off_a(3, 2, tile(p, 3, 2, false, true)); break;
          case 1: put_p(3, 1, tile(p, 3, 1, true, true)); put_off_a(3, 1, tile(p, 3, 1, false, true)); break;
          case 2: put_p(3, 0, tile(p, 3, 0, true, true)); put_off_a(3, 0, tile(p, 3, 0, false, true)); break;
          default: put_p(2, 1, tile(p, 2, 1, true, true)); put_off_a(2, 1, tile(p, 2, 1, false, true)); break;
        }
        diag_tiles_exact<DK, b_scalar>(qb, kb, gb, bb, bsb, kstride, H, c0, nvalid, tid, sAd, sP);
        lds_barrier();
        fresh();
        tinv_block<LDD, LDTT>(sAd + w * 16 * LDD, sId, sT + w * 16 * LDTT, lane);
        rescale(p);
      }
      lds_barrier();
      fresh();
      // ---- phase 2: key tile (DK = 128) and this wave's value tile
      if constexpr (NCT == 8) {
        f4 X[4];
        column(true, w, X);
      }
      column(false, w, Ut);
      lds_barrier();
      fresh();
      // ---- phase 3: the next chunk's Z (its loads were issued in phase 1), then
      // U = U~ - W S, O, state update
      if (more) make_z();
      {
        const bf16* qg = sQg(p);
        const bf16* kg = sKg(p);
        const float* fac = sFac(p);
        bf16x8 Sb[KS];  // state tiles (2s, 2s+1) as K = 32 fragments (channels in phi pairs)
#pragma unroll
        for (int s = 0; s < KS; ++s) Sb[s] = cat8(to_bf4(S[2 * s]), to_bf4(S[2 * s + 1]));
        f4 U[4];
#pragma unroll
        for (int R = 0; R < 4; ++R) {  // sW holds -W, column-major
          U[R] = Ut[R];
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            const bf16* w0 = sW + (32 * s + 4 * g4 + (m16 >> 2)) * LDW + 16 * R + 4 * (m16 & 3);
            U[R] = mma32(cat8(ds_tr4(w0), ds_tr4(w0 + 16 * LDW)), Sb[s], U[R]);
          }
        }
        // O^T = S^T Qg^T + U^T P^T per 16-token block R; lane: token 16R + m16, columns 4g4..
        // (U^T P^T as K = 32 products over token-block pairs: U tiles (2s2, 2s2+1) against the
        // P fragments of the same blocks, zero above the diagonal; all products of one
        // accumulator chain use the one instruction shape)
        const bf16x8 Ub32[2] = {cat8(to_bf4(U[0]), to_bf4(U[1])), cat8(to_bf4(U[2]), to_bf4(U[3]))};
        const bf16x4 zero4 = {};
#pragma unroll
        for (int R = 0; R < 4; ++R) {
          f4 Ot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s)
            Ot = mma32(Sb[s], *reinterpret_cast<const bf16x8*>(qg + KX(16 * R + m16, 32 * s + 8 * g4)), Ot);
#pragma unroll
          for (int s2 = 0; 2 * s2 <= R; ++s2) {
            const bf16x4 p0 = *reinterpret_cast<const bf16x4*>(sP + pair_slot(R, 2 * s2) * 256 + lane * 4);
            const bf16x4 p1 = 2 * s2 + 1 <= R
                                  ? *reinterpret_cast<const bf16x4*>(sP + pair_slot(R, 2 * s2 + 1) * 256 + lane * 4)
                                  : zero4;
            Ot = mma32(Ub32[s2], cat8(p0, p1), Ot);
          }
          const int r = 16 * R + m16;
          if (r < nvalid) {
            const uint2 pk = make_uint2(pack_bf16(Ot[0], Ot[1]), pack_bf16(Ot[2], Ot[3]));
            __builtin_nontemporal_store(__builtin_bit_cast(u32x2, pk),
                                        reinterpret_cast<u32x2*>(ob + (long)(c0 + r) * vstride + 16 * w + 4 * g4));
          }
        }
        // S <- Diag(2^Glast) (S + Kg^T U); on the general path Kg holds K 2^(Glast - G) and
        // S <- Diag(2^Glast) S + Kg^T U
#pragma unroll
        for (int mt = 0; mt < NCT; ++mt) {
          const f4 gam = *reinterpret_cast<const f4*>(fac + Sh::F_GAM * DK + 16 * mt + 4 * g4);
          const int pcol = 32 * (mt >> 1) + 8 * (m16 & 3) + 4 * (mt & 1);  // phi of 16mt + 4(m16&3)
          f4 acc = gen ? S[mt] * gam : S[mt];
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            // rows r and r + 16 share the swizzle
            const bf16* k0 = kg + KX(32 * s2 + 4 * g4 + (m16 >> 2), pcol);
            acc = mma32(cat8(ds_tr4(k0), ds_tr4(k0 + 16 * LDK)), Ub32[s2], acc);
          }
          S[mt] = gen ? acc : acc * gam;
        }
      }
      lds_barrier();
      fresh();
    }
    if (sN != nullptr) {
#pragma unroll
      for (int mt = 0; mt < NCT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sN[sbase + (long)(16 * mt + 4 * g4 + i) * DV] = S[mt][i];
    }
  } else {
    // ======================================================= operand waves (4-7)
    // key side of the operand preparation: channels [8cg, +8) of tokens [TPT*tg, +TPT)
    int pt = tid - 256;
    int cg = pt % CG, tg = pt / CG, blk = tg / Sh::GPB;
    auto fresh = [&]() __attribute__((always_inline)) {
      fresh_lane();
      pt = tid - 256;
      cg = pt % CG;
      tg = pt / CG;
      blk = tg / Sh::GPB;
    };
    Vec8<bf16> rq[TPT], rk[TPT], rb[TPT], rg[TPT], gk[TPT];
    // unconditional prefetch loads (see load_vw): clamped rows, zeroed at use
    auto load_g = [&](int c) __attribute__((always_inline)) {
      const int cc = min(c, nchunks - 1) * C;
#pragma unroll
      for (int j = 0; j < TPT; ++j) {
        const int r = min(tg * TPT + j, len - 1 - cc);
        rg[j].r = kload(gb + (long)cc * kstride, (unsigned)(r * (int)kstride + cg * 8));
      }
    };
    // The loads of a chunk are spread over the three phases, so that the vector memory
    // path of the compute unit never holds one phase's worth of every array in flight at
    // once (measured: loads issued as one burst stall on the L1's pending misses): q and b
    // of the next chunk at the starts of phases 1 and 2, k of the chunk after next token by
    // token inside X.c as it frees the registers, g of the chunk after next at the end of
    // phase 1, and the value side (waves 0-3) at the start of phase 1.
    auto key_off = [&](int c, int j, int& cc) __attribute__((always_inline)) {
      cc = min(c, nchunks - 1) * C;
      const int r = min(tg * TPT + j, len - 1 - cc);
      return (unsigned)(r * (int)kstride + cg * 8);
    };
    auto load_q = [&](int c) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < TPT; ++j) {
        int cc;
        const unsigned off = key_off(c, j, cc);
        rq[j].r = kload(qb + (long)cc * kstride, off);
      }
    };
    auto load_b = [&](int c) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < TPT; ++j) {
        int cc;
        const unsigned off = key_off(c, j, cc);
        if constexpr (b_scalar) {
          const int r = min(tg * TPT + j, len - 1 - cc);
          rb[j].load_one(bsb + (long)cc * H + (unsigned)(r * H));
        } else {
          rb[j].r = kload(bb + (long)cc * kstride, off);
        }
      }
    };
    auto load_k_tok = [&](int c, int j) __attribute__((always_inline)) {
      int cc;
      const unsigned off = key_off(c, j, cc);
      rk[j].r = kload(kb + (long)cc * kstride, off);
    };
    // X.a: this thread's decay total into sTot[tg][channel]; the raw decays are kept (gk)
    // for X.c, since rg is refilled with the chunk after next
    auto xa = [&](int nv) __attribute__((always_inline)) {
      float run[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < TPT; ++j) {
        if (tg * TPT + j >= nv) rg[j].zero();  // past the chunk's end: no decay, no input
        float f[8];
        rg[j].to_float(f);
#pragma unroll
        for (int i = 0; i < 8; ++i) run[i] += fmaxf(f[i] * kLog2e, kMinTokenDecay2);
        gk[j] = rg[j];
      }
      store8(sTot + tg * DK + cg * 8, run);
    };
    // X.b: per-channel exclusive scan over the token groups (in place), factor rows, flag
    auto xb = [&](int p) __attribute__((always_inline)) {
      const int ch = pt;  // one thread per channel
      if (ch < DK) {
        float t[Sh::TG];
#pragma unroll
        for (int x = 0; x < Sh::TG; ++x) t[x] = sTot[x * DK + ch];
        float run = 0.f;
        float* fac = sFac(p);
#pragma unroll
        for (int x = 0; x < Sh::TG; ++x) {
          if (x % Sh::GPB == 0) fac[(Sh::F_GS + x / Sh::GPB) * DK + ch] = run;
          sTot[x * DK + ch] = run;
          run += t[x];
        }
        fac[Sh::F_GL * DK + ch] = run;
        fac[Sh::F_GAM * DK + ch] = fast_exp2(run);
        const float gs1 = fac[(Sh::F_GS + 1) * DK + ch], gs2 = fac[(Sh::F_GS + 2) * DK + ch];
        const float gs3 = fac[(Sh::F_GS + 3) * DK + ch];
        fac[(Sh::F_OFF + 0) * DK + ch] = fast_exp2(gs2 - gs1);  // (2, 0)
        fac[(Sh::F_OFF + 1) * DK + ch] = fast_exp2(gs3 - gs1);  // (3, 0)
        fac[(Sh::F_OFF + 2) * DK + ch] = fast_exp2(gs3 - gs2);  // (3, 1)
        if (-run > kFwdFastDecay2) sFlag[p] = 1;
      }
    };
    // X.c: gated operands of the chunk into Eg, Qg[p], Kg[p] (fast: chunk-referenced;
    // general: block-referenced); then the k loads of chunk cn into the freed registers. Tokens
    // past the chunk's end get K = 0 (so E = 0 too): their rows of Kg, Eg, W and U are then
    // zero and add nothing to the state; their Qg rows only reach outputs that are not stored.
    auto xc_impl = [&](int p, int nv, int cn, auto gen_c) __attribute__((always_inline)) {
      constexpr bool GEN = decltype(gen_c)::value;
      const float* fac = sFac(p);
      float run[8], ox[8], oy[8];
      {
        const f4 a = *reinterpret_cast<const f4*>(sTot + tg * DK + cg * 8);
        const f4 b2 = *reinterpret_cast<const f4*>(sTot + tg * DK + cg * 8 + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) { run[i] = a[i]; run[4 + i] = b2[i]; }
      }
      if constexpr (GEN) {
        const int ge = blk < 3 ? Sh::F_GS + blk + 1 : Sh::F_GL;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ox[i] = fac[(Sh::F_GS + blk) * DK + cg * 8 + i];
          oy[i] = fac[ge * DK + cg * 8 + i];
        }
      }
      bf16* qg = sQg(p);
      bf16* kg = sKg(p);
#pragma unroll
      for (int j = 0; j < TPT; ++j) {
        const int r = tg * TPT + j;
        if (nv < C && r >= nv) rk[j].zero();
        if constexpr (b_scalar) rb[j].splat();
        float fg[8];
        gk[j].to_float(fg);
        // one half (4 channels, contiguous in phi order) of the token at a time
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const bf16x8 vq = __builtin_bit_cast(bf16x8, rq[j].r);
          const bf16x8 vk = __builtin_bit_cast(bf16x8, rk[j].r);
          const bf16x8 vb = __builtin_bit_cast(bf16x8, rb[j].r);
          f4 e1, q1, k1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int ci = 4 * hf + i;
            // (on the fast path no token's decay reaches the clamp: the chunk's total is
            // within kFwdFastDecay2)
            run[ci] = GEN ? run[ci] + fmaxf(fg[ci] * kLog2e, kMinTokenDecay2) : fmaf(fg[ci], kLog2e, run[ci]);
            const float G = run[ci];
            const float xe = fast_exp2(GEN ? G - ox[ci] : G);
            const float ye = fast_exp2(GEN ? oy[ci] - G : -G);
            const float fq = static_cast<float>(vq[ci]), fk = static_cast<float>(vk[ci]);
            e1[i] = static_cast<float>(vb[ci]) * fk * xe;
            q1[i] = fq * xe;
            k1[i] = fk * ye;
          }
          const int o = KX(r, Mma<bf16>::phi(cg * 8) + 8 * hf);
          *reinterpret_cast<bf16x4*>(sEg + o) = to_bf4(e1);
          *reinterpret_cast<bf16x4*>(qg + o) = to_bf4(q1);
          *reinterpret_cast<bf16x4*>(kg + o) = to_bf4(k1);
        }
        load_k_tok(cn, j);
      }
    };
    auto xc = [&](int p, int nv, int cn) __attribute__((always_inline)) {
      if (flag(p)) xc_impl(p, nv, cn, std::true_type{});
      else xc_impl(p, nv, cn, std::false_type{});
    };

    if (nchunks > 0) {  // prologue: chunk 0's operands
      load_g(0);
      load_q(0);
      load_b(0);
#pragma unroll
      for (int j = 0; j < TPT; ++j) load_k_tok(0, j);
      if (tid == 256) sFlag[0] = 0;
      xa(nvalid_of(0));
      load_g(1);
      lds_barrier();
      fresh();
      xb(0);
      lds_barrier();
      fresh();
      xc(0, nvalid_of(0), 1);
      lds_barrier();
      fresh();
    }
    for (int c = 0; c < nchunks; ++c) {
      fresh();
      const int p = c & 1, pn = p ^ 1;
      const int c0 = c * C;
      const int nvalid = nvalid_of(c);
      const bool more = c + 1 < nchunks;
      const bool gen = flag(p);
      const int R4 = wave - 4;
      load_q(c + 1);
      // ---- phase 1: three A / P tiles; next totals
      if (!gen) {
        switch (R4) {
          case 0: put_p(3, 3, tile(p, 3, 3, true, false)); put_p(3, 2, tile(p, 3, 2, true, false)); put_off_a(3, 2, tile(p, 3, 2, false, false)); break;
          case 1: put_p(3, 1, tile(p, 3, 1, true, false)); put_p(3, 0, tile(p, 3, 0, true, false)); put_off_a(3, 1, tile(p, 3, 1, false, false)); break;
          case 2: put_p(2, 2, tile(p, 2, 2, true, false)); put_p(2, 1, tile(p, 2, 1, true, false)); put_off_a(3, 0, tile(p, 3, 0, false, false)); break;
          default: put_p(2, 0, tile(p, 2, 0, true, false)); put_off_a(2, 1, tile(p, 2, 1, false, false)); put_off_a(2, 0, tile(p, 2, 0, false, false)); break;
        }
      } else {
        switch (R4) {
          case 0: put_p(2, 0, tile(p, 2, 0, true, true)); put_off_a(2, 0, tile(p, 2, 0, false, true)); break;
          case 1: put_p(1, 0, tile(p, 1, 0, true, true)); put_off_a(1, 0, tile(p, 1, 0, false, true)); break;
          default: break;
        }
        diag_tiles_exact<DK, b_scalar>(qb, kb, gb, bb, bsb, kstride, H, c0, nvalid, tid, sAd, sP);
        lds_barrier();
        fresh();
        rescale(p);
      }
      if (more) {
        if (tid == 256) sFlag[pn] = 0;
        xa(nvalid_of(c + 1));
      }
      load_g(c + 2);
      lds_barrier();
      fresh();
      // ---- phase 2: a key tile; the next chunk's decay scan
      load_b(c + 1);
      {
        f4 X[4];
        column(true, NCT == 8 ? wave : R4, X);
      }
      if (more) xb(pn);
      lds_barrier();
      fresh();
      // ---- phase 3: the next chunk's operands (and the k loads of the chunk after it; issued
      // on the last chunk too, so that every iteration leaves the same loads in flight and
      // the compiler's waits stay exact)
      if (more) {
        xc(pn, nvalid_of(c + 1), c + 2);
      } else {
#pragma unroll
        for (int j = 0; j < TPT; ++j) load_k_tok(c + 2, j);
      }
      lds_barrier();
      fresh();
    }
  }
}

template <int DK>
static hipError_t launch_fwd(const ChunkArgs& a) {
  const int nslices = a.d_v / 64;
  const long grid = (long)a.N * a.H * nslices;
  auto kern = a.gate_flags == 3 ? gdn2_fwd_kernel<DK, 3>
              : a.gate_flags == 2 ? gdn2_fwd_kernel<DK, 2>
              : a.gate_flags == 1 ? gdn2_fwd_kernel<DK, 1>
                                  : gdn2_fwd_kernel<DK, 0>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), 0, (hipStream_t)a.stream,
                     (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.g,
                     (const bf16*)a.b, (const bf16*)a.w, a.s0, (bf16*)a.o, a.sN, a.cu_seqlens,
                     a.T, a.H, a.d_v, nslices, a.N * a.H);
  return hipGetLastError();
}

bool fwd_pipelined_supported(int dtype, int d_k, int d_v) {
  return dtype == 0 && (d_k == 64 || d_k == 128) && (d_v == 64 || d_v == 128);
}

hipError_t launch_fwd_pipelined(const ChunkArgs& a) {
  if (!fwd_pipelined_supported(a.dtype, a.d_k, a.d_v)) return hipErrorInvalidValue;
  return a.d_k == 128 ? launch_fwd<128>(a) : launch_fwd<64>(a);
}

}  // namespace gdn2
