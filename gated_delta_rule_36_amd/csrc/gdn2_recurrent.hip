// Token-recurrent forward of Gated Delta Rule-2 for fp32 runs with d_k = 128.
//
// The chunk kernels keep a chunk's gated operands in LDS; in fp32 with d_k = 128 those
// operands (E, Q, K and the transposed copies, 64 tokens each) exceed the 160 KB of LDS, so
// this width walks the tokens one by one instead: the per-token procedure of the GDN-2 reading
// note (§3, forward pass; erase along k, see the C header) on an fp32 state slice held in
// registers, exactly as the decode step computes a token:
//   S_bar = Diag(alpha) S,  r = S_bar^T e,  S' = S_bar + k (z - r)^T,
//   o = S'^T q = S_bar^T q + (q . k)(z - r).
// One 256-thread workgroup per (sequence, head, 64 value columns): a thread owns 4 columns of
// d_k / 16 consecutive key rows. Tokens come in blocks of 16: a block's inputs are loaded
// into registers one block ahead, then turned into alpha, e = b*k, q, k, z = w*v and q . k in
// LDS (double-buffered by block parity), so a token step reads LDS only and costs one
// barrier (the partial sums of r and S_bar^T q over the 16 row groups, double-buffered by
// token parity).

#include "gdn2_device.h"
#include "gdn2_launch.h"

namespace gdn2 {

namespace {

template <int DK>
struct RecShape {
  static constexpr int NT = 256;
  static constexpr int NV = 64;           // value columns per workgroup
  static constexpr int CG = NV / 4;       // 16 column groups of 4
  static constexpr int RG = NT / CG;      // 16 row groups
  static constexpr int RPT = DK / RG;     // consecutive key rows per thread
  static constexpr int TB = 16;           // tokens per block
  static constexpr int KL = TB * DK / 4 / NT;  // float4 loads per thread per key-side array
  static_assert(RPT % 4 == 0 && KL >= 1 && TB * NV / 4 == NT, "thread mapping");
};

}  // namespace

template <int DK, int GL>
__global__ void __launch_bounds__(256)
gdn2_recurrent_fwd_kernel(const float* __restrict__ q, const float* __restrict__ k,
                          const float* __restrict__ v, const float* __restrict__ g,
                          const float* __restrict__ bg, const float* __restrict__ wg,
                          const float* s0, float* __restrict__ o, float* sN,
                          const int* __restrict__ cu_seqlens, int T_len, int H, int DV) {
  using Sh = RecShape<DK>;
  constexpr int NT = Sh::NT, NV = Sh::NV, CG = Sh::CG, RG = Sh::RG, RPT = Sh::RPT, TB = Sh::TB;
  constexpr int KL = Sh::KL;
  constexpr bool b_scalar = (GL & kGateBScalar) != 0;
  constexpr bool w_scalar = (GL & kGateWScalar) != 0;
  __shared__ __attribute__((aligned(16))) float s_a[2][TB][DK], s_e[2][TB][DK], s_q[2][TB][DK],
      s_k[2][TB][DK], s_z[2][TB][NV];
  __shared__ float s_qk[2][TB];
  __shared__ __attribute__((aligned(16))) float s_red[2][2][RG][NV];

  const int tid = threadIdx.x;
  const int nslices = DV / NV;
  const int slice = blockIdx.x % nslices;
  const int nh = blockIdx.x / nslices;
  const int h = nh % H, n = nh / H;
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
  const long kstride = (long)H * DK, vstride = (long)H * DV;
  const int col0 = slice * NV;
  const int cg = tid % CG, rg = tid / CG;

  // state: rows rg * RPT + j, columns col0 + 4 cg ..
  f4 s[RPT];
  const long sbase = ((long)n * H + h) * DK * DV + col0 + 4 * cg;
#pragma unroll
  for (int j = 0; j < RPT; ++j)
    s[j] = s0 != nullptr ? *reinterpret_cast<const f4*>(s0 + sbase + (long)(rg * RPT + j) * DV)
                         : f4{0.f, 0.f, 0.f, 0.f};

  // block loads: key side, element (token t, channel 4c..) at index i = tid + NT x; value
  // side, (token tid / CG, columns 4 (tid % CG)..)
  f4 lq[KL], lk[KL], lg[KL], lb[KL], lv, lw;
  auto load_block = [&](int blk) {
    const int t0 = blk * TB;
#pragma unroll
    for (int x = 0; x < KL; ++x) {
      const int i = tid + NT * x, t = i / (DK / 4), c4 = i % (DK / 4);
      const bool ok = t0 + t < len;
      const long off = (row0 + t0 + t) * kstride + (long)h * DK + 4 * c4;
      const f4 z4 = {0.f, 0.f, 0.f, 0.f};
      lq[x] = ok ? *reinterpret_cast<const f4*>(q + off) : z4;
      lk[x] = ok ? *reinterpret_cast<const f4*>(k + off) : z4;
      lg[x] = ok ? *reinterpret_cast<const f4*>(g + off) : z4;
      if constexpr (b_scalar) {
        const float bs = ok ? bg[(row0 + t0 + t) * H + h] : 0.f;
        lb[x] = f4{bs, bs, bs, bs};
      } else {
        lb[x] = ok ? *reinterpret_cast<const f4*>(bg + off) : z4;
      }
    }
    const int t = tid / CG, c4 = tid % CG;
    const bool ok = t0 + t < len;
    const long voff = (row0 + t0 + t) * vstride + (long)h * DV + col0 + 4 * c4;
    const f4 z4 = {0.f, 0.f, 0.f, 0.f};
    lv = ok ? *reinterpret_cast<const f4*>(v + voff) : z4;
    if constexpr (w_scalar) {
      const float ws = ok ? wg[(row0 + t0 + t) * H + h] : 0.f;
      lw = f4{ws, ws, ws, ws};
    } else {
      lw = ok ? *reinterpret_cast<const f4*>(wg + voff) : z4;
    }
  };
  auto store_block = [&](int par) {
#pragma unroll
    for (int x = 0; x < KL; ++x) {
      const int i = tid + NT * x, t = i / (DK / 4), c = 4 * (i % (DK / 4));
      f4 a;
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = __expf(lg[x][e]);
      *reinterpret_cast<f4*>(&s_a[par][t][c]) = a;
      *reinterpret_cast<f4*>(&s_e[par][t][c]) = lb[x] * lk[x];
      *reinterpret_cast<f4*>(&s_q[par][t][c]) = lq[x];
      *reinterpret_cast<f4*>(&s_k[par][t][c]) = lk[x];
    }
    *reinterpret_cast<f4*>(&s_z[par][tid / CG][4 * (tid % CG)]) = lw * lv;
  };

  const int nblocks = (len + TB - 1) / TB;
  if (nblocks > 0) load_block(0);
  int tpar = 0;
  for (int blk = 0; blk < nblocks; ++blk) {
    const int bpar = blk & 1;
    store_block(bpar);
    if (blk + 1 < nblocks) load_block(blk + 1);
    __syncthreads();
    {  // q . k of the block's tokens: 16 lanes per token
      const int t = tid / 16, part = tid % 16;
      float p = 0.f;
#pragma unroll
      for (int c = part; c < DK; c += 16) p += s_q[bpar][t][c] * s_k[bpar][t][c];
#pragma unroll
      for (int m = 8; m > 0; m >>= 1) p += __shfl_xor(p, m, 16);
      if (part == 0) s_qk[bpar][t] = p;
    }
    __syncthreads();
    const int nt = min(TB, len - blk * TB);
    for (int t = 0; t < nt; ++t) {
      f4 r = {0.f, 0.f, 0.f, 0.f}, sq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j4 = 0; j4 < RPT; j4 += 4) {
        const int row = rg * RPT + j4;
        const f4 a = *reinterpret_cast<const f4*>(&s_a[bpar][t][row]);
        const f4 e = *reinterpret_cast<const f4*>(&s_e[bpar][t][row]);
        const f4 qq = *reinterpret_cast<const f4*>(&s_q[bpar][t][row]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          s[j4 + u] = s[j4 + u] * a[u];  // S_bar
          r += e[u] * s[j4 + u];
          sq += qq[u] * s[j4 + u];
        }
      }
      *reinterpret_cast<f4*>(&s_red[tpar][0][rg][4 * cg]) = r;
      *reinterpret_cast<f4*>(&s_red[tpar][1][rg][4 * cg]) = sq;
      __syncthreads();
      r = f4{0.f, 0.f, 0.f, 0.f};
      sq = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int x = 0; x < RG; ++x) {
        r += *reinterpret_cast<const f4*>(&s_red[tpar][0][x][4 * cg]);
        sq += *reinterpret_cast<const f4*>(&s_red[tpar][1][x][4 * cg]);
      }
      const f4 d = *reinterpret_cast<const f4*>(&s_z[bpar][t][4 * cg]) - r;  // z minus the erased read
      if (rg == 0)
        *reinterpret_cast<f4*>(o + (row0 + blk * TB + t) * vstride + (long)h * DV + col0 + 4 * cg) =
            sq + s_qk[bpar][t] * d;
#pragma unroll
      for (int j4 = 0; j4 < RPT; j4 += 4) {
        const f4 kk = *reinterpret_cast<const f4*>(&s_k[bpar][t][rg * RPT + j4]);
#pragma unroll
        for (int u = 0; u < 4; ++u) s[j4 + u] = s[j4 + u] + kk[u] * d;
      }
      tpar ^= 1;
    }
  }
  if (sN != nullptr) {
#pragma unroll
    for (int j = 0; j < RPT; ++j)
      *reinterpret_cast<f4*>(sN + sbase + (long)(rg * RPT + j) * DV) = s[j];
  }
}

template <int DK>
static hipError_t launch_rec(const ChunkArgs& a) {
  const long grid = (long)a.N * a.H * (a.d_v / RecShape<DK>::NV);
  auto kern = a.gate_flags == 3 ? gdn2_recurrent_fwd_kernel<DK, 3>
              : a.gate_flags == 2 ? gdn2_recurrent_fwd_kernel<DK, 2>
              : a.gate_flags == 1 ? gdn2_recurrent_fwd_kernel<DK, 1>
                                  : gdn2_recurrent_fwd_kernel<DK, 0>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)a.stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (const float*)a.g,
                     (const float*)a.b, (const float*)a.w, a.s0, (float*)a.o, a.sN, a.cu_seqlens,
                     a.T, a.H, a.d_v);
  return hipGetLastError();
}

bool fwd_recurrent_used(int dtype, int d_k, int d_v) {
  return dtype == 1 && d_k == 128 && (d_v == 64 || d_v == 128);
}

hipError_t launch_fwd_recurrent(const ChunkArgs& a) {
  if (!fwd_recurrent_used(a.dtype, a.d_k, a.d_v)) return hipErrorInvalidValue;
  return launch_rec<128>(a);
}

}  // namespace gdn2
