// Recurrent decode of Gated Delta Rule-2 on gfx950: one token per call, or L consecutive
// tokens per call against a pool of states.
//
// Per (sequence, head) a token is the recurrence of the GDN-2 reading note's §3
// forward-pass paragraph (erase along k, see the C header):
//   S_bar = Diag(alpha) S,  r = S_bar^T e,  S' = S_bar + k (z - r)^T,  o = S'^T q.
// The readout is formed from the old state in the same pass as r:
//   o = S_bar^T q + (q . k)(z - r)
// so the 64 KB fp32 state is streamed from HBM once and written back once per call;
// everything else (six d-vectors of inputs per token, one d_v output) is negligible
// traffic. The kernels are bandwidth-bound: one workgroup of 256 threads per (sequence,
// head), the state held in registers between the read and the write, and streamed with
// non-temporal loads and stores (read once and written once, it would only evict other
// data from the caches).
//
// Multi-token layout: wave w owns value columns [w d_v / 4, (w + 1) d_v / 4), every key row
// of them; lane l holds 4 columns (column group l / RG) of d_k / RG consecutive rows (row
// group l % RG, RG = 8 for d_v = 128, 16 for d_v = 64). The sums over key rows (r and S_bar^T q)
// run over the RG low lanes of a wave by DPP steps, in registers, so no token needs a
// barrier: each wave stages the token's alpha, e, q, k in LDS of its own (written and read
// by the same wave) and loads the next token's inputs while it computes this one.

#include "gdn2_device.h"
#include "gdn2_launch.h"

namespace gdn2 {

namespace {

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Sum over each group of RG (8 or 16) consecutive lanes, in every lane of the group: lane ^ 1
// and lane ^ 2 by quad permutations, then the mirrored half of the 8-lane half-row, then (RG
// = 16) the mirrored half of the 16-lane row.
template <int RG>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);  // row_half_mirror
  if constexpr (RG == 16) x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}

}  // namespace

// L tokens of one (sequence, head): the state of pool slot indices[n] (slot n without an
// index table) is read, advanced through the tokens, and written back after token
// commit[n] - 1 (commit 0: the pool is left alone; no table: after the last token); with
// step_states every intermediate state is also written out. Returns at once for a slot
// outside [0, P).
template <typename T, int DK, int DV>
__device__ __forceinline__ void decode_tokens(const T* __restrict__ q, const T* __restrict__ k,
                                              const T* __restrict__ v, const T* __restrict__ g,
                                              const T* __restrict__ bg, const T* __restrict__ wg,
                                              float* __restrict__ pool, const int* indices,
                                              const int* commit, T* __restrict__ o,
                                              float* step_states, int L, int H, int P, int gflags) {
  constexpr int CGW = DV / 16;   // 4-column groups per wave
  constexpr int RG = 64 / CGW;   // row groups per wave: the low lane bits
  constexpr int RPL = DK / RG;   // consecutive key rows per lane
  constexpr int EPL = DK / 64;   // key-side channels per lane when a wave stages a token
  static_assert(RPL % 4 == 0 && (RG == 8 || RG == 16) && EPL >= 1, "lane mapping");
  __shared__ __attribute__((aligned(16))) float s_in[4][4][DK];  // [wave][alpha, e, q, k][row]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = blockIdx.x / H, h = blockIdx.x % H;
  const int slot = indices != nullptr ? indices[n] : n;
  if (slot < 0 || slot >= P) return;  // no state for this sequence (uniform)
  int ncommit = commit != nullptr ? commit[n] : L;
  ncommit = ncommit < 0 ? 0 : (ncommit > L ? L : ncommit);
  const int col0 = wave * (DV / 4) + 4 * (lane / RG);
  const int row0 = (lane % RG) * RPL;
  float* S = pool + ((long)slot * H + h) * DK * DV;

  f4 s[RPL];
#pragma unroll
  for (int j = 0; j < RPL; ++j)
    s[j] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(S + (long)(row0 + j) * DV + col0));

  // a token's inputs in registers, loaded one token ahead: EPL channels of each key-side
  // array (lane * EPL ..) and the lane's 4 value columns
  T xk[EPL], xg[EPL], xb[EPL], xq[EPL], xv[4], xw[4];
  auto load_tok = [&](int t) {
    if (t >= L) return;
    const long tk = ((long)n * L + t) * H + h;  // token row of [N, L, H, d]
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int c = lane * EPL + e;
      xk[e] = k[tk * DK + c];
      xg[e] = g[tk * DK + c];
      xb[e] = bg[(gflags & kGateBScalar) ? tk : tk * DK + c];
      xq[e] = q[tk * DK + c];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xv[i] = v[tk * DV + col0 + i];
      xw[i] = wg[(gflags & kGateWScalar) ? tk : tk * DV + col0 + i];
    }
  };
  load_tok(0);
  float* const sa = s_in[wave][0];
  float* const se = s_in[wave][1];
  float* const sq = s_in[wave][2];
  float* const sk = s_in[wave][3];
  for (int t = 0; t < L; ++t) {
    const long tk = ((long)n * L + t) * H + h;
    // stage alpha, e = b k, q, k in this wave's LDS (the previous token's reads of it, by the
    // same wave, are complete: a wave's LDS accesses are in order)
    float qk = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int c = lane * EPL + e;
      const float kk = to_f(xk[e]), qq = to_f(xq[e]);
      sa[c] = __expf(to_f(xg[e]));
      se[c] = to_f(xb[e]) * kk;
      sq[c] = qq;
      sk[c] = kk;
      qk += qq * kk;
    }
    f4 z;
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = to_f(xw[i]) * to_f(xv[i]);
    load_tok(t + 1);
    // q . k over the wave: the 16-lane rows, then the four row sums
    qk = group_sum<16>(qk);
    qk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, qk), 0)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, qk), 16)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, qk), 32)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, qk), 48));
    // S_bar, and this lane's part of r = S_bar^T e and S_bar^T q
    f4 r = {0.f, 0.f, 0.f, 0.f}, sbq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j4 = 0; j4 < RPL; j4 += 4) {
      const f4 a = *reinterpret_cast<const f4*>(sa + row0 + j4);
      const f4 e = *reinterpret_cast<const f4*>(se + row0 + j4);
      const f4 qv = *reinterpret_cast<const f4*>(sq + row0 + j4);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s[j4 + u] = s[j4 + u] * a[u];
        r += e[u] * s[j4 + u];
        sbq += qv[u] * s[j4 + u];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[i] = group_sum<RG>(r[i]);
      sbq[i] = group_sum<RG>(sbq[i]);
    }
    const f4 d = z - r;  // what k writes: z minus the erased read
    if (lane % RG == 0) {
      const f4 out = sbq + qk * d;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[tk * DV + col0 + i] = from_f<T>(out[i]);
    }
#pragma unroll
    for (int j4 = 0; j4 < RPL; j4 += 4) {
      const f4 kk = *reinterpret_cast<const f4*>(sk + row0 + j4);
#pragma unroll
      for (int u = 0; u < 4; ++u) s[j4 + u] = s[j4 + u] + kk[u] * d;
    }
    if (step_states != nullptr) {
      float* St = step_states + tk * DK * DV;
#pragma unroll
      for (int j = 0; j < RPL; ++j)
        __builtin_nontemporal_store(s[j], reinterpret_cast<f4*>(St + (long)(row0 + j) * DV + col0));
    }
    if (t + 1 == ncommit) {
#pragma unroll
      for (int j = 0; j < RPL; ++j)
        __builtin_nontemporal_store(s[j], reinterpret_cast<f4*>(S + (long)(row0 + j) * DV + col0));
    }
  }
}

// One token per (sequence, head), state n of [N, H, d_k, d_v] updated in place. A layout of
// its own: thread (row group rg, column group cg) holds 4 columns of the rows rg + 8 j, so a
// wave reads whole 512-byte rows; the sums over rows go through LDS (two barriers). As a
// pure stream this measured faster than the multi-token kernel's layout specialised to one
// token (92.8 against 98.1 us per step on the decode workload, same box and process).
template <typename T, int DK, int DV>
__global__ void __launch_bounds__(256)
gdn2_decode_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                   const T* __restrict__ g, const T* __restrict__ bg, const T* __restrict__ wg,
                   float* __restrict__ state, T* __restrict__ o, int gflags) {
  constexpr int NT = 256;
  constexpr int CG = DV / 4;        // float4 column groups per row
  constexpr int RG = NT / CG;       // row groups
  constexpr int RPT = DK / RG;      // rows per thread
  __shared__ float s_alpha[DK], s_e[DK], s_q[DK], s_k[DK], s_z[DV];
  __shared__ __attribute__((aligned(16))) float s_red[2][RG][DV];
  __shared__ float s_qk;

  const int tid = threadIdx.x;
  const long unit = blockIdx.x;  // sequence * H + head
  const int cg = tid % CG, rg = tid / CG;
  float* S = state + unit * DK * DV;

  // issue the state loads first: they are the whole cost of the step
  f4 s[RPT];
#pragma unroll
  for (int j = 0; j < RPT; ++j)
    s[j] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(S + (long)(rg + j * RG) * DV + 4 * cg));

  for (int c = tid; c < DK; c += NT) {
    const float kk = to_f(k[unit * DK + c]);
    s_alpha[c] = __expf(to_f(g[unit * DK + c]));
    s_e[c] = to_f(bg[(gflags & kGateBScalar) ? unit : unit * DK + c]) * kk;
    s_q[c] = to_f(q[unit * DK + c]);
    s_k[c] = kk;
  }
  for (int c = tid; c < DV; c += NT)
    s_z[c] = to_f(wg[(gflags & kGateWScalar) ? unit : unit * DV + c]) * to_f(v[unit * DV + c]);
  __syncthreads();

  if (tid < 64) {  // q . k by wave 0
    float p = 0.f;
    for (int c = tid; c < DK; c += 64) p += s_q[c] * s_k[c];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off, 64);
    if (tid == 0) s_qk = p;
  }

  f4 r = {0.f, 0.f, 0.f, 0.f}, sq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int c = rg + j * RG;
    s[j] = s[j] * s_alpha[c];  // S_bar
    r += s_e[c] * s[j];
    sq += s_q[c] * s[j];
  }
  *reinterpret_cast<f4*>(&s_red[0][rg][4 * cg]) = r;
  *reinterpret_cast<f4*>(&s_red[1][rg][4 * cg]) = sq;
  __syncthreads();

  r = f4{0.f, 0.f, 0.f, 0.f};
  sq = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int x = 0; x < RG; ++x) {
    r += *reinterpret_cast<const f4*>(&s_red[0][x][4 * cg]);
    sq += *reinterpret_cast<const f4*>(&s_red[1][x][4 * cg]);
  }
  const f4 z = *reinterpret_cast<const f4*>(&s_z[4 * cg]);
  const f4 d = z - r;  // what k writes: z minus the erased read
  if (rg == 0) {
    const f4 out = sq + s_qk * d;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[unit * DV + 4 * cg + i] = from_f<T>(out[i]);
  }
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int c = rg + j * RG;
    __builtin_nontemporal_store(s[j] + s_k[c] * d, reinterpret_cast<f4*>(S + (long)c * DV + 4 * cg));
  }
}

// L consecutive tokens per (sequence, head) against a pool of states (serving: decode of a
// few tokens at once, or verification of draft tokens).
template <typename T, int DK, int DV>
__global__ void __launch_bounds__(256)
gdn2_decode_tokens_kernel(const T* __restrict__ q, const T* __restrict__ k,
                          const T* __restrict__ v, const T* __restrict__ g,
                          const T* __restrict__ bg, const T* __restrict__ wg,
                          float* __restrict__ pool, const int* __restrict__ indices,
                          const int* __restrict__ commit, T* __restrict__ o,
                          float* __restrict__ step_states, int L, int H, int P, int gflags) {
  decode_tokens<T, DK, DV>(q, k, v, g, bg, wg, pool, indices, commit, o, step_states, L, H, P,
                           gflags);
}

template <typename T, int DK, int DV>
static hipError_t launch_dec(const DecodeArgs& a) {
  hipLaunchKernelGGL((gdn2_decode_kernel<T, DK, DV>), dim3((unsigned)((long)a.N * a.H)), dim3(256),
                     0, (hipStream_t)a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v,
                     (const T*)a.g, (const T*)a.b, (const T*)a.w, a.state, (T*)a.o, a.gate_flags);
  return hipGetLastError();
}

template <typename T>
static hipError_t dispatch_dec(const DecodeArgs& a) {
  if (a.d_k == 64 && a.d_v == 64) return launch_dec<T, 64, 64>(a);
  if (a.d_k == 64 && a.d_v == 128) return launch_dec<T, 64, 128>(a);
  if (a.d_k == 128 && a.d_v == 64) return launch_dec<T, 128, 64>(a);
  if (a.d_k == 128 && a.d_v == 128) return launch_dec<T, 128, 128>(a);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_step(const DecodeArgs& a) {
  return a.dtype == 0 ? dispatch_dec<bf16>(a) : dispatch_dec<float>(a);
}

template <typename T, int DK, int DV>
static hipError_t launch_dec_tokens(const DecodeTokensArgs& a) {
  hipLaunchKernelGGL((gdn2_decode_tokens_kernel<T, DK, DV>), dim3((unsigned)((long)a.N * a.H)),
                     dim3(256), 0, (hipStream_t)a.stream, (const T*)a.q, (const T*)a.k,
                     (const T*)a.v, (const T*)a.g, (const T*)a.b, (const T*)a.w, a.pool,
                     a.indices, a.commit, (T*)a.o, a.step_states, a.L, a.H, a.P, a.gate_flags);
  return hipGetLastError();
}

template <typename T>
static hipError_t dispatch_dec_tokens(const DecodeTokensArgs& a) {
  if (a.d_k == 64 && a.d_v == 64) return launch_dec_tokens<T, 64, 64>(a);
  if (a.d_k == 64 && a.d_v == 128) return launch_dec_tokens<T, 64, 128>(a);
  if (a.d_k == 128 && a.d_v == 64) return launch_dec_tokens<T, 128, 64>(a);
  if (a.d_k == 128 && a.d_v == 128) return launch_dec_tokens<T, 128, 128>(a);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_tokens(const DecodeTokensArgs& a) {
  return a.dtype == 0 ? dispatch_dec_tokens<bf16>(a) : dispatch_dec_tokens<float>(a);
}

}  // namespace gdn2
