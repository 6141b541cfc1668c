// Single-token recurrent decode step of Gated Delta Rule-2 on gfx950.
//
// Per (sequence, head) the step is the token recurrence of the GDN-2 reading note's §3
// forward-pass paragraph (erase along k, see the C header):
//   S_bar = Diag(alpha) S,  r = S_bar^T e,  S' = S_bar + k (z - r)^T,  o = S'^T q.
// The readout is formed from the old state in the same pass as r:
//   o = S_bar^T q + (q . k)(z - r)
// so the 64 KB fp32 state is streamed from HBM once and written back once; everything
// else (six d-vectors of inputs, one d_v output) is negligible traffic. The kernel is
// bandwidth-bound: one workgroup of 256 threads per (sequence, head), the state slice is
// held in registers between the read and the write, float4 accesses make every wave
// touch whole contiguous rows, and the state is streamed with non-temporal loads and
// stores (read once and written once per step, it would only evict other data from the
// caches).

#include "gdn2_device.h"
#include "gdn2_launch.h"

namespace gdn2 {

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
// few tokens at once, or verification of draft tokens). The state of pool slot
// indices[n] is read once, advanced through the L tokens in registers, and, after token
// commit[n] - 1, written back to its slot (commit 0: the pool is left alone); with
// step_states every intermediate state is also written out. Same per-token arithmetic as
// gdn2_decode_kernel; the token inputs are double-buffered in LDS by token parity, so a
// token costs two barriers.
template <typename T, int DK, int DV>
__global__ void __launch_bounds__(256)
gdn2_decode_tokens_kernel(const T* __restrict__ q, const T* __restrict__ k,
                          const T* __restrict__ v, const T* __restrict__ g,
                          const T* __restrict__ bg, const T* __restrict__ wg,
                          float* __restrict__ pool, const int* __restrict__ indices,
                          const int* __restrict__ commit, T* __restrict__ o,
                          float* __restrict__ step_states, int L, int H, int P, int gflags) {
  constexpr int NT = 256;
  constexpr int CG = DV / 4;
  constexpr int RG = NT / CG;
  constexpr int RPT = DK / RG;
  __shared__ float s_alpha[2][DK], s_e[2][DK], s_q[2][DK], s_k[2][DK], s_z[2][DV];
  __shared__ __attribute__((aligned(16))) float s_red[2][2][RG][DV];
  __shared__ float s_qk[2];

  const int tid = threadIdx.x;
  const int n = blockIdx.x / H, h = blockIdx.x % H;
  const int slot = indices != nullptr ? indices[n] : n;
  if (slot < 0 || slot >= P) return;  // no state for this sequence (uniform)
  int ncommit = commit != nullptr ? commit[n] : L;
  ncommit = ncommit < 0 ? 0 : (ncommit > L ? L : ncommit);
  const int cg = tid % CG, rg = tid / CG;
  float* S = pool + ((long)slot * H + h) * DK * DV;

  f4 s[RPT];
#pragma unroll
  for (int j = 0; j < RPT; ++j)
    s[j] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(S + (long)(rg + j * RG) * DV + 4 * cg));

  for (int t = 0; t < L; ++t) {
    const int par = t & 1;
    const long tk = (((long)n * L + t) * H + h);  // token row of [N, L, H, d]
    for (int c = tid; c < DK; c += NT) {
      const float kk = to_f(k[tk * DK + c]);
      s_alpha[par][c] = __expf(to_f(g[tk * DK + c]));
      s_e[par][c] = to_f(bg[(gflags & kGateBScalar) ? tk : tk * DK + c]) * kk;
      s_q[par][c] = to_f(q[tk * DK + c]);
      s_k[par][c] = kk;
    }
    for (int c = tid; c < DV; c += NT)
      s_z[par][c] = to_f(wg[(gflags & kGateWScalar) ? tk : tk * DV + c]) * to_f(v[tk * DV + c]);
    __syncthreads();
    if (tid < 64) {
      float p = 0.f;
      for (int c = tid; c < DK; c += 64) p += s_q[par][c] * s_k[par][c];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off, 64);
      if (tid == 0) s_qk[par] = p;
    }
    f4 r = {0.f, 0.f, 0.f, 0.f}, sq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int c = rg + j * RG;
      s[j] = s[j] * s_alpha[par][c];
      r += s_e[par][c] * s[j];
      sq += s_q[par][c] * s[j];
    }
    *reinterpret_cast<f4*>(&s_red[par][0][rg][4 * cg]) = r;
    *reinterpret_cast<f4*>(&s_red[par][1][rg][4 * cg]) = sq;
    __syncthreads();
    r = f4{0.f, 0.f, 0.f, 0.f};
    sq = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int x = 0; x < RG; ++x) {
      r += *reinterpret_cast<const f4*>(&s_red[par][0][x][4 * cg]);
      sq += *reinterpret_cast<const f4*>(&s_red[par][1][x][4 * cg]);
    }
    const f4 d = *reinterpret_cast<const f4*>(&s_z[par][4 * cg]) - r;
    if (rg == 0) {
      const f4 out = sq + s_qk[par] * d;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[tk * DV + 4 * cg + i] = from_f<T>(out[i]);
    }
#pragma unroll
    for (int j = 0; j < RPT; ++j) s[j] = s[j] + s_k[par][rg + j * RG] * d;
    if (step_states != nullptr) {
      float* St = step_states + tk * DK * DV;
#pragma unroll
      for (int j = 0; j < RPT; ++j)
        __builtin_nontemporal_store(s[j], reinterpret_cast<f4*>(St + (long)(rg + j * RG) * DV + 4 * cg));
    }
    if (t + 1 == ncommit) {
#pragma unroll
      for (int j = 0; j < RPT; ++j) *reinterpret_cast<f4*>(S + (long)(rg + j * RG) * DV + 4 * cg) = s[j];
    }
  }
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
