// Prologue and epilogue of the GDN-2 block around the token mixer, on gfx950.
//
// The block data flow of the GDN-2 reading note (§3, block paragraph): q and k are
// conv -> SiLU -> L2 norm of their projections, v is conv -> SiLU, the decay, erase and
// write gates come from projections of their own, and the mixer output is scaled by an
// RMSNorm with a SiLU gate. The projections themselves are plain GEMMs (not here).
//   conv : causal depthwise, width 4, per sequence (y[t] = sum_j W[c, j] x[t - 3 + j])
//   q, k : l2norm(silu(conv(x)))        over d_k, eps 1e-6
//   v    : silu(conv(x))
//   g    : -scale[c] * softplus(x)      (log alpha)
//   b    : b_max * sigmoid(x),  w : sigmoid(x)
//   y    : o / sqrt(mean(o^2) + 1e-6) * weight[c] * silu(gate)
// Both kernels are elementwise with one reduction per (token, head) row: 16-byte accesses,
// a row of d channels on d/8 consecutive lanes, the reduction by lane shuffles. They are
// HBM-bound: the prologue reads each projection once (plus L2-served conv history) and
// writes each mixer input once; the epilogue reads o and the gate and writes y.

#include "gdn2_device.h"
#include "gdn2_block_launch.h"

namespace gdn2 {

constexpr int kConvWidth = 4;
constexpr float kNormEps = 1e-6f;

// Activations on the hardware exp2 / log2 / reciprocal (about 1 ulp each); both kernels do a
// few of these per element, so full-precision library calls would make them ALU-bound.
__device__ __forceinline__ float sigmoid_f(float x) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-x));  // exp overflow gives rcp(inf) = 0
}
// softplus(x) = max(x, 0) + log(1 + e), e = exp(-|x|) in (0, 1]; log(1 + e) through
// log(u) * e / (u - 1) with u = fl(1 + e), which keeps full relative accuracy for tiny e
// (Goldberg, "What every computer scientist should know about floating-point arithmetic").
__device__ __forceinline__ float softplus_f(float x) {
  const float e = __expf(-fabsf(x));
  const float u = 1.f + e;
  const float lp = u == 1.f ? e : __logf(u) * e * __builtin_amdgcn_rcpf(u - 1.f);
  return fmaxf(x, 0.f) + lp;
}

// Outputs are written once and never read back by these kernels: non-temporal stores.
template <typename T>
__device__ __forceinline__ void store8_t(T* p, const float* f);
template <>
__device__ __forceinline__ void store8_t<bf16>(bf16* p, const float* f) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = static_cast<bf16>(f[i]);
  __builtin_nontemporal_store(v, reinterpret_cast<bf16x8*>(p));
}
template <>
__device__ __forceinline__ void store8_t<float>(float* p, const float* f) {
  __builtin_nontemporal_store(f4{f[0], f[1], f[2], f[3]}, reinterpret_cast<f4*>(p));
  __builtin_nontemporal_store(f4{f[4], f[5], f[6], f[7]}, reinterpret_cast<f4*>(p) + 1);
}

// 8 consecutive channels in the storage dtype, as ext-vector registers (arrays of these stay
// in VGPRs once the loops that index them are unrolled).
template <typename T> struct Raw8;
template <> struct Raw8<bf16> {
  static constexpr int P = 1;  // 16-byte pieces per 8 channels
  typedef bf16x8 piece;
  __device__ static float get(const piece* v, int c) { return static_cast<float>(v[0][c]); }
};
template <> struct Raw8<float> {
  static constexpr int P = 2;
  typedef f4 piece;
  __device__ static float get(const piece* v, int c) { return v[c >> 2][c & 3]; }
};

// Tokens per lane in the prologue: a lane walks R consecutive tokens of one (head, 8-channel
// group), so each projection element is read once (plus 3 history tokens per run) and the
// conv taps and decay scales are loaded once per run.
template <typename T> constexpr int prologue_run() { return 8; }

// blockIdx.y = branch: 0 q, 1 k, 2 v, 3 g, 4 b, 5 w. A "row" is one (run of R tokens, head);
// the D/8 lanes of a row hold its channel groups, so a row's L2 norm is a shuffle reduction
// and the rows of a wave at one token step are adjacent heads (contiguous in memory).
template <typename T, int DK, int DV>
__global__ void __launch_bounds__(256)
gdn2_prologue_kernel(const T* __restrict__ xq, const T* __restrict__ xk,
                     const T* __restrict__ xv, const T* __restrict__ xg,
                     const T* __restrict__ xb, const T* __restrict__ xw,
                     const float* __restrict__ wq, const float* __restrict__ wk,
                     const float* __restrict__ wv, const float* __restrict__ scale, float b_max,
                     T* __restrict__ q, T* __restrict__ k, T* __restrict__ v,
                     T* __restrict__ g, T* __restrict__ b, T* __restrict__ w,
                     const int* __restrict__ cu_seqlens, int N, int T_len, int H, long tokens) {
  constexpr int R = prologue_run<T>();
  constexpr int HIST = kConvWidth - 1;
  typedef Raw8<T> RW;
  typedef typename RW::piece piece;
  const int br = blockIdx.y;
  const bool conv = br <= 2;
  const int D = (br == 2 || br == 5) ? DV : DK;  // uniform per block
  const int TPR = D / 8;                          // lanes per row
  const long rows = (tokens + R - 1) / R * H;
  if ((long)blockIdx.x * (256 / TPR) >= rows) return;  // whole block past the end (narrow branch)
  const long r = (long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const bool live = r < rows;
  const long t0 = live ? r / H * R : 0;
  const int h = (int)(live ? r % H : 0);
  const int c0 = (threadIdx.x % TPR) * 8;
  const long stride = (long)H * D;  // elements from one token to the next
  const T* x = br == 0 ? xq : br == 1 ? xk : br == 2 ? xv : br == 3 ? xg : br == 4 ? xb : xw;
  T* y = br == 0 ? q : br == 1 ? k : br == 2 ? v : br == 3 ? g : br == 4 ? b : w;
  const T* xrow = x + (long)h * D + c0;

  // Issue every load of the run first (clamped in bounds; masked in the arithmetic).
  piece xr[(R + HIST) * RW::P];
#pragma unroll
  for (int i = 0; i < R + HIST; ++i) {
    long t = t0 - HIST + i;
    if (!conv && i < HIST) t = t0;  // gate branches need no history
    t = t < 0 ? 0 : t >= tokens ? tokens - 1 : t;
#pragma unroll
    for (int p = 0; p < RW::P; ++p)
      xr[i * RW::P + p] = reinterpret_cast<const piece*>(xrow + t * stride)[p];
  }
  const long ybase = (long)h * D + c0;
  if (conv) {
    const float* W = br == 0 ? wq : br == 1 ? wk : wv;
    float4 cw[8];  // the 4 taps of each of this lane's 8 channels
#pragma unroll
    for (int i = 0; i < 8; ++i)
      cw[i] = *reinterpret_cast<const float4*>(W + ((long)h * D + c0 + i) * kConvWidth);
    long s0, next;  // bounds [s0, next) of the sequence holding the current token
    int n = 0;
    if (cu_seqlens == nullptr) {
      s0 = t0 - t0 % T_len;
      next = s0 + T_len;
    } else {
      int lo = 0, hi = N;  // largest n < N with cu[n] <= t0 (skips empty sequences)
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu_seqlens[mid] <= t0) lo = mid; else hi = mid;
      }
      n = lo;
      s0 = cu_seqlens[n];
      next = cu_seqlens[n + 1];
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const long t = t0 + i;
      while (t >= next && t < tokens) {  // entering the next non-empty sequence
        s0 = next;
        if (cu_seqlens == nullptr) {
          next += T_len;
        } else {
          ++n;
          next = n < N ? cu_seqlens[n + 1] : tokens;
        }
      }
      const long lim = s0 - t0;  // run-relative offset of the sequence's first token
      float f[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) f[c] = 0.f;
#pragma unroll
      for (int j = 0; j < kConvWidth; ++j) {
        const int slot = i + j;  // token t - HIST + j
        const bool in = slot - HIST >= lim;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float tap = j == 0 ? cw[c].x : j == 1 ? cw[c].y : j == 2 ? cw[c].z : cw[c].w;
          f[c] = in ? fmaf(tap, RW::get(&xr[slot * RW::P], c), f[c]) : f[c];
        }
      }
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        f[c] = f[c] * sigmoid_f(f[c]);  // SiLU
        ss += f[c] * f[c];
      }
      if (br <= 1) {  // L2 norm over the row's D channels (TPR adjacent lanes)
        for (int m = 1; m < TPR; m <<= 1) ss += __shfl_xor(ss, m, 64);
        const float inv = rsqrtf(ss + kNormEps);
#pragma unroll
        for (int c = 0; c < 8; ++c) f[c] *= inv;
      }
      if (live && t < tokens) store8_t<T>(y + t * stride + ybase, f);
    }
  } else if (br == 3) {
    const float4 s0v = *reinterpret_cast<const float4*>(scale + ybase);
    const float4 s1v = *reinterpret_cast<const float4*>(scale + ybase + 4);
#pragma unroll
    for (int i = 0; i < R; ++i) {
      float f[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float sc = c < 4 ? s0v[c] : s1v[c - 4];
        f[c] = -sc * softplus_f(RW::get(&xr[(i + HIST) * RW::P], c));
      }
      if (live && t0 + i < tokens) store8_t<T>(y + (t0 + i) * stride + ybase, f);
    }
  } else {
    const float gain = br == 4 ? b_max : 1.f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      float f[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) f[c] = gain * sigmoid_f(RW::get(&xr[(i + HIST) * RW::P], c));
      if (live && t0 + i < tokens) store8_t<T>(y + (t0 + i) * stride + ybase, f);
    }
  }
}

// Rows per lane in the epilogue (more independent loads in flight per lane).
constexpr int kEpiRows = 1;

template <typename T, int DV>
__global__ void __launch_bounds__(256)
gdn2_epilogue_kernel(const T* __restrict__ o, const T* __restrict__ gate,
                     const float* __restrict__ weight, T* __restrict__ y, long rows) {
  constexpr int TPR = DV / 8;
  constexpr int RPB = 256 / TPR;  // rows per block step
  typedef Raw8<T> RW;
  typedef typename RW::piece piece;
  const int c0 = (threadIdx.x % TPR) * 8;
  const long row0 = (long)blockIdx.x * RPB * kEpiRows + threadIdx.x / TPR;
  piece ov[kEpiRows * RW::P], gv[kEpiRows * RW::P];
#pragma unroll
  for (int i = 0; i < kEpiRows; ++i) {
    long row = row0 + (long)i * RPB;
    row = row < rows ? row : rows - 1;
#pragma unroll
    for (int p = 0; p < RW::P; ++p) {
      ov[i * RW::P + p] = reinterpret_cast<const piece*>(o + row * DV + c0)[p];
      gv[i * RW::P + p] = reinterpret_cast<const piece*>(gate + row * DV + c0)[p];
    }
  }
  const float4 w0 = *reinterpret_cast<const float4*>(weight + c0);
  const float4 w1 = *reinterpret_cast<const float4*>(weight + c0 + 4);
#pragma unroll
  for (int i = 0; i < kEpiRows; ++i) {
    float fo[8];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      fo[c] = RW::get(&ov[i * RW::P], c);
      ss += fo[c] * fo[c];
    }
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) ss += __shfl_xor(ss, m, 64);
    const float inv = rsqrtf(ss / DV + kNormEps);
    float out[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float gf = RW::get(&gv[i * RW::P], c);
      const float wc = c < 4 ? w0[c] : w1[c - 4];
      out[c] = fo[c] * inv * wc * (gf * sigmoid_f(gf));
    }
    const long row = row0 + (long)i * RPB;
    if (row < rows) store8_t<T>(y + row * DV + c0, out);
  }
}

template <typename T, int DK, int DV>
static hipError_t launch_pro(const PrologueArgs& a) {
  const long tokens = (long)a.B * a.T;
  constexpr int R = prologue_run<T>();
  constexpr int RPB = 256 / ((DK > DV ? DK : DV) / 8);  // rows per block of the widest branch
  const long gx = ((tokens + R - 1) / R * a.H + RPB - 1) / RPB;
  hipLaunchKernelGGL((gdn2_prologue_kernel<T, DK, DV>), dim3((unsigned)gx, 6), dim3(256), 0,
                     (hipStream_t)a.stream, (const T*)a.xq, (const T*)a.xk, (const T*)a.xv,
                     (const T*)a.xg, (const T*)a.xb, (const T*)a.xw, a.wq, a.wk, a.wv, a.scale,
                     a.b_max, (T*)a.q, (T*)a.k, (T*)a.v, (T*)a.g, (T*)a.b, (T*)a.w,
                     a.cu_seqlens, a.N, a.T, a.H, tokens);
  return hipGetLastError();
}

template <typename T>
static hipError_t dispatch_pro(const PrologueArgs& a) {
  if (a.d_k == 64 && a.d_v == 64) return launch_pro<T, 64, 64>(a);
  if (a.d_k == 64 && a.d_v == 128) return launch_pro<T, 64, 128>(a);
  if (a.d_k == 128 && a.d_v == 64) return launch_pro<T, 128, 64>(a);
  if (a.d_k == 128 && a.d_v == 128) return launch_pro<T, 128, 128>(a);
  return hipErrorInvalidValue;
}

hipError_t launch_prologue(const PrologueArgs& a) {
  return a.dtype == 0 ? dispatch_pro<bf16>(a) : dispatch_pro<float>(a);
}

template <typename T, int DV>
static hipError_t launch_epi(const EpilogueArgs& a) {
  constexpr int rows_per_block = 256 / (DV / 8) * kEpiRows;
  const long gx = (a.rows + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL((gdn2_epilogue_kernel<T, DV>), dim3((unsigned)gx), dim3(256), 0,
                     (hipStream_t)a.stream, (const T*)a.o, (const T*)a.gate, a.weight, (T*)a.y,
                     a.rows);
  return hipGetLastError();
}

hipError_t launch_epilogue(const EpilogueArgs& a) {
  if (a.dtype == 0) return a.d_v == 64 ? launch_epi<bf16, 64>(a) : launch_epi<bf16, 128>(a);
  return a.d_v == 64 ? launch_epi<float, 64>(a) : launch_epi<float, 128>(a);
}

}  // namespace gdn2
