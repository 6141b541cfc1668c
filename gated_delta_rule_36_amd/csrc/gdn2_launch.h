// Host-side launch interface between the C ABI and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn2 {

struct ChunkArgs {
  const void *q, *k, *v, *g, *b, *w;
  const float* s0;
  void* o;
  float* sN;
  const int32_t* cu_seqlens;
  int B, T, H, d_k, d_v, N;
  int dtype;  // 0 = bf16, 1 = fp32
  int nv;     // value-slice width per workgroup
  void* stream;
};

struct DecodeArgs {
  const void *q, *k, *v, *g, *b, *w;
  float* state;
  void* o;
  int N, H, d_k, d_v;
  int dtype;
  void* stream;
};

// Value-slice widths the chunk kernel is built for, given dtype and d_k.
inline bool chunk_nv_supported(int dtype, int d_k, int d_v, int nv) {
  if (nv > d_v || d_v % nv != 0) return false;
  if (dtype == 0) return (nv == 32 || nv == 64 || nv == 128 || (nv == 16 && d_k == 64));
  return d_k == 64 && (nv == 16 || nv == 32 || nv == 64);
}

hipError_t launch_chunk_fwd(const ChunkArgs& a);
hipError_t launch_decode_step(const DecodeArgs& a);

}  // namespace gdn2
