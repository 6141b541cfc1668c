// Host-side argument blocks and launchers of the block prologue and epilogue kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gdn2 {

struct PrologueArgs {
  const void *xq, *xk, *xv, *xg, *xb, *xw;  // projections, [B, T, H, d]
  const float *wq, *wk, *wv;               // conv taps [H * d, 4]
  const float* scale;                      // decay scale [H * d_k]
  float b_max;
  void *q, *k, *v, *g, *b, *w;             // mixer inputs, [B, T, H, d]
  const int32_t* cu_seqlens;
  int B, T, H, d_k, d_v, N;
  int dtype;
  void* stream;
};

struct EpilogueArgs {
  const void *o, *gate;  // [rows, d_v] (rows = tokens x heads)
  const float* weight;   // [d_v]
  void* y;
  long rows;
  int d_v, dtype;
  void* stream;
};

hipError_t launch_prologue(const PrologueArgs& a);
hipError_t launch_epilogue(const EpilogueArgs& a);

}  // namespace gdn2
