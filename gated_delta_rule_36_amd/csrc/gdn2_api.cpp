// C ABI of the GDN-2 library: argument validation, tile selection, launch.
// Declarations and the contract of every entry point are in include/gdn2.h.
#include "../../include/gdn2.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>

#include "gdn2_block_launch.h"
#include "gdn2_launch.h"

namespace {

constexpr int kChunk = 64;
constexpr int kTargetWorkgroups = 256;  // one per compute unit of an MI355X

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool width_ok(int d) { return d == 64 || d == 128; }

constexpr int kGateMask = GDN2_GATE_B_SCALAR | GDN2_GATE_W_SCALAR;
static_assert(GDN2_GATE_B_SCALAR == gdn2::kGateBScalar && GDN2_GATE_W_SCALAR == gdn2::kGateWScalar,
              "gate layout bits");

// Widest value slice that still yields about one workgroup per compute unit; wider
// slices recompute less key-side work per token, narrower ones expose more chains.
int pick_nv(int dtype, int d_k, int d_v, long chains) {
  const int cands[4] = {128, 64, 32, 16};
  int best = 0;
  for (int nv : cands) {
    if (!gdn2::chunk_nv_supported(dtype, d_k, d_v, nv)) continue;
    best = nv;  // narrowest supported so far
    if (chains * (d_v / nv) >= kTargetWorkgroups) return nv;
  }
  return best;
}

int status_of(hipError_t e) { return e == hipSuccess ? GDN2_OK : GDN2_LAUNCH_FAILED; }

bool split_built(int dtype, int d_k, int d_v) {
  return dtype == GDN2_BF16 && width_ok(d_k) && width_ok(d_v);
}

// Value-slice width of the two-phase path's recurrence kernel: 64 columns per workgroup
// unless that leaves fewer workgroups than compute units.
int pick_split_nv(int d_v, long chains) {
  return chains * (d_v / 64) >= kTargetWorkgroups ? 64 : 32;
}

gdn2::SegPlan seg_plan_for(bool varlen, int T, int H, int d_v, int N) {
  return gdn2::seg_plan(varlen, T, H, d_v, N, kTargetWorkgroups);
}

size_t workspace_need(bool varlen, int B, int T, int H, int d_k, int d_v, int N) {
  const gdn2::SegPlan sp = seg_plan_for(varlen, T, H, d_v, N);
  return gdn2::split_workspace_bytes(varlen, B, T, H, d_k, d_v, N) +
         gdn2::seg_buffer_bytes(sp, N, H, d_k, d_v);
}

int chunk_fwd_impl(const void* q, const void* k, const void* v, const void* log_alpha,
                   const void* b, const void* w, const float* initial_state, void* o,
                   float* final_state, const int32_t* cu_seqlens, int B, int T, int H, int d_k,
                   int d_v, int N, int dtype, void* workspace, size_t workspace_bytes,
                   void* hip_stream, int nv, int gate_layout) {
  if (dtype != GDN2_BF16 && dtype != GDN2_F32) return GDN2_INVALID_ARGUMENT;
  if ((gate_layout & ~kGateMask) != 0) return GDN2_INVALID_ARGUMENT;
  if (B < 0 || T < 0 || H <= 0 || N < 0 || d_k <= 0 || d_v <= 0) return GDN2_INVALID_ARGUMENT;
  if (cu_seqlens == nullptr) {
    if (N != B) return GDN2_INVALID_ARGUMENT;
  } else {
    if (B != 1) return GDN2_INVALID_ARGUMENT;
  }
  if (!width_ok(d_k) || !width_ok(d_v)) return GDN2_UNSUPPORTED;
  // fp32 with d_k = 128 runs the token-recurrent kernel, which has no value-slice choice
  if (nv != 0 && gdn2::fwd_recurrent_used(dtype, d_k, d_v)) return GDN2_UNSUPPORTED;
  const long tokens = (long)B * T;
  if (tokens > 0 && (!q || !k || !v || !log_alpha || !b || !w || !o))
    return GDN2_INVALID_ARGUMENT;
  const void* ptrs[10] = {q, k, v, log_alpha, b, w, o, initial_state, final_state, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN2_INVALID_ARGUMENT;
  if (cu_seqlens && ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0))
    return GDN2_INVALID_ARGUMENT;
  // 64-bit element offsets are used in the kernels; the grid must fit one dimension.
  if (tokens > (long)INT_MAX) return GDN2_INVALID_ARGUMENT;
  const bool split = workspace != nullptr && split_built(dtype, d_k, d_v);
  if (split && workspace_bytes < workspace_need(cu_seqlens != nullptr, B, T, H, d_k, d_v, N))
    return GDN2_WORKSPACE_TOO_SMALL;
  if (N == 0) return GDN2_OK;

  gdn2::ChunkArgs a;
  a.q = q; a.k = k; a.v = v; a.g = log_alpha; a.b = b; a.w = w;
  a.s0 = initial_state; a.o = o; a.sN = final_state; a.cu_seqlens = cu_seqlens;
  a.B = B; a.T = T; a.H = H; a.d_k = d_k; a.d_v = d_v; a.N = N;
  a.dtype = dtype; a.stream = hip_stream; a.gate_flags = gate_layout;
  a.workspace = split ? workspace : nullptr;
  a.workspace_bytes = split ? workspace_bytes : 0;
  if (split) {
    const gdn2::SegPlan sp = seg_plan_for(cu_seqlens != nullptr, T, H, d_v, N);
    a.nseg = sp.nseg;
    a.seg_chunks = sp.seg_chunks;
    a.nv = pick_split_nv(d_v, (long)N * H * sp.nseg);
    if ((long)N * H * sp.nseg * ((d_v + d_k) / 64) > (long)INT_MAX) return GDN2_INVALID_ARGUMENT;
    if ((long)N * H * (d_v / a.nv) > (long)INT_MAX) return GDN2_INVALID_ARGUMENT;
    return status_of(gdn2::launch_chunk_fwd_split(a));
  }
  if (gdn2::fwd_recurrent_used(dtype, d_k, d_v)) {
    if ((long)N * H * (d_v / 64) > (long)INT_MAX) return GDN2_INVALID_ARGUMENT;
    return status_of(gdn2::launch_fwd_recurrent(a));
  }
  // (the pipelined kernel addresses a chunk's value rows through 32-bit buffer offsets)
  if (nv == 0 && gdn2::fwd_pipelined_supported(dtype, d_k, d_v) &&
      (long)H * d_v * kChunk * 2 <= (long)INT_MAX) {
    if ((long)N * H * (d_v / 64) > (long)INT_MAX) return GDN2_INVALID_ARGUMENT;
    a.nv = 64;
    return status_of(gdn2::launch_fwd_pipelined(a));
  }
  if (nv == 0) nv = pick_nv(dtype, d_k, d_v, (long)N * H);
  if (!gdn2::chunk_nv_supported(dtype, d_k, d_v, nv)) return GDN2_UNSUPPORTED;
  const long grid = (long)N * H * (d_v / nv);
  if (grid > (long)INT_MAX) return GDN2_INVALID_ARGUMENT;
  a.nv = nv;
  return status_of(gdn2::launch_chunk_fwd(a));
}

size_t bwd_workspace_need(bool varlen, int B, int T, int H, int d_k, int d_v, int N) {
  // the same segment plan (and buffers) as the two-phase forward: the backward's forward
  // pass and its reverse chain cut long sequences the same way
  const gdn2::SegPlan sp = seg_plan_for(varlen, T, H, d_v, N);
  return gdn2::bwd_workspace_bytes(varlen, B, T, H, d_k, d_v, N) +
         gdn2::seg_buffer_bytes(sp, N, H, d_k, d_v);
}

int chunk_bwd_impl(const void* q, const void* k, const void* v, const void* log_alpha,
                   const void* b, const void* w, const float* initial_state, const void* d_o,
                   const float* d_final_state, void* dq, void* dk, void* dv, void* dlog_alpha,
                   void* db, void* dw, float* d_initial_state, int32_t* range_flag,
                   const int32_t* cu_seqlens, int B, int T, int H, int d_k, int d_v, int N,
                   int dtype, void* workspace, size_t workspace_bytes, void* hip_stream,
                   bool saved, int gate_layout) {
  if (dtype != GDN2_BF16 && dtype != GDN2_F32) return GDN2_INVALID_ARGUMENT;
  if ((gate_layout & ~kGateMask) != 0) return GDN2_INVALID_ARGUMENT;
  if (B < 0 || T < 0 || H <= 0 || N < 0 || d_k <= 0 || d_v <= 0) return GDN2_INVALID_ARGUMENT;
  if (cu_seqlens == nullptr) {
    if (N != B) return GDN2_INVALID_ARGUMENT;
  } else {
    if (B != 1) return GDN2_INVALID_ARGUMENT;
  }
  if (!split_built(dtype, d_k, d_v)) return GDN2_UNSUPPORTED;
  const long tokens = (long)B * T;
  if (tokens > 0 && (!q || !k || !v || !log_alpha || !b || !w || !d_o || !dq || !dk || !dv ||
                     !dlog_alpha || !db || !dw))
    return GDN2_INVALID_ARGUMENT;
  const void* ptrs[17] = {q, k, v, log_alpha, b, w, initial_state, d_o, d_final_state, dq,
                          dk, dv, dlog_alpha, db, dw, d_initial_state, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN2_INVALID_ARGUMENT;
  if ((cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) ||
      (range_flag && (reinterpret_cast<uintptr_t>(range_flag) & 3u) != 0))
    return GDN2_INVALID_ARGUMENT;
  if (tokens > (long)INT_MAX) return GDN2_INVALID_ARGUMENT;
  if (workspace == nullptr ||
      workspace_bytes < bwd_workspace_need(cu_seqlens != nullptr, B, T, H, d_k, d_v, N))
    return GDN2_WORKSPACE_TOO_SMALL;
  if (N == 0) return GDN2_OK;
  const gdn2::SegPlan sp = seg_plan_for(cu_seqlens != nullptr, T, H, d_v, N);
  if ((long)N * H * sp.nseg * ((d_v + d_k) / 64) > (long)INT_MAX) return GDN2_INVALID_ARGUMENT;

  gdn2::BwdArgs a;
  gdn2::ChunkArgs& f = a.fwd;
  f.q = q; f.k = k; f.v = v; f.g = log_alpha; f.b = b; f.w = w;
  f.s0 = initial_state; f.o = nullptr; f.sN = nullptr; f.cu_seqlens = cu_seqlens;
  f.B = B; f.T = T; f.H = H; f.d_k = d_k; f.d_v = d_v; f.N = N;
  f.dtype = dtype; f.nv = 64; f.stream = hip_stream; f.gate_flags = gate_layout;
  f.workspace = workspace; f.workspace_bytes = workspace_bytes;
  f.nseg = sp.nseg; f.seg_chunks = sp.seg_chunks;
  a.d_o = d_o; a.d_sN = d_final_state;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dlog_alpha; a.db = db; a.dw = dw;
  a.d_s0 = d_initial_state; a.range_flag = range_flag; a.saved = saved;
  return status_of(gdn2::launch_chunk_bwd(a));
}

}  // namespace

extern "C" {

size_t gdn2_chunk_fwd_workspace_bytes(int B, int T, int H, int d_k, int d_v, int N,
                                      int dtype) {
  if (B < 0 || T < 0 || H <= 0 || N < 0 || !split_built(dtype, d_k, d_v)) return 0;
  const size_t a = workspace_need(false, B, T, H, d_k, d_v, N);
  const size_t c = workspace_need(true, B, (int)std::min<long>((long)B * T, INT_MAX), H, d_k, d_v, N);
  return a > c ? a : c;
}

int gdn2_chunk_fwd(const void* q, const void* k, const void* v, const void* log_alpha,
                   const void* b, const void* w, const float* initial_state, void* o,
                   float* final_state, const int32_t* cu_seqlens, int B, int T, int H,
                   int d_k, int d_v, int N, int dtype, void* workspace,
                   size_t workspace_bytes, void* hip_stream) {
  return chunk_fwd_impl(q, k, v, log_alpha, b, w, initial_state, o, final_state, cu_seqlens,
                        B, T, H, d_k, d_v, N, dtype, workspace, workspace_bytes, hip_stream, 0, 0);
}

int gdn2_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* log_alpha,
                           const void* b, const void* w, const float* initial_state, void* o,
                           float* final_state, const int32_t* cu_seqlens, int B, int T, int H,
                           int d_k, int d_v, int N, int dtype, int gate_layout,
                           void* hip_stream) {
  if (dtype != GDN2_BF16 && dtype != GDN2_F32) return GDN2_INVALID_ARGUMENT;
  if (B < 0 || T < 0 || H <= 0 || N < 0 || d_k <= 0 || d_v <= 0) return GDN2_INVALID_ARGUMENT;
  if (!split_built(dtype, d_k, d_v)) return GDN2_UNSUPPORTED;
  const size_t need = workspace_need(cu_seqlens != nullptr, B, T, H, d_k, d_v, N);
  if (need > gdn2::scratch_capacity()) return GDN2_WORKSPACE_TOO_SMALL;
  int dev = -1;
  if (hip_stream != nullptr) {
    if (hipStreamGetDevice((hipStream_t)hip_stream, &dev) != hipSuccess)
      return GDN2_INVALID_ARGUMENT;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return GDN2_LAUNCH_FAILED;
  }
  void* scratch = nullptr;
  if (gdn2::scratch_for_device(dev, &scratch) != hipSuccess) return GDN2_LAUNCH_FAILED;
  return chunk_fwd_impl(q, k, v, log_alpha, b, w, initial_state, o, final_state, cu_seqlens,
                        B, T, H, d_k, d_v, N, dtype, scratch, gdn2::scratch_capacity(),
                        hip_stream, 0, gate_layout);
}

size_t gdn2_noalloc_scratch_bytes(void) { return gdn2::scratch_capacity(); }

int gdn2_chunk_fwd_ex(const void* q, const void* k, const void* v, const void* log_alpha,
                      const void* b, const void* w, const float* initial_state, void* o,
                      float* final_state, const int32_t* cu_seqlens, int B, int T, int H,
                      int d_k, int d_v, int N, int dtype, int gate_layout, void* workspace,
                      size_t workspace_bytes, void* hip_stream) {
  return chunk_fwd_impl(q, k, v, log_alpha, b, w, initial_state, o, final_state, cu_seqlens,
                        B, T, H, d_k, d_v, N, dtype, workspace, workspace_bytes, hip_stream, 0,
                        gate_layout);
}

int gdn2_chunk_fwd_sliced(const void* q, const void* k, const void* v, const void* log_alpha,
                          const void* b, const void* w, const float* initial_state, void* o,
                          float* final_state, const int32_t* cu_seqlens, int B, int T, int H,
                          int d_k, int d_v, int N, int dtype, int value_slice,
                          void* hip_stream) {
  if (value_slice < 0) return GDN2_INVALID_ARGUMENT;
  return chunk_fwd_impl(q, k, v, log_alpha, b, w, initial_state, o, final_state, cu_seqlens,
                        B, T, H, d_k, d_v, N, dtype, nullptr, 0, hip_stream, value_slice, 0);
}

size_t gdn2_chunk_bwd_workspace_bytes(int B, int T, int H, int d_k, int d_v, int N,
                                      int dtype) {
  if (B < 0 || T < 0 || H <= 0 || N < 0 || !split_built(dtype, d_k, d_v)) return 0;
  const size_t a = bwd_workspace_need(false, B, T, H, d_k, d_v, N);
  const size_t c = bwd_workspace_need(true, B, (int)std::min<long>((long)B * T, INT_MAX), H, d_k, d_v, N);
  return a > c ? a : c;
}

int gdn2_chunk_bwd(const void* q, const void* k, const void* v, const void* log_alpha,
                   const void* b, const void* w, const float* initial_state, const void* d_o,
                   const float* d_final_state, void* dq, void* dk, void* dv, void* dlog_alpha,
                   void* db, void* dw, float* d_initial_state, int32_t* range_flag,
                   const int32_t* cu_seqlens, int B, int T, int H, int d_k, int d_v, int N,
                   int dtype, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return chunk_bwd_impl(q, k, v, log_alpha, b, w, initial_state, d_o, d_final_state, dq, dk, dv,
                        dlog_alpha, db, dw, d_initial_state, range_flag, cu_seqlens, B, T, H, d_k,
                        d_v, N, dtype, workspace, workspace_bytes, hip_stream, false, 0);
}

int gdn2_chunk_bwd_ex(const void* q, const void* k, const void* v, const void* log_alpha,
                      const void* b, const void* w, const float* initial_state, const void* d_o,
                      const float* d_final_state, void* dq, void* dk, void* dv, void* dlog_alpha,
                      void* db, void* dw, float* d_initial_state, int32_t* range_flag,
                      const int32_t* cu_seqlens, int B, int T, int H, int d_k, int d_v, int N,
                      int dtype, int gate_layout, void* workspace, size_t workspace_bytes,
                      void* hip_stream) {
  return chunk_bwd_impl(q, k, v, log_alpha, b, w, initial_state, d_o, d_final_state, dq, dk, dv,
                        dlog_alpha, db, dw, d_initial_state, range_flag, cu_seqlens, B, T, H, d_k,
                        d_v, N, dtype, workspace, workspace_bytes, hip_stream, false, gate_layout);
}

int gdn2_chunk_bwd_saved(const void* q, const void* k, const void* v, const void* log_alpha,
                         const void* b, const void* w, const float* initial_state,
                         const void* d_o, const float* d_final_state, void* dq, void* dk,
                         void* dv, void* dlog_alpha, void* db, void* dw,
                         float* d_initial_state, int32_t* range_flag,
                         const int32_t* cu_seqlens, int B, int T, int H, int d_k, int d_v,
                         int N, int dtype, int gate_layout, void* workspace,
                         size_t workspace_bytes, void* hip_stream) {
  return chunk_bwd_impl(q, k, v, log_alpha, b, w, initial_state, d_o, d_final_state, dq, dk, dv,
                        dlog_alpha, db, dw, d_initial_state, range_flag, cu_seqlens, B, T, H, d_k,
                        d_v, N, dtype, workspace, workspace_bytes, hip_stream, true, gate_layout);
}

int gdn2_chunk_fwd_train(const void* q, const void* k, const void* v, const void* log_alpha,
                         const void* b, const void* w, const float* initial_state, void* o,
                         float* final_state, const int32_t* cu_seqlens, int B, int T, int H,
                         int d_k, int d_v, int N, int dtype, int gate_layout, void* workspace,
                         size_t workspace_bytes, void* hip_stream) {
  if (dtype != GDN2_BF16 && dtype != GDN2_F32) return GDN2_INVALID_ARGUMENT;
  if ((gate_layout & ~kGateMask) != 0) return GDN2_INVALID_ARGUMENT;
  if (B < 0 || T < 0 || H <= 0 || N < 0 || d_k <= 0 || d_v <= 0) return GDN2_INVALID_ARGUMENT;
  if (cu_seqlens == nullptr ? N != B : B != 1) return GDN2_INVALID_ARGUMENT;
  if (!split_built(dtype, d_k, d_v)) return GDN2_UNSUPPORTED;
  const long tokens = (long)B * T;
  if (tokens > 0 && (!q || !k || !v || !log_alpha || !b || !w || !o)) return GDN2_INVALID_ARGUMENT;
  const void* ptrs[10] = {q, k, v, log_alpha, b, w, o, initial_state, final_state, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN2_INVALID_ARGUMENT;
  if (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return GDN2_INVALID_ARGUMENT;
  if (tokens > (long)INT_MAX) return GDN2_INVALID_ARGUMENT;
  if (workspace == nullptr ||
      workspace_bytes < bwd_workspace_need(cu_seqlens != nullptr, B, T, H, d_k, d_v, N))
    return GDN2_WORKSPACE_TOO_SMALL;
  if (N == 0) return GDN2_OK;
  const gdn2::SegPlan sp = seg_plan_for(cu_seqlens != nullptr, T, H, d_v, N);
  if ((long)N * H * sp.nseg * ((d_v + d_k) / 64) > (long)INT_MAX) return GDN2_INVALID_ARGUMENT;
  if (o == nullptr) return GDN2_INVALID_ARGUMENT;  // (tokens == 0 with N > 0: o still required)
  gdn2::ChunkArgs f;
  f.q = q; f.k = k; f.v = v; f.g = log_alpha; f.b = b; f.w = w;
  f.s0 = initial_state; f.o = o; f.sN = final_state; f.cu_seqlens = cu_seqlens;
  f.B = B; f.T = T; f.H = H; f.d_k = d_k; f.d_v = d_v; f.N = N;
  f.dtype = dtype; f.nv = 64; f.stream = hip_stream; f.gate_flags = gate_layout;
  f.workspace = workspace; f.workspace_bytes = workspace_bytes;
  f.nseg = sp.nseg; f.seg_chunks = sp.seg_chunks;
  return status_of(gdn2::launch_bwd_forward_part(f));
}

int gdn2_decode_step(const void* q, const void* k, const void* v, const void* log_alpha,
                     const void* b, const void* w, float* state, void* o, int N, int H,
                     int d_k, int d_v, int dtype, void* hip_stream) {
  return gdn2_decode_step_ex(q, k, v, log_alpha, b, w, state, o, N, H, d_k, d_v, dtype, 0,
                             hip_stream);
}

int gdn2_decode_step_ex(const void* q, const void* k, const void* v, const void* log_alpha,
                        const void* b, const void* w, float* state, void* o, int N, int H,
                        int d_k, int d_v, int dtype, int gate_layout, void* hip_stream) {
  if (dtype != GDN2_BF16 && dtype != GDN2_F32) return GDN2_INVALID_ARGUMENT;
  if ((gate_layout & ~kGateMask) != 0) return GDN2_INVALID_ARGUMENT;
  if (N < 0 || H <= 0 || d_k <= 0 || d_v <= 0) return GDN2_INVALID_ARGUMENT;
  if (!width_ok(d_k) || !width_ok(d_v)) return GDN2_UNSUPPORTED;
  if (N == 0) return GDN2_OK;
  if (!q || !k || !v || !log_alpha || !b || !w || !state || !o) return GDN2_INVALID_ARGUMENT;
  const void* ptrs[8] = {q, k, v, log_alpha, b, w, state, o};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GDN2_INVALID_ARGUMENT;
  if ((long)N * H > (long)INT_MAX) return GDN2_INVALID_ARGUMENT;
  gdn2::DecodeArgs a;
  a.q = q; a.k = k; a.v = v; a.g = log_alpha; a.b = b; a.w = w;
  a.state = state; a.o = o; a.N = N; a.H = H; a.d_k = d_k; a.d_v = d_v;
  a.dtype = dtype; a.stream = hip_stream; a.gate_flags = gate_layout;
  return status_of(gdn2::launch_decode_step(a));
}

int gdn2_decode_tokens(const void* q, const void* k, const void* v, const void* log_alpha,
                       const void* b, const void* w, float* state_pool,
                       const int32_t* state_indices, const int32_t* commit_len, void* o,
                       float* step_states, int N, int L, int H, int d_k, int d_v, int P,
                       int dtype, void* hip_stream) {
  return gdn2_decode_tokens_ex(q, k, v, log_alpha, b, w, state_pool, state_indices, commit_len,
                               o, step_states, N, L, H, d_k, d_v, P, dtype, 0, hip_stream);
}

int gdn2_decode_tokens_ex(const void* q, const void* k, const void* v, const void* log_alpha,
                          const void* b, const void* w, float* state_pool,
                          const int32_t* state_indices, const int32_t* commit_len, void* o,
                          float* step_states, int N, int L, int H, int d_k, int d_v, int P,
                          int dtype, int gate_layout, void* hip_stream) {
  if (dtype != GDN2_BF16 && dtype != GDN2_F32) return GDN2_INVALID_ARGUMENT;
  if ((gate_layout & ~kGateMask) != 0) return GDN2_INVALID_ARGUMENT;
  if (N < 0 || L < 0 || H <= 0 || P < 0 || d_k <= 0 || d_v <= 0) return GDN2_INVALID_ARGUMENT;
  if (!width_ok(d_k) || !width_ok(d_v)) return GDN2_UNSUPPORTED;
  if (N == 0 || L == 0) return GDN2_OK;
  if (!q || !k || !v || !log_alpha || !b || !w || !state_pool || !o) return GDN2_INVALID_ARGUMENT;
  if (state_indices == nullptr && P < N) return GDN2_INVALID_ARGUMENT;
  const void* ptrs[9] = {q, k, v, log_alpha, b, w, state_pool, o, step_states};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN2_INVALID_ARGUMENT;
  if ((state_indices && (reinterpret_cast<uintptr_t>(state_indices) & 3u) != 0) ||
      (commit_len && (reinterpret_cast<uintptr_t>(commit_len) & 3u) != 0))
    return GDN2_INVALID_ARGUMENT;
  if ((long)N * H > (long)INT_MAX || (long)N * L * H > (long)INT_MAX) return GDN2_INVALID_ARGUMENT;
  gdn2::DecodeTokensArgs a;
  a.q = q; a.k = k; a.v = v; a.g = log_alpha; a.b = b; a.w = w;
  a.pool = state_pool; a.indices = state_indices; a.commit = commit_len; a.o = o;
  a.step_states = step_states; a.N = N; a.L = L; a.H = H; a.d_k = d_k; a.d_v = d_v; a.P = P;
  a.dtype = dtype; a.stream = hip_stream; a.gate_flags = gate_layout;
  return status_of(gdn2::launch_decode_tokens(a));
}

int gdn2_block_prologue(const void* xq, const void* xk, const void* xv, const void* xg,
                        const void* xb, const void* xw, const float* conv_q,
                        const float* conv_k, const float* conv_v, const float* decay_scale,
                        float b_max, void* q, void* k, void* v, void* log_alpha, void* b,
                        void* w, const int32_t* cu_seqlens, int B, int T, int H, int d_k,
                        int d_v, int N, int dtype, void* hip_stream) {
  if (dtype != GDN2_BF16 && dtype != GDN2_F32) return GDN2_INVALID_ARGUMENT;
  if (B < 0 || T < 0 || H <= 0 || N < 0 || d_k <= 0 || d_v <= 0) return GDN2_INVALID_ARGUMENT;
  if (cu_seqlens == nullptr ? N != B : B != 1) return GDN2_INVALID_ARGUMENT;
  if (!width_ok(d_k) || !width_ok(d_v)) return GDN2_UNSUPPORTED;
  const long tokens = (long)B * T;
  if (tokens == 0) return GDN2_OK;
  const void* ptrs[16] = {xq, xk, xv, xg, xb, xw, conv_q, conv_k, conv_v, decay_scale,
                          q, k, v, log_alpha, b, w};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return GDN2_INVALID_ARGUMENT;
  if (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0)
    return GDN2_INVALID_ARGUMENT;
  if (tokens * H > (long)INT_MAX * 8) return GDN2_INVALID_ARGUMENT;
  gdn2::PrologueArgs a;
  a.xq = xq; a.xk = xk; a.xv = xv; a.xg = xg; a.xb = xb; a.xw = xw;
  a.wq = conv_q; a.wk = conv_k; a.wv = conv_v; a.scale = decay_scale; a.b_max = b_max;
  a.q = q; a.k = k; a.v = v; a.g = log_alpha; a.b = b; a.w = w; a.cu_seqlens = cu_seqlens;
  a.B = B; a.T = T; a.H = H; a.d_k = d_k; a.d_v = d_v; a.N = N; a.dtype = dtype;
  a.stream = hip_stream;
  return status_of(gdn2::launch_prologue(a));
}

int gdn2_block_epilogue(const void* o, const void* gate, const float* weight, void* y,
                        long rows, int d_v, int dtype, void* hip_stream) {
  if (dtype != GDN2_BF16 && dtype != GDN2_F32) return GDN2_INVALID_ARGUMENT;
  if (rows < 0 || d_v <= 0) return GDN2_INVALID_ARGUMENT;
  if (!width_ok(d_v)) return GDN2_UNSUPPORTED;
  if (rows == 0) return GDN2_OK;
  const void* ptrs[4] = {o, gate, weight, y};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return GDN2_INVALID_ARGUMENT;
  if (rows > (long)INT_MAX * 16) return GDN2_INVALID_ARGUMENT;
  gdn2::EpilogueArgs a;
  a.o = o; a.gate = gate; a.weight = weight; a.y = y; a.rows = rows; a.d_v = d_v;
  a.dtype = dtype; a.stream = hip_stream;
  return status_of(gdn2::launch_epilogue(a));
}

const char* gdn2_status_string(int status) {
  switch (status) {
    case GDN2_OK: return "ok";
    case GDN2_INVALID_ARGUMENT: return "invalid argument";
    case GDN2_UNSUPPORTED: return "unsupported head width, dtype or value slice";
    case GDN2_WORKSPACE_TOO_SMALL:
      return "workspace too small (for gdn2_chunk_fwd_noalloc: the call needs more than the "
             "library-held scratch, gdn2_noalloc_scratch_bytes())";
    case GDN2_LAUNCH_FAILED: return "kernel launch failed";
    default: return "unknown status";
  }
}

const char* gdn2_version(void) { return "gdn2-mi355x 0.2.0 (gfx950)"; }

}  // extern "C"
