// Host-side launch interface between the C ABI and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn2 {

// Gate layouts (bit set: that gate is one value per (token, head), shared by its channels).
constexpr int kGateBScalar = 1;
constexpr int kGateWScalar = 2;

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
  void* workspace;        // two-phase path only: per-chunk factors (see SplitLayout)
  size_t workspace_bytes;
  int gate_flags = 0;     // kGateBScalar | kGateWScalar
  int nseg = 1;           // two-phase path: segments per sequence (see SegPlan)
  int seg_chunks = 0;     // chunks per segment when nseg > 1
};

struct DecodeArgs {
  const void *q, *k, *v, *g, *b, *w;
  float* state;
  void* o;
  int N, H, d_k, d_v;
  int dtype;
  void* stream;
  int gate_flags = 0;
};

struct DecodeTokensArgs {
  const void *q, *k, *v, *g, *b, *w;  // [N, L, H, d]
  float* pool;                        // [P, H, d_k, d_v]
  const int32_t* indices;             // [N] pool slot per sequence, or null (slot n)
  const int32_t* commit;              // [N] tokens whose update is committed, or null (L)
  void* o;                            // [N, L, H, d_v]
  float* step_states;                 // [N, L, H, d_k, d_v] or null
  int N, L, H, d_k, d_v, P;
  int dtype;
  void* stream;
  int gate_flags = 0;
};

// Value-slice widths the chunk kernel is built for, given dtype and d_k.
inline bool chunk_nv_supported(int dtype, int d_k, int d_v, int nv) {
  if (nv > d_v || d_v % nv != 0) return false;
  if (dtype == 0) return (nv == 32 || nv == 64 || nv == 128 || (nv == 16 && d_k == 64));
  return d_k == 64 && (nv == 16 || nv == 32 || nv == 64);
}

// Two-phase chunk forward (bf16). Phase 1 turns every (64-token chunk, head) into the
// factors the state recurrence needs; phase 2 walks each sequence's chunks in order.
// Per (chunk slot, head) unit the workspace holds, in MFMA fragment order (1 KiB blocks of
// 64 lanes x 8 bf16; key channels / tokens phi-ordered inside each 32-wide K step):
//   -W    [64 tokens][d_k]     blocks (R, s)   R = token tile, s = 32-channel step
//   Qbar  [64 tokens][d_k]     blocks (R, s)   Q 2^G
//   Kt    [d_k][64 tokens]     blocks (m, s)   (K 2^(Glast - G))^T, m = channel tile
//   P     [64][64]             blocks (R, s)
//   U~    D tiles (ct, R) of 16x16, lane-major, 4 bf16 per lane (512 B)
//   gamma [d_k] fp32           2^Glast
struct SplitLayout {
  long w, q, kt, p, u, g, bytes;
  static constexpr int kChunk = 64;
  constexpr SplitLayout(int d_k, int d_v)
      : w(0),
        q(w + 4L * (d_k / 32) * 1024),
        kt(q + 4L * (d_k / 32) * 1024),
        p(kt + (d_k / 16) * 2L * 1024),
        u(p + 8L * 1024),
        g(u + (d_v / 16) * 4L * 512),
        bytes(((g + 4L * d_k) + 255) / 256 * 256) {}
};

// Chunk slots of a call: without cu_seqlens, sequence n owns slots [n*ceil(T/64), ...);
// with cu_seqlens, sequence n owns the slots from floor(cu[n]/64) + n on (disjoint for
// any non-decreasing table, all below floor(T/64) + N).
inline long split_slots(bool varlen, int B, int T, int N) {
  const int C = SplitLayout::kChunk;
  return varlen ? (long)T / C + N : (long)B * ((T + C - 1) / C);
}
// Segments of long sequences (two-phase path, fixed-length batches): when the recurrence
// has fewer chains (sequence x head x 64 value columns) than `target` workgroups, each
// sequence's chunks are cut into nseg segments of seg_chunks (at least 8 chunks each) that
// run in parallel: a transfer pass per segment, a short scan of segment start states,
// then the outputs per segment.
struct SegPlan {
  int nseg, seg_chunks;
};
inline SegPlan seg_plan(bool varlen, int T, int H, int d_v, int N, int target) {
  const int C = SplitLayout::kChunk;
  const int nch = T > 0 ? (T + C - 1) / C : 0;
  const long chains = (long)N * H * (d_v / 64 > 0 ? d_v / 64 : 1);
  if (varlen || N <= 0 || chains <= 0 || chains >= target || nch < 16) return SegPlan{1, nch};
  const long want = (target + chains - 1) / chains;
  const int maxseg = nch / 8;
  const int p = (int)(want < maxseg ? want : maxseg);
  if (p <= 1) return SegPlan{1, nch};
  const int sc = (nch + p - 1) / p;
  return SegPlan{(nch + sc - 1) / sc, sc};
}
// Segment buffers after the factors: end states [N | M] of the transfer pass
// ([units][d_k][d_v + d_k] fp32) and the segment start states ([units][d_k][d_v] fp32).
inline size_t seg_buffer_bytes(const SegPlan& sp, int N, int H, int d_k, int d_v) {
  if (sp.nseg <= 1) return 0;
  return 256 + (size_t)N * H * sp.nseg * d_k * (size_t)(2 * d_v + d_k) * 4;
}
inline size_t split_workspace_bytes(bool varlen, int B, int T, int H, int d_k, int d_v, int N) {
  return (size_t)split_slots(varlen, B, T, N) * H * SplitLayout(d_k, d_v).bytes;
}

// Backward workspace, per (chunk slot, head) unit: the forward factors (SplitLayout) followed
// by the reverse chain's operands, then four per-chunk tensors passed between the kernels.
// All bf16 and in MFMA fragment order unless noted:
//   Kr   Ktil = K 2^(Glast - G)   [64 tokens][d_k]  blocks (R, s), K = channels (phi)
//   Pt   P^T                      [64][64]          blocks (R, s), K = tokens (natural)
//   Qt   Qbar^T                   [d_k][64]         blocks (m, s), K = tokens (natural)
//   Wt   -W^T                     [d_k][64]         blocks (m, s), K = tokens (phi)
//   Bt   back-substitution blocks (R, J), J >= R: (-A_JR)^T for J > R, (T_RR)^T for J = R,
//        16x16 K=16 fragments (64 lanes x 4 bf16)
//   H    state entering the chunk [d_k][d_v]       16x16 accumulator tiles (ct, mt)
//   Ub   U = U~ - W S             [64][d_v]         tiles (ct, R)
//   Db   gradient of the state leaving the chunk [d_k][d_v]  tiles (ct, mt)
//   Zb   dZ = T^T dU              [64][d_v]         tiles (ct, R)
// (accumulator tiles: 64 lanes x 4 bf16 = 512 B, lane l holds column l % 16, rows
// 4 (l / 16) .. + 3, the order the chain kernels hold them in registers)
struct BwdLayout {
  SplitLayout f;
  long kr, pt, qt, wt, bt, factors, h, ub, db, zb, bytes;
  constexpr BwdLayout(int d_k, int d_v)
      : f(d_k, d_v),
        kr(f.bytes),
        pt(kr + 4L * (d_k / 32) * 1024),
        qt(pt + 8L * 1024),
        wt(qt + (d_k / 16) * 2L * 1024),
        bt(wt + (d_k / 16) * 2L * 1024),
        factors(bt + 16L * 512),
        h(factors),
        ub(h + (long)(d_k / 16) * (d_v / 16) * 512),
        db(ub + 4L * (d_v / 16) * 512),
        zb(db + (long)(d_k / 16) * (d_v / 16) * 512),
        bytes(zb + 4L * (d_v / 16) * 512) {}
};

inline size_t bwd_workspace_bytes(bool varlen, int B, int T, int H, int d_k, int d_v, int N) {
  return (size_t)split_slots(varlen, B, T, N) * H * BwdLayout(d_k, d_v).bytes;
}

struct BwdArgs {
  ChunkArgs fwd;            // q..w, s0 (initial state), cu_seqlens, sizes, dtype, stream,
                            // workspace; fwd.o / fwd.sN unused
  const void* d_o;          // [B, T, H, d_v]
  const float* d_sN;        // [N, H, d_k, d_v] or null
  void *dq, *dk, *dv, *dg, *db, *dw;
  float* d_s0;              // [N, H, d_k, d_v] or null
  int* range_flag;          // device int, set to 1 when a chunk is outside the fast range
  bool saved = false;       // the workspace already holds the forward's factors, entering
                            // states and U (written by a training forward): skip that part
};

hipError_t launch_chunk_fwd(const ChunkArgs& a);
// The pipelined fused forward (gdn2_fwd.hip): bf16, d_k and d_v in {64, 128}, 64-column
// value slices.
bool fwd_pipelined_supported(int dtype, int d_k, int d_v);
hipError_t launch_fwd_pipelined(const ChunkArgs& a);
// Token-recurrent forward (gdn2_recurrent.hip): fp32 with d_k = 128, where the chunk
// kernels' fp32 operands do not fit the LDS.
bool fwd_recurrent_used(int dtype, int d_k, int d_v);
hipError_t launch_fwd_recurrent(const ChunkArgs& a);
hipError_t launch_chunk_fwd_split(const ChunkArgs& a);
hipError_t launch_chunk_bwd(const BwdArgs& a);
// pieces of the backward shared with the two-phase forward (gdn2_split.hip)
hipError_t launch_bwd_forward_part(const ChunkArgs& a);
// segment start values by a scan over segments (forward: from s_in = the initial states, in
// segment order; reverse: from s_in = the final states' gradients, last segment first)
hipError_t launch_seg_combine(const float* ebuf, const float* s_in, float* sbuf, int N, int H,
                              int d_k, int d_v, int nseg, bool reverse, void* stream);
int cu_count();  // compute units of the current device
// Library-held scratch (gdn2_noalloc.hip): bytes per device, and this device's address.
size_t scratch_capacity();
hipError_t scratch_for_device(int device, void** ptr);
hipError_t launch_decode_step(const DecodeArgs& a);
hipError_t launch_decode_tokens(const DecodeTokensArgs& a);

}  // namespace gdn2
