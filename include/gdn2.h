/*
 * gdn2.h -- C ABI of the MI355X (gfx950) Gated Delta Rule-2 token mixer.
 *
 * The operation. For every sequence n and head h, with state S (d_k x d_v, fp32) and for
 * each token t in order:
 *     alpha = exp(g_t)              per key channel, g_t = log(alpha_t) <= 0
 *     S_bar = Diag(alpha) S         decay along the key axis
 *     e = b_t * k_t,  z = w_t * v_t gated key (erase gate b, key side) and
 *                                   gated value (write gate w, value side)
 *     r = S_bar^T e                 old read with the gated key
 *     S = S_bar + k_t (z - r)^T     erase that read along k_t, write z along k_t
 *     o_t = S^T q_t                 readout from the updated state
 * This is the Gated Delta Rule-2 of "Gated DeltaNet-2: Decoupling Erase and Write in
 * Linear Attention" (reading note, §2 fast-weight objective and §3 forward pass; the
 * erase runs along k_t, as the objective's minimiser and the (I - k_t e_t^T) factor of
 * §3's backward paragraph fix). No query scale is applied: scale q beforehand if wanted.
 *
 * Conventions common to every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library never
 *     allocates, frees, synchronises, or keeps state between calls. Calls are
 *     asynchronous on `hip_stream` (a hipStream_t; NULL = the null stream).
 *   - Tensors are dense, row-major, contiguous, and 16-byte aligned.
 *   - `dtype` selects the element type of q, k, v, log_alpha, b, w and o:
 *     GDN2_BF16 (bfloat16) or GDN2_F32 (float). States are always fp32.
 *   - Arguments are validated on the host before any launch; on error nothing is
 *     launched and an error status is returned. Gate VALUES are not checked: b and w
 *     outside [0, 1] are computed as given.
 *   - Device faults surface at the caller's next synchronisation.
 *   - Numeric range: every forward entry point (chunked, training, decode) accepts any
 *     log_alpha <= 0, i.e. alpha anywhere in (0, 1], however strong the decay of a chunk
 *     or of a 16-token block; alpha below fp32 range acts as 0 (a full reset). The
 *     chunked backward has a limit of its own (see gdn2_chunk_bwd).
 */
#ifndef GDN2_H_
#define GDN2_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Element type of q, k, v, the gates and o. Entry points take it as a plain int holding a
 * gdn2_dtype value, so that any other value is well defined on both sides of the boundary
 * and is rejected with GDN2_INVALID_ARGUMENT (an enum parameter may be assumed by the
 * compiler to hold only its enumerators, which would let it drop that check).
 */
typedef enum { GDN2_BF16 = 0, GDN2_F32 = 1 } gdn2_dtype;

enum {
  GDN2_OK = 0,
  GDN2_INVALID_ARGUMENT = 1, /* null required pointer, bad sizes, misaligned pointer */
  GDN2_UNSUPPORTED = 2,      /* head widths / dtype combination not built */
  GDN2_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below gdn2_chunk_fwd_workspace_bytes */
  GDN2_LAUNCH_FAILED = 4     /* the HIP runtime rejected a launch */
};

/*
 * Gate layouts for the *_ex entry points (bit set: that gate is one value per token and
 * head, shared by all of its channels, i.e. b = beta * 1 or w = omega * 1, the scalar-gate
 * configurations ablated in the reading note's §4). A scalar b is [..., H] in place of
 * [..., H, d_k]; a scalar w is [..., H] in place of [..., H, d_v]; same dtype, same leading
 * axes. The result equals the per-channel call with the gate broadcast over its channels.
 */
enum { GDN2_GATE_B_SCALAR = 1, GDN2_GATE_W_SCALAR = 2 };

/*
 * Chunkwise-parallel forward over whole sequences (the chunk form of the reading note's
 * §3 chunkwise-training paragraph: a per-channel cumulative decay normalises the state
 * inside a 64-token chunk, the chunk becomes an asymmetric delta recurrence, and the UT
 * transform of the Gated DeltaNet visual reading turns it into triangular-inverse and
 * matrix products). Result equals the token recurrence above up to rounding.
 *
 *   q, k, log_alpha, b : [B, T, H, d_k]   (dtype)
 *   v, w               : [B, T, H, d_v]   (dtype)
 *   initial_state      : [N, H, d_k, d_v] fp32, or NULL for a zero state
 *   o                  : [B, T, H, d_v]   (dtype), written
 *   final_state        : [N, H, d_k, d_v] fp32, or NULL (not written); may alias
 *                        initial_state (each state is read before it is overwritten)
 *   cu_seqlens         : NULL, or device int32 [N+1] offsets into the token axis of a
 *                        packed batch (then B must be 1 and T is the packed length).
 *                        Offsets must be non-decreasing with cu_seqlens[0] = 0 and
 *                        cu_seqlens[N] = T; the kernels clamp them into [0, T] so a bad
 *                        table cannot make them access memory out of bounds (its
 *                        results are then undefined).
 *   workspace          : NULL, or device scratch of at least
 *                        gdn2_chunk_fwd_workspace_bytes(...) bytes (16-byte aligned),
 *                        owned by the caller and free for the call's duration on
 *                        `hip_stream`. With a workspace the call runs the two-phase path:
 *                        one kernel computes every chunk's factors in parallel into the
 *                        workspace, a second walks the chunks of each sequence in order
 *                        (for fixed-length batches with fewer sequence x head chains than
 *                        compute units, each sequence is cut into segments that run in
 *                        parallel: a transfer pass, a scan of segment start states, then
 *                        the outputs). Without one, a single fused kernel does both per
 *                        sequence (for bf16 a kernel that prepares the next chunk's
 *                        operands while it finishes the current one).
 *                        Results agree to rounding. Ignored when
 *                        gdn2_chunk_fwd_workspace_bytes returns 0 for the dtype/widths.
 *   Without cu_seqlens, N must equal B and every sequence has length T.
 *   Supported: d_k, d_v in {64, 128} for both dtypes. GDN2_F32 runs without a workspace
 *   only: the chunk kernel for d_k = 64, and for d_k = 128, whose fp32 chunk operands do
 *   not fit the 160 KB of LDS, the token recurrence itself (one token at a time, fp32
 *   state in registers; exact to fp32 rounding, not chunk-parallel). T = 0 or N = 0 is a
 *   no-op (apart from final_state = initial).
 * Returns GDN2_OK or an error status (GDN2_WORKSPACE_TOO_SMALL when workspace_bytes is
 * below the requirement).
 */
int gdn2_chunk_fwd(const void* q, const void* k, const void* v, const void* log_alpha,
                   const void* b, const void* w, const float* initial_state, void* o,
                   float* final_state, const int32_t* cu_seqlens, int B, int T, int H,
                   int d_k, int d_v, int N, int dtype, void* workspace,
                   size_t workspace_bytes, void* hip_stream);

/*
 * gdn2_chunk_fwd with a gate layout (GDN2_GATE_* bits, 0 = per-channel gates as above):
 * scalar b and / or w are read as [B, T, H] (one value per token and head). Both the fused
 * path and the two-phase path (workspace given) support them. Any other bit gives
 * GDN2_INVALID_ARGUMENT.
 */
int gdn2_chunk_fwd_ex(const void* q, const void* k, const void* v, const void* log_alpha,
                      const void* b, const void* w, const float* initial_state, void* o,
                      float* final_state, const int32_t* cu_seqlens, int B, int T, int H,
                      int d_k, int d_v, int N, int dtype, int gate_layout, void* workspace,
                      size_t workspace_bytes, void* hip_stream);

/*
 * For callers that cannot allocate device memory (work under HIP stream capture, tight
 * serving loops, harnesses that forbid hipMalloc): gdn2_chunk_fwd_ex's two-phase path with
 * its workspace taken from a scratch array that the library holds on each device (a static
 * device array of gdn2_noalloc_scratch_bytes() = 128 MiB, resident from the library's load
 * on that device until the process ends). The call allocates and frees nothing; on its
 * first use on a device it looks up that device's scratch address (hipGetSymbolAddress).
 * The caller still passes every input and output, as for gdn2_chunk_fwd_ex (same
 * arguments without the workspace). Results equal gdn2_chunk_fwd_ex with a workspace.
 *   - Every call on one device shares that device's scratch: calls that may overlap on one
 *     device (different streams, or threads) race and must be serialised by the caller.
 *     The scratch keeps the last call's contents; nothing in it needs to start at zero.
 *   - Sizes whose workspace (gdn2_chunk_fwd_workspace_bytes for the same arguments,
 *     with or without cu_seqlens as given) exceeds the scratch give
 *     GDN2_WORKSPACE_TOO_SMALL and launch nothing; about 1.1 K tokens x heads fit per MiB
 *     at d_k = d_v = 128 (e.g. 4096 tokens x 16 heads in one sequence).
 *   - Built where the two-phase path is: GDN2_BF16 with d_k, d_v in {64, 128}
 *     (GDN2_UNSUPPORTED otherwise; the fused path of gdn2_chunk_fwd needs no workspace).
 */
int gdn2_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* log_alpha,
                           const void* b, const void* w, const float* initial_state, void* o,
                           float* final_state, const int32_t* cu_seqlens, int B, int T, int H,
                           int d_k, int d_v, int N, int dtype, int gate_layout,
                           void* hip_stream);

/* Bytes of the per-device scratch array that gdn2_chunk_fwd_noalloc uses. */
size_t gdn2_noalloc_scratch_bytes(void);

/*
 * Device workspace, in bytes, that the two-phase path of gdn2_chunk_fwd needs for a call
 * with these sizes, with or without cu_seqlens (about 1.13 KiB per token and head at
 * d_k = d_v = 128, plus one chunk per sequence, plus (2 d_v + d_k) d_k fp32 per segment and
 * head when long sequences are cut into segments). 0 when the two-phase path is not built
 * for dtype / d_k / d_v (GDN2_BF16 with d_k, d_v in {64, 128} is) or a size is negative.
 */
size_t gdn2_chunk_fwd_workspace_bytes(int B, int T, int H, int d_k, int d_v, int N,
                                      int dtype);

/*
 * Chunkwise backward: gradients of gdn2_chunk_fwd for upstream gradients of o and of the
 * final states (the gate-aware backward of the reading note's §3: the state gradient flows
 * through the asymmetric factor Diag(alpha_t)(I - e_t k_t^T) of every token; here in chunk
 * form, with one triangular solve per chunk). Inputs and conventions as gdn2_chunk_fwd:
 *
 *   q, k, log_alpha, b, v, w, initial_state, cu_seqlens, B, T, H, d_k, d_v, N : as forward
 *   d_o               : [B, T, H, d_v] (dtype), gradient of o
 *   d_final_state     : [N, H, d_k, d_v] fp32, or NULL for zero
 *   dq, dk, dlog_alpha, db : [B, T, H, d_k] (dtype), written
 *   dv, dw            : [B, T, H, d_v] (dtype), written
 *   d_initial_state   : [N, H, d_k, d_v] fp32, or NULL (not written)
 *   range_flag        : NULL, or a device int32 that the caller clears beforehand. The call
 *                       sets it to 1 when some chunk's total decay, in some key channel,
 *                       exceeds the range of the local-gradient kernel's factors (referenced
 *                       to the middle of each channel's decay over the chunk: about 166 nats
 *                       over 64 tokens); a second kernel then recomputes those chunks'
 *                       gradients with exact pairwise decay factors, so the result is valid
 *                       for any decay either way. The second kernel reads the flag to skip
 *                       its scan when no chunk is out of range (with NULL it always scans).
 *   workspace         : required, at least gdn2_chunk_bwd_workspace_bytes(...) bytes, 16-byte
 *                       aligned, free for the call's duration on `hip_stream`.
 *   Supported: GDN2_BF16 with d_k, d_v in {64, 128}.
 * Returns GDN2_OK or an error status (GDN2_UNSUPPORTED for GDN2_F32,
 * GDN2_WORKSPACE_TOO_SMALL for a missing or short workspace).
 */
int gdn2_chunk_bwd(const void* q, const void* k, const void* v, const void* log_alpha,
                   const void* b, const void* w, const float* initial_state, const void* d_o,
                   const float* d_final_state, void* dq, void* dk, void* dv, void* dlog_alpha,
                   void* db, void* dw, float* d_initial_state, int32_t* range_flag,
                   const int32_t* cu_seqlens, int B, int T, int H, int d_k, int d_v, int N,
                   int dtype, void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Device workspace, in bytes, that gdn2_chunk_bwd (and gdn2_chunk_fwd_train) needs for these
 * sizes, with or without cu_seqlens (about 3.7 KiB per token and head at d_k = d_v = 128, plus
 * one chunk per sequence, plus (2 d_v + d_k) d_k fp32 per segment and head when long
 * sequences are cut into segments, as for the two-phase forward); 0 where the backward is not
 * built.
 */
size_t gdn2_chunk_bwd_workspace_bytes(int B, int T, int H, int d_k, int d_v, int N,
                                      int dtype);

/*
 * gdn2_chunk_bwd with a gate layout (GDN2_GATE_* bits): a scalar b or w is read as
 * [B, T, H], and its gradient db or dw is written as [B, T, H] (the sum over the channels
 * of the per-channel gradient, since the one value is shared by all of them).
 */
int gdn2_chunk_bwd_ex(const void* q, const void* k, const void* v, const void* log_alpha,
                      const void* b, const void* w, const float* initial_state, const void* d_o,
                      const float* d_final_state, void* dq, void* dk, void* dv, void* dlog_alpha,
                      void* db, void* dw, float* d_initial_state, int32_t* range_flag,
                      const int32_t* cu_seqlens, int B, int T, int H, int d_k, int d_v, int N,
                      int dtype, int gate_layout, void* workspace, size_t workspace_bytes,
                      void* hip_stream);

/*
 * Training forward: the same result as gdn2_chunk_fwd (o, and the final state when
 * final_state is not NULL), computed by the two-phase kernels while the backward's
 * intermediates (the chunk factors, every chunk's entering state and U, and for a sequence
 * cut into segments each segment's linear map of the state) are kept in
 * `workspace`, so that gdn2_chunk_bwd_saved can skip the forward recomputation that
 * gdn2_chunk_bwd performs. Same arguments as gdn2_chunk_fwd, except that o is required and
 * workspace is required, of at least gdn2_chunk_bwd_workspace_bytes(...) bytes, and the
 * gate layout (GDN2_GATE_* bits, as for gdn2_chunk_fwd_ex) is given; bf16 only
 * (GDN2_UNSUPPORTED otherwise). The workspace stays owned by the caller and must not be
 * written until the matching gdn2_chunk_bwd_saved has run.
 */
int gdn2_chunk_fwd_train(const void* q, const void* k, const void* v, const void* log_alpha,
                         const void* b, const void* w, const float* initial_state, void* o,
                         float* final_state, const int32_t* cu_seqlens, int B, int T, int H,
                         int d_k, int d_v, int N, int dtype, int gate_layout, void* workspace,
                         size_t workspace_bytes, void* hip_stream);

/*
 * gdn2_chunk_bwd on a workspace written by gdn2_chunk_fwd_train with the same inputs,
 * initial state, cu_seqlens and sizes (the forward recomputation is skipped; nothing checks
 * that the workspace matches, and a mismatched one gives wrong gradients, never an
 * out-of-bounds access). The arguments of gdn2_chunk_bwd_ex, with its errors; the gate layout
 * must be the training forward's.
 */
int gdn2_chunk_bwd_saved(const void* q, const void* k, const void* v, const void* log_alpha,
                         const void* b, const void* w, const float* initial_state,
                         const void* d_o, const float* d_final_state, void* dq, void* dk,
                         void* dv, void* dlog_alpha, void* db, void* dw,
                         float* d_initial_state, int32_t* range_flag,
                         const int32_t* cu_seqlens, int B, int T, int H, int d_k, int d_v,
                         int N, int dtype, int gate_layout, void* workspace,
                         size_t workspace_bytes, void* hip_stream);

/*
 * The fused single-kernel path of gdn2_chunk_fwd (no workspace) with an explicit
 * value-slice width: each workgroup carries
 * `value_slice` columns of the state (16, 32, 64 or 128; a divisor of d_v; 16 only with
 * d_k = 64; at most 64 for GDN2_F32, whose d_k = 128 form has no slices). 0 selects the
 * width automatically, exactly as gdn2_chunk_fwd does. Results do not depend on the width
 * beyond rounding. Returns GDN2_UNSUPPORTED for a width that is not built.
 */
int gdn2_chunk_fwd_sliced(const void* q, const void* k, const void* v, const void* log_alpha,
                          const void* b, const void* w, const float* initial_state, void* o,
                          float* final_state, const int32_t* cu_seqlens, int B, int T, int H,
                          int d_k, int d_v, int N, int dtype, int value_slice,
                          void* hip_stream);

/*
 * One recurrent decode step for N independent sequences (the per-token procedure of
 * the reading note's §3 forward-pass paragraph; constant memory per token, the
 * abstract's decode property). The state is read once and written once in place; the
 * readout is formed from the old state as o = Diag(alpha)-decayed read of q plus
 * (q . k)(z - r), which equals S_t^T q_t.
 *
 *   q, k, log_alpha, b : [N, H, d_k]       (dtype), one token per sequence
 *   v, w               : [N, H, d_v]       (dtype)
 *   state              : [N, H, d_k, d_v]  fp32, read-modify-written in place
 *   o                  : [N, H, d_v]       (dtype), written
 *   Supported: d_k, d_v in {64, 128}, both dtypes. N = 0 is a no-op.
 * Returns GDN2_OK or an error status.
 */
int gdn2_decode_step(const void* q, const void* k, const void* v, const void* log_alpha,
                     const void* b, const void* w, float* state, void* o, int N, int H,
                     int d_k, int d_v, int dtype, void* hip_stream);

/* gdn2_decode_step with a gate layout: scalar b and / or w are [N, H]. */
int gdn2_decode_step_ex(const void* q, const void* k, const void* v, const void* log_alpha,
                        const void* b, const void* w, float* state, void* o, int N, int H,
                        int d_k, int d_v, int dtype, int gate_layout, void* hip_stream);

/*
 * L consecutive tokens for each of N sequences against a pool of recurrent states: decode
 * of a few tokens at once, or verification of draft tokens in speculative decoding (the
 * reading note's §7 names speculative decoding as the serving direction). Per (sequence,
 * head) the state of slot state_indices[n] is read once, advanced through the L tokens with
 * the decode step's arithmetic, and the state after token commit_len[n] - 1 is written back
 * to that slot (commit_len[n] = 0 leaves the slot unchanged). Outputs of all L tokens are
 * written either way.
 *
 *   q, k, log_alpha, b : [N, L, H, d_k]   (dtype)
 *   v, w               : [N, L, H, d_v]   (dtype)
 *   state_pool         : [P, H, d_k, d_v] fp32, read and (partly) written in place
 *   state_indices      : device int32 [N], the slot of each sequence; a negative or >= P
 *                        slot skips the sequence (its outputs are not written). NULL: slot n
 *                        (then P >= N is required). Two sequences must not share a slot.
 *   commit_len         : device int32 [N] in [0, L] (clamped), or NULL for L
 *   o                  : [N, L, H, d_v]   (dtype), written
 *   step_states        : NULL, or [N, L, H, d_k, d_v] fp32: the state after every token
 *                        (so that an accepted prefix can be committed without recomputing)
 *   Supported: d_k, d_v in {64, 128}, both dtypes. N = 0 or L = 0 is a no-op.
 * Returns GDN2_OK or an error status.
 */
int gdn2_decode_tokens(const void* q, const void* k, const void* v, const void* log_alpha,
                       const void* b, const void* w, float* state_pool,
                       const int32_t* state_indices, const int32_t* commit_len, void* o,
                       float* step_states, int N, int L, int H, int d_k, int d_v, int P,
                       int dtype, void* hip_stream);

/* gdn2_decode_tokens with a gate layout: scalar b and / or w are [N, L, H]. */
int gdn2_decode_tokens_ex(const void* q, const void* k, const void* v, const void* log_alpha,
                          const void* b, const void* w, float* state_pool,
                          const int32_t* state_indices, const int32_t* commit_len, void* o,
                          float* step_states, int N, int L, int H, int d_k, int d_v, int P,
                          int dtype, int gate_layout, void* hip_stream);

/*
 * Block prologue: the branches between the block's projections and the mixer (the reading
 * note's §3 block paragraph: q, k = linear -> conv -> SiLU -> L2 norm; v = linear -> conv ->
 * SiLU; per-channel decay, erase and write gates from projections of their own). One pass
 * over the six projected tensors:
 *     q = l2norm(silu(conv(xq))), k = l2norm(silu(conv(xk))), v = silu(conv(xv)),
 *     log_alpha = -decay_scale * softplus(xg), b = b_max * sigmoid(xb), w = sigmoid(xw)
 * with conv the causal depthwise convolution of width 4 over each sequence's tokens
 * (y[t, c] = sum_j conv[c, j] * x[t - 3 + j, c], zero history at every sequence start) and
 * l2norm over d_k with eps 1e-6. (Conv width, eps and the gate activations are this
 * library's readings of what the page leaves open.)
 *
 *   xq, xk, xg, xb     : [B, T, H, d_k]   (dtype) projections
 *   xv, xw             : [B, T, H, d_v]   (dtype)
 *   conv_q, conv_k     : [H * d_k, 4] fp32 taps;  conv_v : [H * d_v, 4] fp32
 *   decay_scale        : [H * d_k] fp32 (positive)
 *   b_max              : 1 nominally, 2 for the widened erase-gate range
 *   q, k, log_alpha, b : [B, T, H, d_k] (dtype), written;  v, w : [B, T, H, d_v] (dtype)
 *   cu_seqlens         : as gdn2_chunk_fwd (B = 1 when given; N = B otherwise)
 * Returns GDN2_OK or an error status.
 */
int gdn2_block_prologue(const void* xq, const void* xk, const void* xv, const void* xg,
                        const void* xb, const void* xw, const float* conv_q,
                        const float* conv_k, const float* conv_v, const float* decay_scale,
                        float b_max, void* q, void* k, void* v, void* log_alpha, void* b,
                        void* w, const int32_t* cu_seqlens, int B, int T, int H, int d_k,
                        int d_v, int N, int dtype, void* hip_stream);

/*
 * Block epilogue: the mixer output scaled by an RMSNorm with a SiLU gate (the reading note's
 * §3 block paragraph): y = o / sqrt(mean_c(o^2) + 1e-6) * weight * silu(gate), the mean over
 * d_v per (token, head).
 *
 *   o, gate, y : [rows, d_v] (dtype), rows = tokens x heads;  weight : [d_v] fp32
 * Returns GDN2_OK or an error status.
 */
int gdn2_block_epilogue(const void* o, const void* gate, const float* weight, void* y,
                        long rows, int d_v, int dtype, void* hip_stream);

/* Human-readable text for a status code (static storage; never NULL). */
const char* gdn2_status_string(int status);

/* Library version string (static storage). */
const char* gdn2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN2_H_ */
