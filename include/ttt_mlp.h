/*
 * ttt_mlp.h -- C ABI of the MI355X (gfx950) In-Place TTT fast-weight MLP layer.
 *
 * The operation (page "In-Place TTT：给LLM装上'临时记忆插槽'，让它边读边学",
 * zhichai.net):
 *   section 3.1  the gated MLP O = SiLU(H W_gate^T) (.) (H W_up^T) W_down^T with
 *                W_down as the fast ("in-place") weight, all else frozen;
 *   section 3.2  chunk-wise schedule: each chunk of C tokens is output with the
 *                current W_down, then W_down takes one update; chunks can be
 *                run in parallel by per-chunk increments and one prefix sum;
 *   section 3.3  the LM-aligned target V^ = Conv1D(X0) W_target and the update
 *                W^(i) = W^(i-1) + eta V^_i^T Z_i.
 * Per-session fast-weight buffers over shared read-only base weights and their
 * reset follow the serving notes of the practitioner blog (blog.travelaiplan.net,
 * section 4 on block-wise updates and multi-request serving, and the TTL/reset
 * item of its safeguards list).
 *
 * Readings fixed by this library where the page is loose:
 *   - Conv1D is depthwise with K taps, U[t][c] = sum_{k<K} taps[c][k] X0[t+1-k][c],
 *     X0 zero outside [0, T) of each sequence, not restarted per chunk, no bias;
 *   - W_target is d x d stored [c_in][j_out] and applied on the right, V^ = U W_target;
 *   - chunk 0 uses W_down0; the last chunk's update is part of the final weight;
 *     a tail chunk shorter than C follows the same rules;
 *   - eta is a plain scalar (no 1/C, no decay).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (HIP, same device as the stream),
 *     row-major, contiguous, 16-byte aligned; the workspace 256-byte aligned.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *     Calls only enqueue work and return; the caller synchronises.
 *   - The caller owns every buffer (inputs, outputs, state, workspace).  The
 *     library allocates no device memory and keeps no device state, apart from
 *     the static 4 MiB buffer per GPU of ttt_mlp_forward_stream_decode_noalloc.
 *     Inputs are never written.  Outputs and the workspace must not overlap
 *     inputs or each other (checked on address ranges).
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error status nothing has been written.  TTT_ERR_HIP means a launch failed
 *     after validation; outputs are then undefined.  ttt_last_error() returns a
 *     message for the calling thread's last non-OK status.
 *   - Nothing throws across the ABI.
 *
 * Number formats: dtype TTT_BF16 means activations (H, X0, O) and weights
 * (W_gate, W_up, W_down0, taps, W_target) are bf16; TTT_F32 means all fp32.
 * The fast-weight state is always fp32.  Contractions run on MFMA with fp32
 * accumulation; Z, eta*V^, each chunk's weight and O are rounded (RNE) to the
 * activation type.
 */
#ifndef TTT_MLP_H
#define TTT_MLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { TTT_F32 = 0, TTT_BF16 = 1 } ttt_dtype_t;

typedef enum {
  TTT_OK = 0,
  TTT_ERR_INVALID_ARGUMENT = -1,
  TTT_ERR_UNSUPPORTED = -2,
  TTT_ERR_WORKSPACE_TOO_SMALL = -3,
  TTT_ERR_HIP = -4
} ttt_status_t;

/* How the chunk recurrence is evaluated.  All give bit-identical results.
 * The chunks of a sequence go in groups of G: a scan over the group streams
 * the exclusive prefix of the per-chunk increments through the fp32 state and
 * writes the weight each chunk uses into a slot; the group's outputs are then
 * computed from its slots, in the same launch as the next group's scan.
 *   SEQUENTIAL      one read-modify-write of the fp32 state in memory per
 *                   chunk (the chunk-by-chunk schedule of section 3.2): each
 *                   chunk's scan is a launch of its own, which writes the
 *                   chunk's slot and the state; a group's outputs run in the
 *                   launch of the next group's first chunk.  Groups as in
 *                   AUTO (G = 1: outputs of chunk i - 1 beside the update of
 *                   chunk i);
 *   CHUNK_PARALLEL  G as large as the workspace holds, up to all chunks (the
 *                   three-step form of section 3.2);
 *   AUTO            chunk-parallel in four groups (fewer if the workspace is
 *                   smaller), so that scans and outputs share launches; one
 *                   group when one scan already has B * ceil(d / 256) *
 *                   ceil(f / 256) >= 1024 weight tiles (many sequences). */
typedef enum {
  TTT_MODE_AUTO = 0,
  TTT_MODE_SEQUENTIAL = 1,
  TTT_MODE_CHUNK_PARALLEL = 2
} ttt_mode_t;

/* Which target the fast weight is trained toward (section 3.3's
 * V^ = Conv1D(X0) W_target, and the variants of the page's ablation table in
 * section 6, read as replacing the left-out part by the identity):
 *   CONV_PROJ  V^ = Conv1D(X0) W_target (the method)
 *   PROJ       V^ = X0 W_target         ("w/o Conv": the token's own embedding)
 *   CONV       V^ = Conv1D(X0)          ("w/o Proj")
 *   EMBED      V^ = X0                  ("w/o Conv, Proj")
 * conv_taps may be NULL when the mode has no conv, W_target when it has no
 * projection. */
typedef enum {
  TTT_TARGET_CONV_PROJ = 0,
  TTT_TARGET_PROJ = 1,
  TTT_TARGET_CONV = 2,
  TTT_TARGET_EMBED = 3
} ttt_target_t;

/* Which token the conv's window ends at (the comparison of the LM-aligned and
 * the reconstruction target in section 4's table):
 *   NEXT  U[t][c] = sum_k taps[c][k] * X0[t+1-k][c]  (the method: tap 0 reads
 *         the next token, the target is aligned with next-token prediction)
 *   SELF  U[t][c] = sum_k taps[c][k] * X0[t-k][c]    (the same window shifted
 *         by one: the reconstruction alignment, tap 0 reads the token itself)
 * Only the targets with a conv depend on it. */
typedef enum {
  TTT_ALIGN_NEXT = 0,
  TTT_ALIGN_SELF = 1
} ttt_align_t;

/* Shapes and scalars of one call.
 *   batch    B >= 1 independent sequences (ttt_mlp_forward requires B == 1);
 *   seq_len  T >= 1 tokens per sequence;
 *   d_model  d, a multiple of 64, at most 2^20;
 *   d_ff     f, a multiple of 64, at most 2^20;
 *            (B*T, d*f and B*ceil(T/C)*ceil64(C) must each stay below 2^31);
 *   chunk    C >= 1 tokens per chunk (the last chunk may be shorter);
 *   conv_k   K taps, 1 <= K <= 8;
 *   eta      finite fast-weight learning rate (0 gives the static MLP);
 *   dtype    TTT_BF16 or TTT_F32 for activations and weights;
 *   mode     see ttt_mode_t;
 *   init_from_w0  (batched only) 1: every W_state[b] is first set to W_down0;
 *                 0: W_state holds each sequence's starting weight on entry;
 *   target   see ttt_target_t (0 for the method itself);
 *   align    see ttt_align_t (0 for the method itself). */
typedef struct {
  int64_t batch;
  int64_t seq_len;
  int64_t d_model;
  int64_t d_ff;
  int32_t chunk;
  int32_t conv_k;
  float eta;
  ttt_dtype_t dtype;
  ttt_mode_t mode;
  int32_t init_from_w0;
  ttt_target_t target;
  ttt_align_t align;
} ttt_mlp_desc_t;

/* Workspace bytes needed for groups of up to `max_group` chunks (0 = the
 * mode's own group: all ceil(T/C) chunks chunk-parallel, a quarter of them
 * (rounded up) auto and sequential).  The workspace holds the activations in
 * the layouts the kernels read, the prepared weights, and one weight slot
 * (B * d * f elements) per chunk of a group, twice over when there is more
 * than one group.  Returns 0 if the descriptor is invalid (see
 * ttt_last_error()).  ttt_mlp_workspace_size(desc, 1) bytes is the minimum. */
size_t ttt_mlp_workspace_size(const ttt_mlp_desc_t* desc, int64_t max_group);

/* Chunks per group the planner would use for this descriptor and workspace
 * size, or a negative ttt_status_t. */
int64_t ttt_mlp_group_size(const ttt_mlp_desc_t* desc, size_t ws_bytes);

/* One sequence (B == 1), starting from W_down0.
 *   H, X0      [T][d]    hidden states entering the MLP / token embeddings X0
 *   W_gate     [f][d]    W_up [f][d]     frozen projections
 *   W_down0    [d][f]    initial fast weight (dtype), read-only
 *   conv_taps  [d][K]    taps[c][k] multiplies X0[t+1-k][c]
 *   W_target   [d][d]    [c_in][j_out]
 *   O          [T][d]    output, dtype
 *   W_down_final [d][f]  fp32, receives W^(N) (the weight after the last chunk)
 *   ws, ws_bytes         workspace (>= ttt_mlp_workspace_size(desc, 1)) */
ttt_status_t ttt_mlp_forward(const ttt_mlp_desc_t* desc, const void* H, const void* X0,
                             const void* W_gate, const void* W_up, const void* W_down0,
                             const void* conv_taps, const void* W_target, void* O,
                             float* W_down_final, void* ws, size_t ws_bytes, void* stream);

/* B independent sequences (sessions), each with its own fp32 fast-weight
 * buffer over shared read-only weights.
 *   H, X0 [B][T][d]; O [B][T][d]; W_state [B][d][f] fp32 in/out: holds each
 *   sequence's W^(0) on entry (or is set from W_down0 when init_from_w0 = 1;
 *   W_down0 may be NULL otherwise) and W^(N) on exit.  Other arguments as in
 *   ttt_mlp_forward. */
ttt_status_t ttt_mlp_forward_batched(const ttt_mlp_desc_t* desc, const void* H, const void* X0,
                                     const void* W_gate, const void* W_up, const void* W_down0,
                                     const void* conv_taps, const void* W_target, void* O,
                                     float* W_state, void* ws, size_t ws_bytes, void* stream);

/* Reset fast-weight buffers: W_state[b] <- fp32(W_down0) for b < batch
 * (session start / periodic reset).  W_down0 [d][f] of w0_dtype; W_state
 * [batch][d][f] fp32.  Same validation and error rules as above (d, f >= 1). */
ttt_status_t ttt_fastweight_state_reset(float* W_state, const void* W_down0,
                                        ttt_dtype_t w0_dtype, int64_t batch, int64_t d_model,
                                        int64_t d_ff, void* stream);

/* ---- Streaming continuation (serving) ----
 * Feeds each of B sessions its tokens over consecutive calls, the way a
 * server reads a long context piece by piece (the page's future-work item on
 * streaming inference, section 9; per-session fast-weight buffers from the
 * practitioner blog's serving notes, section 4).  The final weight equals
 * that of one ttt_mlp_forward_batched call over the concatenated tokens bit
 * for bit, and so do the outputs, except those of decode calls (below), which
 * agree to rounding.
 *
 * The desc describes one call: seq_len = L >= 1 new tokens per session (the
 * same L for all B sessions), chunk = the sessions' chunk size C.  A call at
 * stream position pos (tokens each session has already fed) outputs the L
 * tokens' O rows.  A chunk's update needs the target of its last token, which
 * reads the next token's X0, so the chunk holding a call's last token stays
 * pending: its H and X0 rows (and the few X0 rows before it that the conv
 * reaches back to) go into the caller-owned carry, and the next call
 * re-enters them before its own tokens.  W_state therefore holds the weight
 * after every chunk before the pending one; a call with last = 1 closes the
 * streams (the final chunk is applied with the zero padding of the sequence's
 * end) and leaves the final weight.
 *   pos       tokens the sessions have fed before this call (0: the start;
 *             init_from_w0 = 1 then sets W_state from W_down0, otherwise
 *             init_from_w0 is ignored)
 *   last      1 for the closing call, else 0
 *   carry     ttt_mlp_carry_size(desc) bytes of device memory, 16-byte
 *             aligned, owned by the caller and kept between calls; read when
 *             pos > 0, written when last = 0 (may be NULL if pos = 0 and
 *             last = 1); its contents are opaque.  For bf16 it also holds a
 *             bf16 copy of every session's current weight (B*d_model*d_ff*2
 *             bytes), so W_state must not be changed between the calls of a
 *             stream.
 *   ws        ttt_mlp_stream_workspace_size(desc, 0) bytes (the minimum is
 *             ttt_mlp_stream_workspace_size(desc, 1))
 * A call costs the layer over the pending rows (at most C) plus the new ones,
 * except a decode call: bf16, last = 0, L <= 16 and B*L <= 64, with the new
 * rows staying inside the pending chunk (pos = 0 and L <= C, or fewer than C
 * tokens pending and pending + L <= C).  A decode call computes only the new
 * rows' outputs with the current weight (reading W_gate, W_up and the weight
 * copy once) and appends the rows to the carry; the pending chunk's update
 * comes with the first call that goes past it. */
size_t ttt_mlp_carry_size(const ttt_mlp_desc_t* desc);
size_t ttt_mlp_stream_workspace_size(const ttt_mlp_desc_t* desc, int64_t max_group);
ttt_status_t ttt_mlp_forward_stream(const ttt_mlp_desc_t* desc, int64_t pos, int32_t last,
                                    const void* H, const void* X0, const void* W_gate,
                                    const void* W_up, const void* W_down0, const void* conv_taps,
                                    const void* W_target, void* O, float* W_state, void* carry,
                                    void* ws, size_t ws_bytes, void* stream);

/* Ragged batches: the same call with each session's own position pos[b] and
 * closing flag last[b] (host arrays of B entries), as a server batching
 * sessions that joined and end at different times needs.  A slot whose
 * session closed may start a new one at pos 0 in the next call (its state is
 * set from W_down0 when init_from_w0 = 1, its carry restarts).  Sessions the
 * decode rule above admits are served together by the decode kernels; the
 * others by the full path, one pass per run of consecutive sessions with equal
 * position and flag.  ttt_mlp_forward_stream is this call with every pos[b] =
 * pos and last[b] = last.  ws as for ttt_mlp_forward_stream. */
ttt_status_t ttt_mlp_forward_stream_ragged(const ttt_mlp_desc_t* desc, const int64_t* pos,
                                           const int32_t* last, const void* H, const void* X0,
                                           const void* W_gate, const void* W_up,
                                           const void* W_down0, const void* conv_taps,
                                           const void* W_target, void* O, float* W_state,
                                           void* carry, void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the decode
 * form of ttt_mlp_forward_stream_ragged without a workspace argument.  It
 * serves only calls the decode kernels serve -- bf16, last[b] = 0 for every
 * session, at most 16 new rows per session and 64 in all, every session's new
 * rows inside its pending chunk, and B * L * d_ff * 2 <= 4 MiB -- and returns
 * TTT_ERR_UNSUPPORTED (nothing written) for any other call, which needs
 * ttt_mlp_forward_stream_ragged with a workspace.  Its outputs, state and
 * carry equal that call's bit for bit.  The gated activations go to a
 * library-owned static device buffer of 4 MiB, one per GPU, held until the
 * process ends; it calls no allocator.  All calls on one GPU share that
 * buffer: calls that overlap in time on one GPU (on different streams) race
 * and must be serialised by the caller.  Other arguments as for
 * ttt_mlp_forward_stream_ragged. */
ttt_status_t ttt_mlp_forward_stream_decode_noalloc(
    const ttt_mlp_desc_t* desc, const int64_t* pos, const int32_t* last, const void* H,
    const void* X0, const void* W_gate, const void* W_up, const void* W_down0,
    const void* conv_taps, const void* W_target, void* O, float* W_state, void* carry,
    void* stream);

/* ---- A share of a long sequence (context parallelism) ----
 * The chunk-wise update splits over devices (section 3.2, the note that
 * block-wise updates fit context parallelism): each device takes a
 * contiguous range of whole chunks of the sequences, computes the sum of its
 * own chunks' increments, one exclusive prefix sum over the devices gives
 * each its starting weight, and each then produces its outputs.  These two
 * calls are the per-device parts, on the device's share at its real shape;
 * the prefix sum between them (a collective across devices) is the
 * caller's.  With shares r = 0..R-1 of a sequence, S_r from
 * ttt_mlp_share_increment and W_state of share r set to
 * W_down0 + S_0 + ... + S_{r-1}, ttt_mlp_share_forward gives the outputs of
 * one ttt_mlp_forward_batched call over the whole sequence, and the last
 * share's W_state the final weight (equal up to fp32 summation order; the
 * bf16 weight slots may round differently where the fp32 sums differ).
 *
 * desc describes the share: seq_len = its T_r tokens of each of B
 * sequences, chunk = C (chunks are counted from the share's first token, so a
 * share must start on a chunk boundary of its sequence), and the other
 * fields as for the whole sequence.  H, X0 [B][T_r][d] are the share's rows.
 * The conv's window reaches outside the share; the rows it needs come in
 * ttt_share_t:
 *   X0_left   [B][7][d]: the 7 X0 rows before the share's first token (row 6
 *             is the token just before it); only the last K-2 (alignment
 *             NEXT) or K-1 (SELF) rows are read.  NULL when the share starts
 *             its sequences (zero padding).
 *   X0_right  [B][d]: the X0 row of the token after the share's last token
 *             (the last target looks one token ahead).  NULL when the share
 *             ends its sequences; when given, seq_len must be a multiple of
 *             chunk (the next share starts on a chunk boundary).
 * Both are device pointers, 16-byte aligned, and must not overlap outputs. */
typedef struct {
  const void* X0_left;
  const void* X0_right;
} ttt_share_t;

/* Step 1 of section 3.2 on one device: S [B][d][f] fp32 (overwritten) gets
 * eta * sum over the share's chunks of V^_iᵀ Z_i, the change the share makes
 * to each sequence's fast weight, computed without writing any weight slot.
 * ws: at least ttt_mlp_workspace_size(desc, 1) bytes; on return it holds the
 * share's activations (gated activations and targets in the scans' layouts)
 * for a following ttt_mlp_share_forward with reuse = 1.  W_down0 is not an
 * input: the sum does not depend on the weight. */
ttt_status_t ttt_mlp_share_increment(const ttt_mlp_desc_t* desc, const ttt_share_t* share,
                                     const void* H, const void* X0, const void* W_gate,
                                     const void* W_up, const void* conv_taps,
                                     const void* W_target, float* S, void* ws, size_t ws_bytes,
                                     void* stream);

/* Step 3 of section 3.2 on one device: the share's outputs O [B][T_r][d]
 * from W_state [B][d][f] fp32 (in/out: on entry the weight at the share's
 * first token -- W_down0 plus the increments of every earlier share --, on
 * exit the weight after the share).  reuse = 1: ws holds this share's
 * activations from the ttt_mlp_share_increment call just before it, made on
 * the same stream with the same desc, share rows and weights and not
 * modified since; S1 and S2 are then skipped.  reuse = 0 recomputes them.
 * ws as for ttt_mlp_forward_batched (its size sets the group; keep the same
 * buffer for reuse).  desc.init_from_w0 is ignored. */
ttt_status_t ttt_mlp_share_forward(const ttt_mlp_desc_t* desc, const ttt_share_t* share,
                                   int32_t reuse, const void* H, const void* X0,
                                   const void* W_gate, const void* W_up, const void* conv_taps,
                                   const void* W_target, void* O, float* W_state, void* ws,
                                   size_t ws_bytes, void* stream);

/* ---- Backward pass ----
 * Gradients of a loss L through the layer, given dO = dL/dO and (optionally)
 * dW_final = dL/dW_state after the call, for B sequences laid out as in
 * ttt_mlp_forward_batched.  The backward is the chain rule through the
 * forward the page defines (section 3.1 gated MLP, section 3.3 target and
 * update rule, section 3.2 chunk order): with S_j = dW_final +
 * sum_{m > j} dO_mᵀ Z_m,
 *   dZ_j = dO_j W^(j-1) + eta V^_j S_j,   dV^_j = eta Z_j S_jᵀ,
 *   dW_start = S_{-1},                    deta = sum_j <S_j, V^_jᵀ Z_j>,
 * then through SwiGLU, the projection and the conv.  The forward is
 * recomputed inside the call; S_j comes from the forward's streamed prefix
 * run over the chunks in reverse.
 *   W_down0 / W_start  the starting weight: W_down0 [d][f] (activation dtype)
 *             when init_from_w0 = 1, else W_start [B][d][f] fp32 per sequence
 *             (the other may be NULL)
 *   dO        [B][T][d] activation dtype;  dW_final [B][d][f] fp32 or NULL (0)
 * Outputs (overwritten):
 *   dH, dX0   [B][T][d] activation dtype
 *   dW_gate, dW_up [f][d], dtaps [d][K], dW_target [d][d]: fp32, summed over
 *             the batch (dtaps / dW_target may be NULL when the target has no
 *             conv / projection)
 *   dW_start  [B][d][f] fp32, the gradient of each sequence's starting weight
 *             (with init_from_w0 = 1 the gradient of W_down0 is their sum)
 *   d_eta     one fp32 value in device memory
 *   ws        ttt_mlp_backward_workspace_size(desc) bytes, 256-byte aligned
 * desc.mode is ignored.  Every product runs in the library's own MFMA kernels,
 * in ws; like the forward, the call keeps no state and allocates nothing. */
size_t ttt_mlp_backward_workspace_size(const ttt_mlp_desc_t* desc);
ttt_status_t ttt_mlp_backward_batched(
    const ttt_mlp_desc_t* desc, const void* H, const void* X0, const void* W_gate,
    const void* W_up, const void* W_down0, const float* W_start, const void* conv_taps,
    const void* W_target, const void* dO, const float* dW_final, void* dH, void* dX0,
    float* dW_gate, float* dW_up, float* dW_start, float* dtaps, float* dW_target, float* d_eta,
    void* ws, size_t ws_bytes, void* stream);

/* Message for the calling thread's last non-OK status ("" if none). */
const char* ttt_last_error(void);

/* ---- Stage timing (measurement support) ----
 * While enabled, every forward call records a HIP event pair around each
 * kernel it enqueues, on the caller's stream.  ttt_profile_read() waits for the
 * recorded events, writes per-stage totals (milliseconds and launch counts) for
 * up to max_stages stages, clears them, and returns the number of stages
 * (TTT_NUM_STAGES), or a negative ttt_status_t.  ttt_stage_name() names stage i:
 * 0 state_reset, 1 weight_prep, 2 pad_fill, 3 swiglu (S1), 4 target (S2),
 * 5 prefix_update (the first group's scan, S4/S5), 6 down_proj (the last
 * group's outputs, S3), 7 scan_apply (a group's scan next to the previous
 * group's outputs), 8 scan_target (the first group's scan next to the
 * projection of the later groups' tokens; with a projection and more than one
 * group, stage 4 then projects the first group's tokens only). */
#define TTT_NUM_STAGES 9
ttt_status_t ttt_profile_enable(int enable);
int ttt_profile_read(double* ms_total, int64_t* launches, int max_stages);
const char* ttt_stage_name(int stage);

#ifdef __cplusplus
}
#endif

#endif /* TTT_MLP_H */
