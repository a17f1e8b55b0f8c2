/*
 * gdn.h -- Gated DeltaNet causal mixer for AMD Instinct MI355X (gfx950).
 *
 * The mixer is the linear-attention block that hybrid Qwen-style models run
 * in 48 of their 64 layers: a width-4 causal conv1d with SiLU over the
 * projected q|k|v channels, the gated delta rule, and a gated RMSNorm
 * (haskell-infer-demo README, "Highlights", hybrid-architecture bullet, and
 * "Architecture", kernels gdn_conv.cu, fla_gdn.cu and gdn_norm.cu).
 *
 * Gated delta rule, per sequence and v-head, with state S (d_v x d_k, fp32):
 *     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = scale S_t q_t,
 * a_t = exp(g_t), k_t and q_t L2-normalised when use_qk_l2norm is set.
 *
 * Conventions shared by every entry point
 *   - Every pointer is a DEVICE pointer unless marked (host).  The caller owns
 *     every buffer.  The library allocates nothing, keeps no pointer after a
 *     call returns, never synchronises and never copies device data to the
 *     host.  All work is enqueued on `stream` (a hipStream_t; NULL = the
 *     default stream).
 *   - Sizes are element counts.  Device buffers must be 16-byte aligned.
 *   - Arguments are checked on the host before anything is launched; a call
 *     that returns an error status has written nothing.
 *   - Sequence boundaries (cu_seqlens) and state slots are device data and are
 *     never read on the host: their contents are the caller's guarantee
 *     (cu_seqlens non-decreasing, cu_seqlens[0] = 0, cu_seqlens[n_seq] =
 *     t_total; active slots in range and unique).  This follows the prepared
 *     short-convolution interface of the Flare core-design page (packed
 *     prefill and single-token decode, caller-owned state, explicit slot
 *     mapping, inactive lanes that write no state, no CPU sequence-length
 *     extraction).
 *   - A negative state slot marks an inactive lane: nothing is read for it
 *     and nothing is written, neither state nor output rows.
 *   - Device faults surface at the caller's next synchronisation.
 *   - The library is thread-safe across streams.  Its host-side state is a
 *     thread-local last HIP error and caches filled on first use: the compute
 *     unit count of each device, the resident workgroups per compute unit of
 *     one kernel, the device address of the scratch array of
 *     gdn_chunk_fwd_noalloc on each device (which that entry point, and only
 *     it, shares between calls), and one side stream with two events per
 *     device, on which the chunk entry points run the one-token sequences of
 *     a multi-sequence or pooled call beside the scan (forked from and joined
 *     back into the caller's stream before the call's last kernel; not while
 *     the caller's stream is being captured, and never for
 *     gdn_chunk_fwd_noalloc).  They are held until the process ends.
 *
 * Layouts (row-major, last index fastest)
 *   conv input/output x, y   [t_total, channels], channels ordered q | k | v
 *   conv weights w           [channels, 4], w[c][3] multiplies the current token
 *   conv state               [slots, 3, channels], oldest token first (raw inputs)
 *   q, k                     [t_total, h_qk, d_k] with a token stride (elements)
 *   v                        [t_total, h_v, d_v] with a token stride (elements)
 *   g, beta                  [t_total, h_v] fp32 (log-decay and write strength)
 *   recurrent state          [slots or n_seq, h_v, d_v, d_k] fp32 (S k = v orientation)
 *   o, z, y                  [t_total, h_v, d_v] dense
 *   v-head h reads q/k head h / (h_v / h_qk).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t gdn_status;
#define GDN_OK 0
#define GDN_ERR_NULL 1        /* a required pointer is NULL */
#define GDN_ERR_INVALID 2     /* negative size, h_v % h_qk != 0, bad stride, t_total != n_seq in decode */
#define GDN_ERR_UNSUPPORTED 3 /* head dims / chunk / dtype combination not built */
#define GDN_ERR_ALIGN 4       /* a device pointer or stride breaks 16-byte alignment */
#define GDN_ERR_ALIAS 5       /* an output overlaps an input or another output */
#define GDN_ERR_WORKSPACE 6   /* workspace NULL or smaller than gdn_chunk_fwd_workspace_size */
#define GDN_ERR_HIP 7         /* a launch failed; see gdn_last_hip_error() */

typedef int32_t gdn_dtype;
#define GDN_F32 0
#define GDN_BF16 1

/*
 * gdn_conv1d_fwd -- causal depthwise conv1d of width 4, then SiLU.
 * (haskell-infer-demo README, "Architecture": native causal-conv1d of width 4;
 *  Flare core-design, short-convolution paragraph: raw projected QKV, dilation
 *  1, SiLU, raw input history; the speculative snapshot paragraph: three-token
 *  GDN convolution windows.)
 *
 * For sequence s (tokens cu_seqlens[s] .. cu_seqlens[s+1]-1 of x) with history
 * H = conv_state[slot(s)] (3 raw inputs, oldest first), the padded input is
 * [H; x_s] and output token t is
 *     y[t][c] = SiLU( sum_{i=0..3} w[c][i] * padded[t - start + i][c] ),
 * accumulated in fp32 and rounded once to dt.  Afterwards conv_state[slot(s)]
 * holds the last three rows of the padded input (a sequence shorter than 3
 * shifts its tokens in; a zero-length sequence leaves it bit-identical).
 *
 *   x           [t_total, channels] of dt (read)
 *   dt          GDN_BF16 or GDN_F32; w, conv_state and y use the same dtype
 *   w           [channels, 4] (read)
 *   channels    > 0, multiple of 8
 *   cu_seqlens  [n_seq + 1] int32, or NULL for decode: exactly one token per
 *               sequence, which requires t_total == n_seq
 *   conv_state  [n_slots, 3, channels], read and updated in place
 *   n_slots     number of rows of conv_state (>= n_seq when state_slots is NULL)
 *   state_slots [n_seq] int32 slot per sequence in [0, n_slots), NULL = identity
 *               (slot s); negative = inactive lane (its y rows and state untouched)
 *   y           [t_total, channels] (written); must not overlap x, w or conv_state
 * n_seq == 0 is a no-op.
 */
gdn_status gdn_conv1d_fwd(const void* x, gdn_dtype dt, const void* w, int32_t channels,
                          const int32_t* cu_seqlens, int32_t n_seq, int64_t t_total,
                          void* conv_state, int32_t n_slots, const int32_t* state_slots, void* y,
                          void* stream);

/*
 * gdn_chunk_fwd -- chunked prefill of the gated delta rule over packed sequences.
 * (Recurrence: the formula at the top of this header.  Chunked prefill and
 *  recurrent decode as in haskell-infer-demo README, "Architecture", fla_gdn.cu.
 *  FP32 recurrent state and BF16 intermediates, chunks relative to each call:
 *  Flare core-design, GDN numerics paragraph and Qwen defaults table.  Final
 *  state at the exact consumed length: Flare core-design, the paragraph on
 *  checkpoint endpoints, which are never rounded up to a token group.)
 *
 * Chunks of `chunk` tokens restart at every sequence start.  Within a chunk the
 * kernels use the UT/WY form (intra-chunk triangular solve, then contractions
 * with the fp32 state on the matrix cores); a call boundary that is a multiple
 * of `chunk` leaves results bit-identical to one longer call.
 *
 *   q, k        [t_total, h_qk, d_k] of dt, token stride q_stride / k_stride
 *   v           [t_total, h_v, d_v] of dt, token stride v_stride
 *               (strides in elements; 0 = dense; multiples of 8; at most 2^24)
 *   dt          GDN_BF16 (bf16 operands on the matrix cores, derived operands as
 *               bf16 hi+lo pairs, fp32 accumulation) or GDN_F32 (fp32 matrix cores)
 *   g, beta     [t_total, h_v] fp32: a_t = exp(g_t), write strength beta_t
 *   scale       output scale (1 for the plain rule; models often use d_k^-1/2)
 *   use_qk_l2norm  nonzero: q and k are replaced by x / sqrt(sum x^2 + l2_eps)
 *   (h_qk, h_v) h_v % h_qk == 0; (d_k, d_v, chunk): (128,128,64) for both
 *               dtypes, (16,16,16) for GDN_F32
 *   g           must be finite here (the chunk form takes differences of its
 *               running sums); a hard reset (g = -inf) is exact in gdn_recurrent_step
 *   cu_seqlens  [n_seq + 1] int32; NULL allowed only when n_seq == 1
 *   initial_state [n_seq, h_v, d_v, d_k] fp32 or NULL (zeros)
 *   final_state [n_seq, h_v, d_v, d_k] fp32 or NULL (not wanted); may equal
 *               initial_state exactly (updated in place), no partial overlap.
 *               final_state[s] is the state after exactly len(s) tokens.
 *   o           [t_total, h_v, d_v] of o_dt (GDN_F32 or GDN_BF16): the outputs,
 *               or with z != NULL the gated RMSNorm of the outputs (epilogue)
 *   z           NULL, or [t_total, h_v, d_v] of dt: gate of the gated RMSNorm
 *               y = o / sqrt(mean_dv(o^2) + norm_eps) * norm_w * SiLU(z)
 *   norm_w      [d_v] fp32, required when z != NULL
 *   workspace   device scratch of ws_bytes >= gdn_chunk_fwd_workspace_size(...);
 *               its contents need no initialisation and are not preserved
 * n_seq == 0 is a no-op.  Zero-length sequences are legal: their final state
 * equals their initial state (or zeros).  With t_total == 0 the per-token
 * buffers (q, k, v, g, beta, o, z) may be NULL; the final states are still
 * written.
 */
gdn_status gdn_chunk_fwd(const void* q, const void* k, const void* v,
                         int64_t q_stride, int64_t k_stride, int64_t v_stride, gdn_dtype dt,
                         const float* g, const float* beta, float scale,
                         int32_t use_qk_l2norm, float l2_eps,
                         int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, int32_t chunk,
                         const int32_t* cu_seqlens, int32_t n_seq, int64_t t_total,
                         const float* initial_state, float* final_state,
                         void* o, gdn_dtype o_dt,
                         const void* z, const float* norm_w, float norm_eps,
                         void* workspace, size_t ws_bytes, void* stream);

/*
 * gdn_chunk_fwd_noalloc -- gdn_chunk_fwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.
 *
 * Every argument and result is as for gdn_chunk_fwd, except that there is no
 * workspace argument: the call uses a library-owned device array of
 * GDN_NOALLOC_SCRATCH_BYTES on the current device instead, and allocates
 * nothing (no hipMalloc, no hipFree, no allocating library routine).  The
 * array is placed on each device when the library's code object is first
 * loaded there and is held until the process ends; its address is looked up
 * on the first call on each device.  The kernels need no initialised
 * contents, so nothing is cleared between calls.
 *
 * A call whose workspace (gdn_chunk_fwd_workspace_size for the same
 * arguments) exceeds GDN_NOALLOC_SCRATCH_BYTES returns GDN_ERR_WORKSPACE and
 * writes nothing.  All calls on one device share that device's array: two
 * calls that overlap in time on one device (different streams, threads or
 * processes' copies aside) race and give undefined results, so the caller
 * orders them, e.g. on one stream.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

gdn_status gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                 int64_t q_stride, int64_t k_stride, int64_t v_stride, gdn_dtype dt,
                                 const float* g, const float* beta, float scale,
                                 int32_t use_qk_l2norm, float l2_eps,
                                 int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, int32_t chunk,
                                 const int32_t* cu_seqlens, int32_t n_seq, int64_t t_total,
                                 const float* initial_state, float* final_state,
                                 void* o, gdn_dtype o_dt,
                                 const void* z, const float* norm_w, float norm_eps, void* stream);

/*
 * gdn_chunk_fwd_workspace_size -- (host) bytes of workspace gdn_chunk_fwd needs.
 * An upper bound computed from capacities only (n_seq and t_total), so one
 * allocation serves every call with the same or smaller capacities.
 * with_norm: nonzero if the call will pass z.  Writes *bytes on success.
 */
gdn_status gdn_chunk_fwd_workspace_size(int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v,
                                        int32_t chunk, int32_t n_seq, int64_t t_total,
                                        gdn_dtype dt, int32_t with_norm, size_t* bytes /* host */);

/*
 * gdn_recurrent_step -- one decode token per request, state updated in place.
 * (The recurrence at the top of this header applied to a single token; upstream
 *  recurrent decode: haskell-infer-demo README, "Architecture", fla_gdn.cu;
 *  FP32 recurrent state: Flare core-design, Qwen defaults table.)
 *
 * Each (request, v-head) state of d_v x d_k fp32 is streamed once through
 * registers: read, decayed, corrected by the delta rule, used for the output
 * and written back.
 *
 *   q, k, v, strides, dt, g, beta, scale, use_qk_l2norm, l2_eps, h_qk, h_v,
 *   d_k, d_v: as gdn_chunk_fwd with t_total = n_req; (d_k, d_v) in {(16,16), (128,128)}
 *   state       [n_slots, h_v, d_v, d_k] fp32, read and written in place
 *   n_slots     number of state entries (>= n_req when state_slots is NULL)
 *   state_slots [n_req] int32 slot per request in [0, n_slots), NULL = identity;
 *               negative = inactive lane (reads nothing, writes nothing, o rows
 *               untouched)
 *   o           [n_req, h_v, d_v] of o_dt; with z != NULL the gated RMSNorm output
 *   z, norm_w, norm_eps: as gdn_chunk_fwd
 * n_req == 0 is a no-op.
 */
gdn_status gdn_recurrent_step(const void* q, const void* k, const void* v,
                              int64_t q_stride, int64_t k_stride, int64_t v_stride, gdn_dtype dt,
                              const float* g, const float* beta, float scale,
                              int32_t use_qk_l2norm, float l2_eps,
                              int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, int32_t n_req,
                              float* state, int32_t n_slots, const int32_t* state_slots,
                              void* o, gdn_dtype o_dt,
                              const void* z, const float* norm_w, float norm_eps, void* stream);

/*
 * gdn_chunk_fwd_gated, gdn_recurrent_step_gated -- gdn_chunk_fwd and
 * gdn_recurrent_step with the gate preparation fused into their prologues.
 * (The GDN mixer's B/A gate projections: Flare core-design, the paragraph on
 *  fused projection weights.  The pages give no formula for the gates; the
 *  reading used here is the one that yields a log-decay g < 0 and a write
 *  strength beta in (0, 1).)
 *
 * Instead of fp32 g and beta, each call reads the raw gate projections and
 * forms, per token row t and v-head h, in fp32:
 *     g[t,h]    = -exp(a_log[h]) * softplus(a[t,h] + dt_bias[h])
 *     beta[t,h] = sigmoid(b[t,h])
 * No g or beta tensor is written or needed.  Every other argument, the
 * workspace (gdn_chunk_fwd_workspace_size) and every status are as for the
 * unfused entry point.
 *
 *   a, b        rows of the gate projections: element (t, h) at a[t * ab_stride + h]
 *               (b likewise), [t_total or n_req rows] of ab_dt; only element
 *               alignment is required, so a and b may be the two halves of one
 *               packed [rows, 2 h_v] tensor
 *   ab_stride   row stride of a and b in elements; 0 = h_v; must be >= h_v
 *   ab_dt       GDN_BF16 or GDN_F32
 *   a_log       [h_v] fp32 (4-byte aligned), required
 *   dt_bias     [h_v] fp32 (4-byte aligned), or NULL for a zero bias
 * With t_total == 0 (chunk) a and b may be NULL; a_log is always required.
 */
gdn_status gdn_chunk_fwd_gated(const void* q, const void* k, const void* v,
                               int64_t q_stride, int64_t k_stride, int64_t v_stride, gdn_dtype dt,
                               const void* a, const void* b, int64_t ab_stride, gdn_dtype ab_dt,
                               const float* a_log, const float* dt_bias, float scale,
                               int32_t use_qk_l2norm, float l2_eps,
                               int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, int32_t chunk,
                               const int32_t* cu_seqlens, int32_t n_seq, int64_t t_total,
                               const float* initial_state, float* final_state,
                               void* o, gdn_dtype o_dt,
                               const void* z, const float* norm_w, float norm_eps,
                               void* workspace, size_t ws_bytes, void* stream);

gdn_status gdn_recurrent_step_gated(const void* q, const void* k, const void* v,
                                    int64_t q_stride, int64_t k_stride, int64_t v_stride, gdn_dtype dt,
                                    const void* a, const void* b, int64_t ab_stride, gdn_dtype ab_dt,
                                    const float* a_log, const float* dt_bias, float scale,
                                    int32_t use_qk_l2norm, float l2_eps,
                                    int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, int32_t n_req,
                                    float* state, int32_t n_slots, const int32_t* state_slots,
                                    void* o, gdn_dtype o_dt,
                                    const void* z, const float* norm_w, float norm_eps, void* stream);

/*
 * gdn_recurrent_verify -- speculative verification: n_tok tokens per request
 * from the live state, the state after each token kept in a checkpoint column.
 * (Flare core-design, speculative target state: eight recurrent checkpoint
 *  columns per request, and a round writes the columns of its verification
 *  inputs; the recurrence is the one at the top of this header.)
 *
 * Request r's tokens are rows r * n_tok + t (t = 0 .. n_tok - 1) of q, k, v,
 * g, beta, z and o.  The live state[state_slots[r]] is only read; the state
 * after token t is written to checkpoints[state_slots[r]][t].  Installing an
 * accepted prefix of a tokens is gdn_state_rows_copy of column a - 1 into the
 * live slot.
 *
 *   q, k, v, strides, dt, g, beta, scale, use_qk_l2norm, l2_eps, h_qk, h_v,
 *   d_k, d_v: as gdn_recurrent_step, over n_req * n_tok token rows
 *   n_tok       verification tokens per request, 1 <= n_tok <= n_cols
 *   state       [n_slots, h_v, d_v, d_k] fp32 live states (read only)
 *   state_slots [n_req] int32 slot per request, NULL = identity; negative =
 *               inactive lane (reads nothing, writes nothing, o rows untouched)
 *   checkpoints [n_slots, n_cols, h_v, d_v, d_k] fp32; columns 0 .. n_tok - 1 of
 *               each active slot are written
 *   o           [n_req * n_tok, h_v, d_v] of o_dt (the gated RMSNorm of the
 *               outputs when z != NULL)
 * n_req == 0 is a no-op.  Errors as gdn_recurrent_step; n_tok < 1 or
 * n_tok > n_cols is GDN_ERR_INVALID.
 */
gdn_status gdn_recurrent_verify(const void* q, const void* k, const void* v,
                                int64_t q_stride, int64_t k_stride, int64_t v_stride, gdn_dtype dt,
                                const float* g, const float* beta, float scale,
                                int32_t use_qk_l2norm, float l2_eps,
                                int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v,
                                int32_t n_req, int32_t n_tok,
                                const float* state, int32_t n_slots, const int32_t* state_slots,
                                float* checkpoints, int32_t n_cols,
                                void* o, gdn_dtype o_dt,
                                const void* z, const float* norm_w, float norm_eps, void* stream);

/*
 * gdn_conv1d_verify -- the width-4 conv + SiLU of a speculative verification
 * round: n_tok tokens per request from the live history, which is only read,
 * with the 3-token history after each token kept as that column's window.
 * (Flare core-design, speculative target state: a snapshot copies a column's
 *  three-token GDN convolution window.)
 *
 *   x, y        [n_req * n_tok, channels] of dt (request r: rows r * n_tok + t)
 *   w, channels as gdn_conv1d_fwd
 *   conv_state  [n_slots, 3, channels] of dt, the live histories (read only)
 *   state_slots [n_req] int32 or NULL (identity); negative = inactive lane
 *   windows     [n_slots, n_cols, 3, channels] of dt: windows[slot][t] is the
 *               history after token t (its last three raw inputs, oldest
 *               first); columns 0 .. n_tok - 1 of each active slot are written
 * n_req == 0 is a no-op; 1 <= n_tok <= n_cols.
 */
gdn_status gdn_conv1d_verify(const void* x, gdn_dtype dt, const void* w, int32_t channels,
                             int32_t n_req, int32_t n_tok, const void* conv_state, int32_t n_slots,
                             const int32_t* state_slots, void* y, void* windows, int32_t n_cols,
                             void* stream);

/*
 * gdn_state_rows_copy -- indirect row copy for state maintenance: for each
 * entry e < n, row dst_rows[e] of dst becomes a copy of row src_rows[e] of src,
 * or zeros when src is NULL.  (Flare core-design, prepared state operations:
 * initialize, restore, snapshot and reset are indirect copy kernels driven by
 * device-resident slot-index buffers.)
 *
 * A row is a block of row_bytes (a multiple of 16) at dst + row * row_bytes:
 * a recurrent state slot (h_v * d_v * d_k * 4 bytes), one checkpoint column
 * (row slot * n_cols + column of the checkpoint array), a conv history
 * (3 * channels * element bytes) or one window.  The copy is bit-exact.
 *
 *   dst, n_dst_rows   destination buffer of n_dst_rows rows (16-byte aligned)
 *   dst_rows          [n] int32 destination rows (device)
 *   src, n_src_rows   source buffer of n_src_rows rows, or NULL (zero fill)
 *   src_rows          [n] int32 source rows (device); required when src != NULL
 * An entry whose destination or source row lies outside [0, rows) of its
 * buffer is skipped.  src may be dst itself (copies between rows of one
 * pool); other overlaps are GDN_ERR_ALIAS.  The caller guarantees that no row
 * is written by two entries or written by one entry and read by another.
 * n == 0 is a no-op.
 */
gdn_status gdn_state_rows_copy(void* dst, int64_t n_dst_rows, const int32_t* dst_rows,
                               const void* src, int64_t n_src_rows, const int32_t* src_rows,
                               int64_t row_bytes, int32_t n, void* stream);

/*
 * gdn_conv1d_mixed, gdn_chunk_mixed -- the mixed prefill-plus-decode form of
 * gdn_conv1d_fwd and gdn_chunk_fwd for a serving batch: prompt chunks and
 * single decode tokens packed into one call over caller-owned state pools.
 * (Flare core-design, the short-convolution paragraph and its prepared
 *  interface list: caller-owned state, explicit request-to-state-slot
 *  mapping, a fresh-state flag, device-resident sequence and token counts,
 *  fixed token and sequence capacities, a mixed prefill-plus-decode mode,
 *  inactive lanes that write no state; the state-maintenance paragraph:
 *  padding changes capacity, never logical length, and padded rows take no
 *  part in convolution or recurrent updates.)
 *
 * The host passes capacities only: n_seq is the sequence capacity and
 * t_total the token capacity of the packed buffers.  The live counts are
 * device data: cu_seqlens[n_seq] <= t_total is the number of live token rows
 * (rows past it are padding and keep their contents in every output), and a
 * padded sequence has length 0 and slot -1.  A decode token is a sequence of
 * length 1.  For sequence s with slot p = state_slots[s] >= 0:
 *   - its history / state is zero when fresh[s] != 0 (the pool row is not
 *     read), else conv_state[p] / state[p];
 *   - its rows are computed as by gdn_conv1d_fwd / gdn_chunk_fwd;
 *   - conv_state[p] / state[p] receive its history / state after exactly
 *     len(s) tokens (zero-length: the initial value, zeros when fresh).
 * A sequence with p < 0 is an inactive lane: nothing is read or written for
 * it, and its rows of y / o keep their contents.
 *
 *   gdn_conv1d_mixed: x, dt, w, channels, conv_state, n_slots, y as
 *               gdn_conv1d_fwd; cu_seqlens [n_seq + 1] and state_slots [n_seq]
 *               int32 required; fresh [n_seq] int32 or NULL (none fresh)
 *   gdn_chunk_mixed: q, k, v, strides, dt, g, beta, scale, use_qk_l2norm,
 *               l2_eps, head sizes, chunk, o, o_dt, z, norm_w, norm_eps and
 *               workspace as gdn_chunk_fwd (workspace sized by
 *               gdn_chunk_fwd_workspace_size for the capacities);
 *               state [n_slots, h_v, d_v, d_k] fp32, read and written in place;
 *               cu_seqlens, state_slots required, fresh optional (as above)
 * Active slots must be distinct (caller's guarantee, like the contents of
 * cu_seqlens).  n_seq == 0 is a no-op.  Statuses as the plain entry points;
 * a missing cu_seqlens, state_slots or state is GDN_ERR_NULL.
 */
gdn_status gdn_conv1d_mixed(const void* x, gdn_dtype dt, const void* w, int32_t channels,
                            const int32_t* cu_seqlens, int32_t n_seq, int64_t t_total,
                            void* conv_state, int32_t n_slots, const int32_t* state_slots,
                            const int32_t* fresh, void* y, void* stream);

gdn_status gdn_chunk_mixed(const void* q, const void* k, const void* v,
                           int64_t q_stride, int64_t k_stride, int64_t v_stride, gdn_dtype dt,
                           const float* g, const float* beta, float scale,
                           int32_t use_qk_l2norm, float l2_eps,
                           int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, int32_t chunk,
                           const int32_t* cu_seqlens, int32_t n_seq, int64_t t_total,
                           float* state, int32_t n_slots, const int32_t* state_slots, const int32_t* fresh,
                           void* o, gdn_dtype o_dt,
                           const void* z, const float* norm_w, float norm_eps,
                           void* workspace, size_t ws_bytes, void* stream);

/*
 * gdn_chunk_bwd -- gradients of the gated delta rule over packed sequences
 * (the backward pass for training).  (Recurrence: the formula at the top of
 * this header, as in gdn_chunk_fwd; gradients from the states at chunk
 * boundaries: haskell-infer-demo README, the FLA-derived chunked GDN kernels,
 * and Flare core-design, the chunk-boundary checkpoint paragraph.)
 *
 * For L = sum(d_o * o) + sum(d_final * S_T), with o and S_T what gdn_chunk_fwd
 * returns for the same inputs (no norm epilogue), writes dL/dq, dL/dk (through
 * the L2 normalisation when use_qk_l2norm), dL/dv, dL/dg, dL/dbeta and
 * dL/d(initial_state).  bf16 inputs with d_k = d_v = 128 run the chunked
 * form on the matrix cores: a forward pass writes the state entering every
 * 64-token chunk, a reverse pass over the chunks carries the state gradient
 * (and writes dv), then one pass per (chunk, v-head) forms the other
 * gradients from the chunk algebra; contractions take derived operands as
 * bf16 hi+lo pairs with fp32 accumulation.  fp32 inputs run a token-by-token
 * fp32 reverse chain from checkpoints every 16 tokens.  Sums run in a fixed
 * order (bitwise reproducible).
 *
 *   q, k, v, strides, dt, g, beta, scale, use_qk_l2norm, l2_eps, h_qk, h_v,
 *   cu_seqlens, n_seq, t_total, initial_state: as gdn_chunk_fwd;
 *               (d_k, d_v) = (128, 128) (bf16 or fp32) or (16, 16) (fp32)
 *   d_o         [t_total, h_v, d_v] fp32: gradient of the outputs
 *   d_final     [n_seq, h_v, d_v, d_k] fp32, or NULL (zero)
 *   dq, dk      [t_total, h_qk, d_k] fp32 (written)
 *   dv          [t_total, h_v, d_v] fp32 (written)
 *   dg, dbeta   [t_total, h_v] fp32 (written)
 *   d_initial   [n_seq, h_v, d_v, d_k] fp32, or NULL (not wanted)
 *   workspace   ws_bytes >= gdn_chunk_bwd_workspace_size(...); no
 *               initialisation needed, contents not preserved
 * n_seq == 0 is a no-op.  Outputs must not overlap inputs, each other or the
 * workspace (GDN_ERR_ALIAS).  Other statuses as gdn_chunk_fwd.
 */
gdn_status gdn_chunk_bwd(const void* q, const void* k, const void* v,
                         int64_t q_stride, int64_t k_stride, int64_t v_stride, gdn_dtype dt,
                         const float* g, const float* beta, float scale,
                         int32_t use_qk_l2norm, float l2_eps,
                         int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v,
                         const int32_t* cu_seqlens, int32_t n_seq, int64_t t_total,
                         const float* initial_state, const float* d_o, const float* d_final,
                         float* dq, float* dk, float* dv, float* dg, float* dbeta, float* d_initial,
                         void* workspace, size_t ws_bytes, void* stream);

/*
 * gdn_chunk_bwd_workspace_size -- (host) bytes of workspace gdn_chunk_bwd
 * needs: the block-boundary states ((t_total / 16 + n_seq) x h_v x d_v x d_k
 * fp32) and the per-slice partial sums of dq, dk, dbeta, dg.
 */
gdn_status gdn_chunk_bwd_workspace_size(int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, int32_t n_seq,
                                        int64_t t_total, size_t* bytes /* host */);

/*
 * gdn_conv1d_bwd -- gradients of gdn_conv1d_fwd (width-4 causal conv + SiLU over
 * packed sequences) for training.  (The conv and its raw-input history:
 * haskell-infer-demo README, "Architecture"; Flare core-design,
 * short-convolution paragraph.)
 *
 * For L = sum(dy * y) + sum(d_state_out * state_out), with y and state_out
 * what gdn_conv1d_fwd computes from x, w and the history conv_state_in (the
 * rounding of y to dt is not differentiated), writes dL/dx, dL/dw and
 * dL/d(conv_state_in).  fp32 arithmetic; dw sums per-block partials in a fixed
 * order (bitwise reproducible).
 *
 *   x, dt, w, channels, cu_seqlens, n_seq, t_total: as gdn_conv1d_fwd (packed
 *               prefill; cu_seqlens may be NULL only when n_seq == 1)
 *   conv_state_in [n_seq, 3, channels] of dt (per sequence, oldest first), or
 *               NULL (zeros)
 *   dy          [t_total, channels] fp32
 *   d_state_out [n_seq, 3, channels] fp32, or NULL (zero)
 *   dx          [t_total, channels] fp32 (written)
 *   dw          [channels, 4] fp32 (written)
 *   d_state_in  [n_seq, 3, channels] fp32, or NULL (not wanted)
 *   workspace   ws_bytes >= gdn_conv1d_bwd_workspace_size(...)
 * n_seq == 0 is a no-op.  Outputs must not overlap inputs or each other.
 */
gdn_status gdn_conv1d_bwd(const void* x, gdn_dtype dt, const void* w, int32_t channels,
                          const int32_t* cu_seqlens, int32_t n_seq, int64_t t_total,
                          const void* conv_state_in, const float* dy, const float* d_state_out,
                          float* dx, float* dw, float* d_state_in,
                          void* workspace, size_t ws_bytes, void* stream);

/* gdn_conv1d_bwd_workspace_size -- (host) bytes of workspace gdn_conv1d_bwd needs. */
gdn_status gdn_conv1d_bwd_workspace_size(int32_t channels, int32_t n_seq, int64_t t_total,
                                         size_t* bytes /* host */);

/*
 * gdn_mixer_decode_step -- one decode token of the mixer in one launch: the
 * width-4 conv step with SiLU over the raw projected q|k|v, then the gated
 * delta rule step and, with z, the gated RMSNorm.
 * (Conv: haskell-infer-demo README, "Architecture", and Flare core-design,
 *  short-convolution paragraph; recurrence: the formula at the top of this
 *  header; norm: haskell-infer-demo README, "Highlights".)
 *
 * The results are bit-identical to gdn_conv1d_fwd in decode form (cu_seqlens
 * NULL) into a [n_req, channels] buffer of dt, followed by gdn_recurrent_step
 * on the q, k and v column blocks of that buffer: the conv output is rounded
 * to dt exactly as that buffer would hold it, and the recurrence and norm use
 * the same arithmetic.  The conv output itself is not written.  One workgroup
 * per (request, q/k head) does the conv of the channels it owns and then the
 * recurrent step of the h_v / h_qk v-heads that read that q/k head.
 *
 *   x           [n_req, channels] of dt, channels = 2 h_qk d_k + h_v d_v: the
 *               raw projected q | k | v of one token per request (read)
 *   conv_w      [channels, 4] of dt (read)
 *   conv_state  [n_slots, 3, channels] of dt, updated in place
 *   g, beta, scale, use_qk_l2norm, l2_eps, h_qk, h_v: as gdn_recurrent_step
 *   d_k, d_v    128 and 128; h_v / h_qk at most 8
 *   state       [n_slots, h_v, d_v, d_k] fp32, updated in place
 *   n_slots     rows of conv_state and of state (>= n_req when state_slots is NULL)
 *   state_slots [n_req] int32 slot per request into both conv_state and state,
 *               in [0, n_slots); NULL = identity; negative = inactive lane
 *               (nothing read or written, o rows untouched)
 *   o, o_dt, z, norm_w, norm_eps: as gdn_recurrent_step
 * o must not overlap any input; conv_state and state must not overlap each
 * other or the inputs.  n_req == 0 is a no-op.  Other d_k, d_v or a larger
 * group return GDN_ERR_UNSUPPORTED (the two-call form covers them).
 */
gdn_status gdn_mixer_decode_step(const void* x, gdn_dtype dt, const void* conv_w, void* conv_state,
                                 const float* g, const float* beta, float scale,
                                 int32_t use_qk_l2norm, float l2_eps,
                                 int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v, int32_t n_req,
                                 float* state, int32_t n_slots, const int32_t* state_slots,
                                 void* o, gdn_dtype o_dt,
                                 const void* z, const float* norm_w, float norm_eps, void* stream);

/*
 * gdn_gated_rmsnorm -- y = x / sqrt(mean(x^2) + eps) * w * SiLU(z), per row of d.
 * (The gated RMSNorm of the GDN layers: haskell-infer-demo README,
 *  "Highlights", hybrid-architecture bullet, and "Architecture", gdn_norm.cu;
 *  distinct from the GemmaRMSNorm of flashinfer_norm.cu.)
 *
 *   x   [rows, d] of x_dt (GDN_F32 or GDN_BF16)
 *   z   [rows, d] of z_dt
 *   w   [d] fp32
 *   y   [rows, d] of y_dt; may equal x exactly when x_dt == y_dt (in place)
 *   d in {16, 128}.  rows == 0 is a no-op.
 */
gdn_status gdn_gated_rmsnorm(const void* x, gdn_dtype x_dt, const void* z, gdn_dtype z_dt,
                             const float* w, float eps, int64_t rows, int32_t d,
                             void* y, gdn_dtype y_dt, void* stream);

/* (host) Name of a status code; never NULL. */
const char* gdn_status_string(gdn_status status);

/* (host) hipError_t of the last failed launch on this thread (0 if none). */
int32_t gdn_last_hip_error(void);

/* (host) Library version string. */
const char* gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
