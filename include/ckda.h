/*
 * ckda.h -- C ABI of libckda.so: the Complex KDA (CKDA) token-mixing
 * recurrence on AMD Instinct MI355X (gfx950).
 *
 * The operation (per head; Complex KDA paper page, section 3 "CKDA."
 * paragraph, with DeltaNet's transition from section 2 "Linear RNNs"):
 *
 *     alpha_t = s_t * exp(g_t)          s_t in {+1,-1}^DK, g_t = log|alpha_t|
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *
 * S_t in R^{DK x DV} (row = key channel, column = value channel).  The gate
 * magnitude is passed in log space and the sign separately, and the running
 * product of the signs is pushed onto q and k inside the kernels, as the
 * "complex-kda-1.3B-100B" model card describes; callers always see the true
 * (signed) state unless a call says otherwise.  The pages' ranges are
 * alpha in [-1, 1] and beta in [0, 2] with unit-norm keys; the library does
 * not clamp or normalise anything.
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers (except cu_seqlens_host), dense
 *    and row-major in the layouts stated.  Token tensors: [B, T, H, D];
 *    per-head scalars: [B, T, H]; states: [B, H, DK, DV] float32.
 *  - The caller owns every buffer, the workspace included.  The library never
 *    allocates, frees, or keeps a pointer after the enqueued work is done.
 *  - Work is enqueued on `stream` and the call returns without waiting for it.
 *  - Every argument check runs before anything is enqueued.  On any error
 *    nothing is enqueued, no output is touched and a non-zero status is
 *    returned; ckda_last_error() then describes it (per calling thread).
 *    There is no fallback path: a shape or dtype the kernels do not support
 *    is an error (CKDA_ERR_UNSUPPORTED), never a silent substitute.
 *  - Supported head sizes: DK, DV in {32, 64, 128}.  Chunk length is 64.
 *  - Size limits (the kernels index chains, chunks and tokens in 32 bits):
 *    token-heads (B*T*H or T_total*H), chunk-heads and (sequence, head)
 *    states (B*H or N*H) must each stay below 2^31; larger problems fail
 *    with CKDA_ERR_UNSUPPORTED before anything is enqueued.
 *  - Outputs must not alias inputs (except the in/out decode state).
 *  - Gate range: g must be finite.  The forward and backward calls are exact
 *    over the pages' whole range (g <= 0, i.e. |alpha| <= 1, down to any
 *    magnitude): the intra-chunk products factor exp(b_r - b_i) through
 *    anchors inside each half chunk while every 16-token run of log-gates in
 *    every channel stays above about -66.5 (an average |alpha| above about
 *    0.016), and a chunk that leaves that range (or has any g > 0) is
 *    recomputed entry by entry with the exponent taken whole.  g > 0
 *    (|alpha| > 1) lies outside the pages' range; it is computed exactly
 *    while nothing overflows.
 */
#ifndef CKDA_H
#define CKDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CKDA_ABI_VERSION 12

/* Status codes and dtype codes travel as fixed-width integers (any value a
 * caller passes is well defined on both sides of the boundary; unknown
 * values are errors, not undefined behaviour). */
typedef int32_t ckda_status_t;
#define CKDA_OK 0
#define CKDA_ERR_NULL 1        /* a required pointer is NULL */
#define CKDA_ERR_SHAPE 2       /* a size is negative / inconsistent */
#define CKDA_ERR_DTYPE 3       /* unknown dtype code */
#define CKDA_ERR_UNSUPPORTED 4 /* valid request the kernels do not implement */
#define CKDA_ERR_SEQLENS 5     /* cu_seqlens not 0-based, monotone, ending at T */
#define CKDA_ERR_WORKSPACE 6   /* workspace missing or too small */
#define CKDA_ERR_HIP 7         /* the HIP runtime reported an error */

typedef int32_t ckda_dtype_t;
#define CKDA_F32 0
#define CKDA_BF16 1

/* Options of the forward, decode and backward calls (bitwise OR; 0 = the
 * defaults):
 *  CKDA_GATE_HEAD: one g and one s per (token, head) ([..., H]) instead of
 *      per key channel ([..., H, DK], the CKDA diagonal gate): a signed Gated
 *      DeltaNet (the "Scalar Gate" of the Complex KDA paper page, section 3),
 *      i.e. the channel gate with equal entries.  5 gate bytes per token-head
 *      instead of 640.
 *  CKDA_QK_L2NORM: q and k are normalised per (token, head) over the key
 *      channels, x / ||x|| (a zero vector stays zero), before the recurrence
 *      uses them; the unit keys the pages' stability ranges assume.  The
 *      backward returns gradients w.r.t. the raw q and k.
 *  CKDA_GATE_MAP: g and beta hold pre-activations x and y instead of the
 *      log-gate and beta, and s is not read (it may be NULL): the signed
 *      gate alpha = tanh(x), carried as g = log max(|alpha|, e^-4) and
 *      s = -1 where x < 0 (else +1), and beta = 2 sigmoid(y) in (0, 2).  A
 *      reading of the Complex KDA paper page, section 3 "CKDA." (gates in
 *      [-1, 1], beta in [0, 2], a signed gate with a magnitude floor after
 *      Sarrof et al. and Grazzi et al.), whose formulas and floor the pages
 *      do not carry; the floor e^-4 is this library's choice: it keeps every
 *      16-token run of log-gates inside the fast path's envelope.  The map
 *      runs inside the kernels' loads (no extra pass).  The backward then
 *      returns dg = dL/dx (the plain derivative; 0 on the floor) and
 *      dbeta = dL/dy. */
typedef uint32_t ckda_flags_t;
#define CKDA_GATE_CHANNEL 0u
#define CKDA_GATE_HEAD 1u
#define CKDA_QK_L2NORM 2u
#define CKDA_GATE_MAP 4u
/*  CKDA_CONV_SILU (the ckda_short_conv_* calls only, which accept no other
 *      flag): the convolution's output goes through SiLU, z sigmoid(z). */
#define CKDA_CONV_SILU 8u

/* opaque HIP stream (hipStream_t); NULL = the default stream */
typedef void* ckda_stream_t;

int ckda_abi_version(void);
const char* ckda_status_string(ckda_status_t status);
/* Message of the last failing call on this thread ("" if none). */
const char* ckda_last_error(void);

/* ------------------------------------------------------------------------
 * Gate / sign-fold prep (the first step of every chunk; exposed on its own
 * for testing).  Model card "complex-kda-1.3B-100B": |alpha| is carried in
 * log space and the +-1 part as a running product pushed onto q and k.
 * Per chunk of 64 tokens (the chunk restarts both scans):
 *     b_t  = sum of g over the chunk up to and including t      (float32)
 *     P_t  = product of s over the chunk up to and including t   (+-1)
 *     qf_t = P_t * q_t,  kf_t = P_t * k_t                        (exact)
 * q, k: [B,T,H,DK] in_dtype; g: [B,T,H,DK] f32; s: [B,T,H,DK] int8.
 * Outputs (all [B,T,H,DK]): b f32, p int8 (+-1), qf, kf in_dtype.
 * ---------------------------------------------------------------------- */
ckda_status_t ckda_chunk_prep(int B, int T, int H, int DK, ckda_dtype_t in_dtype,
                              const void* q, const void* k, const float* g, const int8_t* s,
                              float* b_out, int8_t* p_out, void* qf_out, void* kf_out,
                              ckda_stream_t stream);

/* ------------------------------------------------------------------------
 * Chunked forward over B equal-length sequences.
 *   q, k: [B,T,H,DK] in_dtype     v: [B,T,H,DV] in_dtype
 *   g: [B,T,H,DK] f32 (log|alpha|) s: [B,T,H,DK] int8 (+1/-1)
 *      (flags & CKDA_GATE_HEAD: g [B,T,H] f32, s [B,T,H] int8)
 *   beta: [B,T,H] f32             scale: output multiplier
 *   h0: [B,H,DK,DV] f32 or NULL (zero initial state)
 *   o: [B,T,H,DV] f32 (written)   ht: [B,H,DK,DV] f32 or NULL (final state)
 *   h_ckpt: [B,H,NT,DK,DV] f32 or NULL, NT = ceil(T/64): the state at the
 *           start of every chunk (checkpoints for ckda_bwd)
 *   workspace: ckda_fwd_workspace_bytes(B, T, H, DK, DV, in_dtype) bytes of
 *           device memory, 16-byte aligned, owned by the caller; the call
 *           overwrites it.  It carries one record per (chunk, head) from the
 *           chunk-local pass to the state pass, then room for the segmented
 *           state pass (below).  A smaller workspace that still holds the
 *           records is accepted, and the state pass then always walks whole
 *           sequences; less than that fails with CKDA_ERR_WORKSPACE.  Calls
 *           that share a workspace must be ordered on one stream.
 * The chunk-local pass runs over every (chunk, head) at once; the state
 * pass walks the chunks of each sequence.  When a few sequences are much
 * longer than the GPU has parallel work for, the state pass cuts them into
 * segments of G chunks (see ckda_set_segment_chunks): segment maps in
 * parallel, a short scan over the segments, then the segments from their
 * true start states.  Results agree with the whole-sequence pass to
 * rounding.
 * ---------------------------------------------------------------------- */
size_t ckda_fwd_workspace_bytes(int B, int T, int H, int DK, int DV, ckda_dtype_t in_dtype);
ckda_status_t ckda_fwd_chunked(int B, int T, int H, int DK, int DV, ckda_dtype_t in_dtype,
                               ckda_flags_t flags, const void* q, const void* k, const void* v,
                               const float* g, const int8_t* s, const float* beta, float scale,
                               const float* h0, float* o, float* ht, float* h_ckpt,
                               void* workspace, size_t workspace_bytes, ckda_stream_t stream);

/* ------------------------------------------------------------------------
 * ckda_fwd_chunked for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid device allocation.
 * Same arguments and results as ckda_fwd_chunked (whole-chain state pass),
 * without the workspace: the chunk records go to a fixed device array that
 * the library holds on every GPU it runs on until the process ends
 * (CKDA_NOALLOC_SCRATCH_BYTES = 160 MiB, e.g. B * ceil(T/64) * H = 1,024
 * chunk-heads of DK = DV = 128: one 4,096-token sequence of 16 heads).  A
 * call whose records need more (ckda_fwd_workspace_bytes without the
 * segment buffers) fails with CKDA_ERR_UNSUPPORTED before anything is
 * enqueued.  The call allocates nothing: the array's device address is
 * looked up once per device, on the first call there.  Every call on one GPU
 * shares the array, so calls that overlap in time on one GPU (other streams,
 * other threads) race and must be serialised by the caller.
 * ---------------------------------------------------------------------- */
#define CKDA_NOALLOC_SCRATCH_BYTES ((size_t)160 << 20)
ckda_status_t ckda_fwd_chunked_noalloc(int B, int T, int H, int DK, int DV, ckda_dtype_t in_dtype,
                                       ckda_flags_t flags, const void* q, const void* k, const void* v,
                                       const float* g, const int8_t* s, const float* beta, float scale,
                                       const float* h0, float* o, float* ht, float* h_ckpt,
                                       ckda_stream_t stream);

/* ------------------------------------------------------------------------
 * Segment length of the forward's state pass and of the backward's reverse
 * (state-gradient) pass, process-wide (all devices).
 * Per chunk the state map is affine, S' = A_c S + B_c, and the columns of
 * S evolve independently, so a long chain can be split into segments whose
 * maps (A and B composed over the segment) are built in parallel and then
 * chained by a scan: the single-GPU form of sequence sharding.
 *   G = 0   automatic (default): a cost model picks G, or whole chains;
 *   G < 0   never split;
 *   G >= 16 split every chain longer than G chunks into segments of G
 *           chunks (when the workspace has room).
 * 0 < G < 16 is rejected with CKDA_ERR_UNSUPPORTED.  Not synchronised with
 * calls in flight on other threads: set it before enqueueing work.
 * ---------------------------------------------------------------------- */
ckda_status_t ckda_set_segment_chunks(int G);

/* ------------------------------------------------------------------------
 * Varlen forward over N packed documents (training packs documents back to
 * back, "complex-kda-ladder" model card, tokenizer section).  Document n
 * covers tokens cu_seqlens[n] .. cu_seqlens[n+1]-1 of the packed tensors;
 * it starts from h0[n] (or zero) and its final state goes to ht[n].  No state
 * or sign product crosses a document boundary.
 *   cu_seqlens_host: int32 [N+1] in host memory, read during the call to
 *                    validate it (0-based, non-decreasing, ends at T_total)
 *   cu_seqlens_dev:  the same N+1 values in device memory, read by the kernel
 *   q, k, g, s: [T_total,H,DK]; v, o: [T_total,H,DV]; beta: [T_total,H]
 *   (flags & CKDA_GATE_HEAD: g, s [T_total,H])
 *   h0, ht: [N,H,DK,DV] f32, each nullable.  Documents may be empty (their
 *   ht is their h0, or zero).
 *   h_ckpt: nullable; else [ckda_varlen_chunk_slots(N, T_total), H, DK, DV]
 *           f32 receiving the true-frame state at the start of every chunk:
 *           chunk j of document n (tokens cu[n] + 64j ..) is chunk slot
 *           floor(cu[n] / 64) + n + j.  Slots no chunk maps to are not
 *           written.  (Checkpoints for ckda_bwd_varlen.)
 *   workspace: at least ckda_fwd_varlen_workspace_bytes(N, T_total, H, DK,
 *   DV, in_dtype) bytes, as for ckda_fwd_chunked.
 * ---------------------------------------------------------------------- */
int ckda_varlen_chunk_slots(int N, int T_total);
size_t ckda_fwd_varlen_workspace_bytes(int N, int T_total, int H, int DK, int DV, ckda_dtype_t in_dtype);
ckda_status_t ckda_fwd_varlen(int N, int T_total, const int32_t* cu_seqlens_host,
                              const int32_t* cu_seqlens_dev, int H, int DK, int DV,
                              ckda_dtype_t in_dtype, ckda_flags_t flags, const void* q, const void* k,
                              const void* v, const float* g, const int8_t* s, const float* beta,
                              float scale, const float* h0, float* o, float* ht, float* h_ckpt,
                              void* workspace,
                              size_t workspace_bytes, ckda_stream_t stream);

/* ------------------------------------------------------------------------
 * One recurrent (decode) step for N independent sequences.  The state is
 * carried in the folded frame: the true state is Diag(sign_prod) * state.
 * A prefill's final state enters as state = ht, sign_prod = +1.
 *   q, k: [N,H,DK] in_dtype;  v: [N,H,DV] in_dtype
 *   g, s: [N,H,DK] f32 / int8 (flags & CKDA_GATE_HEAD: [N,H]);  beta: [N,H] f32
 *   state: [N,H,DK,DV] f32, updated in place
 *   sign_prod: [N,H,DK] int8 (+1/-1), updated in place (times s; with the
 *              head gate every channel takes the head's s)
 *   o: [N,H,DV] f32
 * Each state element is read once and written once.
 * ---------------------------------------------------------------------- */
ckda_status_t ckda_decode_step(int N, int H, int DK, int DV, ckda_dtype_t in_dtype,
                               ckda_flags_t flags, const void* q, const void* k, const void* v, const float* g,
                               const int8_t* s, const float* beta, float scale, float* state,
                               int8_t* sign_prod, float* o, ckda_stream_t stream);

/* ------------------------------------------------------------------------
 * Backward of the chunked forward: gradients of L = <do, o> + <dht, ht>.
 *   inputs as in ckda_fwd_chunked; h0 nullable (zero)
 *   h_ckpt: [B,H,NT,DK,DV] f32 written by ckda_fwd_chunked on the same
 *           inputs, or NULL: the call then recomputes the checkpoints with
 *           one more forward pass (whole chains) into its workspace
 *   dout: [B,T,H,DV] in_dtype;  dht: [B,H,DK,DV] f32 or NULL (zero)
 *   dq, dk, dg: [B,T,H,DK] f32;  dv: [B,T,H,DV] f32;  dbeta: [B,T,H] f32
 *   (flags & CKDA_GATE_HEAD: g, s and dg are [B,T,H]; dg is then the sum
 *   over channels of the channel-gate gradient)
 *   dh0: [B,H,DK,DV] f32 or NULL
 *   workspace: ckda_bwd_workspace_bytes(...) bytes of device memory: per
 *           (chunk, head) the blocks of the chunk-parallel passes and the
 *           reverse pass's dU and chunk-end state gradient, then room for
 *           recomputed checkpoints, then the segment buffers of the reverse
 *           pass over long chains.  With h_ckpt given,
 *           ckda_bwd_workspace_bytes_given_ckpt(...) bytes suffice (the
 *           segment buffers take the checkpoint room's place); less is
 *           accepted down to the part before that room (the reverse pass then
 *           walks whole chains).
 * dg is the gradient w.r.t. g = log|alpha| (alpha * dL/dalpha); s gets none.
 * ---------------------------------------------------------------------- */
size_t ckda_bwd_workspace_bytes(int B, int T, int H, int DK, int DV);
size_t ckda_bwd_workspace_bytes_given_ckpt(int B, int T, int H, int DK, int DV);
ckda_status_t ckda_bwd(int B, int T, int H, int DK, int DV, ckda_dtype_t in_dtype,
                       ckda_flags_t flags, const void* q, const void* k, const void* v, const float* g,
                       const int8_t* s, const float* beta, float scale, const float* h0,
                       const float* h_ckpt, const void* dout, const float* dht,
                       float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dh0,
                       void* workspace, size_t workspace_bytes, ckda_stream_t stream);

/* The same backward reading the chunk records of the ckda_fwd_chunked call
 * that wrote h_ckpt on the same inputs and flags: fwd_workspace is that
 * call's workspace, unchanged since; its leading part holds the records, and
 * fwd_workspace_bytes must cover at least that part (the least the forward
 * itself accepts; less fails with CKDA_ERR_WORKSPACE).  The backward
 * then skips its own pass over the chunks that writes reverse records (the
 * reverse pass stages the forward's records transposed), trading the memory
 * the caller keeps between the two calls for that pass.  h_ckpt must be given.
 * Results agree with ckda_bwd's to rounding (the two record kinds round the
 * same quantities in different orders). */
ckda_status_t ckda_bwd_with_records(int B, int T, int H, int DK, int DV, ckda_dtype_t in_dtype,
                                    ckda_flags_t flags, const void* q, const void* k, const void* v,
                                    const float* g, const int8_t* s, const float* beta, float scale,
                                    const float* h0, const float* h_ckpt, const void* fwd_workspace,
                                    size_t fwd_workspace_bytes, const void* dout, const float* dht,
                                    float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dh0,
                                    void* workspace, size_t workspace_bytes, ckda_stream_t stream);

/* ------------------------------------------------------------------------
 * Backward of the varlen forward: per document n, gradients of
 * <do, o> + <dht[n], ht[n]> with documents as independent sequences.
 *   cu_seqlens_host / _dev, q .. beta, scale: as in ckda_fwd_varlen
 *   h_ckpt: the per-chunk-slot checkpoints ckda_fwd_varlen wrote on the same
 *           inputs, or NULL (recomputed, as in ckda_bwd)
 *   dout: [T_total,H,DV] in_dtype;  dht: [N,H,DK,DV] f32 or NULL (zero)
 *   dq, dk, dg: [T_total,H,DK] f32;  dv: [T_total,H,DV];  dbeta: [T_total,H]
 *   (flags & CKDA_GATE_HEAD: g, s, dg [T_total,H])
 *   dh0: [N,H,DK,DV] f32 or NULL
 *   workspace: ckda_bwd_varlen_workspace_bytes(...) bytes of device memory,
 *           or ckda_bwd_varlen_workspace_bytes_given_ckpt(...) with h_ckpt
 *           given
 * Conventions and errors as for ckda_bwd and ckda_fwd_varlen.
 * ---------------------------------------------------------------------- */
size_t ckda_bwd_varlen_workspace_bytes(int N, int T_total, int H, int DK, int DV);
size_t ckda_bwd_varlen_workspace_bytes_given_ckpt(int N, int T_total, int H, int DK, int DV);
ckda_status_t ckda_bwd_varlen(int N, int T_total, const int32_t* cu_seqlens_host,
                              const int32_t* cu_seqlens_dev, int H, int DK, int DV,
                              ckda_dtype_t in_dtype, ckda_flags_t flags, const void* q, const void* k,
                              const void* v, const float* g, const int8_t* s, const float* beta,
                              float scale, const float* h0, const float* h_ckpt, const void* dout,
                              const float* dht, float* dq, float* dk, float* dv, float* dg,
                              float* dbeta, float* dh0, void* workspace, size_t workspace_bytes,
                              ckda_stream_t stream);

/* ckda_bwd_varlen reading the records of the ckda_fwd_varlen call that wrote
 * h_ckpt (its workspace), as ckda_bwd_with_records does. */
ckda_status_t ckda_bwd_varlen_with_records(int N, int T_total, const int32_t* cu_seqlens_host,
                                           const int32_t* cu_seqlens_dev, int H, int DK, int DV,
                                           ckda_dtype_t in_dtype, ckda_flags_t flags, const void* q,
                                           const void* k, const void* v, const float* g, const int8_t* s,
                                           const float* beta, float scale, const float* h0,
                                           const float* h_ckpt, const void* fwd_workspace,
                                           size_t fwd_workspace_bytes, const void* dout, const float* dht,
                                           float* dq, float* dk, float* dv, float* dg, float* dbeta,
                                           float* dh0, void* workspace, size_t workspace_bytes,
                                           ckda_stream_t stream);

/* ------------------------------------------------------------------------
 * Short convolution: the optional width-4 part of the pre-mixer prep.  The
 * "complex-kda-1.3B-100B" model card lists a short convolution of width 4
 * among the layer's parts and nothing more; read here as a depthwise causal
 * convolution over tokens with one 4-tap filter per channel, applied to an
 * input of the mixer (q, k or v as [.., H*D] rows), optionally followed by
 * SiLU (CKDA_CONV_SILU):
 *     z_t[c] = sum_{j=0..3} w[c][j] x_{t-3+j}[c],   y_t = z_t or z_t sigmoid(z_t)
 * Before each sequence the history is zero, or the caller's window of the
 * three inputs that preceded it.
 *   Sequences: cu_seqlens_host and cu_seqlens_dev (both, [N+1], as in
 *           ckda_fwd_varlen), or both NULL for N equal sequences of T_total / N
 *           tokens (T_total a multiple of N)
 *   C: channels per token row, a multiple of 4 (H * D for a [.., H, D] tensor)
 *   x: [T_total][C] in_dtype;  w: [C][4] f32 (tap 3 takes the current token)
 *   state0: [N][3][C] in_dtype (x_{-3}, x_{-2}, x_{-1} of each sequence) or NULL
 *   y: [T_total][C] in_dtype (rounded to bf16 for bf16 inputs); must not
 *           overlap x
 *   state_out: [N][3][C] in_dtype or NULL: each sequence's last three inputs
 *           (its window rows where it is shorter than three), for a later
 *           call or ckda_short_conv_step; may be state0 itself (in place)
 * Every pointer 16-byte aligned.  Errors as for the mixer calls (host checks,
 * nothing enqueued on failure).
 * ---------------------------------------------------------------------- */
ckda_status_t ckda_short_conv_fwd(int N, int T_total, const int32_t* cu_seqlens_host,
                                  const int32_t* cu_seqlens_dev, int C, ckda_dtype_t in_dtype,
                                  ckda_flags_t flags, const void* x, const float* w, const void* state0,
                                  void* y, void* state_out, ckda_stream_t stream);

/* Backward of ckda_short_conv_fwd for an upstream gradient dy ([T_total][C]
 * f32): dx [T_total][C] f32, dw [C][4] f32 (summed in a fixed order: the
 * same inputs give the same bits), dstate0 [N][3][C] f32 or NULL.
 *   workspace: ckda_short_conv_bwd_workspace_bytes(T_total, C) bytes (per
 *           64-token run and channel, its part of dw). */
size_t ckda_short_conv_bwd_workspace_bytes(int T_total, int C);
ckda_status_t ckda_short_conv_bwd(int N, int T_total, const int32_t* cu_seqlens_host,
                                  const int32_t* cu_seqlens_dev, int C, ckda_dtype_t in_dtype,
                                  ckda_flags_t flags, const void* x, const float* w, const void* state0,
                                  const float* dy, float* dx, float* dw, float* dstate0, void* workspace,
                                  size_t workspace_bytes, ckda_stream_t stream);

/* One decode step of the convolution for N sequences: x, y [N][C] in_dtype,
 * window [N][3][C] in_dtype (the last three inputs), shifted in place to end
 * with x. */
ckda_status_t ckda_short_conv_step(int N, int C, ckda_dtype_t in_dtype, ckda_flags_t flags, const void* x,
                                   const float* w, void* window, void* y, ckda_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CKDA_H */
