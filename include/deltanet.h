/*
 * deltanet.h -- C ABI of the MI355X (gfx950) delta-rule sequence mixer.
 *
 * The operation (all pages cited are the three web pages this library restates):
 *
 *   Per (sequence, value head) the state S is a d_v x d_k matrix mapping keys to
 *   values.  Each token t updates it by the delta rule of the frankenstein
 *   "DeltaNet Attention" page (module docstring) -- equivalently the error-
 *   correcting form of the mutichung garden "DeltaNet" page, section "The Delta
 *   Rule" -- after first decaying it by the gate of the nnterp "linear_attention"
 *   page (LinearAttention class text; "decays" is the log of the fraction kept):
 *
 *       S'_t = exp(g_t) S_{t-1}
 *       S_t  = S'_t - beta_t (S'_t k_t - v_t) k_t^T
 *       o_t  = scale * S_t q_t                      (read after the write)
 *
 *   With g absent the decay factor is 1 (the plain delta rule).  With DN_GATE_PER_KEY
 *   the gate is taken per key channel (the nnterp page's ChannelGates, [batch, seq,
 *   heads, key_dim], the KDA variant): S'_t = S_{t-1} diag(exp(g_t)), key channel i of
 *   the state keeping exp(g_t[i]).  beta may lie in
 *   (0, 1), or in (0, 2) for the negative-eigenvalue variant (nnterp "betas"); any
 *   real beta is computed as given.  q and k are L2-normalised before the rule (the
 *   frankenstein class text; the "L2 Norm" box right before the "Delta Rule" box of
 *   the mutichung DeltaNet block flowchart): either by the caller (the default), or
 *   inside the call when shape->flags has DN_QK_L2NORM, which replaces every q_t
 *   and k_t by x / sqrt(sum_i x_i^2 + l2norm_eps) before it is used (the nnterp
 *   queries/keys accessors list the conv, activation and head repeat but no
 *   normalisation, so the values at the rule may be raw).
 *
 *   A prompt runs the chunked (chunkwise-parallel) form of the rule over the whole
 *   sequence; a decode step runs the rule for one token against the cached state,
 *   which it overwrites in place (nnterp "state_input": None on a fresh prompt, the
 *   cache's own buffer on a decode step).
 *
 * State layout.  Every state tensor is fp32, [.., Dk, Dv] row-major: element
 * (i, j) is S[j][i], i.e. the library stores M = S^T: a key-dimension by
 * value-dimension matrix for every head, the orientation the nnterp page gives its state.
 *
 * Head sharing.  Hv value heads read Hqk <= Hv query/key heads, Hv % Hqk == 0;
 * value head h reads query/key head h / (Hv / Hqk) (the nnterp queries accessor
 * repeats the query/key heads to the value heads; each query/key head serves that
 * many consecutive value heads).
 *
 * Conventions for every entry point:
 *   - Every tensor pointer is DEVICE memory owned by the caller, contiguous
 *     row-major; q, k, v, o, states and workspace 16-byte aligned, beta, g and
 *     cu_seqlens 4-byte aligned.  The library allocates nothing and keeps no
 *     state between calls; calls on different streams may run concurrently when
 *     their output buffers do not overlap.
 *   - Work is queued on `stream` (a hipStream_t; NULL = the default stream) and
 *     is asynchronous: the call returns before the kernels finish.
 *   - Argument errors are detected on the host and returned synchronously before
 *     anything is launched; nothing is written then.  Data-dependent
 *     preconditions (g <= 0, q/k normalisation, cu_seqlens monotone with
 *     cu_seqlens[0] == 0 and cu_seqlens[N] == T) are not checked on the device.
 */
#ifndef DELTANET_H
#define DELTANET_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DN_OK = 0,
    DN_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, bad or inconsistent sizes     */
    DN_ERR_UNSUPPORTED = 2,  /* a size or dtype outside what the kernels are built for */
    DN_ERR_HIP = 3,          /* the HIP runtime reported an error at launch            */
    DN_ERR_WORKSPACE = 4     /* workspace missing or smaller than required             */
} dn_status;

typedef enum {
    DN_F32 = 0,              /* q, k, v and o are float                                */
    DN_BF16 = 1              /* q, k, v and o are bfloat16 (round to nearest even)     */
} dn_dtype;

/* dn_shape.flags bits */
#define DN_QK_L2NORM 1       /* L2-normalise q_t and k_t inside the call (see above)        */
#define DN_GATE_PER_KEY 2    /* g holds one log decay per key channel: [.., Hv, Dk]          */

/* Sizes of one call.  Supported: Dk, Dv in {16, 32, 64, 128}; chunk_size in
 * {16, 32, 64} (0 selects 64).  beta, g and all states are fp32 regardless of dtype.
 * flags: any of DN_QK_L2NORM, DN_GATE_PER_KEY (other bits are an error; DN_GATE_PER_KEY
 * needs g); l2norm_eps >= 0 (finite) is read
 * only with DN_QK_L2NORM.  With l2norm_eps == 0 a zero q or k vector normalises to
 * zero.  The bf16 Dk = Dv = 128 path folds the normalisation into per-token factors
 * and keeps A's 16x16 diagonal blocks in fp16: their entries are bounded by beta
 * times the ratio of two key norms of one chunk, so key norms within a chunk may
 * differ by up to about 10^4. */
typedef struct {
    int32_t B;           /* batch rows; 1 when cu_seqlens is given                       */
    int32_t T;           /* tokens per row; total packed tokens when cu_seqlens is given */
    int32_t num_seqs;    /* N: B, or len(cu_seqlens) - 1                                  */
    int32_t Hqk;         /* query/key heads                                               */
    int32_t Hv;          /* value heads (multiple of Hqk)                                 */
    int32_t Dk;          /* key dim                                                       */
    int32_t Dv;          /* value dim                                                     */
    int32_t dtype;       /* dn_dtype of q, k, v, o                                        */
    int32_t chunk_size;  /* tokens per chunk of the chunked form                          */
    float scale;         /* multiplies every read; 1.0 reproduces o_t = S_t q_t           */
    int32_t flags;       /* 0, or DN_QK_L2NORM | DN_GATE_PER_KEY                          */
    float l2norm_eps;    /* eps of the in-call normalisation (1e-6 is customary)          */
} dn_shape;

/*
 * dn_chunk_fwd -- the delta rule over whole sequences (prefill), in the
 * chunkwise-parallel form: inside each chunk the updates are solved together as a
 * unit-lower-triangular system, and the state is carried from chunk to chunk.
 * The result equals the token-by-token recurrence above up to rounding.
 *
 *   q, k           [B, T, Hqk, Dk]  dtype
 *   v              [B, T, Hv, Dv]   dtype
 *   beta           [B, T, Hv]       fp32 write strengths
 *   g              [B, T, Hv]       fp32 log decays, or NULL for the plain rule;
 *                  [B, T, Hv, Dk]   with DN_GATE_PER_KEY (never NULL then).  Channel
 *                                   gates run on the matrix cores for bf16 at Dk = 128,
 *                                   Dv a multiple of 32 and 64-token chunks, else on the
 *                                   vector ALUs in 32-token chunks.
 *   initial_state  [N, Hv, Dk, Dv]  fp32 state each sequence starts from, or NULL
 *                                   for the zero state (a fresh prompt)
 *   final_state    [N, Hv, Dk, Dv]  fp32 state after each sequence's last token,
 *                                   or NULL to skip it; may alias initial_state
 *   cu_seqlens     [N + 1] int32 device offsets of N sequences packed along T (B must
 *                                   be 1), or NULL: each batch row is one sequence.
 *                                   A sequence of length 0 returns its initial state.
 *   o              [B, T, Hv, Dv]   dtype, written for every token
 *   workspace      device scratch of dn_chunk_fwd_workspace_bytes(shape) bytes, or
 *                                   NULL (with less, the per-key-channel path runs as
 *                                   one slower kernel); contents on entry are ignored,
 *                                   on exit undefined (two calls in flight on one workspace race)
 *
 * Errors: DN_ERR_INVALID_ARG (null required pointer, non-positive sizes, Hv % Hqk,
 * B != 1 or num_seqs < 1 with cu_seqlens, num_seqs != B without, misaligned
 * pointer, unknown flags, negative or non-finite l2norm_eps), DN_ERR_UNSUPPORTED
 * (Dk, Dv, chunk_size or dtype not supported), DN_ERR_HIP.  A missing or short
 * workspace is not an error: the per-key-channel path then runs as one kernel
 * (dn_chunk_fwd_path tells which kernels a call runs).  T == 0 is valid:
 * final_state = initial_state.
 */
dn_status dn_chunk_fwd(const dn_shape* shape,
                       const void* q, const void* k, const void* v,
                       const float* beta, const float* g,
                       const float* initial_state, float* final_state,
                       const int32_t* cu_seqlens, void* o,
                       void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* Bytes of device workspace dn_chunk_fwd needs for this shape (0 when none).  One bf16
 * path with 64-token chunks uses one, keeping the state-independent operands of each
 * (chunk, value head) there for the sequential pass: DN_GATE_PER_KEY at Dk = 128, Dv a
 * multiple of 32 (68,352 B each; given less, one slower kernel forms them inside its
 * chunk loop). */
size_t dn_chunk_fwd_workspace_bytes(const dn_shape* shape);

/*
 * dn_chunk_fwd_noalloc -- dn_chunk_fwd for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and results as dn_chunk_fwd, without the workspace.  The path that
 * needs scratch (gates per key channel on the matrix cores: 68,352 B per chunk and value
 * head) takes it from a static device array of DN_NOALLOC_SCRATCH_BYTES that each GPU the
 * library runs on holds until the process ends; the call allocates nothing.  A call whose
 * records exceed the array (more than 981 (chunk, value head) pairs) returns
 * DN_ERR_WORKSPACE, before any launch.  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (different streams, or host threads) race and
 * must be serialised by the caller.  Nothing in the array needs clearing between calls.
 *
 * Errors: as dn_chunk_fwd, DN_ERR_WORKSPACE as above, DN_ERR_HIP if the array's device
 * address cannot be looked up.
 */
#define DN_NOALLOC_SCRATCH_BYTES (64u << 20)
dn_status dn_chunk_fwd_noalloc(const dn_shape* shape,
                               const void* q, const void* k, const void* v,
                               const float* beta, const float* g,
                               const float* initial_state, float* final_state,
                               const int32_t* cu_seqlens, void* o, hipStream_t stream);

/* Which kernels dn_chunk_fwd runs for this shape and workspace size (no launch, no
 * device access).  Only bf16 prompts with 64-token chunks run on the matrix cores: at
 * Dk = Dv = 128 or Dk = Dv = 64 in one kernel (with or without DN_QK_L2NORM), and with
 * DN_GATE_PER_KEY at Dk = 128, Dv a multiple of 32; every other supported shape runs the
 * vector-ALU chunked kernel, which is about 100x slower on the same work.  Returns
 * DN_PATH_INVALID for a shape dn_chunk_fwd would reject. */
typedef enum {
    DN_PATH_INVALID = -1,
    DN_PATH_FUSED = 0,                         /* one matrix-core kernel                     */
    DN_PATH_CHANNEL_GATE_TWO_KERNELS = 1,      /* per-key-channel gates, with the workspace  */
    DN_PATH_CHANNEL_GATE_ONE_KERNEL = 2,       /* per-key-channel gates, workspace too small */
    DN_PATH_VECTOR = 3                         /* vector-ALU chunked kernel                  */
} dn_path;
int32_t dn_chunk_fwd_path(const dn_shape* shape, size_t workspace_bytes);

/*
 * dn_decode_step -- one token of the delta rule for each of N sequences against a
 * cached state, updated in place (the nnterp page's token-by-token rule for a decode
 * step: a single token per sequence, fed the cache as its state input).
 *
 *   shape->B = N sequences, shape->T must be 1, num_seqs = N, cu_seqlens unused;
 *   q, k   [N, Hqk, Dk] dtype;  v [N, Hv, Dv] dtype;  beta, g [N, Hv] fp32 (g may be NULL;
 *          [N, Hv, Dk] with DN_GATE_PER_KEY)
 *   state  [N, Hv, Dk, Dv] fp32, read and overwritten with the new state
 *   o      [N, Hv, Dv] dtype
 *
 * Errors: as dn_chunk_fwd (chunk_size is ignored).
 */
dn_status dn_decode_step(const dn_shape* shape,
                         const void* q, const void* k, const void* v,
                         const float* beta, const float* g,
                         float* state, void* o, hipStream_t stream);

/*
 * dn_recurrent_fwd -- the rule token by token over whole sequences (the pages'
 * recurrent route: the frankenstein forward's token loop; the nnterp page's recurrent
 * delta-rule route, which exposes the state after every token).  Same arguments and
 * results as dn_chunk_fwd (chunk_size is ignored, no workspace), plus
 *
 *   state_trace    [B, T, Hv, Dk, Dv] fp32 (B * T tokens), 16-byte aligned, or NULL:
 *                  the state after each token (key-major like every state), written for
 *                  every token of every sequence
 *
 * One workgroup per (sequence, value head) keeps the state in registers and steps through
 * the tokens: it is for inspection and for checking the chunked path, not a fast prompt
 * path (the trace alone is Dk * Dv * 4 bytes per token and head).
 *
 * Errors: as dn_chunk_fwd.
 */
dn_status dn_recurrent_fwd(const dn_shape* shape,
                           const void* q, const void* k, const void* v,
                           const float* beta, const float* g,
                           const float* initial_state, float* final_state,
                           const int32_t* cu_seqlens, void* o, float* state_trace,
                           hipStream_t stream);

/*
 * dn_recurrent_bwd -- the reverse pass of the rule (gradients for training), token by
 * token: given dL/do and dL/d final_state, the gradients of the loss for q, k, v, beta, g
 * and the initial state.  It walks each sequence backwards from the state trace that
 * dn_recurrent_fwd wrote for the same inputs (with the same flags).  One gate per head,
 * one per key channel (DN_GATE_PER_KEY: M' = diag(exp(g_t)) M, so dg_t[i] sums row i of
 * dL/dM' times M') or none.  With DN_QK_L2NORM, dq and dk are the gradients for the raw
 * q and k, taken back through x / sqrt(|x|^2 + eps).
 *
 *   state_trace     [B, T, Hv, Dk, Dv] fp32 from dn_recurrent_fwd (required)
 *   d_o             [B, T, Hv, Dv] dtype (required)
 *   d_final_state   [N, Hv, Dk, Dv] fp32 or NULL (zero)
 *   dq, dk          [B, T, Hqk, Dk] fp32 (summed over the value heads of each q/k head)
 *   dv              [B, T, Hv, Dv] fp32;  dbeta [B, T, Hv] fp32
 *   dg              g's shape ([B, T, Hv], or [B, T, Hv, Dk] per key channel) fp32,
 *                   required when g is given, else ignored
 *   d_initial_state [N, Hv, Dk, Dv] fp32 or NULL
 *   workspace       dn_recurrent_bwd_workspace_bytes(shape) bytes
 *
 * Errors: as dn_recurrent_fwd, DN_ERR_WORKSPACE.
 */
dn_status dn_recurrent_bwd(const dn_shape* shape,
                           const void* q, const void* k, const void* v,
                           const float* beta, const float* g, const float* initial_state,
                           const float* state_trace, const void* d_o,
                           const float* d_final_state, const int32_t* cu_seqlens,
                           float* dq, float* dk, float* dv, float* dbeta, float* dg,
                           float* d_initial_state, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * dn_chunk_bwd -- the reverse pass of the chunked form on the matrix cores (gradients for
 * training; the learned gate and write strengths of the nnterp "linear_attention" page,
 * LinearAttention class text): given dL/do and dL/d final_state, the gradients for q, k,
 * v, beta, g and the initial state, without a per-token state trace.  It reruns the forward
 * chunk chain to keep the state at every chunk start, forms T = (I + A)^-1 and P of every
 * chunk in parallel, walks each sequence's chunks backwards carrying only dL/dM (written
 * out at every chunk), and then forms every gradient of every chunk in parallel from the
 * chunk's start state and dL/dM after it.  dq and dk sum the value heads of a q/k head in a
 * fixed order and no step uses atomics (the result is bitwise reproducible).  With fewer
 * (sequence, value head) pairs than a quarter of the GPU's compute units, the rerun of the
 * forward runs on a second stream of the library's own, forked from and joined to `stream`
 * by events (so the call can be captured into a graph on `stream`); otherwise every step
 * runs on `stream`.
 *
 * Supported: bf16 q/k/v/d_o, Dk = Dv = 128, 64-token chunks, one log decay per head or
 * none, with or without DN_QK_L2NORM (then a first pass writes the normalised q and k,
 * in bf16, and the inverse norms of their rows to the workspace, the reverse pass runs on
 * them, and its last kernel takes dq, dk back through the normalisation to the raw rows
 * as it stores them); DN_GATE_PER_KEY and other shapes
 * return DN_ERR_UNSUPPORTED (dn_recurrent_bwd computes them token by token from a state
 * trace).  Arguments as dn_recurrent_bwd without the trace:
 *
 *   d_o             [B, T, Hv, Dv] bf16 (required)
 *   d_final_state   [N, Hv, Dk, Dv] fp32 or NULL (zero)
 *   dq, dk          [B, T, Hqk, Dk] fp32 (summed over the value heads of each q/k head)
 *   dv              [B, T, Hv, Dv] fp32;  dbeta [B, T, Hv] fp32
 *   dg              [B, T, Hv] fp32, required when g is given, else ignored
 *   d_initial_state [N, Hv, Dk, Dv] fp32 or NULL
 *   workspace       dn_chunk_bwd_workspace_bytes(shape) bytes: per chunk and value head the
 *                   state at the chunk start and dL/dM after the chunk (fp32) and T and P
 *                   (bf16): (2 Dk Dv * 4 + 2 * 64 * 64 * 2) bytes; with DN_QK_L2NORM
 *                   also 2 * B * T * Hqk * Dk * 2 bytes of normalised q and k and
 *                   2 * B * T * Hqk * 4 bytes of inverse norms (rounded up to 256);
 *                   contents on entry ignored, on exit undefined
 *
 * Errors: as dn_chunk_fwd, DN_ERR_UNSUPPORTED as above, DN_ERR_WORKSPACE.
 */
dn_status dn_chunk_bwd(const dn_shape* shape,
                       const void* q, const void* k, const void* v,
                       const float* beta, const float* g, const float* initial_state,
                       const void* d_o, const float* d_final_state, const int32_t* cu_seqlens,
                       float* dq, float* dk, float* dv, float* dbeta, float* dg,
                       float* d_initial_state, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* Bytes of workspace dn_chunk_bwd needs for this shape (0 when the shape is unsupported). */
size_t dn_chunk_bwd_workspace_bytes(const dn_shape* shape);

/* Bytes of workspace dn_recurrent_bwd needs: each value-column slice's share of dq, dk,
 * dbeta and dg before they are added in a fixed order (the shape's flags matter: dg per
 * key channel takes Dk floats per token and head). */
size_t dn_recurrent_bwd_workspace_bytes(const dn_shape* shape);

/*
 * Readout epilogue: the step after the rule, per (token, value head) over the d_v
 * entries of the readout o -- a normalisation (the frankenstein page's layer norm of the
 * recurrent readout; the mutichung block flowchart's RMSNorm after the Delta Rule box),
 * then the silu-gated output gate (frankenstein g_proj):
 *
 *   DN_NORM_RMS:    y = o / sqrt(mean(o^2) + eps) * w
 *   DN_NORM_LAYER:  y = (o - mean(o)) / sqrt(mean((o - mean(o))^2) + eps) * w + b
 *   with a gate z:  y <- y * z / (1 + exp(-z))
 *
 * w and b (length d_v, fp32) are shared by the heads; NULL weight = ones, NULL bias =
 * zeros (a bias is an error with DN_NORM_RMS).  The gate has the readout's shape and
 * dtype, or is NULL (no output gate).  Arithmetic is fp32.
 */
typedef enum { DN_NORM_RMS = 0, DN_NORM_LAYER = 1 } dn_norm_kind;

typedef struct {
    int32_t kind;          /* dn_norm_kind                                               */
    float eps;             /* >= 0 and finite; inside the square root                    */
    const float* weight;   /* [Dv] fp32 device, 4-byte aligned, or NULL (ones)           */
    const float* bias;     /* [Dv] fp32 device, 4-byte aligned, or NULL (zeros)          */
    const void* gate;      /* readout-shaped, dtype, 16-byte aligned, or NULL (no gate)  */
} dn_epilogue;

/*
 * dn_norm_gate -- the epilogue over a prefill's output: o and y are [B, T, Hv, Dv] in
 * shape->dtype (B * T tokens; Hqk, Dk and chunk_size are checked as for dn_chunk_fwd
 * but not used), the gate likewise.  y may alias o.  Bound by HBM bandwidth: it reads o
 * (and the gate) once and writes y once.
 *
 * Errors: as dn_chunk_fwd, and DN_ERR_INVALID_ARG for a NULL or bad epilogue (unknown
 * kind, negative or non-finite eps, a bias with DN_NORM_RMS, misaligned pointer).
 */
dn_status dn_norm_gate(const dn_shape* shape, const dn_epilogue* epilogue,
                       const void* o, void* y, hipStream_t stream);

/*
 * dn_decode_step_ex -- dn_decode_step with the epilogue fused: o receives y (the raw
 * readout is not written).  epilogue == NULL is dn_decode_step.  The decode workgroup
 * holds a head's whole readout, so the epilogue adds no HBM traffic beyond the gate.
 *
 * Errors: as dn_decode_step and dn_norm_gate.
 */
dn_status dn_decode_step_ex(const dn_shape* shape,
                            const void* q, const void* k, const void* v,
                            const float* beta, const float* g,
                            float* state, const dn_epilogue* epilogue, void* o,
                            hipStream_t stream);

/*
 * Short causal depthwise convolution in front of the rule (the mutichung DeltaNet block
 * flowchart: a "Conv" box then a "SiLU" box on the q/k and on the v branch, the
 * convolutions depthwise-separable, generalising the shift SSM).  Per channel c:
 *
 *   y_t[c] = act(b[c] + sum_{j<W} w[c][j] x_{t-W+1+j}[c]),   act = silu or identity
 *
 * Inputs before a sequence's first token come from its conv state, the W - 1 inputs
 * before it, oldest first, [N, C, W - 1] in the dtype of x; a NULL initial state means
 * zeros.  The final state is each sequence's last W - 1 inputs (state entries when the
 * sequence is shorter).  Channels are the last axis of x: q, k and v of one layer can be
 * one [.., Hqk*Dk + Hqk*Dk + Hv*Dv] tensor.  Bound by HBM bandwidth: x is read once and y
 * written once.
 */
typedef struct {
    int32_t B, T;          /* B rows of T tokens; B == 1 with cu_seqlens (T = total tokens)   */
    int32_t num_seqs;      /* N: B, or len(cu_seqlens) - 1                                      */
    int32_t C;             /* channels, a multiple of 8                                          */
    int32_t width;         /* W, 2..8                                                            */
    int32_t dtype;         /* dn_dtype of x, y and the conv states                               */
    int32_t activation;    /* 0: none, 1: silu                                                   */
} dn_conv_shape;

/*
 *   x              [B, T, C] dtype, 16-byte aligned
 *   weight         [C, W] fp32 (4-byte aligned);  bias [C] fp32 or NULL
 *   initial_state  [N, C, W - 1] dtype or NULL;   final_state [N, C, W - 1] dtype or NULL
 *                  (may not alias initial_state: a sequence's last block may be read
 *                  after another's state is written)
 *   cu_seqlens     [N + 1] int32 device or NULL (each batch row is a sequence)
 *   y              [B, T, C] dtype, 16-byte aligned; may not alias x
 * Errors: DN_ERR_INVALID_ARG (null required pointer, sizes, C % 8, misalignment,
 * aliasing), DN_ERR_UNSUPPORTED (W outside 2..8, dtype), DN_ERR_HIP.
 */
dn_status dn_causal_conv(const dn_conv_shape* shape, const void* x, const float* weight,
                         const float* bias, const void* initial_state, void* final_state,
                         const int32_t* cu_seqlens, void* y, hipStream_t stream);

/*
 * dn_conv_qkv -- the whole prologue in front of the rule in one pass (the mutichung
 * "DeltaNet" page, "DeltaNet Transformer" flowchart: Conv, then SiLU, then the L2 norm on
 * the q and k branches, then the delta rule): the convolution of dn_causal_conv over
 * x = [q | k | v] projections, [.., Hqk*Dk + Hqk*Dk + Hv*Dv] channels, its output split
 * into q, k and v tensors in the layout dn_chunk_fwd reads, with q and k L2-normalised per
 * head (x / sqrt(|x|^2 + eps), the normalisation of DN_QK_L2NORM) inside the same pass.
 * x is read once and q, k, v written once; hand the results to dn_chunk_fwd without
 * DN_QK_L2NORM.
 *
 *   shape          as dn_causal_conv, C == 2 Hqk Dk + Hv Dv (activation 1 for the flowchart)
 *   split          heads and head sizes (below); Dk in {16, 32, 64, 128}, Dv a multiple of 8
 *   x, weight, bias, initial_state, final_state, cu_seqlens   as dn_causal_conv
 *   q, k           [B, T, Hqk, Dk] dtype, 16-byte aligned
 *   v              [B, T, Hv, Dv] dtype, 16-byte aligned; none of q, k, v aliases x or another
 * Errors: as dn_causal_conv; DN_ERR_INVALID_ARG also for a split that does not add up to C,
 * eps negative or not finite; DN_ERR_UNSUPPORTED for Dk outside {16, 32, 64, 128}.
 */
typedef struct {
    int32_t Hqk, Hv;       /* q/k heads and value heads                                      */
    int32_t Dk, Dv;        /* head sizes                                                     */
    int32_t qk_l2norm;     /* 1: q and k L2-normalised per head after the conv; 0: not       */
    float eps;             /* the normalisation's epsilon (>= 0, finite)                     */
} dn_qkv_split;

dn_status dn_conv_qkv(const dn_conv_shape* shape, const dn_qkv_split* split, const void* x,
                      const float* weight, const float* bias, const void* initial_state,
                      void* final_state, const int32_t* cu_seqlens, void* q, void* k, void* v,
                      hipStream_t stream);

/*
 * dn_causal_conv_step -- one token per sequence (decode): shape->B = N sequences, T == 1;
 * x, y [N, C]; conv_state [N, C, W - 1] read and overwritten (shifted by one, x appended).
 * Errors: as dn_causal_conv.
 */
dn_status dn_causal_conv_step(const dn_conv_shape* shape, const void* x, const float* weight,
                              const float* bias, void* conv_state, void* y, hipStream_t stream);

/* Static description of a status code. */
const char* dn_status_str(dn_status status);

/* ABI version (major * 10000 + minor * 100 + patch). */
int32_t dn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DELTANET_H */
