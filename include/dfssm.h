/*
 * dfssm.h - C ABI of the DF-SSM inference hot path on AMD Instinct MI355X (gfx950).
 *
 * DF-SSM ("Density Field State Space Models: 1-Bit Distillation, Efficient Inference, and
 * Knowledge Organization in Mamba-2", arXiv 2606.10932) stores every in/out projection of a
 * Mamba-2 layer as a frozen 1-bit scaffold plus an int8 low-rank correction (paper §3.2 Eq. (3),
 * §3.3), keeps the conv and SSM states resident across tokens and runs the whole layer stack as
 * one captured unit per token (paper §4.1). This header exposes that computation.
 *
 * Semantics of one decode step of one layer for one token h (all norms use eps = norm_eps):
 *   u   = RMSNorm(h) * norm_w                                   (fp32 vector, d_model)
 *   a   = max|u|;  q = clamp(rint_even(u * fl32(127/a)), -127, 127);  s = fl32(a/127)
 *         (a == 0 gives q = 0, s = 0)                           (per-token int8 codes)
 *   acc = sign(in) . q   (int32; sign bit 1 -> +1, 0 -> -1)      (1-bit scaffold, §4.1)
 *   t   = lora_dn(in) . q (int32, rank_in values)                (int8 low-rank, §3.3)
 *   Y   = s*row_scale*acc + lora_up_scale * lora_up . (lora_dn_scale * s * t)    (Eq. (3))
 *   Y is split into z[d_inner] | xBC[conv_dim] | dt_raw[nheads] | padding
 *   xBC <- SiLU(causal depthwise conv over (conv state, xBC) + conv_b)   (state shifts by one)
 *   dt = softplus(dt_raw + dt_bias);  A = -exp(A_log);  per head: S <- exp(dt*A) S + (dt x) (x) B,
 *   y = S . C + D x                                          (paper App. B Table 12, row 1)
 *   g = y * SiLU(z);  u2 = RMSNorm(g) * gnorm_w              (gate, then norm: App. B Table 12)
 *   (q2, s2) as above from u2;  h_out = h + projection(out, q2, s2)
 * conv_dim = d_inner + 2*ngroups*d_state; nheads = d_inner / headdim; head h reads B and C of
 * group h*ngroups/nheads.
 *
 * Around the layer: the tied int8 embedding and LM head (dfssm_embed, dfssm_lm_head; paper §3.3,
 * Table 1), the projection with the 17-level scaffold the 1-bit one is binarised from
 * (dfssm_dfw_project; §3.1 Eq. (1)), and the density field codec of the SSM state, standalone
 * (dfssm_state_encode / dfssm_state_decode) and at the chunk boundaries of the prefill scan
 * (dfssm_layer_prefill_ex / dfssm_stack_prefill_ex; §3.4, App. D).
 *
 * Conventions
 *  - Every pointer is a DEVICE pointer (hipMalloc'd or equivalent) unless marked HOST.
 *  - The caller owns all memory. Weights are read-only; states are updated in place; no pointer
 *    is retained after the enqueued work completes. The library allocates no device memory
 *    inside these calls; every intermediate lives in the caller's workspace.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default stream). A return of
 *    DFSSM_OK means the work was enqueued; device faults surface at the caller's next sync.
 *  - Every argument is validated before anything is enqueued, so a call that returns an error
 *    has no side effect.
 *  - Device pointers must be 16-byte aligned.
 *  - Calls are re-entrant across streams when their states, outputs and workspaces differ;
 *    two calls that share a workspace or state must be ordered by the caller.
 */
#ifndef DFSSM_H
#define DFSSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define DFSSM_OK            0
#define DFSSM_EINVAL       (-1)   /* null required pointer, misalignment, non-positive size   */
#define DFSSM_EUNSUPPORTED (-2)   /* shape outside what the kernels implement (see dfssm_dims) */
#define DFSSM_EWORKSPACE   (-3)   /* ws_bytes smaller than dfssm_workspace_bytes()             */
#define DFSSM_EHIP         (-4)   /* a HIP runtime call or launch failed                        */

/* dfssm_workspace_bytes() op codes */
#define DFSSM_OP_LAYER_DECODE  0
#define DFSSM_OP_LAYER_PREFILL 1
#define DFSSM_OP_STACK_DECODE  2
#define DFSSM_OP_STACK_PREFILL 3

/* Status word of a stack decode: the int32 at byte offset DFSSM_STACK_STATUS_OFFSET of the
 * workspace holds, once the call's work has completed on the stream, DFSSM_STATUS_OK or
 * DFSSM_STATUS_TIMEOUT (a wait between the workgroups of a persistent launch ran past its bound,
 * e.g. because the device could not keep the whole grid running; every value of y is then NaN). */
#define DFSSM_STACK_STATUS_OFFSET 0   /* the int32 after it is an internal diagnostic code */
#define DFSSM_STATUS_OK      0
#define DFSSM_STATUS_TIMEOUT 1

/* dfssm_stack_opts.path */
#define DFSSM_PATH_AUTO      0   /* the fastest path that supports the shape and batch            */
#define DFSSM_PATH_FLOW      1   /* batch 1: one persistent launch, two exchanges per layer        */
#define DFSSM_PATH_PER_LAYER 2   /* a launch sequence per layer and token (any batch)              */

/* token input dtypes of dfssm_layer_prefill */
#define DFSSM_F32  0
#define DFSSM_BF16 1

/*
 * Layer shape. Supported: d_model and d_inner multiples of 128 (up to 16384); headdim == 64;
 * d_state in {16, 32, 64, 128, 256}; d_inner == nheads*headdim; nheads % ngroups == 0;
 * d_conv == 4; n_in_proj >= 2*d_inner + 2*ngroups*d_state + nheads (extra rows are padding
 * that is computed and ignored); 1 <= rank_in, rank_out <= 64; norm_eps > 0.
 */
typedef struct dfssm_dims {
    int32_t d_model, d_inner, d_state, headdim, ngroups, d_conv;
    int32_t n_in_proj;
    int32_t rank_in, rank_out;
    float   norm_eps;
} dfssm_dims;

/*
 * One projection (paper §3.2 Eq. (3) with the int8 factors of §3.3; alpha = 1).
 *   sign      [n_out][n_in/8] uint8, row-major; weight k of a row is bit (k%8) of byte k/8
 *             (equivalently bit k%64 of little-endian 64-bit word k/64, the 64-weights-per-8-bytes
 *             packing of paper §4.2); bit 1 -> +1, bit 0 -> -1.
 *   row_scale [n_out] IEEE fp16 bit patterns: per-output-row scaffold scale.
 *   lora_dn   [rank][n_in] int8 row-major (the paper's W_B);  lora_dn_scale [rank] fp32.
 *   lora_up   [n_out][rank] int8 row-major (the paper's W_A); lora_up_scale [n_out] fp32.
 */
typedef struct dfssm_proj {
    const uint8_t  *sign;
    const uint16_t *row_scale;
    const int8_t   *lora_dn;
    const float    *lora_dn_scale;
    const int8_t   *lora_up;
    const float    *lora_up_scale;
} dfssm_proj;

/*
 * Weights of one layer. in_proj: n_out = n_in_proj, n_in = d_model, rank = rank_in.
 * out_proj: n_out = d_model, n_in = d_inner, rank = rank_out. Rows of in_proj are
 * [z | x | B | C | dt | padding].
 *   conv_w [conv_dim][d_conv] fp32 (column d_conv-1 multiplies the newest input), conv_b [conv_dim]
 *   dt_bias, A_log, D [nheads] fp32;  norm_w [d_model] fp32;  gnorm_w [d_inner] fp32
 */
typedef struct dfssm_layer_weights {
    dfssm_proj   in_proj, out_proj;
    const float *conv_w, *conv_b;
    const float *dt_bias, *A_log, *D;
    const float *norm_w, *gnorm_w;
} dfssm_layer_weights;

/*
 * Persistent per-sequence state of one layer (paper §4.1: preallocated, persists across tokens).
 *   conv [batch][conv_dim][d_conv-1] fp32: the last d_conv-1 pre-activation conv inputs, oldest first
 *   ssm  [batch][nheads][headdim][d_state] fp32
 */
typedef struct dfssm_layer_state {
    float *conv;
    float *ssm;
} dfssm_layer_state;

/*
 * Optional debug taps (any member may be NULL; the struct pointer itself may be NULL).
 * For dfssm_layer_decode each buffer holds one record per batch row: [batch][...].
 * For dfssm_layer_prefill: [batch][seqlen][...]. For dfssm_stack_decode:
 * [n_steps][n_layers][batch][...]. Record sizes: h_in, in_u: d_model fp32; in_q: d_model int8;
 * in_s, out_s: 1 fp32; in_acc: n_in_proj int32; in_t: rank_in int32; out_u: d_inner fp32;
 * out_q: d_inner int8; out_acc: d_model int32; out_t: rank_out int32.
 * h_in is the residual entering the layer; u/q/s are exactly the values the quantizer saw and
 * produced; acc/t are the integer scaffold and low-rank sums.
 */
typedef struct dfssm_taps {
    float   *h_in;
    float   *in_u;   int8_t *in_q;   float *in_s;   int32_t *in_acc;  int32_t *in_t;
    float   *out_u;  int8_t *out_q;  float *out_s;  int32_t *out_acc; int32_t *out_t;
} dfssm_taps;

/*
 * Bytes of device workspace `op` needs for this shape, batch, sequence length and layer count
 * (seqlen is ignored by the decode ops, n_layers by the single-layer ops; for the prefill ops the
 * size covers every supported chunk length). Returns 0 for an invalid or unsupported shape.
 * The workspace needs no initialisation and carries nothing from one call to the next (a stack
 * decode leaves its status word, DFSSM_STACK_STATUS_OFFSET, for the caller to read).
 */
size_t dfssm_workspace_bytes(const dfssm_dims *dims, int32_t op, int32_t batch, int32_t seqlen,
                             int32_t n_layers);

/*
 * One decode step of one layer for `batch` independent sequences (paper §4.1, batch = 1 in the
 * paper's headline; Table 2 runs batches up to 512).
 *   dims, w, state, taps: HOST pointers to the structs above (their members are device pointers);
 *   x_in [batch][d_model] fp32 residual input; x_out [batch][d_model] fp32 = x_in + mixer output
 *   (x_out may alias x_in). state is read and updated in place. 1 <= batch <= 4096. Up to 4 tokens
 *   share one pass of a packed-sign GEMV; larger batches (with ranks that are multiples of 8) run the
 *   projections as int8 MFMA GEMMs.
 * Returns DFSSM_OK or a negative status.
 */
int dfssm_layer_decode(const dfssm_dims *dims, const dfssm_layer_weights *w,
                       const dfssm_layer_state *state, const float *x_in, float *x_out,
                       int32_t batch, void *ws, size_t ws_bytes, const dfssm_taps *taps,
                       void *stream);

/*
 * dfssm_layer_decode without a workspace argument, for callers that cannot allocate device memory
 * around the call: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. The intermediates live in a fixed device array of DFSSM_NOALLOC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends (its address is looked up on
 * the first call on each device, so make one call before capturing a graph). The call allocates
 * nothing; a shape and batch whose dfssm_workspace_bytes(DFSSM_OP_LAYER_DECODE) exceeds the array
 * returns DFSSM_EWORKSPACE (the Mamba-2 1.3B layer fits up to batch 64). Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (different streams, or host threads)
 * race and must be ordered by the caller. Arguments and results as dfssm_layer_decode.
 */
#define DFSSM_NOALLOC_SCRATCH_BYTES (16u << 20)
int dfssm_layer_decode_noalloc(const dfssm_dims *dims, const dfssm_layer_weights *w,
                               const dfssm_layer_state *state, const float *x_in, float *x_out,
                               int32_t batch, const dfssm_taps *taps, void *stream);

/*
 * Prefill of `seqlen` tokens per sequence through one layer, starting from `state` and leaving
 * the final conv/SSM state in it. The result equals seqlen successive dfssm_layer_decode steps
 * (quantization is per token); the SSM part is evaluated as a chunked scan with chunk length
 * `chunk` (the state-space-duality block form of Mamba-2, which the paper builds on, §2).
 *   x_in  [batch][seqlen][d_model], fp32 (x_dtype DFSSM_F32) or bf16 bit patterns (DFSSM_BF16)
 *   x_out [batch][seqlen][d_model] fp32 (must not alias x_in)
 *   chunk in {16, 32, 64, 128, 256}; 1 <= seqlen <= 65536; 1 <= batch <= 64; batch*seqlen <= 2^20;
 *   rank_in and rank_out
 *   multiples of 8 (the projections run as int8 MFMA GEMMs over all batch*seqlen tokens).
 */
int dfssm_layer_prefill(const dfssm_dims *dims, const dfssm_layer_weights *w,
                        const dfssm_layer_state *state, const void *x_in, int32_t x_dtype,
                        float *x_out, int32_t batch, int32_t seqlen, int32_t chunk,
                        void *ws, size_t ws_bytes, const dfssm_taps *taps, void *stream);

/*
 * dfssm_layer_prefill with options (opts: HOST pointer, NULL = defaults, which is dfssm_layer_prefill).
 *   state_codec       1: DF-SSD ([DF-SSM] §3.4 "Density Field State Representation", App. D): the SSM
 *                     state entering every chunk after the first passes through the density field
 *                     codec of dfssm_state_encode / dfssm_state_decode (encoded and read back, per
 *                     state row) before the chunk uses it; the state after the last chunk, written
 *                     back to state->ssm, is not coded. 0: off.
 *   reserved          must be 0.
 *   chunk_state_pre   optional (state_codec only), device [n_chunks][batch][nheads][headdim][d_state]
 *                     fp32, n_chunks = ceil(seqlen / chunk): the state entering each chunk before the
 *                     codec (chunk 0: the initial state).
 *   chunk_state_in    optional, the same shape: the state each chunk uses (after the codec).
 * The codec carry runs one wave per (sequence, head), sequentially over the chunks.
 */
typedef struct dfssm_prefill_opts {
    int32_t state_codec;
    int32_t reserved;
    float  *chunk_state_pre;
    float  *chunk_state_in;
} dfssm_prefill_opts;

int dfssm_layer_prefill_ex(const dfssm_dims *dims, const dfssm_layer_weights *w,
                           const dfssm_layer_state *state, const void *x_in, int32_t x_dtype,
                           float *x_out, int32_t batch, int32_t seqlen, int32_t chunk,
                           void *ws, size_t ws_bytes, const dfssm_taps *taps,
                           const dfssm_prefill_opts *opts, void *stream);

/*
 * Kernel selection for dfssm_stack_decode_ex (every path computes the same decode; zero-initialise
 * the struct for the defaults).
 *   path      DFSSM_PATH_*; a path that cannot run the shape and batch is DFSSM_EUNSUPPORTED.
 *   launch    DFSSM_LAUNCH_*: how DFSSM_PATH_FLOW's persistent kernel is launched. Its grid (one
 *             workgroup per compute unit) must be resident all at once; the cooperative launch
 *             (default) has the runtime verify that, the ordinary launch does not (for tools that
 *             cannot follow cooperative launches, e.g. kernel tracers): if the device then leaves
 *             part of the grid waiting, the bounded waits expire and the call's status word reads
 *             DFSSM_STATUS_TIMEOUT. Ignored by the other paths.
 */
#define DFSSM_LAUNCH_COOPERATIVE 0
#define DFSSM_LAUNCH_ORDINARY    1
typedef struct dfssm_stack_opts {
    int32_t path;
    int32_t launch;
} dfssm_stack_opts;

/*
 * Autoregressive-style decode through a stack of n_layers layers for n_steps tokens:
 *   x(0) = x0;  for t: h = x(t); h = layer_l(h) for l = 0..n_layers-1;
 *   y[t] = RMSNorm(h) * final_norm_w;  x(t+1) = y[t].
 * At batch 1 the whole token loop runs as ONE persistent kernel launch (the paper's §4.1 captures
 * the forward pass in a graph to remove per-kernel launch cost; here the layers hand their partial
 * results to each other through tagged words in the workspace instead of kernel boundaries). When
 * the device cannot keep the needed workgroups resident at once, and at batch > 1, the call runs
 * per-layer kernels with the same results. From batch 32 up the batch runs as two halves: the first
 * on `stream`, the second on a stream the library creates once per device (default priority,
 * forked from `stream` by an event at the start of the call and joined back into it at the end),
 * so all of the call's work is still ordered on `stream`. The call's status word
 * (DFSSM_STACK_STATUS_OFFSET) is written in the workspace once its work completes.
 *   layers, states: HOST arrays [n_layers] of the structs above; final_norm_w [d_model] fp32;
 *   x0 [batch][d_model] fp32; y [n_steps][batch][d_model] fp32 (must not alias x0);
 *   taps: NULL or records laid out [n_steps][n_layers][batch][...].
 *   1 <= n_layers <= 1024, 1 <= n_steps <= 1<<20, 1 <= batch <= 4096.
 */
int dfssm_stack_decode(const dfssm_dims *dims, const dfssm_layer_weights *layers,
                       const dfssm_layer_state *states, int32_t n_layers,
                       const float *final_norm_w, const float *x0, float *y,
                       int32_t batch, int32_t n_steps, void *ws, size_t ws_bytes,
                       const dfssm_taps *taps, void *stream);

/* dfssm_stack_decode with an explicit kernel path (opts: HOST pointer, NULL = defaults). */
int dfssm_stack_decode_ex(const dfssm_dims *dims, const dfssm_layer_weights *layers,
                          const dfssm_layer_state *states, int32_t n_layers,
                          const float *final_norm_w, const float *x0, float *y,
                          int32_t batch, int32_t n_steps, void *ws, size_t ws_bytes,
                          const dfssm_taps *taps, const dfssm_stack_opts *opts, void *stream);

/*
 * Prefill of `seqlen` tokens per sequence through a stack of n_layers layers (the pages' §4.1
 * forward over a prompt, batch rows independent), leaving every layer's final conv/SSM state in
 * `states` for the decode that continues from it:
 *   h = x_in;  h = layer_l(h) for l = 0..n_layers-1 (each as dfssm_layer_prefill);
 *   y[b][t] = RMSNorm(h[b][t]) * final_norm_w
 * so y[b][seqlen-1] is the x0 of a dfssm_stack_decode that continues the sequences.
 *   layers, states: HOST arrays [n_layers]; x_in [batch][seqlen][d_model] fp32 or bf16 bit patterns;
 *   y [batch][seqlen][d_model] fp32 (must not alias x_in); taps: NULL or records laid out
 *   [n_layers][batch][seqlen][...]. Limits as for dfssm_layer_prefill; 1 <= n_layers <= 1024.
 */
int dfssm_stack_prefill(const dfssm_dims *dims, const dfssm_layer_weights *layers,
                        const dfssm_layer_state *states, int32_t n_layers,
                        const float *final_norm_w, const void *x_in, int32_t x_dtype, float *y,
                        int32_t batch, int32_t seqlen, int32_t chunk, void *ws, size_t ws_bytes,
                        const dfssm_taps *taps, void *stream);

/* dfssm_stack_prefill with options (opts: HOST pointer, NULL = defaults): state_codec applies DF-SSD
 * (see dfssm_prefill_opts) in every layer; the chunk-state taps must be NULL here (take them from
 * dfssm_layer_prefill_ex). */
int dfssm_stack_prefill_ex(const dfssm_dims *dims, const dfssm_layer_weights *layers,
                           const dfssm_layer_state *states, int32_t n_layers,
                           const float *final_norm_w, const void *x_in, int32_t x_dtype, float *y,
                           int32_t batch, int32_t seqlen, int32_t chunk, void *ws, size_t ws_bytes,
                           const dfssm_taps *taps, const dfssm_prefill_opts *opts, void *stream);

/*
 * The tied int8 embedding / LM head ([DF-SSM] §3.3: the embedding is quantized to int8 per row;
 * Table 1: "Embedding + LM head (tied)", 103 MB for the 1.3B model):
 *   weight[v][k] = codes[v][k] * row_scale[v]
 *   codes [vocab][d_model] int8 row-major; row_scale [vocab] fp32.
 * Supported: d_model a multiple of 128 up to 8192; 1 <= vocab <= 1<<24.
 */
typedef struct dfssm_embedding {
    const int8_t *codes;
    const float  *row_scale;
    int32_t vocab, d_model;
} dfssm_embedding;

/* Optional taps of dfssm_lm_head (any member may be NULL): q [batch][d_model] int8 and s [batch]
 * fp32, the head's codes of y; acc [batch][vocab] int32, the integer row sums. */
typedef struct dfssm_head_taps {
    int8_t  *q;
    float   *s;
    int32_t *acc;
} dfssm_head_taps;

/* x[b] = weight[tokens[b]] (fp32 [batch][d_model]); tokens [batch] int32 on the device (ids outside
 * [0, vocab) are clamped into it). 1 <= batch <= 4096. No workspace. */
int dfssm_embed(const dfssm_embedding *emb, const int32_t *tokens, int32_t batch, float *x, void *stream);

/*
 * The tied LM head over y [batch][d_model] fp32 (the stack's normalised output, dfssm_stack_decode's
 * y[t]): per token the same int8 quantizer as the projections, (q, s) = Qz(y[b]), then
 *   acc[v] = sum_k codes[v][k] q[k] (int32),  logits[b][v] = s * row_scale[v] * acc[v]
 * and next_tokens[b] = the v of the largest logit (the smallest v among equal logits).
 *   logits [batch][vocab] fp32 and next_tokens [batch] int32 may each be NULL (not both);
 *   ws: dfssm_workspace_bytes(dims, DFSSM_OP_LM_HEAD, batch, 0, 0) bytes (dims.d_model == d_model).
 * Every byte of the embedding is read once per call of up to 8 tokens (an HBM-bound GEMV).
 * 1 <= batch <= 4096.
 */
#define DFSSM_OP_LM_HEAD 4
int dfssm_lm_head(const dfssm_embedding *emb, const float *y, int32_t batch, float *logits,
                  int32_t *next_tokens, void *ws, size_t ws_bytes, const dfssm_head_taps *taps,
                  void *stream);

/*
 * Projection with the 17-level scaffold ([DF-SSM] §3.1 Eq. (1): K_w = 16, 17 levels from -1 to +1;
 * §3.2 Eq. (3): y = W_scaffold x + W_A (W_B x)), the scaffold before binarisation.
 * The weight of row n, input i is (k - 8)/8 * row_scale[n], k = the level index 0..16 of Eq. (1)
 * (round(clamp((w+1)/2, 0, 1) * 16)), stored as five bit planes: planes[b][n][i/8] bit i % 8 holds
 * bit b of k (the 1-bit scaffold layout, once per plane; 5/8 byte per weight). Per token b:
 *   (q, s) = the per-token int8 quantizer of x[b] (as in the layer projections, without a norm)
 *   acc[n] = sum_i (k[n][i] - 8) q[i]            (exact int32)
 *   t[j]   = sum_i lora_dn[j][i] q[i]            (exact int32)
 *   y[b][n] = s * row_scale[n] * acc[n] / 8 + lora_up_scale[n] * sum_j lora_up[n][j] * lora_dn_scale[j] * s * t[j]
 * x [batch][n_in] fp32 and y [batch][n_out] fp32 are device buffers.
 * Supported: n_in a multiple of 128, 128..8192; 1 <= n_out <= 1<<20; 1 <= rank <= 64; 1 <= batch <= 256.
 * The five planes are read once per group of up to four tokens. Workspace:
 * dfssm_dfw_workspace_bytes(n_in, rank, batch) bytes. Taps (each member may be NULL): q [batch][n_in],
 * s [batch], acc [batch][n_out], t [batch][rank].
 */
typedef struct dfssm_dfw_proj {
    const uint8_t  *planes;          /* [5][n_out][n_in/8] */
    const uint16_t *row_scale;       /* [n_out] IEEE fp16 */
    const int8_t   *lora_dn;         /* [rank][n_in] */
    const float    *lora_dn_scale;   /* [rank] */
    const int8_t   *lora_up;         /* [n_out][rank] */
    const float    *lora_up_scale;   /* [n_out] */
} dfssm_dfw_proj;

typedef struct dfssm_dfw_taps {
    int8_t  *q;
    float   *s;
    int32_t *acc;
    int32_t *t;
} dfssm_dfw_taps;

size_t dfssm_dfw_workspace_bytes(int32_t n_in, int32_t rank, int32_t batch);
int dfssm_dfw_project(const dfssm_dfw_proj *w, int32_t n_out, int32_t n_in, int32_t rank, const float *x,
                      float *y, int32_t batch, void *ws, size_t ws_bytes, const dfssm_dfw_taps *taps,
                      void *stream);

/*
 * Density field codec of the SSM state ([DF-SSM] §3.4 "Density Field State Representation", App. D).
 * Each state row (the d_state values of one head channel; batch*nheads*headdim rows, in the layout
 * of dfssm_layer_state.ssm) is stored as a K x K bit field, K = round(sqrt(4*d_state)) (23 for
 * d_state 128: 529 bits), plus its fp32 mean and population standard deviation:
 *   x_i = clamp((s_i - (mu - 3 sigma)) / (6 sigma), 0, 1),  t_i = rint(255 x_i)  (8 bits)
 *   value i owns cells floor(i K^2 / d_state) .. floor((i+1) K^2 / d_state) - 1 in raster order;
 *   first-order sigma-delta over the cells with an 8-bit error e (starting at 0):
 *     v = e + t_i;  bit = (v >= 128);  e = v - 255 * bit
 *   readout: s'_i = mu - 3 sigma + 6 sigma * (ones among value i's cells) / (its cells);
 *   a row with sigma = 0 has an all-zero field and reads back as mu.
 *   fields [rows][dfssm_state_field_words(d_state)] uint32: cell c is bit c % 32 of word c / 32;
 *   stats  [rows][2] fp32: mu, sigma.
 * The state of the 1.3B layer (2 MiB per sequence) encodes to 4096 x (68 + 8) bytes = 304 KiB.
 * Supported d_state: 16, 32, 64, 128, 256. 1 <= batch <= 4096. No workspace.
 */
int32_t dfssm_state_field_words(int32_t d_state);
int dfssm_state_encode(const dfssm_dims *dims, const float *ssm, int32_t batch, uint32_t *fields,
                       float *stats, void *stream);
int dfssm_state_decode(const dfssm_dims *dims, const uint32_t *fields, const float *stats,
                       int32_t batch, float *ssm, void *stream);

/* Static, human-readable text of a status code. */
const char *dfssm_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* DFSSM_H */
