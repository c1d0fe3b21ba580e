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
 * (seqlen is ignored by the decode ops, n_layers by the single-layer ops; for the prefill op the
 * size covers every supported chunk length). Returns 0 for an invalid or unsupported shape.
 * The workspace needs no initialisation and holds nothing between calls.
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
 * Autoregressive-style decode through a stack of n_layers layers for n_steps tokens:
 *   x(0) = x0;  for t: h = x(t); h = layer_l(h) for l = 0..n_layers-1;
 *   y[t] = RMSNorm(h) * final_norm_w;  x(t+1) = y[t].
 * The whole token loop runs as ONE persistent kernel launch (the paper's §4.1 captures the forward
 * pass in a graph to remove per-kernel launch cost; here the layers hand their partial results to
 * each other through tagged words in the workspace instead of kernel boundaries). When the device
 * cannot keep the needed workgroups resident at once, the call falls back to per-layer kernels
 * with the same results.
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

/* Static, human-readable text of a status code. */
const char *dfssm_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* DFSSM_H */
