// Internal declarations shared by the DF-SSM HIP translation units (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dfssm.h"

namespace dfssm {

constexpr int kBlock = 256;          // threads per workgroup: 4 wave64
constexpr int kWaves = kBlock / 64;
constexpr int kGemvMaxBatch = 4;     // tokens one packed-sign GEMV pass serves
constexpr int kGemvLdsBytes = 61440; // dynamic LDS budget of one GEMV workgroup
constexpr int kMaxRank = 64;
constexpr int kMaxK = 8192;          // largest d_model / d_inner
constexpr int kConvTaps = 4;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Derived shape quantities used on the host.
struct Shape {
    int D, E, N, P, H, G, W, Cd, Nin, Ninp, Rin, Rout;
    float eps;
};
Shape shape_of(const dfssm_dims &d);

// Workspace carve-up of one decode call for `batch` tokens (device pointers).
struct DecodeWs {
    int32_t *acc_in, *t_in;
    float *s_in;
    float *zbuf, *xbc, *dtbuf, *gbuf;
    int32_t *acc_out, *t_out;
    float *s_out;
    float *hbuf, *xcur;      // stack only
    size_t bytes;
};
DecodeWs carve_decode_ws(const Shape &s, int batch, void *base, bool stack);

// Per-record tap pointers for one (token-group, layer) launch; any member may be null.
struct TapPtrs {
    float *h_in, *in_u, *in_s, *out_u, *out_s;
    int8_t *in_q, *out_q;
    int32_t *in_acc, *in_t, *out_acc, *out_t;
};
TapPtrs tap_offset(const dfssm_taps *t, const Shape &s, int64_t record);

// Enqueue one decode step of one layer for `batch` tokens: x_in -> x_out (may alias).
hipError_t launch_layer_decode(const Shape &s, const dfssm_layer_weights &w,
                               const dfssm_layer_state &st, const float *x_in, float *x_out,
                               int batch, const DecodeWs &ws, const TapPtrs &taps,
                               hipStream_t stream);

// Two-exchange persistent stack decode (flow2.hip), used at batch 1 when the shape fits it.
bool stack2_ok(const Shape &s, int batch);
size_t stack2_extra_ws_bytes(const Shape &s, int batch, int n_layers);
hipError_t launch_stack2(const Shape &s, const dfssm_layer_weights *layers, const dfssm_layer_state *states, int n_layers,
                         const float *final_w, const float *x0, float *y, int batch, int n_steps, void *extra,
                         const dfssm_taps *taps, bool cooperative, int **err_flag, hipStream_t stream);

// After a stack decode: status[0] = *err (0 when err is null), and when *err is set every one of
// the n floats of y becomes NaN, so that a timed-out exchange can never pass as a result.
hipError_t launch_stack_finish(const int *err, int32_t *status, float *y, int64_t n, hipStream_t stream);

// int8-code x (+-1 scaffold) GEMM with the projection epilogue (gemm.hip):
//   y[m][n] = s[m]*row_scale[n]*acc[m][n] + up_scale[n] * sum_j t'[m][j]*lora_up[n][j] (+ res[m][n])
// acc = sum_k sgn[n][k]*q[m][k]; t' = thi + tlo (bf16 split of dn_scale*s*t). rank % 8 == 0, K % 128 == 0.
// When the output has few tiles the K range is split over several workgroups; their exact int32
// partial sums and per-tile arrival counters live in `scratch` (gemm_scratch_bytes of workspace,
// no initialisation needed: the launch clears the counters itself).
struct GemmArgs {
    const int8_t *q;
    int64_t ldq;
    const int32_t *qsum;
    const float *s;
    const uint8_t *sign;
    int M, N, K;
    const uint16_t *row_scale;
    const float *up_scale;
    const int8_t *lora_up;
    int rank;
    const __bf16 *thi, *tlo;
    float *y;
    int64_t ldy;
    const float *res;      // optional
    int64_t ldres;
    int32_t *acc_tap;      // optional
    int64_t ldacc;
    void *scratch;         // split-K scratch (gemm_scratch_bytes), 256-byte aligned
    int counters_zeroed;   // the split-K arrival counters (gemm_counter_words at scratch) are already 0
                           // (every launch leaves them 0 again: the last arrival of a tile resets its counter)
};
size_t gemm_scratch_bytes(int M, int N, int K);
int gemm_counter_words(int M, int N, int K);   // arrival counters the launch needs zeroed (0: none)
hipError_t launch_gemm_pm1(const GemmArgs &a, hipStream_t stream);

// Per-token RMSNorm + int8 quantizer + int8 LoRA-down for M tokens (prefill / batched decode):
// writes codes q [M][K], s, sum of codes, and t' = dn_scale * s * t split into bf16 hi/lo [M][rank].
struct TokQuantArgs {
    const void *X;         // [M][ldx] fp32 or bf16 bit patterns
    int x_bf16;
    int64_t ldx;
    const float *W;        // norm weight [K]
    int M, K;
    float eps;
    const int8_t *lora_dn; // [rank][K]
    const float *dn_scale; // [rank]
    int rank;
    int8_t *q;             // [M][K]
    float *s;
    int32_t *qsum;
    __bf16 *thi, *tlo;     // [M][rank]
    float *tap_h, *tap_u, *tap_s;
    int8_t *tap_q;
    int32_t *tap_t;
    uint32_t *zero_words;  // optional: workgroup 0 sets these nzero words to 0 (the next GEMM's counters)
    int nzero;
};
hipError_t launch_tok_quant(const TokQuantArgs &a, hipStream_t stream);

// Prefill workspace carve-up (tokens M = batch * seqlen, chunk Q; Q = 0 for a decode step, which
// runs no chunked scan and so carves none of its buffers).
struct PrefillWs {
    int8_t *q_in, *q_out;
    float *s_in, *s_out;
    int32_t *qsum_in, *qsum_out;
    __bf16 *thi_in, *tlo_in, *thi_out, *tlo_out;
    float *Y, *xbc, *dt, *cb, *lam_end, *sloc, *gbuf;
    void *gemm_scratch;    // split-K scratch shared by the two projections (they run one after the other)
    size_t bytes;
};
PrefillWs carve_prefill_ws(const Shape &s, int batch, int seqlen, int chunk, void *base);

// DF-SSD: the codec on the state entering every chunk after the first (taps optional)
struct PrefillCodec {
    bool on;
    float *tap_pre, *tap_in;   // [nch][batch][H][P][N]
};
hipError_t launch_layer_prefill(const Shape &s, const dfssm_layer_weights &w, const dfssm_layer_state &st,
                                const void *x_in, int x_bf16, float *x_out, int batch, int seqlen, int chunk,
                                const PrefillWs &ws, const dfssm_taps *taps, hipStream_t stream,
                                const PrefillCodec *codec = nullptr);

// Per-layer SSM step + gate for `batch` tokens from ws.xbc/zbuf/dtbuf into ws.gbuf (decode.hip).
hipError_t launch_ssm_step(const Shape &s, const dfssm_layer_weights &w, const dfssm_layer_state &st,
                           const DecodeWs &ws, int batch, hipStream_t stream);

// One decode step of one layer for many tokens through the int8-MFMA projections (prefill.hip);
// pws is a prefill workspace carved for (batch, seqlen 1, chunk 0).
hipError_t launch_layer_decode_mfma(const Shape &s, const dfssm_layer_weights &w, const dfssm_layer_state &st,
                                    const float *x_in, float *x_out, int batch, const DecodeWs &dws,
                                    const PrefillWs &pws, const TapPtrs &taps, hipStream_t stream);
bool decode_uses_mfma(const Shape &s, int batch);

// Tied int8 embedding and LM head (head.hip).
struct HeadTaps {
    int8_t *q;      // [batch][D] the head's int8 codes of y
    float *s;       // [batch] their scale
    int32_t *acc;   // [batch][V] integer row sums
};
size_t head_ws_bytes(int batch);
hipError_t launch_lm_head(const int8_t *codes, const float *row_scale, int V, int D, const float *y, int batch,
                          float *logits, int32_t *next_tokens, void *ws, const HeadTaps &taps, hipStream_t stream);
hipError_t launch_embed(const int8_t *codes, const float *row_scale, int V, int D, const int32_t *tokens, int batch,
                        float *x, hipStream_t stream);

// Projection with the 17-level scaffold (dfw.hip).
struct DfwWeights {
    const uint8_t *planes;        // [5][n_out][K/8]
    const uint16_t *row_scale;    // [n_out] fp16
    const int8_t *lora_dn;        // [rank][K]
    const float *lora_dn_scale;   // [rank]
    const int8_t *lora_up;        // [n_out][rank]
    const float *lora_up_scale;   // [n_out]
};
struct DfwTaps {
    int8_t *q;      // [batch][K]
    float *s;       // [batch]
    int32_t *acc;   // [batch][n_out]
    int32_t *t;     // [batch][rank]
};
size_t dfw_ws_bytes(int K, int rank, int batch);
hipError_t launch_dfw_project(const DfwWeights &w, int n_out, int K, int rank, const float *x, float *y, int batch,
                              void *ws, const DfwTaps &taps, hipStream_t stream);

// Density field codec of SSM state rows (codec.hip): rows of N = d_state floats.
int codec_field_words(int d_state);   // 32-bit words of one row's K x K field (0: unsupported N)
hipError_t launch_state_encode(const float *ssm, int64_t rows, int N, uint32_t *fields, float *stats,
                               hipStream_t stream);
hipError_t launch_state_decode(const uint32_t *fields, const float *stats, int64_t rows, int N, float *ssm,
                               hipStream_t stream);
// The chunked scan's carry with the codec on the state entering every chunk after the first
// (replaces k_ssd_scan): state [BH][P][N] initial -> final, sloc [BH][nch][P][N] chunk contributions
// -> entering states, lam_end [BH][nch]; taps [nch][BH][P][N] or null. P must be 64.
hipError_t launch_ssd_scan_codec(float *state, float *sloc, const float *lam_end, int BH, int nch, int N, int P,
                                 float *tap_pre, float *tap_in, hipStream_t stream);

// Enqueue y = RMSNorm(h) * w for `batch` rows of length D, also copying y to `y2` when non-null.
hipError_t launch_final_norm(const float *h, const float *w, float *y, float *y2, int D, float eps,
                             int batch, hipStream_t stream);

}  // namespace dfssm
