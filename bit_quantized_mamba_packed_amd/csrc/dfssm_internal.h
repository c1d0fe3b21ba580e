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

// Extra workspace of the persistent stack kernel (layer table, barrier counter, error flag,
// raw B/C values) and its launcher; batch <= kGemvMaxBatch.
size_t stack_extra_ws_bytes(const Shape &s, int batch, int n_layers);
hipError_t launch_stack_persistent(const Shape &s, const dfssm_layer_weights *layers,
                                   const dfssm_layer_state *states, int n_layers, const float *final_w,
                                   const float *x0, float *y, int batch, int n_steps, const DecodeWs &ws,
                                   void *extra, const dfssm_taps *taps, int max_wgs, hipStream_t stream);
bool stack_persistent_ok(const Shape &s, int batch);

// Enqueue y = RMSNorm(h) * w for `batch` rows of length D, also copying y to `y2` when non-null.
hipError_t launch_final_norm(const float *h, const float *w, float *y, float *y2, int D, float eps,
                             int batch, hipStream_t stream);

}  // namespace dfssm
