// C ABI of the DF-SSM hot path: argument validation, workspace carving and launch sequencing.
// Every check happens before the first enqueue, so a rejected call has no side effect.
#include <stdlib.h>

#include <algorithm>

#include "dfssm_internal.h"

namespace dfssm {

Shape shape_of(const dfssm_dims &d) {
    Shape s{};
    s.D = d.d_model;
    s.E = d.d_inner;
    s.N = d.d_state;
    s.P = d.headdim;
    s.H = d.headdim > 0 ? d.d_inner / d.headdim : 0;
    s.G = d.ngroups;
    s.W = d.d_conv;
    s.Cd = d.d_inner + 2 * d.ngroups * d.d_state;
    s.Nin = 2 * d.d_inner + 2 * d.ngroups * d.d_state + s.H;
    s.Ninp = d.n_in_proj;
    s.Rin = d.rank_in;
    s.Rout = d.rank_out;
    s.eps = d.norm_eps;
    return s;
}

namespace {

constexpr size_t kAlign = 256;

int check_dims(const dfssm_dims *d) {
    if (!d) return DFSSM_EINVAL;
    if (d->d_model <= 0 || d->d_inner <= 0 || d->d_state <= 0 || d->headdim <= 0 || d->ngroups <= 0 ||
        d->d_conv <= 0 || d->n_in_proj <= 0 || d->rank_in <= 0 || d->rank_out <= 0)
        return DFSSM_EINVAL;
    if (!(d->norm_eps > 0.f) || d->norm_eps > 1.f) return DFSSM_EINVAL;
    if (d->d_model % 128 || d->d_inner % 128 || d->d_model > kMaxK || d->d_inner > kMaxK) return DFSSM_EUNSUPPORTED;
    if (d->headdim != 64 || d->d_inner % d->headdim) return DFSSM_EUNSUPPORTED;
    const int H = d->d_inner / d->headdim;
    if (d->d_state != 16 && d->d_state != 32 && d->d_state != 64 && d->d_state != 128 && d->d_state != 256)
        return DFSSM_EUNSUPPORTED;
    if (H % d->ngroups) return DFSSM_EUNSUPPORTED;
    if (d->d_conv != kConvTaps) return DFSSM_EUNSUPPORTED;
    const long nat = 2L * d->d_inner + 2L * d->ngroups * d->d_state + H;
    if (d->n_in_proj < nat || d->n_in_proj > (1 << 20)) return DFSSM_EUNSUPPORTED;
    if (d->rank_in > kMaxRank || d->rank_out > kMaxRank) return DFSSM_EUNSUPPORTED;
    return DFSSM_OK;
}

bool bad_ptr(const void *p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }
bool bad_opt_ptr(const void *p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

int check_proj(const dfssm_proj &p) {
    if (bad_ptr(p.sign) || bad_ptr(p.row_scale) || bad_ptr(p.lora_dn) || bad_ptr(p.lora_dn_scale) ||
        bad_ptr(p.lora_up) || bad_ptr(p.lora_up_scale))
        return DFSSM_EINVAL;
    return DFSSM_OK;
}

int check_weights(const dfssm_layer_weights *w) {
    if (!w) return DFSSM_EINVAL;
    int r;
    if ((r = check_proj(w->in_proj)) || (r = check_proj(w->out_proj))) return r;
    if (bad_ptr(w->conv_w) || bad_ptr(w->conv_b) || bad_ptr(w->dt_bias) || bad_ptr(w->A_log) || bad_ptr(w->D) ||
        bad_ptr(w->norm_w) || bad_ptr(w->gnorm_w))
        return DFSSM_EINVAL;
    return DFSSM_OK;
}

int check_state(const dfssm_layer_state *st) {
    if (!st || bad_ptr(st->conv) || bad_ptr(st->ssm)) return DFSSM_EINVAL;
    return DFSSM_OK;
}

int check_taps(const dfssm_taps *t) {
    if (!t) return DFSSM_OK;
    const void *ps[] = {t->h_in, t->in_u, t->in_q, t->in_s, t->in_acc, t->in_t,
                        t->out_u, t->out_q, t->out_s, t->out_acc, t->out_t};
    for (const void *p : ps)
        if (bad_opt_ptr(p)) return DFSSM_EINVAL;
    return DFSSM_OK;
}

size_t decode_ws_bytes(const Shape &s, int batch, bool stack, int n_layers = 0) {
    DecodeWs w = carve_decode_ws(s, batch, nullptr, stack);
    size_t extra = 0;
    if (stack && stack_persistent_ok(s, batch))
        extra = std::max(stack_extra_ws_bytes(s, batch, n_layers), stack2_extra_ws_bytes(s, batch, n_layers));
    else if (decode_uses_mfma(s, batch)) extra = carve_prefill_ws(s, batch, 1, 1, nullptr).bytes;
    return w.bytes + extra;
}

bool chunk_ok(int chunk) { return chunk == 16 || chunk == 32 || chunk == 64 || chunk == 128 || chunk == 256; }

size_t prefill_ws_bytes(const Shape &s, int batch, int seqlen, int chunk) {
    return carve_prefill_ws(s, batch, seqlen, chunk, nullptr).bytes;
}

// One decode step of one layer through whichever projection path suits the batch.
hipError_t decode_step(const Shape &s, const dfssm_layer_weights &w, const dfssm_layer_state &st, const float *x_in,
                       float *x_out, int batch, void *ws, bool stack, const TapPtrs &tp, hipStream_t stream) {
    const DecodeWs d = carve_decode_ws(s, batch, ws, stack);
    if (decode_uses_mfma(s, batch)) {
        const PrefillWs p = carve_prefill_ws(s, batch, 1, 1, static_cast<char *>(ws) + d.bytes);
        return launch_layer_decode_mfma(s, w, st, x_in, x_out, batch, d, p, tp, stream);
    }
    return launch_layer_decode(s, w, st, x_in, x_out, batch, d, tp, stream);
}

int env_int(const char *name, int dflt) {
    const char *v = getenv(name);
    return v ? atoi(v) : dflt;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DFSSM_OK : DFSSM_EHIP; }

}  // namespace

DecodeWs carve_decode_ws(const Shape &s, int batch, void *base, bool stack) {
    DecodeWs w{};
    size_t off = 0;
    char *b = static_cast<char *>(base);
    auto take = [&](size_t bytes) -> void * {
        void *p = b ? b + off : nullptr;
        off += align_up(bytes, kAlign);
        return p;
    };
    const size_t B = (size_t)batch;
    w.acc_in = static_cast<int32_t *>(take(B * s.Ninp * 4));
    w.t_in = static_cast<int32_t *>(take(B * kMaxRank * 4));
    w.s_in = static_cast<float *>(take(B * 4));
    w.zbuf = static_cast<float *>(take(B * s.E * 4));
    w.xbc = static_cast<float *>(take(B * s.Cd * 4));
    w.dtbuf = static_cast<float *>(take(B * s.H * 4));
    w.gbuf = static_cast<float *>(take(B * s.E * 4));
    w.acc_out = static_cast<int32_t *>(take(B * s.D * 4));
    w.t_out = static_cast<int32_t *>(take(B * kMaxRank * 4));
    w.s_out = static_cast<float *>(take(B * 4));
    if (stack) {
        w.hbuf = static_cast<float *>(take(B * s.D * 4));
        w.xcur = static_cast<float *>(take(B * s.D * 4));
    }
    w.bytes = off;
    return w;
}

TapPtrs tap_offset(const dfssm_taps *t, const Shape &s, int64_t rec) {
    TapPtrs p{};
    if (!t) return p;
    p.h_in = t->h_in ? t->h_in + rec * s.D : nullptr;
    p.in_u = t->in_u ? t->in_u + rec * s.D : nullptr;
    p.in_q = t->in_q ? t->in_q + rec * s.D : nullptr;
    p.in_s = t->in_s ? t->in_s + rec : nullptr;
    p.in_acc = t->in_acc ? t->in_acc + rec * s.Ninp : nullptr;
    p.in_t = t->in_t ? t->in_t + rec * s.Rin : nullptr;
    p.out_u = t->out_u ? t->out_u + rec * s.E : nullptr;
    p.out_q = t->out_q ? t->out_q + rec * s.E : nullptr;
    p.out_s = t->out_s ? t->out_s + rec : nullptr;
    p.out_acc = t->out_acc ? t->out_acc + rec * s.D : nullptr;
    p.out_t = t->out_t ? t->out_t + rec * s.Rout : nullptr;
    return p;
}

}  // namespace dfssm

using namespace dfssm;

extern "C" {

size_t dfssm_workspace_bytes(const dfssm_dims *dims, int32_t op, int32_t batch, int32_t seqlen,
                             int32_t n_layers) {
    if (check_dims(dims) != DFSSM_OK || batch <= 0) return 0;
    const Shape s = shape_of(*dims);
    switch (op) {
        case DFSSM_OP_LAYER_DECODE: return decode_ws_bytes(s, batch, false);
        case DFSSM_OP_STACK_DECODE:
            if (n_layers <= 0) return 0;
            return decode_ws_bytes(s, batch, true, n_layers);
        case DFSSM_OP_LAYER_PREFILL:
            if (seqlen <= 0 || seqlen > 65536 || batch > 64 || (int64_t)batch * seqlen > (1 << 20) || s.Rin % 8 ||
                s.Rout % 8)
                return 0;
            {   // enough for every supported chunk length
                size_t mx = 0;
                for (int c = 16; c <= 256; c *= 2) mx = std::max(mx, prefill_ws_bytes(s, batch, seqlen, c));
                return mx;
            }
        default: return 0;
    }
}

int dfssm_layer_decode(const dfssm_dims *dims, const dfssm_layer_weights *w, const dfssm_layer_state *state,
                       const float *x_in, float *x_out, int32_t batch, void *ws, size_t ws_bytes,
                       const dfssm_taps *taps, void *stream) {
    int r;
    if ((r = check_dims(dims))) return r;
    if ((r = check_weights(w)) || (r = check_state(state)) || (r = check_taps(taps))) return r;
    if (bad_ptr(x_in) || bad_ptr(x_out) || batch <= 0) return DFSSM_EINVAL;
    if (batch > 4096) return DFSSM_EUNSUPPORTED;
    if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1))) return DFSSM_EINVAL;
    const Shape s = shape_of(*dims);
    if (ws_bytes < decode_ws_bytes(s, batch, false)) return DFSSM_EWORKSPACE;
    const TapPtrs tp = tap_offset(taps, s, 0);
    return hip_status(decode_step(s, *w, *state, x_in, x_out, batch, ws, false, tp, static_cast<hipStream_t>(stream)));
}

int dfssm_layer_prefill(const dfssm_dims *dims, const dfssm_layer_weights *w, const dfssm_layer_state *state,
                        const void *x_in, int32_t x_dtype, float *x_out, int32_t batch, int32_t seqlen,
                        int32_t chunk, void *ws, size_t ws_bytes, const dfssm_taps *taps, void *stream) {
    int r;
    if ((r = check_dims(dims))) return r;
    if ((r = check_weights(w)) || (r = check_state(state)) || (r = check_taps(taps))) return r;
    if (bad_ptr(x_in) || bad_ptr(x_out) || batch <= 0 || seqlen <= 0) return DFSSM_EINVAL;
    if (x_dtype != DFSSM_F32 && x_dtype != DFSSM_BF16) return DFSSM_EINVAL;
    if (x_in == static_cast<const void *>(x_out)) return DFSSM_EINVAL;
    if (!chunk_ok(chunk)) return DFSSM_EUNSUPPORTED;
    if (seqlen > 65536 || batch > 64 || (int64_t)batch * seqlen > (1 << 20)) return DFSSM_EUNSUPPORTED;
    const Shape s = shape_of(*dims);
    if (s.Rin % 8 || s.Rout % 8) return DFSSM_EUNSUPPORTED;
    if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1))) return DFSSM_EINVAL;
    if (ws_bytes < prefill_ws_bytes(s, batch, seqlen, chunk)) return DFSSM_EWORKSPACE;
    const PrefillWs p = carve_prefill_ws(s, batch, seqlen, chunk, ws);
    return hip_status(launch_layer_prefill(s, *w, *state, x_in, x_dtype == DFSSM_BF16, x_out, batch, seqlen, chunk, p,
                                           taps, static_cast<hipStream_t>(stream)));
}

int dfssm_stack_decode(const dfssm_dims *dims, const dfssm_layer_weights *layers, const dfssm_layer_state *states,
                       int32_t n_layers, const float *final_norm_w, const float *x0, float *y, int32_t batch,
                       int32_t n_steps, void *ws, size_t ws_bytes, const dfssm_taps *taps, void *stream) {
    int r;
    if ((r = check_dims(dims))) return r;
    if (!layers || !states || n_layers <= 0 || n_steps <= 0 || batch <= 0) return DFSSM_EINVAL;
    if (n_layers > 1024 || n_steps > (1 << 20) || batch > 4096) return DFSSM_EUNSUPPORTED;
    for (int l = 0; l < n_layers; ++l)
        if ((r = check_weights(&layers[l])) || (r = check_state(&states[l]))) return r;
    if ((r = check_taps(taps))) return r;
    if (bad_ptr(final_norm_w) || bad_ptr(x0) || bad_ptr(y)) return DFSSM_EINVAL;
    if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1))) return DFSSM_EINVAL;
    const Shape s = shape_of(*dims);
    if (ws_bytes < decode_ws_bytes(s, batch, true, n_layers)) return DFSSM_EWORKSPACE;
    const DecodeWs wsp = carve_decode_ws(s, batch, ws, true);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (stack_persistent_ok(s, batch) && stack2_ok(s, batch))
        return hip_status(launch_stack2(s, layers, states, n_layers, final_norm_w, x0, y, batch, n_steps,
                                        static_cast<char *>(ws) + wsp.bytes, taps, st));
    if (stack_persistent_ok(s, batch)) {
        // DFSSM_STACK_MAX_WGS caps the resident grid (a tuning knob; 0 = as many as useful)
        e = launch_stack_persistent(s, layers, states, n_layers, final_norm_w, x0, y, batch, n_steps, wsp,
                                    static_cast<char *>(ws) + wsp.bytes, taps, env_int("DFSSM_STACK_MAX_WGS", 0), st);
        return hip_status(e);
    }
    const int64_t rowsz = (int64_t)batch * s.D;
    for (int t = 0; t < n_steps; ++t) {
        const float *xin = t == 0 ? x0 : y + (t - 1) * rowsz;
        for (int l = 0; l < n_layers; ++l) {
            const TapPtrs tp = tap_offset(taps, s, ((int64_t)t * n_layers + l) * batch);
            e = decode_step(s, layers[l], states[l], l == 0 ? xin : wsp.hbuf, wsp.hbuf, batch, ws, true, tp, st);
            if (e != hipSuccess) return DFSSM_EHIP;
        }
        e = launch_final_norm(wsp.hbuf, final_norm_w, y + t * rowsz, nullptr, s.D, s.eps, batch, st);
        if (e != hipSuccess) return DFSSM_EHIP;
    }
    return DFSSM_OK;
}

const char *dfssm_strerror(int status) {
    switch (status) {
        case DFSSM_OK: return "success";
        case DFSSM_EINVAL: return "invalid argument (null or misaligned pointer, or non-positive size)";
        case DFSSM_EUNSUPPORTED: return "unsupported shape or size";
        case DFSSM_EWORKSPACE: return "workspace too small";
        case DFSSM_EHIP: return "HIP runtime or kernel launch error";
        default: return "unknown status";
    }
}

}  // extern "C"
