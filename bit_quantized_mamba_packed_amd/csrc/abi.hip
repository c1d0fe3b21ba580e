// C ABI of the DF-SSM hot path: argument validation, workspace carving and launch sequencing.
// Every check happens before the first enqueue, so a rejected call has no side effect.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

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

// Fixed device scratch of dfssm_layer_decode_noalloc: every GPU the library runs on holds its own
// copy until the process ends. In host code `scratch` names a host-side stand-in, never the device
// array: its device address comes from hipGetSymbolAddress, once per device (scratch_on_device).
constexpr size_t kNoAllocScratchBytes = DFSSM_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxScratchDevices = 64;
std::atomic<void *> g_scratch[kMaxScratchDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array, looked up on the first call on that device.
hipError_t scratch_on_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

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

// A batched stack decode of at least kHalvesMinBatch sequences runs as two batch halves on two
// streams (stack_decode_halves).
constexpr int kHalvesMinBatch = 32;

// Bytes one decode_step of `batch` sequences carves from its workspace.
size_t step_ws_bytes(const Shape &s, int batch, bool stack) {
    size_t b = carve_decode_ws(s, batch, nullptr, stack).bytes;
    if (decode_uses_mfma(s, batch)) b += carve_prefill_ws(s, batch, 1, 0, nullptr).bytes;
    return b;
}

// One half's share of a halved stack decode's workspace (the larger half: the second).
size_t half_ws_bytes(const Shape &s, int batch) { return align_up(step_ws_bytes(s, batch - batch / 2, true), kAlign); }

// A stack decode's workspace starts with its status word (kAlign bytes), then the decode carve (the
// persistent kernel's tables and exchange words at batch 1, two half carves at kHalvesMinBatch and up).
size_t decode_ws_bytes(const Shape &s, int batch, bool stack, int n_layers = 0) {
    if (!stack) return step_ws_bytes(s, batch, false);
    size_t b = step_ws_bytes(s, batch, true);
    if (stack2_ok(s, batch)) b += stack2_extra_ws_bytes(s, batch, n_layers);
    if (batch >= kHalvesMinBatch) b = std::max(b, 2 * half_ws_bytes(s, batch));
    return kAlign + b;
}

bool chunk_ok(int chunk) { return chunk == 16 || chunk == 32 || chunk == 64 || chunk == 128 || chunk == 256; }

size_t prefill_ws_bytes(const Shape &s, int batch, int seqlen, int chunk) {
    return carve_prefill_ws(s, batch, seqlen, chunk, nullptr).bytes;
}

bool prefill_size_ok(const Shape &s, int batch, int seqlen) {
    return seqlen > 0 && seqlen <= 65536 && batch > 0 && batch <= 64 && (int64_t)batch * seqlen <= (1 << 20) &&
           s.Rin % 8 == 0 && s.Rout % 8 == 0;
}

// Largest prefill carve over the supported chunk lengths.
size_t prefill_ws_any_chunk(const Shape &s, int batch, int seqlen) {
    size_t mx = 0;
    for (int c = 16; c <= 256; c *= 2) mx = std::max(mx, prefill_ws_bytes(s, batch, seqlen, c));
    return mx;
}

// A stack prefill: one residual buffer [batch][seqlen][D] fp32, then one layer's prefill carve.
size_t stack_prefill_hbuf_bytes(const Shape &s, int batch, int seqlen) {
    return align_up((size_t)batch * seqlen * s.D * 4, kAlign);
}

// Tap pointers of one layer's records inside [n_layers][records_per_layer][...] buffers.
dfssm_taps taps_for_layer(const dfssm_taps *t, const Shape &s, int64_t rec) {
    dfssm_taps o{};
    if (!t) return o;
    const TapPtrs p = tap_offset(t, s, rec);
    o.h_in = p.h_in;
    o.in_u = p.in_u;
    o.in_q = p.in_q;
    o.in_s = p.in_s;
    o.in_acc = p.in_acc;
    o.in_t = p.in_t;
    o.out_u = p.out_u;
    o.out_q = p.out_q;
    o.out_s = p.out_s;
    o.out_acc = p.out_acc;
    o.out_t = p.out_t;
    return o;
}

// One decode step of one layer through whichever projection path suits the batch.
hipError_t decode_step(const Shape &s, const dfssm_layer_weights &w, const dfssm_layer_state &st, const float *x_in,
                       float *x_out, int batch, void *ws, bool stack, const TapPtrs &tp, hipStream_t stream) {
    const DecodeWs d = carve_decode_ws(s, batch, ws, stack);
    if (decode_uses_mfma(s, batch)) {
        const PrefillWs p = carve_prefill_ws(s, batch, 1, 0, static_cast<char *>(ws) + d.bytes);
        return launch_layer_decode_mfma(s, w, st, x_in, x_out, batch, d, p, tp, stream);
    }
    return launch_layer_decode(s, w, st, x_in, x_out, batch, d, tp, stream);
}

int hip_status(hipError_t e) { return e == hipSuccess ? DFSSM_OK : DFSSM_EHIP; }

// The second stream of halved stack decodes, one per device (default priority, created on first
// use, kept until the process ends), and the two events that fork it from the caller's stream and
// join it back. Every call re-records the events, so an enqueue holds g_halves_mu throughout.
constexpr int kMaxHalvesDevices = 64;
struct HalvesStream {
    hipStream_t s;
    hipEvent_t fork, join;
};
HalvesStream g_halves[kMaxHalvesDevices];
std::mutex g_halves_mu;

// A per-layer stack decode as two batch halves [0, b0) and [b0, batch), b0 = batch / 2: the first on
// the caller's stream, the second on the device's halves stream, their launches interleaved layer by
// layer. A half's sequences, states, outputs and tap records are contiguous slices of the caller's,
// and the halves share nothing but the (read-only) weights, so the results are those of the single
// stream; while one half's SSM step streams its state the other's projections and quantizers, which
// do not fill the GPU, run beside it.
hipError_t stack_decode_halves(const Shape &s, const dfssm_layer_weights *layers, const dfssm_layer_state *states,
                               int n_layers, const float *final_norm_w, const float *x0, float *y, int batch,
                               int n_steps, char *wsd, const dfssm_taps *taps, hipStream_t st) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxHalvesDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_halves_mu);
    HalvesStream &hs = g_halves[dev];
    if (!hs.s) {
        if ((e = hipEventCreateWithFlags(&hs.fork, hipEventDisableTiming)) != hipSuccess) return e;
        if ((e = hipEventCreateWithFlags(&hs.join, hipEventDisableTiming)) != hipSuccess) return e;
        if ((e = hipStreamCreateWithFlags(&hs.s, hipStreamNonBlocking)) != hipSuccess) return e;
    }
    const int b0 = batch / 2, nb[2] = {b0, batch - b0};
    const hipStream_t xs[2] = {st, hs.s};
    const size_t hb = half_ws_bytes(s, batch);
    std::vector<dfssm_layer_state> hst(2 * (size_t)n_layers);
    DecodeWs dws[2];
    for (int i = 0; i < 2; ++i) {
        const int64_t first = i ? b0 : 0;
        dws[i] = carve_decode_ws(s, nb[i], wsd + i * hb, true);
        for (int l = 0; l < n_layers; ++l) {
            hst[i * n_layers + l].conv = states[l].conv + first * s.Cd * (kConvTaps - 1);
            hst[i * n_layers + l].ssm = states[l].ssm + first * s.H * s.P * s.N;
        }
    }
    if ((e = hipEventRecord(hs.fork, st)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(hs.s, hs.fork, 0)) != hipSuccess) return e;
    const int64_t rowsz = (int64_t)batch * s.D;
    for (int t = 0; t < n_steps; ++t) {
        for (int l = 0; l < n_layers; ++l)
            for (int i = 0; i < 2; ++i) {
                const int64_t first = i ? b0 : 0;
                const float *xin = (t == 0 ? x0 : y + (t - 1) * rowsz) + first * s.D;
                const TapPtrs tp = tap_offset(taps, s, ((int64_t)t * n_layers + l) * batch + first);
                e = decode_step(s, layers[l], hst[i * n_layers + l], l == 0 ? xin : dws[i].hbuf, dws[i].hbuf, nb[i],
                                wsd + i * hb, true, tp, xs[i]);
                if (e != hipSuccess) return e;
            }
        for (int i = 0; i < 2; ++i) {
            e = launch_final_norm(dws[i].hbuf, final_norm_w, y + t * rowsz + (i ? b0 : 0) * s.D, nullptr, s.D, s.eps,
                                  nb[i], xs[i]);
            if (e != hipSuccess) return e;
        }
    }
    if ((e = hipEventRecord(hs.join, hs.s)) != hipSuccess) return e;
    return hipStreamWaitEvent(st, hs.join, 0);
}

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
            if (!prefill_size_ok(s, batch, seqlen)) return 0;
            return prefill_ws_any_chunk(s, batch, seqlen);
        case DFSSM_OP_LM_HEAD:
            if (batch > 4096) return 0;
            return head_ws_bytes(batch);
        case DFSSM_OP_STACK_PREFILL:
            if (n_layers <= 0 || !prefill_size_ok(s, batch, seqlen)) return 0;
            return stack_prefill_hbuf_bytes(s, batch, seqlen) + prefill_ws_any_chunk(s, batch, seqlen);
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

int dfssm_layer_decode_noalloc(const dfssm_dims *dims, const dfssm_layer_weights *w,
                               const dfssm_layer_state *state, const float *x_in, float *x_out, int32_t batch,
                               const dfssm_taps *taps, void *stream) {
    int r;
    if ((r = check_dims(dims))) return r;
    if ((r = check_weights(w)) || (r = check_state(state)) || (r = check_taps(taps))) return r;
    if (bad_ptr(x_in) || bad_ptr(x_out) || batch <= 0) return DFSSM_EINVAL;
    if (batch > 4096) return DFSSM_EUNSUPPORTED;
    const Shape s = shape_of(*dims);
    if (decode_ws_bytes(s, batch, false) > kNoAllocScratchBytes) return DFSSM_EWORKSPACE;
    void *ws = nullptr;
    if (scratch_on_device(&ws) != hipSuccess) return DFSSM_EHIP;
    const TapPtrs tp = tap_offset(taps, s, 0);
    return hip_status(decode_step(s, *w, *state, x_in, x_out, batch, ws, false, tp, static_cast<hipStream_t>(stream)));
}

int dfssm_layer_prefill(const dfssm_dims *dims, const dfssm_layer_weights *w, const dfssm_layer_state *state,
                        const void *x_in, int32_t x_dtype, float *x_out, int32_t batch, int32_t seqlen,
                        int32_t chunk, void *ws, size_t ws_bytes, const dfssm_taps *taps, void *stream) {
    return dfssm_layer_prefill_ex(dims, w, state, x_in, x_dtype, x_out, batch, seqlen, chunk, ws, ws_bytes, taps,
                                  nullptr, stream);
}

int dfssm_layer_prefill_ex(const dfssm_dims *dims, const dfssm_layer_weights *w, const dfssm_layer_state *state,
                           const void *x_in, int32_t x_dtype, float *x_out, int32_t batch, int32_t seqlen,
                           int32_t chunk, void *ws, size_t ws_bytes, const dfssm_taps *taps,
                           const dfssm_prefill_opts *opts, void *stream) {
    int r;
    const dfssm_prefill_opts o = opts ? *opts : dfssm_prefill_opts{};
    if ((o.state_codec != 0 && o.state_codec != 1) || o.reserved != 0) return DFSSM_EINVAL;
    if (bad_opt_ptr(o.chunk_state_pre) || bad_opt_ptr(o.chunk_state_in)) return DFSSM_EINVAL;
    if (!o.state_codec && (o.chunk_state_pre || o.chunk_state_in)) return DFSSM_EINVAL;
    if ((r = check_dims(dims))) return r;
    if ((r = check_weights(w)) || (r = check_state(state)) || (r = check_taps(taps))) return r;
    if (bad_ptr(x_in) || bad_ptr(x_out) || batch <= 0 || seqlen <= 0) return DFSSM_EINVAL;
    if (x_dtype != DFSSM_F32 && x_dtype != DFSSM_BF16) return DFSSM_EINVAL;
    if (x_in == static_cast<const void *>(x_out)) return DFSSM_EINVAL;
    if (!chunk_ok(chunk)) return DFSSM_EUNSUPPORTED;
    const Shape s = shape_of(*dims);
    if (!prefill_size_ok(s, batch, seqlen)) return DFSSM_EUNSUPPORTED;
    if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1))) return DFSSM_EINVAL;
    if (ws_bytes < prefill_ws_bytes(s, batch, seqlen, chunk)) return DFSSM_EWORKSPACE;
    const PrefillWs p = carve_prefill_ws(s, batch, seqlen, chunk, ws);
    const PrefillCodec pc{o.state_codec == 1, o.chunk_state_pre, o.chunk_state_in};
    return hip_status(launch_layer_prefill(s, *w, *state, x_in, x_dtype == DFSSM_BF16, x_out, batch, seqlen, chunk, p,
                                           taps, static_cast<hipStream_t>(stream), &pc));
}

int dfssm_stack_decode(const dfssm_dims *dims, const dfssm_layer_weights *layers, const dfssm_layer_state *states,
                       int32_t n_layers, const float *final_norm_w, const float *x0, float *y, int32_t batch,
                       int32_t n_steps, void *ws, size_t ws_bytes, const dfssm_taps *taps, void *stream) {
    return dfssm_stack_decode_ex(dims, layers, states, n_layers, final_norm_w, x0, y, batch, n_steps, ws, ws_bytes,
                                 taps, nullptr, stream);
}

int dfssm_stack_decode_ex(const dfssm_dims *dims, const dfssm_layer_weights *layers, const dfssm_layer_state *states,
                          int32_t n_layers, const float *final_norm_w, const float *x0, float *y, int32_t batch,
                          int32_t n_steps, void *ws, size_t ws_bytes, const dfssm_taps *taps,
                          const dfssm_stack_opts *opts, void *stream) {
    int r;
    if ((r = check_dims(dims))) return r;
    if (!layers || !states || n_layers <= 0 || n_steps <= 0 || batch <= 0) return DFSSM_EINVAL;
    if (n_layers > 1024 || n_steps > (1 << 20) || batch > 4096) return DFSSM_EUNSUPPORTED;
    for (int l = 0; l < n_layers; ++l)
        if ((r = check_weights(&layers[l])) || (r = check_state(&states[l]))) return r;
    if ((r = check_taps(taps))) return r;
    if (bad_ptr(final_norm_w) || bad_ptr(x0) || bad_ptr(y)) return DFSSM_EINVAL;
    if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1))) return DFSSM_EINVAL;
    const dfssm_stack_opts o = opts ? *opts : dfssm_stack_opts{};
    if (o.path < DFSSM_PATH_AUTO || o.path > DFSSM_PATH_PER_LAYER) return DFSSM_EINVAL;
    if (o.launch != DFSSM_LAUNCH_COOPERATIVE && o.launch != DFSSM_LAUNCH_ORDINARY) return DFSSM_EINVAL;
    const Shape s = shape_of(*dims);
    if (ws_bytes < decode_ws_bytes(s, batch, true, n_layers)) return DFSSM_EWORKSPACE;
    const bool flow = stack2_ok(s, batch);
    int path = o.path;
    if (path == DFSSM_PATH_AUTO) path = flow ? DFSSM_PATH_FLOW : DFSSM_PATH_PER_LAYER;
    if (path == DFSSM_PATH_FLOW && !flow) return DFSSM_EUNSUPPORTED;
    int32_t *status = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + DFSSM_STACK_STATUS_OFFSET);
    char *wsd = static_cast<char *>(ws) + kAlign;
    const DecodeWs wsp = carve_decode_ws(s, batch, wsd, true);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t ny = (int64_t)n_steps * batch * s.D;
    int *err = nullptr;
    hipError_t e;
    if (path == DFSSM_PATH_FLOW) {
        e = launch_stack2(s, layers, states, n_layers, final_norm_w, x0, y, batch, n_steps, wsd + wsp.bytes, taps,
                          o.launch == DFSSM_LAUNCH_COOPERATIVE, &err, st);
        if (e != hipSuccess) return DFSSM_EHIP;
        return hip_status(launch_stack_finish(err, status, y, ny, st));
    }
    if (batch >= kHalvesMinBatch) {
        e = stack_decode_halves(s, layers, states, n_layers, final_norm_w, x0, y, batch, n_steps, wsd, taps, st);
        if (e != hipSuccess) return DFSSM_EHIP;
        return hip_status(launch_stack_finish(nullptr, status, y, ny, st));
    }
    const int64_t rowsz = (int64_t)batch * s.D;
    for (int t = 0; t < n_steps; ++t) {
        const float *xin = t == 0 ? x0 : y + (t - 1) * rowsz;
        for (int l = 0; l < n_layers; ++l) {
            const TapPtrs tp = tap_offset(taps, s, ((int64_t)t * n_layers + l) * batch);
            e = decode_step(s, layers[l], states[l], l == 0 ? xin : wsp.hbuf, wsp.hbuf, batch, wsd, true, tp, st);
            if (e != hipSuccess) return DFSSM_EHIP;
        }
        e = launch_final_norm(wsp.hbuf, final_norm_w, y + t * rowsz, nullptr, s.D, s.eps, batch, st);
        if (e != hipSuccess) return DFSSM_EHIP;
    }
    return hip_status(launch_stack_finish(nullptr, status, y, ny, st));
}

int dfssm_stack_prefill(const dfssm_dims *dims, const dfssm_layer_weights *layers, const dfssm_layer_state *states,
                        int32_t n_layers, const float *final_norm_w, const void *x_in, int32_t x_dtype, float *y,
                        int32_t batch, int32_t seqlen, int32_t chunk, void *ws, size_t ws_bytes,
                        const dfssm_taps *taps, void *stream) {
    return dfssm_stack_prefill_ex(dims, layers, states, n_layers, final_norm_w, x_in, x_dtype, y, batch, seqlen, chunk,
                                  ws, ws_bytes, taps, nullptr, stream);
}

int dfssm_stack_prefill_ex(const dfssm_dims *dims, const dfssm_layer_weights *layers, const dfssm_layer_state *states,
                           int32_t n_layers, const float *final_norm_w, const void *x_in, int32_t x_dtype, float *y,
                           int32_t batch, int32_t seqlen, int32_t chunk, void *ws, size_t ws_bytes,
                           const dfssm_taps *taps, const dfssm_prefill_opts *opts, void *stream) {
    int r;
    const dfssm_prefill_opts o = opts ? *opts : dfssm_prefill_opts{};
    if ((o.state_codec != 0 && o.state_codec != 1) || o.reserved != 0) return DFSSM_EINVAL;
    if (o.chunk_state_pre || o.chunk_state_in) return DFSSM_EINVAL;   // per-layer taps: the layer call
    if ((r = check_dims(dims))) return r;
    if (!layers || !states || n_layers <= 0 || batch <= 0 || seqlen <= 0) return DFSSM_EINVAL;
    if (n_layers > 1024) return DFSSM_EUNSUPPORTED;
    for (int l = 0; l < n_layers; ++l)
        if ((r = check_weights(&layers[l])) || (r = check_state(&states[l]))) return r;
    if ((r = check_taps(taps))) return r;
    if (bad_ptr(final_norm_w) || bad_ptr(x_in) || bad_ptr(y)) return DFSSM_EINVAL;
    if (x_dtype != DFSSM_F32 && x_dtype != DFSSM_BF16) return DFSSM_EINVAL;
    if (x_in == static_cast<const void *>(y)) return DFSSM_EINVAL;
    if (!chunk_ok(chunk)) return DFSSM_EUNSUPPORTED;
    const Shape s = shape_of(*dims);
    if (!prefill_size_ok(s, batch, seqlen)) return DFSSM_EUNSUPPORTED;
    if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1))) return DFSSM_EINVAL;
    const size_t hb = stack_prefill_hbuf_bytes(s, batch, seqlen);
    if (ws_bytes < hb + prefill_ws_bytes(s, batch, seqlen, chunk)) return DFSSM_EWORKSPACE;
    float *hbuf = static_cast<float *>(ws);
    const PrefillWs p = carve_prefill_ws(s, batch, seqlen, chunk, static_cast<char *>(ws) + hb);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t per_layer = (int64_t)batch * seqlen;
    // layer outputs alternate between y and the workspace buffer so that the last one lands in y,
    // which the stack's final RMSNorm then rewrites in place (row by row, each row read first)
    for (int l = 0; l < n_layers; ++l) {
        const void *src = l == 0 ? x_in : ((n_layers - l) % 2 == 0 ? static_cast<const void *>(y) : hbuf);
        float *dst = (n_layers - 1 - l) % 2 == 0 ? y : hbuf;
        const dfssm_taps tl = taps_for_layer(taps, s, l * per_layer);
        const PrefillCodec pc{o.state_codec == 1, nullptr, nullptr};
        hipError_t e = launch_layer_prefill(s, layers[l], states[l], src, l == 0 && x_dtype == DFSSM_BF16, dst, batch,
                                            seqlen, chunk, p, taps ? &tl : nullptr, st, &pc);
        if (e != hipSuccess) return DFSSM_EHIP;
    }
    return hip_status(launch_final_norm(y, final_norm_w, y, nullptr, s.D, s.eps, (int)per_layer, st));
}

static int check_embedding(const dfssm_embedding *e) {
    if (!e || bad_ptr(e->codes) || bad_ptr(e->row_scale) || e->vocab <= 0 || e->d_model <= 0) return DFSSM_EINVAL;
    if (e->d_model % 128 || e->d_model > kMaxK || e->vocab > (1 << 24)) return DFSSM_EUNSUPPORTED;
    return DFSSM_OK;
}

int dfssm_embed(const dfssm_embedding *emb, const int32_t *tokens, int32_t batch, float *x, void *stream) {
    int r;
    if ((r = check_embedding(emb))) return r;
    if (bad_ptr(tokens) || bad_ptr(x) || batch <= 0) return DFSSM_EINVAL;
    if (batch > 4096) return DFSSM_EUNSUPPORTED;
    return hip_status(launch_embed(emb->codes, emb->row_scale, emb->vocab, emb->d_model, tokens, batch, x,
                                   static_cast<hipStream_t>(stream)));
}

int dfssm_lm_head(const dfssm_embedding *emb, const float *y, int32_t batch, float *logits, int32_t *next_tokens,
                  void *ws, size_t ws_bytes, const dfssm_head_taps *taps, void *stream) {
    int r;
    if ((r = check_embedding(emb))) return r;
    if (bad_ptr(y) || batch <= 0 || bad_opt_ptr(logits) || bad_opt_ptr(next_tokens)) return DFSSM_EINVAL;
    if (!logits && !next_tokens) return DFSSM_EINVAL;
    if (taps && (bad_opt_ptr(taps->q) || bad_opt_ptr(taps->s) || bad_opt_ptr(taps->acc))) return DFSSM_EINVAL;
    if (batch > 4096) return DFSSM_EUNSUPPORTED;
    if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & 255)) return DFSSM_EINVAL;
    if (ws_bytes < head_ws_bytes(batch)) return DFSSM_EWORKSPACE;
    const HeadTaps t{taps ? taps->q : nullptr, taps ? taps->s : nullptr, taps ? taps->acc : nullptr};
    return hip_status(launch_lm_head(emb->codes, emb->row_scale, emb->vocab, emb->d_model, y, batch, logits,
                                     next_tokens, ws, t, static_cast<hipStream_t>(stream)));
}

static bool dfw_shape_ok(int32_t n_out, int32_t n_in, int32_t rank, int32_t batch) {
    return n_in >= 128 && n_in <= 8192 && n_in % 128 == 0 && n_out >= 1 && n_out <= (1 << 20) && rank >= 1 &&
           rank <= 64 && batch >= 1 && batch <= 256;
}

size_t dfssm_dfw_workspace_bytes(int32_t n_in, int32_t rank, int32_t batch) {
    if (!dfw_shape_ok(1, n_in, rank, batch)) return 0;
    return dfw_ws_bytes(n_in, rank, batch);
}

int dfssm_dfw_project(const dfssm_dfw_proj *w, int32_t n_out, int32_t n_in, int32_t rank, const float *x, float *y,
                      int32_t batch, void *ws, size_t ws_bytes, const dfssm_dfw_taps *taps, void *stream) {
    if (!w || bad_ptr(x) || bad_ptr(y) || bad_ptr(ws)) return DFSSM_EINVAL;
    if (bad_ptr(w->planes) || bad_ptr(w->row_scale) || bad_ptr(w->lora_dn) || bad_ptr(w->lora_dn_scale) ||
        bad_ptr(w->lora_up) || bad_ptr(w->lora_up_scale))
        return DFSSM_EINVAL;
    if (n_out <= 0 || n_in <= 0 || rank <= 0 || batch <= 0) return DFSSM_EINVAL;
    if (!dfw_shape_ok(n_out, n_in, rank, batch)) return DFSSM_EUNSUPPORTED;
    if (taps && (bad_opt_ptr(taps->q) || bad_opt_ptr(taps->s) || bad_opt_ptr(taps->acc) || bad_opt_ptr(taps->t)))
        return DFSSM_EINVAL;
    if (ws_bytes < dfw_ws_bytes(n_in, rank, batch)) return DFSSM_EWORKSPACE;
    const DfwWeights dw{w->planes, w->row_scale, w->lora_dn, w->lora_dn_scale, w->lora_up, w->lora_up_scale};
    DfwTaps tp{};
    if (taps) tp = DfwTaps{taps->q, taps->s, taps->acc, taps->t};
    return hip_status(launch_dfw_project(dw, n_out, n_in, rank, x, y, batch, ws, tp,
                                         static_cast<hipStream_t>(stream)));
}

int32_t dfssm_state_field_words(int32_t d_state) { return codec_field_words(d_state); }

int dfssm_state_encode(const dfssm_dims *dims, const float *ssm, int32_t batch, uint32_t *fields, float *stats,
                       void *stream) {
    int r;
    if ((r = check_dims(dims))) return r;
    if (bad_ptr(ssm) || bad_ptr(fields) || bad_ptr(stats) || batch <= 0) return DFSSM_EINVAL;
    if (batch > 4096) return DFSSM_EUNSUPPORTED;
    const Shape s = shape_of(*dims);
    if (codec_field_words(s.N) == 0) return DFSSM_EUNSUPPORTED;
    return hip_status(launch_state_encode(ssm, (int64_t)batch * s.H * s.P, s.N, fields, stats,
                                          static_cast<hipStream_t>(stream)));
}

int dfssm_state_decode(const dfssm_dims *dims, const uint32_t *fields, const float *stats, int32_t batch, float *ssm,
                       void *stream) {
    int r;
    if ((r = check_dims(dims))) return r;
    if (bad_ptr(ssm) || bad_ptr(fields) || bad_ptr(stats) || batch <= 0) return DFSSM_EINVAL;
    if (batch > 4096) return DFSSM_EUNSUPPORTED;
    const Shape s = shape_of(*dims);
    if (codec_field_words(s.N) == 0) return DFSSM_EUNSUPPORTED;
    return hip_status(launch_state_decode(fields, stats, (int64_t)batch * s.H * s.P, s.N, ssm,
                                          static_cast<hipStream_t>(stream)));
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
