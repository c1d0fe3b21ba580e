// DF-SSM layer prefill for M = batch * seqlen tokens on gfx950.
//
// The result is, by definition, seqlen successive decode steps (quantization is per token); the
// SSM part is evaluated with the chunked state-space-duality form of Mamba-2 (the SSD paper the
// DF-SSM paper builds on, §2). Per layer:
//   1 k_tok_quant      per token: RMSNorm + int8 quantizer, int8 LoRA-down, t' split to bf16
//   2 k_gemm_pm1       in_proj over all tokens (int8 MFMA) with the Eq. (3) epilogue -> Y
//   3 k_conv_seq       causal conv over the sequence + SiLU (x, B, C); softplus(dt + dt_bias)
//   4 k_conv_handoff   final conv state = the last d_conv-1 pre-activation inputs
//   5 SSD, chunk length Q, Lam_t = sum_{tau <= t in chunk} dt_tau A (per head):
//       k_ssd_lam      Lam within each chunk and its end value
//       k_ssd_cb       CB[t][s] = C_t . B_s for each chunk and group (shared by the group's heads)
//       k_ssd_ydiag    Y_diag[t] = sum_{s <= t} exp(Lam_t - Lam_s) CB[t][s] dt_s x_s
//       k_ssd_sloc     S_loc = sum_s exp(Lam_end - Lam_s) dt_s x_s (x) B_s
//       k_ssd_scan     S_in(c) = state entering chunk c; S <- exp(Lam_end) S + S_loc (sequential in c)
//       k_ssd_yoff     y = Y_diag + exp(Lam_t) C_t . S_in + D x; g = y * SiLU(z)
//     (exponentials are always taken of differences of Lam)
//   6 k_tok_quant      gated RMSNorm + quantizer + LoRA-down of g
//   7 k_gemm_pm1       out_proj with the residual add -> x_out
#include "decode_device.h"

namespace dfssm {

namespace {

constexpr int TT = 64;  // token / feature tile of the SSD kernels

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

__global__ __launch_bounds__(kBlock) void k_widen_bf16(const uint16_t *x, float *y, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < n) y[i] = bf16_bits_to_float(x[i]);
}

// ------------------------------------------------------------------ 1/6 per-token quantizer
__global__ __launch_bounds__(kBlock) void k_tok_quant(TokQuantArgs a) {
    __shared__ float red[2 * kWaves];
    __shared__ int ired[kWaves];
    __shared__ __align__(16) int8_t sq[kMaxK];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = blockIdx.x;
    const int K = a.K;
    constexpr int KCH = kMaxK / 1024;
    float4 hv[KCH];
    float ss = 0.f, pm = 0.f;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
        const int e = (i * kBlock + tid) * 4;
        if (e < K) {
            if (a.x_bf16) {
                const uint2 r = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(a.X) + (int64_t)m * a.ldx + e);
                hv[i] = make_float4(bf16_bits_to_float(r.x & 0xffffu), bf16_bits_to_float(r.x >> 16),
                                    bf16_bits_to_float(r.y & 0xffffu), bf16_bits_to_float(r.y >> 16));
            } else {
                hv[i] = *reinterpret_cast<const float4 *>(static_cast<const float *>(a.X) + (int64_t)m * a.ldx + e);
            }
            if (a.tap_h) *reinterpret_cast<float4 *>(a.tap_h + (int64_t)m * K + e) = hv[i];
            ss += hv[i].x * hv[i].x + hv[i].y * hv[i].y + hv[i].z * hv[i].z + hv[i].w * hv[i].w;
            const float4 w = *reinterpret_cast<const float4 *>(a.W + e);
            hv[i].x *= w.x;
            hv[i].y *= w.y;
            hv[i].z *= w.z;
            hv[i].w *= w.w;
            pm = fmaxf(pm, fmaxf(fmaxf(fabsf(hv[i].x), fabsf(hv[i].y)), fmaxf(fabsf(hv[i].z), fabsf(hv[i].w))));
        }
    }
    float tot;
    block_sum_max(ss, pm, red, tot, pm);
    // u = fl(fl(h * w) * r) so that max|u| = fl(max|h * w| * r) exactly (r > 0)
    const float r = 1.0f / sqrtf(tot / (float)K + a.eps);
    const float amax = pm * r;
    const float inv = amax > 0.f ? 127.0f / amax : 0.f;
    const float s = amax > 0.f ? amax / 127.0f : 0.f;
    int qs = 0;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
        const int e = (i * kBlock + tid) * 4;
        if (e < K) {
            float4 u = hv[i];
            u.x *= r;
            u.y *= r;
            u.z *= r;
            u.w *= r;
            const int q0 = quant1(u.x, inv), q1 = quant1(u.y, inv), q2 = quant1(u.z, inv), q3 = quant1(u.w, inv);
            qs += q0 + q1 + q2 + q3;
            const uint32_t packed = (uint32_t)(q0 & 255) | ((uint32_t)(q1 & 255) << 8) | ((uint32_t)(q2 & 255) << 16) |
                                    ((uint32_t)(q3 & 255) << 24);
            *reinterpret_cast<uint32_t *>(sq + e) = packed;
            *reinterpret_cast<uint32_t *>(a.q + (int64_t)m * K + e) = packed;
            if (a.tap_u) *reinterpret_cast<float4 *>(a.tap_u + (int64_t)m * K + e) = u;
            if (a.tap_q) *reinterpret_cast<uint32_t *>(a.tap_q + (int64_t)m * K + e) = packed;
        }
    }
    qs = block_isum(qs, ired);
    if (tid == 0) {
        a.s[m] = s;
        a.qsum[m] = qs;
        if (a.tap_s) a.tap_s[m] = s;
    }
    __syncthreads();
    // int8 LoRA-down, one wave per rank row
    for (int j = wave; j < a.rank; j += kWaves) {
        const int8_t *row = a.lora_dn + (int64_t)j * K;
        int acc = 0;
        for (int off = lane * 16; off < K; off += 1024) {
            const int4 lw = *reinterpret_cast<const int4 *>(row + off);
            const int4 qv = *reinterpret_cast<const int4 *>(sq + off);
            acc = __builtin_amdgcn_sdot4(lw.x, qv.x, acc, false);
            acc = __builtin_amdgcn_sdot4(lw.y, qv.y, acc, false);
            acc = __builtin_amdgcn_sdot4(lw.z, qv.z, acc, false);
            acc = __builtin_amdgcn_sdot4(lw.w, qv.w, acc, false);
        }
        acc = wave_isum(acc);
        if (lane == 0) {
            const float tp = a.dn_scale[j] * s * (float)acc;
            const __bf16 hi = (__bf16)tp;
            const __bf16 lo = (__bf16)(tp - (float)hi);
            a.thi[(int64_t)m * a.rank + j] = hi;
            a.tlo[(int64_t)m * a.rank + j] = lo;
            if (a.tap_t) a.tap_t[(int64_t)m * a.rank + j] = acc;
        }
    }
}

// ------------------------------------------------------------------ 3/4 conv over the sequence
struct ConvSeqArgs {
    const float *Y;        // [M][Ninp] in_proj output
    int64_t ldY;
    int E, Cd, H, L, M;
    const float *conv_w, *conv_b, *dt_bias;
    const float *conv_state;  // [B][Cd][3] initial
    float *xbc;            // [M][Cd]
    float *dt;             // [M][H]
};

// One thread per channel and run of kConvRun consecutive tokens of one sequence: the window of
// the last d_conv-1 inputs slides in registers, so every Y element is read about once.
constexpr int kConvRun = 32;
__global__ __launch_bounds__(kBlock) void k_conv_seq(ConvSeqArgs a) {
    const int runs = (a.L + kConvRun - 1) / kConvRun;
    const int b = blockIdx.x / runs, t0 = (blockIdx.x - b * runs) * kConvRun;
    const int col = blockIdx.y * kBlock + threadIdx.x;
    if (col >= a.Cd + a.H) return;
    const int t1 = min(a.L, t0 + kConvRun);
    const int64_t mb = (int64_t)b * a.L;
    if (col < a.Cd) {
        const float4 w = *reinterpret_cast<const float4 *>(a.conv_w + (int64_t)col * kConvTaps);
        const float bias = a.conv_b[col];
        // window = inputs at t0-3, t0-2, t0-1 (conv state entries for negative positions)
        float win[kConvTaps - 1];
#pragma unroll
        for (int k = 0; k < kConvTaps - 1; ++k) {
            const int tok = t0 - (kConvTaps - 1) + k;
            win[k] = tok >= 0 ? a.Y[(mb + tok) * a.ldY + a.E + col]
                              : a.conv_state[((int64_t)b * a.Cd + col) * (kConvTaps - 1) + (kConvTaps - 1) + tok];
        }
        for (int t = t0; t < t1; ++t) {
            const float x = a.Y[(mb + t) * a.ldY + a.E + col];
            const float v = bias + w.x * win[0] + w.y * win[1] + w.z * win[2] + w.w * x;
            a.xbc[(mb + t) * a.Cd + col] = silu_f(v);
            win[0] = win[1];
            win[1] = win[2];
            win[2] = x;
        }
    } else {
        const int h = col - a.Cd;
        const float db = a.dt_bias[h];
        for (int t = t0; t < t1; ++t)
            a.dt[(mb + t) * a.H + h] = softplus_f(a.Y[(mb + t) * a.ldY + a.E + a.Cd + h] + db);
    }
}

// new state[i] = element L + i of the sequence [old state (3) | inputs (L)]
__global__ __launch_bounds__(kBlock) void k_conv_handoff(ConvSeqArgs a, float *state, int batch) {
    const int idx = blockIdx.x * kBlock + threadIdx.x;
    if (idx >= batch * a.Cd) return;
    const int b = idx / a.Cd, c = idx - b * a.Cd;
    float *st = state + (int64_t)idx * (kConvTaps - 1);
    float nv[kConvTaps - 1];
#pragma unroll
    for (int i = 0; i < kConvTaps - 1; ++i) {
        const int p = a.L + i;  // position in the combined sequence
        nv[i] = p < kConvTaps - 1 ? st[p] : a.Y[((int64_t)b * a.L + p - (kConvTaps - 1)) * a.ldY + a.E + c];
    }
#pragma unroll
    for (int i = 0; i < kConvTaps - 1; ++i) st[i] = nv[i];
}

// ------------------------------------------------------------------ 5 SSD
struct SsdArgs {
    int B, L, H, P, N, G, E, Cd, Q, nch;
    const float *xbc;      // [M][Cd]: x | B (G*N) | C (G*N)
    const float *dt;       // [M][H]
    const float *A_log, *D;
    const float *Y;        // in_proj output (z at columns [0, E))
    int64_t ldY;
    float *lam;            // [B][H][L]
    float *lam_end;        // [B][H][nch]
    float *cb;             // [B][G][nch][Q][Q]
    float *ydiag;          // [M][E]
    float *sloc;           // [B][H][nch][P][N]  (becomes the state entering each chunk)
    float *state;          // [B][H][P][N] initial -> final
    float *g;              // [M][E] gated output
};

// Lam_t = inclusive cumsum of dt_t * A within each chunk: one workgroup per (b, h, c), one token
// per thread (chunk <= 256), wave scans combined through LDS.
__global__ __launch_bounds__(kBlock) void k_ssd_lam(SsdArgs a) {
    __shared__ float wsum[kWaves];
    const int idx = blockIdx.x;  // (b, h, c)
    const int c = idx % a.nch, bh = idx / a.nch, h = bh % a.H, b = bh / a.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t = c * a.Q + tid;
    const bool ok = tid < a.Q && t < a.L;
    const float A = -expf(a.A_log[h]);
    float v = ok ? a.dt[((int64_t)b * a.L + t) * a.H + h] * A : 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    for (int w = 0; w < wave; ++w) v += wsum[w];
    if (ok) a.lam[((int64_t)b * a.H + h) * a.L + t] = v;
    const int last = min(a.Q, a.L - c * a.Q) - 1;
    if (tid == last) a.lam_end[idx] = v;
}

// CB tile (ti, si) of chunk c for group g: 64 x 64 outputs, 4 x 4 per thread, N in tiles of 64.
__global__ __launch_bounds__(kBlock) void k_ssd_cb(SsdArgs a) {
    __shared__ __align__(16) float Cs[TT][TT + 4];  // [n][t]
    __shared__ __align__(16) float Bs[TT][TT + 4];  // [n][s]
    const int tq = (a.Q + TT - 1) / TT;
    const int ti = blockIdx.y / tq, si = blockIdx.y % tq;
    const int bgc = blockIdx.x, c = bgc % a.nch, g = (bgc / a.nch) % a.G, b = bgc / (a.nch * a.G);
    if (si > ti) return;
    const int len = min(a.Q, a.L - c * a.Q);
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    float acc[4][4] = {};
    const int64_t mbase = (int64_t)b * a.L + c * a.Q;
    for (int n0 = 0; n0 < a.N; n0 += TT) {
        for (int k = tid; k < TT * TT; k += kBlock) {
            const int r = k / TT, n = k % TT;  // r: token row within the tile
            const int tt = ti * TT + r, ss = si * TT + r;
            const bool nin = n0 + n < a.N;  // d_state below 64 leaves part of the tile empty
            Cs[n][r] = nin && tt < len ? a.xbc[(mbase + tt) * a.Cd + a.E + a.G * a.N + g * a.N + n0 + n] : 0.f;
            Bs[n][r] = nin && ss < len ? a.xbc[(mbase + ss) * a.Cd + a.E + g * a.N + n0 + n] : 0.f;
        }
        __syncthreads();
#pragma unroll 4
        for (int n = 0; n < TT; ++n) {
            const float4 cv = *reinterpret_cast<const float4 *>(&Cs[n][ty * 4]);
            const float4 bv = *reinterpret_cast<const float4 *>(&Bs[n][tx * 4]);
            const float cr[4] = {cv.x, cv.y, cv.z, cv.w}, br[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] += cr[i] * br[j];
        }
        __syncthreads();
    }
    float *out = a.cb + (((int64_t)b * a.G + g) * a.nch + c) * a.Q * a.Q;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = ti * TT + ty * 4 + i;
        if (t >= a.Q) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int s = si * TT + tx * 4 + j;
            if (s < a.Q) out[(int64_t)t * a.Q + s] = acc[i][j];
        }
    }
}

// Y_diag for token tile ti of chunk c, head h: 64 tokens x P(=64) features, 4 x 4 per thread.
__global__ __launch_bounds__(kBlock) void k_ssd_ydiag(SsdArgs a) {
    __shared__ __align__(16) float Ws[TT][TT + 4];  // [s][t]
    __shared__ __align__(16) float Xs[TT][TT + 4];  // [s][p]
    __shared__ float lam_t[TT], lam_s[TT], dts[TT];
    const int tq = (a.Q + TT - 1) / TT;
    const int ti = blockIdx.y;
    const int bhc = blockIdx.x, c = bhc % a.nch, h = (bhc / a.nch) % a.H, b = bhc / (a.nch * a.H);
    if (ti >= tq) return;
    const int len = min(a.Q, a.L - c * a.Q);
    if (ti * TT >= len) return;
    const int g = h * a.G / a.H;
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    const int64_t mbase = (int64_t)b * a.L + c * a.Q;
    const float *lamh = a.lam + ((int64_t)b * a.H + h) * a.L + c * a.Q;
    const float *cbc = a.cb + (((int64_t)b * a.G + g) * a.nch + c) * a.Q * a.Q;
    if (tid < TT) lam_t[tid] = ti * TT + tid < len ? lamh[ti * TT + tid] : 0.f;
    float acc[4][4] = {};
    for (int si = 0; si <= ti; ++si) {
        __syncthreads();
        if (tid < TT) {
            const int s = si * TT + tid;
            lam_s[tid] = s < len ? lamh[s] : 0.f;
            dts[tid] = s < len ? a.dt[(mbase + s) * a.H + h] : 0.f;
        }
        __syncthreads();
        for (int k = tid; k < TT * TT; k += kBlock) {
            const int r = k / TT, q = k % TT;
            // W[t=r][s=q] = CB * exp(lam_t - lam_s) * dt_s  for s <= t (both inside the chunk)
            const int t = ti * TT + r, s = si * TT + q;
            float wv = 0.f;
            if (s <= t && t < len) wv = cbc[(int64_t)t * a.Q + s] * expf(lam_t[r] - lam_s[q]) * dts[q];
            Ws[q][r] = wv;
            Xs[r][q] = si * TT + r < len ? a.xbc[(mbase + si * TT + r) * a.Cd + h * a.P + q] : 0.f;
        }
        __syncthreads();
#pragma unroll 4
        for (int s = 0; s < TT; ++s) {
            const float4 wv = *reinterpret_cast<const float4 *>(&Ws[s][ty * 4]);
            const float4 xv = *reinterpret_cast<const float4 *>(&Xs[s][tx * 4]);
            const float wr[4] = {wv.x, wv.y, wv.z, wv.w}, xr[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] += wr[i] * xr[j];
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = ti * TT + ty * 4 + i;
        if (t >= len) continue;
        *reinterpret_cast<float4 *>(a.ydiag + (mbase + t) * a.E + h * a.P + tx * 4) =
            make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
    }
}

// Chunk-local state S_loc[p][n] = sum_s exp(Lam_end - Lam_s) dt_s x_s[p] B_s[n] for (b, h, c):
// a (P x chunk) x (chunk x N) product, 64 x 64 outputs per workgroup (4 x 4 per thread), s in tiles of 64.
__global__ __launch_bounds__(kBlock) void k_ssd_sloc(SsdArgs a) {
    __shared__ __align__(16) float Xw[TT][TT + 4];  // [s][p], scaled by the decay weight
    __shared__ __align__(16) float Bs[TT][TT + 4];  // [s][n]
    __shared__ float wgt[TT];
    const int bhc = blockIdx.x, c = bhc % a.nch, h = (bhc / a.nch) % a.H, b = bhc / (a.nch * a.H);
    const int n0 = blockIdx.y * TT;
    const int len = min(a.Q, a.L - c * a.Q);
    const int g = h * a.G / a.H;
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    const int64_t mbase = (int64_t)b * a.L + c * a.Q;
    const float *lamh = a.lam + ((int64_t)b * a.H + h) * a.L + c * a.Q;
    const float lend = a.lam_end[((int64_t)b * a.H + h) * a.nch + c];
    float acc[4][4] = {};
    for (int s0 = 0; s0 < len; s0 += TT) {
        __syncthreads();
        if (tid < TT) {
            const int s = s0 + tid;
            wgt[tid] = s < len ? expf(lend - lamh[s]) * a.dt[(mbase + s) * a.H + h] : 0.f;
        }
        __syncthreads();
        for (int k = tid; k < TT * TT; k += kBlock) {
            const int r = k / TT, q = k % TT;  // r: token within the tile, q: feature
            const int s = s0 + r;
            const bool sin_ = s < len;
            Xw[r][q] = sin_ ? a.xbc[(mbase + s) * a.Cd + h * a.P + q] * wgt[r] : 0.f;
            Bs[r][q] = sin_ && n0 + q < a.N ? a.xbc[(mbase + s) * a.Cd + a.E + g * a.N + n0 + q] : 0.f;
        }
        __syncthreads();
#pragma unroll 4
        for (int r = 0; r < TT; ++r) {
            const float4 xv = *reinterpret_cast<const float4 *>(&Xw[r][ty * 4]);
            const float4 bv = *reinterpret_cast<const float4 *>(&Bs[r][tx * 4]);
            const float xr[4] = {xv.x, xv.y, xv.z, xv.w}, br[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] += xr[i] * br[j];
        }
    }
    float *out = a.sloc + (((int64_t)b * a.H + h) * a.nch + c) * a.P * a.N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = ty * 4 + i;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n < a.N) out[(int64_t)p * a.N + n] = acc[i][j];
        }
    }
}

// Sequential carry over chunks; sloc[c] is replaced by the state entering chunk c.
__global__ __launch_bounds__(kBlock) void k_ssd_scan(SsdArgs a) {
    const int64_t PN = (int64_t)a.P * a.N;
    const int bh = blockIdx.y;
    const int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (e >= PN) return;
    float S = a.state[(int64_t)bh * PN + e];
    for (int c = 0; c < a.nch; ++c) {
        float *slot = a.sloc + ((int64_t)bh * a.nch + c) * PN + e;
        const float loc = *slot;
        *slot = S;
        S = expf(a.lam_end[(int64_t)bh * a.nch + c]) * S + loc;
    }
    a.state[(int64_t)bh * PN + e] = S;
}

// y = Y_diag + exp(Lam_t) C_t . S_in + D x ; g = y * SiLU(z), token tile ti of chunk c, head h.
__global__ __launch_bounds__(kBlock) void k_ssd_yoff(SsdArgs a) {
    __shared__ __align__(16) float Cs[TT][TT + 4];  // [n][t]
    __shared__ __align__(16) float Ss[TT][TT + 4];  // [n][p]
    const int tq = (a.Q + TT - 1) / TT;
    const int ti = blockIdx.y;
    const int bhc = blockIdx.x, c = bhc % a.nch, h = (bhc / a.nch) % a.H, b = bhc / (a.nch * a.H);
    const int len = min(a.Q, a.L - c * a.Q);
    if (ti >= tq || ti * TT >= len) return;
    const int g = h * a.G / a.H;
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    const int64_t mbase = (int64_t)b * a.L + c * a.Q;
    const float *sin = a.sloc + (((int64_t)b * a.H + h) * a.nch + c) * a.P * a.N;
    float acc[4][4] = {};
    for (int n0 = 0; n0 < a.N; n0 += TT) {
        __syncthreads();
        for (int k = tid; k < TT * TT; k += kBlock) {
            const int r = k / TT, n = k % TT;
            const int t = ti * TT + r;
            const bool nin = n0 + n < a.N;
            Cs[n][r] = nin && t < len ? a.xbc[(mbase + t) * a.Cd + a.E + a.G * a.N + g * a.N + n0 + n] : 0.f;
            Ss[n][r] = nin ? sin[(int64_t)r * a.N + n0 + n] : 0.f;   // r is p here (P == 64)
        }
        __syncthreads();
#pragma unroll 4
        for (int n = 0; n < TT; ++n) {
            const float4 cv = *reinterpret_cast<const float4 *>(&Cs[n][ty * 4]);
            const float4 sv = *reinterpret_cast<const float4 *>(&Ss[n][tx * 4]);
            const float cr[4] = {cv.x, cv.y, cv.z, cv.w}, sr[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] += cr[i] * sr[j];
        }
    }
    const float *lamh = a.lam + ((int64_t)b * a.H + h) * a.L + c * a.Q;
    const float Dh = a.D[h];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = ti * TT + ty * 4 + i;
        if (t >= len) continue;
        const int64_t m = mbase + t;
        const float el = expf(lamh[t]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int p = tx * 4 + j;
            const int64_t col = h * a.P + p;
            const float x = a.xbc[m * a.Cd + col];
            const float y = a.ydiag[m * a.E + col] + el * acc[i][j] + Dh * x;
            a.g[m * a.E + col] = y * silu_f(a.Y[m * a.ldY + col]);
        }
    }
}

// Decode-step conv from the in_proj output Y [B][Ninp]: z copied out, x|B|C conv + SiLU with the
// per-sequence conv state (shifted in place: one thread per channel), softplus(dt + dt_bias).
struct ConvStepArgs {
    const float *Y;
    int64_t ldY;
    int E, Cd, H;
    const float *conv_w, *conv_b, *dt_bias;
    float *conv_state;     // [B][Cd][3]
    float *zbuf, *xbc, *dtbuf;
};

__global__ __launch_bounds__(kBlock) void k_conv_step_y(ConvStepArgs a) {
    const int b = blockIdx.y;
    const int n = blockIdx.x * kBlock + threadIdx.x;
    if (n >= a.E + a.Cd + a.H) return;
    const float y = a.Y[(int64_t)b * a.ldY + n];
    if (n < a.E) {
        a.zbuf[(int64_t)b * a.E + n] = y;
    } else if (n < a.E + a.Cd) {
        const int ch = n - a.E;
        float *st = a.conv_state + ((int64_t)b * a.Cd + ch) * (kConvTaps - 1);
        const float *w = a.conv_w + (int64_t)ch * kConvTaps;
        const float s0 = st[0], s1 = st[1], s2 = st[2];
        const float pre = a.conv_b[ch] + w[0] * s0 + w[1] * s1 + w[2] * s2 + w[3] * y;
        st[0] = s1;
        st[1] = s2;
        st[2] = y;
        a.xbc[(int64_t)b * a.Cd + ch] = silu_f(pre);
    } else {
        const int h = n - a.E - a.Cd;
        a.dtbuf[(int64_t)b * a.H + h] = softplus_f(y + a.dt_bias[h]);
    }
}

}  // namespace

bool decode_uses_mfma(const Shape &s, int batch) {
    return batch > kGemvMaxBatch && s.Rin % 8 == 0 && s.Rout % 8 == 0;
}

hipError_t launch_layer_decode_mfma(const Shape &s, const dfssm_layer_weights &w, const dfssm_layer_state &st,
                                    const float *x_in, float *x_out, int batch, const DecodeWs &dws,
                                    const PrefillWs &pws, const TapPtrs &tp, hipStream_t stream) {
    hipError_t e;
    {
        TokQuantArgs a{};
        a.X = x_in;
        a.ldx = s.D;
        a.W = w.norm_w;
        a.M = batch;
        a.K = s.D;
        a.eps = s.eps;
        a.lora_dn = w.in_proj.lora_dn;
        a.dn_scale = w.in_proj.lora_dn_scale;
        a.rank = s.Rin;
        a.q = pws.q_in;
        a.s = pws.s_in;
        a.qsum = pws.qsum_in;
        a.thi = pws.thi_in;
        a.tlo = pws.tlo_in;
        a.tap_h = tp.h_in;
        a.tap_u = tp.in_u;
        a.tap_q = tp.in_q;
        a.tap_s = tp.in_s;
        a.tap_t = tp.in_t;
        if ((e = launch_tok_quant(a, stream)) != hipSuccess) return e;
    }
    {
        GemmArgs a{};
        a.q = pws.q_in;
        a.ldq = s.D;
        a.qsum = pws.qsum_in;
        a.s = pws.s_in;
        a.sign = w.in_proj.sign;
        a.M = batch;
        a.N = s.Ninp;
        a.K = s.D;
        a.row_scale = w.in_proj.row_scale;
        a.up_scale = w.in_proj.lora_up_scale;
        a.lora_up = w.in_proj.lora_up;
        a.rank = s.Rin;
        a.thi = pws.thi_in;
        a.tlo = pws.tlo_in;
        a.y = pws.Y;
        a.ldy = s.Ninp;
        a.acc_tap = tp.in_acc;
        a.ldacc = s.Ninp;
        a.scratch = pws.gemm_scratch;
        if ((e = launch_gemm_pm1(a, stream)) != hipSuccess) return e;
    }
    {
        ConvStepArgs a{pws.Y, s.Ninp, s.E, s.Cd, s.H, w.conv_w, w.conv_b, w.dt_bias, st.conv, dws.zbuf, dws.xbc, dws.dtbuf};
        k_conv_step_y<<<dim3((s.Nin + kBlock - 1) / kBlock, batch), kBlock, 0, stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = launch_ssm_step(s, w, st, dws, batch, stream)) != hipSuccess) return e;
    {
        TokQuantArgs a{};
        a.X = dws.gbuf;
        a.ldx = s.E;
        a.W = w.gnorm_w;
        a.M = batch;
        a.K = s.E;
        a.eps = s.eps;
        a.lora_dn = w.out_proj.lora_dn;
        a.dn_scale = w.out_proj.lora_dn_scale;
        a.rank = s.Rout;
        a.q = pws.q_out;
        a.s = pws.s_out;
        a.qsum = pws.qsum_out;
        a.thi = pws.thi_out;
        a.tlo = pws.tlo_out;
        a.tap_u = tp.out_u;
        a.tap_q = tp.out_q;
        a.tap_s = tp.out_s;
        a.tap_t = tp.out_t;
        if ((e = launch_tok_quant(a, stream)) != hipSuccess) return e;
    }
    {
        GemmArgs a{};
        a.q = pws.q_out;
        a.ldq = s.E;
        a.qsum = pws.qsum_out;
        a.s = pws.s_out;
        a.sign = w.out_proj.sign;
        a.M = batch;
        a.N = s.D;
        a.K = s.E;
        a.row_scale = w.out_proj.row_scale;
        a.up_scale = w.out_proj.lora_up_scale;
        a.lora_up = w.out_proj.lora_up;
        a.rank = s.Rout;
        a.thi = pws.thi_out;
        a.tlo = pws.tlo_out;
        a.y = x_out;                // may alias x_in: each element is read then written by one thread
        a.ldy = s.D;
        a.res = x_in;
        a.ldres = s.D;
        a.acc_tap = tp.out_acc;
        a.ldacc = s.D;
        a.scratch = pws.gemm_scratch;
        if ((e = launch_gemm_pm1(a, stream)) != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_tok_quant(const TokQuantArgs &a, hipStream_t stream) {
    if (a.K > kMaxK || a.K % 16 || a.rank > kMaxRank) return hipErrorInvalidValue;
    k_tok_quant<<<a.M, kBlock, 0, stream>>>(a);
    return hipGetLastError();
}

PrefillWs carve_prefill_ws(const Shape &s, int batch, int seqlen, int chunk, void *base) {
    PrefillWs w{};
    size_t off = 0;
    char *bp = static_cast<char *>(base);
    auto take = [&](size_t bytes) -> void * {
        void *p = bp ? bp + off : nullptr;
        off += align_up(bytes, 256);
        return p;
    };
    const size_t M = (size_t)batch * seqlen;
    const int nch = (seqlen + chunk - 1) / chunk;
    w.q_in = static_cast<int8_t *>(take(M * s.D));
    w.s_in = static_cast<float *>(take(M * 4));
    w.qsum_in = static_cast<int32_t *>(take(M * 4));
    w.thi_in = static_cast<__bf16 *>(take(M * s.Rin * 2));
    w.tlo_in = static_cast<__bf16 *>(take(M * s.Rin * 2));
    w.Y = static_cast<float *>(take(M * s.Ninp * 4));
    w.xbc = static_cast<float *>(take(M * s.Cd * 4));
    w.dt = static_cast<float *>(take(M * s.H * 4));
    w.lam = static_cast<float *>(take((size_t)batch * s.H * seqlen * 4));
    w.lam_end = static_cast<float *>(take((size_t)batch * s.H * nch * 4));
    w.cb = static_cast<float *>(take((size_t)batch * s.G * nch * chunk * chunk * 4));
    w.ydiag = static_cast<float *>(take(M * s.E * 4));
    w.sloc = static_cast<float *>(take((size_t)batch * s.H * nch * s.P * s.N * 4));
    w.gbuf = static_cast<float *>(take(M * s.E * 4));
    w.q_out = static_cast<int8_t *>(take(M * s.E));
    w.s_out = static_cast<float *>(take(M * 4));
    w.qsum_out = static_cast<int32_t *>(take(M * 4));
    w.thi_out = static_cast<__bf16 *>(take(M * s.Rout * 2));
    w.tlo_out = static_cast<__bf16 *>(take(M * s.Rout * 2));
    w.gemm_scratch = take(std::max(gemm_scratch_bytes((int)M, s.Ninp, s.D), gemm_scratch_bytes((int)M, s.D, s.E)));
    w.bytes = off;
    return w;
}

hipError_t launch_layer_prefill(const Shape &s, const dfssm_layer_weights &w, const dfssm_layer_state &st,
                                const void *x_in, int x_bf16, float *x_out, int batch, int seqlen, int chunk,
                                const PrefillWs &ws, const dfssm_taps *taps, hipStream_t stream) {
    const int M = batch * seqlen;
    const int nch = (seqlen + chunk - 1) / chunk;
    const TapPtrs tp = tap_offset(taps, s, 0);
    hipError_t e;
    // 1. in: per-token quantizer + LoRA-down
    {
        TokQuantArgs a{};
        a.X = x_in;
        a.x_bf16 = x_bf16;
        a.ldx = s.D;
        a.W = w.norm_w;
        a.M = M;
        a.K = s.D;
        a.eps = s.eps;
        a.lora_dn = w.in_proj.lora_dn;
        a.dn_scale = w.in_proj.lora_dn_scale;
        a.rank = s.Rin;
        a.q = ws.q_in;
        a.s = ws.s_in;
        a.qsum = ws.qsum_in;
        a.thi = ws.thi_in;
        a.tlo = ws.tlo_in;
        a.tap_h = tp.h_in;
        a.tap_u = tp.in_u;
        a.tap_q = tp.in_q;
        a.tap_s = tp.in_s;
        a.tap_t = tp.in_t;
        if ((e = launch_tok_quant(a, stream)) != hipSuccess) return e;
    }
    // 2. in_proj GEMM
    {
        GemmArgs a{};
        a.q = ws.q_in;
        a.ldq = s.D;
        a.qsum = ws.qsum_in;
        a.s = ws.s_in;
        a.sign = w.in_proj.sign;
        a.M = M;
        a.N = s.Ninp;
        a.K = s.D;
        a.row_scale = w.in_proj.row_scale;
        a.up_scale = w.in_proj.lora_up_scale;
        a.lora_up = w.in_proj.lora_up;
        a.rank = s.Rin;
        a.thi = ws.thi_in;
        a.tlo = ws.tlo_in;
        a.y = ws.Y;
        a.ldy = s.Ninp;
        a.acc_tap = tp.in_acc;
        a.ldacc = s.Ninp;
        a.scratch = ws.gemm_scratch;
        if ((e = launch_gemm_pm1(a, stream)) != hipSuccess) return e;
    }
    // 3/4. conv over the sequence, dt, conv-state handoff
    ConvSeqArgs cv{ws.Y, s.Ninp, s.E, s.Cd, s.H, seqlen, M, w.conv_w, w.conv_b, w.dt_bias, st.conv, ws.xbc, ws.dt};
    {
        dim3 grid(batch * ((seqlen + kConvRun - 1) / kConvRun), (s.Cd + s.H + kBlock - 1) / kBlock);
        k_conv_seq<<<grid, kBlock, 0, stream>>>(cv);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        k_conv_handoff<<<(batch * s.Cd + kBlock - 1) / kBlock, kBlock, 0, stream>>>(cv, st.conv, batch);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // 5. chunked SSD
    {
        SsdArgs a{};
        a.B = batch;
        a.L = seqlen;
        a.H = s.H;
        a.P = s.P;
        a.N = s.N;
        a.G = s.G;
        a.E = s.E;
        a.Cd = s.Cd;
        a.Q = chunk;
        a.nch = nch;
        a.xbc = ws.xbc;
        a.dt = ws.dt;
        a.A_log = w.A_log;
        a.D = w.D;
        a.Y = ws.Y;
        a.ldY = s.Ninp;
        a.lam = ws.lam;
        a.lam_end = ws.lam_end;
        a.cb = ws.cb;
        a.ydiag = ws.ydiag;
        a.sloc = ws.sloc;
        a.state = st.ssm;
        a.g = ws.gbuf;
        const int tq = (chunk + TT - 1) / TT;
        const int nbhc = batch * s.H * nch;
        k_ssd_lam<<<nbhc, kBlock, 0, stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        k_ssd_cb<<<dim3(batch * s.G * nch, tq * tq), kBlock, 0, stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        k_ssd_ydiag<<<dim3(nbhc, tq), kBlock, 0, stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        k_ssd_sloc<<<dim3(nbhc, (s.N + TT - 1) / TT), kBlock, 0, stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        k_ssd_scan<<<dim3((s.P * s.N + kBlock - 1) / kBlock, batch * s.H), kBlock, 0, stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        k_ssd_yoff<<<dim3(nbhc, tq), kBlock, 0, stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // 6. out: gated RMSNorm + quantizer + LoRA-down of g
    {
        TokQuantArgs a{};
        a.X = ws.gbuf;
        a.x_bf16 = 0;
        a.ldx = s.E;
        a.W = w.gnorm_w;
        a.M = M;
        a.K = s.E;
        a.eps = s.eps;
        a.lora_dn = w.out_proj.lora_dn;
        a.dn_scale = w.out_proj.lora_dn_scale;
        a.rank = s.Rout;
        a.q = ws.q_out;
        a.s = ws.s_out;
        a.qsum = ws.qsum_out;
        a.thi = ws.thi_out;
        a.tlo = ws.tlo_out;
        a.tap_u = tp.out_u;
        a.tap_q = tp.out_q;
        a.tap_s = tp.out_s;
        a.tap_t = tp.out_t;
        if ((e = launch_tok_quant(a, stream)) != hipSuccess) return e;
    }
    // 7. out_proj GEMM + residual. The residual is the fp32 (or bf16-widened) layer input.
    {
        const float *res = static_cast<const float *>(x_in);
        if (x_bf16) {
            // widen the bf16 input once into x_out, then add in place (the epilogue reads res[m][n]
            // before writing y[m][n] in the same thread)
            k_widen_bf16<<<(unsigned)(((int64_t)M * s.D + kBlock - 1) / kBlock), kBlock, 0, stream>>>(static_cast<const uint16_t *>(x_in), x_out,
                                                                                 (int64_t)M * s.D);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            res = x_out;
        }
        GemmArgs a{};
        a.q = ws.q_out;
        a.ldq = s.E;
        a.qsum = ws.qsum_out;
        a.s = ws.s_out;
        a.sign = w.out_proj.sign;
        a.M = M;
        a.N = s.D;
        a.K = s.E;
        a.row_scale = w.out_proj.row_scale;
        a.up_scale = w.out_proj.lora_up_scale;
        a.lora_up = w.out_proj.lora_up;
        a.rank = s.Rout;
        a.thi = ws.thi_out;
        a.tlo = ws.tlo_out;
        a.y = x_out;
        a.ldy = s.D;
        a.res = res;
        a.ldres = s.D;
        a.acc_tap = tp.out_acc;
        a.ldacc = s.D;
        a.scratch = ws.gemm_scratch;
        if ((e = launch_gemm_pm1(a, stream)) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace dfssm
