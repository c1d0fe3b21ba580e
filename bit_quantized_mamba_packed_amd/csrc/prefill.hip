// DF-SSM layer prefill for M = batch * seqlen tokens on gfx950.
//
// The result is, by definition, seqlen successive decode steps (quantization is per token); the
// SSM part is evaluated with the chunked state-space-duality form of Mamba-2 (the SSD paper the
// DF-SSM paper builds on, §2). Per layer:
//   1 k_tok_quant      per token: RMSNorm + int8 quantizer, int8 LoRA-down, t' split to bf16
//   2 k_gemm_pm1       in_proj over all tokens (int8 MFMA) with the Eq. (3) epilogue -> Y
//   3 k_conv_seq       causal conv over the sequence + SiLU (x, B, C); softplus(dt + dt_bias)
//   4 (C.B^T pass)     final conv state = the last d_conv-1 pre-activation inputs
//   5 SSD, chunk length Q, Lam_t = sum_{tau <= t in chunk} dt_tau A (per head), MFMA:
//     k_ssd_cbm_state, one launch of two independent passes:
//       C.B^T          CB[t][s] = C_t . B_s for each chunk and group (shared by the group's heads)
//       chunk state    S_loc = sum_s exp(Lam_end - Lam_s) dt_s x_s (x) B_s per chunk, and Lam_end
//       k_ssd_scan     S_in(c) = state entering chunk c; S <- exp(Lam_end) S + S_loc (sequential in c)
//       k_ssd_out      y = sum_{s <= t} exp(Lam_t - Lam_s) CB[t][s] dt_s x_s + exp(Lam_t) C_t . S_in
//                      + D x; g = y * SiLU(z)
//     (exponentials only of Lam differences, or of Lam itself: never positive)
//   6 k_tok_quant      gated RMSNorm + quantizer + LoRA-down of g
//   7 k_gemm_pm1       out_proj with the residual add -> x_out
#include <algorithm>

#include "decode_device.h"
#include "gemm_conv.h"

namespace dfssm {

namespace {

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

__global__ __launch_bounds__(kBlock) void k_widen_bf16(const uint16_t *x, float *y, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < n) y[i] = bf16_bits_to_float(x[i]);
}

// ------------------------------------------------------------------ 1/6 per-token quantizer
// TOK tokens per workgroup of NW waves (one or two tokens per wave). Each wave normalises and
// quantizes whole tokens (wave-level reductions only, no barrier), leaving the codes in LDS; then the LoRA-down of
// all of them, t[tok][j] = sum_k q[tok][k] L_dn[j][k], runs on int8 MFMA (32x32x32 blocks, tokens
// as rows 0..7 of the block, rank rows as its columns, the K blocks split over the waves), so each
// workgroup reads L_dn once for TOK tokens (loaded with the rows when TOK = 8 and K <= 4096).
constexpr int kTqTok = 8;   // tokens per workgroup of k_tok_quant
constexpr int kTq1MaxM = 256;   // up to this many tokens: k_tok_quant1 (one token per workgroup)
constexpr int kTqRow = kMaxK + 16;  // LDS bytes per token's codes (the pad spreads rows over the banks)
typedef int tq_v4i __attribute__((ext_vector_type(4)));
typedef int tq_v16i __attribute__((ext_vector_type(16)));

template <int KCH, int TOK, int NW>
__global__ __launch_bounds__(64 * NW) void k_tok_quant(TokQuantArgs a) {
    __shared__ __align__(16) int8_t sq[TOK * kTqRow];
    __shared__ float s_l[TOK];
    __shared__ int tred[NW][kMaxRank / 32][4][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, hsel = lane >> 5;
    const int m0 = blockIdx.x * TOK;
    const int K = a.K;
    if (blockIdx.x == 0)
        for (int i = tid; i < a.nzero; i += 64 * NW) a.zero_words[i] = 0u;
    const int nkw = K / (32 * NW), nrb = (a.rank + 31) / 32;  // K blocks of 32 per wave; rank blocks of 32
    // Loads are issued in the order their results are needed (norm weight, the rows, then the
    // LoRA-down operands), all before any store, with addresses clamped into range and
    // out-of-range values zeroed after, so that the quantizer of the first row starts while the
    // rest is still in flight.
    float dsv[kMaxRank / 32];
#pragma unroll
    for (int rb = 0; rb < kMaxRank / 32; ++rb) dsv[rb] = a.dn_scale[min(rb * 32 + (tid & 31), a.rank - 1)];
    float4 wv[KCH];
#pragma unroll
    for (int i = 0; i < KCH; ++i) wv[i] = *reinterpret_cast<const float4 *>(a.W + min((i * 64 + lane) * 4, K - 4));
    // ---- norm + quantizer: wave w takes tokens w, w + NW, ... (all of them in flight at once when
    // they fit in registers)
    constexpr int TPW = TOK / NW;   // tokens per wave
    constexpr int NU = KCH <= 16 ? TPW : 1;
    // LoRA-down operands (lane: rank row lr, bytes 16 * hsel.. of each 32-wide K block); with one
    // rank block and exactly PRE K blocks per wave they are loaded with the rows
    constexpr int PRE = KCH <= 16 && TOK == 8 ? 8 * KCH / NW : 1;
    const bool pre = KCH <= 16 && TOK == 8 && nrb == 1 && nkw == PRE;
    const int8_t *brow[kMaxRank / 32];
    bool bok[kMaxRank / 32];
#pragma unroll
    for (int rb = 0; rb < kMaxRank / 32; ++rb) {
        const int j = rb * 32 + lr;
        bok[rb] = j < a.rank;
        brow[rb] = a.lora_dn + (int64_t)min(j, a.rank - 1) * K + hsel * 16 + wave * nkw * 32;
    }
    tq_v4i bpre[PRE];
#pragma unroll
    for (int pass = 0; pass < TPW / NU; ++pass) {
        float4 hv[NU][KCH];
        int mrow[NU];
        bool mok[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int m = m0 + wave + (pass * NU + u) * NW;
            mok[u] = m < a.M;
            mrow[u] = min(m, a.M - 1);
        }
        if (a.x_bf16) {
            uint2 raw[NU][KCH];
#pragma unroll
            for (int u = 0; u < NU; ++u)
#pragma unroll
                for (int i = 0; i < KCH; ++i) {
                    const int e = min((i * 64 + lane) * 4, K - 4);
                    raw[u][i] = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(a.X) + (int64_t)mrow[u] * a.ldx + e);
                }
            if (pre) {
#pragma unroll
                for (int c = 0; c < PRE; ++c) bpre[c] = *reinterpret_cast<const tq_v4i *>(brow[0] + c * 32);
            }
#pragma unroll
            for (int u = 0; u < NU; ++u)
#pragma unroll
                for (int i = 0; i < KCH; ++i) {
                    const uint2 r = raw[u][i];
                    hv[u][i] = make_float4(bf16_bits_to_float(r.x & 0xffffu), bf16_bits_to_float(r.x >> 16),
                                           bf16_bits_to_float(r.y & 0xffffu), bf16_bits_to_float(r.y >> 16));
                }
        } else {
#pragma unroll
            for (int u = 0; u < NU; ++u)
#pragma unroll
                for (int i = 0; i < KCH; ++i) {
                    const int e = min((i * 64 + lane) * 4, K - 4);
                    hv[u][i] = *reinterpret_cast<const float4 *>(static_cast<const float *>(a.X) + (int64_t)mrow[u] * a.ldx + e);
                }
            if (pre) {
#pragma unroll
                for (int c = 0; c < PRE; ++c) bpre[c] = *reinterpret_cast<const tq_v4i *>(brow[0] + c * 32);
            }
        }
        float ss[NU], pm[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            ss[u] = 0.f;
            pm[u] = 0.f;
        }
#pragma unroll
        for (int u = 0; u < NU; ++u) {
#pragma unroll
            for (int i = 0; i < KCH; ++i) {
                const bool ok = (i * 64 + lane) * 4 < K && mok[u];
                float4 &h = hv[u][i];
                h.x = ok ? h.x : 0.f;
                h.y = ok ? h.y : 0.f;
                h.z = ok ? h.z : 0.f;
                h.w = ok ? h.w : 0.f;
                ss[u] += h.x * h.x + h.y * h.y + h.z * h.z + h.w * h.w;
            }
        }
        if (a.tap_h) {
#pragma unroll
            for (int u = 0; u < NU; ++u)
#pragma unroll
                for (int i = 0; i < KCH; ++i) {
                    const int e = (i * 64 + lane) * 4;
                    if (e < K && mok[u]) *reinterpret_cast<float4 *>(a.tap_h + (int64_t)mrow[u] * K + e) = hv[u][i];
                }
        }
#pragma unroll
        for (int u = 0; u < NU; ++u) {
#pragma unroll
            for (int i = 0; i < KCH; ++i) {
                float4 &h = hv[u][i];
                const float4 w = wv[i];
                h.x *= w.x;
                h.y *= w.y;
                h.z *= w.z;
                h.w *= w.w;
                pm[u] = fmaxf(pm[u], fmaxf(fmaxf(fabsf(h.x), fabsf(h.y)), fmaxf(fabsf(h.z), fabsf(h.w))));
            }
        }
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int tok = wave + (pass * NU + u) * NW, m = m0 + tok;
            const float tot = dpp_wave_sum(ss[u]), mx = dpp_wave_max(pm[u]);
            // u = fl(fl(h * w) * r) so that max|u| = fl(max|h * w| * r) exactly (r > 0)
            const float r = 1.0f / sqrtf(tot / (float)K + a.eps);
            const float amax = mx * r;
            const float inv = amax > 0.f ? 127.0f / amax : 0.f;
            const float sv = amax > 0.f ? amax / 127.0f : 0.f;
            int qs = 0;
#pragma unroll
            for (int i = 0; i < KCH; ++i) {
                const int e = (i * 64 + lane) * 4;
                if (e < K) {
                    float4 v = hv[u][i];
                    v.x *= r;
                    v.y *= r;
                    v.z *= r;
                    v.w *= r;
                    const int q0 = quant1(v.x, inv), q1 = quant1(v.y, inv), q2 = quant1(v.z, inv), q3 = quant1(v.w, inv);
                    qs += q0 + q1 + q2 + q3;
                    const uint32_t packed = (uint32_t)(q0 & 255) | ((uint32_t)(q1 & 255) << 8) |
                                            ((uint32_t)(q2 & 255) << 16) | ((uint32_t)(q3 & 255) << 24);
                    *reinterpret_cast<uint32_t *>(sq + tok * kTqRow + e) = packed;
                    if (m < a.M) {
                        *reinterpret_cast<uint32_t *>(a.q + (int64_t)m * K + e) = packed;
                        if (a.tap_u) *reinterpret_cast<float4 *>(a.tap_u + (int64_t)m * K + e) = v;
                        if (a.tap_q) *reinterpret_cast<uint32_t *>(a.tap_q + (int64_t)m * K + e) = packed;
                    }
                }
            }
            qs = dpp_wave_isum(qs);
            if (lane == 0) {
                s_l[tok] = sv;
                if (m < a.M) {
                    a.s[m] = sv;
                    a.qsum[m] = qs;
                    if (a.tap_s) a.tap_s[m] = sv;
                }
            }
        }
    }
    __syncthreads();
    // ---- LoRA-down on int8 MFMA: lane supplies row (token) lr and column (rank row) lr of the
    // block; tokens past kTqTok and rank rows past the rank are zero
    const int8_t *arow = sq + (lr & (TOK - 1)) * kTqRow + hsel * 16 + wave * nkw * 32;
    tq_v16i acc[kMaxRank / 32];
#pragma unroll
    for (int rb = 0; rb < kMaxRank / 32; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[rb][r] = 0;
    const tq_v4i zero4 = {0, 0, 0, 0};
    if (pre) {
        tq_v4i av[PRE];
#pragma unroll
        for (int c = 0; c < PRE; ++c) {
            av[c] = *reinterpret_cast<const tq_v4i *>(arow + c * 32);
            if (lr >= TOK) av[c] = zero4;
            if (!bok[0]) bpre[c] = zero4;
        }
#pragma unroll
        for (int c = 0; c < PRE; ++c) acc[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[c], bpre[c], acc[0], 0, 0, 0);
    } else {
        // runs of kTqRun K blocks, a run's loads issued before its MFMAs
        constexpr int kTqRun = 8;
        for (int c0 = 0; c0 < nkw; c0 += kTqRun) {
            tq_v4i av[kTqRun], bv[kTqRun][kMaxRank / 32];
#pragma unroll
            for (int c = 0; c < kTqRun; ++c) {
                const int k = min(c0 + c, nkw - 1) * 32;
                av[c] = *reinterpret_cast<const tq_v4i *>(arow + k);
                if (lr >= TOK) av[c] = zero4;
#pragma unroll
                for (int rb = 0; rb < kMaxRank / 32; ++rb) {
                    if (rb < nrb) {
                        bv[c][rb] = *reinterpret_cast<const tq_v4i *>(brow[rb] + k);
                        if (!bok[rb]) bv[c][rb] = zero4;
                    }
                }
            }
#pragma unroll
            for (int c = 0; c < kTqRun; ++c) {
                if (c0 + c < nkw) {
#pragma unroll
                    for (int rb = 0; rb < kMaxRank / 32; ++rb)
                        if (rb < nrb) acc[rb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[c], bv[c][rb], acc[rb], 0, 0, 0);
                }
            }
        }
    }
    // rows 0..7 of the block (the tokens) sit in accumulator entries r < 4: token 4 * hsel + r
#pragma unroll
    for (int rb = 0; rb < kMaxRank / 32; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) tred[wave][rb][r][lane] = acc[rb][r];
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < kMaxRank / 32; ++rb) {
        if (rb >= nrb || tid >= 256) break;
        const int r = tid >> 6, l = tid & 63;
        int tot = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) tot += tred[w][rb][r][l];   // exact, fixed order
        const int tok = 4 * (l >> 5) + r, j = rb * 32 + (l & 31), m = m0 + tok;
        if (tok < TOK && j < a.rank && m < a.M) {
            const float tp = dsv[rb] * s_l[tok] * (float)tot;
            const __bf16 hi = (__bf16)tp;
            const __bf16 lo = (__bf16)(tp - (float)hi);
            a.thi[(int64_t)m * a.rank + j] = hi;
            a.tlo[(int64_t)m * a.rank + j] = lo;
            if (a.tap_t) a.tap_t[(int64_t)m * a.rank + j] = tot;
        }
    }
}

// The same for few tokens (batched decode): one token per workgroup row, its LoRA-down rows split
// in slices of kTq1Rows over blockIdx.y (so that a few tokens still fill the chip and no workgroup
// reads more than its slice of L_dn). Every slice normalises and quantizes the whole token (the
// same code path, so the same codes); slice 0 writes the codes, scale and code sum. The thread's
// 4 KC codes (4 consecutive per chunk, chunks 1 KB apart) meet the same bytes of each L_dn row in
// sdot4 products, summed over the workgroup in a fixed order (exact integers).
constexpr int kTq1Rows = 8;
template <int KC>
__global__ __launch_bounds__(kBlock) void k_tok_quant1(TokQuantArgs a) {
    __shared__ float red[2 * kWaves];
    __shared__ int ired[kWaves];
    __shared__ int tred[kWaves][kTq1Rows];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = blockIdx.x, slice = blockIdx.y, j0 = slice * kTq1Rows, K = a.K;
    if (m == 0 && slice == 0)
        for (int i = tid; i < a.nzero; i += kBlock) a.zero_words[i] = 0u;
    // loads first: norm weight, the row, the slice's L_dn bytes at the thread's positions (clamped;
    // positions past K and rows past the rank are dropped later)
    float4 wv[KC], hv[KC];
#pragma unroll
    for (int i = 0; i < KC; ++i) wv[i] = *reinterpret_cast<const float4 *>(a.W + min((i * kBlock + tid) * 4, K - 4));
    if (a.x_bf16) {
        uint2 raw[KC];
#pragma unroll
        for (int i = 0; i < KC; ++i)
            raw[i] = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(a.X) + (int64_t)m * a.ldx +
                                                      min((i * kBlock + tid) * 4, K - 4));
#pragma unroll
        for (int i = 0; i < KC; ++i)
            hv[i] = make_float4(bf16_bits_to_float(raw[i].x & 0xffffu), bf16_bits_to_float(raw[i].x >> 16),
                                bf16_bits_to_float(raw[i].y & 0xffffu), bf16_bits_to_float(raw[i].y >> 16));
    } else {
#pragma unroll
        for (int i = 0; i < KC; ++i)
            hv[i] = *reinterpret_cast<const float4 *>(static_cast<const float *>(a.X) + (int64_t)m * a.ldx +
                                                      min((i * kBlock + tid) * 4, K - 4));
    }
    int ld[kTq1Rows][KC];
#pragma unroll
    for (int jj = 0; jj < kTq1Rows; ++jj) {
        const int8_t *lrow = a.lora_dn + (int64_t)min(j0 + jj, a.rank - 1) * K;
#pragma unroll
        for (int i = 0; i < KC; ++i) ld[jj][i] = *reinterpret_cast<const int *>(lrow + min((i * kBlock + tid) * 4, K - 4));
    }
    // ---- RMSNorm statistics and the quantizer
    float ss = 0.f, pm = 0.f;
#pragma unroll
    for (int i = 0; i < KC; ++i) {
        const bool ok = (i * kBlock + tid) * 4 < K;
        float4 &h = hv[i];
        h.x = ok ? h.x : 0.f;
        h.y = ok ? h.y : 0.f;
        h.z = ok ? h.z : 0.f;
        h.w = ok ? h.w : 0.f;
        ss += h.x * h.x + h.y * h.y + h.z * h.z + h.w * h.w;
    }
    const bool writer = slice == 0;
    if (a.tap_h && writer) {
#pragma unroll
        for (int i = 0; i < KC; ++i) {
            const int e = (i * kBlock + tid) * 4;
            if (e < K) *reinterpret_cast<float4 *>(a.tap_h + (int64_t)m * K + e) = hv[i];
        }
    }
#pragma unroll
    for (int i = 0; i < KC; ++i) {
        float4 &h = hv[i];
        h.x *= wv[i].x;
        h.y *= wv[i].y;
        h.z *= wv[i].z;
        h.w *= wv[i].w;
        pm = fmaxf(pm, fmaxf(fmaxf(fabsf(h.x), fabsf(h.y)), fmaxf(fabsf(h.z), fabsf(h.w))));
    }
    ss = dpp_wave_sum(ss);
    pm = dpp_wave_max(pm);
    if (lane == 0) {
        red[wave] = ss;
        red[kWaves + wave] = pm;
    }
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float mx = fmaxf(fmaxf(red[kWaves], red[kWaves + 1]), fmaxf(red[kWaves + 2], red[kWaves + 3]));
    // u = fl(fl(h * w) * r) so that max|u| = fl(max|h * w| * r) exactly (r > 0)
    const float r = 1.0f / sqrtf(tot / (float)K + a.eps);
    const float amax = mx * r;
    const float inv = amax > 0.f ? 127.0f / amax : 0.f;
    const float sv = amax > 0.f ? amax / 127.0f : 0.f;
    int qs = 0;
    int dacc[kTq1Rows];
#pragma unroll
    for (int jj = 0; jj < kTq1Rows; ++jj) dacc[jj] = 0;
#pragma unroll
    for (int i = 0; i < KC; ++i) {
        const int e = (i * kBlock + tid) * 4;
        if (e < K) {
            float4 v = hv[i];
            v.x *= r;
            v.y *= r;
            v.z *= r;
            v.w *= r;
            const int q0 = quant1(v.x, inv), q1 = quant1(v.y, inv), q2 = quant1(v.z, inv), q3 = quant1(v.w, inv);
            qs += q0 + q1 + q2 + q3;
            const uint32_t packed = (uint32_t)(q0 & 255) | ((uint32_t)(q1 & 255) << 8) | ((uint32_t)(q2 & 255) << 16) |
                                    ((uint32_t)(q3 & 255) << 24);
#pragma unroll
            for (int jj = 0; jj < kTq1Rows; ++jj) dacc[jj] = __builtin_amdgcn_sdot4((int)packed, ld[jj][i], dacc[jj], false);
            if (writer) {
                *reinterpret_cast<uint32_t *>(a.q + (int64_t)m * K + e) = packed;
                if (a.tap_u) *reinterpret_cast<float4 *>(a.tap_u + (int64_t)m * K + e) = v;
                if (a.tap_q) *reinterpret_cast<uint32_t *>(a.tap_q + (int64_t)m * K + e) = packed;
            }
        }
    }
    qs = dpp_wave_isum(qs);
#pragma unroll
    for (int jj = 0; jj < kTq1Rows; ++jj) dacc[jj] = dpp_wave_isum(dacc[jj]);
    if (lane == 0) {
        ired[wave] = qs;
#pragma unroll
        for (int jj = 0; jj < kTq1Rows; ++jj) tred[wave][jj] = dacc[jj];
    }
    __syncthreads();
    if (writer && tid == 0) {
        a.s[m] = sv;
        a.qsum[m] = (ired[0] + ired[1]) + (ired[2] + ired[3]);
        if (a.tap_s) a.tap_s[m] = sv;
    }
    if (tid < kTq1Rows && j0 + tid < a.rank) {
        const int j = j0 + tid;
        const int t = ((tred[0][tid] + tred[1][tid]) + tred[2][tid]) + tred[3][tid];
        const float tp = a.dn_scale[j] * sv * (float)t;
        const __bf16 hi = (__bf16)tp;
        const __bf16 lo = (__bf16)(tp - (float)hi);
        a.thi[(int64_t)m * a.rank + j] = hi;
        a.tlo[(int64_t)m * a.rank + j] = lo;
        if (a.tap_t) a.tap_t[(int64_t)m * a.rank + j] = t;
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

// SiLU and softplus for the sequence conv pass, on the hardware exp2 and reciprocal (a few ulp; the
// layer tolerance is 1e-3)
__device__ __forceinline__ float silu_fast(float v) {
    return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * v));
}
__device__ __forceinline__ float softplus_fast(float v) {
    return v > 20.0f ? v : log1pf(__builtin_amdgcn_exp2f(1.4426950408889634f * v));
}

// One thread per channel (or dt column) and run of kConvRun consecutive tokens of one sequence: the
// window of the last d_conv-1 inputs slides in registers (the run re-reads the d_conv-1 inputs
// before it), all of a run's loads before its first store (a load behind a store waits for it).
// Short runs measured fastest (8 tokens: 16.4 us per 2048 x 4416 pass, 32 tokens: 20.8): more
// threads in flight outweigh the re-read window. (Two or four channels per thread with 8- or
// 16-byte accesses measured slower.)
constexpr int kConvRun = 8;
__global__ __launch_bounds__(kBlock) void k_conv_seq(ConvSeqArgs a) {
    const int runs = (a.L + kConvRun - 1) / kConvRun;
    const int b = blockIdx.x / runs, t0 = (blockIdx.x - b * runs) * kConvRun;
    const int col = blockIdx.y * kBlock + threadIdx.x;
    if (col >= a.Cd + a.H) return;
    const int t1 = min(a.L, t0 + kConvRun);
    const int64_t mb = (int64_t)b * a.L;
    const float *yc = a.Y + a.E + col;
    float yv[kConvRun];
#pragma unroll
    for (int i = 0; i < kConvRun; ++i) yv[i] = yc[(mb + min(t0 + i, t1 - 1)) * a.ldY];
    if (col < a.Cd) {
        const float4 w = *reinterpret_cast<const float4 *>(a.conv_w + (int64_t)col * kConvTaps);
        const float bias = a.conv_b[col];
        // window = inputs at t0-3, t0-2, t0-1 (conv state entries for negative positions)
        float win[kConvTaps - 1];
#pragma unroll
        for (int k = 0; k < kConvTaps - 1; ++k) {
            const int tok = t0 - (kConvTaps - 1) + k;
            win[k] = tok >= 0 ? yc[(mb + tok) * a.ldY]
                              : a.conv_state[((int64_t)b * a.Cd + col) * (kConvTaps - 1) + (kConvTaps - 1) + tok];
        }
#pragma unroll
        for (int i = 0; i < kConvRun; ++i) {
            if (t0 + i >= t1) break;
            const float x = yv[i];
            const float v = bias + w.x * win[0] + w.y * win[1] + w.z * win[2] + w.w * x;
            a.xbc[(mb + t0 + i) * a.Cd + col] = silu_fast(v);
            win[0] = win[1];
            win[1] = win[2];
            win[2] = x;
        }
    } else {
        const int h = col - a.Cd;
        const float db = a.dt_bias[h];
#pragma unroll
        for (int i = 0; i < kConvRun; ++i) {
            if (t0 + i >= t1) break;
            a.dt[(mb + t0 + i) * a.H + h] = softplus_fast(yv[i] + db);
        }
    }
}

// ------------------------------------------------------------------ 5 SSD
struct SsdArgs {
    int B, L, H, P, N, G, E, Cd, Q, nch;
    const float *xbc;      // [M][Cd]: x | B (G*N) | C (G*N)
    const float *dt;       // [M][H]
    const float *A_log, *D;
    const float *Y;        // in_proj output (z at columns [0, E))
    int64_t ldY;
    float *cb;             // [B][G][nch][Q][Q]: CB[t][s] = C_t . B_s (s-tiles <= t-tile)
    float *lam_end;        // [B][H][nch] Lam at each chunk's last token
    float *sloc;           // [B][H][nch][P][N] chunk states (become the states entering each chunk)
    float *state;          // [B][H][P][N] initial -> final
    float *g;              // [M][E] gated output
    float *conv_state;     // [B][Cd][3]: replaced by the last d_conv-1 pre-activation inputs (C.B^T pass)
};

constexpr int kSsdMaxQ = 256, kSsdMaxN = 256, kSsdP = 64, kSsdWaves = 8, kSsdBlock = 64 * kSsdWaves;

typedef float f4v __attribute__((ext_vector_type(4)));
// Chunked SSD in three passes, each over every (b, h, chunk) at once (Lam_t = inclusive cumsum of
// dt A within the chunk; exponentials only of Lam differences, or of Lam itself, all <= 0):
//   k_ssd_cbm_state  S_loc = sum_s exp(Lam_end - Lam_s) dt_s x_s (x) B_s of the chunk, and Lam_end
//                (beside the C.B^T pass, in the same launch)
//   k_ssd_scan   S_in(c) = exp(Lam_end(c-1)) S_in(c-1) + S_loc(c-1), in place (sequential in c)
//   k_ssd_out    y_t = sum_{s<=t} exp(Lam_t - Lam_s) CB[t][s] dt_s x_s + exp(Lam_t) C_t . S_in + D x_t,
//                g = y SiLU(z)
// The contractions of the state and output passes run on bf16 MFMA 16x16x32 with every fp32
// operand split as v = hi + lo (hi = bf16(v), lo = bf16(v - hi)) and the product taken as
// a_hi b_hi + a_hi b_lo + a_lo b_hi: about 16 bits of each operand survive, so each product is
// within ~2^-16 relative of the fp32 one, at a sixth of the fp32 MFMA cost. Operands used by many
// products (x, the state) are scaled and split once per chunk into LDS planes; the others (C, CB,
// B) are split as they are loaded.
constexpr int kSsdRow = kSsdMaxQ + 8;   // bf16 per LDS plane row (the pad spreads rows over the banks)
static_assert(kSsdMaxN <= kSsdMaxQ, "state planes share the row length of the x planes");

typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
// bf16 MFMA 16x16x32: lane l supplies row (A) / column (B) l % 16 and the 8 contraction indices
// 8 (l / 16) .. +8, and holds D[4 (l / 16) + r][l % 16] in element r.
__device__ __forceinline__ f4v mfma_bf(const bf8v &a, const bf8v &b, f4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4v mfma_bf3(const bf8v &ah, const bf8v &al, const bf8v &bh, const bf8v &bl, f4v c) {
    c = mfma_bf(al, bh, c);
    c = mfma_bf(ah, bl, c);
    return mfma_bf(ah, bh, c);
}
__device__ __forceinline__ void split8(const float (&v)[8], bf8v &hi, bf8v &lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        hi[e] = (__bf16)v[e];
        lo[e] = (__bf16)(v[e] - (float)hi[e]);
    }
}
__device__ __forceinline__ void split_store2(__bf16 *hi, __bf16 *lo, float v0, float v1) {
    const __bf16 h0 = (__bf16)v0, h1 = (__bf16)v1;
    const __bf16 l0 = (__bf16)(v0 - (float)h0), l1 = (__bf16)(v1 - (float)h1);
    *reinterpret_cast<uint32_t *>(hi) = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    *reinterpret_cast<uint32_t *>(lo) = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
}

// Lam (in log2 units) and dt of the chunk's tokens (DPP block scan over dt_t A, dt_t from
// ssd_dt_load; Q <= kSsdBlock / 2); two barriers inside, the results are visible on return.
__device__ __forceinline__ float ssd_dt_load(const SsdArgs &a, int h, int64_t mbase, int len) {
    const int tid = threadIdx.x;
    const float v = a.dt[(mbase + min(tid, len - 1)) * a.H + h];
    return tid < len ? v : 0.f;
}
__device__ __forceinline__ void ssd_lam(const SsdArgs &a, int h, float dtv, float *lam2, float *dts, float *tot) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float A = -expf(a.A_log[h]);
    float v = dtv * A;
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false));
    if (lane == 63) tot[wave] = v;
    __syncthreads();
    for (int w = 0; w < wave; ++w) v += tot[w];
    if (tid < kSsdMaxQ) {
        constexpr float kLog2e = 1.4426950408889634f;
        lam2[tid] = v * kLog2e;
        dts[tid] = dtv;
    }
    __syncthreads();
}

// x of head h for all kSsdMaxQ token slots of the chunk (zero past its end) into planes [p][t]:
// raw x (hi, lo) when RAW, and x scaled by w_t = dt_t exp(Lam_ref(t) - Lam_t) (hi, lo), with
// ref(t) = the chunk's last token (END) or the last token of t's 32-token block (!END). Thread:
// token pair (2 tp, 2 tp + 1), 16 channels. The loads (ssd_x_load) are issued apart from the
// stores (ssd_x_store) so that they can be in flight during earlier work. No barrier.
struct SsdXRegs {
    float4 v[2][4];
};
__device__ __forceinline__ void ssd_x_load(const SsdArgs &a, int h, int64_t mbase, int len, SsdXRegs &x) {
    const int tid = threadIdx.x, tp = tid & 127, cq = tid >> 7;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const float *xr = a.xbc + (mbase + min(2 * tp + u, len - 1)) * a.Cd + h * a.P + 16 * cq;
#pragma unroll
        for (int j = 0; j < 4; ++j) x.v[u][j] = *reinterpret_cast<const float4 *>(xr + 4 * j);
    }
}
template <bool END, bool RAW>
__device__ __forceinline__ void ssd_x_store(const SsdXRegs &x, int len, const float *lam2, const float *dts, __bf16 *xh,
                                            __bf16 *xl, __bf16 *rh, __bf16 *rl) {
    const int tid = threadIdx.x, tp = tid & 127, cq = tid >> 7;
    const int t0 = 2 * tp;
    float w[2];
    bool in[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int t = t0 + u;
        const int ref = END ? len - 1 : min(t | 31, len - 1);
        in[u] = t < len;
        w[u] = in[u] ? dts[t] * __builtin_amdgcn_exp2f(lam2[ref] - lam2[t]) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float x0[4] = {x.v[0][j].x, x.v[0][j].y, x.v[0][j].z, x.v[0][j].w};
        const float x1[4] = {x.v[1][j].x, x.v[1][j].y, x.v[1][j].z, x.v[1][j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int o = (16 * cq + 4 * j + e) * kSsdRow + t0;
            const float r0 = in[0] ? x0[e] : 0.f, r1 = in[1] ? x1[e] : 0.f;
            split_store2(xh + o, xl + o, r0 * w[0], r1 * w[1]);
            if (RAW) split_store2(rh + o, rl + o, r0, r1);
        }
    }
}

// CB[t][s] = C_t . B_s of one 16-token t-tile of chunk c, group g, on bf16 MFMA with both operands
// split hi/lo: 8 waves, wave w takes the s-tiles w, w + 8, ... <= the t-tile (only those are read);
// the t-tile's C fragments are split once, each s-tile's B fragments as they load (the next
// s-tile's loads in flight while one computes). Also the conv-state hand-off.
constexpr int kCbmSplit = 2;   // workgroups per (chunk, t-tile): 9.0 -> 6.7 us (4: 9.3)
// Workgroup wg of the ncbm = (B G nch) x (Q / 16) x kCbmSplit of this pass (bgc fastest, then the
// t-tile, then the split). NBM: 32-wide blocks of d_state held (N <= 32 NBM).
template <int NBM>
__device__ __forceinline__ void ssd_cbm_body(const SsdArgs &a, int wg, int ncbm) {
    const int nbgc = a.B * a.G * a.nch, ntt = a.Q / 16;
    const int bgc = wg % nbgc, ti = (wg / nbgc) % ntt, zsp = wg / (nbgc * ntt);
    {   // conv-state handoff, per (sequence, channel): new state[i] = element L + i of
        // [old state (3) | the sequence's conv inputs (L)] (the conv pass has read the old state)
        const int nthr = ncbm * kSsdBlock;
        for (int idx = wg * kSsdBlock + threadIdx.x; idx < a.B * a.Cd; idx += nthr) {
            const int bb = idx / a.Cd, ch = idx - bb * a.Cd;
            float *st = a.conv_state + (int64_t)idx * (kConvTaps - 1);
            float nv[kConvTaps - 1];
#pragma unroll
            for (int i = 0; i < kConvTaps - 1; ++i) {
                const int p = a.L + i;
                nv[i] = p < kConvTaps - 1 ? st[p] : a.Y[((int64_t)bb * a.L + p - (kConvTaps - 1)) * a.ldY + a.E + ch];
            }
#pragma unroll
            for (int i = 0; i < kConvTaps - 1; ++i) st[i] = nv[i];
        }
    }
    const int c = bgc % a.nch, g = (bgc / a.nch) % a.G, b = bgc / (a.nch * a.G);
    const int len = min(a.Q, a.L - c * a.Q);
    if (ti * 16 >= len) return;   // no barriers in this pass
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, r = lane & 15, kq = lane >> 4;
    const int64_t mbase = (int64_t)b * a.L + c * a.Q;
    const int N = a.N, NB = (N + 31) / 32;
    // lane: row (C) / column (B) r of its tile, d_state indices 32 nb + 8 kq .. +8 (zero past N)
    auto load8 = [&](const float *row, int nb, float (&v)[8]) {
        const int n = 32 * nb + 8 * kq, nc = min(n, N - 8);
        const float4 v0 = *reinterpret_cast<const float4 *>(row + nc), v1 = *reinterpret_cast<const float4 *>(row + nc + 4);
        const bool ok = n < N;
        v[0] = ok ? v0.x : 0.f; v[1] = ok ? v0.y : 0.f; v[2] = ok ? v0.z : 0.f; v[3] = ok ? v0.w : 0.f;
        v[4] = ok ? v1.x : 0.f; v[5] = ok ? v1.y : 0.f; v[6] = ok ? v1.z : 0.f; v[7] = ok ? v1.w : 0.f;
    };
    const float *Crow = a.xbc + (mbase + min(ti * 16 + r, len - 1)) * a.Cd + a.E + a.G * N + g * N;
    bf8v ch[NBM], cl[NBM];
#pragma unroll
    for (int nb = 0; nb < NBM; ++nb) {
        if (nb < NB) {
            float v[8];
            load8(Crow, nb, v);
            split8(v, ch[nb], cl[nb]);
        }
    }
    float *out = a.cb + (((int64_t)b * a.G + g) * a.nch + c) * a.Q * a.Q;
    // the t-tile's s-tiles are spread over the kCbmSplit workgroups of (chunk, t-tile) and their waves
    for (int si = zsp * kSsdWaves + wave; si <= ti; si += kSsdWaves * kCbmSplit) {
        const float *Brow = a.xbc + (mbase + min(si * 16 + r, len - 1)) * a.Cd + a.E + g * N;
        float bv[NBM][8];
#pragma unroll
        for (int nb = 0; nb < NBM; ++nb)
            if (nb < NB) load8(Brow, nb, bv[nb]);
        f4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nb = 0; nb < NBM; ++nb) {
            if (nb < NB) {
                bf8v bh, bl;
                split8(bv[nb], bh, bl);
                acc = mfma_bf3(ch[nb], cl[nb], bh, bl, acc);
            }
        }
        // lane l holds CB[t = 16 ti + 4 kq + rr][s = 16 si + r]
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) out[(int64_t)(ti * 16 + 4 * kq + rr) * a.Q + si * 16 + r] = acc[rr];
    }
}

// S_loc of one (b, h, chunk) = Xs . B with Xs[p][s] = exp(Lam_end - Lam_s) dt_s x_s (LDS planes)
// and B[s][n] straight from global memory. Wave w takes the n-tiles w, w + 8, ... for all four
// p-tiles, so each split B fragment feeds four p-tiles.
// Workgroup blk of B H nch.
__device__ __forceinline__ void ssd_state_body(const SsdArgs &a, int blk) {
    __shared__ float lam2[kSsdMaxQ], dts[kSsdMaxQ], tot[kSsdWaves];
    __shared__ __align__(16) __bf16 xh[kSsdP * kSsdRow], xl[kSsdP * kSsdRow];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r = lane & 15, kq = lane >> 4;
    const int c = blk % a.nch, bh = blk / a.nch, h = bh % a.H, b = bh / a.H;
    const int g = h * a.G / a.H, Q = a.Q, N = a.N, NT = N / 16;
    const int len = min(Q, a.L - c * Q);
    const int64_t mbase = (int64_t)b * a.L + c * Q;
    const int nsb = (len + 31) / 32;   // 32-token blocks holding the chunk's tokens
    const float *Bbase = a.xbc + mbase * a.Cd + a.E + g * N;
    // B[s][n] of an n-tile, all blocks (rows clamped into the chunk: tokens past its end meet Xs = 0)
    // B[s][n] of one 32-token block of an n-tile (rows clamped into the chunk: tokens past its end
    // meet Xs = 0); two blocks in flight: block sb + 1 loads while block sb computes
    float bq[2][8];
#define SSD_LOAD_B(nt, sb, dst)                                                                                 \
    {                                                                                                           \
        const float *bcol = Bbase + (nt) * 16 + r;                                                              \
        _Pragma("unroll") for (int e = 0; e < 8; ++e)                                                           \
            dst[e] = bcol[(int64_t)min(32 * (sb) + 8 * kq + e, len - 1) * a.Cd];                               \
    }
    const float dtv = ssd_dt_load(a, h, mbase, len);
    SsdXRegs xr;
    ssd_x_load(a, h, mbase, len, xr);
    SSD_LOAD_B(min(wave, NT - 1), 0, bq[0])   // in flight during the prologue
    ssd_lam(a, h, dtv, lam2, dts, tot);
    ssd_x_store<true, false>(xr, len, lam2, dts, xh, xl, nullptr, nullptr);
    if (tid == 0) a.lam_end[(int64_t)bh * a.nch + c] = lam2[len - 1] * 0.6931471805599453f;
    __syncthreads();
    float *out = a.sloc + ((int64_t)bh * a.nch + c) * kSsdP * N;
    for (int nt = wave; nt < NT; nt += kSsdWaves) {
        if (nt != wave) SSD_LOAD_B(nt, 0, bq[0])
        f4v acc[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[pt] = f4v{0.f, 0.f, 0.f, 0.f};
        auto block = [&](int sb, const float (&bv)[8]) {
            const int s0 = 32 * sb + 8 * kq;
            bf8v bhv, blv;
            split8(bv, bhv, blv);
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const int o = (16 * pt + r) * kSsdRow + s0;
                const bf8v ahv = *reinterpret_cast<const bf8v *>(xh + o);
                const bf8v alv = *reinterpret_cast<const bf8v *>(xl + o);
                acc[pt] = mfma_bf3(ahv, alv, bhv, blv, acc[pt]);
            }
        };
#pragma unroll 1
        for (int sb = 0; sb < nsb; sb += 2) {
            if (sb + 1 < nsb) SSD_LOAD_B(nt, sb + 1, bq[1])
            block(sb, bq[0]);
            if (sb + 1 < nsb) {
                if (sb + 2 < nsb) SSD_LOAD_B(nt, sb + 2, bq[0])
                block(sb + 1, bq[1]);
            }
        }
        // lane l holds S_loc[p = 16 pt + 4 kq + rr][n = 16 nt + r]
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) out[(int64_t)(16 * pt + 4 * kq + rr) * N + nt * 16 + r] = acc[pt][rr];
    }
#undef SSD_LOAD_B
}

// The two passes that need only the conv outputs, in one launch: the ncbm C.B^T workgroups first
// (short), then the B H nch chunk-state workgroups, which take the slots the short ones free (one
// launch of 6.8 + 19.7 us became one of about 20). Two workgroups per compute unit (<= 128 registers)
// up to d_state 128; d_state 256 holds twice the C.B^T operands and runs one (no spills).
template <int NBM>
__global__ __launch_bounds__(kSsdBlock) __attribute__((amdgpu_waves_per_eu(NBM <= 4 ? 4 : 2))) void k_ssd_cbm_state(SsdArgs a, int ncbm) {
    const int wg = blockIdx.x;
    if (wg < ncbm) ssd_cbm_body<NBM>(a, wg, ncbm);
    else ssd_state_body(a, wg - ncbm);
}

// Sequential carry over chunks; sloc[c] is replaced by the state entering chunk c. Chunks go in
// groups of kScanGroup whose loads are all issued before the group's stores.
constexpr int kScanGroup = 8;
__global__ __launch_bounds__(kBlock) void k_ssd_scan(SsdArgs a) {
    const int64_t PN = (int64_t)a.P * a.N;   // even (P = 64)
    const int bh = blockIdx.y;
    const int64_t e = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * 2;   // two state entries per thread
    if (e >= PN) return;
    float2 S = *reinterpret_cast<const float2 *>(a.state + (int64_t)bh * PN + e);
    for (int c0 = 0; c0 < a.nch; c0 += kScanGroup) {
        float2 loc[kScanGroup];
        float dec[kScanGroup];
#pragma unroll
        for (int i = 0; i < kScanGroup; ++i) {
            const int c = min(c0 + i, a.nch - 1);
            loc[i] = *reinterpret_cast<const float2 *>(a.sloc + ((int64_t)bh * a.nch + c) * PN + e);
            dec[i] = a.lam_end[(int64_t)bh * a.nch + c];
        }
#pragma unroll
        for (int i = 0; i < kScanGroup; ++i) {
            if (c0 + i >= a.nch) break;
            *reinterpret_cast<float2 *>(a.sloc + ((int64_t)bh * a.nch + c0 + i) * PN + e) = S;
            const float f = expf(dec[i]);
            S.x = f * S.x + loc[i].x;
            S.y = f * S.y + loc[i].y;
        }
    }
    *reinterpret_cast<float2 *>(a.state + (int64_t)bh * PN + e) = S;
}

// Outputs of one (b, h, chunk): wave w owns the 16-token t-tiles {w, 15 - w} (balanced causal
// work) and all four 16-channel p-tiles of each; every term is accumulated already scaled:
//   phase A  exp(Lam_t) C_t . S_in       A = C_t exp(Lam_t) (split on load), B = S_in (LDS planes)
//   phase B  off-diagonal 32-token blocks (s <= e = the block's last token < the tile):
//              sum_s [CB[t][s] exp(Lam_t - Lam_e)] [x_s dt_s exp(Lam_e - Lam_s)]   (B: LDS planes)
//            the diagonal block (the one holding t):
//              sum_{s <= t} [CB[t][s] exp(Lam_t - Lam_s) dt_s] x_s                 (B: x from memory)
// Every exponential is of a non-positive number. The S_in planes and the x planes share 67.5 KB of
// LDS and the kernel keeps to 128 registers, so two workgroups share a compute unit and one
// workgroup's loads overlap the other's MFMA work. NB = 32-wide blocks of d_state (N <= 32 NB).
template <int NB>
__global__ __launch_bounds__(kSsdBlock) __attribute__((amdgpu_waves_per_eu(4))) void k_ssd_out(SsdArgs a) {
    __shared__ float lam2[kSsdMaxQ], dts[kSsdMaxQ], tot[kSsdWaves];
    __shared__ __align__(16) __bf16 pl[2][kSsdP * kSsdRow];   // phase A: S_in hi, lo; phase B: xs hi, lo
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r = lane & 15, kq = lane >> 4;
    const int c = blockIdx.x % a.nch, bh = blockIdx.x / a.nch, h = bh % a.H, b = bh / a.H;
    const int g = h * a.G / a.H, Q = a.Q, N = a.N, QT = Q / 16;
    const int len = min(Q, a.L - c * Q);
    const int64_t mbase = (int64_t)b * a.L + c * Q;
    const float Dh = a.D[h];
    int tiles[2];
    bool live[2];
    tiles[0] = wave;
    tiles[1] = 15 - wave;
#pragma unroll
    for (int k = 0; k < 2; ++k) live[k] = tiles[k] < QT && tiles[k] * 16 < len;
    const float dtv = ssd_dt_load(a, h, mbase, len);
    {   // S_in planes [p][n], zero for n in [N, 32 NB)
        const float *sin = a.sloc + ((int64_t)bh * a.nch + c) * kSsdP * N;
        constexpr int NP = 32 * NB, J = kSsdP * NP / 2 / kSsdBlock;
        float2 sv[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int i = tid + j * kSsdBlock, p = (2 * i) / NP, n = (2 * i) % NP;
            sv[j] = *reinterpret_cast<const float2 *>(sin + (int64_t)p * N + min(n, N - 2));
        }
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int i = tid + j * kSsdBlock, p = (2 * i) / NP, n = (2 * i) % NP;
            if (n >= N) sv[j] = make_float2(0.f, 0.f);
            split_store2(pl[0] + p * kSsdRow + n, pl[1] + p * kSsdRow + n, sv[j].x, sv[j].y);
        }
    }
    ssd_lam(a, h, dtv, lam2, dts, tot);   // its barriers also publish the S_in planes
    f4v y[2][4];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) y[k][pt] = f4v{0.f, 0.f, 0.f, 0.f};
    // ---- phase A: exp(Lam_t) C_t . S_in
    const float *Cbase = a.xbc + mbase * a.Cd + a.E + a.G * N + g * N;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (!live[k]) continue;
        const int t = min(tiles[k] * 16 + r, len - 1);
        const float *Crow = Cbase + (int64_t)t * a.Cd;
        float4 cl[NB][2];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int nc = min(32 * nb + 8 * kq, N - 8);
            cl[nb][0] = *reinterpret_cast<const float4 *>(Crow + nc);
            cl[nb][1] = *reinterpret_cast<const float4 *>(Crow + nc + 4);
        }
        const float et = __builtin_amdgcn_exp2f(lam2[t]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const float e = 32 * nb + 8 * kq < N ? et : 0.f;   // d_state columns past N (clamped loads) count 0
            const float4 c0 = cl[nb][0], c1 = cl[nb][1];
            const float cv[8] = {c0.x * e, c0.y * e, c0.z * e, c0.w * e, c1.x * e, c1.y * e, c1.z * e, c1.w * e};
            bf8v ahv, alv;
            split8(cv, ahv, alv);
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const int o = (16 * pt + r) * kSsdRow + 32 * nb + 8 * kq;
                const bf8v bhv = *reinterpret_cast<const bf8v *>(pl[0] + o);
                const bf8v blv = *reinterpret_cast<const bf8v *>(pl[1] + o);
                y[k][pt] = mfma_bf3(ahv, alv, bhv, blv, y[k][pt]);
            }
        }
    }
    __syncthreads();   // the S_in planes are dead: the scaled x planes take their place
    {
        SsdXRegs xr;
        ssd_x_load(a, h, mbase, len, xr);
        ssd_x_store<false, false>(xr, len, lam2, dts, pl[0], pl[1], nullptr, nullptr);
    }
    __syncthreads();
    // ---- phase B: CB-weighted sums over the chunk's earlier tokens
    const float *cbbase = a.cb + (((int64_t)b * a.G + g) * a.nch + c) * Q * Q;
    const float *xbase = a.xbc + mbase * a.Cd + (int64_t)h * a.P;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (!live[k]) continue;
        const int ti = tiles[k];
        const int t = min(ti * 16 + r, len - 1);
        const float lt = lam2[t];
        const float *cbrow = cbbase + (int64_t)t * Q;
        const int bd = ti >> 1;   // the 32-token block holding the tile
        // z of the tile's outputs (lane l: rows ti*16 + 4 kq + rr, channels 16 pt + r), in flight during the tile
        float zr[4][4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int64_t m = mbase + min(ti * 16 + 4 * kq + rr, len - 1);
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) zr[rr][pt] = a.Y[m * a.ldY + (int64_t)h * a.P + 16 * pt + r];
        }
        // off-diagonal blocks, the next block's CB in flight while one computes
        float4 cn[2];
        {
            const int s0 = min(8 * kq, Q - 8);
            cn[0] = *reinterpret_cast<const float4 *>(cbrow + s0);
            cn[1] = *reinterpret_cast<const float4 *>(cbrow + s0 + 4);
        }
        for (int sb = 0; sb < bd; ++sb) {
            const float4 c0 = cn[0], c1 = cn[1];
            {
                const int s1 = min(32 * (sb + 1) + 8 * kq, Q - 8);
                cn[0] = *reinterpret_cast<const float4 *>(cbrow + s1);
                cn[1] = *reinterpret_cast<const float4 *>(cbrow + s1 + 4);
            }
            const int s0 = 32 * sb + 8 * kq;
            const float f = __builtin_amdgcn_exp2f(lt - lam2[32 * sb + 31]);
            const float cv[8] = {c0.x * f, c0.y * f, c0.z * f, c0.w * f, c1.x * f, c1.y * f, c1.z * f, c1.w * f};
            bf8v ahv, alv;
            split8(cv, ahv, alv);
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                const int o = (16 * pt + r) * kSsdRow + s0;
                const bf8v bhv = *reinterpret_cast<const bf8v *>(pl[0] + o);
                const bf8v blv = *reinterpret_cast<const bf8v *>(pl[1] + o);
                y[k][pt] = mfma_bf3(ahv, alv, bhv, blv, y[k][pt]);
            }
        }
        {   // the diagonal block (cn holds its CB): entries with s > t, or past the chunk, are never
            // read (select, not product); B = x of the block's tokens (rows clamped into the chunk)
            const int s0 = 32 * bd + 8 * kq;
            const float raw[8] = {cn[0].x, cn[0].y, cn[0].z, cn[0].w, cn[1].x, cn[1].y, cn[1].z, cn[1].w};
            float xd[4][8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float *xrow = xbase + (int64_t)min(s0 + e, len - 1) * a.Cd + r;
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) xd[pt][e] = xrow[16 * pt];
            }
            // the skip term D x_t rides on the diagonal entry: A[t][t] = CB[t][t] dt_t + D
            float cv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int s = s0 + e;
                cv[e] = s <= t ? raw[e] * __builtin_amdgcn_exp2f(lt - lam2[s]) * dts[s] + (s == t ? Dh : 0.f) : 0.f;
            }
            bf8v ahv, alv;
            split8(cv, ahv, alv);
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) {
                bf8v bhv, blv;
                split8(xd[pt], bhv, blv);
                y[k][pt] = mfma_bf3(ahv, alv, bhv, blv, y[k][pt]);
            }
        }
        // gate, out: lane l holds row ti*16 + 4 kq + rr, channel 16 pt + r
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int tt = ti * 16 + 4 * kq + rr;
            if (tt < len) {
                const int64_t m = mbase + tt;
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const int64_t col = (int64_t)h * a.P + 16 * pt + r;
                    a.g[m * a.E + col] = y[k][pt][rr] * silu_fast(zr[rr][pt]);
                }
            }
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
        if (batch <= 64) {   // the skinny GEMM runs the conv step in its epilogue
            const ConvEpi c{s.E, s.Cd, s.H, w.conv_w, w.conv_b, w.dt_bias, st.conv, dws.zbuf, dws.xbc, dws.dtbuf};
            if ((e = launch_gemm_pm1_conv(a, c, stream)) != hipSuccess) return e;
        } else {
            if ((e = launch_gemm_pm1(a, stream)) != hipSuccess) return e;
            ConvStepArgs cs{pws.Y, s.Ninp, s.E, s.Cd, s.H, w.conv_w, w.conv_b, w.dt_bias, st.conv, dws.zbuf, dws.xbc, dws.dtbuf};
            k_conv_step_y<<<dim3((s.Nin + kBlock - 1) / kBlock, batch), kBlock, 0, stream>>>(cs);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
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
    if (a.K > kMaxK || a.K % 128 || a.rank > kMaxRank || a.rank <= 0 || a.M <= 0) return hipErrorInvalidValue;
    if (a.M <= kTq1MaxM) {   // few tokens: one per workgroup
        const dim3 grid(a.M, (a.rank + kTq1Rows - 1) / kTq1Rows);
        if (a.K <= 1024) k_tok_quant1<1><<<grid, kBlock, 0, stream>>>(a);
        else if (a.K <= 2048) k_tok_quant1<2><<<grid, kBlock, 0, stream>>>(a);
        else if (a.K <= 4096) k_tok_quant1<4><<<grid, kBlock, 0, stream>>>(a);
        else k_tok_quant1<8><<<grid, kBlock, 0, stream>>>(a);
        return hipGetLastError();
    }
    // one wave per token while the rows fit the registers of 2 waves per SIMD, else two tokens per wave
    const int grid = (a.M + kTqTok - 1) / kTqTok;
    if (a.K <= 1024) k_tok_quant<4, kTqTok, 8><<<grid, 512, 0, stream>>>(a);
    else if (a.K <= 2048) k_tok_quant<8, kTqTok, 8><<<grid, 512, 0, stream>>>(a);
    else if (a.K <= 4096) k_tok_quant<16, kTqTok, 4><<<grid, 256, 0, stream>>>(a);
    else k_tok_quant<32, kTqTok, 4><<<grid, 256, 0, stream>>>(a);
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
    const int nch = chunk > 0 ? (seqlen + chunk - 1) / chunk : 0;   // chunk 0: decode, no scan buffers
    w.q_in = static_cast<int8_t *>(take(M * s.D));
    w.s_in = static_cast<float *>(take(M * 4));
    w.qsum_in = static_cast<int32_t *>(take(M * 4));
    w.thi_in = static_cast<__bf16 *>(take(M * s.Rin * 2));
    w.tlo_in = static_cast<__bf16 *>(take(M * s.Rin * 2));
    w.Y = static_cast<float *>(take(M * s.Ninp * 4));
    w.xbc = static_cast<float *>(take(M * s.Cd * 4));
    w.dt = static_cast<float *>(take(M * s.H * 4));
    w.cb = static_cast<float *>(take((size_t)batch * s.G * nch * chunk * chunk * 4));
    w.lam_end = static_cast<float *>(take((size_t)batch * s.H * nch * 4));
    w.sloc = static_cast<float *>(take((size_t)batch * s.H * nch * s.P * s.N * 4));
    w.gbuf = static_cast<float *>(take(M * s.E * 4));
    w.q_out = static_cast<int8_t *>(take(M * s.E));
    w.s_out = static_cast<float *>(take(M * 4));
    w.qsum_out = static_cast<int32_t *>(take(M * 4));
    w.thi_out = static_cast<__bf16 *>(take(M * s.Rout * 2));
    w.tlo_out = static_cast<__bf16 *>(take(M * s.Rout * 2));
    w.gemm_scratch = take(std::max({gemm_scratch_bytes((int)M, s.Ninp, s.D), gemm_scratch_bytes((int)M, 2 * s.E, s.D),
                                    gemm_scratch_bytes((int)M, s.Ninp - 2 * s.E, s.D), gemm_scratch_bytes((int)M, s.D, s.E)}));
    w.bytes = off;
    return w;
}

hipError_t launch_layer_prefill(const Shape &s, const dfssm_layer_weights &w, const dfssm_layer_state &st,
                                const void *x_in, int x_bf16, float *x_out, int batch, int seqlen, int chunk,
                                const PrefillWs &ws, const dfssm_taps *taps, hipStream_t stream,
                                const PrefillCodec *codec) {
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
        // the split-K counters of this layer's GEMMs (each launch leaves them zero again)
        a.zero_words = static_cast<uint32_t *>(ws.gemm_scratch);
        a.nzero = std::max({gemm_counter_words(M, 2 * s.E, s.D), gemm_counter_words(M, s.Ninp - 2 * s.E, s.D),
                            gemm_counter_words(M, s.D, s.E)});
        if ((e = launch_tok_quant(a, stream)) != hipSuccess) return e;
    }
    // 2. in_proj GEMM
    {
        GemmArgs a{};
        a.q = ws.q_in;
        a.ldq = s.D;
        a.qsum = ws.qsum_in;
        a.s = ws.s_in;
        a.M = M;
        a.K = s.D;
        a.rank = s.Rin;
        a.thi = ws.thi_in;
        a.tlo = ws.tlo_in;
        a.ldy = s.Ninp;
        a.ldacc = s.Ninp;
        a.scratch = ws.gemm_scratch;
        // two GEMMs over the same codes: the z | x rows (wide tiles, a whole number of them) and the
        // B | C | dt rows (few columns: narrow tiles with the K range split), in one launch with the
        // narrow units first, so that neither leaves a short tail of whole tiles behind
        const int cuts[3] = {0, 2 * s.E, s.Ninp};
        GemmArgs part[2];
        for (int k = 0; k < 2; ++k) {
            GemmArgs &g = part[k];
            g = a;
            const int n0 = cuts[k];
            g.N = cuts[k + 1] - n0;
            g.sign = w.in_proj.sign + (int64_t)n0 * (s.D / 8);
            g.row_scale = w.in_proj.row_scale + n0;
            g.up_scale = w.in_proj.lora_up_scale + n0;
            g.lora_up = w.in_proj.lora_up + (int64_t)n0 * s.Rin;
            g.y = ws.Y + n0;
            g.acc_tap = tp.in_acc ? tp.in_acc + n0 : nullptr;
            g.counters_zeroed = 1;
        }
        if (M > 64) {
            if ((e = launch_gemm_pm1_pair(part[0], part[1], stream)) != hipSuccess) return e;
        } else {
            for (int k = 0; k < 2; ++k)
                if ((e = launch_gemm_pm1(part[k], stream)) != hipSuccess) return e;
        }
    }
    // 3/4. conv over the sequence, dt, conv-state handoff
    ConvSeqArgs cv{ws.Y, s.Ninp, s.E, s.Cd, s.H, seqlen, M, w.conv_w, w.conv_b, w.dt_bias, st.conv, ws.xbc, ws.dt};
    {
        dim3 grid(batch * ((seqlen + kConvRun - 1) / kConvRun), (s.Cd + s.H + kBlock - 1) / kBlock);
        k_conv_seq<<<grid, kBlock, 0, stream>>>(cv);
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
        a.cb = ws.cb;
        a.lam_end = ws.lam_end;
        a.sloc = ws.sloc;
        a.state = st.ssm;
        a.g = ws.gbuf;
        a.conv_state = st.conv;
        const int nblk = batch * s.H * nch, ncbm = batch * s.G * nch * (chunk / 16) * kCbmSplit;
        if (s.N <= 32) k_ssd_cbm_state<1><<<ncbm + nblk, kSsdBlock, 0, stream>>>(a, ncbm);
        else if (s.N <= 64) k_ssd_cbm_state<2><<<ncbm + nblk, kSsdBlock, 0, stream>>>(a, ncbm);
        else if (s.N <= 128) k_ssd_cbm_state<4><<<ncbm + nblk, kSsdBlock, 0, stream>>>(a, ncbm);
        else k_ssd_cbm_state<8><<<ncbm + nblk, kSsdBlock, 0, stream>>>(a, ncbm);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (codec && codec->on) {
            e = launch_ssd_scan_codec(st.ssm, ws.sloc, ws.lam_end, batch * s.H, nch, s.N, s.P, codec->tap_pre,
                                      codec->tap_in, stream);
        } else {
            k_ssd_scan<<<dim3((s.P * s.N / 2 + kBlock - 1) / kBlock, batch * s.H), kBlock, 0, stream>>>(a);
            e = hipGetLastError();
        }
        if (e != hipSuccess) return e;
        if (s.N <= 32) k_ssd_out<1><<<nblk, kSsdBlock, 0, stream>>>(a);
        else if (s.N <= 64) k_ssd_out<2><<<nblk, kSsdBlock, 0, stream>>>(a);
        else if (s.N <= 128) k_ssd_out<4><<<nblk, kSsdBlock, 0, stream>>>(a);
        else k_ssd_out<8><<<nblk, kSsdBlock, 0, stream>>>(a);
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
        a.counters_zeroed = 1;
        if ((e = launch_gemm_pm1(a, stream)) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace dfssm
