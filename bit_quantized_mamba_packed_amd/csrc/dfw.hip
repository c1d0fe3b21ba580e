// Projection with the 17-level scaffold ([DF-SSM] §3.1 Eq. (1), K_w = 16; §3.2 Eq. (3)): the weight
// of row n, input i is (k[n][i] - 8)/8 times the row's fp16 scale, k the 5-bit level index 0..16
// held in five bit planes (plane b = bit b of k, each in the 1-bit scaffold layout: bit i % 8 of
// byte i / 8 of the row).
//
//   k_dfw_quant  per token: (q, s) = the per-token int8 quantizer of x (a = max|x|, q = rint(x*127/a)),
//                the eight bit planes of q (two's complement), sum(q), and the LoRA-down
//                t[j] = sum_i L_dn[j][i] q[i] (int32, sdot4; one row per wave, rank / 4 workgroups
//                per token)
//   k_dfw_gemv   acc[n] = sum_i (k[n][i] - 8) q[i]
//                       = sum_{b,p} 2^b w_p popcount(plane_b[n] & qplane_p) - 8 sum(q)
//                (w_p = 2^p, w_7 = -128), exact in int32; then
//                y[n] = s*sc[n]*acc[n]/8 + us[n] * sum_j L_up[n][j] * (ds[j] * s * t[j])
//
// The GEMV streams the five planes once per group of up to four tokens (5/8 byte per weight); a
// lane takes one 16-byte chunk (128 weights) of each plane per row and the lanes of a row add
// their partial sums with DPP. Per 128 weights and token it issues 8 x 5 x 4 AND + bit-count
// pairs, so at one token it is bound by HBM and beyond that by the vector ALU.
#include "decode_device.h"

namespace dfssm {

namespace {

constexpr int kDfwPlanes = 5;
constexpr int kDfwBlock = 128;           // threads of a GEMV workgroup (2 waves)
constexpr int kDfwWaves = kDfwBlock / 64;

struct DfwQuantArgs {
    const float *x;         // [batch][K]
    int K, rank;
    const int8_t *lora_dn;  // [rank][K]
    int8_t *q;              // [batch][K]
    uint32_t *qpl;          // [batch][8][K/32]
    float *s;               // [batch]
    int32_t *qsum;          // [batch]
    int32_t *t;             // [batch][rank]
};

// grid (batch, ceil(rank / kWaves)): every workgroup quantizes its whole token (the same code path,
// so the same codes; the workgroups of slice 0 publish them) and wave w forms LoRA-down row
// blockIdx.y * kWaves + w, so the rows' loads run in parallel across the chip instead of one after
// another in one workgroup.
__global__ __launch_bounds__(kBlock) void k_dfw_quant(DfwQuantArgs a) {
    extern __shared__ __align__(16) int8_t sq[];   // [K]
    __shared__ float red[2 * kWaves];
    __shared__ int ired[kWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x, K = a.K;
    const bool pub = blockIdx.y == 0;
    const float *x = a.x + (int64_t)b * K;
    // LoRA-down row of this wave: its loads go out first
    const int j = blockIdx.y * kWaves + wave;
    const bool has_row = j < a.rank;
    const int8_t *lrow = a.lora_dn + (int64_t)(has_row ? j : 0) * K;
    constexpr int kMaxLc = 8;   // 16-byte chunks per lane: K <= 8192
    int4 lw[kMaxLc];
#pragma unroll
    for (int c = 0; c < kMaxLc; ++c) {
        const int e = 16 * (lane + 64 * c);
        lw[c] = has_row && e < K ? *reinterpret_cast<const int4 *>(lrow + e) : make_int4(0, 0, 0, 0);
    }
    constexpr int kMaxXc = 8;   // float4 chunks of x per thread: K <= 8192
    float4 xv[kMaxXc];
#pragma unroll
    for (int c = 0; c < kMaxXc; ++c) {
        const int e = 4 * (tid + kBlock * c);
        xv[c] = e < K ? *reinterpret_cast<const float4 *>(x + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float m = 0.f;
#pragma unroll
    for (int c = 0; c < kMaxXc; ++c)
        m = fmaxf(m, fmaxf(fmaxf(fabsf(xv[c].x), fabsf(xv[c].y)), fmaxf(fabsf(xv[c].z), fabsf(xv[c].w))));
    m = block_max(m, red);
    const float inv = m > 0.f ? 127.0f / m : 0.f;
    const float s = m > 0.f ? m / 127.0f : 0.f;
    int qs = 0;
#pragma unroll
    for (int c = 0; c < kMaxXc; ++c) {
        const int e = 4 * (tid + kBlock * c);
        if (e >= K) break;
        const float4 v = xv[c];
        const int q0 = quant1(v.x, inv), q1 = quant1(v.y, inv), q2 = quant1(v.z, inv), q3 = quant1(v.w, inv);
        qs += q0 + q1 + q2 + q3;
        const uint32_t packed = (uint32_t)(q0 & 255) | ((uint32_t)(q1 & 255) << 8) | ((uint32_t)(q2 & 255) << 16) |
                                ((uint32_t)(q3 & 255) << 24);
        *reinterpret_cast<uint32_t *>(sq + e) = packed;
        if (pub) *reinterpret_cast<uint32_t *>(a.q + (int64_t)b * K + e) = packed;
    }
    qs = block_isum(qs, ired);   // its barriers also publish sq
    if (pub) {
        if (tid == 0) {
            a.s[b] = s;
            a.qsum[b] = qs;
        }
        // bit planes: wave ballots over 64 consecutive codes
        const int G32 = K >> 5;
        uint32_t *pl = a.qpl + (int64_t)b * 8 * G32;
        for (int c = wave; c < (K >> 6); c += kWaves) {
            const uint32_t v = (uint8_t)sq[c * 64 + lane];
            uint64_t mine = 0;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const uint64_t bal = __ballot((v >> p) & 1u);
                if ((lane & 7) == p) mine = bal;
            }
            if (lane < 16) pl[(lane & 7) * G32 + 2 * c + (lane >> 3)] = lane < 8 ? (uint32_t)mine : (uint32_t)(mine >> 32);
        }
    }
    int acc = 0;
#pragma unroll
    for (int c = 0; c < kMaxLc; ++c) {
        const int e = 16 * (lane + 64 * c);
        if (e < K) {
            const int4 q = *reinterpret_cast<const int4 *>(sq + e);
            acc = __builtin_amdgcn_sdot4(lw[c].x, q.x, acc, false);
            acc = __builtin_amdgcn_sdot4(lw[c].y, q.y, acc, false);
            acc = __builtin_amdgcn_sdot4(lw[c].z, q.z, acc, false);
            acc = __builtin_amdgcn_sdot4(lw[c].w, q.w, acc, false);
        }
    }
    acc = dpp_wave_isum(acc);
    if (has_row && lane == 0) a.t[(int64_t)b * a.rank + j] = acc;
}

struct DfwGemvArgs {
    const uint8_t *planes;      // [5][n_out][K/8]
    const uint16_t *row_scale;  // [n_out] fp16
    const float *dn_scale;      // [rank]
    const int8_t *lora_up;      // [n_out][rank]
    const float *up_scale;      // [n_out]
    int n_out, K, rank, batch;
    int lpr;                    // lanes per row: a power of two <= min(64, K/128)
    const uint32_t *qpl;        // [batch][8][K/32]
    const float *s;             // [batch]
    const int32_t *qsum;        // [batch]
    const int32_t *t;           // [batch][rank]
    float *y;                   // [batch][n_out]
    int32_t *acc_tap;           // [batch][n_out] or null
};

__device__ __forceinline__ uint32_t u4_at(const uint4 &v, int j) { return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w; }

// Sum over groups of w consecutive lanes; the total lands in the group's last lane.
__device__ __forceinline__ int group_isum(int v, int w) { return dpp_group_sum(v, w); }

// grid: (row blocks of kDfwWaves * 64 / lpr rows, token groups of NB)
template <int NB>
__global__ __launch_bounds__(kDfwBlock) void k_dfw_gemv(DfwGemvArgs a) {
    extern __shared__ __align__(16) uint32_t lds[];   // qpl[NB][8][K/32], then v[NB][rank] (fp32)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = a.K, G32 = K >> 5, chunks = K >> 7, lpr = a.lpr;
    const int b0 = blockIdx.y * NB, nb = min(NB, a.batch - b0);
    const int rpw = 64 / lpr;
    const int rin = lane / lpr, lir = lane & (lpr - 1);
    const int n = (blockIdx.x * kDfwWaves + wave) * rpw + rin;
    const bool valid = n < a.n_out;
    const int64_t pstride = (int64_t)a.n_out * (K >> 3);
    const uint8_t *row = a.planes + (int64_t)(valid ? n : 0) * (K >> 3);
    // the first chunk's planes are requested before anything else (they do not depend on the tokens)
    uint4 w[kDfwPlanes];
#pragma unroll
    for (int pb = 0; pb < kDfwPlanes; ++pb)
        w[pb] = valid && lir < chunks ? *reinterpret_cast<const uint4 *>(row + pb * pstride + 16 * lir) : make_uint4(0, 0, 0, 0);

    uint32_t *qpl = lds;
    float *vlo = reinterpret_cast<float *>(lds + NB * 8 * G32);
    for (int i = tid; i < nb * 8 * G32; i += kDfwBlock) qpl[i] = a.qpl[(int64_t)b0 * 8 * G32 + i];
    for (int i = tid; i < NB * 8 * G32; i += kDfwBlock)
        if (i >= nb * 8 * G32) qpl[i] = 0u;
    for (int i = tid; i < NB * a.rank; i += kDfwBlock) {
        const int bb = i / a.rank, j = i - bb * a.rank;
        vlo[i] = bb < nb ? a.dn_scale[j] * a.s[b0 + bb] * (float)a.t[(int64_t)(b0 + bb) * a.rank + j] : 0.f;
    }
    __syncthreads();

    int accp[NB][8];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
        for (int p = 0; p < 8; ++p) accp[bb][p] = 0;
    for (int c = lir; c < chunks; c += lpr) {
        if (c != lir) {
#pragma unroll
            for (int pb = 0; pb < kDfwPlanes; ++pb)
                w[pb] = valid ? *reinterpret_cast<const uint4 *>(row + pb * pstride + 16 * c) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const uint4 x = *reinterpret_cast<const uint4 *>(qpl + (bb * 8 + p) * G32 + 4 * c);
                int cb[kDfwPlanes];
#pragma unroll
                for (int pb = 0; pb < kDfwPlanes; ++pb) {
                    int v = 0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) v += __builtin_popcount(u4_at(w[pb], j) & u4_at(x, j));
                    cb[pb] = v;
                }
                accp[bb][p] += cb[0] + 2 * cb[1] + 4 * cb[2] + 8 * cb[3] + 16 * cb[4];
            }
        }
    }
    // epilogue: lanes of the row reduce; its last lane writes
    const float sc = valid ? half_bits_to_float(a.row_scale[n]) : 0.f;
    const float us = valid ? a.up_scale[n] : 0.f;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
        int acc = accp[bb][0] + 2 * accp[bb][1] + 4 * accp[bb][2] + 8 * accp[bb][3] + 16 * accp[bb][4] +
                  32 * accp[bb][5] + 64 * accp[bb][6] - 128 * accp[bb][7];
        acc = group_isum(acc, lpr);
        float lo = 0.f;
        for (int j = lir; j < a.rank; j += lpr)
            lo += (valid ? (float)a.lora_up[(int64_t)n * a.rank + j] : 0.f) * vlo[bb * a.rank + j];
        lo = dpp_group_sum_f(lo, lpr);
        if (valid && lir == lpr - 1 && bb < nb) {
            const int b = b0 + bb;
            acc -= 8 * a.qsum[b];
            a.y[(int64_t)b * a.n_out + n] = a.s[b] * sc * (float)acc * 0.125f + us * lo;
            if (a.acc_tap) a.acc_tap[(int64_t)b * a.n_out + n] = acc;
        }
    }
}

constexpr size_t kDfwAlign = 256;
size_t dfw_round(size_t v) { return (v + kDfwAlign - 1) / kDfwAlign * kDfwAlign; }

}  // namespace

// Workspace: codes q [batch][K] i8, their bit planes [batch][8][K/32] u32 (K bytes per token),
// s [batch], sum(q) [batch], t [batch][rank].
size_t dfw_ws_bytes(int K, int rank, int batch) {
    return dfw_round((size_t)batch * K) + dfw_round((size_t)batch * K) + dfw_round((size_t)batch * 4) +
           dfw_round((size_t)batch * 4) + dfw_round((size_t)batch * rank * 4);
}

hipError_t launch_dfw_project(const DfwWeights &w, int n_out, int K, int rank, const float *x, float *y, int batch,
                              void *ws, const DfwTaps &taps, hipStream_t stream) {
    char *p = static_cast<char *>(ws);
    int8_t *q = reinterpret_cast<int8_t *>(p);
    p += dfw_round((size_t)batch * K);
    uint32_t *qpl = reinterpret_cast<uint32_t *>(p);
    p += dfw_round((size_t)batch * K);
    float *s = reinterpret_cast<float *>(p);
    p += dfw_round((size_t)batch * 4);
    int32_t *qsum = reinterpret_cast<int32_t *>(p);
    p += dfw_round((size_t)batch * 4);
    int32_t *t = reinterpret_cast<int32_t *>(p);

    DfwQuantArgs qa{x, K, rank, w.lora_dn, q, qpl, s, qsum, t};
    k_dfw_quant<<<dim3((unsigned)batch, (unsigned)((rank + kWaves - 1) / kWaves)), kBlock, (size_t)K, stream>>>(qa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    int lpr = 1;
    while (lpr * 2 <= (K >> 7) && lpr < 64) lpr *= 2;
    DfwGemvArgs ga{w.planes, w.row_scale, w.lora_dn_scale, w.lora_up, w.lora_up_scale, n_out, K, rank, batch, lpr,
                   qpl, s, qsum, t, y, taps.acc};
    const int rows_per_wg = kDfwWaves * (64 / lpr);
    const unsigned gx = (unsigned)((n_out + rows_per_wg - 1) / rows_per_wg);
    const int NB = batch >= 4 ? 4 : batch >= 2 ? 2 : 1;
    const dim3 grid(gx, (unsigned)((batch + NB - 1) / NB));
    const size_t lds = ((size_t)NB * 8 * (K >> 5) + (size_t)NB * rank) * 4;
    if (NB == 4) k_dfw_gemv<4><<<grid, kDfwBlock, lds, stream>>>(ga);
    else if (NB == 2) k_dfw_gemv<2><<<grid, kDfwBlock, lds, stream>>>(ga);
    else k_dfw_gemv<1><<<grid, kDfwBlock, lds, stream>>>(ga);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // taps: the codes, scales and LoRA-down sums are in the workspace; copy them out on request
    if (taps.q) e = hipMemcpyAsync(taps.q, q, (size_t)batch * K, hipMemcpyDeviceToDevice, stream);
    if (e == hipSuccess && taps.s) e = hipMemcpyAsync(taps.s, s, (size_t)batch * 4, hipMemcpyDeviceToDevice, stream);
    if (e == hipSuccess && taps.t)
        e = hipMemcpyAsync(taps.t, t, (size_t)batch * rank * 4, hipMemcpyDeviceToDevice, stream);
    return e;
}

}  // namespace dfssm
