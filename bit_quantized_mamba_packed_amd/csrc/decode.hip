// DF-SSM decode-step kernels for gfx950 (one token per sequence per call).
//
// Per layer and token group the step runs as five kernels:
//   1. k_quant_gemv (in):  RMSNorm + per-token int8 quantizer in every workgroup (prologue),
//                          then the packed-sign GEMV over the in_proj rows and the int8 LoRA-down
//                          rows (DF-SSM paper §4.1 scaffold matmul, §3.3 int8 LoRA)
//   2. k_epi_conv:         rescale + LoRA-up epilogue (Eq. (3)) of every in_proj row, then the
//                          causal conv step + SiLU on x|B|C and softplus on dt
//   3. k_ssm:              selective-state update and readout per (head, row block), gated by
//                          SiLU(z) (paper App. B Table 12: dt-scaled input, gate before the norm)
//   4. k_quant_gemv (out): gated RMSNorm + quantizer prologue, GEMV over out_proj rows + LoRA-down
//   5. k_epi_residual:     rescale + LoRA-up epilogue of out_proj, residual add
//
// The packed-sign GEMV never expands weights to int8: with the activation codes split into
// bit-planes, sum_k sgn_k q_k = 2*sum_{bit_k=1} q_k - sum_k q_k and
// sum_{bit=1} q = sum_p c_p * popcount(bits & plane_p), c_p = 2^p (p < 7), c_7 = -128,
// i.e. one AND and one accumulating popcount per 32 weights per plane.
#include "dfssm_internal.h"

namespace dfssm {

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}
__device__ __forceinline__ int wave_isum(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Block-wide reductions with a fixed combination order, so every workgroup that reduces the
// same data obtains bit-identical results. `red` is >= kWaves floats of LDS.
__device__ __forceinline__ float block_sum(float v, float *red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float r = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return r;
}
__device__ __forceinline__ float block_max(float v, float *red) {
    v = wave_max(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return r;
}
__device__ __forceinline__ int block_isum(int v, int *red) {
    v = wave_isum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    int r = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return r;
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ float silu_f(float v) { return v / (1.0f + expf(-v)); }
__device__ __forceinline__ float softplus_f(float v) { return v > 20.0f ? v : log1pf(expf(v)); }

// int8 code of one value: clamp(rint_half_even(u * inv), -127, 127)
__device__ __forceinline__ int quant1(float u, float inv) {
    float r = rintf(u * inv);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

struct QuantGemvArgs {
    const float *X;       // [batch][x_stride] input vectors (K used)
    int64_t x_stride;
    const float *W;       // [K] norm weight
    int K;
    float eps;
    const uint8_t *sign;  // [n_out][K/8]
    int n_out;
    int rows_per_wg;
    int n_row_wgs;
    const int8_t *lora_dn;  // [rank][K]
    int rank;
    int32_t *acc;         // [batch][n_out]
    int32_t *t;           // [batch][rank]
    float *s;             // [batch]
    // taps, record-major [batch][...]; null when absent
    float *tap_h, *tap_u, *tap_s;
    int8_t *tap_q;
    int32_t *tap_acc, *tap_t;
};

// RMSNorm + quantizer of NB input vectors into LDS: codes sq[NB][K] and bit-planes
// spl[NB][8][K/32] (word g of plane p holds bit p of codes 32g..32g+31), sum of codes sqsum[NB].
template <int NB>
__device__ void norm_quant_prologue(const QuantGemvArgs &a, int8_t *sq, uint32_t *spl, int *sqsum,
                                    float *red, int *ired) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = a.K;
    const bool tap_wg = blockIdx.x == 0;
    for (int b = 0; b < NB; ++b) {
        const float *x = a.X + (int64_t)b * a.x_stride;
        float4 hv[kMaxK / 1024];
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < kMaxK / 1024; ++i) {
            const int e = (i * kBlock + tid) * 4;
            if (e < K) {
                hv[i] = *reinterpret_cast<const float4 *>(x + e);
                ss += hv[i].x * hv[i].x + hv[i].y * hv[i].y + hv[i].z * hv[i].z + hv[i].w * hv[i].w;
            }
        }
        const float tot = block_sum(ss, red);
        const float r = 1.0f / sqrtf(tot / (float)K + a.eps);
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < kMaxK / 1024; ++i) {
            const int e = (i * kBlock + tid) * 4;
            if (e < K) {
                const float4 w = *reinterpret_cast<const float4 *>(a.W + e);
                float4 u;
                u.x = (hv[i].x * r) * w.x;
                u.y = (hv[i].y * r) * w.y;
                u.z = (hv[i].z * r) * w.z;
                u.w = (hv[i].w * r) * w.w;
                hv[i] = u;
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(u.x), fabsf(u.y)), fmaxf(fabsf(u.z), fabsf(u.w))));
            }
        }
        amax = block_max(amax, red);
        const float inv = amax > 0.f ? 127.0f / amax : 0.f;
        const float s = amax > 0.f ? amax / 127.0f : 0.f;
        int qs = 0;
#pragma unroll
        for (int i = 0; i < kMaxK / 1024; ++i) {
            const int e = (i * kBlock + tid) * 4;
            if (e < K) {
                const int q0 = quant1(hv[i].x, inv), q1 = quant1(hv[i].y, inv);
                const int q2 = quant1(hv[i].z, inv), q3 = quant1(hv[i].w, inv);
                qs += q0 + q1 + q2 + q3;
                const uint32_t packed = (uint32_t)(q0 & 255) | ((uint32_t)(q1 & 255) << 8) |
                                        ((uint32_t)(q2 & 255) << 16) | ((uint32_t)(q3 & 255) << 24);
                *reinterpret_cast<uint32_t *>(sq + b * K + e) = packed;
                if (tap_wg) {
                    if (a.tap_u) *reinterpret_cast<float4 *>(a.tap_u + (int64_t)b * K + e) = hv[i];
                    if (a.tap_q) *reinterpret_cast<uint32_t *>(a.tap_q + (int64_t)b * K + e) = packed;
                    if (a.tap_h)
                        *reinterpret_cast<float4 *>(a.tap_h + (int64_t)b * K + e) =
                            *reinterpret_cast<const float4 *>(x + e);
                }
            }
        }
        qs = block_isum(qs, ired);
        if (tid == 0) {
            sqsum[b] = qs;
            if (tap_wg) {
                a.s[b] = s;
                if (a.tap_s) a.tap_s[b] = s;
            }
        }
    }
    __syncthreads();
    // bit-planes via wave ballots over 64 consecutive codes
    const int G32 = K >> 5;
    for (int b = 0; b < NB; ++b) {
        for (int c = wave; c < (K >> 6); c += kWaves) {
            const uint32_t v = (uint8_t)sq[b * K + c * 64 + lane];
            uint64_t mine = 0;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const uint64_t m = __ballot((v >> p) & 1u);
                if ((lane & 7) == p) mine = m;
            }
            if (lane < 16) {
                const int p = lane & 7;
                const uint32_t word = lane < 8 ? (uint32_t)mine : (uint32_t)(mine >> 32);
                spl[(b * 8 + p) * G32 + 2 * c + (lane >> 3)] = word;
            }
        }
    }
    __syncthreads();
}

template <int NB>
__device__ void gemv_rows(const QuantGemvArgs &a, int row_begin, int row_end, const uint32_t *spl,
                          const int *sqsum) {
    const int K = a.K, chunks = K >> 7, G32 = K >> 5;
    int lpr = 1;
    while (lpr * 2 <= chunks && lpr < 64) lpr *= 2;  // lanes per row: power of two
    const int rpw = 64 / lpr;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rin = lane / lpr, lir = lane & (lpr - 1);
    for (int n0 = row_begin + wave * rpw; n0 < row_end; n0 += kWaves * rpw) {
        const int n = n0 + rin;
        const bool valid = n < row_end;
        uint32_t cnt[NB][8];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int p = 0; p < 8; ++p) cnt[b][p] = 0;
        const uint4 *row = reinterpret_cast<const uint4 *>(a.sign + (int64_t)(valid ? n : row_begin) * (K >> 3));
        for (int c = lir; c < chunks; c += lpr) {
            const uint4 bits = valid ? row[c] : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
#pragma unroll
                for (int p = 0; p < 8; ++p) {
                    const uint4 pl = *reinterpret_cast<const uint4 *>(spl + (b * 8 + p) * G32 + c * 4);
                    cnt[b][p] = __popc(bits.x & pl.x) + __popc(bits.y & pl.y) + __popc(bits.z & pl.z) +
                                __popc(bits.w & pl.w) + cnt[b][p];
                }
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            int pos = 0;
#pragma unroll
            for (int p = 0; p < 7; ++p) pos += (int)cnt[b][p] << p;
            pos -= (int)cnt[b][7] << 7;
            for (int m = lpr >> 1; m >= 1; m >>= 1) pos += __shfl_xor(pos, m, 64);
            if (lir == 0 && valid) {
                const int accv = 2 * pos - sqsum[b];
                a.acc[(int64_t)b * a.n_out + n] = accv;
                if (a.tap_acc) a.tap_acc[(int64_t)b * a.n_out + n] = accv;
            }
        }
    }
}

template <int NB>
__device__ void lora_dn_rows(const QuantGemvArgs &a, int j_begin, int j_end, const int8_t *sq) {
    const int K = a.K;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int j = j_begin + wave; j < j_end; j += kWaves) {
        int sacc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) sacc[b] = 0;
        const int8_t *row = a.lora_dn + (int64_t)j * K;
        for (int off = lane * 16; off < K; off += 1024) {
            const int4 lw = *reinterpret_cast<const int4 *>(row + off);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int4 qv = *reinterpret_cast<const int4 *>(sq + b * K + off);
                int v = sacc[b];
                v = __builtin_amdgcn_sdot4(lw.x, qv.x, v, false);
                v = __builtin_amdgcn_sdot4(lw.y, qv.y, v, false);
                v = __builtin_amdgcn_sdot4(lw.z, qv.z, v, false);
                v = __builtin_amdgcn_sdot4(lw.w, qv.w, v, false);
                sacc[b] = v;
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int tv = wave_isum(sacc[b]);
            if (lane == 0) {
                a.t[b * a.rank + j] = tv;
                if (a.tap_t) a.tap_t[(int64_t)b * a.rank + j] = tv;
            }
        }
    }
}

template <int NB>
__global__ __launch_bounds__(kBlock) void k_quant_gemv(QuantGemvArgs a) {
    extern __shared__ __align__(16) char smem[];
    __shared__ float red[kWaves];
    __shared__ int ired[kWaves];
    __shared__ int sqsum[NB];
    int8_t *sq = reinterpret_cast<int8_t *>(smem);
    uint32_t *spl = reinterpret_cast<uint32_t *>(smem + NB * a.K);
    norm_quant_prologue<NB>(a, sq, spl, sqsum, red, ired);
    if ((int)blockIdx.x < a.n_row_wgs) {
        const int r0 = blockIdx.x * a.rows_per_wg;
        gemv_rows<NB>(a, r0, min(r0 + a.rows_per_wg, a.n_out), spl, sqsum);
    } else {
        const int j0 = (blockIdx.x - a.n_row_wgs) * kWaves;
        lora_dn_rows<NB>(a, j0, min(j0 + kWaves, a.rank), sq);
    }
}

// ---------------------------------------------------------------- rescale + LoRA-up epilogue
struct EpiCommon {
    const int32_t *acc;     // [batch][n_out]
    const int32_t *t;       // [batch][rank]
    const float *s;         // [batch]
    int n_out, rank;
    const uint16_t *row_scale;
    const int8_t *lora_up;  // [n_out][rank]
    const float *up_scale, *dn_scale;
};

// v[j] = dn_scale[j] * s * t[j] into LDS (rank <= 64); returns s.
__device__ __forceinline__ float epi_prepare(const EpiCommon &c, int b, float *v) {
    const float s = c.s[b];
    if ((int)threadIdx.x < c.rank) v[threadIdx.x] = c.dn_scale[threadIdx.x] * s * (float)c.t[b * c.rank + threadIdx.x];
    __syncthreads();
    return s;
}

// y[n] = s*row_scale[n]*acc[n] + up_scale[n] * sum_j lora_up[n,j] * v[j]
__device__ __forceinline__ float epi_row(const EpiCommon &c, int b, int n, float s, const float *v) {
    const int8_t *up = c.lora_up + (int64_t)n * c.rank;
    float lr = 0.f;
    if ((c.rank & 15) == 0) {
        for (int j = 0; j < c.rank; j += 16) {
            const int4 w4 = *reinterpret_cast<const int4 *>(up + j);
            const int ws[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int k = 0; k < 4; ++k) lr += (float)(int8_t)(ws[i] >> (8 * k)) * v[j + 4 * i + k];
        }
    } else {
        for (int j = 0; j < c.rank; ++j) lr += (float)up[j] * v[j];
    }
    const float acc = (float)c.acc[(int64_t)b * c.n_out + n];
    return s * half_bits_to_float(c.row_scale[n]) * acc + c.up_scale[n] * lr;
}

struct EpiConvArgs {
    EpiCommon c;
    int E, Cd, H;
    const float *conv_w, *conv_b, *dt_bias;
    float *conv_state;  // [batch][Cd][3]
    float *zbuf, *xbc, *dtbuf;
};

__global__ __launch_bounds__(kBlock) void k_epi_conv(EpiConvArgs a) {
    __shared__ float v[kMaxRank];
    const int b = blockIdx.y;
    const float s = epi_prepare(a.c, b, v);
    const int n = blockIdx.x * kBlock + threadIdx.x;
    if (n >= a.E + a.Cd + a.H) return;
    const float y = epi_row(a.c, b, n, s, v);
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

struct EpiResArgs {
    EpiCommon c;
    const float *h_in;
    float *h_out;       // may alias h_in (same element read then written by one thread)
};

__global__ __launch_bounds__(kBlock) void k_epi_residual(EpiResArgs a) {
    __shared__ float v[kMaxRank];
    const int b = blockIdx.y;
    const float s = epi_prepare(a.c, b, v);
    const int n = blockIdx.x * kBlock + threadIdx.x;
    if (n >= a.c.n_out) return;
    const float y = epi_row(a.c, b, n, s, v);
    const int64_t i = (int64_t)b * a.c.n_out + n;
    a.h_out[i] = a.h_in[i] + y;
}

// ---------------------------------------------------------------- SSM step + gate
struct SsmArgs {
    const float *xbc, *zbuf, *dtbuf;
    float *ssm;          // [batch][H][P][N]
    const float *A_log, *D;
    float *gbuf;         // [batch][E]
    int E, H, P, N, G, Cd;
    int rows_per_wg;     // rows_per_wg * N is a multiple of 1024 (or covers the head)
};

__global__ __launch_bounds__(kBlock) void k_ssm(SsmArgs a) {
    const int b = blockIdx.y;
    const int wg_per_head = a.P / a.rows_per_wg;
    const int h = blockIdx.x / wg_per_head;
    const int p0 = (blockIdx.x % wg_per_head) * a.rows_per_wg;
    const float dt = a.dtbuf[(int64_t)b * a.H + h];
    const float dA = expf(dt * -expf(a.A_log[h]));
    const float Dh = a.D[h];
    const int g = h * a.G / a.H;
    const float *xrow = a.xbc + (int64_t)b * a.Cd;
    const float *Bv = xrow + a.E + g * a.N;
    const float *Cv = xrow + a.E + a.G * a.N + g * a.N;
    const int n4 = a.N >> 2;
    const int nchunks = a.rows_per_wg * n4;
    for (int ci = threadIdx.x; ci < nchunks; ci += kBlock) {
        const int pr = ci / n4, c4 = ci - pr * n4;
        const int p = p0 + pr;
        const float x = xrow[h * a.P + p];
        const float dtx = dt * x;
        float4 *sp = reinterpret_cast<float4 *>(a.ssm + (((int64_t)b * a.H + h) * a.P + p) * a.N) + c4;
        float4 S = *sp;
        const float4 Bn = reinterpret_cast<const float4 *>(Bv)[c4];
        const float4 Cn = reinterpret_cast<const float4 *>(Cv)[c4];
        S.x = dA * S.x + dtx * Bn.x;
        S.y = dA * S.y + dtx * Bn.y;
        S.z = dA * S.z + dtx * Bn.z;
        S.w = dA * S.w + dtx * Bn.w;
        *sp = S;
        float part = (S.x * Cn.x + S.y * Cn.y) + (S.z * Cn.z + S.w * Cn.w);
        for (int m = n4 >> 1; m >= 1; m >>= 1) part += __shfl_xor(part, m, 64);
        if (c4 == 0) {
            const float y = part + Dh * x;
            const float z = a.zbuf[(int64_t)b * a.E + h * a.P + p];
            a.gbuf[(int64_t)b * a.E + h * a.P + p] = y * silu_f(z);
        }
    }
}

// ---------------------------------------------------------------- final RMSNorm of the stack
__global__ __launch_bounds__(kBlock) void k_final_norm(const float *h, const float *w, float *y, float *y2,
                                                       int D, float eps) {
    __shared__ float red[kWaves];
    const int b = blockIdx.x;
    const float *hb = h + (int64_t)b * D;
    float ss = 0.f;
    for (int e = threadIdx.x; e < D; e += kBlock) ss += hb[e] * hb[e];
    const float tot = block_sum(ss, red);
    const float r = 1.0f / sqrtf(tot / (float)D + eps);
    for (int e = threadIdx.x; e < D; e += kBlock) {
        const float v = (hb[e] * r) * w[e];
        y[(int64_t)b * D + e] = v;
        if (y2) y2[(int64_t)b * D + e] = v;
    }
}

template <int NB>
hipError_t launch_qg(const QuantGemvArgs &a, int n_lora_wgs, hipStream_t stream) {
    const size_t lds = (size_t)NB * a.K * 2;
    k_quant_gemv<NB><<<a.n_row_wgs + n_lora_wgs, kBlock, lds, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_quant_gemv(QuantGemvArgs a, int nb, hipStream_t stream) {
    const int chunks = a.K >> 7;
    int lpr = 1;
    while (lpr * 2 <= chunks && lpr < 64) lpr *= 2;
    a.rows_per_wg = kWaves * (64 / lpr);
    a.n_row_wgs = (a.n_out + a.rows_per_wg - 1) / a.rows_per_wg;
    const int n_lora_wgs = (a.rank + kWaves - 1) / kWaves;
    switch (nb) {
        case 1: return launch_qg<1>(a, n_lora_wgs, stream);
        case 2: return launch_qg<2>(a, n_lora_wgs, stream);
        case 3: return launch_qg<3>(a, n_lora_wgs, stream);
        default: return launch_qg<4>(a, n_lora_wgs, stream);
    }
}

}  // namespace

hipError_t launch_layer_decode(const Shape &s, const dfssm_layer_weights &w, const dfssm_layer_state &st,
                               const float *x_in, float *x_out, int batch, const DecodeWs &ws,
                               const TapPtrs &tp, hipStream_t stream) {
    hipError_t e;
    // 1. in-proj: groups of up to kGemvMaxBatch tokens share one pass over the packed weights
    //    (LDS holds 2*K bytes per token of the group: codes + bit-planes)
    const int grp_in = min(kGemvMaxBatch, kGemvLdsBytes / (2 * s.D));
    const int grp_out = min(kGemvMaxBatch, kGemvLdsBytes / (2 * s.E));
    for (int b0 = 0; b0 < batch; b0 += grp_in) {
        const int nb = min(grp_in, batch - b0);
        QuantGemvArgs a{};
        a.X = x_in + (int64_t)b0 * s.D;
        a.x_stride = s.D;
        a.W = w.norm_w;
        a.K = s.D;
        a.eps = s.eps;
        a.sign = w.in_proj.sign;
        a.n_out = s.Ninp;
        a.lora_dn = w.in_proj.lora_dn;
        a.rank = s.Rin;
        a.acc = ws.acc_in + (int64_t)b0 * s.Ninp;
        a.t = ws.t_in + (int64_t)b0 * s.Rin;
        a.s = ws.s_in + b0;
        a.tap_h = tp.h_in ? tp.h_in + (int64_t)b0 * s.D : nullptr;
        a.tap_u = tp.in_u ? tp.in_u + (int64_t)b0 * s.D : nullptr;
        a.tap_q = tp.in_q ? tp.in_q + (int64_t)b0 * s.D : nullptr;
        a.tap_s = tp.in_s ? tp.in_s + b0 : nullptr;
        a.tap_acc = tp.in_acc ? tp.in_acc + (int64_t)b0 * s.Ninp : nullptr;
        a.tap_t = tp.in_t ? tp.in_t + (int64_t)b0 * s.Rin : nullptr;
        if ((e = launch_quant_gemv(a, nb, stream)) != hipSuccess) return e;
    }
    // 2. epilogue + conv + dt
    {
        EpiConvArgs a{};
        a.c = EpiCommon{ws.acc_in, ws.t_in, ws.s_in, s.Ninp, s.Rin, w.in_proj.row_scale, w.in_proj.lora_up,
                        w.in_proj.lora_up_scale, w.in_proj.lora_dn_scale};
        a.E = s.E;
        a.Cd = s.Cd;
        a.H = s.H;
        a.conv_w = w.conv_w;
        a.conv_b = w.conv_b;
        a.dt_bias = w.dt_bias;
        a.conv_state = st.conv;
        a.zbuf = ws.zbuf;
        a.xbc = ws.xbc;
        a.dtbuf = ws.dtbuf;
        dim3 grid((s.Nin + kBlock - 1) / kBlock, batch);
        k_epi_conv<<<grid, kBlock, 0, stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // 3. SSM step + gate
    {
        SsmArgs a{};
        a.xbc = ws.xbc;
        a.zbuf = ws.zbuf;
        a.dtbuf = ws.dtbuf;
        a.ssm = st.ssm;
        a.A_log = w.A_log;
        a.D = w.D;
        a.gbuf = ws.gbuf;
        a.E = s.E;
        a.H = s.H;
        a.P = s.P;
        a.N = s.N;
        a.G = s.G;
        a.Cd = s.Cd;
        a.rows_per_wg = min(s.P, 2048 / s.N);
        dim3 grid(s.H * (s.P / a.rows_per_wg), batch);
        k_ssm<<<grid, kBlock, 0, stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // 4. out-proj
    for (int b0 = 0; b0 < batch; b0 += grp_out) {
        const int nb = min(grp_out, batch - b0);
        QuantGemvArgs a{};
        a.X = ws.gbuf + (int64_t)b0 * s.E;
        a.x_stride = s.E;
        a.W = w.gnorm_w;
        a.K = s.E;
        a.eps = s.eps;
        a.sign = w.out_proj.sign;
        a.n_out = s.D;
        a.lora_dn = w.out_proj.lora_dn;
        a.rank = s.Rout;
        a.acc = ws.acc_out + (int64_t)b0 * s.D;
        a.t = ws.t_out + (int64_t)b0 * s.Rout;
        a.s = ws.s_out + b0;
        a.tap_u = tp.out_u ? tp.out_u + (int64_t)b0 * s.E : nullptr;
        a.tap_q = tp.out_q ? tp.out_q + (int64_t)b0 * s.E : nullptr;
        a.tap_s = tp.out_s ? tp.out_s + b0 : nullptr;
        a.tap_acc = tp.out_acc ? tp.out_acc + (int64_t)b0 * s.D : nullptr;
        a.tap_t = tp.out_t ? tp.out_t + (int64_t)b0 * s.Rout : nullptr;
        if ((e = launch_quant_gemv(a, nb, stream)) != hipSuccess) return e;
    }
    // 5. epilogue + residual
    {
        EpiResArgs a{};
        a.c = EpiCommon{ws.acc_out, ws.t_out, ws.s_out, s.D, s.Rout, w.out_proj.row_scale, w.out_proj.lora_up,
                        w.out_proj.lora_up_scale, w.out_proj.lora_dn_scale};
        a.h_in = x_in;
        a.h_out = x_out;
        dim3 grid((s.D + kBlock - 1) / kBlock, batch);
        k_epi_residual<<<grid, kBlock, 0, stream>>>(a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_final_norm(const float *h, const float *w, float *y, float *y2, int D, float eps, int batch,
                             hipStream_t stream) {
    k_final_norm<<<batch, kBlock, 0, stream>>>(h, w, y, y2, D, eps);
    return hipGetLastError();
}

}  // namespace dfssm
