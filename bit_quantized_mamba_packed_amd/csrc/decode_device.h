// Device-side building blocks of the DF-SSM decode step, shared by the per-layer kernels and
// the persistent stack kernel: deterministic reductions, the RMSNorm + int8 quantizer prologue,
// the packed-sign popcount GEMV, the int8 LoRA-down rows and the rescale + LoRA-up epilogue.
#pragma once

#include "dfssm_internal.h"

namespace dfssm {

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

// Sum over groups of w consecutive lanes (w a power of two <= 64) with DPP row operations; the
// group's total is valid in its last lane (lane % w == w - 1).
__device__ __forceinline__ int dpp_group_sum(int v, int w) {
    if (w >= 2) v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
    if (w >= 4) v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
    if (w >= 8) v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
    if (w >= 16) v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true); // row_shr:8
    if (w >= 32) v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false); // row_bcast:15 into rows 1, 3
    if (w >= 64) v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false); // row_bcast:31 into rows 2, 3
    return v;
}
template <int CTRL, int RMASK, bool BC>
__device__ __forceinline__ float dpp_add_f(float v) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, RMASK, 0xF, BC));
}
__device__ __forceinline__ float dpp_group_sum_f(float v, int w) {
    if (w >= 2) v = dpp_add_f<0xB1, 0xF, true>(v);
    if (w >= 4) v = dpp_add_f<0x4E, 0xF, true>(v);
    if (w >= 8) v = dpp_add_f<0x114, 0xF, true>(v);
    if (w >= 16) v = dpp_add_f<0x118, 0xF, true>(v);
    if (w >= 32) v = dpp_add_f<0x142, 0xA, false>(v);
    if (w >= 64) v = dpp_add_f<0x143, 0xC, false>(v);
    return v;
}

// Whole-wave sum / max by DPP (a few cycles per step, against a full LDS round trip per step for
// lane shuffles); the fixed order makes every workgroup reducing the same data agree bit for bit.
template <int CTRL, int RMASK, bool BC>
__device__ __forceinline__ float dpp_max_f(float v) {
    return fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, RMASK, 0xF, BC)));
}
__device__ __forceinline__ float dpp_wave_sum(float v) {
    v = dpp_group_sum_f(v, 64);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float dpp_wave_max(float v) {   // v >= 0 (lanes past a row edge read 0)
    v = dpp_max_f<0xB1, 0xF, true>(v);
    v = dpp_max_f<0x4E, 0xF, true>(v);
    v = dpp_max_f<0x114, 0xF, true>(v);
    v = dpp_max_f<0x118, 0xF, true>(v);
    v = dpp_max_f<0x142, 0xA, false>(v);
    v = dpp_max_f<0x143, 0xC, false>(v);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ int dpp_wave_isum(int v) { return __builtin_amdgcn_readlane(dpp_group_sum(v, 64), 63); }

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

// Sum of `v` and max of `m` over the block in one reduction round (fixed combination order).
__device__ __forceinline__ void block_sum_max(float v, float m, float *red, float &sum, float &mx) {
    v = wave_sum(v);
    m = wave_max(m);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        red[wave] = v;
        red[kWaves + wave] = m;
    }
    __syncthreads();
    sum = (red[0] + red[1]) + (red[2] + red[3]);
    mx = fmaxf(fmaxf(red[kWaves], red[kWaves + 1]), fmaxf(red[kWaves + 2], red[kWaves + 3]));
    __syncthreads();
}

// Accesses to values exchanged between workgroups inside one kernel (agent-scope coherent: the
// per-XCD L2 caches are not coherent with each other, and these bypass them). Weights and state
// that a single workgroup owns use plain loads and stores.
template <typename T>
__device__ __forceinline__ T ld_x(const T *p) {
    return __hip_atomic_load(const_cast<T *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st_x(T *p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float4 ld_x4(const float *p) {
    return make_float4(ld_x(p), ld_x(p + 1), ld_x(p + 2), ld_x(p + 3));
}

// 2*KCH coherent (sc1) 16-byte loads of a thread's 4*KCH consecutive tagged words, waited for
// inside the same asm block. Word 2j is (r[j].x payload, r[j].y epoch), word 2j+1 is (r[j].z, r[j].w).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <int KCH>
__device__ __forceinline__ void load_words_sc1(const uint64_t *p, u32x4 (&r)[2 * KCH]);
template <>
__device__ __forceinline__ void load_words_sc1<1>(const uint64_t *p, u32x4 (&r)[2]) {
    asm volatile("global_load_dwordx4 %0, %2, off sc1\n\t"
                 "global_load_dwordx4 %1, %2, off offset:16 sc1\n\t"
                 "s_waitcnt vmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1]) : "v"(p) : "memory");
}
template <>
__device__ __forceinline__ void load_words_sc1<2>(const uint64_t *p, u32x4 (&r)[4]) {
    asm volatile("global_load_dwordx4 %0, %4, off sc1\n\t"
                 "global_load_dwordx4 %1, %4, off offset:16 sc1\n\t"
                 "global_load_dwordx4 %2, %4, off offset:32 sc1\n\t"
                 "global_load_dwordx4 %3, %4, off offset:48 sc1\n\t"
                 "s_waitcnt vmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]) : "v"(p) : "memory");
}
template <>
__device__ __forceinline__ void load_words_sc1<4>(const uint64_t *p, u32x4 (&r)[8]) {
    asm volatile("global_load_dwordx4 %0, %8, off sc1\n\t"
                 "global_load_dwordx4 %1, %8, off offset:16 sc1\n\t"
                 "global_load_dwordx4 %2, %8, off offset:32 sc1\n\t"
                 "global_load_dwordx4 %3, %8, off offset:48 sc1\n\t"
                 "global_load_dwordx4 %4, %8, off offset:64 sc1\n\t"
                 "global_load_dwordx4 %5, %8, off offset:80 sc1\n\t"
                 "global_load_dwordx4 %6, %8, off offset:96 sc1\n\t"
                 "global_load_dwordx4 %7, %8, off offset:112 sc1\n\t"
                 "s_waitcnt vmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
                   "=&v"(r[7])
                 : "v"(p)
                 : "memory");
}
template <>
__device__ __forceinline__ void load_words_sc1<8>(const uint64_t *p, u32x4 (&r)[16]) {
    load_words_sc1<4>(p, *reinterpret_cast<u32x4(*)[8]>(&r[0]));
    load_words_sc1<4>(p + 16, *reinterpret_cast<u32x4(*)[8]>(&r[8]));
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

// Element of chunk i (4 consecutive inputs) a thread handles in the norm + quantizer prologue:
// each thread owns KCH chunks in a row, so its inputs are one contiguous run of 4*KCH values.
template <int KCH>
__device__ __forceinline__ int prologue_elem(int i) {
    return ((int)threadIdx.x * KCH + i) * 4;
}

struct QuantGemvArgs {
    const float *X;       // [batch][x_stride] input vectors (K used) for the per-layer kernels
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
    int32_t *acc;         // [batch][n_out]   (per-layer kernels)
    int32_t *t;           // [batch][rank]
    float *s;             // [batch]
    // optional normalisation applied to X before the prologue's own RMSNorm: X <- RMSNorm(X)*pre_w
    // (the stack's final norm folded into the next token's first layer); workgroup 0 stores the
    // normalised vectors to pre_out when it is non-null
    const float *pre_w;
    float *pre_out;
    // taps, record-major [batch][...]; null when absent
    float *tap_h, *tap_u, *tap_s;
    int8_t *tap_q;
    int32_t *tap_acc, *tap_t;
};

// Input of the prologue read from a plain fp32 array (KCH float4 chunks per thread).
template <int KCH>
struct PlainSource {
    const float *X;
    int64_t stride;
    __device__ __forceinline__ void load(int b, int K, float4 *hv) const {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int e = prologue_elem<KCH>(i);
            if (e < K) hv[i] = ld_x4(X + (int64_t)b * stride + e);
        }
    }
};

// Integer results written to plain int32 arrays.
struct PlainSink {
    int32_t *acc, *t;
    int n_out, rank;
    __device__ __forceinline__ void put_acc(int b, int n, int v) const { st_x(acc + (int64_t)b * n_out + n, v); }
    __device__ __forceinline__ void put_t(int b, int j, int v) const { st_x(t + b * rank + j, v); }
};

// RMSNorm + quantizer of NB input vectors into LDS: codes sq[NB][K] and bit-planes
// spl[NB][8][K/32] (word g of plane p holds bit p of codes 32g..32g+31), sum of codes sqsum[NB],
// scale ssc[NB]. When xsave is non-null the (pre-normalised) input is also kept there [NB][K].
// Each thread holds KCH chunks of 4 inputs (K <= 1024 * KCH).
template <int NB, int KCH, class Src>
__device__ void norm_quant_prologue(const QuantGemvArgs &a, const Src &src, int8_t *sq, uint32_t *spl,
                                    int *sqsum, float *ssc, float *red, int *ired, float *xsave) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = a.K;
    const bool tap_wg = blockIdx.x == 0;
    for (int b = 0; b < NB; ++b) {
        float4 hv[KCH];
        src.load(b, K, hv);
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int e = prologue_elem<KCH>(i);
            if (e < K) ss += hv[i].x * hv[i].x + hv[i].y * hv[i].y + hv[i].z * hv[i].z + hv[i].w * hv[i].w;
        }
        if (a.pre_w) {
            const float tot0 = block_sum(ss, red);
            const float r0 = 1.0f / sqrtf(tot0 / (float)K + a.eps);
            ss = 0.f;
#pragma unroll
            for (int i = 0; i < KCH; ++i) {
                const int e = prologue_elem<KCH>(i);
                if (e < K) {
                    const float4 w = *reinterpret_cast<const float4 *>(a.pre_w + e);
                    hv[i].x = (hv[i].x * r0) * w.x;
                    hv[i].y = (hv[i].y * r0) * w.y;
                    hv[i].z = (hv[i].z * r0) * w.z;
                    hv[i].w = (hv[i].w * r0) * w.w;
                    ss += hv[i].x * hv[i].x + hv[i].y * hv[i].y + hv[i].z * hv[i].z + hv[i].w * hv[i].w;
                    if (tap_wg && a.pre_out) *reinterpret_cast<float4 *>(a.pre_out + (int64_t)b * K + e) = hv[i];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int e = prologue_elem<KCH>(i);
            if (e < K) {
                if (tap_wg && a.tap_h) *reinterpret_cast<float4 *>(a.tap_h + (int64_t)b * K + e) = hv[i];
                if (xsave) *reinterpret_cast<float4 *>(xsave + b * K + e) = hv[i];
            }
        }
        // u = fl(fl(h * w) * r): with r > 0 the largest |u| is fl(max|h * w| * r) exactly, so the
        // sum of squares and max|h * w| share one reduction
        float pm = 0.f;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int e = prologue_elem<KCH>(i);
            if (e < K) {
                const float4 w = *reinterpret_cast<const float4 *>(a.W + e);
                hv[i].x = hv[i].x * w.x;
                hv[i].y = hv[i].y * w.y;
                hv[i].z = hv[i].z * w.z;
                hv[i].w = hv[i].w * w.w;
                pm = fmaxf(pm, fmaxf(fmaxf(fabsf(hv[i].x), fabsf(hv[i].y)), fmaxf(fabsf(hv[i].z), fabsf(hv[i].w))));
            }
        }
        float tot;
        block_sum_max(ss, pm, red, tot, pm);
        const float r = 1.0f / sqrtf(tot / (float)K + a.eps);
        const float amax = pm * r;
        const float inv = amax > 0.f ? 127.0f / amax : 0.f;
        const float s = amax > 0.f ? amax / 127.0f : 0.f;
        int qs = 0;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int e = prologue_elem<KCH>(i);
            if (e < K) {
                hv[i].x = hv[i].x * r;
                hv[i].y = hv[i].y * r;
                hv[i].z = hv[i].z * r;
                hv[i].w = hv[i].w * r;
                const int q0 = quant1(hv[i].x, inv), q1 = quant1(hv[i].y, inv);
                const int q2 = quant1(hv[i].z, inv), q3 = quant1(hv[i].w, inv);
                qs += q0 + q1 + q2 + q3;
                const uint32_t packed = (uint32_t)(q0 & 255) | ((uint32_t)(q1 & 255) << 8) |
                                        ((uint32_t)(q2 & 255) << 16) | ((uint32_t)(q3 & 255) << 24);
                *reinterpret_cast<uint32_t *>(sq + b * K + e) = packed;
                if (tap_wg) {
                    if (a.tap_u) *reinterpret_cast<float4 *>(a.tap_u + (int64_t)b * K + e) = hv[i];
                    if (a.tap_q) *reinterpret_cast<uint32_t *>(a.tap_q + (int64_t)b * K + e) = packed;
                }
            }
        }
        qs = block_isum(qs, ired);
        if (tid == 0) {
            sqsum[b] = qs;
            ssc[b] = s;
            if (tap_wg) {
                if (a.s) st_x(a.s + b, s);
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

// Lanes per row of the packed-sign GEMV for K inputs (one 16-byte chunk = 128 weights per lane
// per step; a power of two, at most a wave).
__device__ __host__ __forceinline__ int gemv_lanes_per_row(int K) {
    const int chunks = K >> 7;
    int lpr = 1;
    while (lpr * 2 <= chunks && lpr < 64) lpr *= 2;
    return lpr;
}

// Up to kGemvPre 16-byte sign chunks a lane loads ahead of the GEMV (in the order gemv_rows
// consumes them), so that their HBM latency overlaps whatever the workgroup waits for first.
constexpr int kGemvPre = 2;
struct GemvPre {
    uint4 c[kGemvPre];
};
__device__ __forceinline__ void gemv_prefetch(GemvPre &pre, const uint8_t *sign, int K, int row_begin, int row_end) {
    static_assert(kGemvPre == 2, "gemv_prefetch fills two chunks");
    const int chunks = K >> 7;
    const int lpr = gemv_lanes_per_row(K);
    const int rpw = 64 / lpr;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rin = lane / lpr, lir = lane & (lpr - 1);
    // first chunk: first row pass, chunk lir; second: the next chunk of that row if the lane has
    // one, else chunk lir of the next row pass (the order gemv_rows walks them)
    const int n0 = row_begin + wave * rpw + rin;
    const bool same_row = lir + lpr < chunks;
    const int n1 = same_row ? n0 : n0 + kWaves * rpw;
    const int c1 = same_row ? lir + lpr : lir;
    const int64_t stride = K >> 3;
    const bool v0 = row_begin + wave * rpw < row_end && n0 < row_end;
    const bool v1 = (same_row ? row_begin + wave * rpw : row_begin + wave * rpw + kWaves * rpw) < row_end && n1 < row_end;
    pre.c[0] = v0 ? reinterpret_cast<const uint4 *>(sign + (int64_t)n0 * stride)[lir] : make_uint4(0, 0, 0, 0);
    pre.c[1] = v1 ? reinterpret_cast<const uint4 *>(sign + (int64_t)n1 * stride)[c1] : make_uint4(0, 0, 0, 0);
}

// Packed-sign GEMV over rows [row_begin, row_end): acc[b][n] = sum_k sgn[n,k] q_b[k].
// When use_pre is set the chunks of `pre` (from gemv_prefetch over the same rows) are used first.
template <int NB, class Sink>
__device__ __forceinline__ void gemv_rows(const QuantGemvArgs &a, const Sink &sink, int row_begin, int row_end,
                                          const uint32_t *spl, const int *sqsum, const GemvPre pre, bool use_pre) {
    const int K = a.K, chunks = K >> 7, G32 = K >> 5;
    const int lpr = gemv_lanes_per_row(K);
    const int rpw = 64 / lpr;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rin = lane / lpr, lir = lane & (lpr - 1);
    int k = use_pre ? 0 : kGemvPre;
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
            uint4 bits;
            if (k < kGemvPre) {
                bits = k == 0 ? pre.c[0] : pre.c[1];
                ++k;
            } else {
                bits = valid ? row[c] : make_uint4(0, 0, 0, 0);
            }
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
                sink.put_acc(b, n, accv);
                if (a.tap_acc) a.tap_acc[(int64_t)b * a.n_out + n] = accv;
            }
        }
    }
}

// int8 LoRA-down rows [j_begin, j_end): t[b][j] = sum_k L_dn[j,k] q_b[k] (sdot4).
template <int NB, class Sink>
__device__ void lora_dn_rows(const QuantGemvArgs &a, const Sink &sink, int j_begin, int j_end, const int8_t *sq) {
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
                sink.put_t(b, j, tv);
                if (a.tap_t) a.tap_t[(int64_t)b * a.rank + j] = tv;
            }
        }
    }
}

// ---------------------------------------------------------------- rescale + LoRA-up epilogue
// sum_j lora_up[n,j] * v[j] for one row (rank <= 64), v in LDS.
__device__ __forceinline__ float lowrank_row(const int8_t *lora_up, int rank, int n, const float *v) {
    const int8_t *up = lora_up + (int64_t)n * rank;
    float lr = 0.f;
    if ((rank & 15) == 0) {
        for (int j = 0; j < rank; j += 16) {
            const int4 w4 = *reinterpret_cast<const int4 *>(up + j);
            const int ws[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int k = 0; k < 4; ++k) lr += (float)(int8_t)(ws[i] >> (8 * k)) * v[j + 4 * i + k];
        }
    } else {
        for (int j = 0; j < rank; ++j) lr += (float)up[j] * v[j];
    }
    return lr;
}

// One projection output (paper Eq. (3)): s*row_scale*acc + up_scale * (low-rank sum).
__device__ __forceinline__ float epi_combine(float s, uint16_t row_scale_bits, int acc, float up_scale, float lr) {
    return s * half_bits_to_float(row_scale_bits) * (float)acc + up_scale * lr;
}

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
    const float s = ld_x(c.s + b);
    if ((int)threadIdx.x < c.rank) v[threadIdx.x] = c.dn_scale[threadIdx.x] * s * (float)ld_x(c.t + b * c.rank + threadIdx.x);
    __syncthreads();
    return s;
}

__device__ __forceinline__ float epi_row(const EpiCommon &c, int b, int n, float s, const float *v) {
    const float lr = lowrank_row(c.lora_up, c.rank, n, v);
    return epi_combine(s, c.row_scale[n], ld_x(c.acc + (int64_t)b * c.n_out + n), c.up_scale[n], lr);
}

}  // namespace dfssm
