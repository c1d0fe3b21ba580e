// int8-code x (+-1 scaffold) GEMM with the DF-SSM projection epilogue, on gfx950 MFMA.
//
// For M tokens at once (prefill, batched decode) a projection is a real dense contraction
// (DF-SSM paper §4.1 runs it on INT8 tensor cores). Here:
//   C[m][n] = sum_k q[m][k] * bit[n][k]           v_mfma_i32_32x32x32_i8, bits unpacked to 0/1
//   acc     = 2*C - sum_k q[m][k]                  (sgn = 2*bit - 1)
//   y[m][n] = s[m]*row_scale[n]*acc + up_scale[n] * sum_j t'[m][j] * lora_up[n][j]   (Eq. (3))
// with t' = dn_scale * s * t (the LoRA-down result, fp32) split as t' = hi + lo in bf16 so that
// the rank-r product runs on v_mfma_f32_32x32x16_bf16 (lora_up is int8, exact in bf16; the
// split keeps ~16 mantissa bits of t'). An optional residual is added (out_proj), and the int32
// acc can be written out (taps).
//
// Tiles: 128 x 128 outputs per workgroup, 4 waves as 2 x 2 of 64 x 64 (2 x 2 MFMA blocks each),
// K in steps of 64 through double-buffered LDS. Sign bits are unpacked once per workgroup into
// LDS (bytes 0/1), shared by the two waves of each column half. Ragged M and N are zero-filled.
#include "decode_device.h"

namespace dfssm {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int BM = 128, BN = 128, KT = 64;
constexpr int LDS_ROW = KT + 16;  // bytes per LDS row (padding staggers banks)

__device__ __forceinline__ uint32_t nibble_to_bytes(uint32_t nib) { return (nib * 0x00204081u) & 0x01010101u; }

__global__ __launch_bounds__(kBlock) void k_gemm_pm1(GemmArgs a) {
    __shared__ __align__(16) int8_t As[2][BM * LDS_ROW];
    __shared__ __align__(16) int8_t Bs[2][BN * LDS_ROW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int K = a.K;
    // staging: thread -> row tid/2 of the tile, half (32 k) tid%2
    const int srow = tid >> 1, shalf = tid & 1;
    const int gm = m0 + srow, gn = n0 + srow;
    const bool am = gm < a.M, bn_ok = gn < a.N;
    const int8_t *qrow = a.q + (int64_t)(am ? gm : 0) * a.ldq + shalf * 32;
    const uint8_t *brow = a.sign + (int64_t)(bn_ok ? gn : 0) * (K >> 3) + shalf * 4;
    int4 ra0, ra1;
    uint32_t rb;
    auto gload = [&](int k0) {
        if (am) {
            ra0 = *reinterpret_cast<const int4 *>(qrow + k0);
            ra1 = *reinterpret_cast<const int4 *>(qrow + k0 + 16);
        } else {
            ra0 = make_int4(0, 0, 0, 0);
            ra1 = ra0;
        }
        rb = bn_ok ? *reinterpret_cast<const uint32_t *>(brow + (k0 >> 3)) : 0u;
    };
    auto sstore = [&](int buf) {
        int8_t *ad = As[buf] + srow * LDS_ROW + shalf * 32;
        *reinterpret_cast<int4 *>(ad) = ra0;
        *reinterpret_cast<int4 *>(ad + 16) = ra1;
        int8_t *bd = Bs[buf] + srow * LDS_ROW + shalf * 32;
        int4 w0, w1;
        w0.x = (int)nibble_to_bytes(rb & 15u);
        w0.y = (int)nibble_to_bytes((rb >> 4) & 15u);
        w0.z = (int)nibble_to_bytes((rb >> 8) & 15u);
        w0.w = (int)nibble_to_bytes((rb >> 12) & 15u);
        w1.x = (int)nibble_to_bytes((rb >> 16) & 15u);
        w1.y = (int)nibble_to_bytes((rb >> 20) & 15u);
        w1.z = (int)nibble_to_bytes((rb >> 24) & 15u);
        w1.w = (int)nibble_to_bytes(rb >> 28);
        *reinterpret_cast<int4 *>(bd) = w0;
        *reinterpret_cast<int4 *>(bd + 16) = w1;
    };
    v16i acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;
    const int nk = K / KT;
    gload(0);
    sstore(0);
    __syncthreads();
    const int lr = lane & 31, lk = (lane >> 5) * 16;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * KT);
#pragma unroll
        for (int kk = 0; kk < KT; kk += 32) {
            v4i af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const v4i *>(As[cur] + (wm * 64 + i * 32 + lr) * LDS_ROW + kk + lk);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bf[j] = *reinterpret_cast<const v4i *>(Bs[cur] + (wn * 64 + j * 32 + lr) * LDS_ROW + kk + lk);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }
    // ---- low-rank term on bf16 MFMA: lacc[m][n] = sum_j t'[m][j] * lora_up[n][j]
    v16f lacc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) lacc[i][j][r] = 0.f;
    const int lj = (lane >> 5) * 8;
    for (int kr = 0; kr < a.rank; kr += 16) {
        const bool inr = kr + lj + 8 <= a.rank;
        v8bf ahi[2], alo[2], bup[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int m = m0 + wm * 64 + i * 32 + lr;
            if (inr && m < a.M) {
                ahi[i] = *reinterpret_cast<const v8bf *>(a.thi + (int64_t)m * a.rank + kr + lj);
                alo[i] = *reinterpret_cast<const v8bf *>(a.tlo + (int64_t)m * a.rank + kr + lj);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    ahi[i][e] = (__bf16)0.f;
                    alo[i][e] = (__bf16)0.f;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + wn * 64 + j * 32 + lr;
            uint2 w = make_uint2(0u, 0u);
            if (inr && n < a.N) w = *reinterpret_cast<const uint2 *>(a.lora_up + (int64_t)n * a.rank + kr + lj);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                bup[j][e] = (__bf16)(float)(int8_t)(w.x >> (8 * e));
                bup[j][4 + e] = (__bf16)(float)(int8_t)(w.y >> (8 * e));
            }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                lacc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[i], bup[j], lacc[i][j], 0, 0, 0);
                lacc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo[i], bup[j], lacc[i][j], 0, 0, 0);
            }
    }
    // ---- epilogue: lane holds column lr of each 32-wide block, rows 8*(r/4) + 4*(lane/32) + r%4
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn * 64 + j * 32 + lr;
        if (n >= a.N) continue;
        const float sc = half_bits_to_float(a.row_scale[n]);
        const float us = a.up_scale[n];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m >= a.M) continue;
                const int accv = 2 * acc[i][j][r] - a.qsum[m];
                float v = a.s[m] * sc * (float)accv + us * lacc[i][j][r];
                if (a.res) v += a.res[(int64_t)m * a.ldres + n];
                a.y[(int64_t)m * a.ldy + n] = v;
                if (a.acc_tap) a.acc_tap[(int64_t)m * a.ldacc + n] = accv;
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_pm1(const GemmArgs &a, hipStream_t stream) {
    if (a.K % KT || a.rank % 8 || a.rank > kMaxRank) return hipErrorInvalidValue;
    dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM);
    k_gemm_pm1<<<grid, kBlock, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace dfssm
