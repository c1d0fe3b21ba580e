// Density field codec of the SSM state ([DF-SSM] §3.4 "Density Field State Representation", App. D
// "Density Field Configuration"): each state row (the d_state values of one head channel) becomes
// a K x K bit field with K^2 ~ 4 d_state (K = 23 for d_state 128) plus its mean and standard
// deviation:
//   1. normalisation: x = clamp((s - (mu - 3 sigma)) / (6 sigma), 0, 1), taken to 8 bits t = rint(255 x)
//   2. first-order sigma-delta over the cells in raster order, value i owning cells
//      floor(i K^2 / N) .. floor((i+1) K^2 / N): v = e + t_i, bit = (v >= 128), e = v - 255 bit,
//      e an 8-bit accumulator (it stays in [-128, 127])
//   3. threshold at 0.5 (128 of 256)
//   4. readout: s' = mu - 3 sigma + 6 sigma * popcount(value's cells) / cells (a row with sigma = 0
//      reads back as mu)
// The sigma-delta pass is sequential along a row, so one lane owns one row and holds it in
// registers; the kernels are templated on d_state so that every value-to-cell boundary is a
// compile-time constant and the whole row is straight-line code (no indexed register arrays).
// Global traffic goes through a small LDS tile per wave so that each load or store instruction
// covers whole 128-byte lines: state rows move 32 columns at a time (a [64][33] float tile, odd
// stride so that the 64 lanes walking their rows hit distinct banks) and the fields of the wave's
// 64 consecutive rows, which are contiguous in memory, move as one coalesced block.
#include "decode_device.h"

namespace dfssm {

namespace {

constexpr int kCodecRows = 64;   // rows per workgroup (one wave, one row per lane)

constexpr int codec_side(int n) {
    // K = round(sqrt(4 n)) for the supported n (16, 32, 64, 128, 256): 8, 11, 16, 23, 32
    return n == 16 ? 8 : n == 32 ? 11 : n == 64 ? 16 : n == 128 ? 23 : n == 256 ? 32 : 0;
}
constexpr int codec_words(int n) { return (codec_side(n) * codec_side(n) + 31) / 32; }

// First cell of value i (value i owns cells cell_begin(i) .. cell_begin(i + 1) - 1).
template <int N>
constexpr int cell_begin(int i) {
    return (i * codec_side(N) * codec_side(N)) / N;
}

// Staging geometry: state columns move kT at a time through a [64][kT + 1] float tile (odd
// stride: the 64 lanes walking their own rows hit distinct banks); the wave's fields sit in LDS as
// [64][WS] words, WS the odd one of W, W + 1.
template <int N>
struct Tile {
    static constexpr int kT = N < 32 ? N : 32;             // columns per pass
    static constexpr int kStride = kT + 1;
    static constexpr int kLpr = kT / 4;                     // lanes per row (one float4 each)
    static constexpr int kRpp = kCodecRows / kLpr;          // rows per pass
    static constexpr int W = codec_words(N);
    static constexpr int WS = W | 1;
    static constexpr int kFloats = kCodecRows * (kStride > WS ? kStride : WS);
};

// Rows [r0, r0 + nr) of N floats, columns [c0, c0 + kT): global -> tile[row][col]. Each pass
// covers kRpp rows x kT * 4 contiguous bytes.
template <int N>
__device__ __forceinline__ void tile_load(const float *src, int64_t r0, int nr, int c0, float *tile) {
    using T = Tile<N>;
#pragma unroll
    for (int p = 0; p < kCodecRows / T::kRpp; ++p) {
        const int rr = p * T::kRpp + (int)threadIdx.x / T::kLpr, cc = ((int)threadIdx.x % T::kLpr) * 4;
        if (rr < nr) {
            const float4 v = *reinterpret_cast<const float4 *>(src + (r0 + rr) * N + c0 + cc);
            float *d = tile + rr * T::kStride + cc;
            d[0] = v.x;
            d[1] = v.y;
            d[2] = v.z;
            d[3] = v.w;
        }
    }
}

template <int N>
__device__ __forceinline__ void tile_store(float *dst, int64_t r0, int nr, int c0, const float *tile) {
    using T = Tile<N>;
#pragma unroll
    for (int p = 0; p < kCodecRows / T::kRpp; ++p) {
        const int rr = p * T::kRpp + (int)threadIdx.x / T::kLpr, cc = ((int)threadIdx.x % T::kLpr) * 4;
        if (rr < nr) {
            const float *s = tile + rr * T::kStride + cc;
            *reinterpret_cast<float4 *>(dst + (r0 + rr) * N + c0 + cc) = make_float4(s[0], s[1], s[2], s[3]);
        }
    }
}

// a / b rounded to nearest (the IEEE quotient) from y = RN(1 / b): q0 = RN(a y) is within two ulps;
// one fma correction makes it faithful, and the second is Markstein's step, which then yields the
// correctly rounded quotient (for normal b and quotients that neither overflow nor underflow; the
// codes only depend on quotients in [0, 1], smaller ones clamp to 0). Five operations instead of
// the ten of a full division, for the 8-bit codes of a row that share one divisor.
__device__ __forceinline__ float div_by_recip(float a, float b, float y) {
    const float q0 = a * y;
    const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, b, a), y, q0);
    return __builtin_fmaf(__builtin_fmaf(-q1, b, a), y, q1);
}

// 2^m as a float, -126 <= m <= 127.
__device__ __forceinline__ float pow2f(int m) { return __builtin_bit_cast(float, (uint32_t)(m + 127) << 23); }

// The divisor of a row's codes brought to [1, 2) by an exact power-of-two scale s1 * s2 (applied to
// every dividend as well, so each quotient is unchanged), which keeps RN(1 / divisor) normal for any
// span > 0. A span of 0 (a constant row, whose field is all zero) keeps scale 1.
struct RowDivisor {
    float s1, s2, b, y;
};
__device__ __forceinline__ RowDivisor row_divisor(float span) {
    const int k = span > 0.f ? -ilogbf(span) : 0;
    RowDivisor d;
    d.s1 = pow2f(k >> 1);
    d.s2 = pow2f(k - (k >> 1));
    d.b = (span * d.s1) * d.s2;
    d.y = 1.0f / d.b;
    return d;
}
__device__ __forceinline__ float row_quotient(float a, const RowDivisor &d) {
    return div_by_recip((a * d.s1) * d.s2, d.b, d.y);
}

// Readout of one row's field: lo + span * (ones among the value's cells) / cells.
template <int N>
__device__ __forceinline__ void row_decode(const uint32_t (&word)[codec_words(N)], float mu, float sigma,
                                           float (&out)[N]) {
    const float lo = mu - 3.0f * sigma, span = 6.0f * sigma;
    const bool flat = !(sigma != 0.f);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int c0 = cell_begin<N>(i), c1 = cell_begin<N>(i + 1);
        // cells c0 .. c1 - 1 span at most two words (a value owns fewer than 32 cells)
        const int w0 = c0 >> 5, w1 = (c1 - 1) >> 5, b0 = c0 & 31;
        int ones;
        if (w0 == w1) {
            const uint32_t m = (c1 - c0 == 32) ? 0xffffffffu : ((1u << (c1 - c0)) - 1u);
            ones = __builtin_popcount((word[w0] >> b0) & m);
        } else {
            const int n1 = c1 - (w1 << 5);
            ones = __builtin_popcount(word[w0] >> b0) + __builtin_popcount(word[w1] & ((1u << n1) - 1u));
        }
        const float dens = (float)ones * (1.0f / (float)(c1 - c0));
        out[i] = flat ? mu : lo + span * dens;
    }
}

template <int N>
__global__ __launch_bounds__(kCodecRows) void k_state_encode(const float *__restrict__ ssm, int64_t rows,
                                                            uint32_t *__restrict__ fields, float *__restrict__ stats) {
#pragma clang fp contract(off)
    using T = Tile<N>;
    constexpr int K2 = codec_side(N) * codec_side(N), W = T::W;
    __shared__ float lds[T::kFloats];
    const int64_t r0 = (int64_t)blockIdx.x * kCodecRows;
    const int nr = (int)min((int64_t)kCodecRows, rows - r0);
    const int lane = threadIdx.x;

    float v[N];
#pragma unroll
    for (int c0 = 0; c0 < N; c0 += T::kT) {
        tile_load<N>(ssm, r0, nr, c0, lds);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < T::kT; ++j) v[c0 + j] = lds[lane * T::kStride + j];
        __syncthreads();
    }

    // mean and population standard deviation, summed in element order
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) acc = acc + v[i];
    const float mu = acc / (float)N;
    float acc2 = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float d = v[i] - mu;
        acc2 = acc2 + d * d;
    }
    const float sigma = sqrtf(acc2 / (float)N);
    const float lo = mu - 3.0f * sigma, span = 6.0f * sigma;

    // 8-bit codes, kept as t - 128 so that a cell's decision is the sign of e + (t - 128)
    int tm[N];
    const RowDivisor dv = row_divisor(span);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float x = fminf(fmaxf(row_quotient(v[i] - lo, dv), 0.f), 1.f);
        tm[i] = (int)rintf(x * 255.0f) - 128;
    }

    // sigma-delta over the cells; bits collected inverted (a set bit of `inv` is a 0 cell)
    uint32_t word[W];
    int e = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) word[w] = 0u;
#pragma unroll
    for (int i = 0; i < N; ++i) {
#pragma unroll
        for (int c = cell_begin<N>(i); c < cell_begin<N>(i + 1); ++c) {
            const int u = e + tm[i];            // v - 128
            const int neg = u >> 31;            // -1 where v < 128 (bit 0), else 0
            e = u - 127 + (neg & 255);          // v - 255 * bit
            word[c >> 5] |= (uint32_t)neg & (1u << (c & 31));
        }
    }
    const bool flat = !(sigma != 0.f);   // sigma == 0: all-zero field, readout mu
    constexpr uint32_t kTailMask = (K2 & 31) ? ((1u << (K2 & 31)) - 1u) : 0xffffffffu;
#pragma unroll
    for (int w = 0; w < W; ++w) {
        const uint32_t valid = (w == W - 1) ? kTailMask : 0xffffffffu;
        lds[lane * T::WS + w] = __builtin_bit_cast(float, flat ? 0u : (~word[w] & valid));
    }
    if (lane < nr) *reinterpret_cast<float2 *>(stats + 2 * (r0 + lane)) = make_float2(mu, sigma);
    __syncthreads();
    // the wave's nr rows of fields are nr * W contiguous words
    uint32_t *dst = fields + r0 * W;
    for (int k = lane; k < nr * W; k += kCodecRows) {
        const int rr = k / W, w = k - rr * W;
        dst[k] = __builtin_bit_cast(uint32_t, lds[rr * T::WS + w]);
    }
}

template <int N>
__global__ __launch_bounds__(kCodecRows) void k_state_decode(const uint32_t *__restrict__ fields,
                                                            const float *__restrict__ stats, int64_t rows,
                                                            float *__restrict__ ssm) {
    using T = Tile<N>;
    constexpr int W = T::W;
    __shared__ float lds[T::kFloats];
    const int64_t r0 = (int64_t)blockIdx.x * kCodecRows;
    const int nr = (int)min((int64_t)kCodecRows, rows - r0);
    const int lane = threadIdx.x;

    const uint32_t *srcw = fields + r0 * W;
    for (int k = lane; k < nr * W; k += kCodecRows) {
        const int rr = k / W, w = k - rr * W;
        lds[rr * T::WS + w] = __builtin_bit_cast(float, srcw[k]);
    }
    float2 ms = make_float2(0.f, 0.f);
    if (lane < nr) ms = *reinterpret_cast<const float2 *>(stats + 2 * (r0 + lane));
    __syncthreads();
    uint32_t word[W];
#pragma unroll
    for (int w = 0; w < W; ++w) word[w] = __builtin_bit_cast(uint32_t, lds[lane * T::WS + w]);
    __syncthreads();

    float out[N];
    row_decode<N>(word, ms.x, ms.y, out);
#pragma unroll
    for (int c0 = 0; c0 < N; c0 += T::kT) {
#pragma unroll
        for (int j = 0; j < T::kT; ++j) lds[lane * T::kStride + j] = out[c0 + j];
        __syncthreads();
        tile_store<N>(ssm, r0, nr, c0, lds);
        __syncthreads();
    }
}

// DF-SSD carry ([DF-SSM] §3.4, App. D: the codec at chunk boundaries of the chunked scan). One wave
// per R rows of a (sequence, head) -- every state row is coded on its own -- and one lane per state
// row (the head's 64 channels): S starts as the layer's
// state; for every chunk c the state entering it is S itself for c = 0 and codec(S) after that,
// and it is written over sloc[c] (which held the chunk's own contribution S_loc, read first), then
// S = exp(Lam_end(c)) * entering + S_loc(c); the state after the last chunk is the layer's new state.
// Optional taps: the state entering each chunk before and after the codec.
struct ScanCodecArgs {
    float *state;            // [BH][64][N] initial -> final
    float *sloc;             // [BH][nch][64][N] chunk contributions -> entering states
    const float *lam_end;    // [BH][nch]
    int BH, nch;
    float *tap_pre, *tap_in; // [nch][BH][64][N] or null
};

// A whole [R][N] block (R rows of one chunk's S_loc of a head) in flight at once: the loads of every
// tile pass land in registers (rows kRpp apart, kT columns per pass), and later go to an [R][N + 1]
// LDS array (odd stride: each lane then reads its own row without bank conflicts). R is a multiple
// of kRpp; src points at the block's first row.
template <int N, int R>
struct BlockRegs {
    static constexpr int kLoads = (N / Tile<N>::kT) * (R / Tile<N>::kRpp);
    float4 v[kLoads];
};
template <int N, int R>
__device__ __forceinline__ void block_issue(const float *src, BlockRegs<N, R> &b) {
    using T = Tile<N>;
    const int rr0 = (int)threadIdx.x / T::kLpr, cc = ((int)threadIdx.x % T::kLpr) * 4;
#pragma unroll
    for (int c0 = 0; c0 < N / T::kT; ++c0)
#pragma unroll
        for (int p = 0; p < R / T::kRpp; ++p)
            b.v[c0 * (R / T::kRpp) + p] =
                *reinterpret_cast<const float4 *>(src + (int64_t)(p * T::kRpp + rr0) * N + c0 * T::kT + cc);
}
template <int N, int R>
__device__ __forceinline__ void block_to_lds(const BlockRegs<N, R> &b, float *full) {
    using T = Tile<N>;
    const int rr0 = (int)threadIdx.x / T::kLpr, cc = ((int)threadIdx.x % T::kLpr) * 4;
#pragma unroll
    for (int c0 = 0; c0 < N / T::kT; ++c0)
#pragma unroll
        for (int p = 0; p < R / T::kRpp; ++p) {
            const float4 v = b.v[c0 * (R / T::kRpp) + p];
            float *d = full + (p * T::kRpp + rr0) * (N + 1) + c0 * T::kT + cc;
            d[0] = v.x;
            d[1] = v.y;
            d[2] = v.z;
            d[3] = v.w;
        }
}

template <int N, int R>
__global__ __launch_bounds__(kCodecRows) void k_ssd_scan_codec(ScanCodecArgs a) {
#pragma clang fp contract(off)
    using T = Tile<N>;
    __shared__ float lds[T::kFloats];
    // up to d_state 128 the next chunk's S_loc is in flight while the current chunk's state is
    // coded (a whole block in registers: 128 more per lane); d_state 256 loads it pass by pass
    constexpr bool kAhead = N <= 128;
    __shared__ float full[kAhead ? R * (N + 1) : 1];
    // rows [r0, r0 + R) of head bh; lanes past R repeat row R - 1's arithmetic and store nothing
    constexpr int kParts = kCodecRows / R;
    const int bh = blockIdx.x / kParts, r0 = (blockIdx.x % kParts) * R, lane = threadIdx.x;
    const int row = lane < R ? lane : R - 1;
    constexpr int64_t PN = (int64_t)kCodecRows * N;
    BlockRegs<kAhead ? N : 16, kAhead ? R : 16> nxt;
    if constexpr (kAhead) block_issue<N, R>(a.sloc + (int64_t)bh * a.nch * PN + (int64_t)r0 * N, nxt);
    float S[N];
#pragma unroll
    for (int c0 = 0; c0 < N; c0 += T::kT) {
        tile_load<N>(a.state + bh * PN, r0, R, c0, lds);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < T::kT; ++j) S[c0 + j] = lds[row * T::kStride + j];
        __syncthreads();
    }
    for (int c = 0; c < a.nch; ++c) {
        const int64_t slot = ((int64_t)c * a.BH + bh) * PN;
        if (a.tap_pre) {
#pragma unroll
            for (int c0 = 0; c0 < N; c0 += T::kT) {
#pragma unroll
                for (int j = 0; j < T::kT; ++j) lds[lane * T::kStride + j] = S[c0 + j];
                __syncthreads();
                tile_store<N>(a.tap_pre + slot, r0, R, c0, lds);
                __syncthreads();
            }
        }
        if (c > 0) {
            // ---- encode (mean and population standard deviation in element order, 8-bit codes,
            // sigma-delta), then read back in place
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < N; ++i) acc = acc + S[i];
            const float mu = acc / (float)N;
            float acc2 = 0.f;
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const float d = S[i] - mu;
                acc2 = acc2 + d * d;
            }
            const float sigma = sqrtf(acc2 / (float)N);
            const float lo = mu - 3.0f * sigma, span = 6.0f * sigma;
            int tm[N];
            const RowDivisor dv = row_divisor(span);
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const float x = fminf(fmaxf(row_quotient(S[i] - lo, dv), 0.f), 1.f);
                tm[i] = (int)rintf(x * 255.0f) - 128;
            }
            // The field is only read back here, so the sigma-delta runs one step per value: with
            // U = e + 127 in [0, 254] at a value's first cell, each of its c cells adds t (0..255)
            // to U and emits a 1 exactly when U reaches 255 (then U -= 255), so the value's cells
            // hold (U + c t) div 255 ones and leave U' = (U + c t) mod 255 -- the same bits' count
            // as the cell-by-cell pass, without the 529-step chain.
            const bool flat = !(sigma != 0.f);
            uint32_t U = 127u;
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const uint32_t cells = (uint32_t)(cell_begin<N>(i + 1) - cell_begin<N>(i));
                const uint32_t sum = U + cells * (uint32_t)(tm[i] + 128);
                const uint32_t ones = sum / 255u;
                U = sum - 255u * ones;
                const float dens = (float)ones * (1.0f / (float)cells);
                S[i] = flat ? mu : lo + span * dens;
            }
        }
        // S_loc of this chunk (loaded ahead; read before its slot is overwritten), the entering state
        // out, the carry
        const float f = expf(a.lam_end[(int64_t)bh * a.nch + c]);
        float *sl = a.sloc + ((int64_t)bh * a.nch + c) * PN;
        if constexpr (kAhead) {
            block_to_lds<N, R>(nxt, full);
            __syncthreads();
            float loc[N];
#pragma unroll
            for (int j = 0; j < N; ++j) loc[j] = full[row * (N + 1) + j];
            if (c + 1 < a.nch) block_issue<N, R>(sl + PN + (int64_t)r0 * N, nxt);
#pragma unroll
            for (int c0 = 0; c0 < N; c0 += T::kT) {
#pragma unroll
                for (int j = 0; j < T::kT; ++j) lds[lane * T::kStride + j] = S[c0 + j];
                __syncthreads();
                tile_store<N>(sl, r0, R, c0, lds);
                if (a.tap_in) tile_store<N>(a.tap_in + slot, r0, R, c0, lds);
                __syncthreads();
#pragma unroll
                for (int j = 0; j < T::kT; ++j) S[c0 + j] = f * S[c0 + j] + loc[c0 + j];
            }
        } else {
#pragma unroll
            for (int c0 = 0; c0 < N; c0 += T::kT) {
                tile_load<N>(sl, r0, R, c0, lds);
                __syncthreads();
                float loc[T::kT];
#pragma unroll
                for (int j = 0; j < T::kT; ++j) loc[j] = lds[row * T::kStride + j];
                __syncthreads();
#pragma unroll
                for (int j = 0; j < T::kT; ++j) lds[lane * T::kStride + j] = S[c0 + j];
                __syncthreads();
                tile_store<N>(sl, r0, R, c0, lds);
                if (a.tap_in) tile_store<N>(a.tap_in + slot, r0, R, c0, lds);
                __syncthreads();
#pragma unroll
                for (int j = 0; j < T::kT; ++j) S[c0 + j] = f * S[c0 + j] + loc[j];
            }
        }
    }
#pragma unroll
    for (int c0 = 0; c0 < N; c0 += T::kT) {
#pragma unroll
        for (int j = 0; j < T::kT; ++j) lds[lane * T::kStride + j] = S[c0 + j];
        __syncthreads();
        tile_store<N>(a.state + bh * PN, r0, R, c0, lds);
        __syncthreads();
    }
}

// The same carry with a row's values split over lanes (d_state >= 64): L = N / 32 lanes per state
// row, lane q of a row holding values [32 q, 32 q + 32), so a one-wave workgroup takes RW = 64 / L
// rows of a head and each lane runs a quarter (L = 4) of the per-value code. The row's mu and sigma
// keep their element order: the running sum passes from lane q to lane q + 1 after q's segment.
// The sigma-delta's U at a segment's first value is (127 + sum of c t over the row's earlier values)
// mod 255 -- the same U as the serial pass, from an exact integer prefix over the row's lanes. Every
// value gets the arithmetic of the row kernel above, so the states are bit-identical to it.
template <int N, int R>
__device__ __forceinline__ void block_to_seg_lds(const BlockRegs<N, R> &b, float *full) {
    using T = Tile<N>;
    constexpr int RS = N + N / 32;   // one pad float per 32-value segment
    const int rr0 = (int)threadIdx.x / T::kLpr, cc = ((int)threadIdx.x % T::kLpr) * 4;
#pragma unroll
    for (int c0 = 0; c0 < N / T::kT; ++c0)
#pragma unroll
        for (int p = 0; p < R / T::kRpp; ++p) {
            const float4 v = b.v[c0 * (R / T::kRpp) + p];
            float *d = full + (p * T::kRpp + rr0) * RS + c0 * (T::kT + 1) + cc;
            d[0] = v.x;
            d[1] = v.y;
            d[2] = v.z;
            d[3] = v.w;
        }
}
template <int N, int R>
__device__ __forceinline__ void seg_lds_store(float *dst, const float *full) {   // dst: the block's first row
    using T = Tile<N>;
    constexpr int RS = N + N / 32;
    const int rr0 = (int)threadIdx.x / T::kLpr, cc = ((int)threadIdx.x % T::kLpr) * 4;
#pragma unroll
    for (int c0 = 0; c0 < N / T::kT; ++c0)
#pragma unroll
        for (int p = 0; p < R / T::kRpp; ++p) {
            const float *d = full + (p * T::kRpp + rr0) * RS + c0 * (T::kT + 1) + cc;
            *reinterpret_cast<float4 *>(dst + (int64_t)(p * T::kRpp + rr0) * N + c0 * T::kT + cc) =
                make_float4(d[0], d[1], d[2], d[3]);
        }
}

template <int N>
__global__ __launch_bounds__(kCodecRows) void k_ssd_scan_codec_seg(ScanCodecArgs a) {
#pragma clang fp contract(off)
    static_assert(N >= 64 && Tile<N>::kT == 32, "segments of 32 values, one column tile each");
    constexpr int L = N / 32, RW = kCodecRows / L, RS = N + L;
    constexpr int K2 = codec_side(N) * codec_side(N), CMIN = K2 / N;
    static_assert(K2 < (N << 5), "a value owns fewer than 32 cells");
    __shared__ float full[RW * RS];
    const int lane = threadIdx.x, q = lane % L, rl = lane / L;
    const int bh = blockIdx.x / L, r0 = (blockIdx.x % L) * RW, i0 = 32 * q;
    constexpr int64_t PN = (int64_t)kCodecRows * N;
    float *seg = full + rl * RS + q * 33;
    float S[32];
    {
        BlockRegs<N, RW> cur;
        block_issue<N, RW>(a.state + bh * PN + (int64_t)r0 * N, cur);
        block_to_seg_lds<N, RW>(cur, full);
    }
    BlockRegs<N, RW> nxt;
    block_issue<N, RW>(a.sloc + (int64_t)bh * a.nch * PN + (int64_t)r0 * N, nxt);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 32; ++j) S[j] = seg[j];
    __syncthreads();
    for (int c = 0; c < a.nch; ++c) {
        const int64_t slot = ((int64_t)c * a.BH + bh) * PN + (int64_t)r0 * N;
        if (a.tap_pre) {
#pragma unroll
            for (int j = 0; j < 32; ++j) seg[j] = S[j];
            __syncthreads();
            seg_lds_store<N, RW>(a.tap_pre + slot, full);
            __syncthreads();
        }
        if (c > 0) {
            // mean in element order: L stages, stage s summing lane s's segment onto the sum of the
            // values before it (the other lanes' results of that stage are not used)
            float run = 0.f, tot = 0.f;
#pragma unroll
            for (int st = 0; st < L; ++st) {
                float acc = run;
#pragma unroll
                for (int j = 0; j < 32; ++j) acc = acc + S[j];
                const float up = __shfl_up(acc, 1);
                if (q == st + 1) run = up;
                tot = acc;
            }
            const float mu = __shfl(tot, rl * L + L - 1) / (float)N;
            float dd[32];
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const float d = S[j] - mu;
                dd[j] = d * d;
            }
            run = 0.f;
#pragma unroll
            for (int st = 0; st < L; ++st) {
                float acc = run;
#pragma unroll
                for (int j = 0; j < 32; ++j) acc = acc + dd[j];
                const float up = __shfl_up(acc, 1);
                if (q == st + 1) run = up;
                tot = acc;
            }
            const float sigma = sqrtf(__shfl(tot, rl * L + L - 1) / (float)N);
            const float lo = mu - 3.0f * sigma, span = 6.0f * sigma;
            const RowDivisor dv = row_divisor(span);
            uint32_t ct[32];
            uint32_t part = 0u;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const float x = fminf(fmaxf(row_quotient(S[j] - lo, dv), 0.f), 1.f);
                const uint32_t t = (uint32_t)(int)rintf(x * 255.0f);
                const int i = i0 + j;
                const uint32_t cells = (uint32_t)((i + 1) * K2) / N - (uint32_t)(i * K2) / N;
                ct[j] = cells * t;
                part += ct[j];
            }
            uint32_t incl = part;   // inclusive prefix of the row's per-lane sums
#pragma unroll
            for (int d = 1; d < L; d <<= 1) {
                const uint32_t o = __shfl_up(incl, d);
                if (q >= d) incl += o;
            }
            uint32_t U = (127u + (incl - part)) % 255u;
            const bool flat = !(sigma != 0.f);
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const int i = i0 + j;
                const uint32_t cells = (uint32_t)((i + 1) * K2) / N - (uint32_t)(i * K2) / N;
                const uint32_t sum = U + ct[j];
                const uint32_t ones = sum / 255u;
                U = sum - 255u * ones;
                const float rc = cells == (uint32_t)CMIN ? 1.0f / (float)CMIN : 1.0f / (float)(CMIN + 1);
                const float dens = (float)ones * rc;
                S[j] = flat ? mu : lo + span * dens;
            }
        }
        const float f = expf(a.lam_end[(int64_t)bh * a.nch + c]);
        float *sl = a.sloc + ((int64_t)bh * a.nch + c) * PN + (int64_t)r0 * N;
        block_to_seg_lds<N, RW>(nxt, full);
        __syncthreads();
        float loc[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) loc[j] = seg[j];
        __syncthreads();
        if (c + 1 < a.nch) block_issue<N, RW>(sl + PN, nxt);
#pragma unroll
        for (int j = 0; j < 32; ++j) seg[j] = S[j];
        __syncthreads();
        seg_lds_store<N, RW>(sl, full);
        if (a.tap_in) seg_lds_store<N, RW>(a.tap_in + slot, full);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 32; ++j) S[j] = f * S[j] + loc[j];
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) seg[j] = S[j];
    __syncthreads();
    seg_lds_store<N, RW>(a.state + bh * PN + (int64_t)r0 * N, full);
}

template <int N>
hipError_t scan_codec_n(const ScanCodecArgs &a, hipStream_t stream) {
    // d_state >= 64: rows split over lanes; below: one lane per row, one wave per kRpp rows while
    // that keeps to 2,048 workgroups (the carry is bound by each wave's arithmetic), else per head
    constexpr int kR = Tile<N>::kRpp;
    if constexpr (N >= 64)
        k_ssd_scan_codec_seg<N><<<(unsigned)(a.BH * (N / 32)), kCodecRows, 0, stream>>>(a);
    else if ((int64_t)a.BH * (kCodecRows / kR) <= 2048)
        k_ssd_scan_codec<N, kR><<<(unsigned)(a.BH * (kCodecRows / kR)), kCodecRows, 0, stream>>>(a);
    else
        k_ssd_scan_codec<N, kCodecRows><<<(unsigned)a.BH, kCodecRows, 0, stream>>>(a);
    return hipGetLastError();
}

template <int N>
hipError_t encode_n(const float *ssm, int64_t rows, uint32_t *fields, float *stats, hipStream_t stream) {
    const int64_t grid = (rows + kCodecRows - 1) / kCodecRows;
    k_state_encode<N><<<(unsigned)grid, kCodecRows, 0, stream>>>(ssm, rows, fields, stats);
    return hipGetLastError();
}

template <int N>
hipError_t decode_n(const uint32_t *fields, const float *stats, int64_t rows, float *ssm, hipStream_t stream) {
    const int64_t grid = (rows + kCodecRows - 1) / kCodecRows;
    k_state_decode<N><<<(unsigned)grid, kCodecRows, 0, stream>>>(fields, stats, rows, ssm);
    return hipGetLastError();
}

}  // namespace

int codec_field_words(int d_state) { return codec_side(d_state) ? codec_words(d_state) : 0; }

hipError_t launch_state_encode(const float *ssm, int64_t rows, int N, uint32_t *fields, float *stats,
                               hipStream_t stream) {
    switch (N) {
    case 16: return encode_n<16>(ssm, rows, fields, stats, stream);
    case 32: return encode_n<32>(ssm, rows, fields, stats, stream);
    case 64: return encode_n<64>(ssm, rows, fields, stats, stream);
    case 128: return encode_n<128>(ssm, rows, fields, stats, stream);
    case 256: return encode_n<256>(ssm, rows, fields, stats, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_ssd_scan_codec(float *state, float *sloc, const float *lam_end, int BH, int nch, int N, int P,
                                 float *tap_pre, float *tap_in, hipStream_t stream) {
    if (P != kCodecRows) return hipErrorInvalidValue;
    const ScanCodecArgs a{state, sloc, lam_end, BH, nch, tap_pre, tap_in};
    switch (N) {
    case 16: return scan_codec_n<16>(a, stream);
    case 32: return scan_codec_n<32>(a, stream);
    case 64: return scan_codec_n<64>(a, stream);
    case 128: return scan_codec_n<128>(a, stream);
    case 256: return scan_codec_n<256>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_state_decode(const uint32_t *fields, const float *stats, int64_t rows, int N, float *ssm,
                               hipStream_t stream) {
    switch (N) {
    case 16: return decode_n<16>(fields, stats, rows, ssm, stream);
    case 32: return decode_n<32>(fields, stats, rows, ssm, stream);
    case 64: return decode_n<64>(fields, stats, rows, ssm, stream);
    case 128: return decode_n<128>(fields, stats, rows, ssm, stream);
    case 256: return decode_n<256>(fields, stats, rows, ssm, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace dfssm
