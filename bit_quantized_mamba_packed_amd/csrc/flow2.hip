// Persistent stack decode with two exchanges per layer, for one token per step (batch 1: every
// weight and state a workgroup needs stays in registers or LDS without spilling).
//
// One cooperative launch runs every step of every layer. The workgroups have two roles:
//   role 1, item w < n1: head h = w / S, channels [p0, p0 + pr) of that head (pr = P / S):
//            gather the residual h (all D values), RMSNorm + int8 quantizer, LoRA-down t, the
//            packed-sign GEMV of its share (q rows) of the B and C rows -> rescale + LoRA-up, conv
//            step, publish them at once; then the rows only it consumes (its z and x channels, its
//            head's dt row) while those travel; gather its group's B and C, SSM update + readout,
//            SiLU(z) gate -> publish this item's gated outputs g
//   role 2, item w >= n1: out_proj rows [(w - n1) * R2, ...): gather g (all E values), gated
//            RMSNorm + quantizer, LoRA-down, GEMV of its rows, epilogue, residual add -> publish
//            those rows of h (it keeps them: they are its next residual input)
// Each exchange (h, B/C, g) is an all-gather of tagged 64-bit words {payload, epoch}, written with
// agent-coherent stores and read with 16-byte agent-coherent loads until every epoch matches;
// there are no flags and no barriers. The h and g producers write their words as whole 128-byte
// lines in one store instruction (a role-2 workgroup's 16 rows of h; an item's gated outputs,
// staged in LDS first): coherent stores of partial lines take microseconds longer to be visible. Every layer has its own word slots, rewritten one token
// later; every workgroup reads all of a layer's words before anything of the next token's same
// layer can be produced, so a slot is never rewritten while a reader still needs it.
//
// A workgroup works on one phase per layer, so right after publishing it loads what its next
// layer needs that does not depend on the token (sign rows and LoRA-down factors straight into
// LDS, scales, conv taps and windows, SSM state into registers): that latency hides behind the
// other role's work. Every wait is bounded: on a timeout the kernel sets the workspace's error
// flag and every later wait gives up at once, so every wave still reaches the end; the launch that
// follows the kernel (launch_stack_finish) reports the flag and fills y with NaN.

#include <atomic>

#include "decode_device.h"

namespace dfssm {

namespace {

// Threads per workgroup: eight waves, two on each SIMD, so that one wave's LDS, DPP and memory
// latencies are covered by the other's work (with one wave per SIMD every one of them is exposed).
constexpr int F2_T = 512;
constexpr int F2_W = F2_T / 64;
// in_proj rows per GEMV thread (rows rg + NG * i, the B/C rows first): with CPR lanes per row
// (CPR = d_model / 128, NG = F2_T / CPR row groups) an item may hold up to 96, 64 or 128 rows
constexpr int f2_maxi(int cpr) { return cpr >= 16 ? 3 : 1; }
constexpr int F2_SBLK = 4;    // 1 KB blocks of in_proj sign rows each wave copies per layer
constexpr int F2_UPC = 2;     // LoRA-up chunks (16 B) per row: rank <= 32
// out_proj rows per GEMV thread: a role-2 workgroup holds d_model / 128 rows
constexpr int f2_maxo(int cpr) { return cpr >= 64 ? 2 : 1; }
constexpr int F2_FPT = 2;     // SSM state float4s per thread and token
constexpr int F2_BCW = 2;     // first wave of the B/C gather (rows past 128 would share a wave with it)
constexpr int F2_ROWS = 512;  // item rows (incl. padding rows) per workgroup, at most
constexpr unsigned kSpin2 = 1u << 21;
constexpr int kSleep2 = 1;
constexpr int kTable2 = 16;
constexpr int kMaxDevices2 = 64;
constexpr size_t kF2MaxLds = 159 * 1024;

struct Entry2 {
    dfssm_layer_weights w;
    dfssm_layer_state st;
};
struct Chunk2 {
    Entry2 e[kTable2];
};

struct F2Args {
    int n_layers, n_steps, batch;
    int D, E, N, P, H, G, Cd, Nin, Ninp, Rin, Rout;
    float eps;
    int S, pr, q, R1, npad, R2, fpt, n1, n2;
    const Entry2 *layers;
    const float *final_w, *x0;
    float *y;
    uint64_t *hx, *gx;  // [L][batch][D], [L][batch][E] tagged words
    uint64_t *rx;       // the stack's final RMSNorm factor of the previous token (tagged)
    uint64_t *bcx;      // [L][batch][2GN] tagged words: the conv'd B and C of every group
    int *err;
    dfssm_taps taps;
};

// Weights and state are reached through pointers read from the layer table, which the compiler
// cannot place in an address space: accessed as generic (flat) memory, every store would hold up the
// next LDS wait until it is acknowledged. These helpers state that they are global memory, and the
// table itself is read through the constant address space (scalar loads: it does not change while
// the kernel runs). The host pass of the single-source compile has no address spaces for class
// types and only needs the declarations.
#define F2_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ T gld(const T *p) {
#if __HIP_DEVICE_COMPILE__
    return *(const F2_GLOBAL T *)p;
#else
    return *p;
#endif
}
template <typename T>
__device__ __forceinline__ void gst(T *p, const T &v) {
#if __HIP_DEVICE_COMPILE__
    *(F2_GLOBAL T *)p = v;
#else
    *p = v;
#endif
}
__device__ __forceinline__ Entry2 f2_entry(const F2Args &a, int l) {
#if __HIP_DEVICE_COMPILE__
    return ((const __attribute__((address_space(4))) Entry2 *)a.layers)[l];
#else
    return a.layers[l];
#endif
}

__device__ __forceinline__ size_t f2_round_kb(size_t v) { return (v + 1023) & ~(size_t)1023; }
__device__ __forceinline__ uint64_t tag2(uint32_t bits, uint32_t tag) { return ((uint64_t)tag << 32) | bits; }
__device__ __forceinline__ uint32_t fbits2(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float bitsf2(uint32_t b) { return __builtin_bit_cast(float, b); }

__device__ void f2_error(const F2Args &a) { __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// This thread's 4*KCH consecutive words at p, reloaded until every epoch equals `tag` (bounded).
template <int KCH>
__device__ __forceinline__ void f2_gather(const F2Args &a, const uint64_t *p, uint32_t tag, u32x4 (&r)[2 * KCH]) {
    unsigned spins = 0;
    for (;;) {
        load_words_sc1<KCH>(p, r);
        bool ok = true;
#pragma unroll
        for (int j = 0; j < 2 * KCH; ++j) ok = ok && r[j].y == tag && r[j].w == tag;
        if (ok) return;
        __builtin_amdgcn_s_sleep(kSleep2);
        ++spins;
        if ((spins & 63) == 0 && ld_x(a.err)) return;
        if (spins > kSpin2) {
            f2_error(a);
            return;
        }
    }
}

// 8x8 bit transpose (delta swaps, Hacker's Delight 7-3): with code j in byte j of x, byte p of the
// result holds bit p of every code, code j in bit j.
__device__ __forceinline__ uint64_t transpose8(uint64_t x) {
    uint64_t t = (x ^ (x >> 7)) & 0x00AA00AA00AA00AAull;
    x ^= t ^ (t << 7);
    t = (x ^ (x >> 14)) & 0x0000CCCC0000CCCCull;
    x ^= t ^ (t << 14);
    t = (x ^ (x >> 28)) & 0x00000000F0F0F0F0ull;
    x ^= t ^ (t << 28);
    return x;
}

// Bit-plane words of 32 consecutive codes from registers: the thread holds 4*KCH consecutive codes
// (packed four to a word, lowest code in the low byte); the 32/(4*KCH) threads of one plane word
// merge their bits with DPP row shifts, and the first of them returns the eight words (bit j of
// plane p = bit p of code 32w + j).
template <int KCH>
__device__ __forceinline__ void code_planes(const uint32_t (&pk)[KCH], uint32_t (&pw)[8]) {
    constexpr int NP = KCH >= 2 ? KCH / 2 : 1, BL = 4 * KCH;
    uint64_t y[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k)
        y[k] = transpose8((uint64_t)pk[2 * k < KCH ? 2 * k : 0] | (2 * k + 1 < KCH ? (uint64_t)pk[2 * k + 1] << 32 : 0ull));
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        uint32_t v = 0;
#pragma unroll
        for (int k = 0; k < NP; ++k) v |= (uint32_t)((y[k] >> (8 * p)) & 0xFFu) << (8 * k);
        if (BL < 32) v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x101, 0xF, 0xF, true) << (BL & 31);        // lane + 1
        if (BL < 16) v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x102, 0xF, 0xF, true) << ((2 * BL) & 31);  // lane + 2
        if (BL < 8) v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x104, 0xF, 0xF, true) << ((4 * BL) & 31);   // lane + 4
        pw[p] = v;
    }
}

// Sum over groups of w consecutive lanes (w a power of two <= 64, uniform across the wave but not
// known at compile time), total in the group's last lane: every DPP step runs and the steps past w
// add zero, so the reduction has no branches.
template <int CTRL, int RMASK, bool BC>
__device__ __forceinline__ float f2_dpp_step(float v, int keep) {
    const int d = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, RMASK, 0xF, BC);
    return v + __builtin_bit_cast(float, d & keep);
}
__device__ __forceinline__ float f2_group_sum(float v, int w) {
    v = f2_dpp_step<0xB1, 0xF, true>(v, -(w >= 2));
    v = f2_dpp_step<0x4E, 0xF, true>(v, -(w >= 4));
    v = f2_dpp_step<0x114, 0xF, true>(v, -(w >= 8));
    v = f2_dpp_step<0x118, 0xF, true>(v, -(w >= 16));
    v = f2_dpp_step<0x142, 0xA, false>(v, -(w >= 32));
    v = f2_dpp_step<0x143, 0xC, false>(v, -(w >= 64));
    return v;
}

__device__ __forceinline__ float f2_ss(const float4 &v) { return v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w; }

// The F2_W per-wave partials in a fixed pairwise order (every workgroup gets the same bits).
__device__ __forceinline__ float f2_sum8(const float *v) {
    return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
}
__device__ __forceinline__ float f2_max8(const float *v) {
    return fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])), fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
}
__device__ __forceinline__ int f2_isum8(const int *v) {
    return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
}
static_assert(F2_W == 8, "the partial combinations take eight waves");

// RMSNorm factor (mean of squares + eps)^-1/2 by the hardware reciprocal square root (about one
// ulp): the factor needs no correctly rounded value, since the quantizer's decisions are taken on
// the u this workgroup forms with it, and the last token's final RMSNorm uses the same expression.
__device__ __forceinline__ float f2_rnorm(float sumsq, int K, float eps) {
    return __builtin_amdgcn_rsqf(sumsq / (float)K + eps);
}

// The stack's final RMSNorm, (h * r) * w, of one gathered vector: the thread layout and the order of
// the sum of squares are the prologue's, so that the last token's output is bit-identical to what
// the next token's prologue would form from the same words.
// One barrier: the per-wave partials go to slots (F2_W floats) that nothing writes again before
// the caller's next barrier; the combination order is fixed, so every workgroup reducing the same
// data gets the same bits.
template <int KCH>
__device__ __forceinline__ float f2_norm_factor(const F2Args &a, const float4 (&hv)[KCH], int K, float *slot) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < KCH; ++i) ss += f2_ss(hv[i]);
    ss = dpp_wave_sum(ss);
    if ((threadIdx.x & 63) == 0) slot[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = f2_sum8(slot);
    return f2_rnorm(tot, K, a.eps);
}

// Gather NB vectors of K tagged words, RMSNorm (after the stack's final RMSNorm when pre_w is set),
// int8 quantizer -> codes sq[b][K], bit-planes spl[b][8][K/32]; every thread gets the sum of the
// codes and the scale. wr: this thread's norm weights. Taps are written by workgroup tapwg. red:
// 3 * F2_W floats, ired: NB * F2_W ints of LDS. Two barriers per vector (three with pre_w).
template <int NB, int KCH>
__device__ void f2_prologue(const F2Args &a, const uint64_t *X, int K, uint32_t tag, const float4 (&wr)[KCH],
                            const float *pre_w, float *pre_out, int8_t *sq, uint32_t *spl, int (&qsum)[NB],
                            float (&scale)[NB], float *red, int *ired, bool tapwg, float *r0_out, float *tap_h,
                            float *tap_u, int8_t *tap_q, float *tap_s) {
    const int tid = threadIdx.x;
    const int e0 = prologue_elem<KCH>(0);
    const bool mine = e0 < K;   // K is a multiple of 4*KCH: a thread has all of its chunks or none
    for (int b = 0; b < NB; ++b) {
        float4 hv[KCH];
        if (mine) {
            u32x4 r[2 * KCH];
            f2_gather<KCH>(a, X + (int64_t)b * K + e0, tag, r);
#pragma unroll
            for (int i = 0; i < KCH; ++i)
                hv[i] = make_float4(bitsf2(r[2 * i].x), bitsf2(r[2 * i].z), bitsf2(r[2 * i + 1].x), bitsf2(r[2 * i + 1].z));
        } else {
#pragma unroll
            for (int i = 0; i < KCH; ++i) hv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        float ss = 0.f;
        if (pre_w) {
            const float r0 = f2_norm_factor<KCH>(a, hv, K, red + 2 * F2_W);
            if (r0_out && tid == 0) *r0_out = r0;
            if (mine) {
#pragma unroll
                for (int i = 0; i < KCH; ++i) {
                    const int e = prologue_elem<KCH>(i);
                    const float4 w = *reinterpret_cast<const float4 *>(pre_w + e);
                    hv[i].x = (hv[i].x * r0) * w.x;
                    hv[i].y = (hv[i].y * r0) * w.y;
                    hv[i].z = (hv[i].z * r0) * w.z;
                    hv[i].w = (hv[i].w * r0) * w.w;
                    if (tapwg && pre_out) *reinterpret_cast<float4 *>(pre_out + (int64_t)b * K + e) = hv[i];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < KCH; ++i) ss += f2_ss(hv[i]);
        float pm = 0.f;
        if (mine) {
#pragma unroll
            for (int i = 0; i < KCH; ++i) {
                const int e = prologue_elem<KCH>(i);
                if (tapwg && tap_h) *reinterpret_cast<float4 *>(tap_h + (int64_t)b * K + e) = hv[i];
                const float4 w = wr[i];
                hv[i].x = hv[i].x * w.x;
                hv[i].y = hv[i].y * w.y;
                hv[i].z = hv[i].z * w.z;
                hv[i].w = hv[i].w * w.w;
                pm = fmaxf(pm, fmaxf(fmaxf(fabsf(hv[i].x), fabsf(hv[i].y)), fmaxf(fabsf(hv[i].z), fabsf(hv[i].w))));
            }
        }
        // u = fl(fl(h * w) * r): with r > 0 the largest |u| is fl(max|h * w| * r) exactly
        ss = dpp_wave_sum(ss);
        pm = dpp_wave_max(pm);
        if ((tid & 63) == 0) {
            red[tid >> 6] = ss;
            red[F2_W + (tid >> 6)] = pm;
        }
        __syncthreads();
        const float tot = f2_sum8(red);
        pm = f2_max8(red + F2_W);
        const float r = f2_rnorm(tot, K, a.eps);
        const float amax = pm * r;
        const float inv = amax > 0.f ? 127.0f / amax : 0.f;
        const float s = amax > 0.f ? amax / 127.0f : 0.f;
        int qs = 0;
        uint32_t pk[KCH];
#pragma unroll
        for (int i = 0; i < KCH; ++i) pk[i] = 0;
        if (mine) {
#pragma unroll
            for (int i = 0; i < KCH; ++i) {
                const int e = prologue_elem<KCH>(i);
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
                pk[i] = packed;
                if (tapwg) {
                    if (tap_u) *reinterpret_cast<float4 *>(tap_u + (int64_t)b * K + e) = hv[i];
                    if (tap_q) *reinterpret_cast<uint32_t *>(tap_q + (int64_t)b * K + e) = packed;
                }
            }
        }
        {
            uint32_t pw[8];
            code_planes<KCH>(pk, pw);
            constexpr int NL = KCH >= 8 ? 1 : 8 / KCH;   // threads per plane word
            if (mine && tid % NL == 0) {
                const int w = tid * KCH / 8, G32 = K >> 5;
#pragma unroll
                for (int p = 0; p < 8; ++p) spl[(b * 8 + p) * G32 + w] = pw[p];
            }
        }
        qs = dpp_wave_isum(qs);
        if ((tid & 63) == 0) ired[b * F2_W + (tid >> 6)] = qs;
        scale[b] = s;
        if (tapwg && tap_s && tid == 0) tap_s[b] = s;
        if (NB > 1) __syncthreads();   // red is reused by the next vector
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < NB; ++b)
        qsum[b] = f2_isum8(ired + b * F2_W);
}

// sum_k sgn * q of one 16-byte sign chunk against the bit-planes of the same 128 codes:
// 2 * (sum over set bits of q) - sum(q) is finished by the caller; this returns sum over set bits.
__device__ __forceinline__ int chunk_pos(const uint4 &bits, const uint4 (&pl)[8]) {
    int pos = 0;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int c = __popc(bits.x & pl[p].x) + __popc(bits.y & pl[p].y) + __popc(bits.z & pl[p].z) +
                      __popc(bits.w & pl[p].w);
        pos += p < 7 ? (c << p) : -(c << 7);
    }
    return pos;
}

__device__ __forceinline__ int sdot_chunk(const uint4 &w, const int4 &q, int acc) {
    acc = __builtin_amdgcn_sdot4((int)w.x, q.x, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.y, q.y, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.z, q.z, acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.w, q.w, acc, false);
    return acc;
}

// LoRA-down sums t[j] = L_dn[j] . q of a factor held in LDS ([rank][K] int8, rank <= 32) against
// codes in LDS: wave jg takes rows jg + 8 * jj (jj < 4), lane cl the 16-byte chunks cl + 64 * m
// (K = 4 * KCH * F2_T, so 2 * KCH chunks per lane), so each code chunk is read once for four rows
// and all of a thread's reads are issued before the first is used. The sums end in lane 63.
template <int KCH>
__device__ __forceinline__ void lora_down_sums(const char *ldn, const int8_t *q, int K, int rank, int (&part)[4]) {
    const int jg = threadIdx.x >> 6, cl = threadIdx.x & 63, C16 = K >> 4;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) part[jj] = 0;
    // no branches (they would split the reads into separately waited blocks): chunks past the row
    // end are read clamped with zero codes, rows past the rank clamped (their sums are not used)
#pragma unroll
    for (int m = 0; m < 2 * KCH; ++m) {
        const bool in = cl + 64 * m < C16;
        const int cc = in ? cl + 64 * m : C16 - 1;
        int4 qv = *reinterpret_cast<const int4 *>(q + cc * 16);
        if (!in) qv = make_int4(0, 0, 0, 0);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            part[jj] = sdot_chunk(*reinterpret_cast<const uint4 *>(ldn + (size_t)min(jg + 8 * jj, rank - 1) * K + cc * 16), qv,
                                  part[jj]);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) part[jj] = dpp_group_sum(part[jj], 64);
}

template <int KCH>
__device__ __forceinline__ void load_norm_w(float4 (&wr)[KCH], const float *w, int K) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
        const int e = prologue_elem<KCH>(i);
        wr[i] = e < K ? gld(reinterpret_cast<const float4 *>(w + e)) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

// Direct-to-LDS copies (no registers): a wave instruction moves 64 lanes x 16 bytes into 1 KB of
// consecutive LDS. Chunk i of the destination comes from src(i); lanes past n copy chunk 0 into the
// padding (regions are whole KB). Every workgroup reads the same weights at the same moment, so each
// starts at a different 1 KB block (rot) and wraps: the concurrent requests spread over all L2
// channels instead of queueing on the one that holds the block everybody wants.
__device__ __forceinline__ int f2_rot(int nblk) { return nblk > 0 ? (int)((blockIdx.x * 37u) % (unsigned)nblk) : 0; }

__device__ __forceinline__ void lds_copy_contig(char *dst, const char *src, int n16) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nblk = (n16 + 63) >> 6, rot = f2_rot(nblk);
    for (int k = wave; k < nblk; k += F2_W) {
        int kb = k + rot;
        if (kb >= nblk) kb -= nblk;
        const int base = kb * 64, i = base + lane;
        __builtin_amdgcn_global_load_lds(src + (size_t)(i < n16 ? i : 0) * 16, dst + (size_t)base * 16, 16, 0, 0);
    }
}

// sum_j L_up[n][j] * v[j] over the (at most 32) low-rank terms; v (16-byte aligned LDS) is read as
// eight 16-byte vectors before the first product, so the reads are in flight together.
__device__ __forceinline__ float up_dot2(const int4 (&w)[F2_UPC], int rank, const float *v) {
    float4 vv[4 * F2_UPC];
#pragma unroll
    for (int i = 0; i < 4 * F2_UPC; ++i) vv[i] = reinterpret_cast<const float4 *>(v)[i];
    float lr = 0.f;
#pragma unroll
    for (int i = 0; i < F2_UPC; ++i) {
        // no rank test: past the rank both the weights (zero-padded) and v (zeroed) are zero
        const int ws[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 x = vv[4 * i + q];
            lr += (float)(int8_t)(ws[q]) * x.x;
            lr += (float)(int8_t)(ws[q] >> 8) * x.y;
            lr += (float)(int8_t)(ws[q] >> 16) * x.z;
            lr += (float)(int8_t)(ws[q] >> 24) * x.w;
        }
    }
    return lr;
}

__device__ __forceinline__ void load_up(int4 (&w)[F2_UPC], const int8_t *lora_up, int rank, int n) {
    const int8_t *p = lora_up + (int64_t)n * rank;
#pragma unroll
    for (int i = 0; i < F2_UPC; ++i) {
        if (i * 16 < rank) {
            if (i * 16 + 16 <= rank) {
                w[i] = gld(reinterpret_cast<const int4 *>(p) + i);
            } else {   // rank 8: half a chunk
                const int2 h = gld(reinterpret_cast<const int2 *>(p) + 2 * i);
                w[i] = make_int4(h.x, h.y, 0, 0);
            }
        } else {
            w[i] = make_int4(0, 0, 0, 0);
        }
    }
}

// Row of row group g (of ng) in GEMV pass i: passes 0 and 1 in group order, later ones reversed.
__device__ __forceinline__ int f2_pass_row(int g, int i, int ng) { return ng * i + (i >= 2 ? ng - 1 - g : g); }

// Which in_proj row / conv channel the r-th row of an item covers: first the item's share of the B
// and C rows (all groups' B rows, then all groups' C rows, spread over the items), then its z
// channels, its x channels, its head's dt row, and (workgroup 0, with taps) the padding rows.
struct ItemRow {
    int n, ch;  // in_proj row, conv channel (-1: z, dt or padding row; -2: no row)
};
__device__ __forceinline__ ItemRow item_row(const F2Args &a, int r, int h, int p0, int bc0) {
    const int pr = a.pr, q = a.q, E = a.E;
    ItemRow m{0, -1};
    if (r < q) {
        const int bc = bc0 + r;
        m.ch = bc < 2 * a.G * a.N ? E + bc : -2;
    } else if (r < q + pr) {
        m.n = h * a.P + p0 + (r - q);
    } else if (r < q + 2 * pr) {
        m.ch = h * a.P + p0 + (r - q - pr);
    } else if (r == q + 2 * pr) {
        m.n = E + a.Cd + h;
    } else {
        m.n = a.Nin + (r - a.R1);   // padding row (computed only for the taps)
    }
    if (m.ch >= 0) m.n = E + m.ch;
    return m;
}

// Per-thread parameters of one in_proj row of the item, loaded a layer ahead. The fp16 row scale
// stays in its bits until used, so that no load has to complete inside the prefetch.
template <int NB>
struct RowRegs {
    ItemRow m;
    uint32_t scb;
    float us, cb;
    float4 cw;
    int4 up[F2_UPC];
    float win[NB][3];
};

template <int NB>
__device__ __forceinline__ void load_row(RowRegs<NB> &R, const ItemRow &m, const Entry2 &Ly, int rank, int Cd) {
    const dfssm_proj &pin = Ly.w.in_proj;
    R.m = m;
    if (m.ch == -2) return;
    R.scb = gld(pin.row_scale + m.n);
    R.us = gld(pin.lora_up_scale + m.n);
    load_up(R.up, pin.lora_up, rank, m.n);
    if (m.ch >= 0) {
        R.cw = gld(reinterpret_cast<const float4 *>(Ly.w.conv_w + (int64_t)m.ch * kConvTaps));
        R.cb = gld(Ly.w.conv_b + m.ch);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float *w = Ly.st.conv + ((int64_t)b * Cd + m.ch) * (kConvTaps - 1);
            R.win[b][0] = gld(w);
            R.win[b][1] = gld(w + 1);
            R.win[b][2] = gld(w + 2);
        }
    }
}

// Scaffold + low-rank output of one in_proj row (Eq. 3); for a conv channel also the conv step:
// the window moves on in the caller's state and the SiLU activation is returned.
template <int NB>
__device__ __forceinline__ float finish_row(const RowRegs<NB> &R, int b, int acc, float s, const float *tvb, int rank,
                                            float *conv_state, int Cd) {
    const float yv = s * half_bits_to_float((uint16_t)R.scb) * (float)acc + R.us * up_dot2(R.up, rank, tvb);
    if (R.m.ch < 0) return yv;
    const float pre = R.cb + R.cw.x * R.win[b][0] + R.cw.y * R.win[b][1] + R.cw.z * R.win[b][2] + R.cw.w * yv;
    float *w = conv_state + ((int64_t)b * Cd + R.m.ch) * (kConvTaps - 1);
    gst(w, R.win[b][1]);
    gst(w + 1, R.win[b][2]);
    gst(w + 2, yv);
    return silu_f(pre);
}

// TAPS: whether any debug tap is set; without them the tap code (and the registers holding its
// pointers) is compiled out of the launch that carries no taps.
template <int NB, int KCH1, int KCH2, int CPR1, int CPR2, bool TAPS>
__global__ __launch_bounds__(F2_T, 1) void k_flow2(F2Args a) {
    constexpr int F2_MAXI = f2_maxi(CPR1), F2_MAXO = f2_maxo(CPR2);
    constexpr int NG1 = F2_T / CPR1, NG2 = F2_T / CPR2;
    extern __shared__ __align__(16) char smem[];
    __shared__ float red[3 * F2_W];
    __shared__ int ired[NB * F2_W];
    __shared__ float dtl[NB];
    __shared__ float gsh[NB][64];   // the item's gated outputs, published by one coalesced store
    int sqsum[NB];
    float ssc[NB];
    __shared__ float r0s;
    const int D = a.D, E = a.E, N = a.N, P = a.P;
    const int Kmax = D > E ? D : E;
    int8_t *sq = reinterpret_cast<int8_t *>(smem);                          // [NB][Kmax]
    uint32_t *spl = reinterpret_cast<uint32_t *>(smem + NB * Kmax);         // [NB][8][Kmax/32]
    int *accl = reinterpret_cast<int *>(smem + 2 * NB * Kmax);              // [NB][F2_ROWS]
    float *tv = reinterpret_cast<float *>(accl + NB * F2_ROWS);             // [NB][64]
    float *zl = tv + NB * 64;                                               // [NB][P]
    float *xl = zl + NB * P;                                                // [NB][P]
    float *Bl = xl + NB * P;                                                // [NB][N]
    float *Cl = Bl + NB * N;                                                // [NB][N]
    char *wreg = reinterpret_cast<char *>(Cl + NB * N);                     // sign rows, then LoRA-down rows
    const int tid = threadIdx.x, wg = blockIdx.x;
    const int L = a.n_layers, B = a.batch;
    const dfssm_taps T = TAPS ? a.taps : dfssm_taps{};
    const int64_t n_tok = (int64_t)a.n_steps * L;
    const int nbc = 2 * a.G * N;
    for (int i = tid; i < NB * 64; i += F2_T) tv[i] = 0.f;   // entries past the rank stay zero
    if (wg < a.n1) {
        // ====================================================================== role 1
        const int h = wg / a.S, p0 = (wg % a.S) * a.pr, g = h * a.G / a.H;
        const int q = a.q, bc0 = wg * q;
        const bool pad_rows = wg == 0 && T.in_acc != nullptr;
        const int R1t = a.R1 + (pad_rows ? a.npad : 0), nrest = R1t - q;
        const int c1 = tid % CPR1, rg1 = tid / CPR1;
        const int C16_1 = D >> 4;
        const int N4 = N >> 2, nf = a.pr * N4;
        // the lane that completes a B/C row's sum also finishes that row; thread r finishes rest row q + r
        const bool bc_lane = c1 == CPR1 - 1 && rg1 < q;
        const ItemRow m_bc = item_row(a, min(rg1, q - 1), h, p0, bc0);
        const ItemRow m_rest = item_row(a, min(q + tid, R1t - 1), h, p0, bc0);
        // fixed per workgroup: byte offsets (in a layer's in_proj sign matrix) of the 16-byte chunks
        // this lane copies into LDS, block by block (rotated start)
        const int s16 = R1t * CPR1, sblk = (s16 + 63) >> 6, srot = f2_rot(sblk);
        int soff[F2_SBLK];
#pragma unroll
        for (int j = 0; j < F2_SBLK; ++j) {
            const int k = (tid >> 6) + F2_W * j;
            soff[j] = 0;
            if (k < sblk) {
                int kb = k + srot;
                if (kb >= sblk) kb -= sblk;
                const int i = kb * 64 + (tid & 63) < s16 ? kb * 64 + (tid & 63) : 0;
                const int r = i / CPR1, c = i - r * CPR1;
                const ItemRow m = item_row(a, r, h, p0, bc0);
                soff[j] = (m.ch == -2 ? 0 : m.n) * (D >> 3) + c * 16;
            }
        }
        char *sgn1 = wreg;
        char *ldn1 = wreg + f2_round_kb((size_t)R1t * (D >> 3));
        // ---- per-layer loads that do not depend on the token: issued one layer ahead
        RowRegs<NB> rb, rr;
        float4 st[F2_FPT][NB];
        float4 wr[KCH1];
        float dsc1[4], dtb = 0.f, alog = 0.f, Dh = 0.f;
        auto prefetch = [&](int l) {
            const Entry2 Ly = f2_entry(a, l);
            const dfssm_proj &pin = Ly.w.in_proj;
            // register loads first (their waits come at first use), then the direct-to-LDS copies
            load_norm_w<KCH1>(wr, Ly.w.norm_w, D);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) dsc1[jj] = (tid >> 6) + 8 * jj < a.Rin ? gld(pin.lora_dn_scale + (tid >> 6) + 8 * jj) : 0.f;
            if (bc_lane) load_row(rb, m_bc, Ly, a.Rin, a.Cd);
            if (tid < nrest) load_row(rr, m_rest, Ly, a.Rin, a.Cd);
            dtb = gld(Ly.w.dt_bias + h);
            alog = gld(Ly.w.A_log + h);
            Dh = gld(Ly.w.D + h);
#pragma unroll
            for (int i = 0; i < F2_FPT; ++i) {
                const int f = tid + F2_T * i;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    st[i][b] = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (i < a.fpt && f < nf) {
                        const int p = f / N4, n4 = f - p * N4;
                        st[i][b] = gld(reinterpret_cast<const float4 *>(Ly.st.ssm + (((int64_t)b * a.H + h) * P + p0 + p) * N) + n4);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < F2_SBLK; ++j) {
                const int k = (tid >> 6) + F2_W * j;
                if (k < sblk) {
                    int kb = k + srot;
                    if (kb >= sblk) kb -= sblk;
                    __builtin_amdgcn_global_load_lds(pin.sign + soff[j], sgn1 + (size_t)kb * 64 * 16, 16, 0, 0);
                }
            }
            lds_copy_contig(ldn1, reinterpret_cast<const char *>(pin.lora_dn), a.Rin * C16_1);
        };
        prefetch(0);
        for (int t = 0; t < a.n_steps; ++t)
        for (int l = 0; l < L; ++l) {
            const int64_t it = (int64_t)t * L + l;
            const Entry2 Ly = f2_entry(a, l);
            const uint32_t tag = (uint32_t)(it + 1);
            const int lp = l == 0 ? L - 1 : l - 1;
            const int64_t rec = it * B;
            const uint64_t *hx_prev = a.hx + (int64_t)lp * B * D;
            uint64_t *gxl = a.gx + (int64_t)l * B * E;
            uint64_t *bcxl = a.bcx + (int64_t)l * B * nbc;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's direct-to-LDS copies are in
            __syncthreads();
            // ---- residual in, norm, quantizer
            {
                const bool fold = l == 0 && t > 0;   // the previous token's stack output through the final RMSNorm
                f2_prologue<NB, KCH1>(a, hx_prev, D, tag - 1, wr, fold ? a.final_w : nullptr,
                                      fold ? a.y + (int64_t)(t - 1) * B * D : nullptr, sq, spl, sqsum, ssc, red, ired,
                                      wg == 0, fold ? &r0s : nullptr, T.h_in ? T.h_in + rec * D : nullptr,
                                      T.in_u ? T.in_u + rec * D : nullptr, T.in_q ? T.in_q + rec * D : nullptr,
                                      T.in_s ? T.in_s + rec : nullptr);
                if (fold && wg == 0 && tid == 0) st_x(a.rx, tag2(fbits2(r0s), tag));
            }
            // LoRA-down t[j] = L_dn[j] . q (sdot4, factors in LDS)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                int part[4];
                lora_down_sums<KCH1>(ldn1, sq + b * D, D, a.Rin, part);
                if ((tid & 63) == 63) {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int j = (tid >> 6) + 8 * jj;
                        if (j < a.Rin) {
                            tv[b * 64 + j] = dsc1[jj] * ssc[b] * (float)part[jj];
                            if (wg == 0 && T.in_t) T.in_t[(rec + b) * a.Rin + j] = part[jj];
                        }
                    }
                }
            }
            __syncthreads();
            // packed-sign GEMV over the item's rows, pass i taking rows [NG1 * i, NG1 * (i + 1)) (the
            // B/C rows are r < q, all in the first pass of wave 0): the lane that completes a B/C row's
            // sum finishes and publishes it at once, then the other passes run while the B/C words
            // travel. Passes after the second run in reverse group order, so that the few rows of a
            // last, partial pass fall to the last waves rather than to the one finishing the B/C rows,
            // and a wave skips a pass in which none of its groups has a row.
            {
                const int G32 = D >> 5;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    uint4 pl[8];
#pragma unroll
                    for (int p = 0; p < 8; ++p) pl[p] = *reinterpret_cast<const uint4 *>(spl + (b * 8 + p) * G32 + c1 * 4);
                    // every sign chunk is read before the first is used (rows past the item's end are
                    // read clamped and their sums dropped)
                    uint4 bits[F2_MAXI];
                    int pos[F2_MAXI];
#pragma unroll
                    for (int i = 0; i < F2_MAXI; ++i)
                        bits[i] = *reinterpret_cast<const uint4 *>(sgn1 + (size_t)min(f2_pass_row(rg1, i, NG1), R1t - 1) * (D >> 3) + c1 * 16);
                    pos[0] = dpp_group_sum(chunk_pos(bits[0], pl), CPR1);
                    if (bc_lane && rb.m.ch != -2) {
                        const int acc = 2 * pos[0] - sqsum[b];
                        const float act = finish_row(rb, b, acc, ssc[b], tv + b * 64, a.Rin, Ly.st.conv, a.Cd);
                        st_x(bcxl + (int64_t)b * nbc + (rb.m.ch - E), tag2(fbits2(act), tag));
                        if (T.in_acc) T.in_acc[(rec + b) * a.Ninp + rb.m.n] = acc;
                    }
#pragma unroll
                    for (int i = 1; i < F2_MAXI; ++i) {
                        pos[i] = 0;
                        if (__any(f2_pass_row(rg1, i, NG1) < R1t)) pos[i] = dpp_group_sum(chunk_pos(bits[i], pl), CPR1);
                    }
#pragma unroll
                    for (int i = 0; i < F2_MAXI; ++i) {
                        const int r = f2_pass_row(rg1, i, NG1);
                        if (NG1 * i < R1t && c1 == CPR1 - 1 && r >= q && r < R1t) accl[b * F2_ROWS + r - q] = 2 * pos[i] - sqsum[b];
                    }
                }
            }
            __syncthreads();
            // the other rows' epilogue (z, conv step of x, dt), then the group's B and C from the exchange
            if (tid < nrest) {
                const int r = q + tid;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int acc = accl[b * F2_ROWS + tid];
                    if (T.in_acc) T.in_acc[(rec + b) * a.Ninp + rr.m.n] = acc;
                    if (r >= a.R1) continue;   // padding row
                    const float v = finish_row(rr, b, acc, ssc[b], tv + b * 64, a.Rin, Ly.st.conv, a.Cd);
                    if (r < q + a.pr) zl[b * P + (r - q)] = silu_f(v);   // the gate SiLU(z)
                    else if (r < q + 2 * a.pr) xl[b * P + (r - q - a.pr)] = v;
                    else dtl[b] = softplus_f(v + dtb);
                }
            }
            // the group's B and C: gathered by the waves past the epilogue rows (the words were published
            // during the GEMV), while the first waves finish their rows
            const int tbc = tid - F2_BCW * 64;
            if (tbc >= 0 && tbc < (N >> 1)) {
                const int c = tbc < N4 ? 0 : 1, k = (tbc - c * N4) * 4;   // B or C, first of 4 words
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    u32x4 w[2];
                    f2_gather<1>(a, bcxl + (int64_t)b * nbc + c * a.G * N + g * N + k, tag, w);
                    *reinterpret_cast<float4 *>((c ? Cl : Bl) + b * N + k) =
                        make_float4(bitsf2(w[0].x), bitsf2(w[0].z), bitsf2(w[1].x), bitsf2(w[1].z));
                }
            }
            __syncthreads();
            // SSM update + readout, gate, publish g
            const float Ah = -expf(alog);
            float dtv[NB], dAv[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                dtv[b] = dtl[b];
                dAv[b] = expf(dtv[b] * Ah);
            }
            // every LDS operand first (one wait), then the updates; a thread's n4 is the same for
            // all of its state rows (F2_T is a multiple of N / 4)
            const int n4 = tid % N4;
            float xs[F2_FPT][NB], zs[F2_FPT][NB];
            float4 Bv[NB], Cv[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                Bv[b] = *reinterpret_cast<const float4 *>(Bl + b * N + n4 * 4);
                Cv[b] = *reinterpret_cast<const float4 *>(Cl + b * N + n4 * 4);
#pragma unroll
                for (int i = 0; i < F2_FPT; ++i) {
                    const int p = min((tid + F2_T * i) / N4, a.pr - 1);
                    xs[i][b] = xl[b * P + p];
                    zs[i][b] = zl[b * P + p];
                }
            }
#pragma unroll
            for (int i = 0; i < F2_FPT; ++i) {
                const int f = tid + F2_T * i;
                const bool ok = i < a.fpt && f < nf;
                const int p = ok ? f / N4 : 0;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const float dt = dtv[b];
                    const float dA = dAv[b];
                    const float x = xs[i][b];
                    const float dtx = dt * x;
                    const float4 Bn = Bv[b];
                    const float4 Cn = Cv[b];
                    float4 v = st[i][b];
                    v.x = dA * v.x + dtx * Bn.x;
                    v.y = dA * v.y + dtx * Bn.y;
                    v.z = dA * v.z + dtx * Bn.z;
                    v.w = dA * v.w + dtx * Bn.w;
                    st[i][b] = v;
                    float part = ok ? (v.x * Cn.x + v.y * Cn.y) + (v.z * Cn.z + v.w * Cn.w) : 0.f;
                    part = f2_group_sum(part, N4);
                    if (ok && n4 == N4 - 1) gsh[b][p] = (part + Dh * x) * zs[i][b];
                }
            }
            // the gated outputs go out as one store of pr consecutive words (whole cache lines: the
            // item's slot starts on a 256-byte boundary), then the new state
            __syncthreads();
            if (tid < a.pr) {
#pragma unroll
                for (int b = 0; b < NB; ++b) st_x(gxl + (int64_t)b * E + h * P + p0 + tid, tag2(fbits2(gsh[b][tid]), tag));
            }
#pragma unroll
            for (int i = 0; i < F2_FPT; ++i) {
                const int f = tid + F2_T * i;
                if (i < a.fpt && f < nf) {
                    const int p = f / N4;
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                        gst(reinterpret_cast<float4 *>(Ly.st.ssm + (((int64_t)b * a.H + h) * P + p0 + p) * N) + n4, st[i][b]);
                }
            }
            // ---- the next layer's weights and state, while the other role works on this one
            if (it + 1 < n_tok) {
                __syncthreads();   // every wave is done with this layer's LDS
                prefetch(l + 1 < L ? l + 1 : 0);
            }
        }
        // the stack's final RMSNorm of the last token
        if (wg == 0) {
            const uint32_t tag = (uint32_t)n_tok;
            const uint64_t *hl = a.hx + (int64_t)(L - 1) * B * D;
            float *yt = a.y + (int64_t)(a.n_steps - 1) * B * D;
            const int e0 = prologue_elem<KCH1>(0);
            const bool mine = e0 < D;
            for (int b = 0; b < B; ++b) {
                float4 hv[KCH1];
                if (mine) {
                    u32x4 r[2 * KCH1];
                    f2_gather<KCH1>(a, hl + (int64_t)b * D + e0, tag, r);
#pragma unroll
                    for (int i = 0; i < KCH1; ++i)
                        hv[i] = make_float4(bitsf2(r[2 * i].x), bitsf2(r[2 * i].z), bitsf2(r[2 * i + 1].x), bitsf2(r[2 * i + 1].z));
                } else {
#pragma unroll
                    for (int i = 0; i < KCH1; ++i) hv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
                }
                const float r0 = f2_norm_factor<KCH1>(a, hv, D, red + 2 * F2_W);
                if (mine) {
#pragma unroll
                    for (int i = 0; i < KCH1; ++i) {
                        const int e = prologue_elem<KCH1>(i);
                        const float4 w = *reinterpret_cast<const float4 *>(a.final_w + e);
                        *reinterpret_cast<float4 *>(yt + (int64_t)b * D + e) =
                            make_float4((hv[i].x * r0) * w.x, (hv[i].y * r0) * w.y, (hv[i].z * r0) * w.z, (hv[i].w * r0) * w.w);
                    }
                }
                __syncthreads();   // the reduction slots are reused by the next row
            }
        }
        return;
    }
    // ========================================================================== role 2
    const int w2 = wg - a.n1, n_out0 = w2 * a.R2;
    const int R2t = max(0, min(a.R2, D - n_out0));
    const int c2 = tid % CPR2, rg2 = tid / CPR2;
    const int C16_2 = E >> 4;
    const bool tap2 = w2 == 0;
    char *sgn2 = wreg;
    char *ldn2 = wreg + f2_round_kb((size_t)a.R2 * (E >> 3));
    const int on = n_out0 + tid;
    const bool orow = tid < R2t;
    float dsc2[4], ous = 0.f;
    uint32_t oscb = 0;
    int4 oup[F2_UPC];
    float4 wr[KCH2];
    auto prefetch = [&](int l) {
        const Entry2 Ly = f2_entry(a, l);
        const dfssm_proj &pout = Ly.w.out_proj;
        load_norm_w<KCH2>(wr, Ly.w.gnorm_w, E);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) dsc2[jj] = (tid >> 6) + 8 * jj < a.Rout ? gld(pout.lora_dn_scale + (tid >> 6) + 8 * jj) : 0.f;
        if (orow) {
            oscb = gld(pout.row_scale + on);
            ous = gld(pout.lora_up_scale + on);
            load_up(oup, pout.lora_up, a.Rout, on);
        }
        if (R2t > 0)
            lds_copy_contig(sgn2, reinterpret_cast<const char *>(pout.sign + (int64_t)n_out0 * (E >> 3)), R2t * CPR2);
        lds_copy_contig(ldn2, reinterpret_cast<const char *>(pout.lora_dn), a.Rout * C16_2);
    };
    // this workgroup's rows of the residual stream (the token input x0 to begin with)
    float hold[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) hold[b] = orow ? a.x0[(int64_t)b * D + on] : 0.f;
    const float fw = orow ? a.final_w[on] : 0.f;
    prefetch(0);
    for (int t = 0; t < a.n_steps; ++t)
    for (int l = 0; l < L; ++l) {
        const int64_t it = (int64_t)t * L + l;
        const uint32_t tag = (uint32_t)(it + 1);
        const int64_t rec = it * B;
        const uint64_t *gxl = a.gx + (int64_t)l * B * E;
        uint64_t *hxl = a.hx + (int64_t)l * B * D;
        if (l == 0 && t > 0) {
            // the residual input of layer 0 is the previous token's output through the final RMSNorm,
            // whose factor role-1 workgroup 0 publishes (the product is the one its prologue forms)
            uint64_t w = ld_x(a.rx);
            unsigned spins = 0;
            while ((uint32_t)(w >> 32) != tag && spins <= kSpin2) {
                __builtin_amdgcn_s_sleep(kSleep2);
                if (++spins > kSpin2) f2_error(a);
                w = ld_x(a.rx);
            }
            const float r0 = bitsf2((uint32_t)w);
#pragma unroll
            for (int b = 0; b < NB; ++b) hold[b] = (hold[b] * r0) * fw;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's direct-to-LDS copies are in
        __syncthreads();
        f2_prologue<NB, KCH2>(a, gxl, E, tag, wr, nullptr, nullptr, sq, spl, sqsum, ssc, red, ired, tap2, nullptr,
                              nullptr, T.out_u ? T.out_u + rec * E : nullptr, T.out_q ? T.out_q + rec * E : nullptr,
                              T.out_s ? T.out_s + rec : nullptr);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            int part[4];
            lora_down_sums<KCH2>(ldn2, sq + b * E, E, a.Rout, part);
            if ((tid & 63) == 63) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int j = (tid >> 6) + 8 * jj;
                    if (j < a.Rout) {
                        tv[b * 64 + j] = dsc2[jj] * ssc[b] * (float)part[jj];
                        if (tap2 && T.out_t) T.out_t[(rec + b) * a.Rout + j] = part[jj];
                    }
                }
            }
        }
        {
            const int G32 = E >> 5;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                uint4 pl[8];
#pragma unroll
                for (int p = 0; p < 8; ++p) pl[p] = *reinterpret_cast<const uint4 *>(spl + (b * 8 + p) * G32 + c2 * 4);
                uint4 bits[F2_MAXO];
#pragma unroll
                for (int i = 0; i < F2_MAXO; ++i)
                    bits[i] = *reinterpret_cast<const uint4 *>(sgn2 + (size_t)min(rg2 + NG2 * i, max(R2t - 1, 0)) * (E >> 3) + c2 * 16);
#pragma unroll
                for (int i = 0; i < F2_MAXO; ++i) {
                    const int r = rg2 + NG2 * i;
                    const int pos = dpp_group_sum(chunk_pos(bits[i], pl), CPR2);
                    if (c2 == CPR2 - 1 && r < R2t) accl[b * F2_ROWS + r] = 2 * pos - sqsum[b];
                }
            }
        }
        __syncthreads();
        if (orow) {
            const float osc = half_bits_to_float((uint16_t)oscb);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int acc = accl[b * F2_ROWS + tid];
                const float yv = ssc[b] * osc * (float)acc + ous * up_dot2(oup, a.Rout, tv + b * 64);
                if (T.out_acc) T.out_acc[(rec + b) * D + on] = acc;
                hold[b] = hold[b] + yv;
                st_x(hxl + (int64_t)b * D + on, tag2(fbits2(hold[b]), tag));
            }
        }
        if (it + 1 < n_tok) {
            __syncthreads();   // every wave is done with this layer's LDS
            prefetch(l + 1 < L ? l + 1 : 0);
        }
    }
}

__global__ void k_store2(Entry2 *dst, Chunk2 c, int n) {
    if ((int)threadIdx.x < n) dst[threadIdx.x] = c.e[threadIdx.x];
}

// The exchange words are cleared (and seeded) with the same agent-coherent stores the exchange
// itself uses, so no earlier run's tagged words can be observed by the polling loads.
__global__ void k_zero2(uint64_t *p, int64_t n, int *err, uint64_t *rx) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        st_x(p + i, (uint64_t)0);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        st_x(err, 0);
        st_x(rx, (uint64_t)0);
    }
}

__global__ void k_seed2(uint64_t *hx_last, const float *x0, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        st_x(hx_last + i, (uint64_t)__builtin_bit_cast(uint32_t, x0[i]));
}

bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

size_t f2_lds_base(const Shape &s, int nb) {
    const int kmax = s.D > s.E ? s.D : s.E;
    return (size_t)2 * nb * kmax + (size_t)nb * F2_ROWS * 4 + (size_t)nb * 64 * 4 + (size_t)nb * 2 * (s.P + s.N) * 4;
}
size_t f2_round_kb_host(size_t v) { return (v + 1023) & ~(size_t)1023; }
// weight region: max over the two phases of (sign rows + LoRA-down factors), each whole KB
// (also the last token's residual, D floats, for the stack's final RMSNorm)
size_t f2_wreg_bytes(const Shape &s, int R1max, int R2) {
    const size_t p1 = f2_round_kb_host((size_t)R1max * (s.D >> 3)) + f2_round_kb_host((size_t)s.Rin * s.D);
    const size_t p2 = f2_round_kb_host((size_t)R2 * (s.E >> 3)) + f2_round_kb_host((size_t)s.Rout * s.E);
    const size_t m = p1 > p2 ? p1 : p2;
    return m > (size_t)s.D * 4 ? m : (size_t)s.D * 4;
}

// Slices per head (a power of two dividing headdim) for `slots` workgroups, 0 if unsupported.
int f2_slices(const Shape &s, int slots) {
    if (slots < s.H) return 0;
    int S = 1;
    while (S * 2 <= s.P && s.H * S * 2 <= slots && s.P % (S * 2) == 0) S *= 2;
    return S;
}

struct F2Plan {
    int S, pr, q, R1, npad, R2, fpt, n1, n2;
};

bool f2_plan(const Shape &s, int batch, int slots, F2Plan &p) {
    if (batch != 1) return false;
    if (!pow2(s.D) || s.D < 256 || s.D > 4096 || s.E != 2 * s.D) return false;
    if (!pow2(s.Rin) || !pow2(s.Rout) || s.Rin < 8 || s.Rout < 8 || s.Rin > 16 * F2_UPC || s.Rout > 16 * F2_UPC) return false;
    if (s.N % 4 || s.N / 4 > 64 || !pow2(s.N / 4)) return false;
    // half the resident workgroups (at most) for the SSM items, the rest for out_proj row blocks
    p.S = f2_slices(s, slots / 2);
    if (p.S == 0) return false;
    p.n1 = s.H * p.S;
    p.pr = s.P / p.S;
    p.q = (2 * s.G * s.N + p.n1 - 1) / p.n1;
    p.R1 = p.q + 2 * p.pr + 1;
    p.npad = s.Ninp - s.Nin;
    const int CPR1 = s.D >> 7, NG1 = F2_T / CPR1, rest = p.R1 + p.npad - p.q;
    if (p.q > NG1 || p.R1 + p.npad > NG1 * f2_maxi(CPR1) || rest > F2_T || rest > F2_ROWS) return false;
    if ((p.R1 + p.npad) * CPR1 > F2_SBLK * F2_W * 64) return false;
    const int avail = slots - p.n1;
    if (avail < 1) return false;
    p.R2 = (s.D + avail - 1) / avail;
    p.n2 = (s.D + p.R2 - 1) / p.R2;
    if (p.R2 > F2_T || p.R2 > (F2_T / (s.E >> 7)) * f2_maxo(s.E >> 7)) return false;
    const int nf = p.pr * (s.N / 4);
    p.fpt = (nf + F2_T - 1) / F2_T;
    if (p.fpt > F2_FPT) return false;
    return f2_lds_base(s, batch) + f2_wreg_bytes(s, p.R1 + p.npad, p.R2) <= kF2MaxLds;
}


// The grid (one workgroup per slot the plan counted as resident) is the same either way; the
// cooperative API also verifies that the device keeps all of it resident. The ordinary launch is
// for tools that cannot follow cooperative launches: should part of the grid not be resident, the
// bounded waits time out and the call reports DFSSM_STATUS_TIMEOUT.
bool f2_any_tap(const dfssm_taps &t) {
    return t.in_u || t.in_q || t.in_s || t.in_acc || t.in_t || t.out_u || t.out_q || t.out_s || t.out_acc || t.out_t ||
           t.h_in;
}

template <int NB, int KCH1, int KCH2, int CPR1, int CPR2>
hipError_t f2_launch(F2Args &a, const Shape &s, bool cooperative, hipStream_t stream) {
    const size_t lds = f2_lds_base(s, NB) + f2_wreg_bytes(s, a.R1 + a.npad, a.R2);
    void *args[] = {&a};
    const void *fn = f2_any_tap(a.taps) ? reinterpret_cast<const void *>(&k_flow2<NB, KCH1, KCH2, CPR1, CPR2, true>)
                                        : reinterpret_cast<const void *>(&k_flow2<NB, KCH1, KCH2, CPR1, CPR2, false>);
    if (cooperative) return hipLaunchCooperativeKernel(fn, dim3(a.n1 + a.n2), dim3(F2_T), args, lds, stream);
    return hipLaunchKernel(fn, dim3(a.n1 + a.n2), dim3(F2_T), args, lds, stream);
}

template <int NB, int KCH1, int KCH2, int CPR1, int CPR2>
int f2_resident() {
    static std::atomic<int> memo[kMaxDevices2];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices2) return 0;
    int v = memo[dev].load(std::memory_order_relaxed);
    if (v != 0) return v;
    int ncu = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    // with the largest LDS a supported shape may use (registers bound the occupancy to one per CU anyway)
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(&k_flow2<NB, KCH1, KCH2, CPR1, CPR2, true>),
                                                     F2_T, kF2MaxLds) != hipSuccess)
        return 0;
    v = per_cu * ncu;
    memo[dev].store(v, std::memory_order_relaxed);
    return v;
}

// The (D, E = 2D) shapes the kernel is built for: KCH1 = D / 2048, KCH2 = E / 2048 (at least 1),
// CPR = lanes per sign row (D / 128, E / 128). D = 4096 would mean 128 heads, whose items hold more
// rows than the GEMV loop takes (f2_plan).
int f2_slots(const Shape &s, int batch) {
    if (batch != 1 || s.E != 2 * s.D) return 0;
    switch (s.D) {
    case 256: return f2_resident<1, 1, 1, 2, 4>();
    case 512: return f2_resident<1, 1, 1, 4, 8>();
    case 1024: return f2_resident<1, 1, 1, 8, 16>();
    case 2048: return f2_resident<1, 1, 2, 16, 32>();
    default: return 0;
    }
}

hipError_t f2_launch_any(F2Args &a, const Shape &s, bool coop, hipStream_t stream) {
    switch (s.D) {
    case 256: return f2_launch<1, 1, 1, 2, 4>(a, s, coop, stream);
    case 512: return f2_launch<1, 1, 1, 4, 8>(a, s, coop, stream);
    case 1024: return f2_launch<1, 1, 1, 8, 16>(a, s, coop, stream);
    case 2048: return f2_launch<1, 1, 2, 16, 32>(a, s, coop, stream);
    default: return hipErrorInvalidConfiguration;
    }
}

}  // namespace

bool stack2_ok(const Shape &s, int batch) {
    F2Plan p{};
    return f2_plan(s, batch, f2_slots(s, batch), p);
}

size_t stack2_extra_ws_bytes(const Shape &s, int batch, int n_layers) {
    F2Plan p{};
    if (!f2_plan(s, batch, f2_slots(s, batch), p)) return 0;
    const size_t L = n_layers;
    return align_up(L * sizeof(Entry2), 256) + 256 + align_up(L * batch * (size_t)(s.D + s.E + 2 * s.G * s.N) * 8, 256);
}

hipError_t launch_stack2(const Shape &s, const dfssm_layer_weights *layers, const dfssm_layer_state *states, int n_layers,
                         const float *final_w, const float *x0, float *y, int batch, int n_steps, void *extra,
                         const dfssm_taps *taps, bool cooperative, int **err_flag, hipStream_t stream) {
    F2Plan p{};
    if (!f2_plan(s, batch, f2_slots(s, batch), p)) return hipErrorInvalidConfiguration;
    char *q = static_cast<char *>(extra);
    const size_t L = n_layers;
    Entry2 *table = reinterpret_cast<Entry2 *>(q);
    q += align_up(L * sizeof(Entry2), 256);
    int *err = reinterpret_cast<int *>(q);
    q += 256;
    uint64_t *words = reinterpret_cast<uint64_t *>(q);
    const int64_t nwords = (int64_t)L * batch * (s.D + s.E + 2 * s.G * s.N);
    q += align_up((size_t)nwords * 8, 256);
    F2Args a{};
    a.n_layers = n_layers;
    a.n_steps = n_steps;
    a.batch = batch;
    a.D = s.D;
    a.E = s.E;
    a.N = s.N;
    a.P = s.P;
    a.H = s.H;
    a.G = s.G;
    a.Cd = s.Cd;
    a.Nin = s.Nin;
    a.Ninp = s.Ninp;
    a.Rin = s.Rin;
    a.Rout = s.Rout;
    a.eps = s.eps;
    a.S = p.S;
    a.pr = p.pr;
    a.q = p.q;
    a.R1 = p.R1;
    a.npad = p.npad;
    a.R2 = p.R2;
    a.fpt = p.fpt;
    a.n1 = p.n1;
    a.n2 = p.n2;
    a.layers = table;
    a.final_w = final_w;
    a.x0 = x0;
    a.rx = reinterpret_cast<uint64_t *>(err) + 8;
    a.y = y;
    a.hx = words;
    a.gx = words + L * batch * s.D;
    a.bcx = a.gx + L * batch * s.E;
    a.err = err;
    *err_flag = err;
    if (taps) a.taps = *taps;
    hipError_t e;
    for (int l0 = 0; l0 < n_layers; l0 += kTable2) {
        Chunk2 c{};
        const int n = min(kTable2, n_layers - l0);
        for (int i = 0; i < n; ++i) c.e[i] = Entry2{layers[l0 + i], states[l0 + i]};
        k_store2<<<1, 64, 0, stream>>>(table + l0, c, n);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    k_zero2<<<256, 256, 0, stream>>>(words, nwords, err, a.rx);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_seed2<<<64, 256, 0, stream>>>(a.hx + (int64_t)(L - 1) * batch * s.D, x0, (int64_t)batch * s.D);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return f2_launch_any(a, s, cooperative, stream);
}

}  // namespace dfssm
