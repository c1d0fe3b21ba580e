// int8-code x (+-1 scaffold) GEMM with the DF-SSM projection epilogue, on gfx950 MFMA.
//
// For M tokens at once (prefill, batched decode) a projection is a real dense contraction
// (the DF-SSM paper's §4.1 runs it on INT8 tensor cores). Here:
//   C[m][n] = sum_k q[m][k] * bit[n][k]           v_mfma_i32_32x32x32_i8, bits expanded to 0/1 bytes
//   acc     = 2*C - sum_k q[m][k]                  (sgn = 2*bit - 1)
//   y[m][n] = s[m]*row_scale[n]*acc + up_scale[n] * sum_j t'[m][j] * lora_up[n][j]   (Eq. (3))
// with t' = dn_scale * s * t (the LoRA-down result, fp32) split as t' = hi + lo in bf16 so that
// the rank-r product runs on v_mfma_f32_32x32x16_bf16 (lora_up is int8, exact in bf16; the split
// keeps ~16 mantissa bits of t'). An optional residual is added (out_proj) and the int32 acc can
// be written out (taps).
//
// Operand paths. The codes (A, int8 [M][K]) are staged through LDS, shared by the waves of a
// workgroup. The sign bits (B) never touch LDS: each lane loads the 16 bytes (128 k) of its
// column's bit row for the current K step straight into registers and expands the 16 bits each
// MFMA needs into 16 bytes with a multiply-and-mask, so LDS carries only A.
//
// k_gemm_tile (M > 64): workgroup tile 128 x (64*WNB), 4 waves side by side along N, each wave
// 128 x (16*WNB) = 4 x WNB/2 MFMA blocks, so every wave expands only its own columns' sign bits
// (no two waves expand the same bits); K in steps of 128 through double-buffered LDS, one barrier
// per step.
// The ragged last column tile is dispatched first so that the short workgroups do not trail.
// k_gemm_tile_ext (prefill in_proj): the z|x GEMM's 128 x 256 tiles fill exactly one round of
// two workgroups per compute unit at 2,048 tokens; the B|C|dt GEMM (a few 32-column blocks) rides
// along, each block with the first column tiles (one 32 x 32 block per wave, over the whole K), so
// its work needs neither a second round of tiles nor a split K range (k_gemm_tile_pair, which runs
// the narrow GEMM as K-split units ahead of the wide tiles, remains for other shapes).
// k_gemm_skinny (M <= 64): one workgroup of 16 waves (8 when M <= 32: one 32-row block) per 32
// columns (per 64 when that would leave more workgroups than compute units); A and the sign bits go
// through LDS in K chunks of 1024 by direct loads, the waves split the K steps of every chunk, and
// their int32 partial sums meet in LDS (exact, so in any order).
#include <algorithm>

#include "decode_device.h"
#include "gemm_conv.h"

namespace dfssm {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int BM = 128, KT = 128;

__device__ __forceinline__ uint32_t nibble_to_bytes(uint32_t nib) { return (nib * 0x00204081u) & 0x01010101u; }

// 16 sign bits -> 16 bytes of 0/1, byte e = bit e
__device__ __forceinline__ v4i expand16(uint32_t b16) {
    v4i r;
    r.x = (int)nibble_to_bytes(b16 & 15u);
    r.y = (int)nibble_to_bytes((b16 >> 4) & 15u);
    r.z = (int)nibble_to_bytes((b16 >> 8) & 15u);
    r.w = (int)nibble_to_bytes((b16 >> 12) & 15u);
    return r;
}

template <typename T>
__device__ __forceinline__ T *at_bytes(T *base, uint32_t off) {
    return reinterpret_cast<T *>(reinterpret_cast<char *>(base) + off);
}
template <typename T>
__device__ __forceinline__ const T *at_bytes(const T *base, uint32_t off) {
    return reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + off);
}

__device__ __forceinline__ uint32_t u4_get(const uint4 &v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Low-rank term of one 32 x 32 block (rows m0.., columns n0..) on bf16 MFMA from global memory:
// lacc[r] = sum_j t'[m][j] * lora_up[n][j] for this lane's 16 outputs (used by the skinny kernel).
// The operands are loaded first (addresses clamped) and multiplied later (operands past the rank or
// the matrix zeroed), so that their latency can hide behind other work.
// Q = rank / 16 rounded up (at most kMaxRank / 16).
constexpr int kLrQ = kMaxRank / 16;
template <int Q>
struct LowrankOps {
    uint4 h[Q], l[Q];
    uint2 w[Q];
};
template <int Q>
__device__ __forceinline__ LowrankOps<Q> lowrank_load(const GemmArgs &a, int mrow, int ncol, int lane) {
    const int lj = (lane >> 5) * 8;
    const int mc = min(mrow, a.M - 1), nc = min(ncol, a.N - 1);
    LowrankOps<Q> o;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int kr = min(16 * q + lj, a.rank - 8);
        o.h[q] = *reinterpret_cast<const uint4 *>(a.thi + (int64_t)mc * a.rank + kr);
        o.l[q] = *reinterpret_cast<const uint4 *>(a.tlo + (int64_t)mc * a.rank + kr);
        o.w[q] = *reinterpret_cast<const uint2 *>(a.lora_up + (int64_t)nc * a.rank + kr);
    }
    return o;
}
template <int Q>
__device__ __forceinline__ v16f lowrank_mma(const GemmArgs &a, const LowrankOps<Q> &o, int mrow, int ncol, int lane) {
    const int lj = (lane >> 5) * 8;
    v16f lacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) lacc[r] = 0.f;
    const bool rok = mrow < a.M, cok = ncol < a.N;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        if (16 * q >= a.rank) break;
        const bool inr = 16 * q + lj + 8 <= a.rank;
        v8bf ahi = __builtin_bit_cast(v8bf, o.h[q]), alo = __builtin_bit_cast(v8bf, o.l[q]), bup;
        if (!(inr && rok)) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ahi[e] = (__bf16)0.f;
                alo[e] = (__bf16)0.f;
            }
        }
        const uint2 wq = inr && cok ? o.w[q] : make_uint2(0u, 0u);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bup[e] = (__bf16)(float)(int8_t)(wq.x >> (8 * e));
            bup[4 + e] = (__bf16)(float)(int8_t)(wq.y >> (8 * e));
        }
        lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, bup, lacc, 0, 0, 0);
        lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, bup, lacc, 0, 0, 0);
    }
    return lacc;
}

// LDS of the tile kernel. Main loop: A[2][BM][KT] int8 codes (16-byte columns of row r stored at
// column ^ (r & 7), so the fragment reads of 8 consecutive rows hit 8 different bank groups),
// B[2][max(BN, 256)][16] sign bytes; both are written by direct global->LDS loads.
// Epilogue operands: s[BM] f32, qsum[BM] i32, thi/tlo [BM][rank+8] bf16, lora_up [BN][rank+8] int8.
// For rank <= 32 they get their own region behind the main-loop buffers and are loaded before the
// main loop (their latency hides behind it); larger ranks reuse the main-loop buffers afterwards.
constexpr int A_BYTES = BM * KT;
template <int BN>
constexpr int b_bytes() { return (BN > 256 ? BN : 256) * 16; }
constexpr int kCntBytes = 4096;
template <int BN>
constexpr int main_lds() { return 2 * A_BYTES + 2 * b_bytes<BN>(); }
constexpr int kEarlyRank = 32;
template <int BN>
constexpr int epi_lds_bytes(int rank) { return 1024 + 2 * BM * (rank + 8) * 2 + BN * (rank + 8); }
template <int BN>
constexpr int tile_smem() { return main_lds<BN>() + epi_lds_bytes<BN>(kEarlyRank); }
static_assert(epi_lds_bytes<256>(kMaxRank) <= tile_smem<256>() && epi_lds_bytes<128>(kMaxRank) <= tile_smem<128>(),
              "tile LDS");

typedef __attribute__((address_space(3))) char lds_char;

// Direct global->LDS load of 16 bytes per lane: the wave's 64 lanes fill 1 KB of LDS from `lds`
// (wave-uniform) in lane order. Written as inline asm so that the compiler does not make every
// later LDS read wait for it (it cannot tell which LDS bytes the load writes); the waits are
// explicit: dma_barrier before any read of what it wrote, and before it overwrites anything read.
__device__ __forceinline__ void lds_dma16(const void *g, void *lds) {
    const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_char *)lds);
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(base) : "memory");
}

// Workgroup barrier after direct global->LDS loads: those count as vector-memory loads, so every
// wave waits for its own to land (vmcnt) and its LDS reads to finish before the barrier.
__device__ __forceinline__ void dma_barrier() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Stage the epilogue operands of tile (m0, n0) into LDS at `base`.
template <int BN>
__device__ __forceinline__ void stage_epilogue(const GemmArgs &a, char *base, int m0, int n0, int tid) {
    const int rank = a.rank, RS = rank + 8, rc = rank >> 3;
    float *s_l = reinterpret_cast<float *>(base);
    int *q_l = reinterpret_cast<int *>(base + 512);
    __bf16 *th_l = reinterpret_cast<__bf16 *>(base + 1024);
    __bf16 *tl_l = th_l + BM * RS;
    int8_t *u_l = reinterpret_cast<int8_t *>(tl_l + BM * RS);
    // every load first, then every LDS store (the trip counts are fixed so the loads are in flight together)
    constexpr int NT = BM * (kMaxRank / 8) / kBlock, NU = BN * (kMaxRank / 8) / kBlock;
    uint4 h[NT], l[NT];
    uint2 w[NU];
    float sv = 0.f;
    int qv = 0;
    if (tid < BM && m0 + tid < a.M) {
        sv = a.s[m0 + tid];
        qv = a.qsum[m0 + tid];
    }
#pragma unroll
    for (int it = 0; it < NT; ++it) {
        const int idx = tid + it * kBlock, row = idx / rc, c = idx - row * rc, m = m0 + row;
        h[it] = make_uint4(0u, 0u, 0u, 0u);
        l[it] = h[it];
        if (idx < BM * rc && m < a.M) {
            h[it] = *reinterpret_cast<const uint4 *>(a.thi + (int64_t)m * rank + c * 8);
            l[it] = *reinterpret_cast<const uint4 *>(a.tlo + (int64_t)m * rank + c * 8);
        }
    }
#pragma unroll
    for (int it = 0; it < NU; ++it) {
        const int idx = tid + it * kBlock, col = idx / rc, c = idx - col * rc, n = n0 + col;
        w[it] = make_uint2(0u, 0u);
        if (idx < BN * rc && n < a.N) w[it] = *reinterpret_cast<const uint2 *>(a.lora_up + (int64_t)n * rank + c * 8);
    }
    if (tid < BM) {
        s_l[tid] = sv;
        q_l[tid] = qv;
    }
#pragma unroll
    for (int it = 0; it < NT; ++it) {
        const int idx = tid + it * kBlock, row = idx / rc, c = idx - row * rc;
        if (idx < BM * rc) {
            *reinterpret_cast<uint4 *>(th_l + row * RS + c * 8) = h[it];
            *reinterpret_cast<uint4 *>(tl_l + row * RS + c * 8) = l[it];
        }
    }
#pragma unroll
    for (int it = 0; it < NU; ++it) {
        const int idx = tid + it * kBlock, col = idx / rc, c = idx - col * rc;
        if (idx < BN * rc) *reinterpret_cast<uint2 *>(u_l + col * RS + c * 8) = w[it];
    }
}

// two waves per SIMD (<= 256 registers incl. accumulators), so two workgroups share a compute unit
// One workgroup's tile: tile index bid, K slice z of splitk; smem holds tile_smem<64 WNB>() bytes.
// EXT: the tiles of column tiles tn < next also compute the 32 columns [32 tn, 32 tn + 32) of a second
// GEMM `nar` over the same codes (one 32 x 32 block per wave: rows 32 w .. 32 w + 31), so that a
// narrow GEMM rides along the wide one's single round of tiles; its sign bits take a 1 KB LDS slot
// per K buffer after the tile's own LDS (kExtLds).
template <int WNB, bool SPLIT, bool RES, bool EXT = false>
__device__ __forceinline__ void gemm_tile_body(const GemmArgs &a, int ntm, int ntn, int splitk, int bid, int z,
                                               char *smem, int &last_flag, const GemmArgs *nar = nullptr,
                                               int next = 0) {
    constexpr int BN = 64 * WNB, NBW = WNB / 2;   // N blocks of 32 per wave
    constexpr int BDMA = b_bytes<BN>() / 4096;   // 1 KB sign-bit loads per wave and K step
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave;
    const int lr = lane & 31, hsel = lane >> 5;
    // tile order: the ragged last column tile of every row first, then row-fastest
    int tm, tn;
    {
        const bool ragged = (a.N % BN) != 0;
        if (ragged && bid < ntm) {
            tm = bid;
            tn = ntn - 1;
        } else {
            const int idx = ragged ? bid - ntm : bid;
            tm = idx % ntm;
            tn = idx / ntm;
        }
    }
    const int m0 = tm * BM, n0 = tn * BN;
    const int K = a.K, nk = K / KT;
    const bool ext = EXT && tn < next;   // uniform over the workgroup
    const int wvu = __builtin_amdgcn_readfirstlane(wave);
    uint8_t *const bx0 = reinterpret_cast<uint8_t *>(smem) + tile_smem<BN>();
    const uint8_t *xsrc = nullptr;
    if (EXT) xsrc = nar->sign + (int64_t)min(32 * tn + lr, nar->N - 1) * (K >> 3);
    const int kt0 = z * nk / splitk, kt1 = (z + 1) * nk / splitk;
    auto As = [&](int b) { return reinterpret_cast<int8_t *>(smem) + b * A_BYTES; };
    auto Bs = [&](int b) { return reinterpret_cast<uint8_t *>(smem) + 2 * A_BYTES + b * b_bytes<BN>(); };
    // Direct global->LDS loads (16 bytes per lane, 1 KB per wave and instruction, written to LDS in
    // lane order). A: wave w, load i covers rows 8 (4 w + i) .. + 8; lane l fills LDS column l & 7
    // of row l >> 3 with the code bytes of column (l & 7) ^ (l >> 3) (the swizzle). B: wave w, load
    // c covers bit rows 64 (4 c + w) + l. Rows and columns past the matrix are clamped into it:
    // they only feed outputs that are never stored.
    const int8_t *asrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 8 * (4 * wave + i) + (lane >> 3);
        asrc[i] = a.q + (int64_t)min(m0 + row, a.M - 1) * a.ldq + (((lane & 7) ^ (lane >> 3)) << 4);
    }
    const uint8_t *bsrc[BDMA];
#pragma unroll
    for (int c = 0; c < BDMA; ++c) bsrc[c] = a.sign + (int64_t)min(n0 + 64 * (4 * c + wave) + lane, a.N - 1) * (K >> 3);
    auto dma = [&](int buf, int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            lds_dma16(asrc[i] + k0, As(buf) + 1024 * (4 * wave + i));
#pragma unroll
        for (int c = 0; c < BDMA; ++c)
            lds_dma16(bsrc[c] + (k0 >> 3), Bs(buf) + 1024 * (4 * c + wave));
        // ext: lane l writes the 16 bytes of column l & 31 (lanes 32..63 repeat 0..31)
        if (EXT && ext && wvu == 0) lds_dma16(xsrc + (k0 >> 3), bx0 + 1024 * buf);
    };
    v16i acc[4][NBW];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;
    v16i accx;
#pragma unroll
    for (int r = 0; r < 16; ++r) accx[r] = 0;
    dma(0, kt0 * KT);
    const bool early = a.rank <= kEarlyRank;
    char *epi = smem + (early ? main_lds<BN>() : 0);
    if (early) stage_epilogue<BN>(a, epi, m0, n0, tid);
    // per-column scales of the epilogue, loaded now so that no load follows the epilogue's stores
    float sc[NBW], us[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
        const int n = min(n0 + wn * (32 * NBW) + j * 32 + lr, a.N - 1);
        sc[j] = half_bits_to_float(a.row_scale[n]);
        us[j] = a.up_scale[n];
    }
    dma_barrier();
    // one K step: the A fragments of sub-step s + 1 are read from LDS while sub-step s multiplies
    auto step = [&](int cur) {
        // row i * 32 + lr, 16-byte column 2 s + hsel, stored at column (2 s + hsel) ^ (lr & 7)
        const int8_t *abase = As(cur) + lr * KT + ((hsel ^ (lr & 1)) << 4);
        const int sx = (lr >> 1) & 3;
        uint4 bw[NBW];
#pragma unroll
        for (int j = 0; j < NBW; ++j)
            bw[j] = *reinterpret_cast<const uint4 *>(Bs(cur) + (wn * (32 * NBW) + j * 32 + lr) * 16);
        uint4 bwx = make_uint4(0u, 0u, 0u, 0u);
        if (EXT && ext) bwx = *reinterpret_cast<const uint4 *>(bx0 + 1024 * cur + lr * 16);
        v4i af[2][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[0][i] = *reinterpret_cast<const v4i *>(abase + i * 32 * KT + (sx << 5));
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < 3) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    af[(s + 1) & 1][i] = *reinterpret_cast<const v4i *>(abase + i * 32 * KT + (((s + 1) ^ sx) << 5));
            }
            // keep the next sub-step's reads ahead of this sub-step's MFMAs (the scheduler would
            // otherwise sink each read to just before its use)
            __builtin_amdgcn_sched_barrier(0);
            v4i bf[NBW];
#pragma unroll
            for (int j = 0; j < NBW; ++j) bf[j] = expand16((u4_get(bw[j], s) >> (16 * hsel)) & 0xffffu);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NBW; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[s & 1][i], bf[j], acc[i][j], 0, 0, 0);
            if (EXT && ext) {   // the wave's rows 32 w .. 32 w + 31 are A fragment w
                const v4i bfx = expand16((u4_get(bwx, s) >> (16 * hsel)) & 0xffffu);
                switch (wvu) {
                    case 0: accx = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[s & 1][0], bfx, accx, 0, 0, 0); break;
                    case 1: accx = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[s & 1][1], bfx, accx, 0, 0, 0); break;
                    case 2: accx = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[s & 1][2], bfx, accx, 0, 0, 0); break;
                    default: accx = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[s & 1][3], bfx, accx, 0, 0, 0); break;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    for (int kt = kt0; kt < kt1; ++kt) {
        const int cur = (kt - kt0) & 1;
        const bool more = kt + 1 < kt1;
        if (more) dma(cur ^ 1, (kt + 1) * KT);
        step(cur);
        dma_barrier();
    }
    // ---- split K: publish the exact int32 partial sums; the last workgroup of the tile to arrive
    // adds the others' and runs the epilogue (no workgroup ever waits for another)
    if (SPLIT) {
        const int tile = bid;
        const int64_t tsz = (int64_t)BM * BN;
        uint32_t *cnt = static_cast<uint32_t *>(a.scratch);
        int32_t *part = reinterpret_cast<int32_t *>(static_cast<char *>(a.scratch) + kCntBytes);
        int32_t *mine = part + ((int64_t)tile * splitk + z) * tsz;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < NBW; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) st_x(mine + ((((wave * 4 + i) * NBW + j) * 16 + r) * 64 + lane), acc[i][j][r]);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) {
            const uint32_t old = __hip_atomic_fetch_add(cnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last_flag = old == (uint32_t)(splitk - 1);
        }
        __syncthreads();
        if (!last_flag) return;
        if (tid == 0) cnt[tile] = 0u;   // every other arrival is in: the counter is free for the next launch
        for (int z2 = 0; z2 < splitk; ++z2) {
            if (z2 == z) continue;
            const int32_t *o = part + ((int64_t)tile * splitk + z2) * tsz;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NBW; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] += ld_x(o + ((((wave * 4 + i) * NBW + j) * 16 + r) * 64 + lane));
        }
    }
    // ---- epilogue: operands from LDS (staged before the main loop, or now for ranks above 32)
    if (!early) {
        stage_epilogue<BN>(a, epi, m0, n0, tid);
        __syncthreads();
    }
    const int rank = a.rank, RS = rank + 8;
    const float *s_l = reinterpret_cast<const float *>(epi);
    const int *q_l = reinterpret_cast<const int *>(epi + 512);
    const __bf16 *th_l = reinterpret_cast<const __bf16 *>(epi + 1024);
    const __bf16 *tl_l = th_l + BM * RS;
    const int8_t *u_l = reinterpret_cast<const int8_t *>(tl_l + BM * RS);
    const int lj = hsel * 8;
    // Element (local row ml, local column cl) of the tile is at byte ml * ld * 4 + cl * 4 from the
    // tile's corner: uniform 64-bit corners, 32-bit per-lane offsets.
    const bool mfull = m0 + BM <= a.M;
    float *const yt = a.y + (int64_t)m0 * a.ldy + n0;
    const float *const rt = RES ? a.res + (int64_t)m0 * a.ldres + n0 : nullptr;
    int32_t *const tt = a.acc_tap ? a.acc_tap + (int64_t)m0 * a.ldacc + n0 : nullptr;
    constexpr int NIT = 4 * NBW;
    // Residual of block `it` (clamped into the matrix, so every load is in bounds). The loads of
    // block it + 1 are issued before the stores of block it: a load behind stores would make its
    // wait cover the stores as well.
    float rv[2][16];
    auto load_res = [&](int it, float (&dst)[16]) {
        const int clc = min(wn * (32 * NBW) + (it >> 2) * 32 + lr, a.N - 1 - n0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int mlc = min((it & 3) * 32 + 8 * (r >> 2) + 4 * hsel + (r & 3), a.M - 1 - m0);
            dst[r] = *at_bytes(rt, (uint32_t)(mlc * (int)a.ldres + clc) * 4u);
        }
    };
    if (RES) load_res(0, rv[0]);
    // ext block operands, loaded now so that their latency hides behind the main epilogue
    LowrankOps<kLrQ> xops;
    float scx = 0.f, usx = 0.f;
    if (EXT && ext) {
        const int nc = min(32 * tn + lr, nar->N - 1);
        xops = lowrank_load<kLrQ>(*nar, m0 + 32 * wvu + lr, 32 * tn + lr, lane);
        scx = half_bits_to_float(nar->row_scale[nc]);
        usx = nar->up_scale[nc];
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int i = it & 3, j = it >> 2;
        const int rl = i * 32, cl = wn * (32 * NBW) + j * 32 + lr;
        v16f lacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) lacc[r] = 0.f;
        for (int kr = 0; kr < rank; kr += 16) {
            const bool inr = kr + lj + 8 <= rank;
            v8bf ahi, alo, bup;
            uint2 w = make_uint2(0u, 0u);
            if (inr) {
                ahi = *reinterpret_cast<const v8bf *>(th_l + (rl + lr) * RS + kr + lj);
                alo = *reinterpret_cast<const v8bf *>(tl_l + (rl + lr) * RS + kr + lj);
                w = *reinterpret_cast<const uint2 *>(u_l + cl * RS + kr + lj);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    ahi[e] = (__bf16)0.f;
                    alo[e] = (__bf16)0.f;
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                bup[e] = (__bf16)(float)(int8_t)(w.x >> (8 * e));
                bup[4 + e] = (__bf16)(float)(int8_t)(w.y >> (8 * e));
            }
            lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, bup, lacc, 0, 0, 0);
            lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, bup, lacc, 0, 0, 0);
        }
        if (RES && it + 1 < NIT) load_res(it + 1, rv[(it + 1) & 1]);
        if (n0 + cl < a.N) {
            float v[16];
            int accv[16];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int ml = rl + 8 * g + 4 * hsel;
                const float4 sv = *reinterpret_cast<const float4 *>(s_l + ml);
                const int4 qv = *reinterpret_cast<const int4 *>(q_l + ml);
                const float svs[4] = {sv.x, sv.y, sv.z, sv.w};
                const int qvs[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    accv[r] = 2 * acc[i][j][r] - qvs[e];
                    v[r] = svs[e] * sc[j] * (float)accv[r] + us[j] * lacc[r];
                    if (RES) v[r] += rv[it & 1][r];
                }
            }
            // byte offset = lane part ((4 * hsel) rows, column cl) + uniform part (row rl + 8 g + e)
            const uint32_t ly = (uint32_t)(4 * hsel * (int)a.ldy + cl) * 4u;
            const uint32_t lt = (uint32_t)(4 * hsel * (int)a.ldacc + cl) * 4u;
            if (mfull) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    *at_bytes(yt, ly + (uint32_t)((rl + 8 * (r >> 2) + (r & 3)) * (int)a.ldy) * 4u) = v[r];
                if (tt) {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        *at_bytes(tt, lt + (uint32_t)((rl + 8 * (r >> 2) + (r & 3)) * (int)a.ldacc) * 4u) = accv[r];
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int mr = rl + 8 * (r >> 2) + (r & 3);
                    if (m0 + mr + 4 * hsel >= a.M) continue;
                    *at_bytes(yt, ly + (uint32_t)(mr * (int)a.ldy) * 4u) = v[r];
                    if (tt) *at_bytes(tt, lt + (uint32_t)(mr * (int)a.ldacc) * 4u) = accv[r];
                }
            }
        }
    }
    if (EXT && ext) {
        // the wave's ext block: rows m0 + 32 w + 8 (r >> 2) + 4 hsel + (r & 3), column 32 tn + lr of nar
        const GemmArgs &b = *nar;
        const int rl = 32 * wvu, n = 32 * tn + lr;
        const v16f lacc = lowrank_mma<kLrQ>(b, xops, m0 + rl + lr, n, lane);
        if (n < b.N) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ml = rl + 8 * (r >> 2) + 4 * hsel + (r & 3), m = m0 + ml;
                if (m < b.M) {
                    const int accv = 2 * accx[r] - q_l[ml];
                    b.y[(int64_t)m * b.ldy + n] = s_l[ml] * scx * (float)accv + usx * lacc[r];
                    if (b.acc_tap) b.acc_tap[(int64_t)m * b.ldacc + n] = accv;
                }
            }
        }
    }
}

template <int WNB, bool SPLIT, bool RES>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm_tile(GemmArgs a, int ntm,
                                                                                              int ntn, int splitk) {
    __shared__ __align__(16) char smem[tile_smem<64 * WNB>()];
    __shared__ int last_flag;
    gemm_tile_body<WNB, SPLIT, RES>(a, ntm, ntn, splitk, blockIdx.x, blockIdx.y, smem, last_flag);
}

// Two independent GEMMs of one input in one launch: the nsmall K-split units of the narrow one
// (128 x 128 tiles) first, then the wide one's 128 x 256 tiles, so that the short units end early
// and their slots take the wide tiles that did not fit the first round (instead of a second launch
// whose few workgroups leave most compute units idle).
constexpr int kPairLds = tile_smem<256>() > tile_smem<128>() ? tile_smem<256>() : tile_smem<128>();
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm_tile_pair(
    GemmArgs wide, int ntm_w, int ntn_w, GemmArgs narrow, int ntm_n, int ntn_n, int splitk_n) {
    __shared__ __align__(16) char smem[kPairLds];
    __shared__ int last_flag;
    const int tiles_n = ntm_n * ntn_n, nsmall = tiles_n * splitk_n;
    const int bid = blockIdx.x;
    if (bid < nsmall) gemm_tile_body<2, true, false>(narrow, ntm_n, ntn_n, splitk_n, bid % tiles_n, bid / tiles_n, smem, last_flag);
    else gemm_tile_body<4, false, false>(wide, ntm_w, ntn_w, 1, bid - nsmall, 0, smem, last_flag);
}

// The same pair as one round of wide tiles: the narrow GEMM's 32-column blocks ride along the first
// `next` column tiles (EXT), so no tile waits for a second round and no K range is split.
constexpr int kExtLds = 2048;
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm_tile_ext(
    GemmArgs wide, int ntm_w, int ntn_w, GemmArgs narrow, int next) {
    __shared__ __align__(16) char smem[tile_smem<256>() + kExtLds];
    __shared__ int last_flag;
    // the tiles that carry a narrow block (column tiles 0 .. next - 1) come first: tile order is
    // row-fastest
    gemm_tile_body<4, false, false, true>(wide, ntm_w, ntn_w, 1, blockIdx.x, 0, smem, last_flag, &narrow, next);
}

__global__ void k_clear_u32(uint32_t *p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// M <= 64: one workgroup of NW waves per 32 output columns; wave w takes the K steps
// [w nk / NW, (w + 1) nk / NW), all of its loads issued (kSkRun steps at a time) before
// its first MFMA. The int32 partial sums meet in LDS; waves 0 and 1 each finish one 32-row block,
// with their epilogue operands loaded before the reduction barrier.
// NW = 16 waves for M <= 64 (two 32-row blocks), 8 for M <= 32 (one: half the code bytes and MFMAs)
template <int NW>
constexpr int sk_block() { return 64 * NW; }
constexpr int kSkChunk = 1024;   // K bytes of A per LDS chunk (8 K steps of 128)
template <int CB>
constexpr int sk_lds_bytes(int NW) { return 2 * (4 * NW * kSkChunk + CB * 32 * (kSkChunk / 8)); }

// M <= 64 rows (NW = 16 waves, NRB = 2 row blocks of 32) or M <= 32 (NW = 8, NRB = 1), CB blocks
// of 32 columns per workgroup. K runs in chunks of 1024 through two LDS buffers: A[32 NRB][1024]
// (row r's 16-byte column c stored at c ^ (r & 7)) and the sign bits B[CB * 32][128] (column n's
// 16-byte piece p stored at p ^ (n & 7)), both written by direct global->LDS loads that read whole
// rows (coalesced), chunk c + 1 in flight while chunk c is multiplied. Wave w computes output block
// w % (NRB CB) (row block w % NRB, column block (w % (NRB CB)) / NRB) over the K steps kg, kg + KG,
// ... of every chunk (kg = w / (NRB CB), KG = 8 / CB), so the partial sums of only KG waves meet
// per output, in LDS after the last chunk.
template <int CB, bool CONV, int NW>
__global__ __launch_bounds__(sk_block<NW>()) void k_gemm_skinny(GemmArgs a, ConvEpi cv) {
    constexpr int NRB = NW / 8, NBLK = NRB * CB, KG = NW / NBLK, A_BUF = 4 * NW * kSkChunk, B_BUF = CB * 32 * (kSkChunk / 8);
    static_assert(NW == 8 || NW == 16, "8 waves (one row block) or 16 (two)");
    __shared__ __align__(16) char smem[sk_lds_bytes<CB>(NW)];
    // the wave index is uniform: in a scalar register, so are the row pointers and block indices
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31, hsel = lane >> 5;
    const int n0 = blockIdx.x * 32 * CB;
    const int K = a.K, nkt = K / KT, nch = (K + kSkChunk - 1) / kSkChunk;
    auto As = [&](int b) { return reinterpret_cast<int8_t *>(smem) + b * A_BUF; };
    auto Bs = [&](int b) { return reinterpret_cast<uint8_t *>(smem) + 2 * A_BUF + b * B_BUF; };
    // loads of chunk c: A rows wave + NW i (i < 4), lane l -> 16-byte column l ^ (row & 7); B: wave
    // w < 4 CB loads columns 8 w + l / 8, lane l -> piece (l & 7) ^ (column & 7). Rows past M and
    // columns past N read row / column clamped into the matrix (outputs never stored); bytes past K
    // in a short last chunk read clamped addresses (K steps never used).
    const int8_t *arow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) arow[i] = a.q + (int64_t)min(wave + NW * i, a.M - 1) * a.ldq;
    const int asw = 16 * (lane ^ (wave & 7));   // row & 7 == wave & 7 for every row of this wave
    const int bcol = 8 * wave + (lane >> 3);
    const uint8_t *brow = a.sign + (int64_t)min(n0 + bcol, a.N - 1) * (K >> 3);
    const int bsw = 16 * ((lane & 7) ^ (bcol & 7));
    auto dma = [&](int c) {
        const int b = c & 1, k0 = c * kSkChunk;
        const int aoff = min(k0 + asw, K - 16), boff = min((k0 >> 3) + bsw, (K >> 3) - 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) lds_dma16(arow[i] + aoff, As(b) + (wave + NW * i) * kSkChunk);
        if (wave < 4 * CB) lds_dma16(brow + boff, Bs(b) + wave * 1024);
    };
    // epilogue operands of this wave's quarter of a block, loaded before the chunks (so that waiting
    // for them never waits for a chunk) and used after the last one: block fb = wave / 4 (row block
    // fb % NRB, column block fb / NRB), accumulator entries r in [4 rq, 4 rq + 4), rows
    // 8 rq + 4 (lane / 32) + 0..3
    const int nb = a.M > 32 ? 2 : 1;
    const int fb = wave >> 2, fib = fb % NRB, fcb = fb / NRB, rq = wave & 3;
    const bool fin = fb < NBLK && fib < nb;
    const int n = n0 + fcb * 32 + lr;
    float sv[4], rv[4], us = 0.f;
    int qv[4];
    uint16_t scb = 0;   // fp16 bits of the row scale, widened after the chunks (no wait before their loads)
    // the low-rank operands too when the rank is at most 32 (registers), else after the last chunk
    const bool lr_pre = a.rank <= 32;
    LowrankOps<2> lops;
    if (fin) {
        const int nc = min(n, a.N - 1);
        scb = a.row_scale[nc];
        us = a.up_scale[nc];
        const float *rrow = a.res ? a.res : a.s;   // a valid address either way; the value is dropped without res
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int mc = min(fib * 32 + 8 * rq + 4 * hsel + e, a.M - 1);
            sv[e] = a.s[mc];
            qv[e] = a.qsum[mc];
            rv[e] = rrow[a.res ? (int64_t)mc * a.ldres + nc : 0];
        }
        if (lr_pre) lops = lowrank_load<2>(a, fib * 32 + lr, n, lane);
    }
    // conv step operands of this lane's column (kind 0: z, 1: conv, 2: dt, 3: past them)
    int kind = 3;
    float4 cw = make_float4(0.f, 0.f, 0.f, 0.f);
    float cbias = 0.f;
    if (CONV && fin) {
        kind = n < cv.E ? 0 : n < cv.E + cv.Cd ? 1 : n < cv.E + cv.Cd + cv.H ? 2 : 3;
        const int ch = min(max(n - cv.E, 0), cv.Cd - 1), hh = min(max(n - cv.E - cv.Cd, 0), cv.H - 1);
        cw = *reinterpret_cast<const float4 *>(cv.conv_w + (int64_t)ch * kConvTaps);
        cbias = kind == 2 ? cv.dt_bias[hh] : cv.conv_b[ch];
    }
    dma(0);
    if (nch > 1) dma(1);
    constexpr int TPC = 8 / KG;   // K steps per wave and chunk
    const int blk = wave % NBLK, kg = wave / NBLK, rb = blk % NRB, cb = blk / NRB;
    v16i acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0;
    for (int c = 0; c < nch; ++c) {
        if (c == 0 && nch > 1) {
            // chunk 0 has landed once only this wave's loads of chunk 1 (the youngest) are pending
            if (wave < 4 * CB) asm volatile("s_waitcnt vmcnt(5) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        } else {
            dma_barrier();   // chunk c has landed; every wave is done with the buffer chunk c + 1 goes to
            if (c >= 1 && c + 1 < nch) dma(c + 1);
        }
        const int b = c & 1, ntc = min(8, nkt - 8 * c);
        const int8_t *abase = As(b) + (rb * 32 + lr) * kSkChunk;
        const uint8_t *bbase = Bs(b) + (cb * 32 + lr) * (kSkChunk / 8);
        uint4 bw[TPC];
        v4i af[TPC][4];
#pragma unroll
        for (int j = 0; j < TPC; ++j) {
            const int t = min(kg + KG * j, ntc - 1);   // a K step past a short chunk is read clamped, then dropped
#pragma unroll
            for (int s = 0; s < 4; ++s) af[j][s] = *reinterpret_cast<const v4i *>(abase + 16 * (8 * t + ((2 * s + hsel) ^ (lr & 7))));
            bw[j] = *reinterpret_cast<const uint4 *>(bbase + 16 * (t ^ (lr & 7)));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < TPC; ++j) {
            if (kg + KG * j >= ntc) bw[j] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[j][s], expand16((u4_get(bw[j], s) >> (16 * hsel)) & 0xffffu), acc, 0, 0, 0);
        }
    }
    // the conv state of this lane's outputs, loaded while the partial sums meet
    float cst[4][3];
    if (CONV && fin) {
        const int ch = min(max(n - cv.E, 0), cv.Cd - 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int mc = min(fib * 32 + 8 * rq + 4 * hsel + e, a.M - 1);
            const float *sp = cv.conv_state + ((int64_t)mc * cv.Cd + ch) * (kConvTaps - 1);
#pragma unroll
            for (int k = 0; k < kConvTaps - 1; ++k) cst[e][k] = sp[k];
        }
    }
    // the KG partial sums of every output meet in LDS (over the A buffers, once every wave is done)
    __syncthreads();
    int *red = reinterpret_cast<int *>(smem);   // [wave][16][64]
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(wave * 16 + r) * 64 + lane] = acc[r];
    v16f lacc;
    if (fin) {
        if (lr_pre) lacc = lowrank_mma<2>(a, lops, fib * 32 + lr, n, lane);
        else lacc = lowrank_mma<kLrQ>(a, lowrank_load<kLrQ>(a, fib * 32 + lr, n, lane), fib * 32 + lr, n, lane);
    }
    __syncthreads();
    if (!fin || n >= a.N) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = 4 * rq + e, m = fib * 32 + 8 * rq + 4 * hsel + e;
        if (m >= a.M) continue;
        int t = 0;
#pragma unroll
        for (int g = 0; g < KG; ++g) t += red[((g * NBLK + fb) * 16 + r) * 64 + lane];
        const int accv = 2 * t - qv[e];
        const float sc = half_bits_to_float(scb);
        float v = sv[e] * sc * (float)accv + us * lacc[r];
        if (a.res) v += rv[e];
        if (a.acc_tap) a.acc_tap[(int64_t)m * a.ldacc + n] = accv;
        if (!CONV) {
            a.y[(int64_t)m * a.ldy + n] = v;
        } else if (kind == 0) {
            cv.zbuf[(int64_t)m * cv.E + n] = v;
        } else if (kind == 1) {
            const int ch = n - cv.E;
            const float pre = cbias + cw.x * cst[e][0] + cw.y * cst[e][1] + cw.z * cst[e][2] + cw.w * v;
            float *sp = cv.conv_state + ((int64_t)m * cv.Cd + ch) * (kConvTaps - 1);
            sp[0] = cst[e][1];
            sp[1] = cst[e][2];
            sp[2] = v;
            cv.xbc[(int64_t)m * cv.Cd + ch] = silu_f(pre);
        } else if (kind == 2) {
            cv.dtbuf[(int64_t)m * cv.H + (n - cv.E - cv.Cd)] = softplus_f(v + cbias);
        }
    }
}

}  // namespace

namespace {

// Launch plan of the tile kernel: column-tile width, tile count and K split (only with <= 256 tiles,
// so the arrival counters fit the fixed kCntBytes block at the start of the scratch).
struct GemmPlan {
    int wnb, ntm, ntn, splitk;
};

GemmPlan plan_gemm(int M, int N, int K) {
    GemmPlan p{};
    p.ntm = (M + BM - 1) / BM;
    const int nk = K / KT;
    const int64_t wide = (int64_t)p.ntm * ((N + 255) / 256);
    // wide tiles (128 x 256) when they still give two workgroups per compute unit
    if (wide >= 512) {
        p.wnb = 4;
        p.ntn = (N + 255) / 256;
        p.splitk = 1;
        return p;
    }
    p.wnb = 2;
    p.ntn = (N + 127) / 128;
    const int64_t tiles = (int64_t)p.ntm * p.ntn;
    p.splitk = 1;
    // K split only below one tile per compute unit: at 256 tiles (the 2,048-token out_proj) the
    // split's partial-sum exchange costs more than the second workgroup per compute unit gains
    // (32.9 -> 30.8 us without it)
    if (tiles < 256)
        while (tiles * p.splitk * 2 <= 512 && p.splitk * 2 <= nk && p.splitk < 4) p.splitk *= 2;
    return p;
}

}  // namespace

int gemm_counter_words(int M, int N, int K) {
    if (M <= 64) return 0;
    const GemmPlan p = plan_gemm(M, N, K);
    return p.splitk > 1 ? p.ntm * p.ntn : 0;
}

size_t gemm_scratch_bytes(int M, int N, int K) {
    if (M <= 64) return 0;
    const GemmPlan p = plan_gemm(M, N, K);
    if (p.splitk == 1) return 0;
    const size_t tiles = (size_t)p.ntm * p.ntn;
    return kCntBytes + tiles * p.splitk * BM * (64 * p.wnb) * 4;
}

hipError_t launch_gemm_pm1(const GemmArgs &a, hipStream_t stream) {
    if (a.K % KT || a.rank % 8 || a.rank <= 0 || a.rank > kMaxRank || a.M <= 0 || a.N <= 0) return hipErrorInvalidValue;
    // the tile kernel addresses its outputs with 32-bit byte offsets from the tile corner
    const int64_t ldmax = std::max(a.ldy, std::max(a.res ? a.ldres : 0, a.acc_tap ? a.ldacc : 0));
    if (ldmax > (int64_t)1 << 22) return hipErrorInvalidValue;
    if (a.M <= 64) {
        // two column blocks per workgroup when one each would not fit one workgroup per compute unit
        const int ncb = (a.N + 31) / 32;
        if (a.M <= 32) {
            if (ncb > 256) k_gemm_skinny<2, false, 8><<<(ncb + 1) / 2, sk_block<8>(), 0, stream>>>(a, ConvEpi{});
            else k_gemm_skinny<1, false, 8><<<ncb, sk_block<8>(), 0, stream>>>(a, ConvEpi{});
        } else {
            if (ncb > 256) k_gemm_skinny<2, false, 16><<<(ncb + 1) / 2, sk_block<16>(), 0, stream>>>(a, ConvEpi{});
            else k_gemm_skinny<1, false, 16><<<ncb, sk_block<16>(), 0, stream>>>(a, ConvEpi{});
        }
        return hipGetLastError();
    }
    const GemmPlan p = plan_gemm(a.M, a.N, a.K);
    const int tiles = p.ntm * p.ntn;
    if (p.splitk > 1) {
        if (!a.scratch || tiles * 4 > kCntBytes) return hipErrorInvalidValue;
        if (!a.counters_zeroed)
            k_clear_u32<<<(tiles + kBlock - 1) / kBlock, kBlock, 0, stream>>>(static_cast<uint32_t *>(a.scratch), tiles);
    }
    const dim3 grid(tiles, p.splitk);
    const bool res = a.res != nullptr;
    if (p.wnb == 4) {
        if (res) k_gemm_tile<4, false, true><<<grid, kBlock, 0, stream>>>(a, p.ntm, p.ntn, 1);
        else k_gemm_tile<4, false, false><<<grid, kBlock, 0, stream>>>(a, p.ntm, p.ntn, 1);
    } else if (p.splitk > 1) {
        if (res) k_gemm_tile<2, true, true><<<grid, kBlock, 0, stream>>>(a, p.ntm, p.ntn, p.splitk);
        else k_gemm_tile<2, true, false><<<grid, kBlock, 0, stream>>>(a, p.ntm, p.ntn, p.splitk);
    } else {
        if (res) k_gemm_tile<2, false, true><<<grid, kBlock, 0, stream>>>(a, p.ntm, p.ntn, 1);
        else k_gemm_tile<2, false, false><<<grid, kBlock, 0, stream>>>(a, p.ntm, p.ntn, 1);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_pm1_conv(const GemmArgs &a, const ConvEpi &c, hipStream_t stream) {
    if (a.K % KT || a.rank % 8 || a.rank <= 0 || a.rank > kMaxRank || a.M <= 0 || a.M > 64 || a.N <= 0)
        return hipErrorInvalidValue;
    if (c.E <= 0 || c.Cd <= 0 || c.H <= 0 || c.E + c.Cd + c.H > a.N) return hipErrorInvalidValue;
    const int ncb = (a.N + 31) / 32;
    if (a.M <= 32) {
        if (ncb > 256) k_gemm_skinny<2, true, 8><<<(ncb + 1) / 2, sk_block<8>(), 0, stream>>>(a, c);
        else k_gemm_skinny<1, true, 8><<<ncb, sk_block<8>(), 0, stream>>>(a, c);
    } else {
        if (ncb > 256) k_gemm_skinny<2, true, 16><<<(ncb + 1) / 2, sk_block<16>(), 0, stream>>>(a, c);
        else k_gemm_skinny<1, true, 16><<<ncb, sk_block<16>(), 0, stream>>>(a, c);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_pm1_pair(const GemmArgs &wide, const GemmArgs &narrow, hipStream_t stream) {
    for (const GemmArgs *a : {&wide, &narrow}) {
        if (a->K % KT || a->rank % 8 || a->rank <= 0 || a->rank > kMaxRank || a->M <= 64 || a->N <= 0 || a->res)
            return hipErrorInvalidValue;
        const int64_t ldmax = std::max(a->ldy, a->acc_tap ? a->ldacc : (int64_t)0);
        if (ldmax > (int64_t)1 << 22) return hipErrorInvalidValue;
    }
    const GemmPlan pw = plan_gemm(wide.M, wide.N, wide.K), pn = plan_gemm(narrow.M, narrow.N, narrow.K);
    if (pw.wnb != 4 || pw.splitk != 1 || pn.wnb != 2 || pn.splitk < 2) {   // not the shapes the pair serves
        hipError_t e = launch_gemm_pm1(wide, stream);
        return e != hipSuccess ? e : launch_gemm_pm1(narrow, stream);
    }
    const int next = (narrow.N + 31) / 32;
    if (narrow.M == wide.M && narrow.K == wide.K && narrow.rank == wide.rank && wide.N % 256 == 0 && next <= pw.ntn) {
        k_gemm_tile_ext<<<pw.ntm * pw.ntn, kBlock, 0, stream>>>(wide, pw.ntm, pw.ntn, narrow, next);
        return hipGetLastError();
    }
    const int tiles_n = pn.ntm * pn.ntn;
    if (!narrow.scratch || tiles_n * 4 > kCntBytes) return hipErrorInvalidValue;
    if (!narrow.counters_zeroed)
        k_clear_u32<<<(tiles_n + kBlock - 1) / kBlock, kBlock, 0, stream>>>(static_cast<uint32_t *>(narrow.scratch), tiles_n);
    const int grid = tiles_n * pn.splitk + pw.ntm * pw.ntn;
    k_gemm_tile_pair<<<grid, kBlock, 0, stream>>>(wide, pw.ntm, pw.ntn, narrow, pn.ntm, pn.ntn, pn.splitk);
    return hipGetLastError();
}

}  // namespace dfssm
