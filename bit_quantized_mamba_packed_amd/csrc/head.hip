// Tied int8 embedding and LM head ([DF-SSM] §3.3: the embedding quantized to int8 per row;
// Table 1: "Embedding + LM head (tied)", 103 MB at d_model 2048).
//
//   k_embed    x[b] = row_scale[tok[b]] * codes[tok[b]]
//   k_lm_head  per token: (q, s) = the per-token int8 quantizer of y (the stack's normalised
//              output), acc[v] = sum_k codes[v][k] q[k] (int32, sdot4), logits[v] = s*row_scale[v]*acc[v],
//              and each workgroup's best (logit, row) per token
//   k_argmax   per token: the best row over the workgroups (the smallest row among equal logits)
//
// The head streams every byte of the embedding once per call: one wave reads whole rows (64 lanes x
// 16 bytes = 1 KB per load instruction, fully coalesced), each lane keeps the codes of the token for
// its columns in registers, and four rows' loads are in flight before their dot products. It is
// bound by HBM bandwidth (V * d_model bytes per call, whatever the batch up to kHeadTok tokens).
#include "decode_device.h"

namespace dfssm {

namespace {

constexpr int kHeadTok = 8;      // tokens per launch of the head
constexpr int kHeadRows = 4;     // rows per wave in flight
constexpr int kHeadWgs = 2048;   // most workgroups of one launch (partials per token in the workspace)

struct HeadArgs {
    const int8_t *codes;
    const float *row_scale;
    int V, D, nb;           // vocabulary, d_model, tokens in this launch
    const float *y;         // [nb][D]
    float *logits;          // [nb][V] or null
    int32_t *acc_tap;       // [nb][V] or null
    int8_t *q_tap;          // [nb][D] or null
    float *s_tap;           // [nb] or null
    float2 *part;           // [nb][gridDim.x]: (best logit, best row as float bits)
};

typedef int i32x4_nt __attribute__((ext_vector_type(4)));
// A 16-byte load that is not kept in the caches (every row is read once per call).
__device__ __forceinline__ int4 ld_stream16(const int8_t *p) {
    const i32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const i32x4_nt *>(p));
    return make_int4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ int sdot16(const int4 &w, const int4 &q, int acc) {
    acc = __builtin_amdgcn_sdot4(w.x, q.x, acc, false);
    acc = __builtin_amdgcn_sdot4(w.y, q.y, acc, false);
    acc = __builtin_amdgcn_sdot4(w.z, q.z, acc, false);
    return __builtin_amdgcn_sdot4(w.w, q.w, acc, false);
}

// (value, row) pairs: the larger value wins, the smaller row among equal values.
__device__ __forceinline__ bool better(float v, int r, float bv, int br) { return v > bv || (v == bv && r < br); }

template <int NB, int KC>
__global__ __launch_bounds__(kBlock) void k_lm_head(HeadArgs a) {
    __shared__ float bestv[kWaves][NB];
    __shared__ int bestr[kWaves][NB];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int D = a.D, C16 = D >> 4;
    // ---- the per-token quantizer of y (every workgroup forms the same codes; workgroup 0 taps them)
    int4 q[NB][KC];
    float s[NB];
    for (int b = 0; b < NB; ++b) {
        float4 v[KC][4];
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < KC; ++j) {
            const int c = lane + 64 * j;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v[j][k] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (b < a.nb && c < C16) v[j][k] = *reinterpret_cast<const float4 *>(a.y + (int64_t)b * D + c * 16 + 4 * k);
                m = fmaxf(m, fmaxf(fmaxf(fabsf(v[j][k].x), fabsf(v[j][k].y)), fmaxf(fabsf(v[j][k].z), fabsf(v[j][k].w))));
            }
        }
        // every wave holds the whole row (64 lanes x KC chunks): no cross-wave reduction needed
        m = dpp_wave_max(m);
        const float inv = m > 0.f ? 127.0f / m : 0.f;
        s[b] = m > 0.f ? m / 127.0f : 0.f;
#pragma unroll
        for (int j = 0; j < KC; ++j) {
            int w[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int q0 = quant1(v[j][k].x, inv), q1 = quant1(v[j][k].y, inv);
                const int q2 = quant1(v[j][k].z, inv), q3 = quant1(v[j][k].w, inv);
                w[k] = (q0 & 255) | ((q1 & 255) << 8) | ((q2 & 255) << 16) | ((q3 & 255) << 24);
            }
            q[b][j] = make_int4(w[0], w[1], w[2], w[3]);
            const int c = lane + 64 * j;
            if (blockIdx.x == 0 && wave == 0 && b < a.nb && c < C16 && a.q_tap)
                *reinterpret_cast<int4 *>(a.q_tap + (int64_t)b * D + c * 16) = q[b][j];
        }
        if (blockIdx.x == 0 && tid == 0 && b < a.nb && a.s_tap) a.s_tap[b] = s[b];
    }
    // ---- rows: wave gw of the grid takes rows gw, gw + W, ... in groups of kHeadRows
    const int W = gridDim.x * kWaves, gw = blockIdx.x * kWaves + wave;
    float bv[NB];
    int br[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        bv[b] = -__builtin_inff();
        br[b] = 0x7fffffff;
    }
    for (int r0 = gw * kHeadRows; r0 < a.V; r0 += W * kHeadRows) {
        int4 w[kHeadRows][KC];
        float sc[kHeadRows];
#pragma unroll
        for (int i = 0; i < kHeadRows; ++i) {
            const int v = min(r0 + i, a.V - 1);
            sc[i] = a.row_scale[v];
#pragma unroll
            for (int j = 0; j < KC; ++j) {
                const int c = lane + 64 * j;
                w[i][j] = c < C16 ? ld_stream16(a.codes + (int64_t)v * D + c * 16) : make_int4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < kHeadRows; ++i) {
            const int v = r0 + i;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                int acc = 0;
#pragma unroll
                for (int j = 0; j < KC; ++j) acc = sdot16(w[i][j], q[b][j], acc);
                acc = dpp_wave_isum(acc);
                const float lg = s[b] * sc[i] * (float)acc;
                if (v < a.V && b < a.nb) {
                    if (better(lg, v, bv[b], br[b])) {
                        bv[b] = lg;
                        br[b] = v;
                    }
                    if (lane == 0) {
                        if (a.logits) a.logits[(int64_t)b * a.V + v] = lg;
                        if (a.acc_tap) a.acc_tap[(int64_t)b * a.V + v] = acc;
                    }
                }
            }
        }
    }
    // ---- the workgroup's best row per token
    if (lane == 0) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            bestv[wave][b] = bv[b];
            bestr[wave][b] = br[b];
        }
    }
    __syncthreads();
    if (tid < NB && tid < a.nb) {
        float v = bestv[0][tid];
        int r = bestr[0][tid];
        for (int k = 1; k < kWaves; ++k)
            if (better(bestv[k][tid], bestr[k][tid], v, r)) {
                v = bestv[k][tid];
                r = bestr[k][tid];
            }
        a.part[(int64_t)tid * gridDim.x + blockIdx.x] = make_float2(v, __int_as_float(r));
    }
}

__global__ __launch_bounds__(kBlock) void k_argmax(const float2 *part, int nwg, int32_t *out) {
    __shared__ float sv[kBlock];
    __shared__ int sr[kBlock];
    const int b = blockIdx.x, tid = threadIdx.x;
    float v = -__builtin_inff();
    int r = 0x7fffffff;
    for (int i = tid; i < nwg; i += kBlock) {
        const float2 p = part[(int64_t)b * nwg + i];
        if (better(p.x, __float_as_int(p.y), v, r)) {
            v = p.x;
            r = __float_as_int(p.y);
        }
    }
    sv[tid] = v;
    sr[tid] = r;
    __syncthreads();
    for (int st = kBlock / 2; st > 0; st >>= 1) {
        if (tid < st && better(sv[tid + st], sr[tid + st], sv[tid], sr[tid])) {
            sv[tid] = sv[tid + st];
            sr[tid] = sr[tid + st];
        }
        __syncthreads();
    }
    if (tid == 0) out[b] = sr[0];
}

__global__ __launch_bounds__(kBlock) void k_embed(const int8_t *codes, const float *row_scale, int V, int D,
                                                  const int32_t *tokens, float *x) {
    const int b = blockIdx.y;
    const int e = (blockIdx.x * kBlock + threadIdx.x) * 4;
    if (e >= D) return;
    const int t = tokens[b];
    const int v = t < 0 ? 0 : (t >= V ? V - 1 : t);   // ids are validated by the caller; clamp keeps reads in range
    const float sc = row_scale[v];
    const char4 c = *reinterpret_cast<const char4 *>(codes + (int64_t)v * D + e);
    *reinterpret_cast<float4 *>(x + (int64_t)b * D + e) =
        make_float4(sc * (float)c.x, sc * (float)c.y, sc * (float)c.z, sc * (float)c.w);
}

template <int NB>
hipError_t launch_head_nb(const HeadArgs &a, int nwg, hipStream_t stream) {
    // chunks of 16 codes per lane: the next power of two of D / 1024 (lanes past the row end idle)
    if (a.D <= 1024) k_lm_head<NB, 1><<<nwg, kBlock, 0, stream>>>(a);
    else if (a.D <= 2048) k_lm_head<NB, 2><<<nwg, kBlock, 0, stream>>>(a);
    else if (a.D <= 4096) k_lm_head<NB, 4><<<nwg, kBlock, 0, stream>>>(a);
    else if (a.D <= kMaxK) k_lm_head<NB, 8><<<nwg, kBlock, 0, stream>>>(a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

size_t head_ws_bytes(int batch) { return align_up((size_t)batch * kHeadWgs * sizeof(float2), 256); }

hipError_t launch_lm_head(const int8_t *codes, const float *row_scale, int V, int D, const float *y, int batch,
                          float *logits, int32_t *next_tokens, void *ws, const HeadTaps &taps, hipStream_t stream) {
    float2 *part = static_cast<float2 *>(ws);
    // workgroups: every wave takes the same number of kHeadRows-row groups (the last one partial)
    const int per_round = kHeadRows * kWaves;
    const int rounds = (V + per_round * kHeadWgs - 1) / (per_round * kHeadWgs);
    const int nwg = (V + per_round * rounds - 1) / (per_round * rounds);
    hipError_t e;
    for (int b0 = 0; b0 < batch; b0 += kHeadTok) {
        HeadArgs a{};
        a.codes = codes;
        a.row_scale = row_scale;
        a.V = V;
        a.D = D;
        a.nb = min(kHeadTok, batch - b0);
        a.y = y + (int64_t)b0 * D;
        a.logits = logits ? logits + (int64_t)b0 * V : nullptr;
        a.acc_tap = taps.acc ? taps.acc + (int64_t)b0 * V : nullptr;
        a.q_tap = taps.q ? taps.q + (int64_t)b0 * D : nullptr;
        a.s_tap = taps.s ? taps.s + b0 : nullptr;
        a.part = part + (int64_t)b0 * nwg;
        if (a.nb == 1) e = launch_head_nb<1>(a, nwg, stream);
        else if (a.nb == 2) e = launch_head_nb<2>(a, nwg, stream);
        else if (a.nb <= 4) e = launch_head_nb<4>(a, nwg, stream);
        else e = launch_head_nb<8>(a, nwg, stream);
        if (e != hipSuccess) return e;
    }
    if (next_tokens) {
        k_argmax<<<batch, kBlock, 0, stream>>>(part, nwg, next_tokens);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_embed(const int8_t *codes, const float *row_scale, int V, int D, const int32_t *tokens, int batch,
                        float *x, hipStream_t stream) {
    k_embed<<<dim3((D / 4 + kBlock - 1) / kBlock, batch), kBlock, 0, stream>>>(codes, row_scale, V, D, tokens, x);
    return hipGetLastError();
}

}  // namespace dfssm
