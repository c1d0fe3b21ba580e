// Sustained MFMA rate of the part: every wave of a full grid (1 or 2 workgroups of 4 waves per compute
// unit) issues iters x 8 independent MFMAs on register operands, no memory traffic; the printed
// TOP/s is the ceiling the GEMM and SSD kernels are compared against, beside the published peak.
// Build and run (standalone, not part of the library):
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops mfma_rate.hip -o mfma_rate
#include <hip/hip_runtime.h>
#include <cstdio>
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
template <int KIND>
__global__ __launch_bounds__(256) void k_rate(int iters, int *out) {
    const int lane = threadIdx.x & 63;
    v4i a = {lane, lane + 1, lane + 2, lane + 3}, b = {lane * 3, 7, 9, lane};
    v8bf ab, bb;
    for (int e = 0; e < 8; ++e) { ab[e] = (__bf16)(float)(lane + e); bb[e] = (__bf16)(float)(e - lane); }
    v16i acc[8];
    v16f facc[8];
    for (int j = 0; j < 8; ++j) for (int r = 0; r < 16; ++r) { acc[j][r] = 0; facc[j][r] = 0.f; }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (KIND == 0) acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[j], 0, 0, 0);
            else facc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, bb, facc[j], 0, 0, 0);
        }
    }
    int s = 0;
    for (int j = 0; j < 8; ++j) for (int r = 0; r < 16; ++r) s += acc[j][r] + (int)facc[j][r];
    if (s == 0x12345) out[threadIdx.x] = s;
}
int main() {
    int *out; hipMalloc(&out, 4096);
    hipEvent_t e0, e1; hipEventCreate(&e0); hipEventCreate(&e1);
    const int iters = 2000;
    for (int kind = 0; kind < 2; ++kind)
        for (int wps = 1; wps <= 2; ++wps) {   // workgroups (of 4 waves) per CU
            const int grid = 256 * wps;
            for (int rep = 0; rep < 2; ++rep) {
                hipEventRecord(e0);
                if (kind == 0) k_rate<0><<<grid, 256>>>(iters, out); else k_rate<1><<<grid, 256>>>(iters, out);
                hipEventRecord(e1);
                hipEventSynchronize(e1);
                float ms; hipEventElapsedTime(&ms, e0, e1);
                const double mfmas = (double)grid * 4 * iters * 8;
                const double ops = mfmas * (kind == 0 ? 65536.0 : 32768.0);
                if (rep) printf("%s  %d WG/CU: %.3f ms  %.1f cycles/MFMA/SIMD at 2.4 GHz  %.0f TOP/s\n", kind ? "bf16 32x32x16" : "i8 32x32x32 ", wps, ms,
                                ms * 1e-3 * 2.4e9 / (mfmas / 1024), ops / (ms * 1e-3) / 1e12);
            }
        }
    return 0;
}
