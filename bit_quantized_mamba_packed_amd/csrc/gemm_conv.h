// Projection GEMM launch variants. The skinny GEMM (M <= 64 tokens) with the decode conv step in
// its epilogue: the in_proj outputs of one decode step go straight to the consumers of the SSM step
// instead of through the in_proj output buffer and a separate conv-step pass (Mamba-2 layer,
// depthwise causal conv1d of width d_conv = 4 over x | B | C, then SiLU; softplus(dt + dt_bias)).
// And the two in_proj GEMMs of a prefill in one launch.
#pragma once

#include "dfssm_internal.h"

namespace dfssm {

struct ConvEpi {
    int E, Cd, H;                        // z columns [0, E), conv columns [E, E + Cd), dt columns after
    const float *conv_w, *conv_b;        // [Cd][4], [Cd]
    const float *dt_bias;                // [H]
    float *conv_state;                   // [M][Cd][3], shifted by one input
    float *zbuf, *xbc, *dtbuf;           // [M][E], [M][Cd] (after SiLU), [M][H] (after softplus)
};

// Same contract as launch_gemm_pm1 for a.M <= 64 (otherwise hipErrorInvalidValue), except that
// a.y is not written: column n of row m goes to zbuf, through the conv step to xbc (and the conv
// state), or through softplus to dtbuf; columns past E + Cd + H are dropped.
hipError_t launch_gemm_pm1_conv(const GemmArgs &a, const ConvEpi &c, hipStream_t stream);

// Two GEMMs of M > 64 rows over the same codes (the z | x and the B | C | dt rows of in_proj) in one
// launch, each with the contract of launch_gemm_pm1 (no residual). When their launch plans are not
// a wide-tile GEMM and a K-split narrow-tile GEMM it runs them as two launches.
hipError_t launch_gemm_pm1_pair(const GemmArgs &wide, const GemmArgs &narrow, hipStream_t stream);

}  // namespace dfssm
