// dev_common.h -- small device helpers shared by the gconv kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace gconv {

constexpr int kWave = 64;

// Butterfly sum over all 64 lanes of a wavefront; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Butterfly sum over one 32-lane half of a wavefront (lanes 0-31 or 32-63).
__device__ __forceinline__ float half_wave_sum(float v) {
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Logistic function 1/(1+exp(-t)) (the sigmoid of the conv + bias + scale
// + sigmoid + GroupNorm chain), with the hardware base-2 exponential and
// reciprocal: exp(-t) = 2^(-t*log2(e)).  Both are accurate to about one ulp;
// the result is within a few ulp of the exact logistic, far inside what the
// GroupNorm output tolerance allows after the 1/sigma amplification.  Large
// |t| saturates correctly: 2^(+big) = inf gives 0, 2^(-big) = 0 gives 1.
__device__ __forceinline__ float sigmoidf(float t) {
    const float e = __builtin_amdgcn_exp2f(-t * 1.44269504088896340736f);
    return __builtin_amdgcn_rcpf(1.0f + e);
}

// Sum over a 256-thread block in a fixed order: every thread gets the total.
// `scratch` holds at least 4 floats of LDS; the call contains barriers and
// must be reached by every thread of the block.
__device__ __forceinline__ float block256_sum(float v, float *scratch) {
    v = wave_sum(v);
    const int wave = threadIdx.x >> 6;
    __syncthreads();  // scratch may still be read from a previous call
    if ((threadIdx.x & 63) == 0) scratch[wave] = v;
    __syncthreads();
    return (scratch[0] + scratch[1]) + (scratch[2] + scratch[3]);
}

}  // namespace gconv
