// Shared device helpers for the gfx950 kernels (wave64, CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

#define WAVE 64

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
    return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

__device__ __forceinline__ float4 ld4(const float* p) {
    return *reinterpret_cast<const float4*>(p);
}
__device__ __forceinline__ void st4(float* p, float4 v) {
    *reinterpret_cast<float4*>(p) = v;
}

// tanh-form GELU and its derivative.  sqrt(2/pi) is the constant of the
// definition; tanh comes from the HIP device math library.
#define GELU_K0 0.7978845608028654f
#define GELU_K1 0.044715f

__device__ __forceinline__ float gelu_f(float x) {
    float u = GELU_K0 * (x + GELU_K1 * x * x * x);
    return 0.5f * x * (1.0f + tanhf(u));
}

__device__ __forceinline__ float gelu_grad_f(float x) {
    float u = GELU_K0 * (x + GELU_K1 * x * x * x);
    float th = tanhf(u);
    float du = GELU_K0 * (1.0f + 3.0f * GELU_K1 * x * x);
    return 0.5f * (1.0f + th) + 0.5f * x * (1.0f - th * th) * du;
}

// Maps a linear workgroup id to a logical tile id so that the 8 XCDs (which
// receive workgroups round-robin) each process one contiguous range of tiles
// and so share operands in their own L2.  Bijective on [0, n).
__device__ __forceinline__ int xcd_remap(int wg, int n) {
    int q = n >> 3;
    return wg < (q << 3) ? (wg & 7) * q + (wg >> 3) : wg;
}
