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

// Streaming (non-temporal) forms for single-use sweeps over large arrays.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld4_nt(const float* p) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st4_nt(float* p, float4 v) {
    const f32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<f32x4_t*>(p));
}

// tanh-form GELU and its derivative:
//   GELU(x) = 0.5 x (1 + tanh(u)),  u = sqrt(2/pi) (x + 0.044715 x^3).
// Since (1 + tanh(u)) / 2 = 1 / (1 + e^(-2u)) = s, GELU(x) = x s, and
//   GELU'(x) = s + x s (1 - s) du2,  du2 = d(2u)/dx = 2 sqrt(2/pi) (1 + 3 * 0.044715 x^2).
// e^(-2u) = 2^z with z = x (A + B x^2), A = -2 sqrt(2/pi) log2(e), B = 0.044715 A.
// One hardware base-2 exponential and one reciprocal per element (a few
// fp32 ulps), half the other arithmetic of the tanh form: these run in the
// matmul epilogues.  Both ends saturate cleanly: x -> -inf gives 2^z = inf,
// s = 0; x -> +inf gives s = 1.
#define GELU_A (-2.302208198144325f)
#define GELU_B (-0.1029432395800235f)
#define GELU_D0 1.5957691216057308f   // 2 sqrt(2/pi)
#define GELU_D1 0.21406444881780076f  // 2 sqrt(2/pi) * 3 * 0.044715

__device__ __forceinline__ float gelu_sigmoid(float x, float x2) {
    const float z = x * fmaf(GELU_B, x2, GELU_A);
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z));
}

__device__ __forceinline__ float gelu_f(float x) { return x * gelu_sigmoid(x, x * x); }

__device__ __forceinline__ float gelu_grad_f(float x) {
    const float x2 = x * x;
    const float s = gelu_sigmoid(x, x2);
    return fmaf(x * fmaf(GELU_D1, x2, GELU_D0), fmaf(-s, s, s), s);
}

// Maps a linear workgroup id to a logical tile id so that the 8 XCDs (which
// receive workgroups round-robin) each process one contiguous range of tiles
// and so share operands in their own L2.  Bijective on [0, n).
__device__ __forceinline__ int xcd_remap(int wg, int n) {
    int q = n >> 3;
    return wg < (q << 3) ? (wg & 7) * q + (wg >> 3) : wg;
}

// Tile and K-split index of a split-K workgroup (grid: tiles x 1 x nz).
// With nz a multiple of 8 each XCD takes whole K chunks: XCD x runs every
// tile of chunks x, x + 8, ... in tile order, so the workgroups resident on
// one XCD read the same A and B chunk panels through its L2.  Otherwise the
// tiles of each chunk are spread by xcd_remap.  Bijective on both forms.
__device__ __forceinline__ void split_remap(int bx, int bz, int tiles, int nz, int& tile,
                                            int& kz) {
    if (nz > 1 && (nz & 7) == 0) {
        const int lin = bx + tiles * bz;  // dispatch order
        const int j = lin >> 3;
        kz = (lin & 7) + 8 * (j / tiles);
        tile = j - (j / tiles) * tiles;
    } else {
        kz = bz;
        tile = xcd_remap(bx, tiles);
    }
}

// ---- 16-bit storage -------------------------------------------------------
#include "dtype.h"

// ---- bf16 storage ----------------------------------------------------------
// bf16 is kept as raw uint16_t bits: the top half of an IEEE fp32.  Rounding
// from fp32 is to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Loads and stores of four consecutive activations as fp32, whatever the
// storage type (float or bf16 bits).
template <class T>
struct Act;

template <>
struct Act<float> {
    static __device__ __forceinline__ float4 ld(const float* p) { return ld4(p); }
    static __device__ __forceinline__ void st(float* p, float4 v) { st4(p, v); }
    static __device__ __forceinline__ float ld1(const float* p) { return *p; }
    static __device__ __forceinline__ void st1(float* p, float v) { *p = v; }
};

template <>
struct Act<uint16_t> {
    static __device__ __forceinline__ float4 ld(const uint16_t* p) {
        const uint2 u = *reinterpret_cast<const uint2*>(p);
        return make_float4(bf2f(u.x & 0xffffu), bf2f(u.x >> 16), bf2f(u.y & 0xffffu),
                           bf2f(u.y >> 16));
    }
    static __device__ __forceinline__ void st(uint16_t* p, float4 v) {
        *reinterpret_cast<uint2*>(p) = make_uint2(f2bf(v.x) | ((uint32_t)f2bf(v.y) << 16),
                                                  f2bf(v.z) | ((uint32_t)f2bf(v.w) << 16));
    }
    static __device__ __forceinline__ float ld1(const uint16_t* p) { return bf2f(*p); }
    static __device__ __forceinline__ void st1(uint16_t* p, float v) { *p = f2bf(v); }
};

// IEEE fp16 storage; conversion from fp32 rounds to nearest, ties to even.
template <>
struct Act<_Float16> {
    static __device__ __forceinline__ float4 ld(const _Float16* p) {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        const h4 u = *reinterpret_cast<const h4*>(p);
        return make_float4((float)u[0], (float)u[1], (float)u[2], (float)u[3]);
    }
    static __device__ __forceinline__ void st(_Float16* p, float4 v) {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        h4 u = {(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
        *reinterpret_cast<h4*>(p) = u;
    }
    static __device__ __forceinline__ float ld1(const _Float16* p) { return (float)*p; }
    static __device__ __forceinline__ void st1(_Float16* p, float v) { *p = (_Float16)v; }
};

// The same four-element accesses through a buffer resource: the row base
// and byte size sit in scalar registers and each lane supplies one 32-bit
// byte offset (plus a uniform one), so a thread's many loads of one row
// share a single address register.  Callers keep every access inside the
// size they give the resource.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

// Cache policy of the streaming buffer accesses below: non-temporal (the
// data is touched once).  On the vocabulary softmax (3.3 GB read, 3.3 GB
// written) it measured 1182 against 1293 us with the default policy.
constexpr int BUF_NT = 2;

template <class T>
struct BufAct;

template <>
struct BufAct<float> {
    static constexpr int BYTES = 16;  // four elements
    static __device__ __forceinline__ float4 ld(__amdgpu_buffer_rsrc_t r, int vo, int so) {
        const u32x4_t u = __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, BUF_NT);
        return make_float4(__uint_as_float(u[0]), __uint_as_float(u[1]), __uint_as_float(u[2]),
                           __uint_as_float(u[3]));
    }
    static __device__ __forceinline__ void st(__amdgpu_buffer_rsrc_t r, int vo, int so, float4 v) {
        const u32x4_t u = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                           __float_as_uint(v.w)};
        __builtin_amdgcn_raw_buffer_store_b128(u, r, vo, so, BUF_NT);
    }
};

template <>
struct BufAct<uint16_t> {
    static constexpr int BYTES = 8;
    static __device__ __forceinline__ float4 ld(__amdgpu_buffer_rsrc_t r, int vo, int so) {
        const u32x2_t u = __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, BUF_NT);
        return make_float4(__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u),
                           __uint_as_float(u[1] << 16), __uint_as_float(u[1] & 0xffff0000u));
    }
    static __device__ __forceinline__ void st(__amdgpu_buffer_rsrc_t r, int vo, int so, float4 v) {
        const u32x2_t u = {f2bf(v.x) | ((uint32_t)f2bf(v.y) << 16),
                           f2bf(v.z) | ((uint32_t)f2bf(v.w) << 16)};
        __builtin_amdgcn_raw_buffer_store_b64(u, r, vo, so, BUF_NT);
    }
};

template <>
struct BufAct<_Float16> {
    static constexpr int BYTES = 8;
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    static __device__ __forceinline__ float4 ld(__amdgpu_buffer_rsrc_t r, int vo, int so) {
        const h4 u = __builtin_bit_cast(h4, __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, BUF_NT));
        return make_float4((float)u[0], (float)u[1], (float)u[2], (float)u[3]);
    }
    static __device__ __forceinline__ void st(__amdgpu_buffer_rsrc_t r, int vo, int so, float4 v) {
        const h4 u = {(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, u), r, vo, so, BUF_NT);
    }
};

// The 16-bit formats as matrix-core operands: bits <-> fp32, a packed pair,
// and the 32x32x16 MFMA with fp32 accumulation.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

struct HBF16 {
    static constexpr int dt = DT_BF16;
    static __device__ __forceinline__ float f(uint32_t h) { return bf2f(h & 0xFFFFu); }
    static __device__ __forceinline__ uint16_t h(float x) { return f2bf(x); }
    static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
    static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
    static __device__ __forceinline__ uint32_t pk(float a, float b) {
        const f32x2_t v = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    }
    static __device__ __forceinline__ floatx16 mma(uint4 a, uint4 b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
};

struct HF16 {
    static constexpr int dt = DT_F16;
    static __device__ __forceinline__ float f(uint32_t h) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xFFFFu));
    }
    static __device__ __forceinline__ uint16_t h(float x) {
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    }
    static __device__ __forceinline__ float lo(uint32_t w) { return f(w); }
    static __device__ __forceinline__ float hi(uint32_t w) { return f(w >> 16); }
    static __device__ __forceinline__ uint32_t pk(float a, float b) {
        const f32x2_t v = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
    }
    static __device__ __forceinline__ floatx16 mma(uint4 a, uint4 b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
};

// Runs f with a value of the storage type of dt (float, bf16 bits or fp16).
template <class F>
inline hipError_t by_dt(int dt, F&& f) {
    switch (dt) {
        case DT_BF16: return f(uint16_t{});
        case DT_F16: return f(_Float16{});
        default: return f(float{});
    }
}
