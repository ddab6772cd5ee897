// LayerNorm forward and backward (the layer the llm.c articles walk through
// as the worked example: yinghuohong.cn article "OpenAI创始大神手搓千行C代码
// 训练GPT", section "脚动完成每一个层前向/反向流传"; ujoy.net article "徒手用
// 1000 行 C 语言实现", section "用C语言实现LLM").
//
//   forward:  y = (x - mean) * rstd * w + b,  rstd = 1/sqrt(var + 1e-5),
//             biased variance, mean taken first and variance second;
//   backward: with xhat = (x - mean) rstd and g = dy w,
//             dx = rstd (g - mean(g) - xhat mean(g xhat)),
//             dw += sum_rows dy xhat,  db += sum_rows dy.
//
// The backward can also sum its own output over rows: the residual-stream
// gradient it leaves behind is the output gradient of the projection whose
// result was added into that stream, so that column sum is the projection's
// bias gradient, taken here without reading the stream again.
//
// One wave per row; the row stays in registers between the two reductions,
// so x is read once.  The backward's column sums are deterministic: each
// workgroup reduces its rows to one partial row, a second kernel adds the
// partial rows in order.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

constexpr float LN_EPS = 1e-5f;

// The value a store of v leaves in memory, back in fp32.
template <class T>
__device__ __forceinline__ float4 as_stored(float4 v);
template <>
__device__ __forceinline__ float4 as_stored<float>(float4 v) {
    return v;
}
template <>
__device__ __forceinline__ float4 as_stored<uint16_t>(float4 v) {
    return make_float4(bf2f(f2bf(v.x)), bf2f(f2bf(v.y)), bf2f(f2bf(v.z)), bf2f(f2bf(v.w)));
}
template <>
__device__ __forceinline__ float4 as_stored<_Float16>(float4 v) {
    return make_float4((float)(_Float16)v.x, (float)(_Float16)v.y, (float)(_Float16)v.z,
                       (float)(_Float16)v.w);
}

template <int NCH, class T>  // float4 chunks per lane: C <= 256 * NCH
__global__ __launch_bounds__(256) void ln_fwd_kernel(T* __restrict__ out,
                                                     float* __restrict__ mean,
                                                     float* __restrict__ rstd,
                                                     const T* __restrict__ inp,
                                                     const float* __restrict__ w,
                                                     const float* __restrict__ b, int N,
                                                     int C) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= N) return;
    const int C4 = C >> 2;
    const T* x = inp + (int64_t)row * C;
    float4 v[NCH], wv[NCH], bv[NCH];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; i++) {
        const int c4 = lane + 64 * i;
        v[i] = c4 < C4 ? Act<T>::ld(x + 4 * c4) : make_float4(0.f, 0.f, 0.f, 0.f);
        // the affine parameters load alongside the row, not after its reductions
        wv[i] = c4 < C4 ? ld4(w + 4 * c4) : make_float4(0.f, 0.f, 0.f, 0.f);
        bv[i] = c4 < C4 ? ld4(b + 4 * c4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < NCH; i++) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    const float m = wave_sum(s) / C;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; i++) {
        const int c4 = lane + 64 * i;
        if (c4 < C4) {
            const float a = v[i].x - m, bb = v[i].y - m, c = v[i].z - m, d = v[i].w - m;
            ss += (a * a + bb * bb) + (c * c + d * d);
        }
    }
    const float var = wave_sum(ss) / C;
    const float r = 1.0f / sqrtf(var + LN_EPS);
    T* y = out + (int64_t)row * C;
#pragma unroll
    for (int i = 0; i < NCH; i++) {
        const int c4 = lane + 64 * i;
        if (c4 < C4) {
            const float4 ww = wv[i], bb = bv[i];
            Act<T>::st(y + 4 * c4, make_float4((v[i].x - m) * r * ww.x + bb.x,
                                        (v[i].y - m) * r * ww.y + bb.y,
                                        (v[i].z - m) * r * ww.z + bb.z,
                                        (v[i].w - m) * r * ww.w + bb.w));
        }
    }
    if (lane == 0) {
        mean[row] = m;
        rstd[row] = r;
    }
}

// Rows per backward workgroup: enough workgroups to fill the chip, few
// enough partial rows to keep the second stage small.
inline int ln_rows_per_block(int N) {
    int r = (N + 1023) / 1024;
    r = (r + 3) & ~3;
    return r < 4 ? 4 : r;
}

// nsum = 2: partial rows of (dw, db); nsum = 3: (dw, db, column sums of the
// stored dres rows).  The third sum runs in the wave's own LDS row rather
// than in registers, which keeps four waves per SIMD.
template <int NCH, class T>
__global__ __launch_bounds__(256) void ln_bwd_kernel(
    T* __restrict__ dres, int accumulate, float* __restrict__ partials,
    const T* __restrict__ dout, const T* __restrict__ inp, const float* __restrict__ w,
    const float* __restrict__ mean, const float* __restrict__ rstd, int N, int C, int rpb,
    int nsum) {
    extern __shared__ float red[];  // [4 waves][nsum][C]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int C4 = C >> 2;
    float* osum = red + (wave * nsum + 2) * C;  // this wave's output sums (nsum == 3)
    if (nsum == 3)
        for (int c4 = lane; c4 < C4; c4 += 64) st4(osum + 4 * c4, make_float4(0.f, 0.f, 0.f, 0.f));
    float4 pw[NCH], pb[NCH], wv[NCH];
#pragma unroll
    for (int i = 0; i < NCH; i++) {
        pw[i] = pb[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        const int c4 = lane + 64 * i;
        wv[i] = c4 < C4 ? ld4(w + 4 * c4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const int r0 = blockIdx.x * rpb;
    const int r1 = min(N, r0 + rpb);
    for (int row = r0 + wave; row < r1; row += 4) {
        const float m = mean[row], rs = rstd[row];
        const T* dy = dout + (int64_t)row * C;
        const T* x = inp + (int64_t)row * C;
        T* dx = dres + (int64_t)row * C;
        float4 g[NCH], xh[NCH], dd[NCH], xv[NCH], old[NCH];
        float sg = 0.f, sgx = 0.f;
        // every load of the row is issued before the first use
#pragma unroll
        for (int i = 0; i < NCH; i++) {
            const int c4 = lane + 64 * i;
            dd[i] = xv[i] = old[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (c4 < C4) {
                dd[i] = Act<T>::ld(dy + 4 * c4);
                xv[i] = Act<T>::ld(x + 4 * c4);
                if (accumulate) old[i] = Act<T>::ld(dx + 4 * c4);
            }
        }
#pragma unroll
        for (int i = 0; i < NCH; i++) {
            const float4 d = dd[i], xx = xv[i];
            xh[i] = make_float4((xx.x - m) * rs, (xx.y - m) * rs, (xx.z - m) * rs,
                                (xx.w - m) * rs);
            g[i] = make_float4(d.x * wv[i].x, d.y * wv[i].y, d.z * wv[i].z, d.w * wv[i].w);
            sg += (g[i].x + g[i].y) + (g[i].z + g[i].w);
            sgx += (g[i].x * xh[i].x + g[i].y * xh[i].y) + (g[i].z * xh[i].z + g[i].w * xh[i].w);
            pw[i].x += d.x * xh[i].x;
            pw[i].y += d.y * xh[i].y;
            pw[i].z += d.z * xh[i].z;
            pw[i].w += d.w * xh[i].w;
            pb[i].x += d.x;
            pb[i].y += d.y;
            pb[i].z += d.z;
            pb[i].w += d.w;
        }
        const float mg = wave_sum(sg) / C, mgx = wave_sum(sgx) / C;
#pragma unroll
        for (int i = 0; i < NCH; i++) {
            const int c4 = lane + 64 * i;
            if (c4 < C4) {
                float4 o = make_float4(rs * (g[i].x - mg - xh[i].x * mgx),
                                       rs * (g[i].y - mg - xh[i].y * mgx),
                                       rs * (g[i].z - mg - xh[i].z * mgx),
                                       rs * (g[i].w - mg - xh[i].w * mgx));
                o.x += old[i].x;  // zero unless accumulating
                o.y += old[i].y;
                o.z += old[i].z;
                o.w += old[i].w;
                Act<T>::st(dx + 4 * c4, o);
                if (nsum == 3) {
                    const float4 v = as_stored<T>(o);
                    float4 t = ld4(osum + 4 * c4);
                    t.x += v.x;
                    t.y += v.y;
                    t.z += v.z;
                    t.w += v.w;
                    st4(osum + 4 * c4, t);
                }
            }
        }
    }
    // reduce the four waves' column partials, in wave order
#pragma unroll
    for (int i = 0; i < NCH; i++) {
        const int c4 = lane + 64 * i;
        if (c4 < C4) {
            st4(red + (wave * nsum) * C + 4 * c4, pw[i]);
            st4(red + (wave * nsum + 1) * C + 4 * c4, pb[i]);
        }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < nsum * C; c += blockDim.x) {
        const int k = c / C, cc = c - k * C;
        float s = red[(0 * nsum + k) * C + cc];
        s += red[(1 * nsum + k) * C + cc];
        s += red[(2 * nsum + k) * C + cc];
        s += red[(3 * nsum + k) * C + cc];
        partials[(int64_t)blockIdx.x * nsum * C + c] = s;
    }
}

template <class T>
hipError_t ln_fwd_launch(hipStream_t s, T* out, float* mean, float* rstd, const T* inp,
                         const float* w, const float* b, int N, int C) {
    dim3 grid((N + 3) / 4), block(256);
    switch ((C + 255) / 256) {
        case 1: launch((ln_fwd_kernel<1, T>), grid, block, 0, s, out, mean, rstd, inp, w, b, N, C); break;
        case 2: launch((ln_fwd_kernel<2, T>), grid, block, 0, s, out, mean, rstd, inp, w, b, N, C); break;
        case 3: launch((ln_fwd_kernel<3, T>), grid, block, 0, s, out, mean, rstd, inp, w, b, N, C); break;
        case 4: launch((ln_fwd_kernel<4, T>), grid, block, 0, s, out, mean, rstd, inp, w, b, N, C); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <class T>
hipError_t ln_bwd_launch(hipStream_t s, T* dres, int accumulate, float* partials, const T* dout,
                         const T* inp, const float* w, const float* mean, const float* rstd,
                         int N, int C, int rpb, int nb, int nsum) {
    const size_t shm = (size_t)4 * nsum * C * sizeof(float);
    dim3 grid(nb), block(256);
    switch ((C + 255) / 256) {
        case 1: launch((ln_bwd_kernel<1, T>), grid, block, shm, s, dres, accumulate, partials, dout, inp, w, mean, rstd, N, C, rpb, nsum); break;
        case 2: launch((ln_bwd_kernel<2, T>), grid, block, shm, s, dres, accumulate, partials, dout, inp, w, mean, rstd, N, C, rpb, nsum); break;
        case 3: launch((ln_bwd_kernel<3, T>), grid, block, shm, s, dres, accumulate, partials, dout, inp, w, mean, rstd, N, C, rpb, nsum); break;
        case 4: launch((ln_bwd_kernel<4, T>), grid, block, shm, s, dres, accumulate, partials, dout, inp, w, mean, rstd, N, C, rpb, nsum); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t layernorm_forward(hipStream_t s, void* out, float* mean, float* rstd, const void* inp,
                             const float* w, const float* b, int N, int C, int dt) {
    if (N <= 0) return hipSuccess;
    return by_dt(dt, [&](auto e) {
        using E = decltype(e);
        return ln_fwd_launch<E>(s, (E*)out, mean, rstd, (const E*)inp, w, b, N, C);
    });
}

hipError_t layernorm_backward(hipStream_t s, void* dres, int accumulate, float* dw, float* db,
                              float* dbias, float* partials, const void* dout, const void* inp,
                              const float* w, const float* mean, const float* rstd, int N,
                              int C, int dt) {
    if (N <= 0) return hipSuccess;
    const int rpb = ln_rows_per_block(N);
    const int nb = (N + rpb - 1) / rpb;
    const int nsum = dbias ? 3 : 2;
    hipError_t e = by_dt(dt, [&](auto x) {
        using E = decltype(x);
        return ln_bwd_launch<E>(s, (E*)dres, accumulate, partials, (const E*)dout,
                                (const E*)inp, w, mean, rstd, N, C, rpb, nb, nsum);
    });
    if (e != hipSuccess) return e;
    return colsum_add(s, dw, db, dbias, C, partials, nb, nsum * C);
}

}  // namespace gk
