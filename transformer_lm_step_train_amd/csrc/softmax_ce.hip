// Fused softmax + cross-entropy over the vocabulary, forward and backward in
// one pass (ujoy.net article "徒手用 1000 行 C 语言实现", section "用C语言实现
// LLM": the softmax and cross-entropy layers; section "训练过程": the mean
// "train loss" printed each step).
//
// Per position n with logits z (V values) and target y:
//   lse = max z + log sum_v exp(z_v - max z),  loss_n = lse - z_y,
//   d(mean loss)/dz_v = (exp(z_v - lse) - [v == y]) / N.
// This equals the materialized softmax followed by -log p_y.  One workgroup
// holds a whole row in registers (one HBM read), and writes the gradient over
// the logits (one HBM write).  The evaluation variant (no gradient) only
// reads the row and leaves the logits as they are.
#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

template <int NT>
__device__ __forceinline__ float block_max(float v, float* sh) {
    v = wave_max(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) sh[wave] = v;
    __syncthreads();
    float r = sh[0];
#pragma unroll
    for (int i = 1; i < NT / 64; i++) r = fmaxf(r, sh[i]);
    return r;
}

template <int NT, int NJ, bool GRAD, class T, int WPE = 4>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(WPE))) void softmax_ce_kernel(T* __restrict__ logits,
                                                        float* __restrict__ losses,
                                                        const int32_t* __restrict__ targets,
                                                        int V, int ldv, float dscale,
                                                        const float* __restrict__ gscale,
                                                        int* __restrict__ flag) {
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr int NW = NT / 64;
    __shared__ float shm[NW], shs[NW];
    const int64_t row = blockIdx.x;
    if (gscale) dscale *= *gscale;  // loss scaling of the fp16 model
    // row-uniform values are kept in scalar registers (the row fills the
    // vector registers)
    dscale = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(dscale)));
    T* z = logits + row * ldv;
    const int V4 = ldv >> 2;
    const auto zr = buf_rsrc(z, (uint32_t)ldv * sizeof(T));
    constexpr int JB = NT * BufAct<T>::BYTES;  // byte stride between a thread's groups
    const int vo = threadIdx.x * BufAct<T>::BYTES;
    const int tgt = targets[row];
    const bool bad = tgt < 0 || tgt >= V;
    // the thread whose groups hold the target column reads its logit
    const bool owner = !bad && threadIdx.x == (tgt >> 2) % NT;
    float4 v[NJ];
#pragma unroll
    for (int j = 0; j < NJ; j++) {
        // Groups wholly inside the row (a uniform test) load unconditionally.
        if (NT * (j + 1) <= V4 || threadIdx.x + NT * j < V4)
            v[j] = BufAct<T>::ld(zr, vo, JB * j);
        else
            v[j] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
    const float zt = __int_as_float(
        __builtin_amdgcn_readfirstlane(__float_as_int(bad ? 0.f : Act<T>::ld1(z + tgt))));
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < NJ; j++) {
        if (4 * NT * (j + 1) > V) {  // a group reaching the padding columns
            const int c = 4 * (threadIdx.x + NT * j);
            if (c >= V) v[j].x = -INFINITY;
            if (c + 1 >= V) v[j].y = -INFINITY;
            if (c + 2 >= V) v[j].z = -INFINITY;
            if (c + 3 >= V) v[j].w = -INFINITY;
        }
        m = fmaxf(m, fmaxf(fmaxf(v[j].x, v[j].y), fmaxf(v[j].z, v[j].w)));
    }
    // A thread whose columns are all padding has m = -inf: shift by 0 so that
    // its exponentials are exp(-inf) = 0 rather than NaN.
    const float ms = m == -INFINITY ? 0.f : m * LOG2E;
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; j++) {
        v[j].x = __builtin_amdgcn_exp2f(fmaf(v[j].x, LOG2E, -ms));
        v[j].y = __builtin_amdgcn_exp2f(fmaf(v[j].y, LOG2E, -ms));
        v[j].z = __builtin_amdgcn_exp2f(fmaf(v[j].z, LOG2E, -ms));
        v[j].w = __builtin_amdgcn_exp2f(fmaf(v[j].w, LOG2E, -ms));
        s += (v[j].x + v[j].y) + (v[j].z + v[j].w);
        __builtin_amdgcn_sched_barrier(0);  // in place, one group at a time
    }
    // Merge (m, s) over the wave, then over the waves.
    const float mw = wave_max(m);
    float sw = wave_sum(m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f((m - mw) * LOG2E));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        shm[wave] = mw;
        shs[wave] = sw;
    }
    __syncthreads();
    // every wave merges the NW pairs across its lanes (few registers while
    // the row is held)
    const float mi = lane < NW ? shm[lane] : -INFINITY;
    const float M = wave_max(mi);
    const float S = wave_sum(mi == -INFINITY ? 0.f : shs[lane < NW ? lane : 0] *
                                                      __builtin_amdgcn_exp2f((mi - M) * LOG2E));
    const float lse = M + logf(S);
    if (owner) losses[row] = lse - zt;
    if (bad && threadIdx.x == 0) {
        losses[row] = 0.f;
        atomicOr(flag, 2);
    }
    if constexpr (!GRAD) return;
    // exp(z - lse) = e * exp(m_t - lse); the padding columns give 0.
    const float f = bad || m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - lse) * LOG2E) * dscale;
#pragma unroll
    for (int j = 0; j < NJ; j++) {
        v[j].x *= f;
        v[j].y *= f;
        v[j].z *= f;
        v[j].w *= f;
        if (NT * (j + 1) <= V4 || threadIdx.x + NT * j < V4) BufAct<T>::st(zr, vo, JB * j, v[j]);
        __builtin_amdgcn_sched_barrier(0);  // one group at a time
    }
    // The target column, stored again by the thread that wrote it: the same
    // exponential (same operands and instructions as in its group) times f,
    // minus the scaled one-hot.
    if (owner) Act<T>::st1(z + tgt, __builtin_amdgcn_exp2f(fmaf(zt, LOG2E, -ms)) * f - dscale);
}

template <int NT, int NJ, class T, int WPE = 4>
hipError_t launch_ce(hipStream_t s, T* logits, float* losses, const int32_t* targets, int N,
                     int V, int ldv, float dscale, const float* gscale, int* flag) {
    if (dscale != 0.f)
        launch((softmax_ce_kernel<NT, NJ, true, T, WPE>), dim3(N), dim3(NT), 0, s, logits, losses,
               targets, V, ldv, dscale, gscale, flag);
    else
        launch((softmax_ce_kernel<NT, NJ, false, T, WPE>), dim3(N), dim3(NT), 0, s, logits,
               losses, targets, V, ldv, dscale, gscale, flag);
    return hipGetLastError();
}

// Two rows share a compute unit, so that one row's loads overlap the other's
// reduction and stores: 512-thread workgroups, except the 16-bit rows of up
// to 53248 columns (1024 threads) and rows past 51200 columns (1024 threads,
// one row per compute unit).
template <class T>
hipError_t softmax_ce_t(hipStream_t s, T* logits, float* losses, const int32_t* targets, int N,
                        int V, int ldv, float dscale, const float* gs, int* flag) {
    const int V4 = ldv / 4;
    if (V4 <= 256) return launch_ce<256, 1>(s, logits, losses, targets, N, V, ldv, dscale, gs, flag);
    const int nj = (V4 + 511) / 512;
    if (nj <= 1) return launch_ce<512, 1>(s, logits, losses, targets, N, V, ldv, dscale, gs, flag);
    if (nj <= 2) return launch_ce<512, 2>(s, logits, losses, targets, N, V, ldv, dscale, gs, flag);
    if (nj <= 4) return launch_ce<512, 4>(s, logits, losses, targets, N, V, ldv, dscale, gs, flag);
    if (nj <= 8) return launch_ce<512, 8>(s, logits, losses, targets, N, V, ldv, dscale, gs, flag);
    if (nj <= 16) return launch_ce<512, 16>(s, logits, losses, targets, N, V, ldv, dscale, gs, flag);
    // 16-bit rows up to 53248 columns: 1024 threads of 13 groups and two rows
    // per compute unit (8 waves per SIMD, 64 VGPRs: three of one group's
    // exponentials spill to scratch once per row).  On GPT-2's 50304-wide
    // rows 677 against 827 us in bf16 (standalone), where the 512-thread rows
    // keep too few bytes in flight; in fp32 the gain is 3%, so fp32 keeps the
    // spill-free 512-thread rows.
    if (sizeof(T) == 2 && (V4 + 1023) / 1024 <= 13)
        return launch_ce<1024, 13, T, 8>(s, logits, losses, targets, N, V, ldv, dscale, gs, flag);
    if (nj <= 25) return launch_ce<512, 25>(s, logits, losses, targets, N, V, ldv, dscale, gs, flag);
    // rows past 51200 columns (up to 65536): one 1024-thread workgroup per
    // compute unit, 16 groups per thread, so the row still fits in registers
    if ((V4 + 1023) / 1024 <= 16)
        return launch_ce<1024, 16>(s, logits, losses, targets, N, V, ldv, dscale, gs, flag);
    return hipErrorInvalidValue;
}

__global__ __launch_bounds__(1024) void mean_kernel(float* __restrict__ out,
                                                    const float* __restrict__ x, int n) {
    __shared__ double sh[16];
    double s = 0.0;
    for (int i = threadIdx.x; i < n; i += 1024) s += (double)x[i];
    s = wave_sum_d(s);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        for (int i = 0; i < 16; i++) t += sh[i];
        out[0] = (float)(t / n);
    }
}

// One draw from softmax(z) over a row of V logits by the inverse CDF: the
// smallest v with coin * sum_u p_u < sum_{u <= v} p_u, or V - 1 if rounding
// leaves none.  Each of the 1024 threads owns a contiguous run of the row;
// the exponentials are fp32 and every sum is fp64 (run sums, then an ordered
// exclusive scan over the runs), so the draw is deterministic and the CDF is
// far more precise than the spacing between its steps.
template <class T>
__global__ __launch_bounds__(1024) void sample_kernel(const T* __restrict__ z, int V, float coin,
                                                      int32_t* __restrict__ out) {
    __shared__ float shm[16];
    __shared__ double run[1024];
    __shared__ double total;
    __shared__ int best;
    const int tid = threadIdx.x;
    const int per = (V + 1023) / 1024;
    const int b0 = min(V, tid * per), b1 = min(V, b0 + per);
    float mx = -INFINITY;
    for (int v = b0; v < b1; v++) mx = fmaxf(mx, Act<T>::ld1(z + v));
    mx = block_max<1024>(mx, shm);
    double s = 0.0;
    for (int v = b0; v < b1; v++) s += (double)expf(Act<T>::ld1(z + v) - mx);
    run[tid] = s;
    __syncthreads();
    if (tid == 0) {  // exclusive scan over the runs, in thread order
        double acc = 0.0;
        for (int i = 0; i < 1024; i++) {
            const double t = run[i];
            run[i] = acc;
            acc += t;
        }
        total = acc;
        best = V - 1;
    }
    __syncthreads();
    const double target = (double)coin * total;
    double c = run[tid];
    for (int v = b0; v < b1; v++) {
        c += (double)expf(Act<T>::ld1(z + v) - mx);
        if (target < c) {
            atomicMin(&best, v);
            break;
        }
    }
    __syncthreads();
    if (tid == 0) *out = best;
}

}  // namespace

hipError_t sample_row(hipStream_t s, const void* logits, int V, float coin, int32_t* out,
                      int dt) {
    if (V <= 0) return hipErrorInvalidValue;
    return by_dt(dt, [&](auto e) {
        using E = decltype(e);
        launch(sample_kernel<E>, dim3(1), dim3(1024), 0, s, (const E*)logits, V, coin,
                           out);
        return hipGetLastError();
    });
}

hipError_t softmax_ce(hipStream_t s, void* logits, float* losses, const int32_t* targets,
                      int N, int V, int ldv, float dscale, const float* gscale, int* flag,
                      int dt) {
    if (N <= 0) return hipSuccess;
    if (V <= 0 || ldv < V || (ldv & 3) != 0) return hipErrorInvalidValue;
    return by_dt(dt, [&](auto e) {
        using E = decltype(e);
        return softmax_ce_t<E>(s, (E*)logits, losses, targets, N, V, ldv, dscale, gscale, flag);
    });
}

hipError_t mean_reduce(hipStream_t s, float* out, const float* x, int n) {
    launch(mean_kernel, dim3(1), dim3(1024), 0, s, out, x, n);
    return hipGetLastError();
}

}  // namespace gk
