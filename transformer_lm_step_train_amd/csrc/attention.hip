// Causal multi-head self-attention, forward and backward, on the fp32
// matrix cores (v_mfma_f32_32x32x2_f32).
//
// The layer is GPT-2's masked self-attention (ujoy.net article "徒手用 1000 行
// C 语言实现", section "用C语言实现LLM": self-attention is one of the layers
// with a forward and a backward).  Per sequence b and head h, with q, k, v
// the head's slices of the QKV rows and s = q_t . k_u / sqrt(hs) for u <= t:
//   out_t = sum_u softmax_u(s) v_u,   lse_t = log sum_u exp(s_tu).
// Instead of materializing the (T, T) score matrix, the forward walks key
// tiles with a running maximum and sum (online softmax) and keeps only lse;
// the backward recomputes the probabilities from lse.
//
// Layout trick: scores are computed transposed, S^T = K Q^T, so each lane
// owns one query (one column of the 32x32 accumulator) and holds 16 of its
// 32 keys in registers.  The row statistics are then per-lane scalars, and
// the same registers are directly the B operand of O^T = V^T P^T.  The
// key/value kernel of the backward uses the mirror image (lane owns a key).
//
// Backward: D_t = dout_t . out_t;  P = exp(s - lse);  dS = P (dP - D) with
// dP = dout V^T;  dQ = dS K / sqrt(hs);  dK = dS^T Q / sqrt(hs);  dV = P^T dout.
// dQ and (dK, dV) come from two kernels that each own their output rows, so
// no output is accumulated with atomics and results are deterministic.
#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

constexpr int QB = 64;  // rows owned per workgroup (two waves of 32)
constexpr int KT = 64;  // rows per staged tile

__device__ __forceinline__ floatx16 mfma(float a, float b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void zero16(floatx16& x) {
#pragma unroll
    for (int e = 0; e < 16; e++) x[e] = 0.f;
}

// Copy rows r0..r0+63 (row r at base + r*ld, HS floats each) into LDS with
// row stride HS+4; rows at or past T are zero.
template <int HS>
__device__ __forceinline__ void stage_rows(float* sm, const float* __restrict__ base,
                                           int64_t ld, int r0, int T) {
    constexpr int C4 = HS / 4;
    for (int i = threadIdx.x; i < KT * C4; i += blockDim.x) {
        const int r = i / C4, c = (i - r * C4) * 4;
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (r0 + r < T) x = ld4(base + (int64_t)(r0 + r) * ld + c);
        st4(sm + r * (HS + 4) + c, x);
    }
}

template <int HS>
__global__ __launch_bounds__(128) void attn_fwd_kernel(float* __restrict__ out,
                                                       float* __restrict__ lse,
                                                       const float* __restrict__ qkv,
                                                       int T, int C, int NH, float scale) {
    constexpr int LD = HS + 4, HALF = HS / 2, NDB = (HS + 31) / 32;
    __shared__ __attribute__((aligned(16))) float ks[KT * LD];
    __shared__ __attribute__((aligned(16))) float vs[KT * LD];

    const int nqb = (T + QB - 1) / QB;
    const int id = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = id / nqb;
    const int qb = nqb - 1 - (id - bh * nqb);  // longest rows first
    const int b = bh / NH, h = bh - b * NH;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 31, g = lane >> 5;
    const int64_t ld = 3 * (int64_t)C;
    const float* qbase = qkv + (int64_t)b * T * ld + h * HS;
    const int q = qb * QB + wave * 32 + li;

    float qr[HALF];
#pragma unroll
    for (int s = 0; s < HALF; s += 4) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (q < T) x = ld4(qbase + (int64_t)q * ld + g * HALF + s);
        qr[s] = x.x * scale;
        qr[s + 1] = x.y * scale;
        qr[s + 2] = x.z * scale;
        qr[s + 3] = x.w * scale;
    }
    floatx16 o[NDB];
#pragma unroll
    for (int d = 0; d < NDB; d++) zero16(o[d]);
    float m = -INFINITY, l = 0.f;

    for (int kt = 0; kt <= qb; kt++) {
        __syncthreads();
        stage_rows<HS>(ks, qbase + C, ld, kt * KT, T);
        stage_rows<HS>(vs, qbase + 2 * C, ld, kt * KT, T);
        __syncthreads();
        floatx16 sc[2];
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
            zero16(sc[kb]);
            const float* kr = ks + (kb * 32 + li) * LD + g * HALF;
#pragma unroll
            for (int s = 0; s < HALF; s += 4) {
                const float4 kf = ld4(kr + s);
                sc[kb] = mfma(kf.x, qr[s], sc[kb]);
                sc[kb] = mfma(kf.y, qr[s + 1], sc[kb]);
                sc[kb] = mfma(kf.z, qr[s + 2], sc[kb]);
                sc[kb] = mfma(kf.w, qr[s + 3], sc[kb]);
            }
        }
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int key = kt * KT + kb * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                if (key > q || key >= T) sc[kb][e] = -INFINITY;
                mt = fmaxf(mt, sc[kb][e]);
            }
        mt = fmaxf(mt, __shfl_xor(mt, 32, WAVE));
        const float mn = fmaxf(m, mt);
        const float corr = expf(m - mn);
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const float p = expf(sc[kb][e] - mn);
                sc[kb][e] = p;
                ls += p;
            }
        ls += __shfl_xor(ls, 32, WAVE);
        l = l * corr + ls;
        m = mn;
#pragma unroll
        for (int d = 0; d < NDB; d++)
#pragma unroll
            for (int e = 0; e < 16; e++) o[d][e] *= corr;
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int kl = kb * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
#pragma unroll
                for (int d = 0; d < NDB; d++) {
                    const int dim = d * 32 + li;
                    const float va = dim < HS ? vs[kl * LD + dim] : 0.f;
                    o[d] = mfma(va, sc[kb][e], o[d]);
                }
            }
    }
    if (q < T) {
        const float inv = 1.f / l;
        float* orow = out + ((int64_t)b * T + q) * C + h * HS;
#pragma unroll
        for (int d = 0; d < NDB; d++)
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const int dim0 = d * 32 + 8 * c + 4 * g;
                if (dim0 < HS)
                    st4(orow + dim0, make_float4(o[d][4 * c] * inv, o[d][4 * c + 1] * inv,
                                                 o[d][4 * c + 2] * inv, o[d][4 * c + 3] * inv));
            }
        if (g == 0) lse[((int64_t)b * NH + h) * T + q] = m + logf(l);
    }
}

// D[b,h,t] = dout[b,t,h-slice] . out[b,t,h-slice]
__global__ __launch_bounds__(256) void attn_rowdot_kernel(float* __restrict__ D,
                                                          const float* __restrict__ dout,
                                                          const float* __restrict__ out,
                                                          int B, int T, int C, int NH,
                                                          int HS) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= (int64_t)B * T * NH) return;
    const int h = (int)(i % NH);
    const int64_t bt = i / NH;
    const int b = (int)(bt / T), t = (int)(bt - (int64_t)b * T);
    const float* x = dout + bt * C + h * HS;
    const float* y = out + bt * C + h * HS;
    float s = 0.f;
    for (int d = 0; d < HS; d += 4) {
        const float4 a = ld4(x + d), c = ld4(y + d);
        s += a.x * c.x + a.y * c.y + a.z * c.z + a.w * c.w;
    }
    D[((int64_t)b * NH + h) * T + t] = s;
}

template <int HS>
__global__ __launch_bounds__(128) void attn_bwd_dq_kernel(
    float* __restrict__ dqkv, const float* __restrict__ dout, const float* __restrict__ qkv,
    const float* __restrict__ lse, const float* __restrict__ D, int T, int C, int NH,
    float scale) {
    constexpr int LD = HS + 4, HALF = HS / 2, NDB = (HS + 31) / 32;
    __shared__ __attribute__((aligned(16))) float ks[KT * LD];
    __shared__ __attribute__((aligned(16))) float vs[KT * LD];

    const int nqb = (T + QB - 1) / QB;
    const int id = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = id / nqb;
    const int qb = nqb - 1 - (id - bh * nqb);
    const int b = bh / NH, h = bh - b * NH;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 31, g = lane >> 5;
    const int64_t ld = 3 * (int64_t)C;
    const float* qbase = qkv + (int64_t)b * T * ld + h * HS;
    const float* dobase = dout + (int64_t)b * T * C + h * HS;
    const int q = qb * QB + wave * 32 + li;

    float qr[HALF], dr[HALF];
#pragma unroll
    for (int s = 0; s < HALF; s += 4) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f), y = x;
        if (q < T) {
            x = ld4(qbase + (int64_t)q * ld + g * HALF + s);
            y = ld4(dobase + (int64_t)q * C + g * HALF + s);
        }
        qr[s] = x.x * scale;
        qr[s + 1] = x.y * scale;
        qr[s + 2] = x.z * scale;
        qr[s + 3] = x.w * scale;
        dr[s] = y.x;
        dr[s + 1] = y.y;
        dr[s + 2] = y.z;
        dr[s + 3] = y.w;
    }
    const int64_t srow = ((int64_t)b * NH + h) * T;
    const float lq = q < T ? lse[srow + q] : 0.f;
    const float Dq = q < T ? D[srow + q] : 0.f;
    floatx16 dq[NDB];
#pragma unroll
    for (int d = 0; d < NDB; d++) zero16(dq[d]);

    for (int kt = 0; kt <= qb; kt++) {
        __syncthreads();
        stage_rows<HS>(ks, qbase + C, ld, kt * KT, T);
        stage_rows<HS>(vs, qbase + 2 * C, ld, kt * KT, T);
        __syncthreads();
        floatx16 sc[2], dp[2];
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
            zero16(sc[kb]);
            zero16(dp[kb]);
            const float* kr = ks + (kb * 32 + li) * LD + g * HALF;
            const float* vr = vs + (kb * 32 + li) * LD + g * HALF;
#pragma unroll
            for (int s = 0; s < HALF; s += 4) {
                const float4 kf = ld4(kr + s);
                const float4 vf = ld4(vr + s);
                sc[kb] = mfma(kf.x, qr[s], sc[kb]);
                sc[kb] = mfma(kf.y, qr[s + 1], sc[kb]);
                sc[kb] = mfma(kf.z, qr[s + 2], sc[kb]);
                sc[kb] = mfma(kf.w, qr[s + 3], sc[kb]);
                dp[kb] = mfma(vf.x, dr[s], dp[kb]);
                dp[kb] = mfma(vf.y, dr[s + 1], dp[kb]);
                dp[kb] = mfma(vf.z, dr[s + 2], dp[kb]);
                dp[kb] = mfma(vf.w, dr[s + 3], dp[kb]);
            }
        }
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int key = kt * KT + kb * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                const float p = (key <= q && key < T) ? expf(sc[kb][e] - lq) : 0.f;
                sc[kb][e] = p * (dp[kb][e] - Dq);
            }
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int kl = kb * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
#pragma unroll
                for (int d = 0; d < NDB; d++) {
                    const int dim = d * 32 + li;
                    const float ka = dim < HS ? ks[kl * LD + dim] : 0.f;
                    dq[d] = mfma(ka, sc[kb][e], dq[d]);
                }
            }
    }
    if (q < T) {
        float* row = dqkv + ((int64_t)b * T + q) * ld + h * HS;
#pragma unroll
        for (int d = 0; d < NDB; d++)
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const int dim0 = d * 32 + 8 * c + 4 * g;
                if (dim0 < HS)
                    st4(row + dim0,
                        make_float4(dq[d][4 * c] * scale, dq[d][4 * c + 1] * scale,
                                    dq[d][4 * c + 2] * scale, dq[d][4 * c + 3] * scale));
            }
    }
}

template <int HS>
__global__ __launch_bounds__(128) void attn_bwd_dkdv_kernel(
    float* __restrict__ dqkv, const float* __restrict__ dout, const float* __restrict__ qkv,
    const float* __restrict__ lse, const float* __restrict__ D, int T, int C, int NH,
    float scale) {
    constexpr int LD = HS + 4, HALF = HS / 2, NDB = (HS + 31) / 32;
    __shared__ __attribute__((aligned(16))) float qs[KT * LD];
    __shared__ __attribute__((aligned(16))) float dos[KT * LD];
    __shared__ float lsm[KT], dsm[KT];

    const int nkb = (T + QB - 1) / QB;
    const int id = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = id / nkb;
    const int kb0 = id - bh * nkb;  // lowest key block = most query tiles: first
    const int b = bh / NH, h = bh - b * NH;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 31, g = lane >> 5;
    const int64_t ld = 3 * (int64_t)C;
    const float* qbase = qkv + (int64_t)b * T * ld + h * HS;
    const float* dobase = dout + (int64_t)b * T * C + h * HS;
    const int64_t srow = ((int64_t)b * NH + h) * T;
    const int key = kb0 * QB + wave * 32 + li;

    float kr[HALF], vr[HALF];
#pragma unroll
    for (int s = 0; s < HALF; s += 4) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f), y = x;
        if (key < T) {
            x = ld4(qbase + C + (int64_t)key * ld + g * HALF + s);
            y = ld4(qbase + 2 * C + (int64_t)key * ld + g * HALF + s);
        }
        kr[s] = x.x;
        kr[s + 1] = x.y;
        kr[s + 2] = x.z;
        kr[s + 3] = x.w;
        vr[s] = y.x;
        vr[s + 1] = y.y;
        vr[s + 2] = y.z;
        vr[s + 3] = y.w;
    }
    floatx16 dk[NDB], dv[NDB];
#pragma unroll
    for (int d = 0; d < NDB; d++) {
        zero16(dk[d]);
        zero16(dv[d]);
    }
    const int nqt = (T + KT - 1) / KT;
    for (int qt = kb0; qt < nqt; qt++) {
        __syncthreads();
        stage_rows<HS>(qs, qbase, ld, qt * KT, T);
        stage_rows<HS>(dos, dobase, C, qt * KT, T);
        for (int i = threadIdx.x; i < KT; i += blockDim.x) {
            const int t = qt * KT + i;
            lsm[i] = t < T ? lse[srow + t] : 0.f;
            dsm[i] = t < T ? D[srow + t] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int qh = 0; qh < 2; qh++) {
            floatx16 sc, dp;
            zero16(sc);
            zero16(dp);
            const float* qrow = qs + (qh * 32 + li) * LD + g * HALF;
            const float* drow = dos + (qh * 32 + li) * LD + g * HALF;
#pragma unroll
            for (int s = 0; s < HALF; s += 4) {
                const float4 qf = ld4(qrow + s);
                const float4 df = ld4(drow + s);
                sc = mfma(qf.x * scale, kr[s], sc);
                sc = mfma(qf.y * scale, kr[s + 1], sc);
                sc = mfma(qf.z * scale, kr[s + 2], sc);
                sc = mfma(qf.w * scale, kr[s + 3], sc);
                dp = mfma(df.x, vr[s], dp);
                dp = mfma(df.y, vr[s + 1], dp);
                dp = mfma(df.z, vr[s + 2], dp);
                dp = mfma(df.w, vr[s + 3], dp);
            }
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int ql = qh * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                const int qa = qt * KT + ql;
                const float p = (qa < T && key <= qa) ? expf(sc[e] - lsm[ql]) : 0.f;
                sc[e] = p;
                dp[e] = p * (dp[e] - dsm[ql]);
            }
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int ql = qh * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
#pragma unroll
                for (int d = 0; d < NDB; d++) {
                    const int dim = d * 32 + li;
                    const float da = dim < HS ? dos[ql * LD + dim] : 0.f;
                    const float qa = dim < HS ? qs[ql * LD + dim] : 0.f;
                    dv[d] = mfma(da, sc[e], dv[d]);
                    dk[d] = mfma(qa, dp[e], dk[d]);
                }
            }
        }
    }
    if (key < T) {
        float* row = dqkv + ((int64_t)b * T + key) * ld + h * HS;
#pragma unroll
        for (int d = 0; d < NDB; d++)
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const int dim0 = d * 32 + 8 * c + 4 * g;
                if (dim0 < HS) {
                    st4(row + C + dim0,
                        make_float4(dk[d][4 * c] * scale, dk[d][4 * c + 1] * scale,
                                    dk[d][4 * c + 2] * scale, dk[d][4 * c + 3] * scale));
                    st4(row + 2 * C + dim0, make_float4(dv[d][4 * c], dv[d][4 * c + 1],
                                                        dv[d][4 * c + 2], dv[d][4 * c + 3]));
                }
            }
    }
}

template <int HS>
hipError_t fwd_hs(hipStream_t s, float* out, float* lse, const float* qkv, int B, int T,
                  int C, int NH) {
    const int nqb = (T + QB - 1) / QB;
    const float scale = 1.0f / sqrtf((float)HS);
    hipLaunchKernelGGL((attn_fwd_kernel<HS>), dim3(B * NH * nqb), dim3(128), 0, s, out, lse,
                       qkv, T, C, NH, scale);
    return hipGetLastError();
}

template <int HS>
hipError_t bwd_hs(hipStream_t s, float* dqkv, float* D, const float* dout, const float* qkv,
                  const float* out, const float* lse, int B, int T, int C, int NH) {
    const int nb = (T + QB - 1) / QB;
    const float scale = 1.0f / sqrtf((float)HS);
    const int64_t rows = (int64_t)B * T * NH;
    hipLaunchKernelGGL(attn_rowdot_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0,
                       s, D, dout, out, B, T, C, NH, HS);
    hipLaunchKernelGGL((attn_bwd_dq_kernel<HS>), dim3(B * NH * nb), dim3(128), 0, s, dqkv,
                       dout, qkv, lse, D, T, C, NH, scale);
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<HS>), dim3(B * NH * nb), dim3(128), 0, s, dqkv,
                       dout, qkv, lse, D, T, C, NH, scale);
    return hipGetLastError();
}

}  // namespace

hipError_t attention_forward(hipStream_t s, float* out, float* lse, const float* qkv, int B,
                             int T, int C, int NH) {
    if (B <= 0 || T <= 0) return hipSuccess;
    switch (C / NH) {
        case 16: return fwd_hs<16>(s, out, lse, qkv, B, T, C, NH);
        case 32: return fwd_hs<32>(s, out, lse, qkv, B, T, C, NH);
        case 64: return fwd_hs<64>(s, out, lse, qkv, B, T, C, NH);
        default: return hipErrorInvalidValue;
    }
}

hipError_t attention_backward(hipStream_t s, float* dqkv, float* dpre, const float* dout,
                              const float* qkv, const float* out, const float* lse, int B,
                              int T, int C, int NH) {
    if (B <= 0 || T <= 0) return hipSuccess;
    switch (C / NH) {
        case 16: return bwd_hs<16>(s, dqkv, dpre, dout, qkv, out, lse, B, T, C, NH);
        case 32: return bwd_hs<32>(s, dqkv, dpre, dout, qkv, out, lse, B, T, C, NH);
        case 64: return bwd_hs<64>(s, dqkv, dpre, dout, qkv, out, lse, B, T, C, NH);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gk
