// fp32 matrix multiply on the CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// Every linear layer of the model (QKV, attention projection, MLP fc and
// projection, tied LM head) runs its forward, input-gradient and
// weight-gradient products here (ujoy.net article "徒手用 1000 行 C 语言实现",
// section "用C语言实现LLM": the matmul layer, forward and backward).
//
// Tiling: a 256-thread workgroup owns a 128x128 output tile; its four waves
// each own 64x64 (2x2 blocks of the 32x32 MFMA).  The reduction runs in
// steps of 32, staged through LDS with a register prefetch of the next step
// (two LDS stages, one barrier per step).  Within a step the two 32-lane
// halves of a wave own k = 0..15 and k = 16..31, so an operand stored
// k-contiguous is read from LDS as float4 (four MFMA steps per read).
//
// Operands whose reduction index is contiguous in HBM are stored in LDS as
// [row][k] (36-float rows); operands whose free index is contiguous are
// stored as [k][row] (132-float rows).  Both are written with float4.
//
// Epilogues fuse what the layer does next: bias, residual add, GELU (writing
// both pre- and post-activation), the GELU derivative of the backward, or +=
// into a gradient.  Large reductions over few output tiles are split over K
// into a workspace and summed in a fixed order by a second kernel, so results
// are deterministic.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

constexpr int BM = 128, BN = 128, BK = 32, NTHR = 256;
constexpr int FM_LD = BK + 4;    // [row][k] tile row stride
constexpr int KM_LD = 128 + 4;   // [k][row] tile row stride
constexpr int EPI_PARTIAL = 100; // internal: write split-K partial sums

__device__ __forceinline__ floatx16 mfma(float a, float b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <bool KC>
struct Tile;

// Reduction index contiguous: element (r, k) at g[r*ld + k].
template <>
struct Tile<true> {
    static constexpr int FLOATS = 128 * FM_LD;
    float4 v[4];
    __device__ __forceinline__ void load(const float* __restrict__ g, int64_t ld,
                                         int r0, int R, int k0, int K) {
        const int t = threadIdx.x;
        const int k = k0 + (t & 7) * 4;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int r = r0 + (t >> 3) + 32 * i;
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (r < R) {
                const float* p = g + (int64_t)r * ld + k;
                if (k + 3 < K) {
                    x = ld4(p);
                } else {
                    if (k < K) x.x = p[0];
                    if (k + 1 < K) x.y = p[1];
                    if (k + 2 < K) x.z = p[2];
                }
            }
            v[i] = x;
        }
    }
    __device__ __forceinline__ void store(float* s) const {
        const int t = threadIdx.x;
#pragma unroll
        for (int i = 0; i < 4; i++)
            st4(s + ((t >> 3) + 32 * i) * FM_LD + (t & 7) * 4, v[i]);
    }
    // k = 16*g + 4*q + (0..3) at tile row r
    __device__ static __forceinline__ float4 frag(const float* s, int r, int g, int q) {
        return ld4(s + r * FM_LD + 16 * g + 4 * q);
    }
};

// Free index contiguous: element (r, k) at g[k*ld + r].
template <>
struct Tile<false> {
    static constexpr int FLOATS = BK * KM_LD;
    float4 v[4];
    __device__ __forceinline__ void load(const float* __restrict__ g, int64_t ld,
                                         int r0, int R, int k0, int K) {
        const int t = threadIdx.x;
        const int r = r0 + (t & 31) * 4;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int k = k0 + (t >> 5) + 8 * i;
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (k < K) {
                const float* p = g + (int64_t)k * ld + r;
                if (r + 3 < R) {
                    x = ld4(p);
                } else {
                    if (r < R) x.x = p[0];
                    if (r + 1 < R) x.y = p[1];
                    if (r + 2 < R) x.z = p[2];
                }
            }
            v[i] = x;
        }
    }
    __device__ __forceinline__ void store(float* s) const {
        const int t = threadIdx.x;
#pragma unroll
        for (int i = 0; i < 4; i++)
            st4(s + ((t >> 5) + 8 * i) * KM_LD + (t & 31) * 4, v[i]);
    }
    __device__ static __forceinline__ float4 frag(const float* s, int r, int g, int q) {
        const float* p = s + (16 * g + 4 * q) * KM_LD + r;
        return make_float4(p[0], p[KM_LD], p[2 * KM_LD], p[3 * KM_LD]);
    }
};

template <int OP, int EPI>
__global__ __launch_bounds__(NTHR, 2) void gemm_kernel(const GemmArgs a, int tiles_m,
                                                       int tiles_n, int kchunk,
                                                       float* __restrict__ partial) {
    constexpr bool AKC = (OP != GEMM_TN);
    constexpr bool BKC = (OP == GEMM_NT);
    __shared__ __attribute__((aligned(16))) float smA[2][Tile<AKC>::FLOATS];
    __shared__ __attribute__((aligned(16))) float smB[2][Tile<BKC>::FLOATS];

    // tile order: XCD-contiguous ranges, then groups of 8 tile-rows
    const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    constexpr int GM = 8;
    const int per_group = GM * tiles_n;
    const int group = tile / per_group;
    const int first_m = group * GM;
    const int gm = min(tiles_m - first_m, GM);
    const int in_g = tile - group * per_group;
    const int m0 = (first_m + in_g % gm) * BM;
    const int n0 = (in_g / gm) * BN;

    const int k_begin = blockIdx.z * kchunk;
    const int k_end = min(a.K, k_begin + kchunk);
    const int nk = k_end > k_begin ? (k_end - k_begin + BK - 1) / BK : 0;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    const int li = lane & 31, g = lane >> 5;

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[i][j][e] = 0.f;

    Tile<AKC> ta;
    Tile<BKC> tb;
    if (nk > 0) {
        ta.load(a.A, a.lda, m0, a.M, k_begin, k_end);
        tb.load(a.B, a.ldb, n0, a.N, k_begin, k_end);
        ta.store(smA[0]);
        tb.store(smB[0]);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; kt++) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            const int kn = k_begin + (kt + 1) * BK;
            ta.load(a.A, a.lda, m0, a.M, kn, k_end);
            tb.load(a.B, a.ldb, n0, a.N, kn, k_end);
        }
        const float* sa = smA[cur];
        const float* sb = smB[cur];
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const float4 a0 = Tile<AKC>::frag(sa, wm + li, g, q);
            const float4 a1 = Tile<AKC>::frag(sa, wm + 32 + li, g, q);
            const float4 b0 = Tile<BKC>::frag(sb, wn + li, g, q);
            const float4 b1 = Tile<BKC>::frag(sb, wn + 32 + li, g, q);
            acc[0][0] = mfma(a0.x, b0.x, acc[0][0]);
            acc[0][1] = mfma(a0.x, b1.x, acc[0][1]);
            acc[1][0] = mfma(a1.x, b0.x, acc[1][0]);
            acc[1][1] = mfma(a1.x, b1.x, acc[1][1]);
            acc[0][0] = mfma(a0.y, b0.y, acc[0][0]);
            acc[0][1] = mfma(a0.y, b1.y, acc[0][1]);
            acc[1][0] = mfma(a1.y, b0.y, acc[1][0]);
            acc[1][1] = mfma(a1.y, b1.y, acc[1][1]);
            acc[0][0] = mfma(a0.z, b0.z, acc[0][0]);
            acc[0][1] = mfma(a0.z, b1.z, acc[0][1]);
            acc[1][0] = mfma(a1.z, b0.z, acc[1][0]);
            acc[1][1] = mfma(a1.z, b1.z, acc[1][1]);
            acc[0][0] = mfma(a0.w, b0.w, acc[0][0]);
            acc[0][1] = mfma(a0.w, b1.w, acc[0][1]);
            acc[1][0] = mfma(a1.w, b0.w, acc[1][0]);
            acc[1][1] = mfma(a1.w, b1.w, acc[1][1]);
        }
        if (kt + 1 < nk) {
            ta.store(smA[cur ^ 1]);
            tb.store(smB[cur ^ 1]);
        }
        __syncthreads();
    }

    // 32x32 accumulator layout: lane holds column li, rows 8*(e/4) + 4*g + e%4
#pragma unroll
    for (int bn = 0; bn < 2; bn++) {
        const int col = n0 + wn + 32 * bn + li;
        if (col >= a.N) continue;
        float bcol = 0.f;
        if (EPI == EPI_RESID || EPI == EPI_GELU || (EPI == EPI_STORE && a.bias))
            bcol = a.bias[col];
#pragma unroll
        for (int bm = 0; bm < 2; bm++) {
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int row = m0 + wm + 32 * bm + 8 * (e >> 2) + 4 * g + (e & 3);
                if (row >= a.M) continue;
                const float v = acc[bm][bn][e];
                if (EPI == EPI_PARTIAL) {
                    partial[(int64_t)blockIdx.z * a.M * a.N + (int64_t)row * a.N + col] = v;
                } else {
                    const int64_t idx = (int64_t)row * a.ldc + col;
                    if (EPI == EPI_STORE) {
                        a.C[idx] = v + bcol;
                    } else if (EPI == EPI_RESID) {
                        a.C[idx] = v + bcol + a.aux[(int64_t)row * a.ldaux + col];
                    } else if (EPI == EPI_GELU) {
                        const float pre = v + bcol;
                        a.C[idx] = pre;
                        a.out2[idx] = gelu_f(pre);
                    } else if (EPI == EPI_GELU_BWD) {
                        a.C[idx] = v * gelu_grad_f(a.aux[(int64_t)row * a.ldaux + col]);
                    } else if (EPI == EPI_ACCUM) {
                        a.C[idx] += v;
                    }
                }
            }
        }
    }
}

// C (+)= sum over splits of partial, in split order.  N % 4 == 0.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(
    float* __restrict__ C, int64_t ldc, const float* __restrict__ partial, int splits,
    int M, int N, int accumulate) {
    const int64_t n4 = (int64_t)M * (N / 4);
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / (N / 4);
        const int col = (int)(i - row * (N / 4)) * 4;
        float4 s = ld4(partial + row * N + col);
        for (int z = 1; z < splits; z++) {
            const float4 p = ld4(partial + (int64_t)z * M * N + row * N + col);
            s.x += p.x;
            s.y += p.y;
            s.z += p.z;
            s.w += p.w;
        }
        float* c = C + row * ldc + col;
        if (accumulate) {
            const float4 o = ld4(c);
            s.x += o.x;
            s.y += o.y;
            s.z += o.z;
            s.w += o.w;
        }
        st4(c, s);
    }
}

inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Split the reduction when there are too few output tiles to fill the chip
// (weight gradients of the C x C and 4C x C layers, whose K is B*T).
int choose_splits(int op, int M, int N, int K) {
    if (op != GEMM_TN || (N % 4) != 0) return 1;
    const int tiles = cdiv(M, BM) * cdiv(N, BN);
    const int target = 768;
    if (tiles >= target / 2) return 1;
    int splits = cdiv(target, tiles);
    const int max_splits = K / (BK * 4);  // at least 4 reduction steps each
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
    return splits;
}

int split_chunk(int K, int splits) {
    int c = cdiv(K, splits);
    return cdiv(c, BK) * BK;
}

template <int OP, int EPI>
hipError_t launch(hipStream_t s, const GemmArgs& a, int splits, float* ws) {
    const int tm = cdiv(a.M, BM), tn = cdiv(a.N, BN);
    const int chunk = splits > 1 ? split_chunk(a.K, splits) : (a.K > 0 ? a.K : 1);
    const int nz = splits > 1 ? cdiv(a.K, chunk) : 1;
    dim3 grid(tm * tn, 1, nz);
    hipLaunchKernelGGL((gemm_kernel<OP, EPI>), grid, dim3(NTHR), 0, s, a, tm, tn, chunk,
                       ws);
    return hipGetLastError();
}

}  // namespace

size_t gemm_workspace_bytes(int op, int M, int N, int K) {
    const int splits = choose_splits(op, M, N, K);
    if (splits <= 1) return 0;
    const int chunk = split_chunk(K, splits);
    const int nz = cdiv(K, chunk);
    return (size_t)nz * M * N * sizeof(float);
}

hipError_t gemm(hipStream_t s, const GemmArgs& a, float* ws, size_t ws_bytes) {
    if (a.M <= 0 || a.N <= 0) return hipSuccess;
    int splits = choose_splits(a.op, a.M, a.N, a.K);
    if (splits > 1 && gemm_workspace_bytes(a.op, a.M, a.N, a.K) > ws_bytes) splits = 1;
    if (splits > 1) {
        // only weight gradients are split; they store or accumulate
        if (a.epi != EPI_ACCUM && a.epi != EPI_STORE) return hipErrorInvalidValue;
        hipError_t e = launch<GEMM_TN, EPI_PARTIAL>(s, a, splits, ws);
        if (e != hipSuccess) return e;
        const int chunk = split_chunk(a.K, splits);
        const int nz = cdiv(a.K, chunk);
        const int64_t n4 = (int64_t)a.M * (a.N / 4);
        int blocks = (int)std::min<int64_t>((n4 + 255) / 256, 4096);
        hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, s, a.C, a.ldc,
                           ws, nz, a.M, a.N, a.epi == EPI_ACCUM ? 1 : 0);
        return hipGetLastError();
    }
    switch (a.op) {
        case GEMM_NT:
            switch (a.epi) {
                case EPI_STORE: return launch<GEMM_NT, EPI_STORE>(s, a, 1, ws);
                case EPI_RESID: return launch<GEMM_NT, EPI_RESID>(s, a, 1, ws);
                case EPI_GELU: return launch<GEMM_NT, EPI_GELU>(s, a, 1, ws);
                default: return hipErrorInvalidValue;
            }
        case GEMM_NN:
            switch (a.epi) {
                case EPI_STORE: return launch<GEMM_NN, EPI_STORE>(s, a, 1, ws);
                case EPI_GELU_BWD: return launch<GEMM_NN, EPI_GELU_BWD>(s, a, 1, ws);
                default: return hipErrorInvalidValue;
            }
        case GEMM_TN:
            switch (a.epi) {
                case EPI_STORE: return launch<GEMM_TN, EPI_STORE>(s, a, 1, ws);
                case EPI_ACCUM: return launch<GEMM_TN, EPI_ACCUM>(s, a, 1, ws);
                default: return hipErrorInvalidValue;
            }
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gk
