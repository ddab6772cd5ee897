// fp32 matrix multiply on the CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// Every linear layer of the model (QKV, attention projection, MLP fc and
// projection, tied LM head) runs its forward, input-gradient and
// weight-gradient products here (ujoy.net article "徒手用 1000 行 C 语言实现",
// section "用C语言实现LLM": the matmul layer, forward and backward).
//
// Tiling: a 256-thread workgroup owns a 128x128 output tile; its four waves
// each own 64x64 (2x2 blocks of the 32x32 MFMA).  The reduction runs in
// steps of BK (16, or 32 for the LM head's long-K input gradient) staged
// through two LDS buffers (one barrier per step) while the global loads of
// the step after next are in flight in registers.  Within a step the two
// 32-lane halves of a wave own k = 0..BK/2-1 and k = BK/2..BK-1, so an
// operand stored k-contiguous is read from LDS as float4 (four MFMA steps
// per read).  The main loop loads only whole reduction steps, with rows past
// the matrix clamped to its last row, so every step issues the same loads
// and the wait for the registers of the previous step is exact; a partial
// last step is loaded with zero padding after the loop.
//
// Operands whose reduction index is contiguous in HBM are stored in LDS as
// [row][k] (rows of BK floats, padded by 4 floats after every 256 bytes);
// operands whose free index is contiguous are stored as [k][row] (132-float
// rows).  Both are written with float4 and read without bank conflicts.
// At BK = 16 the workgroup needs 35 KB of LDS and at most 168 VGPRs, so
// three share a compute unit.
//
// The epilogue stages each wave's 64x64 block through LDS in two 32-row
// halves and then works along rows with float4 loads and stores, fusing
// what the layer does next: bias, residual add, GELU (writing both pre- and
// post-activation), the GELU derivative of the backward, or += into a
// gradient.  Large reductions over few output tiles are split over K into a
// workspace and summed in a fixed order by a second kernel, so results are
// deterministic.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

constexpr int BM = kGemmTile, BN = kGemmTile, NTHR = 256;
constexpr int PF = 2;            // register prefetch depth (tiles in flight)
constexpr int EPI_PARTIAL = 100; // internal: write split-K partial sums

__device__ __forceinline__ floatx16 mfma(float a, float b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <bool KC, int R, int NT, int BK>
struct Tile;

template <int R, int NT, int BK>
struct Tile<true, R, NT, BK> {
    // [row][k]: rows of BK floats in groups of G = 64 / BK rows (256 bytes,
    // all 64 banks) followed by 4 floats of padding.  A 16-lane float4 store
    // (G rows of whole steps) and a 16-lane fragment read (one float4 of 16
    // consecutive rows) then both touch 16 distinct groups of four banks.
    static constexpr int G = 64 / BK;
    static_assert(64 % BK == 0 && R % G == 0, "whole row groups");
    static constexpr int KV = BK / 4;     // float4 per row per step
    static constexpr int FLOATS = R * BK + (R / G) * 4;
    static __device__ __forceinline__ int off(int r) { return r * BK + (r / G) * 4; }
    static constexpr int PER = R * KV / NT;
    float4 v[PER];
    // Rows past the matrix read its last row instead (their products land
    // only in outputs that are never stored).  TAIL loads a last, partial
    // step of the reduction and zeroes k >= K; the main loop loads only
    // whole steps and so always issues the same loads.
    template <bool TAIL>
    __device__ __forceinline__ void load(const float* __restrict__ g, int64_t ld, int r0, int Rn,
                                         int k0, int K) {
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int idx = threadIdx.x + NT * i;
            const int r = min(r0 + idx / KV, Rn - 1);
            const int k = k0 + (idx % KV) * 4;
            if (!TAIL) {
                v[i] = ld4(g + (int64_t)r * ld + k);
            } else {
                float4 x = ld4(g + (int64_t)r * ld + (k < K ? k : 0));
                x.x = k < K ? x.x : 0.f;
                x.y = k + 1 < K ? x.y : 0.f;
                x.z = k + 2 < K ? x.z : 0.f;
                x.w = k + 3 < K ? x.w : 0.f;
                v[i] = x;
            }
        }
    }
    __device__ __forceinline__ void store(float* s) const {
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int idx = threadIdx.x + NT * i;
            st4(s + off(idx / KV) + (idx % KV) * 4, v[i]);
        }
    }
    __device__ static __forceinline__ float4 frag(const float* s, int r, int g, int q) {
        return ld4(s + off(r) + (BK / 2) * g + 4 * q);
    }
};

template <int R, int NT, int BK>
struct Tile<false, R, NT, BK> {
    static constexpr int LDK = R + 4;
    static constexpr int FLOATS = BK * LDK;
    static constexpr int PER = BK * R / 4 / NT;
    static constexpr int R4 = R / 4;
    float4 v[PER];
    // A float4 that starts inside the matrix but runs past its last row
    // reads the row's padding (leading dimensions are multiples of 4); one
    // that starts past it reads the last whole float4 instead.
    template <bool TAIL>
    __device__ __forceinline__ void load(const float* __restrict__ g, int64_t ld, int r0, int Rn,
                                         int k0, int K) {
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int idx = threadIdx.x + NT * i;
            const int k = k0 + idx / R4;
            int r = r0 + (idx % R4) * 4;
            r = r < Rn ? r : ((Rn - 1) & ~3);
            if (!TAIL) {
                v[i] = ld4(g + (int64_t)k * ld + r);
            } else {
                const float4 x = ld4(g + (int64_t)(k < K ? k : 0) * ld + r);
                v[i] = k < K ? x : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    }
    __device__ __forceinline__ void store(float* s) const {
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int idx = threadIdx.x + NT * i;
            st4(s + (idx / R4) * LDK + (idx % R4) * 4, v[i]);
        }
    }
    __device__ static __forceinline__ float4 frag(const float* s, int r, int g, int q) {
        const float* p = s + ((BK / 2) * g + 4 * q) * LDK + r;
        return make_float4(p[0], p[LDK], p[2 * LDK], p[3 * LDK]);
    }
};

// Returns the values stored into C (used for the EPI_GELU_BWD column sums).
template <int EPI>
__device__ __forceinline__ float4 epi_store(const GemmArgs& a, float* __restrict__ partial,
                                            int row, int col, float4 v) {
    if (EPI == EPI_PARTIAL) {
        st4(partial + (int64_t)row * a.N + col, v);
        return v;
    }
    float* c = a.C + (int64_t)row * a.ldc + col;
    if (EPI == EPI_ACCUM) {
        const float4 o = ld4(c);
        st4(c, make_float4(o.x + v.x, o.y + v.y, o.z + v.z, o.w + v.w));
        return v;
    }
    if (EPI == EPI_GELU_BWD) {
        const float4 x = ld4(a.aux + (int64_t)row * a.ldaux + col);
        const float4 o = make_float4(v.x * gelu_grad_f(x.x), v.y * gelu_grad_f(x.y),
                                     v.z * gelu_grad_f(x.z), v.w * gelu_grad_f(x.w));
        st4(c, o);
        return o;
    }
    float4 bb = make_float4(0.f, 0.f, 0.f, 0.f);
    if (EPI != EPI_STORE || a.bias) bb = ld4(a.bias + col);
    v = make_float4(v.x + bb.x, v.y + bb.y, v.z + bb.z, v.w + bb.w);
    if (EPI == EPI_RESID) {
        const float4 x = ld4(a.aux + (int64_t)row * a.ldaux + col);
        v = make_float4(v.x + x.x, v.y + x.y, v.z + x.z, v.w + x.w);
    }
    st4(c, v);
    if (EPI == EPI_GELU)
        st4(a.out2 + (int64_t)row * a.ldc + col,
            make_float4(gelu_f(v.x), gelu_f(v.y), gelu_f(v.z), gelu_f(v.w)));
    return v;
}

template <int EPI>
__device__ __forceinline__ float epi_scalar(const GemmArgs& a, float* __restrict__ partial,
                                            int row, int col, float v) {
    if (EPI == EPI_PARTIAL) {
        partial[(int64_t)row * a.N + col] = v;
        return v;
    }
    const int64_t idx = (int64_t)row * a.ldc + col;
    if (EPI == EPI_ACCUM) { a.C[idx] += v; return v; }
    if (EPI == EPI_GELU_BWD) {
        const float o = v * gelu_grad_f(a.aux[(int64_t)row * a.ldaux + col]);
        a.C[idx] = o;
        return o;
    }
    float bb = 0.f;
    if (EPI != EPI_STORE || a.bias) bb = a.bias[col];
    v += bb;
    if (EPI == EPI_RESID) v += a.aux[(int64_t)row * a.ldaux + col];
    a.C[idx] = v;
    if (EPI == EPI_GELU) a.out2[idx] = gelu_f(v);
    return v;
}

template <int OP, int EPI, int BK>
__global__ __launch_bounds__(NTHR, BK == 16 ? 3 : 2) void gemm_kernel(
    const GemmArgs a, int tiles_m, int tiles_n, int kchunk, float* __restrict__ partial) {
    constexpr int NT = NTHR;
    constexpr bool AKC = (OP != GEMM_TN);
    constexpr bool BKC = (OP == GEMM_NT);
    using TA = Tile<AKC, BM, NT, BK>;
    using TB = Tile<BKC, BN, NT, BK>;
    constexpr int MAIN = 2 * (TA::FLOATS + TB::FLOATS);
    constexpr int EPIF = (NT / 64) * 32 * 68;  // epilogue staging, one 32x68 half-block per wave
    constexpr int SMEM = MAIN > EPIF ? MAIN : EPIF;
    __shared__ __attribute__((aligned(16))) float sm[SMEM];

    int tile, kz;
    split_remap(blockIdx.x, blockIdx.z, tiles_m * tiles_n, gridDim.z, tile, kz);
    constexpr int GM = 8;
    const int per_group = GM * tiles_n;
    const int group = tile / per_group;
    const int first_m = group * GM;
    const int gm = min(tiles_m - first_m, GM);
    const int in_g = tile - group * per_group;
    const int m0 = (first_m + in_g % gm) * BM;
    const int n0 = (in_g / gm) * BN;

    const int k_begin = kz * kchunk;
    // this split's partial-sum slice (EPI_PARTIAL)
    float* const part = EPI == EPI_PARTIAL ? partial + (int64_t)kz * a.M * a.N : nullptr;
    const int k_end = min(a.K, k_begin + kchunk);

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

    TA ta[PF];
    TB tb[PF];
    const int nfull = (k_end - k_begin) / BK;  // whole reduction steps
    // Every step of the main loop issues the same loads (past the last
    // whole step it reloads that step, never stored), so the wait for the
    // previous step's registers is exact and two steps of loads stay in
    // flight.
    auto issue = [&](auto slotc, int kt) {
        constexpr int S = decltype(slotc)::value;
        const int kk = k_begin + min(kt, nfull - 1) * BK;
        ta[S].template load<false>(a.A, a.lda, m0, a.M, kk, k_end);
        tb[S].template load<false>(a.B, a.ldb, n0, a.N, kk, k_end);
    };
    auto compute = [&](const float* sa, const float* sb) {
#pragma unroll
        for (int q = 0; q < BK / 8; q++) {
            const float4 a0 = TA::frag(sa, wm + li, g, q);
            const float4 a1 = TA::frag(sa, wm + 32 + li, g, q);
            const float4 b0 = TB::frag(sb, wn + li, g, q);
            const float4 b1 = TB::frag(sb, wn + 32 + li, g, q);
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
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    if (nfull > 0) {
        issue(I0{}, 0);
        ta[0].store(sm);
        tb[0].store(sm + 2 * TA::FLOATS);
        issue(I1{}, 1);
    }
    __syncthreads();
    // Tile j's registers live in slot j & 1: while step j computes from LDS,
    // tile j+2 is loading into the slot step j-1 just emptied into LDS.
    auto step = [&](int kt, auto slotc) {
        constexpr int S = decltype(slotc)::value;
        constexpr int NS = S ^ 1;
        const int cur = kt & 1;
        issue(slotc, kt + 2);
        compute(sm + cur * TA::FLOATS, sm + 2 * TA::FLOATS + cur * TB::FLOATS);
        // Unconditional, so that no path reaches the next step's loads with
        // this slot still pending (after the last step the buffer is unused).
        ta[NS].store(sm + (cur ^ 1) * TA::FLOATS);
        tb[NS].store(sm + 2 * TA::FLOATS + (cur ^ 1) * TB::FLOATS);
        __syncthreads();
    };
    int kt = 0;
    for (; kt + 1 < nfull; kt += 2) {
        step(kt, I0{});
        step(kt + 1, I1{});
    }
    if (kt < nfull) step(kt, I0{});
    if (k_begin + nfull * BK < k_end) {  // partial last step, zero-padded
        const int kk = k_begin + nfull * BK;
        ta[0].template load<true>(a.A, a.lda, m0, a.M, kk, k_end);
        tb[0].template load<true>(a.B, a.ldb, n0, a.N, kk, k_end);
        ta[0].store(sm);
        tb[0].store(sm + 2 * TA::FLOATS);
        __syncthreads();
        compute(sm, sm + 2 * TA::FLOATS);
        __syncthreads();
    }

    // Stage this wave's 64x64 block in LDS one 32-row half at a time (the
    // main loop's buffers are free after its last barrier), then apply the
    // epilogue along rows with float4.
    float* ws = sm + wave * 32 * 68;
    // EPI_GELU_BWD column sums: a lane keeps columns 4*(lane & 15) .. +3 of
    // the wave's block through both halves
    const bool csum = EPI == EPI_GELU_BWD && a.colsum != nullptr;
    float4 cs = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int bm = 0; bm < 2; bm++) {
        if (bm == 1) __syncthreads();  // every wave has read its first half
#pragma unroll
        for (int bn = 0; bn < 2; bn++)
#pragma unroll
            for (int e = 0; e < 16; e++)
                ws[(8 * (e >> 2) + 4 * g + (e & 3)) * 68 + 32 * bn + li] = acc[bm][bn][e];
        __syncthreads();
#pragma unroll 4
        for (int j = 0; j < 8; j++) {
            const int idx = lane + 64 * j;
            const int r = idx >> 4, c4 = (idx & 15) * 4;
            const float4 v = ld4(ws + r * 68 + c4);
            const int row = m0 + wm + 32 * bm + r, col = n0 + wn + c4;
            if (row >= a.M) continue;
            float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
            if (col + 3 < a.N) {
                o = epi_store<EPI>(a, part, row, col, v);
            } else {
                if (col < a.N) o.x = epi_scalar<EPI>(a, part, row, col, v.x);
                if (col + 1 < a.N) o.y = epi_scalar<EPI>(a, part, row, col + 1, v.y);
                if (col + 2 < a.N) o.z = epi_scalar<EPI>(a, part, row, col + 2, v.z);
            }
            if (csum) {
                cs.x += o.x;
                cs.y += o.y;
                cs.z += o.z;
                cs.w += o.w;
            }
        }
    }
    if (csum) {
        // the four lanes that share columns, added in a fixed order
#pragma unroll
        for (int off = 16; off < 64; off <<= 1) {
            cs.x += __shfl_xor(cs.x, off, WAVE);
            cs.y += __shfl_xor(cs.y, off, WAVE);
            cs.z += __shfl_xor(cs.z, off, WAVE);
            cs.w += __shfl_xor(cs.w, off, WAVE);
        }
        const int col = n0 + wn + (lane & 15) * 4;
        if (lane < 16 && m0 + wm < a.M) {
            float* p = a.colsum + (int64_t)((m0 + wm) >> 6) * a.N + col;
            if (col + 3 < a.N) {
                st4(p, cs);
            } else {
                if (col < a.N) p[0] = cs.x;
                if (col + 1 < a.N) p[1] = cs.y;
                if (col + 2 < a.N) p[2] = cs.z;
            }
        }
    }
}

// Sum of the split-K partials in split order, then the epilogue of the
// matmul (store with optional bias, residual add, or += into a gradient).
// N % 4 == 0.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const GemmArgs a,
                                                            const float* __restrict__ partial,
                                                            int splits) {
    // One group of four outputs per thread over a grid that covers them all
    // (the host keeps M * N / 4 below 2^31); the partial sums of a group are
    // loaded four splits at a time, and added in split order.
    const int N4 = a.N / 4;
    const int64_t MN = (int64_t)a.M * a.N;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= a.M * N4) return;
    const int row = i / N4;
    const int col = (i - row * N4) * 4;
    const float* p0 = partial + (int64_t)row * a.N + col;
    float4 s = ld4(p0);
    int z = 1;
    for (; z + 3 < splits; z += 4) {
        const float4 q1 = ld4(p0 + z * MN), q2 = ld4(p0 + (z + 1) * MN),
                     q3 = ld4(p0 + (z + 2) * MN), q4 = ld4(p0 + (z + 3) * MN);
        s.x = (((s.x + q1.x) + q2.x) + q3.x) + q4.x;
        s.y = (((s.y + q1.y) + q2.y) + q3.y) + q4.y;
        s.z = (((s.z + q1.z) + q2.z) + q3.z) + q4.z;
        s.w = (((s.w + q1.w) + q2.w) + q3.w) + q4.w;
    }
    for (; z < splits; z++) {
        const float4 q = ld4(p0 + z * MN);
        s.x += q.x;
        s.y += q.y;
        s.z += q.z;
        s.w += q.w;
    }
    epi_store<EPI>(a, nullptr, (int)row, col, s);
}

}  // namespace

// Compute units of the current device (read once; 256 if unknown).
int device_cu_count() {
    static int cus = 0;
    if (!cus) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            n > 0)
            cus = n;
        else
            cus = 256;
    }
    return cus;
}

namespace {

// Reduction steps of 16 let three workgroups share a compute unit (40 KB of
// LDS each) and measured 2-5% faster on every product of the step but one:
// the input gradient of the LM head (K = V), whose A operand streams from
// HBM, keeps steps of 32 so that each row is fetched in 128-byte pieces.
template <int OP, int EPI>
hipError_t launch(hipStream_t s, const GemmArgs& a, int splits, float* ws) {
    const int tm = cdiv(a.M, BM), tn = cdiv(a.N, BN);
    const int chunk = splits > 1 ? gemm_split_chunk(a.K, splits) : (a.K > 0 ? a.K : 1);
    const int nz = splits > 1 ? cdiv(a.K, chunk) : 1;
    dim3 grid(tm * tn, 1, nz);
    if constexpr (OP == GEMM_NN) {
        if (a.K >= 8192) {
            launch((gemm_kernel<OP, EPI, 32>), grid, dim3(NTHR), 0, s, a, tm, tn, chunk, ws);
            return hipGetLastError();
        }
    }
    launch((gemm_kernel<OP, EPI, 16>), grid, dim3(NTHR), 0, s, a, tm, tn, chunk, ws);
    return hipGetLastError();
}

}  // namespace

template <int OP>
hipError_t launch_split(hipStream_t s, const GemmArgs& a, int splits, float* ws) {
    hipError_t e = launch<OP, EPI_PARTIAL>(s, a, splits, ws);
    if (e != hipSuccess) return e;
    const int nz = cdiv(a.K, gemm_split_chunk(a.K, splits));
    const int64_t n4 = (int64_t)a.M * (a.N / 4);
    if (n4 >= (int64_t)1 << 31) return hipErrorInvalidValue;
    const int blocks = (int)((n4 + 255) / 256);
    switch (a.epi) {
        case EPI_STORE:
            launch(splitk_reduce_kernel<EPI_STORE>, dim3(blocks), dim3(256), 0, s, a,
                               ws, nz);
            break;
        case EPI_RESID:
            launch(splitk_reduce_kernel<EPI_RESID>, dim3(blocks), dim3(256), 0, s, a,
                               ws, nz);
            break;
        case EPI_ACCUM:
            launch(splitk_reduce_kernel<EPI_ACCUM>, dim3(blocks), dim3(256), 0, s, a,
                               ws, nz);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t gemm(hipStream_t s, const GemmArgs& a, float* ws, size_t ws_bytes) {
    if (a.M <= 0 || a.N <= 0) return hipSuccess;
    // float4 access: leading dimensions are multiples of 4 and cover the
    // contiguous extent of each operand.
    if (((a.lda | a.ldb | a.ldc) & 3) != 0) return hipErrorInvalidValue;
    if (a.lda < (a.op == GEMM_TN ? a.M : a.K) || a.ldb < (a.op == GEMM_NT ? a.K : a.N) ||
        a.ldc < a.N)
        return hipErrorInvalidValue;
    const int cus = device_cu_count();
    int splits = gemm_choose_splits(a.op, a.epi, a.M, a.N, a.K, cus);
    if (splits > 1 && gemm_workspace_bytes(a.op, a.epi, a.M, a.N, a.K, cus) > ws_bytes)
        splits = 1;
    if (a.colsum) {
        if (a.epi != EPI_GELU_BWD) return hipErrorInvalidValue;
        splits = 1;  // the column sums are taken in the matmul's own epilogue
    }
    if (splits > 1) {
        switch (a.op) {
            case GEMM_NT: return launch_split<GEMM_NT>(s, a, splits, ws);
            case GEMM_NN: return launch_split<GEMM_NN>(s, a, splits, ws);
            case GEMM_TN: return launch_split<GEMM_TN>(s, a, splits, ws);
            default: return hipErrorInvalidValue;
        }
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
