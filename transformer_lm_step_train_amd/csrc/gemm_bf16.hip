// bf16 matrix multiply with fp32 accumulation on the CDNA4 matrix cores
// (v_mfma_f32_32x32x16_bf16), for the mixed-precision model: activations and
// weight copies in bf16, every sum in fp32 (ujoy.net article "徒手用 1000 行
// C 语言实现", section "用C语言实现LLM": the matmul layer; the reduced-precision
// extension is named by yinghuohong.cn, section "脚动完成每一个层前向/反向流传").
//
// The kernels share the operand conventions of the fp32 one (NT forward,
// NN input gradient, TN weight gradient) and its fused epilogues; outputs
// are bf16 activations or fp32 weight gradients (+=).  Which kernel takes a
// product (launch_h and launch_big at the end of the file):
//   - QKV and fc forwards, and input gradients with K >= 1536 or N >= 2048:
//     gemm_bf16_t128_lds_kernel (128x128, stages loaded straight into LDS);
//   - the LM-head forward: gemm_bf16_nt_stream_kernel (persistent 256x256);
//   - the other forwards with K < 2048 and input gradients:
//     gemm_bf16_k32_kernel (128x128, register-staged 32-deep steps);
//   - forwards with K >= 2048 and operands the above cannot take:
//     gemm_bf16_kernel (128x128, 64-deep steps);
//   - weight gradients and the LM-head input gradient (K split):
//     gemm_bf16_lds_kernel (256x256, stages straight into LDS), or
//     gemm_bf16_big_kernel when the split chunks are not whole stages or
//     the operands not 16-byte aligned; splitk_reduce_bf16_kernel sums the
//     splits in order.
// The kernels that can take the same product (with the same K split) add
// the same k in the same order, so they give bitwise-equal results.
//
// The forward and input-gradient products use a 128x128 output tile per
// 256-thread workgroup, 64x64 per wave (2x2 blocks of the 32x32 MFMA), and
// reduction steps staged through two LDS buffers with a two-deep register
// prefetch (whole steps only in the main loop, rows past the matrix clamped
// to its last row; a partial last step is zero-padded after the loop).
// Operands contiguous in k are stored [row][k] in LDS, so each MFMA operand
// (8 consecutive k of one row) is one 16-byte read.  The B operand of the
// input gradients (NN: the weight, contiguous along n) stays [k][n] in LDS
// and is read with gfx950's transposing LDS loads (frag_tr below).
//   - Steps of 32, three workgroups per CU: the forward products with
//     K < 2048 and the input gradients whose weight allows the transposing
//     reads (gemm_bf16_k32_kernel).
//   - Steps of 64, two workgroups per CU: the rest (gemm_bf16_kernel), where
//     operands contiguous in the free index are loaded as 8 rows of k by 4
//     columns per thread and transposed in registers before the LDS store.
//
// Weight gradients and the LM-head input gradient split K and take the
// 256x256 kernel further below.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

constexpr int BM = 128, BN = 128, BK = 64, NTHR = 256;
static_assert(BK == kGemm16Step, "the split plan counts 64-deep steps");
constexpr int LDH = BK + 8;       // LDS row stride, bf16 elements (144 bytes)
constexpr int EPI_PARTIAL = 100;  // internal: fp32 split-K partial sums

template <bool KC>
struct TileH;

// Reduction index contiguous: element (r, k) at g[r*ld + k].  Thread loads
// 8 consecutive k of one row (16 bytes).
template <>
struct TileH<true> {
    static constexpr int ELEMS = 128 * LDH;
    uint4 v[4];
    // Rows past the matrix read its last row (their products reach only
    // outputs that are never stored); TAIL zeroes k >= K of a partial last
    // reduction step.
    template <bool TAIL>
    __device__ __forceinline__ void load(const uint16_t* __restrict__ g, int64_t ld, int r0,
                                         int R, int k0, int K) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int idx = threadIdx.x + NTHR * i;
            const int r = min(r0 + (idx >> 3), R - 1);
            const int k = k0 + (idx & 7) * 8;
            if (!TAIL) {
                v[i] = *reinterpret_cast<const uint4*>(g + (int64_t)r * ld + k);
            } else {
                const uint4 x =
                    *reinterpret_cast<const uint4*>(g + (int64_t)r * ld + (k < K ? k : 0));
                const uint32_t w[4] = {x.x, x.y, x.z, x.w};
                uint32_t o[4];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const uint32_t lo = k + 2 * j < K ? (w[j] & 0xFFFFu) : 0u;
                    const uint32_t hi = k + 2 * j + 1 < K ? (w[j] & 0xFFFF0000u) : 0u;
                    o[j] = lo | hi;
                }
                v[i] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    }
    __device__ __forceinline__ void store(uint16_t* s) const {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int idx = threadIdx.x + NTHR * i;
            *reinterpret_cast<uint4*>(s + (idx >> 3) * LDH + (idx & 7) * 8) = v[i];
        }
    }
};

// Free index contiguous: element (r, k) at g[k*ld + r].  Thread loads 4
// consecutive rows at each of 8 consecutive k (8 bytes each) and stores the 4
// rows' 8-k runs after a register transpose.
template <>
struct TileH<false> {
    static constexpr int ELEMS = 128 * LDH;
    uint2 v[8];
    // A run of 4 that starts inside the matrix but passes its last row reads
    // the row's padding (leading dimensions are multiples of 4); one that
    // starts past it reads the last whole run instead.
    template <bool TAIL>
    __device__ __forceinline__ void load(const uint16_t* __restrict__ g, int64_t ld, int r0,
                                         int R, int k0, int K) {
        const int t = threadIdx.x;
        int r = r0 + (t & 31) * 4;
        r = r < R ? r : ((R - 1) & ~3);
        const int kb = k0 + (t >> 5) * 8;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int k = kb + i;
            if (!TAIL) {
                v[i] = *reinterpret_cast<const uint2*>(g + (int64_t)k * ld + r);
            } else {
                const uint2 x = *reinterpret_cast<const uint2*>(g + (int64_t)(k < K ? k : 0) * ld + r);
                v[i] = k < K ? x : make_uint2(0u, 0u);
            }
        }
    }
    __device__ __forceinline__ void store(uint16_t* s) const {
        const int t = threadIdx.x;
        const int r = (t & 31) * 4;
        const int kb = (t >> 5) * 8;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            uint32_t e[8];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const uint32_t w = j < 2 ? v[i].x : v[i].y;
                e[i] = (w >> (16 * (j & 1))) & 0xFFFFu;
            }
            *reinterpret_cast<uint4*>(s + (r + j) * LDH + kb) =
                make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                           e[6] | (e[7] << 16));
        }
    }
};

__device__ __forceinline__ uint4 frag(const uint16_t* s, int r, int g, int q) {
    return *reinterpret_cast<const uint4*>(s + r * LDH + 16 * q + 8 * g);
}

// Free index contiguous, kept in LDS as it lies in HBM: [k][n], 16-byte runs
// of 8 consecutive n (leading dimension a multiple of 8, base 16-byte
// aligned).  The MFMA operand (8 consecutive k of one column) is gathered by
// two transposing LDS reads (ds_read_b64_tr_b16).  In each 16-lane group of
// such a read, lane r addresses 4 consecutive columns of one k-row, and lane
// j receives element j of each 16-element row of the group's 16x4 block.
// Lane r at (k0 + r/4, n0 + 4*(r%4)) therefore hands lane j the four values
// (k0..k0+3, n0 + j).
constexpr int LDN_T = BN + 16;  // LDS row stride along n of such a tile, bf16 elements

typedef short tr4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) tr4_t* lds_tr4_ptr;

// Operand of columns nb..nb+31 (lane li = column nb + li), k = 16q + 8g .. +7,
// from a [k][n] tile with row stride LDN_T.
__device__ __forceinline__ uint4 frag_tr(const uint16_t* s, int nb, int q, int lane) {
    const int grp = lane >> 4, r = lane & 15;
    const int n = nb + 16 * (grp & 1) + 4 * (r & 3);
    const int k = 16 * q + 8 * (grp >> 1) + (r >> 2);
    const uint16_t* p = s + k * LDN_T + n;
    const tr4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr4_ptr)p);
    const tr4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr4_ptr)(p + 4 * LDN_T));
    const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
    return make_uint4(a.x, a.y, b.x, b.y);
}

template <class H>
__device__ __forceinline__ float4 ld4h(const uint16_t* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(H::lo(u.x), H::hi(u.x), H::lo(u.y), H::hi(u.y));
}
template <class H>
__device__ __forceinline__ void st4h(uint16_t* p, float4 v) {
    *reinterpret_cast<uint2*>(p) = make_uint2(H::pk(v.x, v.y), H::pk(v.z, v.w));
}

// Epilogue on 4 consecutive columns.  bf16 outputs: STORE, RESID, GELU,
// GELU_BWD.  fp32 outputs: ACCUM (gradient +=), STORE when out_f32, PARTIAL.
// GELU_BWD returns the values as stored (for its column sums).
template <int EPI, class H>
__device__ __forceinline__ float4 epi4(const GemmArgsH& a, float* __restrict__ partial, int row,
                                       int col, float4 v) {
    if (EPI == EPI_PARTIAL) {  // partial: this split's M x N slice
        st4(partial + (int64_t)row * a.N + col, v);
        return v;
    }
    const int64_t idx = (int64_t)row * a.ldc + col;
    if (EPI == EPI_ACCUM) {
        float* c = reinterpret_cast<float*>(a.C) + idx;
        const float4 o = ld4(c);
        st4(c, make_float4(o.x + v.x, o.y + v.y, o.z + v.z, o.w + v.w));
        return v;
    }
    if (EPI == EPI_GELU_BWD) {
        const float4 x = ld4h<H>(a.aux + (int64_t)row * a.ldaux + col);
        const uint2 u = make_uint2(H::pk(v.x * gelu_grad_f(x.x), v.y * gelu_grad_f(x.y)),
                                   H::pk(v.z * gelu_grad_f(x.z), v.w * gelu_grad_f(x.w)));
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.C) + idx) = u;
        return make_float4(H::lo(u.x), H::hi(u.x), H::lo(u.y), H::hi(u.y));
    }
    if (EPI == EPI_RESID || EPI == EPI_GELU || (EPI == EPI_STORE && a.bias)) {
        const float4 bb = ld4(a.bias + col);
        v = make_float4(v.x + bb.x, v.y + bb.y, v.z + bb.z, v.w + bb.w);
    }
    if (EPI == EPI_RESID) {
        const float4 x = ld4h<H>(a.aux + (int64_t)row * a.ldaux + col);
        v = make_float4(v.x + x.x, v.y + x.y, v.z + x.z, v.w + x.w);
    }
    if (EPI == EPI_STORE && a.out_f32) {
        st4(reinterpret_cast<float*>(a.C) + idx, v);
        return v;
    }
    st4h<H>(reinterpret_cast<uint16_t*>(a.C) + idx, v);
    if (EPI == EPI_GELU)
        st4h<H>(a.out2 + idx, make_float4(gelu_f(v.x), gelu_f(v.y), gelu_f(v.z), gelu_f(v.w)));
    return v;
}

template <int EPI, class H>
__device__ __forceinline__ float epi1(const GemmArgsH& a, float* __restrict__ partial, int row,
                                      int col, float v) {
    if (EPI == EPI_PARTIAL) {
        partial[(int64_t)row * a.N + col] = v;
        return v;
    }
    const int64_t idx = (int64_t)row * a.ldc + col;
    if (EPI == EPI_ACCUM) {
        reinterpret_cast<float*>(a.C)[idx] += v;
        return v;
    }
    if (EPI == EPI_GELU_BWD) {
        const uint16_t o = H::h(v * gelu_grad_f(H::f(a.aux[(int64_t)row * a.ldaux + col])));
        reinterpret_cast<uint16_t*>(a.C)[idx] = o;
        return H::f(o);
    }
    if (EPI == EPI_RESID || EPI == EPI_GELU || (EPI == EPI_STORE && a.bias)) v += a.bias[col];
    if (EPI == EPI_RESID) v += H::f(a.aux[(int64_t)row * a.ldaux + col]);
    if (EPI == EPI_STORE && a.out_f32) {
        reinterpret_cast<float*>(a.C)[idx] = v;
        return v;
    }
    reinterpret_cast<uint16_t*>(a.C)[idx] = H::h(v);
    if (EPI == EPI_GELU) a.out2[idx] = H::h(gelu_f(v));
    return v;
}

// The epilogues that read an input of the output's shape (the residual of
// EPI_RESID, the GELU input of EPI_GELU_BWD) find it cold in HBM: it was
// written long before, and its loads, a few in flight per lane, would stall
// the epilogue.  Right after the main loop each thread of the 128x128
// workgroup loads one value of its tile's rows instead, so that all the
// tile's 128-byte lines (two per 256-byte row run) are requested at once
// while the accumulators go through LDS; the epilogue's own loads then hit
// in L2.  The value is consumed by an empty asm at the kernel's end so the
// load stays.  Measured with caches flushed before each launch, the GELU'
// input gradient went from 170 to 149 us and the attention projection from
// 57 to 47 us, with bitwise-equal outputs.
template <int EPI>
__device__ __forceinline__ uint32_t touch_aux_tile(const GemmArgsH& a, int m0, int n0) {
    static_assert(NTHR == 256 && BM == 128 && BN == 128, "two lines per row of the tile");
    if constexpr (EPI == EPI_GELU_BWD || EPI == EPI_RESID) {
        const int r = min(m0 + (int)(threadIdx.x >> 1), a.M - 1);
        const int c = min(n0 + 64 * (int)(threadIdx.x & 1), a.N - 1);
        return a.aux[(int64_t)r * a.ldaux + c];
    }
    return 0u;
}

template <int OP, int EPI, class H>
__global__ __launch_bounds__(NTHR, 2) void gemm_bf16_kernel(const GemmArgsH a, int tiles_m,
                                                            int tiles_n, int kchunk,
                                                            float* __restrict__ partial) {
    constexpr bool AKC = (OP != GEMM_TN);
    constexpr bool BKC = (OP == GEMM_NT);
    using TA = TileH<AKC>;
    using TB = TileH<BKC>;
    constexpr int MAIN_BYTES = 2 * (TA::ELEMS + TB::ELEMS) * 2;
    constexpr int EPI_BYTES = 4 * 64 * 68 * 4;
    constexpr int SMEM = MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES;
    __shared__ __attribute__((aligned(16))) unsigned char smraw[SMEM];
    uint16_t* smh = reinterpret_cast<uint16_t*>(smraw);

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
    float* const part = EPI == EPI_PARTIAL ? partial + (int64_t)blockIdx.z * a.M * a.N : nullptr;
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

    TA ta[2];
    TB tb[2];
    const int nfull = (k_end - k_begin) / BK;  // whole reduction steps
    // Every main-loop step issues the same loads (past the last whole step
    // it reloads that step), so the wait for the previous step's registers
    // is exact and two steps of loads stay in flight.
    auto issue = [&](auto slotc, int kt) {
        constexpr int S = decltype(slotc)::value;
        const int kk = k_begin + min(kt, nfull - 1) * BK;
        ta[S].template load<false>(a.A, a.lda, m0, a.M, kk, k_end);
        tb[S].template load<false>(a.B, a.ldb, n0, a.N, kk, k_end);
    };
    auto compute = [&](const uint16_t* sa, const uint16_t* sb) {
#pragma unroll
        for (int q = 0; q < BK / 16; q++) {
            const uint4 a0 = frag(sa, wm + li, g, q);
            const uint4 a1 = frag(sa, wm + 32 + li, g, q);
            const uint4 b0 = frag(sb, wn + li, g, q);
            const uint4 b1 = frag(sb, wn + 32 + li, g, q);
            acc[0][0] = H::mma(a0, b0, acc[0][0]);
            acc[0][1] = H::mma(a0, b1, acc[0][1]);
            acc[1][0] = H::mma(a1, b0, acc[1][0]);
            acc[1][1] = H::mma(a1, b1, acc[1][1]);
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    if (nfull > 0) {
        issue(I0{}, 0);
        ta[0].store(smh);
        tb[0].store(smh + 2 * TA::ELEMS);
        issue(I1{}, 1);
    }
    __syncthreads();
    auto step = [&](int kt, auto slotc) {
        constexpr int S = decltype(slotc)::value;
        constexpr int NS = S ^ 1;
        const int cur = kt & 1;
        issue(slotc, kt + 2);
        compute(smh + cur * TA::ELEMS, smh + 2 * TA::ELEMS + cur * TB::ELEMS);
        // unconditional: no path reaches the next loads with this slot pending
        ta[NS].store(smh + (cur ^ 1) * TA::ELEMS);
        tb[NS].store(smh + 2 * TA::ELEMS + (cur ^ 1) * TB::ELEMS);
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
        ta[0].store(smh);
        tb[0].store(smh + 2 * TA::ELEMS);
        __syncthreads();
        compute(smh, smh + 2 * TA::ELEMS);
        __syncthreads();
    }

    const uint32_t aux_touch = touch_aux_tile<EPI>(a, m0, n0);
    // stage each wave's 64x64 fp32 block in LDS, then work along rows;
    // EPI_GELU_BWD column sums: a lane keeps columns 4*(lane & 15) .. +3
    const bool csum = EPI == EPI_GELU_BWD && a.colsum != nullptr;
    float4 cs = make_float4(0.f, 0.f, 0.f, 0.f);
    float* ws = reinterpret_cast<float*>(smraw) + wave * 64 * 68;
#pragma unroll
    for (int bm = 0; bm < 2; bm++)
#pragma unroll
        for (int bn = 0; bn < 2; bn++)
#pragma unroll
            for (int e = 0; e < 16; e++)
                ws[(32 * bm + 8 * (e >> 2) + 4 * g + (e & 3)) * 68 + 32 * bn + li] = acc[bm][bn][e];
    __syncthreads();
#pragma unroll 4
    for (int j = 0; j < 16; j++) {
        const int idx = lane + 64 * j;
        const int r = idx >> 4, c4 = (idx & 15) * 4;
        const float4 v = ld4(ws + r * 68 + c4);
        const int row = m0 + wm + r, col = n0 + wn + c4;
        if (row >= a.M) continue;
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        if (col + 3 < a.N) {
            o = epi4<EPI, H>(a, part, row, col, v);
        } else {
            if (col < a.N) o.x = epi1<EPI, H>(a, part, row, col, v.x);
            if (col + 1 < a.N) o.y = epi1<EPI, H>(a, part, row, col + 1, v.y);
            if (col + 2 < a.N) o.z = epi1<EPI, H>(a, part, row, col + 2, v.z);
        }
        if (csum) {
            cs.x += o.x;
            cs.y += o.y;
            cs.z += o.z;
            cs.w += o.w;
        }
    }
    if (csum) {
        // the four lanes that share columns, added in a fixed order; one
        // partial row per 64 output rows
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
    asm volatile("" ::"v"(aux_touch));
}

// ---- 32-deep reduction steps, three workgroups per CU --------------------
//
// The same 128x128 tile and wave layout with reduction steps of 32: 40 KB of
// LDS (rows of 40 bf16, 80 bytes, keep the 16-byte reads aligned) and 134
// VGPRs, so three workgroups share a compute unit and each waits less on
// its own barrier.  The epilogue stages each wave's block in two 32-row
// halves to stay inside that LDS.  Bit-identical to the 64-step kernel (the
// MFMAs see the same k order); 6% faster over the step's NT and NN shapes,
// except the forward at K = 3072, which stays on the 64-step kernel.
constexpr int SBK = 32, LDHS = SBK + 8;

// Reduction index contiguous: [row][k], rows of LDHS.
struct TileH32 {
    static constexpr int ELEMS = 128 * LDHS;
    uint4 v[2];
    template <bool TAIL>
    __device__ __forceinline__ void load(const uint16_t* __restrict__ g, int64_t ld, int r0,
                                         int R, int k0, int K) {
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int idx = threadIdx.x + NTHR * i;
            const int r = min(r0 + (idx >> 2), R - 1);
            const int k = k0 + (idx & 3) * 8;
            if (!TAIL) {
                v[i] = *reinterpret_cast<const uint4*>(g + (int64_t)r * ld + k);
            } else {
                const uint4 x =
                    *reinterpret_cast<const uint4*>(g + (int64_t)r * ld + (k < K ? k : 0));
                const uint32_t w[4] = {x.x, x.y, x.z, x.w};
                uint32_t o[4];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const uint32_t lo = k + 2 * j < K ? (w[j] & 0xFFFFu) : 0u;
                    const uint32_t hi = k + 2 * j + 1 < K ? (w[j] & 0xFFFF0000u) : 0u;
                    o[j] = lo | hi;
                }
                v[i] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    }
    __device__ __forceinline__ void store(uint16_t* s) const {
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int idx = threadIdx.x + NTHR * i;
            *reinterpret_cast<uint4*>(s + (idx >> 2) * LDHS + (idx & 3) * 8) = v[i];
        }
    }
    __device__ static __forceinline__ uint4 frag(const uint16_t* s, int r, int g, int q) {
        return *reinterpret_cast<const uint4*>(s + r * LDHS + 16 * q + 8 * g);
    }
};

// Free index contiguous, [k][n] (read with frag_tr), 32 k-rows: a thread
// moves 16-byte runs of 8 consecutive n.  Runs past the last column read the
// last whole run instead (their products reach only outputs that are never
// stored); TAIL zeroes k >= K of a partial last reduction step.
struct TileT32 {
    static constexpr int ELEMS = SBK * LDN_T;
    uint4 v[2];
    template <bool TAIL>
    __device__ __forceinline__ void load(const uint16_t* __restrict__ g, int64_t ld, int n0,
                                         int N, int k0, int K) {
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int idx = threadIdx.x + NTHR * i;
            const int k = k0 + (idx >> 4);
            int n = n0 + (idx & 15) * 8;
            n = n < N ? n : ((N - 1) & ~7);
            if (!TAIL) {
                v[i] = *reinterpret_cast<const uint4*>(g + (int64_t)k * ld + n);
            } else {
                const uint4 x = *reinterpret_cast<const uint4*>(g + (int64_t)(k < K ? k : 0) * ld + n);
                v[i] = k < K ? x : make_uint4(0u, 0u, 0u, 0u);
            }
        }
    }
    __device__ __forceinline__ void store(uint16_t* s) const {
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int idx = threadIdx.x + NTHR * i;
            *reinterpret_cast<uint4*>(s + (idx >> 4) * LDN_T + (idx & 15) * 8) = v[i];
        }
    }
};

// NT, or NN with the B operand read through the transposing loads.
// NT, or NN with the B operand read through the transposing loads.
template <int OP, int EPI, class H, int PF>
__global__ __launch_bounds__(NTHR, 3) void gemm_bf16_k32_kernel(const GemmArgsH a, int tiles_m,
                                                               int tiles_n) {
    static_assert(OP == GEMM_NT || OP == GEMM_NN, "NT, or NN with the transposing reads");
    using TA = TileH32;
    using TB = std::conditional_t<OP == GEMM_NN, TileT32, TileH32>;
    constexpr int MAIN_BYTES = 2 * (TA::ELEMS + TB::ELEMS) * 2;
    constexpr int EPI_BYTES = 4 * 32 * 68 * 4;
    constexpr int SMEM = MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES;
    __shared__ __attribute__((aligned(16))) unsigned char smraw[SMEM];
    uint16_t* smh = reinterpret_cast<uint16_t*>(smraw);

    const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    constexpr int GM = 8;
    const int per_group = GM * tiles_n;
    const int group = tile / per_group;
    const int first_m = group * GM;
    const int gm = min(tiles_m - first_m, GM);
    const int in_g = tile - group * per_group;
    const int m0 = (first_m + in_g % gm) * BM;
    const int n0 = (in_g / gm) * BN;

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

    // PF register slots of global loads in flight: the loads of step kt + PF
    // are issued while step kt computes
    static_assert(PF == 2 || PF == 3, "prefetch depth");
    TA ta[PF];
    TB tb[PF];
    const int nfull = a.K / SBK;
    auto issue = [&](auto slotc, int kt) {
        constexpr int S = decltype(slotc)::value;
        const int kk = min(kt, nfull - 1) * SBK;
        ta[S].template load<false>(a.A, a.lda, m0, a.M, kk, a.K);
        tb[S].template load<false>(a.B, a.ldb, n0, a.N, kk, a.K);
    };
    auto compute = [&](const uint16_t* sa, const uint16_t* sb) {
#pragma unroll
        for (int q = 0; q < SBK / 16; q++) {
            const uint4 a0 = TA::frag(sa, wm + li, g, q);
            const uint4 a1 = TA::frag(sa, wm + 32 + li, g, q);
            uint4 b0, b1;
            if constexpr (OP == GEMM_NN) {
                b0 = frag_tr(sb, wn, q, lane);
                b1 = frag_tr(sb, wn + 32, q, lane);
            } else {
                b0 = TB::frag(sb, wn + li, g, q);
                b1 = TB::frag(sb, wn + 32 + li, g, q);
            }
            acc[0][0] = H::mma(a0, b0, acc[0][0]);
            acc[0][1] = H::mma(a0, b1, acc[0][1]);
            acc[1][0] = H::mma(a1, b0, acc[1][0]);
            acc[1][1] = H::mma(a1, b1, acc[1][1]);
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2 % PF>;
    if (nfull > 0) {
        issue(I0{}, 0);
        ta[0].store(smh);
        tb[0].store(smh + 2 * TA::ELEMS);
        issue(I1{}, 1);
        if constexpr (PF == 3) issue(I2{}, 2);
    }
    __syncthreads();
    // Step kt computes from LDS buffer kt & 1, issues step kt + PF's loads
    // into the slot that held step kt, and stores step kt + 1 (slot
    // (kt + 1) % PF) into the other buffer.
    auto step = [&](int kt, auto slotc) {
        constexpr int S = decltype(slotc)::value;
        constexpr int NS = (S + 1) % PF;
        const int cur = kt & 1;
        issue(slotc, kt + PF);
        compute(smh + cur * TA::ELEMS, smh + 2 * TA::ELEMS + cur * TB::ELEMS);
        // unconditional: no path reaches the next loads with this slot pending
        ta[NS].store(smh + (cur ^ 1) * TA::ELEMS);
        tb[NS].store(smh + 2 * TA::ELEMS + (cur ^ 1) * TB::ELEMS);
        __syncthreads();
    };
    int kt = 0;
    for (; kt + PF <= nfull; kt += PF) {
        step(kt, I0{});
        step(kt + 1, I1{});
        if constexpr (PF == 3) step(kt + 2, I2{});
    }
    if (kt < nfull) step(kt++, I0{});
    if constexpr (PF == 3) {
        if (kt < nfull) step(kt++, I1{});
    }
    if (nfull * SBK < a.K) {  // partial last step, zero-padded
        const int kk = nfull * SBK;
        ta[0].template load<true>(a.A, a.lda, m0, a.M, kk, a.K);
        tb[0].template load<true>(a.B, a.ldb, n0, a.N, kk, a.K);
        ta[0].store(smh);
        tb[0].store(smh + 2 * TA::ELEMS);
        __syncthreads();
        compute(smh, smh + 2 * TA::ELEMS);
        __syncthreads();
    }

    const uint32_t aux_touch = touch_aux_tile<EPI>(a, m0, n0);
    // each wave's 64x64 block through LDS in two 32-row halves; EPI_GELU_BWD
    // column sums as in the 64-step kernel (same rows in the same order)
    const bool csum = EPI == EPI_GELU_BWD && a.colsum != nullptr;
    float4 cs = make_float4(0.f, 0.f, 0.f, 0.f);
    float* ws = reinterpret_cast<float*>(smraw) + wave * 32 * 68;
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
                o = epi4<EPI, H>(a, nullptr, row, col, v);
            } else {
                if (col < a.N) o.x = epi1<EPI, H>(a, nullptr, row, col, v.x);
                if (col + 1 < a.N) o.y = epi1<EPI, H>(a, nullptr, row, col + 1, v.y);
                if (col + 2 < a.N) o.z = epi1<EPI, H>(a, nullptr, row, col + 2, v.z);
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
    asm volatile("" ::"v"(aux_touch));
}

// ---- large tiles for the weight-gradient and long-K products -------------
//
// The products above use 128x128 tiles (2 x 2 MFMA blocks per wave).  The
// weight gradients (K = B*T, few output tiles) and the LM-head input
// gradient (K = V) split K; there a 256x256 tile per workgroup (4 x 4 blocks
// per wave, one workgroup per CU) halves the operand traffic per MFMA from
// LDS and L2 and measured 10-45% faster.  Operands contiguous in k sit in LDS
// as rows of 64 bf16 with the eight 16-byte chunks permuted by
// chunk ^ ((row >> 1) & 7), so their reads and stores avoid bank conflicts
// without padding.  Operands contiguous in the free index (both operands of
// the weight gradients, the weight of the LM-head input gradient) stay
// [k][row] and are read with the transposing LDS loads; against an 8 x 8
// register transpose that took these products from 8.2 to 7.4 ms per step
// with bit-identical results.
// element offset of 16-byte chunk c (0..7) of row r
__device__ __forceinline__ int sw(int r, int c) { return r * BK + 8 * (c ^ ((r >> 1) & 7)); }

template <bool KC, int R>
struct TileS;

// Reduction index contiguous: element (r, k) at g[r*ld + k].  A thread moves
// 16-byte chunks (8 consecutive k of one row).
template <int R>
struct TileS<true, R> {
    static constexpr int ELEMS = R * BK;
    static constexpr int PER = R * 8 / NTHR;
    uint4 v[PER];
    template <bool TAIL>
    __device__ __forceinline__ void load(const uint16_t* __restrict__ g, int64_t ld, int r0,
                                         int Rn, int k0, int K) {
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int idx = threadIdx.x + NTHR * i;
            const int r = min(r0 + (idx >> 3), Rn - 1);
            const int k = k0 + (idx & 7) * 8;
            if (!TAIL) {
                v[i] = *reinterpret_cast<const uint4*>(g + (int64_t)r * ld + k);
            } else {
                const uint4 x =
                    *reinterpret_cast<const uint4*>(g + (int64_t)r * ld + (k < K ? k : 0));
                const uint32_t w[4] = {x.x, x.y, x.z, x.w};
                uint32_t o[4];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const uint32_t lo = k + 2 * j < K ? (w[j] & 0xFFFFu) : 0u;
                    const uint32_t hi = k + 2 * j + 1 < K ? (w[j] & 0xFFFF0000u) : 0u;
                    o[j] = lo | hi;
                }
                v[i] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    }
    __device__ __forceinline__ void store(uint16_t* s) const {
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int idx = threadIdx.x + NTHR * i;
            *reinterpret_cast<uint4*>(s + sw(idx >> 3, idx & 7)) = v[i];
        }
    }
};

__device__ __forceinline__ uint4 frag_s(const uint16_t* s, int r, int g, int q) {
    return *reinterpret_cast<const uint4*>(s + sw(r, 2 * q + g));
}

// Free index contiguous, kept [k][r] in LDS (rows of R + 16 values) and read
// with the transposing LDS loads, as TileT32 above: a thread moves 16-byte runs
// of 8 consecutive r at one k.
template <int R>
struct TileSTr {
    static constexpr int LDR = R + 16;
    static constexpr int ELEMS = BK * LDR;
    static constexpr int RUNS = R / 8;              // runs per k-row
    static constexpr int PER = BK * RUNS / NTHR;
    uint4 v[PER];
    template <bool TAIL>
    __device__ __forceinline__ void load(const uint16_t* __restrict__ g, int64_t ld, int r0,
                                         int Rn, int k0, int K) {
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int idx = threadIdx.x + NTHR * i;
            const int k = k0 + idx / RUNS;
            int r = r0 + (idx % RUNS) * 8;
            r = r < Rn ? r : ((Rn - 1) & ~7);
            if (!TAIL) {
                v[i] = *reinterpret_cast<const uint4*>(g + (int64_t)k * ld + r);
            } else {
                const uint4 x = *reinterpret_cast<const uint4*>(g + (int64_t)(k < K ? k : 0) * ld + r);
                v[i] = k < K ? x : make_uint4(0u, 0u, 0u, 0u);
            }
        }
    }
    __device__ __forceinline__ void store(uint16_t* s) const {
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int idx = threadIdx.x + NTHR * i;
            *reinterpret_cast<uint4*>(s + (idx / RUNS) * LDR + (idx % RUNS) * 8) = v[i];
        }
    }
    // operand of rows rb..rb+31 (lane li = row rb + li), k = 16q + 8g .. +7
    __device__ static __forceinline__ uint4 frag(const uint16_t* s, int rb, int q, int lane) {
        const int grp = lane >> 4, rr = lane & 15;
        const int r = rb + 16 * (grp & 1) + 4 * (rr & 3);
        const int k = 16 * q + 8 * (grp >> 1) + (rr >> 2);
        const uint16_t* p = s + k * LDR + r;
        const tr4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr4_ptr)p);
        const tr4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr4_ptr)(p + 4 * LDR));
        const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
        return make_uint4(a.x, a.y, b.x, b.y);
    }
};

template <int MI, int NI>
struct Shape {
    static constexpr int BM = 64 * MI, BN = 64 * NI;
    static constexpr int WM = 32 * MI, WN = 32 * NI;
    static constexpr int STAGE = (BM + BN) * BK;   // bf16 elements per LDS stage
    static constexpr int EPI_LD = WN + 4;          // fp32 staging row stride
    static constexpr int EPI_F = 4 * 32 * EPI_LD;  // staging floats (4 waves x 32 rows)
    static constexpr int LDS_BYTES = 2 * STAGE * 2 > EPI_F * 4 ? 2 * STAGE * 2 : EPI_F * 4;
    static constexpr int OCC = LDS_BYTES <= 80 * 1024 ? 2 : 1;  // workgroups per CU
};

template <int OP, int EPI, int MI, int NI, class H>
__global__ __launch_bounds__(NTHR, (Shape<MI, NI>::OCC)) void gemm_bf16_big_kernel(
    const GemmArgsH a, int tiles_m, int tiles_n, int kchunk, float* __restrict__ partial) {
    using SH = Shape<MI, NI>;
    constexpr bool AKC = (OP != GEMM_TN);
    constexpr bool BKC = (OP == GEMM_NT);
    // Fragment pipelining: bit-identical, 3-5% faster on the weight
    // gradients, 1-2% slower on the long-K input gradient.
    constexpr bool PIPE = (OP == GEMM_TN);
    using TA = std::conditional_t<AKC, TileS<true, SH::BM>, TileSTr<SH::BM>>;
    using TB = std::conditional_t<BKC, TileS<true, SH::BN>, TileSTr<SH::BN>>;
    constexpr int STAGE = TA::ELEMS + TB::ELEMS;  // bf16 elements per LDS stage
    constexpr int LDS_BYTES = 2 * STAGE * 2 > SH::EPI_F * 4 ? 2 * STAGE * 2 : SH::EPI_F * 4;
    __shared__ __attribute__((aligned(16))) unsigned char smraw[LDS_BYTES];
    uint16_t* smh = reinterpret_cast<uint16_t*>(smraw);

    const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    constexpr int GM = 8;
    const int per_group = GM * tiles_n;
    const int group = tile / per_group;
    const int first_m = group * GM;
    const int gm = min(tiles_m - first_m, GM);
    const int in_g = tile - group * per_group;
    const int m0 = (first_m + in_g % gm) * SH::BM;
    const int n0 = (in_g / gm) * SH::BN;

    const int k_begin = blockIdx.z * kchunk;
    float* const part = EPI == EPI_PARTIAL ? partial + (int64_t)blockIdx.z * a.M * a.N : nullptr;
    const int k_end = min(a.K, k_begin + kchunk);
    const int nfull = (k_end - k_begin) / BK;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = (wave >> 1) * SH::WM, wn = (wave & 1) * SH::WN;
    const int li = lane & 31, g = lane >> 5;

    floatx16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; i++)
#pragma unroll
        for (int j = 0; j < NI; j++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[i][j][e] = 0.f;

    TA ta[2];
    TB tb[2];
    auto issue = [&](auto slotc, int kt) {
        constexpr int S = decltype(slotc)::value;
        const int kk = k_begin + min(kt, nfull - 1) * BK;
        ta[S].template load<false>(a.A, a.lda, m0, a.M, kk, k_end);
        tb[S].template load<false>(a.B, a.ldb, n0, a.N, kk, k_end);
    };
    auto rd = [&](uint4 (&af)[MI], uint4 (&bf)[NI], const uint16_t* sa, const uint16_t* sb,
                  int q) {
#pragma unroll
        for (int i = 0; i < MI; i++) {
            if constexpr (AKC) af[i] = frag_s(sa, wm + 32 * i + li, g, q);
            else af[i] = TA::frag(sa, wm + 32 * i, q, lane);
        }
#pragma unroll
        for (int j = 0; j < NI; j++) {
            if constexpr (BKC) bf[j] = frag_s(sb, wn + 32 * j + li, g, q);
            else bf[j] = TB::frag(sb, wn + 32 * j, q, lane);
        }
    };
    auto mm = [&](const uint4 (&af)[MI], const uint4 (&bf)[NI]) {
#pragma unroll
        for (int i = 0; i < MI; i++)
#pragma unroll
            for (int j = 0; j < NI; j++) acc[i][j] = H::mma(af[i], bf[j], acc[i][j]);
    };
    // One reduction step from LDS.  PIPE: the fragments of sub-step q + 1 are
    // read before the MFMAs of sub-step q, so their LDS latency overlaps the
    // matrix work; the next stage's LDS stores (st) go in the middle of the
    // step.  Otherwise each sub-step reads its fragments and then multiplies,
    // and st runs after the step.
    auto compute = [&](const uint16_t* sa, const uint16_t* sb, auto st) {
        if constexpr (PIPE) {
            uint4 af[2][MI], bf[2][NI];
            rd(af[0], bf[0], sa, sb, 0);
#pragma unroll
            for (int q = 0; q < BK / 16; q++) {
                if (q + 1 < BK / 16) rd(af[(q + 1) & 1], bf[(q + 1) & 1], sa, sb, q + 1);
                mm(af[q & 1], bf[q & 1]);
                if (q == 1) st();
            }
        } else {
#pragma unroll
            for (int q = 0; q < BK / 16; q++) {
                uint4 af[MI], bf[NI];
                rd(af, bf, sa, sb, q);
                mm(af, bf);
            }
            st();
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    auto sA = [&](int b) { return smh + b * STAGE; };
    auto sB = [&](int b) { return smh + b * STAGE + TA::ELEMS; };
    if (nfull > 0) {
        issue(I0{}, 0);
        ta[0].store(sA(0));
        tb[0].store(sB(0));
        issue(I1{}, 1);
    }
    __syncthreads();
    auto step = [&](int kt, auto slotc) {
        constexpr int S = decltype(slotc)::value;
        constexpr int NS = S ^ 1;
        const int cur = kt & 1;
        issue(slotc, kt + 2);
        __builtin_amdgcn_sched_barrier(0);  // loads stay ahead of the MFMAs
        // The stores fill the other buffer, which every wave finished reading
        // before the previous barrier; unconditional, so no path reaches the
        // next loads with this slot pending.
        compute(sA(cur), sB(cur), [&]() {
            ta[NS].store(sA(cur ^ 1));
            tb[NS].store(sB(cur ^ 1));
        });
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
        ta[0].store(sA(0));
        tb[0].store(sB(0));
        __syncthreads();
        compute(sA(0), sB(0), []() {});
        __syncthreads();
    }

    // Epilogue: each wave stages one 32-row strip (32 x WN fp32) at a time in
    // its own LDS region and applies the epilogue along rows (the main
    // loop's buffers are free after the last barrier; a wave reads back only
    // what it wrote).
    float* ws = reinterpret_cast<float*>(smraw) + wave * 32 * SH::EPI_LD;
#pragma unroll
    for (int i = 0; i < MI; i++) {
#pragma unroll
        for (int j = 0; j < NI; j++)
#pragma unroll
            for (int e = 0; e < 16; e++)
                ws[(8 * (e >> 2) + 4 * g + (e & 3)) * SH::EPI_LD + 32 * j + li] = acc[i][j][e];
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the strip is in LDS
        __builtin_amdgcn_wave_barrier();
        constexpr int C4 = SH::WN / 4;
#pragma unroll 4
        for (int idx = lane; idx < 32 * C4; idx += 64) {
            const int r = idx / C4, c4 = (idx % C4) * 4;
            const float4 v = ld4(ws + r * SH::EPI_LD + c4);
            const int row = m0 + wm + 32 * i + r, col = n0 + wn + c4;
            if (row >= a.M) continue;
            if (col + 3 < a.N) {
                epi4<EPI, H>(a, part, row, col, v);
            } else {
                if (col < a.N) epi1<EPI, H>(a, part, row, col, v.x);
                if (col + 1 < a.N) epi1<EPI, H>(a, part, row, col + 1, v.y);
                if (col + 2 < a.N) epi1<EPI, H>(a, part, row, col + 2, v.z);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// ---- 256x256 products with the stages loaded straight into LDS ----------
//
// The weight gradients (TN) and the long-K input gradient (NN, K = V) on the
// same 256x256 tiles, 4x4 blocks per wave and fragment reads as the kernel
// above, but each 32-deep stage goes from memory to LDS with
// global_load_lds_dwordx4 (lane l writes bytes 16l..16l+15 after the wave's
// LDS base), so no registers hold a stage on its way and no LDS store
// instructions are issued: at one wave per SIMD every instruction of the
// wave is on its critical path.  Four stages, loaded three steps ahead; one
// raw barrier per step.  Such a load writes 1 KB of LDS contiguously, so the
// stage rows are not padded; their 16-byte chunks are permuted instead, and
// each lane fetches the chunk that belongs at its place:
//   - free index contiguous ([k][256]: both TN operands, the NN weight),
//     chunk c of row k at c ^ 2 (k & 3), the bank spread of 16 elements of
//     padding for the transposing reads;
//   - reduction index contiguous ([256][32]: the NN A operand), chunk c of
//     row r at c ^ ((r >> 2) & 3), so the 8 rows one 16-byte read serves at
//     a time fall on distinct banks.
// A partial last stage (K not a multiple of 32, the last split only) is
// loaded through registers with zero padding into the same layout.  The
// k order is that of the kernel above, so results are bitwise equal.
// Needs split chunks that are multiples of 32, leading dimensions that are
// multiples of 8 and 16-byte aligned operands.
constexpr int LBK = 32;               // k per stage
constexpr int LSTAGE = LBK * 256;     // bf16 elements per operand per stage

// element offset of (k, r) in a [32][256] stage
__device__ __forceinline__ int lds_off(int k, int r) {
    return k * 256 + (((r >> 3) ^ ((k & 3) << 1)) << 3) + (r & 7);
}
// element offset of (r, k) in a [256][32] stage
__device__ __forceinline__ int lds_off_kc(int r, int k) {
    return r * LBK + (((k >> 3) ^ ((r >> 2) & 3)) << 3) + (k & 7);
}

// operand of rows rb..rb+31 (lane li = row rb + li), k = 16q + 8g .. +7,
// from a [32][256] stage, with two transposing reads
__device__ __forceinline__ uint4 lds_frag(const uint16_t* s, int rb, int q, int lane) {
    const int grp = lane >> 4, rr = lane & 15;
    const int r = rb + 16 * (grp & 1) + 4 * (rr & 3);
    const int k = 16 * q + 8 * (grp >> 1) + (rr >> 2);
    const tr4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr4_ptr)(s + lds_off(k, r)));
    const tr4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr4_ptr)(s + lds_off(k + 4, r)));
    const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
    return make_uint4(a.x, a.y, b.x, b.y);
}
// the same operand from a [256][32] stage: one 16-byte read
__device__ __forceinline__ uint4 lds_frag_kc(const uint16_t* s, int rb, int q, int lane) {
    return *reinterpret_cast<const uint4*>(s + lds_off_kc(rb + (lane & 31), 16 * q + 8 * (lane >> 5)));
}

// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, the others at maximum)
constexpr unsigned kVm0 = 0x0f70, kVm8 = 0x0f78, kVm16 = 0x4f70, kLgkm0 = 0xc07f;

// Tile and K chunk of a split workgroup (grid: tiles x 1 x nz).  The hardware
// hands workgroups to the 8 XCDs round-robin in dispatch order; here XCD x
// takes one contiguous run of the chunk-major order (chunk, tile), so the
// workgroups resident on one XCD are, for all but two chunks of the run, the
// tiles of one chunk, and read that chunk's A and B rows through its L2 at
// the same time.  Bijective for any nz (whole chunks per XCD need nz a
// multiple of 8, which costs the 16-bit products a second round of
// workgroups).
__device__ __forceinline__ void chunk_major_remap(int bx, int bz, int tiles, int nz, int& tile,
                                                  int& kz) {
    if (nz <= 1) {
        kz = 0;
        tile = xcd_remap(bx, tiles);
        return;
    }
    const int lin = bx + tiles * bz;  // dispatch order
    const int total = tiles * nz;
    const int x = lin & 7, base = total >> 3, extra = total & 7;
    const int o = x * base + min(x, extra) + (lin >> 3);  // XCD y holds base + (y < extra)
    kz = o / tiles;
    tile = o - kz * tiles;
}

template <int OP, int EPI, class H>
__global__ __launch_bounds__(NTHR, 1) void gemm_bf16_lds_kernel(const GemmArgsH a, int tiles_m,
                                                               int tiles_n, int kchunk,
                                                               float* __restrict__ partial) {
    static_assert(OP == GEMM_TN || OP == GEMM_NN, "TN or NN");
    constexpr bool AKC = OP == GEMM_NN;  // A contiguous along k
    using SH = Shape<4, 4>;
    constexpr int MI = 4, NI = 4;
    // Eight distinct arrays, so that the compiler can tell the stage being
    // refilled from the stage being read (with one array it waits for every
    // load in flight before each read).
    __shared__ __attribute__((aligned(16))) uint16_t SA0[LSTAGE], SA1[LSTAGE], SA2[LSTAGE],
        SA3[LSTAGE], SB0[LSTAGE], SB1[LSTAGE], SB2[LSTAGE], SB3[LSTAGE];

    int tile, kz;
    chunk_major_remap(blockIdx.x, blockIdx.z, tiles_m * tiles_n, gridDim.z, tile, kz);
    constexpr int GM = 8;
    const int per_group = GM * tiles_n;
    const int group = tile / per_group;
    const int first_m = group * GM;
    const int gm = min(tiles_m - first_m, GM);
    const int in_g = tile - group * per_group;
    const int m0 = (first_m + in_g % gm) * 256;
    const int n0 = (in_g / gm) * 256;

    const int k_begin = kz * kchunk;
    float* const part = EPI == EPI_PARTIAL ? partial + (int64_t)kz * a.M * a.N : nullptr;
    const int k_end = min(a.K, k_begin + kchunk);
    const int nsteps = (k_end - k_begin) / LBK;  // whole stages; the rest is the tail

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = (wave >> 1) * SH::WM, wn = (wave & 1) * SH::WN;
    const int li = lane & 31, g = lane >> 5;

    // Load j = wave + 4i (i = 0..3) of a stage fills 1 KB of it.
    //   [32][256]: rows 2j and 2j + 1; lane l writes physical chunk l % 32 of
    //   row k = 2j + l / 32, the place of logical chunk (l % 32) ^ 2 (k & 3),
    //   with k & 3 = (2 wave + l / 32) & 3 for every i.  Columns past the
    //   matrix read its last whole run of 8.
    //   [256][32] (NN A): rows 16j .. 16j + 15; lane l writes physical chunk
    //   l % 4 of row r = 16j + l / 4, the place of logical chunk
    //   (l % 4) ^ ((r >> 2) & 3) = (l % 4) ^ ((l >> 4) & 3).  Rows past the
    //   matrix read its last row.
    // (Both only reach outputs that are never stored.)
    const int kl = lane >> 5;
    const int fchunk = (lane & 31) ^ (((2 * wave + kl) & 3) << 1);
    int rbn = n0 + 8 * fchunk;
    rbn = rbn < a.N ? rbn : ((a.N - 1) & ~7);
    const uint16_t* gb = a.B + (int64_t)(k_begin + kl) * a.ldb + rbn;
    const uint16_t* ga[4];
    int64_t astep;  // elements per stage along the A pointer
    if constexpr (AKC) {
        const int kc = (lane & 3) ^ ((lane >> 4) & 3);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int r = min(m0 + 16 * (wave + 4 * i) + (lane >> 2), a.M - 1);
            ga[i] = a.A + (int64_t)r * a.lda + k_begin + 8 * kc;
        }
        astep = LBK;
    } else {
        int ra = m0 + 8 * fchunk;
        ra = ra < a.M ? ra : ((a.M - 1) & ~7);
#pragma unroll
        for (int i = 0; i < 4; i++)
            ga[i] = a.A + (int64_t)(k_begin + kl + 2 * (wave + 4 * i)) * a.lda + ra;
        astep = (int64_t)LBK * a.lda;
    }
    auto issue = [&](int t, uint16_t* sa, uint16_t* sb) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int j = wave + 4 * i;
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1)))*)(ga[i] + t * astep),
                (void __attribute__((address_space(3)))*)(sa + j * 512), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1)))*)(gb + ((int64_t)t * LBK + 2 * j) *
                                                                      a.ldb),
                (void __attribute__((address_space(3)))*)(sb + j * 512), 16, 0, 0);
        }
    };

    floatx16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; i++)
#pragma unroll
        for (int j = 0; j < NI; j++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[i][j][e] = 0.f;
    auto fa = [&](const uint16_t* sa, int i, int q) {
        if constexpr (AKC) return lds_frag_kc(sa, wm + 32 * i, q, lane);
        else return lds_frag(sa, wm + 32 * i, q, lane);
    };
    // one stage: the fragments of the second 16-deep sub-step are read before
    // the MFMAs of the first
    auto compute = [&](const uint16_t* sa, const uint16_t* sb) {
        uint4 af[2][MI], bf[2][NI];
#pragma unroll
        for (int i = 0; i < MI; i++) af[0][i] = fa(sa, i, 0);
#pragma unroll
        for (int j = 0; j < NI; j++) bf[0][j] = lds_frag(sb, wn + 32 * j, 0, lane);
#pragma unroll
        for (int q = 0; q < 2; q++) {
            if (q == 0) {
#pragma unroll
                for (int i = 0; i < MI; i++) af[1][i] = fa(sa, i, 1);
#pragma unroll
                for (int j = 0; j < NI; j++) bf[1][j] = lds_frag(sb, wn + 32 * j, 1, lane);
            }
#pragma unroll
            for (int i = 0; i < MI; i++)
#pragma unroll
                for (int j = 0; j < NI; j++) acc[i][j] = H::mma(af[q][i], bf[q][j], acc[i][j]);
        }
    };
    auto barrier = [&]() {  // raw: __syncthreads() would also wait for the loads in flight
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // Before step t: this wave's loads of step t have landed once at most
    // the loads of the (up to two) later steps already issued are in flight
    // (eight per step); after the barrier every wave's have, and every wave
    // has finished step t - 1, so stage (t + 3) % 4 = (t - 1) % 4 is free.
    auto sync = [&](int later) {
        if (later >= 2) __builtin_amdgcn_s_waitcnt(kVm16);
        else if (later == 1) __builtin_amdgcn_s_waitcnt(kVm8);
        else __builtin_amdgcn_s_waitcnt(kVm0);
        __builtin_amdgcn_s_waitcnt(kLgkm0);
        barrier();
    };
    if (nsteps > 0) issue(0, SA0, SB0);
    if (nsteps > 1) issue(1, SA1, SB1);
    if (nsteps > 2) issue(2, SA2, SB2);
    int t = 0;
    for (; t + 7 < nsteps; t += 4) {  // every step refills a stage: no branches
        sync(2);
        issue(t + 3, SA3, SB3);
        compute(SA0, SB0);
        sync(2);
        issue(t + 4, SA0, SB0);
        compute(SA1, SB1);
        sync(2);
        issue(t + 5, SA1, SB1);
        compute(SA2, SB2);
        sync(2);
        issue(t + 6, SA2, SB2);
        compute(SA3, SB3);
    }
    uint16_t* const sas[4] = {SA0, SA1, SA2, SA3};
    uint16_t* const sbs[4] = {SB0, SB1, SB2, SB3};
#pragma unroll
    for (int u = 0; u < 8; u++) {  // the last steps (at most seven; t % 4 == 0)
        if (t + u < nsteps) {
            sync(min(nsteps - 1 - (t + u), 2));
            if (t + u + 3 < nsteps) issue(t + u + 3, sas[(u + 3) & 3], sbs[(u + 3) & 3]);
            compute(sas[u & 3], sbs[u & 3]);
        }
    }
    __builtin_amdgcn_s_waitcnt(kLgkm0);
    barrier();  // every wave is done with the stages
    const int kt = k_begin + nsteps * LBK;
    if (kt < k_end) {  // partial last stage through registers, zero past k_end
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int idx = threadIdx.x + NTHR * i;
            {  // B: [32][256], 8 consecutive columns of one k-row
                const int k = idx >> 5, c = idx & 31;
                int n = n0 + 8 * c;
                n = n < a.N ? n : ((a.N - 1) & ~7);
                uint4 v = make_uint4(0u, 0u, 0u, 0u);
                if (kt + k < k_end)
                    v = *reinterpret_cast<const uint4*>(a.B + (int64_t)(kt + k) * a.ldb + n);
                *reinterpret_cast<uint4*>(SB0 + lds_off(k, 8 * c)) = v;
            }
            if constexpr (AKC) {  // A: [256][32], 8 consecutive k of one row
                const int r = idx >> 2, c = idx & 3, k = kt + 8 * c;
                const int row = min(m0 + r, a.M - 1);
                const uint4 x = *reinterpret_cast<const uint4*>(
                    a.A + (int64_t)row * a.lda + (k < k_end ? k : k_begin));
                const uint32_t w[4] = {x.x, x.y, x.z, x.w};
                uint32_t o[4];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const uint32_t lo = k + 2 * j < k_end ? (w[j] & 0xFFFFu) : 0u;
                    const uint32_t hi = k + 2 * j + 1 < k_end ? (w[j] & 0xFFFF0000u) : 0u;
                    o[j] = lo | hi;
                }
                *reinterpret_cast<uint4*>(SA0 + lds_off_kc(r, 8 * c)) =
                    make_uint4(o[0], o[1], o[2], o[3]);
            } else {  // A: [32][256] like B
                const int k = idx >> 5, c = idx & 31;
                int m = m0 + 8 * c;
                m = m < a.M ? m : ((a.M - 1) & ~7);
                uint4 v = make_uint4(0u, 0u, 0u, 0u);
                if (kt + k < k_end)
                    v = *reinterpret_cast<const uint4*>(a.A + (int64_t)(kt + k) * a.lda + m);
                *reinterpret_cast<uint4*>(SA0 + lds_off(k, 8 * c)) = v;
            }
        }
        __syncthreads();
        compute(SA0, SB0);
        __syncthreads();  // before the epilogue stages into SA0
    }

    // Epilogue as in the kernel above; each wave stages its 32 x 128 fp32
    // strips (16 KB, unpadded) in its own A stage.
    constexpr int ELD = SH::WN;
    float* ws = reinterpret_cast<float*>(wave == 0 ? SA0 : wave == 1 ? SA1 : wave == 2 ? SA2 : SA3);
#pragma unroll
    for (int i = 0; i < MI; i++) {
#pragma unroll
        for (int j = 0; j < NI; j++)
#pragma unroll
            for (int e = 0; e < 16; e++)
                ws[(8 * (e >> 2) + 4 * g + (e & 3)) * ELD + 32 * j + li] = acc[i][j][e];
        __builtin_amdgcn_s_waitcnt(kLgkm0);  // the strip is in LDS
        __builtin_amdgcn_wave_barrier();
        constexpr int C4 = SH::WN / 4;
#pragma unroll 4
        for (int idx = lane; idx < 32 * C4; idx += 64) {
            const int r = idx / C4, c4 = (idx % C4) * 4;
            const float4 v = ld4(ws + r * ELD + c4);
            const int row = m0 + wm + 32 * i + r, col = n0 + wn + c4;
            if (row >= a.M) continue;
            if (col + 3 < a.N) {
                epi4<EPI, H>(a, part, row, col, v);
            } else {
                if (col < a.N) epi1<EPI, H>(a, part, row, col, v.x);
                if (col + 1 < a.N) epi1<EPI, H>(a, part, row, col + 1, v.y);
                if (col + 2 < a.N) epi1<EPI, H>(a, part, row, col + 2, v.z);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// ---- persistent 256x256 forward products, stages straight into LDS -------
//
// The NT products (both operands contiguous along k) with a short reduction:
// one workgroup per compute unit walks its tiles (tile = the i-th virtual
// workgroup blockIdx.x + i * gridDim.x, mapped as the other kernels map
// their workgroups) as one stream of 32-deep steps, so the loads of a tile's
// first stages overlap the previous tile's last steps and its epilogue.
// Stages as in the kernel above ([256][32] rows, chunks permuted by
// (r >> 2) mod 4, loaded three steps ahead); both operands are read with
// 16-byte fragment reads.  The epilogue stages one 32x32 block per wave at a
// time in a separate LDS area.  Needs K a multiple of 128 (every tile starts
// on stage 0) and at least 256, leading dimensions that are multiples of 8
// and 16-byte aligned operands.  The k order is that of the 128x128 kernels, so the
// results are bitwise the same.
template <int EPI, class H>
__global__ __launch_bounds__(NTHR, 1) void gemm_bf16_nt_stream_kernel(const GemmArgsH a,
                                                                     int tiles_m, int tiles_n) {
    using SH = Shape<4, 4>;
    constexpr int MI = 4, NI = 4;
    constexpr int ELD = 36;  // epilogue staging row stride (floats)
    __shared__ __attribute__((aligned(16))) uint16_t SA0[LSTAGE], SA1[LSTAGE], SA2[LSTAGE],
        SA3[LSTAGE], SB0[LSTAGE], SB1[LSTAGE], SB2[LSTAGE], SB3[LSTAGE];
    __shared__ __attribute__((aligned(16))) float EP[4 * 32 * ELD];

    const int ntiles = tiles_m * tiles_n;
    const int G = gridDim.x;
    const int my_tiles = (ntiles - (int)blockIdx.x + G - 1) / G;  // >= 1: the grid has no more WGs than tiles
    const int S = a.K / LBK;                                       // steps per tile, a multiple of 4

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = (wave >> 1) * SH::WM, wn = (wave & 1) * SH::WN;
    const int li = lane & 31, g = lane >> 5;
    const int kc = (lane & 3) ^ ((lane >> 4) & 3);  // the logical chunk this lane fetches

    struct Ptrs {
        const uint16_t* a[4];
        const uint16_t* b[4];
        int m0, n0;
    };
    // load j = wave + 4i of a stage fills rows 16j .. 16j + 15 (1 KB); rows
    // past the matrix read its last row (only outputs never stored see them)
    auto tile_ptrs = [&](int ti, Ptrs& p) {
        const int tile = xcd_remap((int)blockIdx.x + ti * G, ntiles);
        constexpr int GM = 8;
        const int per_group = GM * tiles_n;
        const int group = tile / per_group;
        const int first_m = group * GM;
        const int gm = min(tiles_m - first_m, GM);
        const int in_g = tile - group * per_group;
        p.m0 = (first_m + in_g % gm) * 256;
        p.n0 = (in_g / gm) * 256;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int r = 16 * (wave + 4 * i) + (lane >> 2);
            p.a[i] = a.A + (int64_t)min(p.m0 + r, a.M - 1) * a.lda + 8 * kc;
            p.b[i] = a.B + (int64_t)min(p.n0 + r, a.N - 1) * a.ldb + 8 * kc;
        }
    };
    auto issue = [&](const Ptrs& p, int ks, uint16_t* sa, uint16_t* sb) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int j = wave + 4 * i;
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1)))*)(p.a[i] + ks * LBK),
                (void __attribute__((address_space(3)))*)(sa + j * 512), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1)))*)(p.b[i] + ks * LBK),
                (void __attribute__((address_space(3)))*)(sb + j * 512), 16, 0, 0);
        }
    };

    floatx16 acc[MI][NI];
    auto zero_acc = [&]() {
#pragma unroll
        for (int i = 0; i < MI; i++)
#pragma unroll
            for (int j = 0; j < NI; j++)
#pragma unroll
                for (int e = 0; e < 16; e++) acc[i][j][e] = 0.f;
    };
    auto compute = [&](const uint16_t* sa, const uint16_t* sb) {
        uint4 af[2][MI], bf[2][NI];
#pragma unroll
        for (int i = 0; i < MI; i++) af[0][i] = lds_frag_kc(sa, wm + 32 * i, 0, lane);
#pragma unroll
        for (int j = 0; j < NI; j++) bf[0][j] = lds_frag_kc(sb, wn + 32 * j, 0, lane);
#pragma unroll
        for (int q = 0; q < 2; q++) {
            if (q == 0) {
#pragma unroll
                for (int i = 0; i < MI; i++) af[1][i] = lds_frag_kc(sa, wm + 32 * i, 1, lane);
#pragma unroll
                for (int j = 0; j < NI; j++) bf[1][j] = lds_frag_kc(sb, wn + 32 * j, 1, lane);
            }
#pragma unroll
            for (int i = 0; i < MI; i++)
#pragma unroll
                for (int j = 0; j < NI; j++) acc[i][j] = H::mma(af[q][i], bf[q][j], acc[i][j]);
        }
    };
    auto barrier = [&]() {  // raw: __syncthreads() would also wait for the loads in flight
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // Before step s: this wave's loads of step s have landed once at most the
    // loads of the (up to two) later steps already issued are in flight
    // (eight per step; epilogue stores issued after them only make the wait
    // longer); after the barrier every wave's have, and every wave has
    // finished step s - 1, whose stage the step refills.
    auto sync = [&](int later) {
        if (later >= 2) __builtin_amdgcn_s_waitcnt(kVm16);
        else if (later == 1) __builtin_amdgcn_s_waitcnt(kVm8);
        else __builtin_amdgcn_s_waitcnt(kVm0);
        __builtin_amdgcn_s_waitcnt(kLgkm0);
        barrier();
    };
    // Epilogue of one tile: each wave stages its 32x32 blocks one at a time
    // and stores them along rows (4 columns per lane).
    float* ep = EP + wave * 32 * ELD;
    auto epilogue = [&](int m0, int n0) {
#pragma unroll
        for (int i = 0; i < MI; i++)
#pragma unroll
            for (int j = 0; j < NI; j++) {
#pragma unroll
                for (int e = 0; e < 16; e++)
                    ep[(8 * (e >> 2) + 4 * g + (e & 3)) * ELD + li] = acc[i][j][e];
                __builtin_amdgcn_s_waitcnt(kLgkm0);
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const int idx = lane + 64 * u, r = idx >> 3, c4 = (idx & 7) * 4;
                    const float4 v = ld4(ep + r * ELD + c4);
                    const int row = m0 + wm + 32 * i + r, col = n0 + wn + 32 * j + c4;
                    if (row >= a.M) continue;
                    if (col + 3 < a.N) {
                        epi4<EPI, H>(a, nullptr, row, col, v);
                    } else {
                        if (col < a.N) epi1<EPI, H>(a, nullptr, row, col, v.x);
                        if (col + 1 < a.N) epi1<EPI, H>(a, nullptr, row, col + 1, v.y);
                        if (col + 2 < a.N) epi1<EPI, H>(a, nullptr, row, col + 2, v.z);
                    }
                }
                __builtin_amdgcn_s_waitcnt(kLgkm0);
                __builtin_amdgcn_wave_barrier();
            }
    };

    Ptrs cur, nxt;
    tile_ptrs(0, cur);
    zero_acc();
    issue(cur, 0, SA0, SB0);
    issue(cur, 1, SA1, SB1);
    issue(cur, 2, SA2, SB2);
    // four steps whose refills all fall in this tile: no branches
    auto body = [&](int ks) {
        sync(2);
        issue(cur, ks + 3, SA3, SB3);
        compute(SA0, SB0);
        sync(2);
        issue(cur, ks + 4, SA0, SB0);
        compute(SA1, SB1);
        sync(2);
        issue(cur, ks + 5, SA1, SB1);
        compute(SA2, SB2);
        sync(2);
        issue(cur, ks + 6, SA2, SB2);
        compute(SA3, SB3);
    };
    for (int ti = 0; ti < my_tiles; ti++) {
        const bool more = ti + 1 < my_tiles;
        if (more) tile_ptrs(ti + 1, nxt);
        // The first four steps stay out of the loop: the previous tile's
        // epilogue stores may still be in flight there, and with stores and
        // loads both pending the compiler waits for everything before a
        // stage read; peeled, it does so once per tile and not at the
        // loop's head on every pass.
        body(0);
        for (int ks = 4; ks + 8 <= S; ks += 4) body(ks);
        // the tile's last four steps refill with the next tile's first three
        sync(2);
        issue(cur, S - 1, SA3, SB3);
        compute(SA0, SB0);
        sync(2);
        if (more) issue(nxt, 0, SA0, SB0);
        compute(SA1, SB1);
        sync(more ? 2 : 1);
        if (more) issue(nxt, 1, SA1, SB1);
        compute(SA2, SB2);
        sync(more ? 2 : 0);
        if (more) issue(nxt, 2, SA2, SB2);
        compute(SA3, SB3);
        epilogue(cur.m0, cur.n0);
        zero_acc();
        cur = nxt;
    }
}

constexpr unsigned kVm4 = 0x0f74;  // s_waitcnt vmcnt(4)
constexpr int ST128 = 128 * LBK;   // bf16 elements per operand per 128-row stage
// element offset of (k, r) in a [32][128] stage (chunks permuted as in
// [32][256] stages)
__device__ __forceinline__ int lds_off128(int k, int r) {
    return k * 128 + (((r >> 3) ^ ((k & 3) << 1)) << 3) + (r & 7);
}
// operand of rows rb..rb+31, k = 16q + 8g .. +7, from a [32][128] stage
__device__ __forceinline__ uint4 lds_frag128(const uint16_t* s, int rb, int q, int lane) {
    const int grp = lane >> 4, rr = lane & 15;
    const int r = rb + 16 * (grp & 1) + 4 * (rr & 3);
    const int k = 16 * q + 8 * (grp >> 1) + (rr >> 2);
    const tr4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr4_ptr)(s + lds_off128(k, r)));
    const tr4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr4_ptr)(s + lds_off128(k + 4, r)));
    const uint2 x = __builtin_bit_cast(uint2, lo), y = __builtin_bit_cast(uint2, hi);
    return make_uint4(x.x, x.y, y.x, y.y);
}
// ---- 128x128 products with the stages loaded straight into LDS ----------
//
// The forward (NT) and input-gradient (NN) products on the 128x128 tile,
// 64x64 per wave, with the k order of the 32-deep kernel above (so the
// results, the fused column sums included, are bitwise the same), but each
// 32-deep stage goes from memory to LDS with global_load_lds_dwordx4 as in
// the 256x256 kernels: no staging registers and no LDS store instructions.
// Three stages, loaded two steps ahead, one raw barrier per step; 48 KB of
// LDS, so three workgroups share a compute unit (four stages at two
// workgroups per CU were 2-14% slower).  Stages of operands
// contiguous in k are [128][32] (chunks permuted by (r >> 2) mod 4, read
// with 16-byte fragment reads); the NN weight stays [32][128] (chunks
// permuted by 2 (k mod 4), read with the transposing loads).  The epilogue
// stages 16-row quarters of each wave's block (16 x 68 floats) in the
// wave's own stage buffer.  Needs K a multiple of 32, leading dimensions
// that are multiples of 8 and 16-byte aligned operands.
template <int OP, int EPI, class H>
__global__ __launch_bounds__(NTHR, 3) void gemm_bf16_t128_lds_kernel(const GemmArgsH a,
                                                                    int tiles_m, int tiles_n) {
    static_assert(OP == GEMM_NT || OP == GEMM_NN, "NT or NN");
    // six distinct arrays, so the compiler can tell the stage being refilled
    // from the stage being read
    __shared__ __attribute__((aligned(16))) uint16_t SA0[ST128], SA1[ST128], SA2[ST128],
        SB0[ST128], SB1[ST128], SB2[ST128];
    const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    constexpr int GM = 8;
    const int per_group = GM * tiles_n;
    const int group = tile / per_group;
    const int first_m = group * GM;
    const int gm = min(tiles_m - first_m, GM);
    const int in_g = tile - group * per_group;
    const int m0 = (first_m + in_g % gm) * BM;
    const int n0 = (in_g / gm) * BN;
    const int nsteps = a.K / LBK;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    const int li = lane & 31, g = lane >> 5;
    const int kc = (lane & 3) ^ ((lane >> 4) & 3);
    const uint16_t* ga[2];
    const uint16_t* gb[2];
    int64_t bstep;
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int r = 16 * (wave + 4 * i) + (lane >> 2);
        ga[i] = a.A + (int64_t)min(m0 + r, a.M - 1) * a.lda + 8 * kc;
        if constexpr (OP == GEMM_NT) {
            gb[i] = a.B + (int64_t)min(n0 + r, a.N - 1) * a.ldb + 8 * kc;
        } else {
            // [32][128]: load j fills k-rows 4j .. 4j + 3; lane l writes
            // physical chunk l % 16 of k-row 4j + l / 16, the place of
            // logical chunk (l % 16) ^ 2 ((l / 16) & 3)
            const int kr = 4 * (wave + 4 * i) + (lane >> 4);
            const int fc = (lane & 15) ^ (((lane >> 4) & 3) << 1);
            int n = n0 + 8 * fc;
            n = n < a.N ? n : ((a.N - 1) & ~7);
            gb[i] = a.B + (int64_t)kr * a.ldb + n;
        }
    }
    if constexpr (OP == GEMM_NT) bstep = LBK;
    else bstep = (int64_t)LBK * a.ldb;
    auto issue = [&](int t, uint16_t* sa, uint16_t* sb) {
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int j = wave + 4 * i;
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1)))*)(ga[i] + t * LBK),
                (void __attribute__((address_space(3)))*)(sa + j * 512), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1)))*)(gb[i] + t * bstep),
                (void __attribute__((address_space(3)))*)(sb + j * 512), 16, 0, 0);
        }
    };
    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[i][j][e] = 0.f;
    auto compute = [&](const uint16_t* sa, const uint16_t* sb) {
#pragma unroll
        for (int q = 0; q < 2; q++) {
            const uint4 a0 = lds_frag_kc(sa, wm, q, lane), a1 = lds_frag_kc(sa, wm + 32, q, lane);
            uint4 b0, b1;
            if constexpr (OP == GEMM_NT) {
                b0 = lds_frag_kc(sb, wn, q, lane);
                b1 = lds_frag_kc(sb, wn + 32, q, lane);
            } else {
                b0 = lds_frag128(sb, wn, q, lane);
                b1 = lds_frag128(sb, wn + 32, q, lane);
            }
            acc[0][0] = H::mma(a0, b0, acc[0][0]);
            acc[0][1] = H::mma(a0, b1, acc[0][1]);
            acc[1][0] = H::mma(a1, b0, acc[1][0]);
            acc[1][1] = H::mma(a1, b1, acc[1][1]);
        }
    };
    auto barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // Before step t: this wave's loads of step t have landed once at most the
    // loads of step t + 1, if issued, are in flight (four per step); after the
    // barrier every wave's have, and every wave has finished step t - 1, so
    // its stage, (t + 2) % 3, can be refilled.
    auto sync = [&](int later) {
        if (later >= 1) __builtin_amdgcn_s_waitcnt(kVm4);
        else __builtin_amdgcn_s_waitcnt(kVm0);
        __builtin_amdgcn_s_waitcnt(kLgkm0);
        barrier();
    };
    uint16_t* const sas[3] = {SA0, SA1, SA2};
    uint16_t* const sbs[3] = {SB0, SB1, SB2};
    if (nsteps > 0) issue(0, SA0, SB0);
    if (nsteps > 1) issue(1, SA1, SB1);
    int t = 0;
    for (; t + 5 < nsteps; t += 3) {  // every step refills a stage: no branches
        sync(1);
        issue(t + 2, SA2, SB2);
        compute(SA0, SB0);
        sync(1);
        issue(t + 3, SA0, SB0);
        compute(SA1, SB1);
        sync(1);
        issue(t + 4, SA1, SB1);
        compute(SA2, SB2);
    }
#pragma unroll
    for (int u = 0; u < 6; u++) {  // the last steps (at most five; t % 3 == 0)
        if (t + u < nsteps) {
            sync(min(nsteps - 1 - (t + u), 1));
            if (t + u + 2 < nsteps) issue(t + u + 2, sas[(u + 2) % 3], sbs[(u + 2) % 3]);
            compute(sas[u % 3], sbs[u % 3]);
        }
    }
    const uint32_t aux_touch = touch_aux_tile<EPI>(a, m0, n0);
    __builtin_amdgcn_s_waitcnt(kLgkm0);
    barrier();  // every wave is done with the stages
    // epilogue: each wave stages 16-row quarters of its 64x64 block (16 x 68
    // floats); the column sums of EPI_GELU_BWD add the same rows in the same
    // order as the 32-deep kernel's
    constexpr int ELD = 68;
    float* ws = reinterpret_cast<float*>(wave == 0 ? SA0 : wave == 1 ? SA1 : wave == 2 ? SA2 : SB0);
    const bool csum = EPI == EPI_GELU_BWD && a.colsum != nullptr;
    float4 cs = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int bm = 0; bm < 2; bm++)
#pragma unroll
        for (int hf = 0; hf < 2; hf++) {
#pragma unroll
            for (int bn = 0; bn < 2; bn++)
#pragma unroll
                for (int e = 8 * hf; e < 8 * hf + 8; e++)
                    ws[(8 * ((e >> 2) & 1) + 4 * g + (e & 3)) * ELD + 32 * bn + li] = acc[bm][bn][e];
            __builtin_amdgcn_s_waitcnt(kLgkm0);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int idx = lane + 64 * j;
                const int r = idx >> 4, c4 = (idx & 15) * 4;
                const float4 v = ld4(ws + r * ELD + c4);
                const int row = m0 + wm + 32 * bm + 16 * hf + r, col = n0 + wn + c4;
                if (row >= a.M) continue;
                float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
                if (col + 3 < a.N) {
                    o = epi4<EPI, H>(a, nullptr, row, col, v);
                } else {
                    if (col < a.N) o.x = epi1<EPI, H>(a, nullptr, row, col, v.x);
                    if (col + 1 < a.N) o.y = epi1<EPI, H>(a, nullptr, row, col + 1, v.y);
                    if (col + 2 < a.N) o.z = epi1<EPI, H>(a, nullptr, row, col + 2, v.z);
                }
                if (csum) {
                    cs.x += o.x;
                    cs.y += o.y;
                    cs.z += o.z;
                    cs.w += o.w;
                }
            }
            __builtin_amdgcn_s_waitcnt(kLgkm0);
            __builtin_amdgcn_wave_barrier();
        }
    if (csum) {
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
    asm volatile("" ::"v"(aux_touch));
}

template <int EPI, class H>
__global__ __launch_bounds__(256) void splitk_reduce_bf16_kernel(const GemmArgsH a,
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
    epi4<EPI, H>(a, nullptr, (int)row, col, s);
}

template <int OP, int EPI, class H>
hipError_t launch_h(hipStream_t s, const GemmArgsH& a, float* ws) {
    const int tm = cdiv(a.M, BM), tn = cdiv(a.N, BN);
    // 32-deep steps at three workgroups per CU: the forward products with a
    // short reduction and the input gradients that take the transposing
    // reads.  A very wide output (the LM-head forward, whose weight operand
    // streams 77 MB from memory) keeps three steps of loads in flight:
    // 687 against 622 TFLOP/s there, while at N = 2304 and 3072 the deeper
    // prefetch was 13-24% slower (standalone sweep, bitwise-equal outputs).
    if constexpr (OP == GEMM_NT || OP == GEMM_NN) {
        const bool k32 = (OP == GEMM_NT && a.K < 2048) ||
                         (OP == GEMM_NN && a.ldb % 8 == 0 && ((uintptr_t)a.B & 15) == 0);
        if (k32) {
            // The LM-head forward (no bias) on the persistent 256x256 kernel:
            // 1987 -> 1650 us standalone, bitwise equal.
            if constexpr (OP == GEMM_NT && EPI == EPI_STORE) {
                if (a.N >= kGemm16DeepPrefetchN && !a.bias && a.K % 128 == 0 && a.K >= 256 &&
                    a.lda % 8 == 0 && a.ldb % 8 == 0 &&
                    (((uintptr_t)a.A | (uintptr_t)a.B) & 15) == 0) {
                    const int tm2 = cdiv(a.M, 256), tn2 = cdiv(a.N, 256);
                    launch((gemm_bf16_nt_stream_kernel<EPI, H>),
                           dim3(std::min(tm2 * tn2, device_cu_count())), dim3(NTHR), 0, s, a, tm2,
                           tn2);
                    return hipGetLastError();
                }
            }
            // Stages straight into LDS, bitwise equal to the 32-deep kernel:
            // 4-13% faster standalone on the QKV and fc forwards and on the
            // input gradients with K >= 2304 or N = 3072; 2-5% slower on the
            // 768 x 768 products (one round of workgroups), which keep the
            // register-staged kernel.
            const bool lds_ok = a.K % LBK == 0 && a.lda % 8 == 0 && a.ldb % 8 == 0 &&
                                (((uintptr_t)a.A | (uintptr_t)a.B) & 15) == 0;
            const bool lds_pays = OP == GEMM_NT ? (a.N >= 2048 && a.N < kGemm16DeepPrefetchN)
                                                : (a.N >= 2048 || a.K >= 1536);
            if (lds_ok && lds_pays) {
                launch((gemm_bf16_t128_lds_kernel<OP, EPI, H>), dim3(tm * tn), dim3(NTHR), 0,
                       s, a, tm, tn);
                return hipGetLastError();
            }
            if (a.N >= kGemm16DeepPrefetchN)
                launch((gemm_bf16_k32_kernel<OP, EPI, H, 3>), dim3(tm * tn), dim3(NTHR), 0, s, a,
                       tm, tn);
            else
                launch((gemm_bf16_k32_kernel<OP, EPI, H, 2>), dim3(tm * tn), dim3(NTHR), 0, s, a,
                       tm, tn);
            return hipGetLastError();
        }
    }
    launch((gemm_bf16_kernel<OP, EPI, H>), dim3(tm * tn, 1, 1), dim3(NTHR), 0, s, a, tm, tn,
           a.K > 0 ? a.K : 1, ws);
    return hipGetLastError();
}

template <int OP, int EPI, class H>
hipError_t launch_big(hipStream_t s, const GemmArgsH& a, int splits, float* ws) {
    const int tm = cdiv(a.M, 256), tn = cdiv(a.N, 256);
    const int chunk = splits > 1 ? gemm16_split_chunk(a.K, splits) : (a.K > 0 ? a.K : 1);
    const int nz = splits > 1 ? cdiv(a.K, chunk) : 1;
    // the stages straight into LDS when the split chunks are whole stages
    // and the operands aligned
    if (chunk % LBK == 0 && a.lda % 8 == 0 && a.ldb % 8 == 0 &&
        (((uintptr_t)a.A | (uintptr_t)a.B) & 15) == 0) {
        launch((gemm_bf16_lds_kernel<OP, EPI, H>), dim3(tm * tn, 1, nz), dim3(NTHR), 0, s, a, tm,
               tn, chunk, ws);
        return hipGetLastError();
    }
    launch((gemm_bf16_big_kernel<OP, EPI, 4, 4, H>), dim3(tm * tn, 1, nz), dim3(NTHR), 0,
                       s, a, tm, tn, chunk, ws);
    return hipGetLastError();
}

template <class H>
hipError_t run_big(hipStream_t s, const GemmArgsH& a, int splits, float* ws) {
    if (splits > 1) {
        switch (a.op) {
            case GEMM_NN: return launch_big<GEMM_NN, EPI_PARTIAL, H>(s, a, splits, ws);
            case GEMM_TN: return launch_big<GEMM_TN, EPI_PARTIAL, H>(s, a, splits, ws);
            default: return hipErrorInvalidValue;
        }
    }
    switch (a.op) {
        case GEMM_NN:
            switch (a.epi) {
                case EPI_STORE: return launch_big<GEMM_NN, EPI_STORE, H>(s, a, 1, ws);
                case EPI_GELU_BWD: return launch_big<GEMM_NN, EPI_GELU_BWD, H>(s, a, 1, ws);
                default: return hipErrorInvalidValue;
            }
        case GEMM_TN:
            switch (a.epi) {
                case EPI_STORE: return launch_big<GEMM_TN, EPI_STORE, H>(s, a, 1, ws);
                case EPI_ACCUM: return launch_big<GEMM_TN, EPI_ACCUM, H>(s, a, 1, ws);
                default: return hipErrorInvalidValue;
            }
        default: return hipErrorInvalidValue;
    }
}

template <class H>
hipError_t run_small(hipStream_t s, const GemmArgsH& a, float* ws) {
    switch (a.op) {
        case GEMM_NT:
            switch (a.epi) {
                case EPI_STORE: return launch_h<GEMM_NT, EPI_STORE, H>(s, a, ws);
                case EPI_RESID: return launch_h<GEMM_NT, EPI_RESID, H>(s, a, ws);
                case EPI_GELU: return launch_h<GEMM_NT, EPI_GELU, H>(s, a, ws);
                default: return hipErrorInvalidValue;
            }
        case GEMM_NN:
            switch (a.epi) {
                case EPI_STORE: return launch_h<GEMM_NN, EPI_STORE, H>(s, a, ws);
                case EPI_GELU_BWD: return launch_h<GEMM_NN, EPI_GELU_BWD, H>(s, a, ws);
                default: return hipErrorInvalidValue;
            }
        case GEMM_TN:
            switch (a.epi) {
                case EPI_STORE: return launch_h<GEMM_TN, EPI_STORE, H>(s, a, ws);
                case EPI_ACCUM: return launch_h<GEMM_TN, EPI_ACCUM, H>(s, a, ws);
                default: return hipErrorInvalidValue;
            }
        default: return hipErrorInvalidValue;
    }
}

template <class H>
hipError_t run(hipStream_t s, const GemmArgsH& a, const PlanH& p, float* ws) {
    if (!p.big) return run_small<H>(s, a, ws);
    hipError_t e = run_big<H>(s, a, p.splits, ws);
    if (e != hipSuccess || p.splits <= 1) return e;
    const int nz = cdiv(a.K, gemm16_split_chunk(a.K, p.splits));
    const int64_t n4 = (int64_t)a.M * (a.N / 4);
    if (n4 >= (int64_t)1 << 31) return hipErrorInvalidValue;
    const int blocks = (int)((n4 + 255) / 256);
    if (a.epi == EPI_ACCUM)
        launch((splitk_reduce_bf16_kernel<EPI_ACCUM, H>), dim3(blocks), dim3(256), 0,
                           s, a, ws, nz);
    else
        launch((splitk_reduce_bf16_kernel<EPI_STORE, H>), dim3(blocks), dim3(256), 0,
                           s, a, ws, nz);
    return hipGetLastError();
}

}  // namespace

hipError_t gemm_bf16(hipStream_t s, const GemmArgsH& a, float* ws, size_t ws_bytes) {
    if (a.M <= 0 || a.N <= 0) return hipSuccess;
    // 16-byte runs along k for k-contiguous operands, 8-byte runs of 4 along
    // the free index otherwise; leading dimensions cover each extent.
    const int64_t lda_al = a.op == GEMM_TN ? 4 : 8, ldb_al = a.op == GEMM_NT ? 8 : 4;
    if (a.lda % lda_al || a.ldb % ldb_al || (a.ldc & 3)) return hipErrorInvalidValue;
    if (a.lda < (a.op == GEMM_TN ? a.M : a.K) || a.ldb < (a.op == GEMM_NT ? a.K : a.N) ||
        a.ldc < a.N)
        return hipErrorInvalidValue;
    PlanH p = gemm16_plan(a.op, a.epi, a.M, a.N, a.K, a.lda, a.ldb, device_cu_count());
    if (p.splits > 1 &&
        (size_t)cdiv(a.K, gemm16_split_chunk(a.K, p.splits)) * a.M * a.N * sizeof(float) > ws_bytes)
        p.splits = 1;
    if (a.colsum) {
        if (a.epi != EPI_GELU_BWD) return hipErrorInvalidValue;
        p = {false, 1};  // the column sums are taken in the 128x128 kernel's epilogue
    }
    return a.f16 ? run<HF16>(s, a, p, ws) : run<HBF16>(s, a, p, ws);
}

}  // namespace gk
