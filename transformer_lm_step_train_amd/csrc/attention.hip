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
// Scores are kept in base 2 (log2(e) is folded into the query scale), so the
// exponentials are single v_exp_f32 instructions.
//
// Backward: D_t = dout_t . out_t;  P = exp(s - lse);  dS = P (dP - D) with
// dP = dout V^T;  dQ = dS K / sqrt(hs);  dK = dS^T Q / sqrt(hs);  dV = P^T dout.
// dQ (with D) and (dK, dV) come from two kernels that each own their output
// rows, so no output is accumulated with atomics and results are
// deterministic.  With a dS workspace the order is: D (one row dot per
// position and head), then the key/value kernel, which also stores dS^T,
// then dQ = dS K as a plain product over the stored dS: 5 matmul-sized
// passes instead of 7 (the dQ kernel no longer recomputes S and dP).
// Without one, the dQ kernel recomputes S and dP and also writes D.
//
// Each workgroup is four waves owning 128 consecutive rows; the other operand
// streams through LDS in 64-row tiles (V transposed in the forward, so one
// float4 read feeds four MFMA steps), double-buffered with a register
// prefetch of the next tile (one barrier per tile).  Tiles (and, in the
// key/value kernel, 32-query blocks) that the causal mask empties completely
// are skipped.
#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

constexpr int AQ = 128;  // rows owned per workgroup (four waves of 32)
static_assert(AQ == kAttnBlock, "dS^T blocks are one workgroup's rows");
constexpr int AT = 64;   // rows per staged tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ floatx16 mfma(float a, float b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void zero16(floatx16& x) {
#pragma unroll
    for (int e = 0; e < 16; e++) x[e] = 0.f;
}

// One 64-row tile of one head (HS floats per row), held in registers between
// its global load and its LDS store.
template <int HS>
struct TileRegs {
    static constexpr int C4 = HS / 4;
    static constexpr int PER = AT * C4 / 256;  // float4 per thread
    float4 v[PER];
    // Rows past the sequence read its last row instead: every product they
    // enter is masked (their scores are -inf, their probabilities and dS 0),
    // so any finite values serve, and the loads need no branches.
    template <class E>
    __device__ __forceinline__ void load(const E* __restrict__ base, int64_t ld, int r0, int T) {
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int idx = threadIdx.x + 256 * i;
            const int r = idx / C4, c = (idx - r * C4) * 4;
            v[i] = Act<E>::ld(base + (int64_t)min(r0 + r, T - 1) * ld + c);
        }
    }
    __device__ __forceinline__ void store(float* sm) const {
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int idx = threadIdx.x + 256 * i;
            const int r = idx / C4, c = (idx - r * C4) * 4;
            st4(sm + r * (HS + 4) + c, v[i]);
        }
    }
    // transposed: element (row r, column c) at sm[c * (AT + 4) + r]
    __device__ __forceinline__ void store_t(float* sm) const {
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int idx = threadIdx.x + 256 * i;
            const int r = idx / C4, c = (idx - r * C4) * 4;
            sm[(c + 0) * (AT + 4) + r] = v[i].x;
            sm[(c + 1) * (AT + 4) + r] = v[i].y;
            sm[(c + 2) * (AT + 4) + r] = v[i].z;
            sm[(c + 3) * (AT + 4) + r] = v[i].w;
        }
    }
};

// Write a lane's 32-row accumulator block(s) of one row: the lane holds
// columns d*32 + 8*(e/4) + 4*g + e%4 of its row, i.e. float4 runs.
template <int HS, int NDB, class E>
__device__ __forceinline__ void store_row(E* row, const floatx16 (&acc)[NDB], int g, float mul) {
#pragma unroll
    for (int d = 0; d < NDB; d++)
#pragma unroll
        for (int c = 0; c < 4; c++) {
            const int dim0 = d * 32 + 8 * c + 4 * g;
            if (dim0 < HS)
                Act<E>::st(row + dim0,
                           make_float4(acc[d][4 * c] * mul, acc[d][4 * c + 1] * mul,
                                       acc[d][4 * c + 2] * mul, acc[d][4 * c + 3] * mul));
        }
}

template <int HS, class E>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(E* __restrict__ out,
                                                          float* __restrict__ lse,
                                                          const E* __restrict__ qkv, int T,
                                                          int C, int NH, float qscale, int qb0) {
    constexpr int LD = HS + 4, HALF = HS / 2, NDB = (HS + 31) / 32;
    constexpr int LDT = AT + 4;        // V^T row stride (keys)
    constexpr int VROWS = NDB * 32;    // V^T rows (head dims, padded to 32)
    __shared__ __attribute__((aligned(16))) float ks[2][AT * LD];
    __shared__ __attribute__((aligned(16))) float vs[2][VROWS * LDT];

    // Longest-first over the whole grid: all heads' last query blocks (the
    // most key tiles) are dispatched first, the first blocks fill the tail.
    // Plain round-robin dispatch then gives every XCD the same mix.  Query
    // blocks before qb0 are not computed (their rows are already stored).
    const int nqb = (T + AQ - 1) / AQ;
    const int nbh = gridDim.x / (nqb - qb0);
    const int bh = blockIdx.x % nbh;
    const int qb = nqb - 1 - blockIdx.x / nbh;
    if (VROWS > HS) {  // padding rows of V^T stay zero
        for (int i = threadIdx.x; i < (VROWS - HS) * LDT; i += blockDim.x) {
            vs[0][HS * LDT + i] = 0.f;
            vs[1][HS * LDT + i] = 0.f;
        }
    }
    const int b = bh / NH, h = bh - b * NH;
    // the wave index in a scalar register, so that every per-wave offset
    // is scalar (buffer offsets then need no per-lane loop)
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 31, g = lane >> 5;
    const int64_t ld = 3 * (int64_t)C;
    const E* qbase = qkv + (int64_t)b * T * ld + h * HS;
    const int q0 = qb * AQ;
    const int qw = q0 + wave * 32;
    const int q = qw + li;
    const int qmax = qw < T ? min(qw + 31, T - 1) : -1;  // last query of this wave
    const int nkt = (min(q0 + AQ, T) - 1) / AT + 1;

    float qr[HALF];
#pragma unroll
    for (int s = 0; s < HALF; s += 4) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (q < T) x = Act<E>::ld(qbase + (int64_t)q * ld + g * HALF + s);
        qr[s] = x.x * qscale;
        qr[s + 1] = x.y * qscale;
        qr[s + 2] = x.z * qscale;
        qr[s + 3] = x.w * qscale;
    }
    floatx16 o[NDB];
#pragma unroll
    for (int d = 0; d < NDB; d++) zero16(o[d]);
    float m = -INFINITY, l = 0.f;

    TileRegs<HS> kreg, vreg;
    kreg.load(qbase + C, ld, 0, T);
    vreg.load(qbase + 2 * C, ld, 0, T);
    kreg.store(ks[0]);
    vreg.store_t(vs[0]);
    __syncthreads();
    for (int kt = 0; kt < nkt; kt++) {
        const int cur = kt & 1;
        if (kt + 1 < nkt) {
            kreg.load(qbase + C, ld, (kt + 1) * AT, T);
            vreg.load(qbase + 2 * C, ld, (kt + 1) * AT, T);
        }
        const int k0 = kt * AT;
        if (k0 <= qmax) {
            const float* ksm = ks[cur];
            const float* vsm = vs[cur];
            // S^T for both 32-key blocks as two interleaved MFMA chains
            floatx16 sc[2];
            zero16(sc[0]);
            zero16(sc[1]);
            const float* kr0 = ksm + li * LD + g * HALF;
            const float* kr1 = kr0 + 32 * LD;
#pragma unroll
            for (int s = 0; s < HALF; s += 4) {
                const float4 k0f = ld4(kr0 + s);
                const float4 k1f = ld4(kr1 + s);
                sc[0] = mfma(k0f.x, qr[s], sc[0]);
                sc[1] = mfma(k1f.x, qr[s], sc[1]);
                sc[0] = mfma(k0f.y, qr[s + 1], sc[0]);
                sc[1] = mfma(k1f.y, qr[s + 1], sc[1]);
                sc[0] = mfma(k0f.z, qr[s + 2], sc[0]);
                sc[1] = mfma(k1f.z, qr[s + 2], sc[1]);
                sc[0] = mfma(k0f.w, qr[s + 3], sc[0]);
                sc[1] = mfma(k1f.w, qr[s + 3], sc[1]);
            }
            if ((k0 + AT - 1 > qw) || (k0 + AT > T)) {  // tile touches the mask
#pragma unroll
                for (int kb = 0; kb < 2; kb++)
#pragma unroll
                    for (int e = 0; e < 16; e++) {
                        const int key = k0 + kb * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                        const bool dead = (key > q) | (key >= T);
                        sc[kb][e] = dead ? -INFINITY : sc[kb][e];
                    }
            }
            float mt = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int e = 0; e < 16; e++) mt = fmaxf(mt, sc[kb][e]);
            mt = fmaxf(mt, __shfl_xor(mt, 32, WAVE));
            const float mn = fmaxf(m, mt);
            const float corr = exp2_fast(m - mn);
            float ls = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    const float p = exp2_fast(sc[kb][e] - mn);
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
            // O^T += V^T P^T: steps e = 4c..4c+3 use keys 8c+4g+(0..3) of a
            // block, one float4 of a V^T row
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int c = 0; c < 4; c++)
#pragma unroll
                    for (int d = 0; d < NDB; d++) {
                        const float4 va =
                            ld4(vsm + (d * 32 + li) * LDT + kb * 32 + 8 * c + 4 * g);
                        o[d] = mfma(va.x, sc[kb][4 * c], o[d]);
                        o[d] = mfma(va.y, sc[kb][4 * c + 1], o[d]);
                        o[d] = mfma(va.z, sc[kb][4 * c + 2], o[d]);
                        o[d] = mfma(va.w, sc[kb][4 * c + 3], o[d]);
                    }
        }
        if (kt + 1 < nkt) {
            kreg.store(ks[cur ^ 1]);
            vreg.store_t(vs[cur ^ 1]);
        }
        __syncthreads();
    }
    if (q < T) {
        store_row<HS, NDB>(out + ((int64_t)b * T + q) * C + h * HS, o, g, 1.f / l);
        if (g == 0) lse[((int64_t)b * NH + h) * T + q] = (m + log2f(l)) * LN2;
    }
}

// dQ, and D = rowsum(dout * out) for the key/value kernel.
template <int HS, class E>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(
    E* __restrict__ dqkv, float* __restrict__ Dout, const E* __restrict__ dout,
    const E* __restrict__ out, const E* __restrict__ qkv, const float* __restrict__ lse,
    int T, int C, int NH, float qscale, float scale) {
    constexpr int LD = HS + 4, HALF = HS / 2, NDB = (HS + 31) / 32;
    __shared__ __attribute__((aligned(16))) float ks[2][AT * LD];
    __shared__ __attribute__((aligned(16))) float vs[2][AT * LD];

    const int nqb = (T + AQ - 1) / AQ;
    const int nbh = gridDim.x / nqb;
    const int bh = blockIdx.x % nbh;
    const int qb = nqb - 1 - blockIdx.x / nbh;  // longest first
    const int b = bh / NH, h = bh - b * NH;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 31, g = lane >> 5;
    const int64_t ld = 3 * (int64_t)C;
    const E* qbase = qkv + (int64_t)b * T * ld + h * HS;
    const E* dobase = dout + (int64_t)b * T * C + h * HS;
    const E* obase = out + (int64_t)b * T * C + h * HS;
    const int q0 = qb * AQ;
    const int qw = q0 + wave * 32;
    const int q = qw + li;
    const int qmax = qw < T ? min(qw + 31, T - 1) : -1;
    const int nkt = (min(q0 + AQ, T) - 1) / AT + 1;

    float qr[HALF], dr[HALF];
    float dsum = 0.f;
#pragma unroll
    for (int s = 0; s < HALF; s += 4) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f), y = x, z = x;
        if (q < T) {
            x = Act<E>::ld(qbase + (int64_t)q * ld + g * HALF + s);
            y = Act<E>::ld(dobase + (int64_t)q * C + g * HALF + s);
            z = Act<E>::ld(obase + (int64_t)q * C + g * HALF + s);
        }
        qr[s] = x.x * qscale;
        qr[s + 1] = x.y * qscale;
        qr[s + 2] = x.z * qscale;
        qr[s + 3] = x.w * qscale;
        dr[s] = y.x;
        dr[s + 1] = y.y;
        dr[s + 2] = y.z;
        dr[s + 3] = y.w;
        dsum += (y.x * z.x + y.y * z.y) + (y.z * z.z + y.w * z.w);
    }
    const float Dq = dsum + __shfl_xor(dsum, 32, WAVE);
    const int64_t srow = ((int64_t)b * NH + h) * T;
    if (q < T && g == 0) Dout[srow + q] = Dq;
    const float lq = q < T ? lse[srow + q] * LOG2E : 0.f;
    floatx16 dq[NDB];
#pragma unroll
    for (int d = 0; d < NDB; d++) zero16(dq[d]);

    TileRegs<HS> kreg, vreg;
    kreg.load(qbase + C, ld, 0, T);
    vreg.load(qbase + 2 * C, ld, 0, T);
    kreg.store(ks[0]);
    vreg.store(vs[0]);
    __syncthreads();
    for (int kt = 0; kt < nkt; kt++) {
        const int cur = kt & 1;
        if (kt + 1 < nkt) {
            kreg.load(qbase + C, ld, (kt + 1) * AT, T);
            vreg.load(qbase + 2 * C, ld, (kt + 1) * AT, T);
        }
        const int k0 = kt * AT;
        if (k0 <= qmax) {
            const float* ksm = ks[cur];
            const float* vsm = vs[cur];
            floatx16 sc[2], dp[2];
#pragma unroll
            for (int kb = 0; kb < 2; kb++) {
                zero16(sc[kb]);
                zero16(dp[kb]);
            }
            const float* kr0 = ksm + li * LD + g * HALF;
            const float* vr0 = vsm + li * LD + g * HALF;
#pragma unroll
            for (int s = 0; s < HALF; s += 4) {
#pragma unroll
                for (int kb = 0; kb < 2; kb++) {
                    const float4 kf = ld4(kr0 + kb * 32 * LD + s);
                    const float4 vf = ld4(vr0 + kb * 32 * LD + s);
                    sc[kb] = mfma(kf.x, qr[s], sc[kb]);
                    dp[kb] = mfma(vf.x, dr[s], dp[kb]);
                    sc[kb] = mfma(kf.y, qr[s + 1], sc[kb]);
                    dp[kb] = mfma(vf.y, dr[s + 1], dp[kb]);
                    sc[kb] = mfma(kf.z, qr[s + 2], sc[kb]);
                    dp[kb] = mfma(vf.z, dr[s + 2], dp[kb]);
                    sc[kb] = mfma(kf.w, qr[s + 3], sc[kb]);
                    dp[kb] = mfma(vf.w, dr[s + 3], dp[kb]);
                }
            }
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    const int key = k0 + kb * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                    const bool live = (key <= q) & (key < T);
                    const float p = exp2_fast(sc[kb][e] - lq);
                    sc[kb][e] = live ? p * (dp[kb][e] - Dq) : 0.f;
                }
#pragma unroll
            for (int kb = 0; kb < 2; kb++) {
                float ka[16][NDB];  // all reads of the block issued before its MFMAs
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    const int kl = kb * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
#pragma unroll
                    for (int d = 0; d < NDB; d++) {
                        const int dim = d * 32 + li;
                        ka[e][d] = dim < HS ? ksm[kl * LD + dim] : 0.f;
                    }
                }
#pragma unroll
                for (int e = 0; e < 16; e++)
#pragma unroll
                    for (int d = 0; d < NDB; d++) dq[d] = mfma(ka[e][d], sc[kb][e], dq[d]);
            }
        }
        if (kt + 1 < nkt) {
            kreg.store(ks[cur ^ 1]);
            vreg.store(vs[cur ^ 1]);
        }
        __syncthreads();
    }
    if (q < T) store_row<HS, NDB>(dqkv + ((int64_t)b * T + q) * ld + h * HS, dq, g, scale);
}

// The dS workspace (the key/value kernel writes it, the dQ kernel reads it),
// per (sequence, head):
//  - dS^T in the 128 x 128 blocks on or below the diagonal, block (key block
//    kb, query block qb) at qb(qb+1)/2 + kb, each [key][query] row-major.
//    The 32 x 32 tiles that the mask empties are never written and never
//    read.  The writer stores float4 runs of queries; a reading lane (one
//    query) loads one value per key, 128 contiguous bytes per half-wave.
//  - then K in the dQ product's operand order, per 32-key block and 32 head
//    dimensions (1024 floats): K[key 2 st + g][dim i] at (32 g + i) * 16 + st,
//    so a lane loads its 16 values as four float4.
__device__ __forceinline__ int64_t ds_block(int qb, int kb) {
    return ((int64_t)(qb * (qb + 1) / 2 + kb)) * (AQ * AQ);
}

template <int HS, class E, bool STORE_DS>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkdv_kernel(
    E* __restrict__ dqkv, const E* __restrict__ dout, const E* __restrict__ qkv,
    const float* __restrict__ lse, const float* __restrict__ D, int T, int C, int NH,
    float qscale, float scale, float* __restrict__ dsT, int64_t ds_stride, int64_t kf_off) {
    constexpr int LD = HS + 4, HALF = HS / 2, NDB = (HS + 31) / 32;
    __shared__ __attribute__((aligned(16))) float qs[2][AT * LD];
    __shared__ __attribute__((aligned(16))) float dos[2][AT * LD];
    __shared__ __attribute__((aligned(16))) float lsm[2][AT], dsm[2][AT];

    const int nkb = (T + AQ - 1) / AQ;
    const int nbh = gridDim.x / nkb;
    const int bh = blockIdx.x % nbh;
    const int kb0 = blockIdx.x / nbh;  // lowest keys = most query tiles: first
    const int b = bh / NH, h = bh - b * NH;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 31, g = lane >> 5;
    const int64_t ld = 3 * (int64_t)C;
    const E* qbase = qkv + (int64_t)b * T * ld + h * HS;
    const E* dobase = dout + (int64_t)b * T * C + h * HS;
    const int64_t srow = ((int64_t)b * NH + h) * T;
    const int kw = kb0 * AQ + wave * 32;  // first key of this wave
    const int key = kw + li;

    float kr[HALF], vr[HALF];
    // this (sequence, head)'s slice of the dS workspace, addressed by one
    // lane offset plus wave-uniform ones (its size is under 2 GiB)
    const __amdgpu_buffer_rsrc_t wsr =
        buf_rsrc(dsT + (STORE_DS ? (int64_t)bh * ds_stride : 0),
                 STORE_DS ? (uint32_t)(ds_stride * 4) : 0u);
    const int lane_off = ((li & 1) * 512 + (li >> 1)) * 4;  // bytes: key 2 st + (li & 1), st = li / 2
    // this wave's keys in the dQ product's operand order (keys past T zero)
    const bool kfrag = STORE_DS && kw < T;
    const int kf_so = (int)((kf_off + (int64_t)(kw / 32) * NDB * 1024) * 4);
#pragma unroll
    for (int s = 0; s < HALF; s += 4) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f), y = x;
        if (key < T) {
            x = Act<E>::ld(qbase + C + (int64_t)key * ld + g * HALF + s);
            y = Act<E>::ld(qbase + 2 * C + (int64_t)key * ld + g * HALF + s);
        }
        if (kfrag) {
            const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const int dim = g * HALF + s + c;
                __builtin_amdgcn_raw_buffer_store_b32(
                    __float_as_uint(xs[c]), wsr, lane_off + ((dim >> 5) * 1024 + (dim & 31) * 16) * 4,
                    kf_so, 0);
            }
        }
        kr[s] = x.x * qscale;  // the score scale folded into the key once
        kr[s + 1] = x.y * qscale;
        kr[s + 2] = x.z * qscale;
        kr[s + 3] = x.w * qscale;
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
    const int qt0 = (kb0 * AQ) / AT;
    const int nqt = (T + AT - 1) / AT;
    TileRegs<HS> qreg, dreg;
    float sreg = 0.f;  // one lse (wave 0) or D (the other waves) value per thread
    // wave 0 loads the tile's lse, the other waves its D (waves 2 and 3
    // redundantly); positions past the sequence read its last one (their
    // probabilities are masked to 0).  The base-2 scaling waits for the LDS
    // store, so the load stays in flight with the tile's.
    auto load_stats = [&](int qt) {
        const int t = min(qt * AT + lane, T - 1);
        sreg = (wave == 0 ? lse : D)[srow + t];
    };
    auto store_stats = [&](int buf) {
        if (wave == 0) lsm[buf][lane] = sreg * LOG2E;
        else if (wave == 1) dsm[buf][lane] = sreg;
    };
    qreg.load(qbase, ld, qt0 * AT, T);
    dreg.load(dobase, C, qt0 * AT, T);
    load_stats(qt0);
    qreg.store(qs[0]);
    dreg.store(dos[0]);
    store_stats(0);
    __syncthreads();
    for (int qt = qt0; qt < nqt; qt++) {
        const int cur = (qt - qt0) & 1;
        if (qt + 1 < nqt) {
            load_stats(qt + 1);  // first, so that its wait is not behind the dS stores
            qreg.load(qbase, ld, (qt + 1) * AT, T);
            dreg.load(dobase, C, (qt + 1) * AT, T);
        }
        const float* qsm = qs[cur];
        const float* dsmem = dos[cur];
#pragma unroll
        for (int qh = 0; qh < 2; qh++) {
            const int qlo = qt * AT + qh * 32;
            const bool run = kw < T && qlo + 31 >= kw && qlo < T;  // else empty under the mask
            floatx16 sc, dp;
            zero16(sc);
            zero16(dp);
            if (run) {
                const float* qrow = qsm + (qh * 32 + li) * LD + g * HALF;
                const float* drow = dsmem + (qh * 32 + li) * LD + g * HALF;
#pragma unroll
                for (int s = 0; s < HALF; s += 4) {
                    const float4 qf = ld4(qrow + s);
                    const float4 df = ld4(drow + s);
                    sc = mfma(qf.x, kr[s], sc);
                    sc = mfma(qf.y, kr[s + 1], sc);
                    sc = mfma(qf.z, kr[s + 2], sc);
                    sc = mfma(qf.w, kr[s + 3], sc);
                    dp = mfma(df.x, vr[s], dp);
                    dp = mfma(df.y, vr[s + 1], dp);
                    dp = mfma(df.z, vr[s + 2], dp);
                    dp = mfma(df.w, vr[s + 3], dp);
                }
                // steps e = 4c..4c+3 hold queries qh*32 + 8c + 4g + (0..3): one
                // float4 of each statistic
#pragma unroll
                for (int c = 0; c < 4; c++) {
                    const int ql = qh * 32 + 8 * c + 4 * g;
                    const float4 l4 = ld4(&lsm[cur][ql]), d4 = ld4(&dsm[cur][ql]);
                    const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const int e = 4 * c + j;
                        const float p = exp2_fast(sc[e] - lv[j]);
                        sc[e] = p;
                        dp[e] = p * (dp[e] - dv4[j]);
                    }
                }
                // the mask as selects (masked infinities do not survive), only
                // on blocks that touch it: the diagonal and the sequence end
                // (the same test for the whole wave)
                if (qlo < kw + 31 || qlo + 31 >= T) {
#pragma unroll
                    for (int e = 0; e < 16; e++) {
                        const int qa = qt * AT + qh * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                        const bool live = (qa < T) & (key <= qa);
                        sc[e] = live ? sc[e] : 0.f;
                        dp[e] = live ? dp[e] : 0.f;
                    }
                }
            }
            if (qh == 0 && qt + 1 < nqt) {
                // The next tile goes into the other buffer (free since the last
                // barrier) before any dS store of this tile: waiting for its
                // loads then never waits for those stores as well.
                qreg.store(qs[cur ^ 1]);
                dreg.store(dos[cur ^ 1]);
                store_stats(cur ^ 1);
            }
            if (!run) continue;
            if constexpr (STORE_DS) {  // this wave's 32 keys x 32 queries of dS^T
                const int so = (int)((ds_block(qt >> 1, kb0) + (wave * 32) * AQ) * 4);
                const int vo = (li * AQ + (qt & 1) * AT + qh * 32 + 4 * g) * 4;
#pragma unroll
                for (int c = 0; c < 4; c++)
                    BufAct<float>::st(wsr, vo + 32 * c, so,
                                      make_float4(dp[4 * c], dp[4 * c + 1], dp[4 * c + 2],
                                                  dp[4 * c + 3]));
            }
#pragma unroll
            for (int half = 0; half < 2; half++) {
                float da[8][NDB], qa[8][NDB];  // reads issued before the MFMAs
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    const int e = half * 8 + i;
                    const int ql = qh * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
#pragma unroll
                    for (int d = 0; d < NDB; d++) {
                        const int dim = d * 32 + li;
                        da[i][d] = dim < HS ? dsmem[ql * LD + dim] : 0.f;
                        qa[i][d] = dim < HS ? qsm[ql * LD + dim] : 0.f;
                    }
                }
#pragma unroll
                for (int i = 0; i < 8; i++)
#pragma unroll
                    for (int d = 0; d < NDB; d++) {
                        dv[d] = mfma(da[i][d], sc[half * 8 + i], dv[d]);
                        dk[d] = mfma(qa[i][d], dp[half * 8 + i], dk[d]);
                    }
            }
        }
        __syncthreads();
    }
    if (key < T) {
        E* row = dqkv + ((int64_t)b * T + key) * ld + h * HS;
        store_row<HS, NDB>(row + C, dk, g, scale);
        store_row<HS, NDB>(row + 2 * C, dv, g, 1.f);
    }
}

// D_t = dout_t . out_t per position and head (one wave per position; the
// HS/4 lanes of a head reduce their float4 partial dots).
template <int HS, class E>
__global__ __launch_bounds__(256) void attn_rowdot_kernel(float* __restrict__ D,
                                                          const E* __restrict__ dout,
                                                          const E* __restrict__ out, int M,
                                                          int T, int C, int NH) {
    constexpr int G = HS / 4;  // lanes per head
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= M) return;  // whole wave
    const int b = r / T, t = r - b * T;
    const E* dr = dout + (int64_t)r * C;
    const E* orow = out + (int64_t)r * C;
    for (int j0 = 0; j0 < C / 4; j0 += 64) {
        const int j = j0 + lane;
        float v = 0.f;
        if (j < C / 4) {
            const float4 x = Act<E>::ld(dr + 4 * j), y = Act<E>::ld(orow + 4 * j);
            v = (x.x * y.x + x.y * y.y) + (x.z * y.z + x.w * y.w);
        }
#pragma unroll
        for (int o = 1; o < G; o <<= 1) v += __shfl_xor(v, o, WAVE);
        if (j < C / 4 && (lane & (G - 1)) == 0) D[((int64_t)b * NH + j / G) * T + t] = v;
    }
}

// dQ = dS K / sqrt(hs) from the dS workspace.  Each wave owns 32 queries and
// runs over 32-key blocks up to its diagonal, loading a block's operands
// straight from the workspace in MFMA order (16 coalesced dS values and four
// float4 of K per 32 head dimensions per lane), PF blocks ahead.  No LDS, no
// barriers.
template <int HS, class E, int PF>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_ds_kernel(
    E* __restrict__ dqkv, const float* __restrict__ dsT, int64_t ds_stride, int64_t kf_off, int T,
    int C, int NH, float scale) {
    constexpr int NDB = (HS + 31) / 32;
    const int nqb = (T + AQ - 1) / AQ;
    const int nbh = gridDim.x / nqb;
    const int bh = blockIdx.x % nbh;
    const int qb = nqb - 1 - blockIdx.x / nbh;  // longest first
    const int b = bh / NH, h = bh - b * NH;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 31, g = lane >> 5;
    const int qw = qb * AQ + wave * 32;
    if (qw >= T) return;  // whole wave
    const int64_t ld = 3 * (int64_t)C;
    // this (sequence, head)'s slice of the workspace (under 2 GiB)
    const __amdgpu_buffer_rsrc_t wsr =
        buf_rsrc(dsT + (int64_t)bh * ds_stride, (uint32_t)(ds_stride * 4));
    const int kvo = (g * 32 + li) * 16 * 4;  // this lane's 16 key values of a block, bytes
    const int dvo = (g * AQ + (qw - qb * AQ) + li) * 4;  // its query's column, key 2 st + g
    const int ds_so = (int)(ds_block(qb, 0) * 4);
    const int kf_so = (int)(kf_off * 4);
    const int nblk = qw / 32 + 1;  // 32-key blocks up to the diagonal

    float av[PF][16], kv[PF][NDB][16];
    auto load = [&](int u, int kblk) {
        const int a = ds_so + ((kblk >> 2) * (AQ * AQ) + (kblk & 3) * 32 * AQ) * 4;
#pragma unroll
        for (int st = 0; st < 16; st++)
            av[u][st] = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(wsr, dvo, a + st * 2 * AQ * 4, BUF_NT));
#pragma unroll
        for (int d = 0; d < NDB; d++)
#pragma unroll
            for (int c = 0; c < 4; c++) {
                // keys are read by every wave of the sequence: default cache policy
                const u32x4_t k = __builtin_amdgcn_raw_buffer_load_b128(
                    wsr, kvo + 16 * c, kf_so + (kblk * NDB + d) * 4096, 0);
                float4 x = make_float4(__uint_as_float(k[0]), __uint_as_float(k[1]),
                                       __uint_as_float(k[2]), __uint_as_float(k[3]));
                if (HS < 32 && li >= HS) x = make_float4(0.f, 0.f, 0.f, 0.f);
                kv[u][d][4 * c] = x.x;
                kv[u][d][4 * c + 1] = x.y;
                kv[u][d][4 * c + 2] = x.z;
                kv[u][d][4 * c + 3] = x.w;
            }
    };
    floatx16 dq[NDB];
#pragma unroll
    for (int d = 0; d < NDB; d++) zero16(dq[d]);
#pragma unroll
    for (int u = 0; u < PF; u++)
        if (u < nblk) load(u, u);
    for (int kblk = 0; kblk < nblk; kblk += PF) {
#pragma unroll
        for (int u = 0; u < PF; u++) {
            if (kblk + u < nblk) {
#pragma unroll
                for (int st = 0; st < 16; st++)
#pragma unroll
                    for (int d = 0; d < NDB; d++) dq[d] = mfma(kv[u][d][st], av[u][st], dq[d]);
                if (kblk + u + PF < nblk) load(u, kblk + u + PF);
            }
        }
    }
    const int q = qw + li;
    if (q < T) store_row<HS, NDB>(dqkv + ((int64_t)b * T + q) * ld + h * HS, dq, g, scale);
}

template <int HS, class E>
hipError_t fwd_hs(hipStream_t s, E* out, float* lse, const E* qkv, int B, int T, int C,
                  int NH, int q_first) {
    const int nqb = (T + AQ - 1) / AQ;
    const int qb0 = q_first / AQ;
    const float qscale = LOG2E / sqrtf((float)HS);
    launch((attn_fwd_kernel<HS, E>), dim3(B * NH * (nqb - qb0)), dim3(256), 0, s, out, lse,
           qkv, T, C, NH, qscale, qb0);
    return hipGetLastError();
}

template <int HS, class E>
hipError_t bwd_hs(hipStream_t s, E* dqkv, float* D, const E* dout, const E* qkv, const E* out,
                  const float* lse, int B, int T, int C, int NH, float* dsT, int64_t ds_stride) {
    const int nb = (T + AQ - 1) / AQ;
    const float scale = 1.0f / sqrtf((float)HS);
    const float qscale = LOG2E * scale;
    if (dsT) {
        const int M = B * T;
        launch((attn_rowdot_kernel<HS, E>), dim3((M + 3) / 4), dim3(256), 0, s, D, dout, out, M,
               T, C, NH);
        launch((attn_bwd_dkdv_kernel<HS, E, true>), dim3(B * NH * nb), dim3(256), 0, s, dqkv,
               dout, qkv, lse, (const float*)D, T, C, NH, qscale, scale, dsT, ds_stride,
               attn_ds_blocks_floats(T));
        launch((attn_bwd_dq_ds_kernel<HS, E, 3>), dim3(B * NH * nb), dim3(256), 0, s, dqkv,
               (const float*)dsT, ds_stride, attn_ds_blocks_floats(T), T, C, NH, scale);
        return hipGetLastError();
    }
    launch((attn_bwd_dq_kernel<HS, E>), dim3(B * NH * nb), dim3(256), 0, s, dqkv, D,
                       dout, out, qkv, lse, T, C, NH, qscale, scale);
    launch((attn_bwd_dkdv_kernel<HS, E, false>), dim3(B * NH * nb), dim3(256), 0, s, dqkv,
                       dout, qkv, lse, D, T, C, NH, qscale, scale, nullptr, (int64_t)0,
                       (int64_t)0);
    return hipGetLastError();
}

template <class E>
hipError_t forward_t(hipStream_t s, E* out, float* lse, const E* qkv, int B, int T, int C,
                     int NH, int q_first) {
    switch (C / NH) {
        case 16: return fwd_hs<16, E>(s, out, lse, qkv, B, T, C, NH, q_first);
        case 32: return fwd_hs<32, E>(s, out, lse, qkv, B, T, C, NH, q_first);
        case 64: return fwd_hs<64, E>(s, out, lse, qkv, B, T, C, NH, q_first);
        default: return hipErrorInvalidValue;
    }
}

template <class E>
hipError_t backward_t(hipStream_t s, E* dqkv, float* D, const E* dout, const E* qkv,
                      const E* out, const float* lse, int B, int T, int C, int NH, float* dsT,
                      int64_t ds_stride) {
    switch (C / NH) {
        case 16: return bwd_hs<16, E>(s, dqkv, D, dout, qkv, out, lse, B, T, C, NH, dsT, ds_stride);
        case 32: return bwd_hs<32, E>(s, dqkv, D, dout, qkv, out, lse, B, T, C, NH, dsT, ds_stride);
        case 64: return bwd_hs<64, E>(s, dqkv, D, dout, qkv, out, lse, B, T, C, NH, dsT, ds_stride);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t attention_forward(hipStream_t s, void* out, float* lse, const void* qkv, int B, int T,
                             int C, int NH, int dt, int q_first) {
    if (B <= 0 || T <= 0) return hipSuccess;
    if (q_first < 0 || q_first >= T) return hipErrorInvalidValue;
    if (dt != DT_F32)
        return attention_forward_half(s, (uint16_t*)out, lse, (const uint16_t*)qkv, B, T, C, NH,
                                      dt, q_first);
    return forward_t<float>(s, (float*)out, lse, (const float*)qkv, B, T, C, NH, q_first);
}

hipError_t attention_backward(hipStream_t s, void* dqkv, float* dpre, const void* dout,
                              const void* qkv, const void* out, const float* lse, int B, int T,
                              int C, int NH, int dt, float* ds_ws, int64_t ds_stride) {
    if (B <= 0 || T <= 0) return hipSuccess;
    if (dt != DT_F32)
        return attention_backward_half(s, (uint16_t*)dqkv, dpre, (const uint16_t*)dout,
                                       (const uint16_t*)qkv, (const uint16_t*)out, lse, B, T, C,
                                       NH, dt);
    if (ds_ws && (NH <= 0 || ds_stride < attn_ds_stride(T, C / NH))) return hipErrorInvalidValue;
    return backward_t<float>(s, (float*)dqkv, dpre, (const float*)dout, (const float*)qkv,
                             (const float*)out, lse, B, T, C, NH, ds_ws, ds_stride);
}

}  // namespace gk
