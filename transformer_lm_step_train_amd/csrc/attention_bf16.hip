// Causal multi-head self-attention of the mixed-precision model on the bf16
// matrix cores (v_mfma_f32_32x32x16_bf16): bf16 q, k, v, out and gradients,
// fp32 accumulation and fp32 softmax statistics.
//
// The layer is GPT-2's masked self-attention (ujoy.net article "徒手用 1000 行
// C 语言实现", section "用C语言实现LLM"; the reduced-precision extension is
// named by yinghuohong.cn, section "脚动完成每一个层前向/反向流传").  The
// algorithm is the one of the fp32 kernels: per sequence and head, an online
// softmax over key tiles that keeps only the row log-sum-exp, and a backward
// that recomputes the probabilities from it:
//   s = q.k / sqrt(hs) (keys <= query),  out = softmax(s) v,
//   D = rowsum(dout * out),  dS = P (dout v^T - D),
//   dq = dS k / sqrt(hs),  dk = dS^T q / sqrt(hs),  dv = P^T dout.
//
// MFMA layout.  A 32x32x16 product takes, per lane l (column/row l % 32,
// half g = l / 32), eight consecutive reduction elements 8g..8g+7 of its
// row of A and of its column of B.  Scores are formed transposed, S^T = K
// Q^T (lane owns a query), as in the fp32 kernels; each lane then holds 16
// keys of a 32-key block: {0-3, 8-11, 16-19, 24-27} + 4g.  Those registers
// become the B operand of the next product (P^T or dS^T) without any lane
// exchange, because the reduction over keys may run in any order: within
// each group of 16 keys the reduction position 8g + i is given to key
// 8(i / 4) + 4g + i % 4.  Every tile is stored in LDS once, as rows
// [row][dim] (NDB*32 + 8 bf16 per row).  The operands along head dimensions
// are read from it as 16 bytes; the operands along rows (V^T, K^T, Q^T,
// dout^T) are gathered in the permuted order above by gfx950's transposing
// LDS reads (frag_rt).  Against transposed copies written with 16-bit LDS
// stores this took the attention from 3.61 to 2.82 ms per step, with
// bit-identical results, and halved the backward kernels' LDS, so their
// workgroups now fit three per compute unit.
//
// P and dS are rounded to bf16 for their products; the row statistics, the
// exponentials and every sum stay fp32.  As in the fp32 kernels each
// workgroup is four waves owning 128 rows, tiles of 64 rows stream through
// two LDS buffers with a register prefetch of the next tile (rows past T
// read row T - 1: their scores are masked or their weights are zero), the
// grid runs longest-first, and every output row has one owner, so results
// are deterministic.
#include "common.h"
#include "kernels.h"

namespace gk {
namespace {


constexpr int RQ = 128;  // rows owned per workgroup (four waves of 32)
constexpr int RT = 64;   // rows per staged tile
constexpr float L2E = 1.4426950408889634f;
constexpr float LN_2 = 0.6931471805599453f;


__device__ __forceinline__ void zero(floatx16& x) {
#pragma unroll
    for (int e = 0; e < 16; e++) x[e] = 0.f;
}


// Eight registers of a 32-row accumulator block, e = 8h..8h+7, as a bf16
// B operand (reduction positions 8g..8g+7 of the 16-row group h).
template <class H>
__device__ __forceinline__ uint4 pack8(const floatx16& x, int h) {
    return make_uint4(H::pk(x[8 * h], x[8 * h + 1]), H::pk(x[8 * h + 2], x[8 * h + 3]),
                      H::pk(x[8 * h + 4], x[8 * h + 5]), H::pk(x[8 * h + 6], x[8 * h + 7]));
}

// A 64-row tile of one head (HS bf16 per row) held in registers between its
// global load (16 bytes per access, rows clamped to T - 1) and its LDS store.
template <int HS>
struct Tile16 {
    static constexpr int CH = HS / 8;             // 16-byte chunks per row
    static constexpr int N = RT * CH;             // chunks per tile
    static constexpr int PER = (N + 255) / 256;   // per thread
    // A native vector, not the uint4 struct: a struct is copied as a memcpy,
    // and the optimizer then forwards global -> registers -> LDS into one
    // global-to-LDS copy at the LDS store, which issues the load there
    // instead of a whole step ahead.
    typedef unsigned int chunk_t __attribute__((ext_vector_type(4)));
    chunk_t v[PER];
    __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int64_t ld, int r0,
                                         int T) {
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int idx = threadIdx.x + 256 * i;
            if (N % 256 == 0 || idx < N) {
                const int r = min(r0 + idx / CH, T - 1), c = (idx % CH) * 8;
                v[i] = *reinterpret_cast<const chunk_t*>(base + (int64_t)r * ld + c);
            }
        }
    }
    // [row][dim], row stride LD
    template <int LD>
    __device__ __forceinline__ void store_rows(uint16_t* sm) const {
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int idx = threadIdx.x + 256 * i;
            if (N % 256 == 0 || idx < N)
                *reinterpret_cast<chunk_t*>(sm + (idx / CH) * LD + (idx % CH) * 8) = v[i];
        }
    }
};

// 16-byte LDS operand read
__device__ __forceinline__ uint4 rd(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}

typedef short tr4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) tr4_t* lds_tr4_ptr;

// MFMA operand of head dims db..db+31 (lane li = dim db + li) over reduction
// positions 8g..8g+7 of the 16-row group starting at row kb16, from a tile
// stored as rows [row][dim] (stride ld), with two transposing LDS reads
// (ds_read_b64_tr_b16).  In each 16-lane group of such a read, lane r
// addresses 4 consecutive dims of one row and lane j receives element j of
// each 16-element row of the group's 16x4 block, so lane r at
// (row0 + r/4, dim0 + 4*(r%4)) hands lane j rows row0..row0+3 of dim0 + j.
// Reduction positions 8g..8g+3 and 8g+4..8g+7 are rows kb16 + 4g + 0..3 and
// kb16 + 8 + 4g + 0..3: the order in which the score registers feed the
// other operand.
__device__ __forceinline__ uint4 frag_rt(const uint16_t* s, int ld, int db, int kb16, int lane) {
    const int grp = lane >> 4, r = lane & 15;
    const int dim = db + 16 * (grp & 1) + 4 * (r & 3);
    const int row = kb16 + 4 * (grp >> 1) + (r >> 2);
    const uint16_t* p = s + row * ld + dim;
    const tr4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr4_ptr)p);
    const tr4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr4_ptr)(p + 8 * ld));
    const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
    return make_uint4(a.x, a.y, b.x, b.y);
}

// Zero dims HS..NDB*32-1 of every row of a [row][dim] tile (read by the
// MFMA as padding head dimensions whose outputs are discarded).
template <int HS, int NDB, int LD>
__device__ __forceinline__ void zero_pad_cols(uint16_t* sm) {
    if (NDB * 32 > HS)
        for (int i = threadIdx.x; i < RT * (NDB * 32 - HS); i += blockDim.x)
            sm[(i / (NDB * 32 - HS)) * LD + HS + i % (NDB * 32 - HS)] = 0;
}

// Write one lane's accumulator blocks (rows = head dims d*32 + 8(e/4) +
// 4g + e%4 of this lane's row) as bf16, scaled.
template <int HS, int NDB, class H>
__device__ __forceinline__ void put_row(uint16_t* row, const floatx16 (&acc)[NDB], int g,
                                        float mul) {
#pragma unroll
    for (int d = 0; d < NDB; d++)
#pragma unroll
        for (int c = 0; c < 4; c++) {
            const int dim0 = d * 32 + 8 * c + 4 * g;
            if (dim0 < HS)
                *reinterpret_cast<uint2*>(row + dim0) =
                    make_uint2(H::pk(acc[d][4 * c] * mul, acc[d][4 * c + 1] * mul),
                               H::pk(acc[d][4 * c + 2] * mul, acc[d][4 * c + 3] * mul));
        }
}

template <int HS, class H>
__global__ __launch_bounds__(256, 2) void attn16_fwd_kernel(uint16_t* __restrict__ out,
                                                            float* __restrict__ lse,
                                                            const uint16_t* __restrict__ qkv,
                                                            int T, int C, int NH, float qscale,
                                                            int qb0) {
    constexpr int NKS = HS / 16, NDB = (HS + 31) / 32, LDK = NDB * 32 + 8;
    __shared__ __attribute__((aligned(16))) uint16_t ks[2][RT * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t vs[2][RT * LDK];

    // query blocks before qb0 are not computed (their rows are already stored)
    const int nqb = (T + RQ - 1) / RQ;
    const int nbh = gridDim.x / (nqb - qb0);
    const int bh = blockIdx.x % nbh;
    const int qb = nqb - 1 - blockIdx.x / nbh;  // longest first
    const int b = bh / NH, h = bh - b * NH;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 31, g = lane >> 5;
    const int64_t ld = 3 * (int64_t)C;
    const uint16_t* base = qkv + (int64_t)b * T * ld + h * HS;
    const int q0 = qb * RQ;
    const int qw = q0 + wave * 32;
    const int q = qw + li;
    const int qmax = qw < T ? min(qw + 31, T - 1) : -1;
    const int nkt = (min(q0 + RQ, T) - 1) / RT + 1;
    zero_pad_cols<HS, NDB, LDK>(vs[0]);
    zero_pad_cols<HS, NDB, LDK>(vs[1]);

    uint4 qv[NKS];  // this lane's query, dims 16j + 8g .. +7
#pragma unroll
    for (int j = 0; j < NKS; j++)
        qv[j] = rd(base + (int64_t)min(q, T - 1) * ld + 16 * j + 8 * g);
    floatx16 o[NDB];
#pragma unroll
    for (int d = 0; d < NDB; d++) zero(o[d]);
    float m = -INFINITY, l = 0.f;

    Tile16<HS> kreg, vreg;
    kreg.load(base + C, ld, 0, T);
    vreg.load(base + 2 * C, ld, 0, T);
    kreg.template store_rows<LDK>(ks[0]);
    vreg.template store_rows<LDK>(vs[0]);
    __syncthreads();
    for (int kt = 0; kt < nkt; kt++) {
        const int cur = kt & 1;
        const int nxt = min(kt + 1, nkt - 1) * RT;  // the last tile reloads itself
        kreg.load(base + C, ld, nxt, T);
        vreg.load(base + 2 * C, ld, nxt, T);
        const int k0 = kt * RT;
        if (k0 <= qmax) {
            const uint16_t* kr = ks[cur] + li * LDK + 8 * g;
            floatx16 sc[2];
            zero(sc[0]);
            zero(sc[1]);
#pragma unroll
            for (int j = 0; j < NKS; j++) {
                sc[0] = H::mma(rd(kr + 16 * j), qv[j], sc[0]);
                sc[1] = H::mma(rd(kr + 32 * LDK + 16 * j), qv[j], sc[1]);
            }
            if ((k0 + RT - 1 > qw) || (k0 + RT > T)) {  // tile touches the mask
#pragma unroll
                for (int kb = 0; kb < 2; kb++)
#pragma unroll
                    for (int e = 0; e < 16; e++) {
                        const int key = k0 + kb * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                        sc[kb][e] = ((key > q) | (key >= T)) ? -INFINITY : sc[kb][e];
                    }
            }
            float mt = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int e = 0; e < 16; e++) mt = fmaxf(mt, sc[kb][e]);
            mt = fmaxf(mt, __shfl_xor(mt, 32, WAVE)) * qscale;
            const float mn = fmaxf(m, mt);
            const float corr = __builtin_amdgcn_exp2f(m - mn);
            float ls = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(sc[kb][e], qscale, -mn));
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
                for (int hh = 0; hh < 2; hh++) {
                    const uint4 pb = pack8<H>(sc[kb], hh);
#pragma unroll
                    for (int d = 0; d < NDB; d++)
                        o[d] = H::mma(frag_rt(vs[cur], LDK, d * 32, kb * 32 + 16 * hh, lane), pb,
                                      o[d]);
                }
        }
        kreg.template store_rows<LDK>(ks[cur ^ 1]);
        vreg.template store_rows<LDK>(vs[cur ^ 1]);
        __syncthreads();
    }
    if (q < T) {
        put_row<HS, NDB, H>(out + ((int64_t)b * T + q) * C + h * HS, o, g, 1.f / l);
        if (g == 0) lse[((int64_t)b * NH + h) * T + q] = (m + log2f(l)) * LN_2;
    }
}

// dQ (lane owns a query) and D = rowsum(dout * out) for the key/value
// kernel.  K is staged as rows, read as 16 bytes for S^T = K Q^T and with
// the transposing reads for dQ^T = K^T dS^T; V as rows for dP^T = V dout^T.
template <int HS, class H>
__global__ __launch_bounds__(256, 3) void attn16_dq_kernel(
    uint16_t* __restrict__ dqkv, float* __restrict__ Dout, const uint16_t* __restrict__ dout,
    const uint16_t* __restrict__ out, const uint16_t* __restrict__ qkv,
    const float* __restrict__ lse, int T, int C, int NH, float qscale, float scale) {
    constexpr int NKS = HS / 16, NDB = (HS + 31) / 32, LDK = NDB * 32 + 8;
    __shared__ __attribute__((aligned(16))) uint16_t ks[2][RT * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t vs[2][RT * LDK];

    const int nqb = (T + RQ - 1) / RQ;
    const int nbh = gridDim.x / nqb;
    const int bh = blockIdx.x % nbh;
    const int qb = nqb - 1 - blockIdx.x / nbh;  // longest first
    const int b = bh / NH, h = bh - b * NH;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 31, g = lane >> 5;
    const int64_t ld = 3 * (int64_t)C;
    const uint16_t* base = qkv + (int64_t)b * T * ld + h * HS;
    const uint16_t* dobase = dout + (int64_t)b * T * C + h * HS;
    const uint16_t* obase = out + (int64_t)b * T * C + h * HS;
    const int q0 = qb * RQ;
    const int qw = q0 + wave * 32;
    const int q = qw + li;
    const int qc = min(q, T - 1);
    const int qmax = qw < T ? min(qw + 31, T - 1) : -1;
    const int nkt = (min(q0 + RQ, T) - 1) / RT + 1;
    zero_pad_cols<HS, NDB, LDK>(ks[0]);
    zero_pad_cols<HS, NDB, LDK>(ks[1]);

    uint4 qv[NKS], dv[NKS];
    float dsum = 0.f;
#pragma unroll
    for (int j = 0; j < NKS; j++) {
        qv[j] = rd(base + (int64_t)qc * ld + 16 * j + 8 * g);
        dv[j] = rd(dobase + (int64_t)qc * C + 16 * j + 8 * g);
        const uint4 ov = rd(obase + (int64_t)qc * C + 16 * j + 8 * g);
        const uint32_t dw[4] = {dv[j].x, dv[j].y, dv[j].z, dv[j].w};
        const uint32_t ow[4] = {ov.x, ov.y, ov.z, ov.w};
#pragma unroll
        for (int i = 0; i < 4; i++)
            dsum += H::lo(dw[i]) * H::lo(ow[i]) + H::hi(dw[i]) * H::hi(ow[i]);
    }
    const float Dq = dsum + __shfl_xor(dsum, 32, WAVE);
    const int64_t srow = ((int64_t)b * NH + h) * T;
    if (q < T && g == 0) Dout[srow + q] = Dq;
    const float lq = lse[srow + qc] * L2E;
    floatx16 dq[NDB];
#pragma unroll
    for (int d = 0; d < NDB; d++) zero(dq[d]);

    Tile16<HS> kreg, vreg;
    kreg.load(base + C, ld, 0, T);
    vreg.load(base + 2 * C, ld, 0, T);
    kreg.template store_rows<LDK>(ks[0]);
    vreg.template store_rows<LDK>(vs[0]);
    __syncthreads();
    for (int kt = 0; kt < nkt; kt++) {
        const int cur = kt & 1;
        const int nxt = min(kt + 1, nkt - 1) * RT;
        kreg.load(base + C, ld, nxt, T);
        vreg.load(base + 2 * C, ld, nxt, T);
        const int k0 = kt * RT;
        if (k0 <= qmax) {
            const uint16_t* kr = ks[cur] + li * LDK + 8 * g;
            const uint16_t* vr = vs[cur] + li * LDK + 8 * g;
            floatx16 sc[2], dp[2];
#pragma unroll
            for (int kb = 0; kb < 2; kb++) {
                zero(sc[kb]);
                zero(dp[kb]);
            }
#pragma unroll
            for (int j = 0; j < NKS; j++)
#pragma unroll
                for (int kb = 0; kb < 2; kb++) {
                    sc[kb] = H::mma(rd(kr + kb * 32 * LDK + 16 * j), qv[j], sc[kb]);
                    dp[kb] = H::mma(rd(vr + kb * 32 * LDK + 16 * j), dv[j], dp[kb]);
                }
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    const int key = k0 + kb * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                    const bool live = (key <= q) & (key < T);
                    const float p = __builtin_amdgcn_exp2f(fmaf(sc[kb][e], qscale, -lq));
                    sc[kb][e] = live ? p * (dp[kb][e] - Dq) : 0.f;
                }
#pragma unroll
            for (int kb = 0; kb < 2; kb++)
#pragma unroll
                for (int hh = 0; hh < 2; hh++) {
                    const uint4 sb = pack8<H>(sc[kb], hh);
#pragma unroll
                    for (int d = 0; d < NDB; d++)
                        dq[d] = H::mma(frag_rt(ks[cur], LDK, d * 32, kb * 32 + 16 * hh, lane), sb,
                                       dq[d]);
                }
        }
        kreg.template store_rows<LDK>(ks[cur ^ 1]);
        vreg.template store_rows<LDK>(vs[cur ^ 1]);
        __syncthreads();
    }
    if (q < T) put_row<HS, NDB, H>(dqkv + ((int64_t)b * T + q) * ld + h * HS, dq, g, scale);
}

// dK and dV (lane owns a key).  Q and dout are staged as rows, read as 16
// bytes for S = Q K^T and dP = dout V^T (queries down the accumulator) and
// with the transposing reads for dK^T = Q^T dS and dV^T = dout^T P.  With
// the next tile's loads issued a whole step ahead it needs 200 VGPRs, so two
// workgroups share a compute unit (capped for three it spills, and the spill
// reloads then wait for the prefetch).
template <int HS, class H>
__global__ __launch_bounds__(256, 2) void attn16_dkdv_kernel(
    uint16_t* __restrict__ dqkv, const uint16_t* __restrict__ dout,
    const uint16_t* __restrict__ qkv, const float* __restrict__ lse, const float* __restrict__ D,
    int T, int C, int NH, float qscale, float scale) {
    constexpr int NKS = HS / 16, NDB = (HS + 31) / 32, LDK = NDB * 32 + 8;
    __shared__ __attribute__((aligned(16))) uint16_t qs[2][RT * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t ds[2][RT * LDK];
    __shared__ __attribute__((aligned(16))) float lsm[2][RT], dsm[2][RT];

    const int nkb = (T + RQ - 1) / RQ;
    const int nbh = gridDim.x / nkb;
    const int bh = blockIdx.x % nbh;
    const int kb0 = blockIdx.x / nbh;  // lowest keys = most query tiles: first
    const int b = bh / NH, h = bh - b * NH;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 31, g = lane >> 5;
    const int64_t ld = 3 * (int64_t)C;
    const uint16_t* base = qkv + (int64_t)b * T * ld + h * HS;
    const uint16_t* dobase = dout + (int64_t)b * T * C + h * HS;
    const int64_t srow = ((int64_t)b * NH + h) * T;
    const int kw = kb0 * RQ + wave * 32;  // first key of this wave
    const int key = kw + li;
    const int kc = min(key, T - 1);
    zero_pad_cols<HS, NDB, LDK>(qs[0]);
    zero_pad_cols<HS, NDB, LDK>(qs[1]);
    zero_pad_cols<HS, NDB, LDK>(ds[0]);
    zero_pad_cols<HS, NDB, LDK>(ds[1]);

    uint4 kv[NKS], vv[NKS];
#pragma unroll
    for (int j = 0; j < NKS; j++) {
        kv[j] = rd(base + C + (int64_t)kc * ld + 16 * j + 8 * g);
        vv[j] = rd(base + 2 * C + (int64_t)kc * ld + 16 * j + 8 * g);
    }
    floatx16 dk[NDB], dvv[NDB];
#pragma unroll
    for (int d = 0; d < NDB; d++) {
        zero(dk[d]);
        zero(dvv[d]);
    }
    const int qt0 = (kb0 * RQ) / RT;
    const int nqt = (T + RT - 1) / RT;
    Tile16<HS> qreg, dreg;
    float sreg = 0.f;  // one lse (wave 0) or D (the other waves) value per thread
    // every thread loads (a fixed count per step); the base-2 scaling of lse
    // waits for the LDS store, so the load stays in flight with the tile's
    auto load_stats = [&](int qt) {
        const int t = min(qt * RT + lane, T - 1);
        sreg = (wave == 0 ? lse : D)[srow + t];
    };
    auto store_stats = [&](int buf) {
        if (wave == 0) lsm[buf][lane] = sreg * L2E;
        else if (wave == 1) dsm[buf][lane] = sreg;
    };
    qreg.load(base, ld, qt0 * RT, T);
    dreg.load(dobase, C, qt0 * RT, T);
    load_stats(qt0);
    qreg.template store_rows<LDK>(qs[0]);
    dreg.template store_rows<LDK>(ds[0]);
    store_stats(0);
    __syncthreads();
    for (int qt = qt0; qt < nqt; qt++) {
        const int cur = (qt - qt0) & 1;
        const int nxt = min(qt + 1, nqt - 1);
        load_stats(nxt);
        qreg.load(base, ld, nxt * RT, T);
        dreg.load(dobase, C, nxt * RT, T);
#pragma unroll
        for (int qh = 0; qh < 2; qh++) {
            const int qlo = qt * RT + qh * 32;
            if (kw >= T || qlo + 31 < kw || qlo >= T) continue;  // empty under the mask
            const uint16_t* qr = qs[cur] + (qh * 32 + li) * LDK + 8 * g;
            const uint16_t* dr = ds[cur] + (qh * 32 + li) * LDK + 8 * g;
            floatx16 sc, dp;
            zero(sc);
            zero(dp);
#pragma unroll
            for (int j = 0; j < NKS; j++) {
                sc = H::mma(rd(qr + 16 * j), kv[j], sc);
                dp = H::mma(rd(dr + 16 * j), vv[j], dp);
            }
            // steps e = 4c..4c+3 hold queries qh*32 + 8c + 4g + (0..3): one
            // float4 of each statistic; the mask is a select, not a branch
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const int ql = qh * 32 + 8 * c + 4 * g;
                const float4 l4 = *reinterpret_cast<const float4*>(&lsm[cur][ql]);
                const float4 d4 = *reinterpret_cast<const float4*>(&dsm[cur][ql]);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int e = 4 * c + j;
                    const float p = __builtin_amdgcn_exp2f(fmaf(sc[e], qscale, -lv[j]));
                    sc[e] = p;
                    dp[e] = p * (dp[e] - dv4[j]);
                }
            }
            // the mask (selects, so masked infinities do not survive) only on
            // blocks that touch it: the diagonal and the sequence end (the
            // same test for the whole wave)
            if (qlo < kw + 31 || qlo + 31 >= T) {
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    const int qa = qt * RT + qh * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                    const bool live = (qa < T) & (key <= qa);
                    sc[e] = live ? sc[e] : 0.f;
                    dp[e] = live ? dp[e] : 0.f;
                }
            }
#pragma unroll
            for (int hh = 0; hh < 2; hh++) {
                const uint4 pb = pack8<H>(sc, hh), sb = pack8<H>(dp, hh);
#pragma unroll
                for (int d = 0; d < NDB; d++) {
                    dvv[d] = H::mma(frag_rt(ds[cur], LDK, d * 32, qh * 32 + 16 * hh, lane), pb,
                                    dvv[d]);
                    dk[d] = H::mma(frag_rt(qs[cur], LDK, d * 32, qh * 32 + 16 * hh, lane), sb,
                                   dk[d]);
                }
            }
        }
        qreg.template store_rows<LDK>(qs[cur ^ 1]);
        dreg.template store_rows<LDK>(ds[cur ^ 1]);
        store_stats(cur ^ 1);
        __syncthreads();
    }
    if (key < T) {
        uint16_t* row = dqkv + ((int64_t)b * T + key) * ld + h * HS;
        put_row<HS, NDB, H>(row + C, dk, g, scale);
        put_row<HS, NDB, H>(row + 2 * C, dvv, g, 1.f);
    }
}

template <int HS, class H>
hipError_t bwd16(hipStream_t s, uint16_t* dqkv, float* D, const uint16_t* dout,
                 const uint16_t* qkv, const uint16_t* out, const float* lse, int B, int T, int C,
                 int NH) {
    const int nb = (T + RQ - 1) / RQ;
    const float scale = 1.0f / sqrtf((float)HS);
    const float qscale = L2E * scale;
    launch((attn16_dq_kernel<HS, H>), dim3(B * NH * nb), dim3(256), 0, s, dqkv, D, dout,
                       out, qkv, lse, T, C, NH, qscale, scale);
    launch((attn16_dkdv_kernel<HS, H>), dim3(B * NH * nb), dim3(256), 0, s, dqkv, dout,
                       qkv, lse, D, T, C, NH, qscale, scale);
    return hipGetLastError();
}

template <int HS, class H>
hipError_t fwd16(hipStream_t s, uint16_t* out, float* lse, const uint16_t* qkv, int B, int T,
                 int C, int NH, int q_first) {
    const int nqb = (T + RQ - 1) / RQ;
    const int qb0 = q_first / RQ;
    const float qscale = L2E / sqrtf((float)HS);
    launch((attn16_fwd_kernel<HS, H>), dim3(B * NH * (nqb - qb0)), dim3(256), 0, s, out, lse,
           qkv, T, C, NH, qscale, qb0);
    return hipGetLastError();
}


template <class H>
hipError_t fwd_h(hipStream_t s, uint16_t* out, float* lse, const uint16_t* qkv, int B, int T,
                 int C, int NH, int q_first) {
    switch (C / NH) {
        case 16: return fwd16<16, H>(s, out, lse, qkv, B, T, C, NH, q_first);
        case 32: return fwd16<32, H>(s, out, lse, qkv, B, T, C, NH, q_first);
        case 64: return fwd16<64, H>(s, out, lse, qkv, B, T, C, NH, q_first);
        default: return hipErrorInvalidValue;
    }
}

template <class H>
hipError_t bwd_h(hipStream_t s, uint16_t* dqkv, float* D, const uint16_t* dout,
                 const uint16_t* qkv, const uint16_t* out, const float* lse, int B, int T, int C,
                 int NH) {
    switch (C / NH) {
        case 16: return bwd16<16, H>(s, dqkv, D, dout, qkv, out, lse, B, T, C, NH);
        case 32: return bwd16<32, H>(s, dqkv, D, dout, qkv, out, lse, B, T, C, NH);
        case 64: return bwd16<64, H>(s, dqkv, D, dout, qkv, out, lse, B, T, C, NH);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t attention_forward_half(hipStream_t s, uint16_t* out, float* lse, const uint16_t* qkv,
                                  int B, int T, int C, int NH, int dt, int q_first) {
    if (B <= 0 || T <= 0) return hipSuccess;
    if (q_first < 0 || q_first >= T) return hipErrorInvalidValue;
    return dt == DT_F16 ? fwd_h<HF16>(s, out, lse, qkv, B, T, C, NH, q_first)
                        : fwd_h<HBF16>(s, out, lse, qkv, B, T, C, NH, q_first);
}

hipError_t attention_backward_half(hipStream_t s, uint16_t* dqkv, float* D,
                                   const uint16_t* dout, const uint16_t* qkv,
                                   const uint16_t* out, const float* lse, int B, int T, int C,
                                   int NH, int dt) {
    if (B <= 0 || T <= 0) return hipSuccess;
    return dt == DT_F16 ? bwd_h<HF16>(s, dqkv, D, dout, qkv, out, lse, B, T, C, NH)
                        : bwd_h<HBF16>(s, dqkv, D, dout, qkv, out, lse, B, T, C, NH);
}

}  // namespace gk
