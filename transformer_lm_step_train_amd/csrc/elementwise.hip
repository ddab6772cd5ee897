// Bandwidth-bound kernels: token+position embedding (forward, and its
// deterministic scatter-add backward), bias-gradient column sums, zeroing of
// the gradient arena and the AdamW sweep over the flat parameter arena.
//
// Embedding (ujoy.net article "徒手用 1000 行 C 语言实现", section "用C语言实现
// LLM": the encoder layer):  x[b,t] = wte[tok[b,t]] + wpe[t];  the backward
// adds each position's gradient into its token row and its position row.
// Rows of wte hit by several positions are summed in position order after a
// sort of (token, position) keys, so the result does not depend on timing.
//
// AdamW (section "训练过程" runs Adam at lr 1e-4; decoupled weight decay as in
// Loshchilov & Hutter): per element, with bias corrections c1 = 1 - b1^step
// and c2 = 1 - b2^step computed once on the host,
//   m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
//   p -= lr ((m/c1) / (sqrt(v/c2) + eps) + wd p).
#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

template <class E>
__global__ __launch_bounds__(256) void encoder_fwd_kernel(E* __restrict__ out,
                                                          const int32_t* __restrict__ tok,
                                                          const float* __restrict__ wte,
                                                          const float* __restrict__ wpe,
                                                          int B, int T, int C, int V,
                                                          int* __restrict__ flag) {
    const int C4 = C >> 2;
    const int64_t n = (int64_t)B * T * C4;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t bt = i / C4;
        const int c = (int)(i - bt * C4) * 4;
        const int t = (int)(bt % T);
        const int id = tok[bt];
        float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
        if (id >= 0 && id < V) {
            const float4 a = ld4(wte + (int64_t)id * C + c);
            const float4 p = wpe ? ld4(wpe + (int64_t)t * C + c) : make_float4(0.f, 0.f, 0.f, 0.f);
            r = make_float4(a.x + p.x, a.y + p.y, a.z + p.z, a.w + p.w);
        } else if (c == 0) {
            atomicOr(flag, 1);
        }
        Act<E>::st(out + bt * C + c, r);
    }
}

// Sort of the (token << pos_bits | position) keys, one workgroup of 1024
// threads.  Ids outside [0, V) get the token field V so the backward skips
// them; slots past n get all bits set and sort last.  The keys are built in
// position order and are unique, so a stable sort on the token field alone
// gives them in (token, position) order: a least-significant-digit radix
// sort, 4 bits per pass.  Thread t holds keys [t*EPT, (t+1)*EPT) in
// registers; each pass counts its digits into a [16][1024] table in LDS,
// scans the table in digit-major order (so equal digits keep thread order)
// and scatters the keys through LDS.
template <int EPT>
__global__ __launch_bounds__(1024) void encoder_sort_kernel(uint32_t* __restrict__ keys,
                                                            const int32_t* __restrict__ tok,
                                                            int n, int V, int pos_bits,
                                                            int n_pow2, int passes) {
    constexpr int NT = 1024, NK = EPT * NT;
    extern __shared__ uint32_t sm[];
    uint32_t* sk = sm;                                      // NK keys
    uint16_t* cnt = reinterpret_cast<uint16_t*>(sm + NK);   // [16][NT] counts
    // The 16 wave totals of the scan borrow the first slots of the key area:
    // between a pass's last read of sk (the barrier that ends the previous
    // pass) and its scatter (after the scan's last barrier) nothing else
    // touches it.  This keeps the 32-key variant at exactly 160 KiB.
    uint32_t* wsum = sm;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    uint32_t k[EPT];
#pragma unroll
    for (int e = 0; e < EPT; e++) {
        const int i = t * EPT + e;
        uint32_t key = 0xFFFFFFFFu;
        if (i < n) {
            const int id = tok[i];
            const uint32_t tf = (id >= 0 && id < V) ? (uint32_t)id : (uint32_t)V;
            key = (tf << pos_bits) | (uint32_t)i;
        }
        k[e] = key;
    }
    for (int pass = 0; pass < passes; pass++) {
        const int sh = pos_bits + 4 * pass;
        // digit counts of this thread's keys
        uint32_t total = 0;
#pragma unroll
        for (int d = 0; d < 16; d++) {
            uint32_t c = 0;
#pragma unroll
            for (int e = 0; e < EPT; e++) c += ((k[e] >> sh) & 15u) == (uint32_t)d;
            cnt[d * NT + t] = (uint16_t)c;
        }
        __syncthreads();
        // exclusive scan of the 16*NT counts in index order: thread t owns
        // entries [16t, 16t + 16)
        uint32_t v[16];
#pragma unroll
        for (int j = 0; j < 16; j++) {
            v[j] = cnt[16 * t + j];
            total += v[j];
        }
        uint32_t incl = total;  // inclusive scan of the per-thread totals over the wave
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t up = __shfl_up(incl, off, 64);
            if (lane >= off) incl += up;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        uint32_t base = incl - total;
        for (int w = 0; w < wave; w++) base += wsum[w];
#pragma unroll
        for (int j = 0; j < 16; j++) {
            cnt[16 * t + j] = (uint16_t)base;
            base += v[j];
        }
        __syncthreads();
        // stable scatter: each thread's keys of digit d go, in order, to the
        // slots its scanned count for d starts at
#pragma unroll
        for (int e = 0; e < EPT; e++) {
            const uint32_t d = (k[e] >> sh) & 15u;
            const uint32_t dst = cnt[d * NT + t];
            cnt[d * NT + t] = (uint16_t)(dst + 1);
            sk[dst] = k[e];
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < EPT; e++) k[e] = sk[t * EPT + e];
        __syncthreads();
    }
#pragma unroll
    for (int e = 0; e < EPT; e++) {
        const int i = t * EPT + e;
        if (i < n_pow2) keys[i] = k[e];
    }
}

// Embedding backward into wte, in two fixed-order stages over the sorted
// (token, position) keys cut into chunks of EB_CHUNK consecutive keys, so
// that a token repeated r times (frequent tokens of real text) costs about
// r / EB_CHUNK serial row additions instead of r.
//   Stage 1, one wave per chunk: the chunk's keys form pieces of runs of
//   equal tokens; each piece's gradient rows are summed in key (= position)
//   order.  A piece that is a whole run is added into its wte row at once
//   (no other chunk holds that token).  A piece that continues from the
//   previous chunk goes to the chunk's slot 0; one that continues into the
//   next chunk and not from the previous one to slot 1.
//   Stage 2, one wave per chunk where a run spanning later chunks starts:
//   the run's slot 1, then slot 0 of each later chunk it reaches, summed in
//   chunk order and added into the run's wte row.
// Ids outside [0, V) were sorted with the token field V and are skipped.
constexpr int EB_CHUNK = 16;

template <int NCH, class E>
__global__ __launch_bounds__(256) void encoder_bwd_chunk_kernel(float* __restrict__ dwte,
                                                                float* __restrict__ ws,
                                                                const E* __restrict__ dx,
                                                                const uint32_t* __restrict__ keys,
                                                                int n, int C, int V,
                                                                int pos_bits) {
    const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int i0 = c * EB_CHUNK;
    if (i0 >= n) return;
    const int cnt = min(n - i0, EB_CHUNK);
    const uint32_t pmask = (1u << pos_bits) - 1u;
    const int C4 = C >> 2;
    const uint32_t kl = lane < cnt ? keys[i0 + lane] : 0xFFFFFFFFu;
    const uint32_t tprev = i0 > 0 ? keys[i0 - 1] >> pos_bits : 0xFFFFFFFFu;
    const uint32_t tnext = i0 + cnt < n ? keys[i0 + cnt] >> pos_bits : 0xFFFFFFFFu;
    float4 acc[NCH], pre[NCH];
#pragma unroll
    for (int ch = 0; ch < NCH; ch++) acc[ch] = make_float4(0.f, 0.f, 0.f, 0.f);
    uint32_t cur = (uint32_t)__shfl((int)kl, 0, 64) >> pos_bits;
    int start = 0;  // first key of the current piece, relative to i0
    // The wte row of the current piece's token is read when the piece starts,
    // so the read overlaps the piece's own row sums (used if the piece turns
    // out to be a whole run).
    auto prefetch = [&]() {
#pragma unroll
        for (int ch = 0; ch < NCH; ch++) {
            const int c4 = lane + 64 * ch;
            pre[ch] = cur < (uint32_t)V && c4 < C4 ? ld4(dwte + (int64_t)cur * C + 4 * c4)
                                                   : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    prefetch();
    // piece [start, end) of token cur, summed in acc
    auto flush = [&](int end) {
        if (cur >= (uint32_t)V) return;
        const bool left = start == 0 && tprev == cur;
        const bool right = end == cnt && tnext == cur;
        float* out = (!left && !right) ? dwte + (int64_t)cur * C
                                       : ws + ((int64_t)c * 2 + (left ? 0 : 1)) * C;
#pragma unroll
        for (int ch = 0; ch < NCH; ch++) {
            const int c4 = lane + 64 * ch;
            if (c4 >= C4) continue;
            float4 o = acc[ch];
            if (!left && !right) {
                const float4 w = pre[ch];
                o = make_float4(w.x + o.x, w.y + o.y, w.z + o.z, w.w + o.w);
            }
            st4(out + 4 * c4, o);
        }
    };
    for (int g = 0; g < cnt; g += 4) {
        // the rows of four keys are loaded before any is added
        uint32_t kk[4];
        float4 r[4][NCH];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            kk[u] = (uint32_t)__shfl((int)kl, g + u, 64);
            const bool live = g + u < cnt && (kk[u] >> pos_bits) < (uint32_t)V;
            const E* row = dx + (int64_t)(kk[u] & pmask) * C;
#pragma unroll
            for (int ch = 0; ch < NCH; ch++) {
                const int c4 = lane + 64 * ch;
                r[u][ch] = live && c4 < C4 ? Act<E>::ld(row + 4 * c4)
                                           : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; u++) {
            if (g + u >= cnt) break;
            const uint32_t tok = kk[u] >> pos_bits;
            if (tok != cur) {
                flush(g + u);
#pragma unroll
                for (int ch = 0; ch < NCH; ch++) acc[ch] = make_float4(0.f, 0.f, 0.f, 0.f);
                cur = tok;
                start = g + u;
                prefetch();
            }
#pragma unroll
            for (int ch = 0; ch < NCH; ch++) {
                acc[ch].x += r[u][ch].x;
                acc[ch].y += r[u][ch].y;
                acc[ch].z += r[u][ch].z;
                acc[ch].w += r[u][ch].w;
            }
        }
    }
    flush(cnt);
}

template <int NCH>
__global__ __launch_bounds__(256) void encoder_bwd_span_kernel(float* __restrict__ dwte,
                                                               const float* __restrict__ ws,
                                                               const uint32_t* __restrict__ keys,
                                                               int n, int C, int V,
                                                               int pos_bits) {
    const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int nc = (n + EB_CHUNK - 1) / EB_CHUNK;
    if (c + 1 >= nc) return;  // no later chunk
    const int i0 = c * EB_CHUNK, i1 = i0 + EB_CHUNK;
    const uint32_t tok = keys[i1 - 1] >> pos_bits;
    if (tok >= (uint32_t)V || (keys[i1] >> pos_bits) != tok) return;
    // the run started before this chunk: its owner is an earlier chunk
    if (i0 > 0 && (keys[i0] >> pos_bits) == tok && (keys[i0 - 1] >> pos_bits) == tok) return;
    // the run's last chunk: the first later chunk not followed by another key of tok
    int last = -1;
    for (int base = c + 1; base < nc && last < 0; base += 64) {
        const int cc = base + lane;
        bool ends = true;
        if (cc < nc) {
            const int next = min(n, (cc + 1) * EB_CHUNK);  // first key after chunk cc
            ends = next >= n || (keys[next] >> pos_bits) != tok;
        }
        const unsigned long long m = __ballot(ends);
        if (m) last = base + __builtin_ctzll(m);
    }
    const int C4 = C >> 2;
    float4 acc[NCH];
#pragma unroll
    for (int ch = 0; ch < NCH; ch++) {
        const int c4 = lane + 64 * ch;
        acc[ch] = c4 < C4 ? ld4(ws + ((int64_t)c * 2 + 1) * C + 4 * c4)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int cc = c + 1; cc <= last; cc += 4) {
        float4 r[4][NCH];
#pragma unroll
        for (int u = 0; u < 4; u++)
#pragma unroll
            for (int ch = 0; ch < NCH; ch++) {
                const int c4 = lane + 64 * ch;
                r[u][ch] = cc + u <= last && c4 < C4
                               ? ld4(ws + ((int64_t)(cc + u) * 2) * C + 4 * c4)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
        for (int u = 0; u < 4; u++)
#pragma unroll
            for (int ch = 0; ch < NCH; ch++) {
                acc[ch].x += r[u][ch].x;
                acc[ch].y += r[u][ch].y;
                acc[ch].z += r[u][ch].z;
                acc[ch].w += r[u][ch].w;
            }
    }
    float* out = dwte + (int64_t)tok * C;
#pragma unroll
    for (int ch = 0; ch < NCH; ch++) {
        const int c4 = lane + 64 * ch;
        if (c4 >= C4) continue;
        float4 o = ld4(out + 4 * c4);
        o.x += acc[ch].x;
        o.y += acc[ch].y;
        o.z += acc[ch].z;
        o.w += acc[ch].w;
        st4(out + 4 * c4, o);
    }
}

// dwpe[t] += sum over b of dx[b,t], b in order.
template <class E>
__global__ __launch_bounds__(256) void encoder_bwd_wpe_kernel(float* __restrict__ dwpe,
                                                              const E* __restrict__ dx,
                                                              int B, int T, int C) {
    const int C4 = C >> 2;
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= (int64_t)T * C4) return;
    const int t = (int)(i / C4), c = (int)(i - (int64_t)t * C4) * 4;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int b = 0; b < B; b++) {
        const float4 d = Act<E>::ld(dx + ((int64_t)b * T + t) * C + c);
        s.x += d.x;
        s.y += d.y;
        s.z += d.z;
        s.w += d.w;
    }
    float* o = dwpe + (int64_t)t * C + c;
    float4 r = ld4(o);
    r.x += s.x;
    r.y += s.y;
    r.z += s.z;
    r.w += s.w;
    st4(o, r);
}

// Column sums of dy (M rows, N % 4 == 0 columns, leading dim ld): each
// workgroup sums a chunk of rows for 256 columns (four waves, rows strided by
// four), then a second kernel adds the chunk partials in chunk order.
constexpr int BIAS_ROWS = kBiasRows;

template <class E>
__global__ __launch_bounds__(256) void bias_partial_kernel(float* __restrict__ part,
                                                           const E* __restrict__ dy, int M,
                                                           int N, int64_t ld) {
    __shared__ float4 sh[4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = (blockIdx.x * 64 + lane) * 4;
    const int r0 = blockIdx.y * BIAS_ROWS;
    const int r1 = min(M, r0 + BIAS_ROWS);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (col < N) {
        for (int r = r0 + wave; r < r1; r += 4) {
            const float4 d = Act<E>::ld(dy + (int64_t)r * ld + col);
            s.x += d.x;
            s.y += d.y;
            s.z += d.z;
            s.w += d.w;
        }
    }
    sh[wave][lane] = s;
    __syncthreads();
    if (wave == 0 && col < N) {
        float4 t = sh[0][lane];
        for (int w = 1; w < 4; w++) {
            t.x += sh[w][lane].x;
            t.y += sh[w][lane].y;
            t.z += sh[w][lane].z;
            t.w += sh[w][lane].w;
        }
        st4(part + (int64_t)blockIdx.y * N + col, t);
    }
}

// out[c] += sum over rows r of part[r*ncols + c], into out_k[c - k*split]
// with k = c / split (0, 1 or 2).  One workgroup per 64 columns; its 16
// waves sum interleaved rows (wave w takes rows w, w+16, ...) and are then
// added in wave order, so the result is the same on every run.
__global__ __launch_bounds__(1024) void colsum_finish_kernel(float* __restrict__ out0,
                                                             float* __restrict__ out1,
                                                             float* __restrict__ out2,
                                                             int split,
                                                             const float* __restrict__ part,
                                                             int nrows, int ncols) {
    __shared__ float sh[16][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = blockIdx.x * 64 + lane;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    if (c < ncols) {
        int r = wave;
        for (; r + 48 < nrows; r += 64) {
            s0 += part[(int64_t)r * ncols + c];
            s1 += part[(int64_t)(r + 16) * ncols + c];
            s2 += part[(int64_t)(r + 32) * ncols + c];
            s3 += part[(int64_t)(r + 48) * ncols + c];
        }
        for (; r < nrows; r += 16) s0 += part[(int64_t)r * ncols + c];
    }
    sh[wave][lane] = (s0 + s1) + (s2 + s3);
    __syncthreads();
    if (wave == 0 && c < ncols) {
        float t = sh[0][lane];
        for (int w = 1; w < 16; w++) t += sh[w][lane];
        const int k = c / split;
        float* o = k == 0 ? out0 : k == 1 ? out1 : out2;
        o[c - k * split] += t;
    }
}

// The same sums when ncols % 4 == 0, with four columns per load: one
// workgroup per 32 columns, 8 column lanes x 128 row lanes (lane l takes rows
// l, l+128, ...), then a fixed pairwise tree over the row lanes, so the
// result is the same on every run.
__global__ __launch_bounds__(1024) void colsum4_finish_kernel(float* __restrict__ out0,
                                                              float* __restrict__ out1,
                                                              float* __restrict__ out2,
                                                              int split,
                                                              const float* __restrict__ part,
                                                              int nrows, int ncols) {
    __shared__ float4 sh[128][8];
    const int cl = threadIdx.x & 7, rl = threadIdx.x >> 3;
    const int c = blockIdx.x * 32 + cl * 4;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < ncols)
        for (int r = rl; r < nrows; r += 128) {
            const float4 v = ld4(part + (int64_t)r * ncols + c);
            s.x += v.x;
            s.y += v.y;
            s.z += v.z;
            s.w += v.w;
        }
    sh[rl][cl] = s;
    __syncthreads();
    for (int h = 64; h > 0; h >>= 1) {
        if (rl < h) {
            const float4 a = sh[rl][cl], b = sh[rl + h][cl];
            sh[rl][cl] = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
        }
        __syncthreads();
    }
    if (rl == 0 && c < ncols) {
        const float4 t = sh[0][cl];
        const float v[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int k = (c + j) / split;
            float* o = k == 0 ? out0 : k == 1 ? out1 : out2;
            o[c + j - k * split] += v[j];
        }
    }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
    const int64_t n4 = n >> 2;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += stride)
        st4(p + 4 * i, make_float4(0.f, 0.f, 0.f, 0.f));
    for (int64_t i = 4 * n4 + blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += stride)
        p[i] = 0.f;
}

__device__ __forceinline__ float adamw_one(float& p, float g, float& m, float& v, float lr,
                                           float b1, float b2, float eps, float wd, float ibc1,
                                           float ibc2) {
    m = fmaf(b1, m, (1.f - b1) * g);
    v = fmaf(b2, v, (1.f - b2) * g * g);
    const float mhat = m * ibc1;
    const float vhat = v * ibc2;
    // Hardware square root and reciprocal (about 1 ulp each).
    p -= lr * fmaf(mhat, __builtin_amdgcn_rcpf(__builtin_amdgcn_sqrtf(vhat) + eps), wd * p);
    return p;
}

// shadow (optional): bf16 copy of the updated parameters for the matmuls of
// the mixed-precision model.
// The AdamW sweep.  S is the storage type of the optional 16-bit weight copy
// written in the same pass (uint16_t bf16 bits or _Float16; float = none).
// With loss scaling (fp16 model) the gradients hold scale * dL/dp: they are
// divided by *gscale, and the whole sweep is skipped when *skip is set (a
// non-finite gradient was found).
template <class S>
__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ p,
                                                    const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v,
                                                    S* __restrict__ shadow, int64_t n,
                                                    float lr, float b1, float b2, float eps,
                                                    float wd, float bc1, float bc2,
                                                    const float* __restrict__ gscale,
                                                    const int* __restrict__ skip) {
    if (skip && *skip) return;
    const float ig = gscale ? 1.0f / *gscale : 1.0f;
    const float ibc1 = 1.0f / bc1, ibc2 = 1.0f / bc2;
    // One group of four per thread over the whole grid (no grid-stride
    // loop: a grid of every group keeps the most loads in flight), with
    // streaming loads and stores; the n % 4 tail goes to the next threads.
    const int64_t n4 = n >> 2;
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i < n4) {
        float4 pp = ld4_nt(p + 4 * i), gg = ld4_nt(g + 4 * i), mm = ld4_nt(m + 4 * i),
               vv = ld4_nt(v + 4 * i);
        gg = make_float4(gg.x * ig, gg.y * ig, gg.z * ig, gg.w * ig);
        adamw_one(pp.x, gg.x, mm.x, vv.x, lr, b1, b2, eps, wd, ibc1, ibc2);
        adamw_one(pp.y, gg.y, mm.y, vv.y, lr, b1, b2, eps, wd, ibc1, ibc2);
        adamw_one(pp.z, gg.z, mm.z, vv.z, lr, b1, b2, eps, wd, ibc1, ibc2);
        adamw_one(pp.w, gg.w, mm.w, vv.w, lr, b1, b2, eps, wd, ibc1, ibc2);
        st4_nt(p + 4 * i, pp);
        st4_nt(m + 4 * i, mm);
        st4_nt(v + 4 * i, vv);
        if (shadow) Act<S>::st(shadow + 4 * i, pp);
    } else if (i - n4 < (n & 3)) {
        const int64_t t = 4 * n4 + (i - n4);
        adamw_one(p[t], g[t] * ig, m[t], v[t], lr, b1, b2, eps, wd, ibc1, ibc2);
        if (shadow) Act<S>::st1(shadow + t, p[t]);
    }
}

template <class S>
__global__ __launch_bounds__(256) void to_half_kernel(S* __restrict__ out,
                                                      const float* __restrict__ in, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += stride)
        Act<S>::st1(out + i, in[i]);
}

// *flag = 1 if any of g[0..n) is not finite (inf or NaN).  One group of
// four per thread over the whole grid; the n % 4 tail goes to the next
// threads.
__global__ __launch_bounds__(256) void check_finite_kernel(const float* __restrict__ g, int64_t n,
                                                           int* __restrict__ flag) {
    const int64_t n4 = n >> 2;
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    bool bad = false;
    if (i < n4) {
        const float4 x = ld4_nt(g + 4 * i);
        bad = !(__builtin_isfinite(x.x) && __builtin_isfinite(x.y) && __builtin_isfinite(x.z) &&
                __builtin_isfinite(x.w));
    } else if (i - n4 < (n & 3)) {
        bad = !__builtin_isfinite(g[4 * n4 + (i - n4)]);
    }
    if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flag, 1);
}

// Dynamic loss scaling, one step: st = {scale (float bits), good steps,
// found_inf, skipped}.  A step with a non-finite gradient is skipped and
// halves the scale; `interval` clean steps in a row double it.  found_inf is
// cleared for the next step.
__global__ void loss_scale_kernel(float* __restrict__ scale, int* __restrict__ good,
                                  int* __restrict__ found, int* __restrict__ skipped,
                                  int interval, float min_scale) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    if (*found) {
        *scale = fmaxf(*scale * 0.5f, min_scale);
        *good = 0;
        *skipped = 1;
    } else {
        *skipped = 0;
        if (++*good >= interval) {
            *scale = *scale * 2.0f;
            *good = 0;
        }
    }
    *found = 0;
}

inline unsigned grid_for(int64_t work, int per_block, unsigned cap) {
    int64_t g = (work + per_block - 1) / per_block;
    if (g < 1) g = 1;
    return (unsigned)(g > cap ? cap : g);
}

// Rotary position embedding of the q and k slices of each qkv row, in place
// (RoFormer: Su et al. 2021).  Within every head, the pair of channels
// (2i, 2i+1) of a row at position t is rotated by the angle t * theta_i,
// theta_i = 10000^(-2i/hs); dir = -1 applies the inverse rotation, which is
// the backward of the forward rotation (an orthogonal map).  cs holds
// (cos, sin) of t * theta_i for t < T, i < hs/2, computed on the host in
// double.  One thread per pair.
template <class E>
__global__ __launch_bounds__(256) void rope_kernel(E* __restrict__ qkv, const float2* __restrict__ cs,
                                                   int M, int T, int C, int hs, int64_t ld,
                                                   float dir) {
    const int half = hs >> 1;
    const int64_t n = (int64_t)M * C;  // pairs per row: C/2 of q and C/2 of k
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / C;
        const int k = (int)(i - row * C);           // pair index within q|k
        const int col = 2 * k;                       // 0 .. 2C-1 over [q | k]
        const int t = (int)(row % T);
        const int pi = (col % hs) >> 1;              // pair index within the head
        const float2 r = cs[(int64_t)t * half + pi];
        E* p = qkv + row * ld + col;
        const float x = Act<E>::ld1(p), y = Act<E>::ld1(p + 1);
        const float sn = dir * r.y;
        Act<E>::st1(p, x * r.x - y * sn);
        Act<E>::st1(p + 1, x * sn + y * r.x);
    }
}

}  // namespace

hipError_t encoder_forward(hipStream_t s, void* out, const int32_t* tok, const float* wte,
                           const float* wpe, int B, int T, int C, int V, int* flag, int dt) {
    const int64_t n = (int64_t)B * T * (C / 4);
    if (n <= 0) return hipSuccess;
    const dim3 grid(grid_for(n, 256, 65535));
    return by_dt(dt, [&](auto e) {
        using E = decltype(e);
        launch(encoder_fwd_kernel<E>, grid, dim3(256), 0, s, (E*)out, tok, wte, wpe,
                           B, T, C, V, flag);
        return hipGetLastError();
    });
}

// keys per thread of the sort for n_pow2 slots (1024 threads)
inline int sort_ept(int n_pow2) { return n_pow2 <= 1024 ? 1 : n_pow2 / 1024; }
// keys, then the [16][1024] 16-bit count table: 163,840 bytes (gfx950's LDS
// per workgroup) at 32 keys per thread
inline size_t sort_lds(int ept) { return (size_t)ept * 1024 * 4 + 16 * 1024 * 2; }
static_assert(32 * 1024 * 4 + 16 * 1024 * 2 <= 163840, "sort fits the LDS");

template <int EPT>
hipError_t sort_attr() {
    return hipFuncSetAttribute((const void*)encoder_sort_kernel<EPT>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)sort_lds(EPT));
}

// A forward may run fewer positions than the arenas hold, which picks a
// smaller variant, so every variant up to the largest gets its LDS limit.
hipError_t encoder_sort_prepare(int n_pow2) {
    const int top = sort_ept(n_pow2);
    if (top > 32) return hipErrorInvalidValue;
    hipError_t e = sort_attr<1>();
    if (e == hipSuccess && top >= 2) e = sort_attr<2>();
    if (e == hipSuccess && top >= 4) e = sort_attr<4>();
    if (e == hipSuccess && top >= 8) e = sort_attr<8>();
    if (e == hipSuccess && top >= 16) e = sort_attr<16>();
    if (e == hipSuccess && top >= 32) e = sort_attr<32>();
    return e;
}

hipError_t encoder_sort(hipStream_t s, uint32_t* keys, const int32_t* tok, int n, int V,
                        int pos_bits, int n_pow2) {
    if (n <= 0) return hipSuccess;
    // 4-bit passes over the token field, whose largest value is V
    int bits = 1;
    while (bits < 32 && ((uint64_t)V >> bits) != 0) bits++;
    const int passes = (bits + 3) / 4;
    const int ept = sort_ept(n_pow2);
    const size_t lds = sort_lds(ept);
    switch (ept) {
#define SORT_CASE(E)                                                                          \
    case E:                                                                                   \
        launch(encoder_sort_kernel<E>, dim3(1), dim3(1024), lds, s, keys, tok, n, V, pos_bits, \
               n_pow2, passes);                                                               \
        break;
        SORT_CASE(1)
        SORT_CASE(2)
        SORT_CASE(4)
        SORT_CASE(8)
        SORT_CASE(16)
        SORT_CASE(32)
#undef SORT_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <class E>
hipError_t encoder_backward_t(hipStream_t s, float* dwte, float* dwpe, float* ws, const E* dx,
                              const uint32_t* keys, int B, int T_, int C, int V, int pos_bits) {
    const int n = B * T_;
    const int nc = (n + EB_CHUNK - 1) / EB_CHUNK;
    const dim3 grid((nc + 3) / 4), block(256);
#define EB_CASE(N)                                                                            \
    case N:                                                                                   \
        launch((encoder_bwd_chunk_kernel<N, E>), grid, block, 0, s, dwte, ws, dx, keys, n, C, \
               V, pos_bits);                                                                  \
        launch((encoder_bwd_span_kernel<N>), grid, block, 0, s, dwte, (const float*)ws, keys, \
               n, C, V, pos_bits);                                                            \
        break;
    switch ((C + 255) / 256) {
        EB_CASE(1)
        EB_CASE(2)
        EB_CASE(3)
        EB_CASE(4)
        default: return hipErrorInvalidValue;
    }
#undef EB_CASE
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !dwpe) return e;  // no position table (rotary model)
    const int64_t nw = (int64_t)T_ * (C / 4);
    launch(encoder_bwd_wpe_kernel<E>, dim3(grid_for(nw, 256, 1u << 30)), dim3(256),
                       0, s, dwpe, dx, B, T_, C);
    return hipGetLastError();
}

hipError_t encoder_backward(hipStream_t s, float* dwte, float* dwpe, float* ws, const void* dx,
                            const uint32_t* keys, int B, int T, int C, int V, int pos_bits,
                            int dt) {
    if (B * T <= 0) return hipSuccess;
    static_assert(EB_CHUNK == kEmbedChunk, "chunk of the embedding backward");
    return by_dt(dt, [&](auto e) {
        using E = decltype(e);
        return encoder_backward_t<E>(s, dwte, dwpe, ws, (const E*)dx, keys, B, T, C, V,
                                     pos_bits);
    });
}

hipError_t rope_apply(hipStream_t s, void* qkv, const float* cs, int B, int T, int C, int NH,
                      int dir, int dt) {
    const int64_t n = (int64_t)B * T * C;
    if (n <= 0) return hipSuccess;
    const dim3 grid(grid_for(n, 256, 65535));
    const int hs = C / NH;
    return by_dt(dt, [&](auto e) {
        using E = decltype(e);
        launch(rope_kernel<E>, grid, dim3(256), 0, s, (E*)qkv, (const float2*)cs,
                           B * T, T, C, hs, (int64_t)3 * C, (float)dir);
        return hipGetLastError();
    });
}

hipError_t bias_grad(hipStream_t s, float* db, float* part, const void* dy, int M, int N,
                     int64_t ld, int dt) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const int nchunks = (M + BIAS_ROWS - 1) / BIAS_ROWS;
    dim3 grid((N / 4 + 63) / 64, nchunks);
    hipError_t e = by_dt(dt, [&](auto x) {
        using E = decltype(x);
        launch(bias_partial_kernel<E>, grid, dim3(256), 0, s, part, (const E*)dy, M,
                           N, ld);
        return hipGetLastError();
    });
    if (e != hipSuccess) return e;
    return colsum_add(s, db, nullptr, nullptr, N, part, nchunks, N);
}

hipError_t colsum_add(hipStream_t s, float* out0, float* out1, float* out2, int split,
                      const float* part, int nrows, int ncols) {
    if (nrows <= 0 || ncols <= 0) return hipSuccess;
    if (split <= 0 || ncols > 3 * split || (ncols > split && !out1) ||
        (ncols > 2 * split && !out2))
        return hipErrorInvalidValue;
    if ((ncols & 3) == 0)
        launch(colsum4_finish_kernel, dim3((ncols + 31) / 32), dim3(1024), 0, s, out0, out1,
               out2, split, part, nrows, ncols);
    else
        launch(colsum_finish_kernel, dim3((ncols + 63) / 64), dim3(1024), 0, s, out0, out1,
               out2, split, part, nrows, ncols);
    return hipGetLastError();
}

hipError_t fill_zero(hipStream_t s, float* p, int64_t n) {
    if (n <= 0) return hipSuccess;
    launch(fill_zero_kernel, dim3(grid_for(n / 4 + 1, 256, 8192)), dim3(256), 0, s,
                       p, n);
    return hipGetLastError();
}

hipError_t adamw(hipStream_t s, float* p, const float* g, float* m, float* v, void* shadow,
                 int shadow_dt, int64_t n, float lr, float b1, float b2, float eps, float wd,
                 float bc1, float bc2, const float* gscale, const int* skip) {
    if (n <= 0) return hipSuccess;
    // one thread per group of four, plus up to three for the tail
    const dim3 grid(grid_for((n >> 2) + (n & 3), 256, 1u << 30));
    if (!shadow) shadow_dt = DT_F32;
    return by_dt(shadow_dt, [&](auto e) {
        using S = decltype(e);
        launch(adamw_kernel<S>, grid, dim3(256), 0, s, p, g, m, v, (S*)shadow, n, lr,
                           b1, b2, eps, wd, bc1, bc2, gscale, skip);
        return hipGetLastError();
    });
}

hipError_t to_half(hipStream_t s, void* out, const float* in, int64_t n, int dt) {
    if (n <= 0) return hipSuccess;
    return by_dt(dt, [&](auto e) {
        using S = decltype(e);
        launch(to_half_kernel<S>, dim3(grid_for(n, 256, 8192)), dim3(256), 0, s,
                           (S*)out, in, n);
        return hipGetLastError();
    });
}

hipError_t check_finite(hipStream_t s, const float* g, int64_t n, int* flag) {
    if (n <= 0) return hipSuccess;
    launch(check_finite_kernel, dim3(grid_for((n >> 2) + (n & 3), 256, 1u << 30)), dim3(256), 0,
           s, g, n, flag);
    return hipGetLastError();
}

hipError_t loss_scale_update(hipStream_t s, float* scale, int* good, int* found, int* skipped,
                             int interval, float min_scale) {
    launch(loss_scale_kernel, dim3(1), dim3(64), 0, s, scale, good, found, skipped,
                       interval, min_scale);
    return hipGetLastError();
}

}  // namespace gk
