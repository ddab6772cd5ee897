/*
 * gpt2_oracle.c -- plain CPU reference ("oracle") for one GPT-2 training step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark load it.  It shares no code, header or constant with the
 * HIP path.
 *
 * What it computes, and where the pages state it:
 *   - one flat 1-D arena for all weights and one for all activations,
 *     allocated once up front, every tensor a pointer into it
 *     (yinghuohong.cn article "OpenAI创始大神手搓千行C代码训练GPT", section
 *     "脚动完成每一个层前向/反向流传" (manually
 *     completing each layer's forward/backward pass); ujoy.net article "徒手用 1000 行 C 语言
 *     实现", section "用C语言实现LLM");
 *   - a forward and a backward for each of: encoder, layernorm, matmul,
 *     self-attention, gelu, residual, softmax, cross-entropy, chained into a
 *     model (ujoy.net, section "用C语言实现LLM");
 *   - the forward / zero-grad / backward / update loop with Adam at lr 1e-4
 *     and the GPT-2 124M config printout (ujoy.net, section "训练过程").
 * The pages print no formulas; every layer below is the textbook definition of
 * GPT-2 (pre-LN blocks, tied LM head, tanh GELU), the plainest reading of
 * "matches the PyTorch reference" on the same page.
 *
 * Style: plain loops in source order, one output element per loop body, no
 * blocking and no fusion.  OpenMP only splits independent output rows or
 * columns between threads, so results do not depend on the thread count.
 *
 * Precision: `real` is float (the pages train in fp32); building with
 * -DORACLE_FP64 makes it double, for finite-difference gradient checks.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef ORACLE_FP64
typedef double real;
#define R_EXP exp
#define R_LOG log
#define R_SQRT sqrt
#define R_TANH tanh
#define R_POW pow
#else
typedef float real;
#define R_EXP expf
#define R_LOG logf
#define R_SQRT sqrtf
#define R_TANH tanhf
#define R_POW powf
#endif

#define EXPORT __attribute__((visibility("default")))

EXPORT int oracle_real_size(void) { return (int)sizeof(real); }

/* OpenMP threads for the following calls (timing runs only; results do
 * not depend on the count). */
#ifdef _OPENMP
#include <omp.h>
EXPORT void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
#else
EXPORT void oracle_set_threads(int n) { (void)n; }
#endif

/* ------------------------------------------------------------------------ */
/* Layer definitions                                                         */
/* ------------------------------------------------------------------------ */

/* Token + position embedding: out[b,t,:] = wte[tok[b,t],:] + wpe[t,:].
 * Every sequence in the batch starts at position 0.  wpe may be NULL (the
 * rotary model has no position table): then out = wte[tok]. */
EXPORT void oracle_encoder_forward(real* out, const int* tok, const real* wte,
                                   const real* wpe, int B, int T, int C) {
    for (int b = 0; b < B; b++) {
        for (int t = 0; t < T; t++) {
            real* o = out + ((size_t)b * T + t) * C;
            const real* we = wte + (size_t)tok[b * T + t] * C;
            for (int c = 0; c < C; c++)
                o[c] = wpe ? we[c] + wpe[(size_t)t * C + c] : we[c];
        }
    }
}

/* Gradient of the embedding: each position adds its output gradient into the
 * row of the token it read and into the row of its position. */
EXPORT void oracle_encoder_backward(real* dwte, real* dwpe, const real* dout,
                                    const int* tok, int B, int T, int C) {
    for (int b = 0; b < B; b++) {
        for (int t = 0; t < T; t++) {
            const real* d = dout + ((size_t)b * T + t) * C;
            real* dwe = dwte + (size_t)tok[b * T + t] * C;
            for (int c = 0; c < C; c++) {
                dwe[c] += d[c];
                if (dwpe) dwpe[(size_t)t * C + c] += d[c];
            }
        }
    }
}

/* LayerNorm over the last axis, eps 1e-5, biased variance, mean first and
 * variance second:  y = (x - mean) * rstd * w + b,  rstd = 1/sqrt(var + eps).
 * mean and rstd of each row are kept for the backward. */
EXPORT void oracle_layernorm_forward(real* out, real* mean, real* rstd,
                                     const real* inp, const real* w,
                                     const real* bias, int N, int C) {
    const real eps = (real)1e-5;
#pragma omp parallel for
    for (int n = 0; n < N; n++) {
        const real* x = inp + (size_t)n * C;
        real m = 0;
        for (int c = 0; c < C; c++) m += x[c];
        m = m / C;
        real v = 0;
        for (int c = 0; c < C; c++) {
            real d = x[c] - m;
            v += d * d;
        }
        v = v / C;
        real s = 1 / R_SQRT(v + eps);
        real* y = out + (size_t)n * C;
        for (int c = 0; c < C; c++) y[c] = (x[c] - m) * s * w[c] + bias[c];
        mean[n] = m;
        rstd[n] = s;
    }
}

/* LayerNorm backward.  With xhat = (x-mean)*rstd and g = dy*w:
 *   dx  += rstd * (g - mean(g) - xhat * mean(g*xhat))
 *   dw  += sum_rows dy*xhat,   db += sum_rows dy. */
EXPORT void oracle_layernorm_backward(real* dinp, real* dw, real* db,
                                      const real* dout, const real* inp,
                                      const real* w, const real* mean,
                                      const real* rstd, int N, int C) {
    for (int n = 0; n < N; n++) {
        const real* dy = dout + (size_t)n * C;
        const real* x = inp + (size_t)n * C;
        real* dx = dinp + (size_t)n * C;
        real m = mean[n], s = rstd[n];
        real g_mean = 0, gx_mean = 0;
        for (int c = 0; c < C; c++) {
            real xhat = (x[c] - m) * s;
            real g = dy[c] * w[c];
            g_mean += g;
            gx_mean += g * xhat;
        }
        g_mean = g_mean / C;
        gx_mean = gx_mean / C;
        for (int c = 0; c < C; c++) {
            real xhat = (x[c] - m) * s;
            real g = dy[c] * w[c];
            dx[c] += s * (g - g_mean - xhat * gx_mean);
            dw[c] += dy[c] * xhat;
            db[c] += dy[c];
        }
    }
}

/* Linear layer, weight stored (out, in) row-major:
 *   out[n,o] = bias[o] + sum_c inp[n,c] * w[o,c]     (bias may be NULL). */
EXPORT void oracle_matmul_forward(real* out, const real* inp, const real* w,
                                  const real* bias, int N, int C, int OC) {
#pragma omp parallel for collapse(2)
    for (int n = 0; n < N; n++) {
        for (int o = 0; o < OC; o++) {
            const real* x = inp + (size_t)n * C;
            const real* wr = w + (size_t)o * C;
            real acc = 0;
            for (int c = 0; c < C; c++) acc += x[c] * wr[c];
            out[(size_t)n * OC + o] = acc + (bias ? bias[o] : 0);
        }
    }
}

/* Linear layer backward:
 *   dinp[n,c] += sum_o dout[n,o] * w[o,c]
 *   dw[o,c]   += sum_n dout[n,o] * inp[n,c]
 *   db[o]     += sum_n dout[n,o]              (db may be NULL). */
EXPORT void oracle_matmul_backward(real* dinp, real* dw, real* db,
                                   const real* dout, const real* inp,
                                   const real* w, int N, int C, int OC) {
#pragma omp parallel for
    for (int n = 0; n < N; n++) {
        real* dx = dinp + (size_t)n * C;
        const real* dy = dout + (size_t)n * OC;
        for (int o = 0; o < OC; o++) {
            const real* wr = w + (size_t)o * C;
            real d = dy[o];
            for (int c = 0; c < C; c++) dx[c] += d * wr[c];
        }
    }
#pragma omp parallel for
    for (int o = 0; o < OC; o++) {
        real* dwr = dw + (size_t)o * C;
        for (int n = 0; n < N; n++) {
            const real* x = inp + (size_t)n * C;
            real d = dout[(size_t)n * OC + o];
            for (int c = 0; c < C; c++) dwr[c] += d * x[c];
        }
        if (db) {
            real s = 0;
            for (int n = 0; n < N; n++) s += dout[(size_t)n * OC + o];
            db[o] += s;
        }
    }
}

/* Causal multi-head self-attention.  qkv rows are [q | k | v], each C wide;
 * head h owns channels [h*hs, (h+1)*hs).  For query t and key t2 <= t:
 *   preatt[b,h,t,t2] = q_t . k_t2 / sqrt(hs)
 *   att[b,h,t,:]     = softmax over t2 <= t (row max subtracted), 0 above
 *   out[b,t,h-slice] = sum_t2 att[b,h,t,t2] * v_t2.
 * Positions t2 > t are stored as exactly 0 in both preatt and att.  No
 * attention crosses from one sequence of the batch to another. */
EXPORT void oracle_attention_forward(real* out, real* preatt, real* att,
                                     const real* qkv, int B, int T, int C,
                                     int NH) {
    const int hs = C / NH;
    const real scale = 1 / R_SQRT((real)hs);
#pragma omp parallel for collapse(3)
    for (int b = 0; b < B; b++) {
        for (int h = 0; h < NH; h++) {
            for (int t = 0; t < T; t++) {
                const real* q = qkv + ((size_t)b * T + t) * 3 * C + h * hs;
                real* pre = preatt + (((size_t)b * NH + h) * T + t) * T;
                real* a = att + (((size_t)b * NH + h) * T + t) * T;
                real maxv = -INFINITY;
                for (int t2 = 0; t2 <= t; t2++) {
                    const real* k = qkv + ((size_t)b * T + t2) * 3 * C + C + h * hs;
                    real s = 0;
                    for (int i = 0; i < hs; i++) s += q[i] * k[i];
                    s = s * scale;
                    pre[t2] = s;
                    if (s > maxv) maxv = s;
                }
                real sum = 0;
                for (int t2 = 0; t2 <= t; t2++) {
                    real e = R_EXP(pre[t2] - maxv);
                    a[t2] = e;
                    sum += e;
                }
                for (int t2 = 0; t2 <= t; t2++) a[t2] = a[t2] / sum;
                for (int t2 = t + 1; t2 < T; t2++) {
                    pre[t2] = 0;
                    a[t2] = 0;
                }
                real* o = out + ((size_t)b * T + t) * C + h * hs;
                for (int i = 0; i < hs; i++) {
                    real acc = 0;
                    for (int t2 = 0; t2 <= t; t2++) {
                        const real* v = qkv + ((size_t)b * T + t2) * 3 * C + 2 * C + h * hs;
                        acc += a[t2] * v[i];
                    }
                    o[i] = acc;
                }
            }
        }
    }
}

/* Attention backward through the stored softmax:
 *   datt[t2]   = dout_t . v_t2           dv_t2 += att[t2] * dout_t
 *   dpre[t2]   = att[t2] * (datt[t2] - sum_t3 att[t3]*datt[t3])
 *   dq_t      += sum_t2 dpre[t2] * k_t2 / sqrt(hs)
 *   dk_t2     += dpre[t2] * q_t / sqrt(hs). */
EXPORT void oracle_attention_backward(real* dqkv, real* dpreatt, real* datt,
                                      const real* dout, const real* qkv,
                                      const real* att, int B, int T, int C,
                                      int NH) {
    const int hs = C / NH;
    const real scale = 1 / R_SQRT((real)hs);
#pragma omp parallel for collapse(2)
    for (int b = 0; b < B; b++) {
        for (int h = 0; h < NH; h++) {
            for (int t = 0; t < T; t++) {
                const real* a = att + (((size_t)b * NH + h) * T + t) * T;
                real* da = datt + (((size_t)b * NH + h) * T + t) * T;
                real* dpre = dpreatt + (((size_t)b * NH + h) * T + t) * T;
                const real* dy = dout + ((size_t)b * T + t) * C + h * hs;
                const real* q = qkv + ((size_t)b * T + t) * 3 * C + h * hs;
                real* dq = dqkv + ((size_t)b * T + t) * 3 * C + h * hs;
                for (int t2 = 0; t2 <= t; t2++) {
                    const real* v = qkv + ((size_t)b * T + t2) * 3 * C + 2 * C + h * hs;
                    real* dv = dqkv + ((size_t)b * T + t2) * 3 * C + 2 * C + h * hs;
                    real s = 0;
                    for (int i = 0; i < hs; i++) {
                        s += dy[i] * v[i];
                        dv[i] += a[t2] * dy[i];
                    }
                    da[t2] += s;
                }
                real dot = 0;
                for (int t3 = 0; t3 <= t; t3++) dot += a[t3] * da[t3];
                for (int t2 = 0; t2 <= t; t2++) dpre[t2] += a[t2] * (da[t2] - dot);
                for (int t2 = 0; t2 <= t; t2++) {
                    const real* k = qkv + ((size_t)b * T + t2) * 3 * C + C + h * hs;
                    real* dk = dqkv + ((size_t)b * T + t2) * 3 * C + C + h * hs;
                    for (int i = 0; i < hs; i++) {
                        dq[i] += dpre[t2] * k[i] * scale;
                        dk[i] += dpre[t2] * q[i] * scale;
                    }
                }
            }
        }
    }
}

/* GELU, tanh form:  0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))). */
static real gelu_k0(void) { return (real)sqrt(2.0 / M_PI); }

EXPORT void oracle_gelu_forward(real* out, const real* inp, int64_t n) {
    const real k0 = gelu_k0(), k1 = (real)0.044715;
#pragma omp parallel for
    for (int64_t i = 0; i < n; i++) {
        real x = inp[i];
        out[i] = (real)0.5 * x * (1 + R_TANH(k0 * (x + k1 * x * x * x)));
    }
}

/* d/dx of the tanh GELU:
 *   0.5 (1 + tanh u) + 0.5 x (1 - tanh^2 u) sqrt(2/pi) (1 + 3*0.044715 x^2),
 *   u = sqrt(2/pi) (x + 0.044715 x^3);   dinp += dout * that. */
EXPORT void oracle_gelu_backward(real* dinp, const real* inp, const real* dout,
                                 int64_t n) {
    const real k0 = gelu_k0(), k1 = (real)0.044715;
#pragma omp parallel for
    for (int64_t i = 0; i < n; i++) {
        real x = inp[i];
        real u = k0 * (x + k1 * x * x * x);
        real th = R_TANH(u);
        real du = k0 * (1 + 3 * k1 * x * x);
        real g = (real)0.5 * (1 + th) + (real)0.5 * x * (1 - th * th) * du;
        dinp[i] += dout[i] * g;
    }
}

EXPORT void oracle_residual_forward(real* out, const real* a, const real* b,
                                    int64_t n) {
    for (int64_t i = 0; i < n; i++) out[i] = a[i] + b[i];
}

/* The gradient of a sum reaches both addends unchanged. */
EXPORT void oracle_residual_backward(real* da, real* db, const real* dout,
                                     int64_t n) {
    for (int64_t i = 0; i < n; i++) {
        da[i] += dout[i];
        db[i] += dout[i];
    }
}

/* Row softmax over the vocabulary, row maximum subtracted first. */
EXPORT void oracle_softmax_forward(real* probs, const real* logits, int N,
                                   int V) {
#pragma omp parallel for
    for (int n = 0; n < N; n++) {
        const real* z = logits + (size_t)n * V;
        real* p = probs + (size_t)n * V;
        real maxv = -INFINITY;
        for (int v = 0; v < V; v++)
            if (z[v] > maxv) maxv = z[v];
        real sum = 0;
        for (int v = 0; v < V; v++) {
            p[v] = R_EXP(z[v] - maxv);
            sum += p[v];
        }
        for (int v = 0; v < V; v++) p[v] = p[v] / sum;
    }
}

/* Per-position cross-entropy: loss[n] = -ln probs[n, target[n]]. */
EXPORT void oracle_crossentropy_forward(real* losses, const real* probs,
                                        const int* targets, int N, int V) {
    for (int n = 0; n < N; n++)
        losses[n] = -R_LOG(probs[(size_t)n * V + targets[n]]);
}

/* Softmax followed by cross-entropy, backward to the logits:
 *   dlogits[n,v] += (probs[n,v] - [v == target[n]]) * dloss[n]. */
EXPORT void oracle_crossentropy_softmax_backward(real* dlogits,
                                                 const real* dlosses,
                                                 const real* probs,
                                                 const int* targets, int N,
                                                 int V) {
#pragma omp parallel for
    for (int n = 0; n < N; n++) {
        real* dz = dlogits + (size_t)n * V;
        const real* p = probs + (size_t)n * V;
        for (int v = 0; v < V; v++) {
            real onehot = (v == targets[n]) ? 1 : 0;
            dz[v] += (p[v] - onehot) * dlosses[n];
        }
    }
}

/* AdamW (Adam with decoupled weight decay), one step, 1-based step count:
 *   m = b1 m + (1-b1) g;   v = b2 v + (1-b2) g^2
 *   mhat = m / (1 - b1^step);   vhat = v / (1 - b2^step)
 *   p -= lr * (mhat / (sqrt(vhat) + eps) + wd * p).
 * The pages run Adam at lr 1e-4 (ujoy.net, section "训练过程"); with wd = 0
 * this is exactly Adam. */
EXPORT void oracle_adamw(real* p, const real* g, real* m, real* v, int64_t n,
                         real lr, real b1, real b2, real eps, real wd,
                         int step) {
    real c1 = 1 - R_POW(b1, (real)step);
    real c2 = 1 - R_POW(b2, (real)step);
#pragma omp parallel for
    for (int64_t i = 0; i < n; i++) {
        m[i] = b1 * m[i] + (1 - b1) * g[i];
        v[i] = b2 * v[i] + (1 - b2) * g[i] * g[i];
        real mhat = m[i] / c1;
        real vhat = v[i] / c2;
        p[i] -= lr * (mhat / (R_SQRT(vhat) + eps) + wd * p[i]);
    }
}

/* Rotary position embedding (RoFormer, Su et al. 2021), the architectural
 * extension named by yinghuohong.cn (section "脚动完成每一个层前向/反向流传").
 * In place on the q and k slices of each qkv row (B*T rows of 3C): in every
 * head of size hs, the channel pair (2i, 2i+1) of the row at position t is
 * rotated by the angle t * 10000^(-2i/hs):
 *   x' = x cos a - y sin a,   y' = x sin a + y cos a.
 * Angles and their cosines are taken in double. */
static void rope_rotate(real* qkv, int B, int T, int C, int NH, double sign) {
    const int hs = C / NH;
    for (int b = 0; b < B; b++)
        for (int t = 0; t < T; t++) {
            real* row = qkv + ((size_t)b * T + t) * 3 * C;
            for (int part = 0; part < 2; part++)      /* q, then k */
                for (int h = 0; h < NH; h++)
                    for (int i = 0; i < hs / 2; i++) {
                        real* x = row + part * C + h * hs + 2 * i;
                        const double a = t * pow(10000.0, -2.0 * i / hs);
                        const double cs = cos(a), sn = sign * sin(a);
                        const double x0 = x[0], x1 = x[1];
                        x[0] = (real)(x0 * cs - x1 * sn);
                        x[1] = (real)(x0 * sn + x1 * cs);
                    }
        }
}

EXPORT void oracle_rope_forward(real* qkv, int B, int T, int C, int NH) {
    rope_rotate(qkv, B, T, C, NH, 1.0);
}

/* The rotation is orthogonal, so its backward is the inverse rotation of the
 * q and k gradients (the v gradient passes through). */
EXPORT void oracle_rope_backward(real* dqkv, int B, int T, int C, int NH) {
    rope_rotate(dqkv, B, T, C, NH, -1.0);
}

/* ------------------------------------------------------------------------ */
/* Model: arenas and the chained step                                        */
/* ------------------------------------------------------------------------ */

typedef struct {
    int max_seq_len, vocab_size, num_layers, num_heads, channels;
    int rope; /* 1: rotary position embedding instead of the wpe table */
} OracleConfig;

enum { NPARAM = 16, NACT = 23 };

/* Parameter tensors in arena order; per-layer tensors are stacked over L.
 * Linear weights are (out, in). */
EXPORT int64_t oracle_param_sizes(const OracleConfig* cfg, int64_t* sizes) {
    int64_t L = cfg->num_layers, C = cfg->channels, V = cfg->vocab_size;
    int64_t maxT = cfg->max_seq_len;
    int64_t s[NPARAM] = {
        V * C,         /* wte      */
        cfg->rope ? 0 : maxT * C, /* wpe (none in the rotary model) */
        L * C,         /* ln1w     */
        L * C,         /* ln1b     */
        L * 3 * C * C, /* qkvw     */
        L * 3 * C,     /* qkvb     */
        L * C * C,     /* attprojw */
        L * C,         /* attprojb */
        L * C,         /* ln2w     */
        L * C,         /* ln2b     */
        L * 4 * C * C, /* fcw      */
        L * 4 * C,     /* fcb      */
        L * C * 4 * C, /* fcprojw  */
        L * C,         /* fcprojb  */
        C,             /* lnfw     */
        C,             /* lnfb     */
    };
    int64_t total = 0;
    for (int i = 0; i < NPARAM; i++) {
        if (sizes) sizes[i] = s[i];
        total += s[i];
    }
    return total;
}

/* Every activation the backward reads, fully materialized (attention
 * scores included), in arena order. */
EXPORT int64_t oracle_act_sizes(const OracleConfig* cfg, int B, int T,
                                int64_t* sizes) {
    int64_t L = cfg->num_layers, C = cfg->channels, V = cfg->vocab_size;
    int64_t NH = cfg->num_heads, BT = (int64_t)B * T;
    int64_t s[NACT] = {
        BT * C,              /* encoded   */
        L * BT * C,          /* ln1       */
        L * BT,              /* ln1_mean  */
        L * BT,              /* ln1_rstd  */
        L * BT * 3 * C,      /* qkv       */
        L * BT * C,          /* atty      */
        L * B * NH * T * T,  /* preatt    */
        L * B * NH * T * T,  /* att       */
        L * BT * C,          /* attproj   */
        L * BT * C,          /* residual2 */
        L * BT * C,          /* ln2       */
        L * BT,              /* ln2_mean  */
        L * BT,              /* ln2_rstd  */
        L * BT * 4 * C,      /* fch       */
        L * BT * 4 * C,      /* fch_gelu  */
        L * BT * C,          /* fcproj    */
        L * BT * C,          /* residual3 */
        BT * C,              /* lnf       */
        BT,                  /* lnf_mean  */
        BT,                  /* lnf_rstd  */
        BT * V,              /* logits    */
        BT * V,              /* probs     */
        BT,                  /* losses    */
    };
    int64_t total = 0;
    for (int i = 0; i < NACT; i++) {
        if (sizes) sizes[i] = s[i];
        total += s[i];
    }
    return total;
}

typedef struct {
    OracleConfig cfg;
    int B, T;
    int64_t param_sizes[NPARAM], act_sizes[NACT];
    int64_t num_params, num_acts;
    real *params, *grads, *m, *v;  /* four parameter-shaped arenas */
    real *acts, *dacts;             /* activations and their gradients */
    real* p[NPARAM];                /* tensor views into params */
    real* g[NPARAM];                /* tensor views into grads */
    real* a[NACT];                  /* tensor views into acts */
    real* da[NACT];                 /* tensor views into dacts */
    int* tokens;
    int* targets;
    int have_targets;
    double mean_loss;
} OracleModel;

enum {
    P_WTE, P_WPE, P_LN1W, P_LN1B, P_QKVW, P_QKVB, P_ATTPROJW, P_ATTPROJB,
    P_LN2W, P_LN2B, P_FCW, P_FCB, P_FCPROJW, P_FCPROJB, P_LNFW, P_LNFB
};
enum {
    A_ENCODED, A_LN1, A_LN1_MEAN, A_LN1_RSTD, A_QKV, A_ATTY, A_PREATT, A_ATT,
    A_ATTPROJ, A_RESIDUAL2, A_LN2, A_LN2_MEAN, A_LN2_RSTD, A_FCH, A_FCH_GELU,
    A_FCPROJ, A_RESIDUAL3, A_LNF, A_LNF_MEAN, A_LNF_RSTD, A_LOGITS, A_PROBS,
    A_LOSSES
};

static void carve(real* base, const int64_t* sizes, int n, real** views) {
    int64_t off = 0;
    for (int i = 0; i < n; i++) {
        views[i] = base + off;
        off += sizes[i];
    }
}

EXPORT void oracle_destroy(OracleModel* M);

/* Allocates every arena once; returns NULL on a bad config or no memory. */
EXPORT OracleModel* oracle_create(const OracleConfig* cfg, int B, int T) {
    if (cfg->num_heads <= 0 || cfg->channels % cfg->num_heads != 0) return NULL;
    if (B <= 0 || T <= 0 || T > cfg->max_seq_len) return NULL;
    OracleModel* M = (OracleModel*)calloc(1, sizeof(OracleModel));
    if (!M) return NULL;
    M->cfg = *cfg;
    M->B = B;
    M->T = T;
    M->num_params = oracle_param_sizes(cfg, M->param_sizes);
    M->num_acts = oracle_act_sizes(cfg, B, T, M->act_sizes);
    size_t pb = (size_t)M->num_params * sizeof(real);
    size_t ab = (size_t)M->num_acts * sizeof(real);
    M->params = (real*)calloc(1, pb);
    M->grads = (real*)calloc(1, pb);
    M->m = (real*)calloc(1, pb);
    M->v = (real*)calloc(1, pb);
    M->acts = (real*)calloc(1, ab);
    M->dacts = (real*)calloc(1, ab);
    M->tokens = (int*)calloc((size_t)B * T, sizeof(int));
    M->targets = (int*)calloc((size_t)B * T, sizeof(int));
    if (!M->params || !M->grads || !M->m || !M->v || !M->acts || !M->dacts ||
        !M->tokens || !M->targets) {
        oracle_destroy(M);
        return NULL;
    }
    carve(M->params, M->param_sizes, NPARAM, M->p);
    carve(M->grads, M->param_sizes, NPARAM, M->g);
    carve(M->acts, M->act_sizes, NACT, M->a);
    carve(M->dacts, M->act_sizes, NACT, M->da);
    return M;
}

EXPORT void oracle_destroy(OracleModel* M) {
    if (!M) return;
    free(M->params);
    free(M->grads);
    free(M->m);
    free(M->v);
    free(M->acts);
    free(M->dacts);
    free(M->tokens);
    free(M->targets);
    free(M);
}

EXPORT int64_t oracle_num_params(const OracleModel* M) { return M->num_params; }
EXPORT int64_t oracle_num_acts(const OracleModel* M) { return M->num_acts; }
EXPORT real* oracle_params(OracleModel* M) { return M->params; }
EXPORT real* oracle_grads(OracleModel* M) { return M->grads; }
EXPORT real* oracle_adam_m(OracleModel* M) { return M->m; }
EXPORT real* oracle_adam_v(OracleModel* M) { return M->v; }
EXPORT real* oracle_acts(OracleModel* M) { return M->acts; }
EXPORT real* oracle_act_grads(OracleModel* M) { return M->dacts; }

/* Forward pass.  targets may be NULL (then no loss; returns NaN).  Returns
 * the mean over B*T positions of the per-position loss, summed in double. */
EXPORT double oracle_forward(OracleModel* M, const int* tokens,
                             const int* targets) {
    const int B = M->B, T = M->T, L = M->cfg.num_layers, C = M->cfg.channels;
    const int NH = M->cfg.num_heads, V = M->cfg.vocab_size;
    const int BT = B * T;
    const int64_t BTC = (int64_t)BT * C;
    const int64_t att_sz = (int64_t)B * NH * T * T;
    real** p = M->p;
    real** a = M->a;
    memcpy(M->tokens, tokens, sizeof(int) * BT);
    M->have_targets = targets != NULL;
    if (targets) memcpy(M->targets, targets, sizeof(int) * BT);

    oracle_encoder_forward(a[A_ENCODED], tokens, p[P_WTE], M->cfg.rope ? NULL : p[P_WPE],
                           B, T, C);
    for (int l = 0; l < L; l++) {
        const real* resid = l == 0 ? a[A_ENCODED] : a[A_RESIDUAL3] + (l - 1) * BTC;
        real* ln1 = a[A_LN1] + l * BTC;
        real* ln1_mean = a[A_LN1_MEAN] + (int64_t)l * BT;
        real* ln1_rstd = a[A_LN1_RSTD] + (int64_t)l * BT;
        real* qkv = a[A_QKV] + l * 3 * BTC;
        real* atty = a[A_ATTY] + l * BTC;
        real* preatt = a[A_PREATT] + l * att_sz;
        real* att = a[A_ATT] + l * att_sz;
        real* attproj = a[A_ATTPROJ] + l * BTC;
        real* resid2 = a[A_RESIDUAL2] + l * BTC;
        real* ln2 = a[A_LN2] + l * BTC;
        real* ln2_mean = a[A_LN2_MEAN] + (int64_t)l * BT;
        real* ln2_rstd = a[A_LN2_RSTD] + (int64_t)l * BT;
        real* fch = a[A_FCH] + l * 4 * BTC;
        real* fch_gelu = a[A_FCH_GELU] + l * 4 * BTC;
        real* fcproj = a[A_FCPROJ] + l * BTC;
        real* resid3 = a[A_RESIDUAL3] + l * BTC;

        oracle_layernorm_forward(ln1, ln1_mean, ln1_rstd, resid,
                                 p[P_LN1W] + l * C, p[P_LN1B] + l * C, BT, C);
        oracle_matmul_forward(qkv, ln1, p[P_QKVW] + (int64_t)l * 3 * C * C,
                              p[P_QKVB] + l * 3 * C, BT, C, 3 * C);
        if (M->cfg.rope) oracle_rope_forward(qkv, B, T, C, NH);
        oracle_attention_forward(atty, preatt, att, qkv, B, T, C, NH);
        oracle_matmul_forward(attproj, atty, p[P_ATTPROJW] + (int64_t)l * C * C,
                              p[P_ATTPROJB] + l * C, BT, C, C);
        oracle_residual_forward(resid2, resid, attproj, BTC);
        oracle_layernorm_forward(ln2, ln2_mean, ln2_rstd, resid2,
                                 p[P_LN2W] + l * C, p[P_LN2B] + l * C, BT, C);
        oracle_matmul_forward(fch, ln2, p[P_FCW] + (int64_t)l * 4 * C * C,
                              p[P_FCB] + l * 4 * C, BT, C, 4 * C);
        oracle_gelu_forward(fch_gelu, fch, 4 * BTC);
        oracle_matmul_forward(fcproj, fch_gelu,
                              p[P_FCPROJW] + (int64_t)l * C * 4 * C,
                              p[P_FCPROJB] + l * C, BT, 4 * C, C);
        oracle_residual_forward(resid3, resid2, fcproj, BTC);
    }
    const real* last = a[A_RESIDUAL3] + (L - 1) * BTC;
    oracle_layernorm_forward(a[A_LNF], a[A_LNF_MEAN], a[A_LNF_RSTD], last,
                             p[P_LNFW], p[P_LNFB], BT, C);
    /* LM head shares the token embedding matrix (V, C); it has no bias. */
    oracle_matmul_forward(a[A_LOGITS], a[A_LNF], p[P_WTE], NULL, BT, C, V);
    oracle_softmax_forward(a[A_PROBS], a[A_LOGITS], BT, V);
    if (!targets) {
        M->mean_loss = NAN;
        return M->mean_loss;
    }
    oracle_crossentropy_forward(a[A_LOSSES], a[A_PROBS], targets, BT, V);
    double sum = 0;
    for (int i = 0; i < BT; i++) sum += (double)a[A_LOSSES][i];
    M->mean_loss = sum / BT;
    return M->mean_loss;
}

/* Dynamic loss scaling for the fp16 model, one update: the reading taken
 * for the pages' "fp16" extension (yinghuohong.cn, section
 * "脚动完成每一个层前向/反向流传") is the schedule of Micikevicius et al.
 * (2018).  A step whose scaled gradients hold an inf or NaN is not applied
 * and halves the scale (not below min_scale) and restarts the count of
 * clean steps; a clean step is applied, and the interval-th clean step in a
 * row doubles the scale.  Returns 1 if the update is applied. */
EXPORT int oracle_loss_scale_step(double* scale, int* good, int found_inf, int interval,
                                  double min_scale) {
    if (found_inf) {
        *scale = *scale / 2 < min_scale ? min_scale : *scale / 2;
        *good = 0;
        return 0;
    }
    *good += 1;
    if (*good >= interval) {
        *scale *= 2;
        *good = 0;
    }
    return 1;
}

/* One draw from a probability row by the inverse CDF: the smallest v with
 * coin * sum_u probs[u] < sum_{u <= v} probs[u] (sums in double, in index
 * order), or V - 1 if rounding leaves none.  The pages show the trainer
 * sampling text from the model after training (ujoy.net, section
 * "训练过程": the "generated:" line); drawing from the softmax
 * probabilities with a uniform coin is the plainest reading. */
EXPORT int oracle_sample(const real* probs, int V, double coin) {
    double total = 0;
    for (int v = 0; v < V; v++) total += (double)probs[v];
    const double target = coin * total;
    double cum = 0;
    for (int v = 0; v < V; v++) {
        cum += (double)probs[v];
        if (target < cum) return v;
    }
    return V - 1;
}

/* Generation for a B = 1 model: tokens[0 .. prompt_len) is the prompt; for
 * t = prompt_len .. n-1, run the forward over all T positions (tokens at
 * positions >= t do not reach position t-1 under the causal mask) and set
 * tokens[t] = oracle_sample(probs at position t-1, coins[t - prompt_len]).
 * tokens has M->T entries.  Returns 0, or -1 on a bad argument. */
EXPORT int oracle_generate(OracleModel* M, int* tokens, int prompt_len, int n,
                           const double* coins) {
    const int V = M->cfg.vocab_size;
    if (M->B != 1 || prompt_len < 1 || n < prompt_len || n > M->T) return -1;
    for (int t = prompt_len; t < n; t++) {
        oracle_forward(M, tokens, NULL);
        const real* probs = M->a[A_PROBS] + (int64_t)(t - 1) * V;
        tokens[t] = oracle_sample(probs, V, coins[t - prompt_len]);
    }
    return 0;
}

EXPORT void oracle_zero_grad(OracleModel* M) {
    memset(M->grads, 0, (size_t)M->num_params * sizeof(real));
}

/* Backward pass of the mean loss, in exact reverse order of the forward.
 * Parameter gradients accumulate (+=); activation gradients are cleared
 * first because they are scratch for this one pass.  Returns 0, or -1 if the
 * last forward had no targets. */
EXPORT int oracle_backward(OracleModel* M) {
    if (!M->have_targets) return -1;
    const int B = M->B, T = M->T, L = M->cfg.num_layers, C = M->cfg.channels;
    const int NH = M->cfg.num_heads, V = M->cfg.vocab_size;
    const int BT = B * T;
    const int64_t BTC = (int64_t)BT * C;
    const int64_t att_sz = (int64_t)B * NH * T * T;
    real** p = M->p;
    real** g = M->g;
    real** a = M->a;
    real** da = M->da;
    memset(M->dacts, 0, (size_t)M->num_acts * sizeof(real));

    /* d(mean loss)/d(loss_n) = 1/(B*T) */
    for (int i = 0; i < BT; i++) da[A_LOSSES][i] = (real)1 / BT;
    oracle_crossentropy_softmax_backward(da[A_LOGITS], da[A_LOSSES], a[A_PROBS],
                                         M->targets, BT, V);
    oracle_matmul_backward(da[A_LNF], g[P_WTE], NULL, da[A_LOGITS], a[A_LNF],
                           p[P_WTE], BT, C, V);
    const real* last = a[A_RESIDUAL3] + (L - 1) * BTC;
    real* dlast = da[A_RESIDUAL3] + (L - 1) * BTC;
    oracle_layernorm_backward(dlast, g[P_LNFW], g[P_LNFB], da[A_LNF], last,
                              p[P_LNFW], a[A_LNF_MEAN], a[A_LNF_RSTD], BT, C);

    for (int l = L - 1; l >= 0; l--) {
        const real* resid = l == 0 ? a[A_ENCODED] : a[A_RESIDUAL3] + (l - 1) * BTC;
        real* dresid = l == 0 ? da[A_ENCODED] : da[A_RESIDUAL3] + (l - 1) * BTC;
        const real* ln1 = a[A_LN1] + l * BTC;
        const real* ln1_mean = a[A_LN1_MEAN] + (int64_t)l * BT;
        const real* ln1_rstd = a[A_LN1_RSTD] + (int64_t)l * BT;
        const real* qkv = a[A_QKV] + l * 3 * BTC;
        const real* atty = a[A_ATTY] + l * BTC;
        const real* att = a[A_ATT] + l * att_sz;
        const real* resid2 = a[A_RESIDUAL2] + l * BTC;
        const real* ln2 = a[A_LN2] + l * BTC;
        const real* ln2_mean = a[A_LN2_MEAN] + (int64_t)l * BT;
        const real* ln2_rstd = a[A_LN2_RSTD] + (int64_t)l * BT;
        const real* fch = a[A_FCH] + l * 4 * BTC;
        const real* fch_gelu = a[A_FCH_GELU] + l * 4 * BTC;

        real* dln1 = da[A_LN1] + l * BTC;
        real* dqkv = da[A_QKV] + l * 3 * BTC;
        real* datty = da[A_ATTY] + l * BTC;
        real* dpreatt = da[A_PREATT] + l * att_sz;
        real* datt = da[A_ATT] + l * att_sz;
        real* dattproj = da[A_ATTPROJ] + l * BTC;
        real* dresid2 = da[A_RESIDUAL2] + l * BTC;
        real* dln2 = da[A_LN2] + l * BTC;
        real* dfch = da[A_FCH] + l * 4 * BTC;
        real* dfch_gelu = da[A_FCH_GELU] + l * 4 * BTC;
        real* dfcproj = da[A_FCPROJ] + l * BTC;
        real* dresid3 = da[A_RESIDUAL3] + l * BTC;

        oracle_residual_backward(dresid2, dfcproj, dresid3, BTC);
        oracle_matmul_backward(dfch_gelu, g[P_FCPROJW] + (int64_t)l * C * 4 * C,
                               g[P_FCPROJB] + l * C, dfcproj, fch_gelu,
                               p[P_FCPROJW] + (int64_t)l * C * 4 * C, BT, 4 * C, C);
        oracle_gelu_backward(dfch, fch, dfch_gelu, 4 * BTC);
        oracle_matmul_backward(dln2, g[P_FCW] + (int64_t)l * 4 * C * C,
                               g[P_FCB] + l * 4 * C, dfch, ln2,
                               p[P_FCW] + (int64_t)l * 4 * C * C, BT, C, 4 * C);
        oracle_layernorm_backward(dresid2, g[P_LN2W] + l * C, g[P_LN2B] + l * C,
                                  dln2, resid2, p[P_LN2W] + l * C, ln2_mean,
                                  ln2_rstd, BT, C);
        oracle_residual_backward(dresid, dattproj, dresid2, BTC);
        oracle_matmul_backward(datty, g[P_ATTPROJW] + (int64_t)l * C * C,
                               g[P_ATTPROJB] + l * C, dattproj, atty,
                               p[P_ATTPROJW] + (int64_t)l * C * C, BT, C, C);
        oracle_attention_backward(dqkv, dpreatt, datt, datty, qkv, att, B, T, C,
                                  NH);
        if (M->cfg.rope) oracle_rope_backward(dqkv, B, T, C, NH);
        oracle_matmul_backward(dln1, g[P_QKVW] + (int64_t)l * 3 * C * C,
                               g[P_QKVB] + l * 3 * C, dqkv, ln1,
                               p[P_QKVW] + (int64_t)l * 3 * C * C, BT, C, 3 * C);
        oracle_layernorm_backward(dresid, g[P_LN1W] + l * C, g[P_LN1B] + l * C,
                                  dln1, resid, p[P_LN1W] + l * C, ln1_mean,
                                  ln1_rstd, BT, C);
    }
    oracle_encoder_backward(g[P_WTE], M->cfg.rope ? NULL : g[P_WPE], da[A_ENCODED], M->tokens,
                            B, T, C);
    return 0;
}

EXPORT void oracle_update(OracleModel* M, double lr, double b1, double b2,
                          double eps, double wd, int step) {
    oracle_adamw(M->params, M->grads, M->m, M->v, M->num_params, (real)lr,
                 (real)b1, (real)b2, (real)eps, (real)wd, step);
}
