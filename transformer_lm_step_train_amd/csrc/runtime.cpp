// Host runtime behind the C ABI (include/gpt2.h): one device allocation laid
// out by host.cpp, and the launch sequence of one training step on one HIP
// stream.
//
// The arenas follow the llm.c design of allocating everything once as flat
// 1-D memory and pointing every tensor into it (yinghuohong.cn article
// "OpenAI创始大神手搓千行C代码训练GPT", section "脚动完成每一个层前向/反向流传";
// ujoy.net article "徒手用 1000 行 C 语言实现", section "用C语言实现LLM").  The
// activation arena differs from a CPU layout: attention keeps one
// log-sum-exp per query row instead of the (T, T) probabilities, the residual
// adds and GELU are produced by the matmul epilogues, and the LM-head logits
// are overwritten in place by their gradient.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cerrno>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/gpt2.h"
#include "dtype.h"
#include "host.h"
#include "kernels.h"

namespace gk {
LaunchEvents& launch_events() {
    static thread_local LaunchEvents e;
    return e;
}
}  // namespace gk

// Compute units the split plans are made for: the current device's.
int gh::host_cu_count() { return gk::device_cu_count(); }

namespace {

// config checks, the arena layout, parameter indices P_*, error messages
using namespace gh;

constexpr int kEventPool = 4096;

struct Prof {
    bool on = false;
    int mask = 0;  // classes whose launches carry timing events
    std::vector<hipEvent_t> ev;
    struct Rec {
        int kc;
        double flops, bytes;
    };
    std::vector<Rec> recs;
    double ms[GPT2_KC_COUNT] = {}, fl[GPT2_KC_COUNT] = {}, by[GPT2_KC_COUNT] = {};
    int64_t n[GPT2_KC_COUNT] = {};
};

}  // namespace

struct gpt2_model {
    gpt2_config cfg;
    Layout lay;
    hipStream_t stream = nullptr;
    gpt2_allocator alloc{};
    bool custom_alloc = false;
    char* base = nullptr;
    int32_t* h_stage = nullptr;  // pinned: tokens then targets
    float* h_scal = nullptr;     // pinned: loss, flag
    hipEvent_t stage_done = nullptr;
    bool stage_pending = false;
    int B = 0, T = 0;
    bool have_fwd = false, have_targets = false, have_loss = false;
    bool logits_valid = false;  // last forward had no targets: logits intact
    Prof prof;

    template <class X>
    X* at(size_t off) const {
        return reinterpret_cast<X*>(base + off);
    }
    float* P(int i) const { return at<float>(lay.params) + lay.poff[i]; }
    // weight operand of the matmuls: the fp32 master, or its 16-bit copy
    const void* W(int i) const {
        return lay.half ? (const void*)(at<uint16_t>(lay.shadow) + lay.poff[i]) : (const void*)P(i);
    }
    // activation buffer at byte offset `off`, element `idx`
    char* A(size_t off, size_t idx = 0) const { return base + off + idx * lay.es; }
    float* G(int i) const { return at<float>(lay.grads) + lay.poff[i]; }
    int* flag() const { return at<int>(lay.scalars + 4); }
    int32_t* drawn() const { return at<int32_t>(lay.scalars + 8); }
    // dynamic loss scaling of the fp16 model: scale, clean steps in a row,
    // non-finite gradient found this step, last update skipped
    float* lscale() const { return at<float>(lay.scalars + 12); }
    int* lgood() const { return at<int>(lay.scalars + 16); }
    int* lfound() const { return at<int>(lay.scalars + 20); }
    int* lskipped() const { return at<int>(lay.scalars + 24); }
    int growth_interval = 2000;
    float* dloss() const { return at<float>(lay.scalars); }
};

namespace {

// ---- per-launch timing ------------------------------------------------------

void prof_flush(gpt2_model* md) {
    Prof& p = md->prof;
    if (p.recs.empty()) return;
    hipEventSynchronize(p.ev[2 * p.recs.size() - 1]);
    for (size_t i = 0; i < p.recs.size(); i++) {
        float ms = 0.f;
        hipEventElapsedTime(&ms, p.ev[2 * i], p.ev[2 * i + 1]);
        const int kc = p.recs[i].kc;
        p.ms[kc] += ms;
        p.n[kc] += 1;
        p.fl[kc] += p.recs[i].flops;
        p.by[kc] += p.recs[i].bytes;
    }
    p.recs.clear();
}

// Times the launches of one library call: the first kernel's dispatch
// carries the start event and the last one's the stop event (a call that
// launches nothing records nothing).
struct Scope {
    gpt2_model* md;
    int kc;
    double flops, bytes;
    bool on, timed;
    Scope(gpt2_model* m, int k, double f, double b) : md(m), kc(k), flops(f), bytes(b) {
        on = md->prof.on;
        timed = on && ((md->prof.mask >> kc) & 1);
        gk::LaunchEvents& le = gk::launch_events();
        le = gk::LaunchEvents{};
        if (!timed) return;
        if (2 * (md->prof.recs.size() + 1) > md->prof.ev.size()) prof_flush(md);
        le.start = md->prof.ev[2 * md->prof.recs.size()];
        le.stop = md->prof.ev[2 * md->prof.recs.size() + 1];
    }
    ~Scope() {
        if (!on) return;
        Prof& p = md->prof;
        gk::LaunchEvents& le = gk::launch_events();
        if (timed) {
            if (le.launched > 0) p.recs.push_back({kc, flops, bytes});
        } else if (le.launched > 0) {  // counted, not timed
            p.n[kc] += 1;
            p.fl[kc] += flops;
            p.by[kc] += bytes;
        }
        le = gk::LaunchEvents{};
    }
};

#define LAUNCH(md, kc, flops, bytes, call)                                                \
    do {                                                                                  \
        hipError_t e_;                                                                    \
        {                                                                                 \
            Scope sc_(md, kc, (double)(flops), (double)(bytes));                          \
            e_ = (call);                                                                  \
        }                                                                                 \
        if (e_ != hipSuccess)                                                             \
            return fail(GPT2_EDEVICE, "%s: %s", #call, hipGetErrorString(e_));            \
    } while (0)

int hip_check(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(GPT2_EDEVICE, "%s: %s", what, hipGetErrorString(e));
    return GPT2_OK;
}

// One matmul of the step, independent of the precision: activations and
// weights as untyped pointers (fp32, or bf16 in the mixed-precision model),
// gradients (EPI_ACCUM outputs), biases and everything else fp32.
struct Mm {
    int op, epi, M, N, K;
    const void* A;
    int64_t lda;
    const void* B;
    int64_t ldb;
    void* C;
    int64_t ldc;
    const float* bias = nullptr;
    const void* aux = nullptr;
    int64_t ldaux = 0;
    void* out2 = nullptr;
    float* colsum = nullptr;  // EPI_GELU_BWD: per-64-row column sums of C
};

Mm mm(int op, int epi, int M, int N, int K, const void* A, int64_t lda, const void* B,
      int64_t ldb, void* C, int64_t ldc) {
    Mm x;
    x.op = op;
    x.epi = epi;
    x.M = M;
    x.N = N;
    x.K = K;
    x.A = A;
    x.lda = lda;
    x.B = B;
    x.ldb = ldb;
    x.C = C;
    x.ldc = ldc;
    return x;
}

int run_gemm(gpt2_model* md, const Mm& x) {
    const double flops = 2.0 * x.M * x.N * (double)x.K;
    const double es = (double)md->lay.es;
    const double bytes = es * ((double)x.M * x.K + (double)x.K * x.N) +
                         (x.epi == gk::EPI_ACCUM ? 8.0 : es) * (double)x.M * x.N;
    float* ws = md->at<float>(md->lay.gemm_ws);
    const size_t wsb = md->lay.gemm_ws_bytes;
    if (md->lay.half) {
        gk::GemmArgsH a{};
        a.f16 = md->lay.dt == DT_F16;
        a.op = x.op;
        a.epi = x.epi;
        a.M = x.M;
        a.N = x.N;
        a.K = x.K;
        a.A = (const uint16_t*)x.A;
        a.lda = x.lda;
        a.B = (const uint16_t*)x.B;
        a.ldb = x.ldb;
        a.C = x.C;
        a.ldc = x.ldc;
        a.out_f32 = 0;
        a.bias = x.bias;
        a.aux = (const uint16_t*)x.aux;
        a.ldaux = x.ldaux;
        a.out2 = (uint16_t*)x.out2;
        a.colsum = x.colsum;
        LAUNCH(md, GPT2_KC_GEMM, flops, bytes, gk::gemm_bf16(md->stream, a, ws, wsb));
    } else {
        gk::GemmArgs a{};
        a.op = x.op;
        a.epi = x.epi;
        a.M = x.M;
        a.N = x.N;
        a.K = x.K;
        a.A = (const float*)x.A;
        a.lda = x.lda;
        a.B = (const float*)x.B;
        a.ldb = x.ldb;
        a.C = (float*)x.C;
        a.ldc = x.ldc;
        a.bias = x.bias;
        a.aux = (const float*)x.aux;
        a.ldaux = x.ldaux;
        a.out2 = (float*)x.out2;
        a.colsum = x.colsum;
        LAUNCH(md, GPT2_KC_GEMM, flops, bytes, gk::gemm(md->stream, a, ws, wsb));
    }
    return GPT2_OK;
}

#define TRY(x)                        \
    do {                              \
        int r_ = (x);                 \
        if (r_ != GPT2_OK) return r_; \
    } while (0)

// ---- forward ---------------------------------------------------------------

// What a forward computes after the logits: nothing (inference: the logits
// stay for sampling), the loss with the logits' gradient written over them
// and the embedding keys sorted for the backward (training), or the loss
// alone (evaluation: the logits stay, no backward state).
enum FwdMode { FWD_INFER = 0, FWD_TRAIN = 1, FWD_EVAL = 2 };

// Rows before r0 (only with B = 1 and no targets) are taken as already
// computed for the same leading tokens by an earlier forward: every row-wise
// kernel starts at row r0, and attention reads the keys and values of all T
// rows from the qkv activations (a key/value cache) but computes only the
// outputs from r0's query block on.  Each row's arithmetic is the same as in
// a whole forward, so the results are identical.
int forward_impl(gpt2_model* md, const int32_t* tok, const int32_t* tgt, int B, int T,
                 int mode, int r0 = 0) {
    const Layout& y = md->lay;
    const int L = y.L, C = y.C, NH = y.NH, V = y.V;
    const int M = B * T - r0;  // rows computed
    const size_t ro = (size_t)r0;
    const int h = y.dt;
    const size_t MC = (size_t)y.M * C;  // per-layer capacity stride, elements
    const double es = (double)y.es;
    hipStream_t s = md->stream;
    void* enc = md->A(y.encoded, ro * C);
    const int hsz = C / NH;

    LAUNCH(md, GPT2_KC_OTHER, 0, 4.0, gk::fill_zero(s, (float*)md->flag(), 1));
    LAUNCH(md, GPT2_KC_OTHER, 0, 8.0 * M * C + es * M * C + 4.0 * M,
           gk::encoder_forward(s, enc, tok + ro, md->P(P_WTE),
                               y.rope ? nullptr : md->P(P_WPE) + ro * C, B, T - r0, C, V,
                               md->flag(), h));
    for (int l = 0; l < L; l++) {
        const void* resid = l == 0 ? enc : (const void*)md->A(y.res3, (l - 1) * MC + ro * C);
        void* ln1 = md->A(y.ln1, l * MC + ro * C);
        float* ln1m = md->at<float>(y.ln1_mean) + (size_t)l * y.M + ro;
        float* ln1r = md->at<float>(y.ln1_rstd) + (size_t)l * y.M + ro;
        void* qkv_l = md->A(y.qkv, l * 3 * MC);
        void* qkv = md->A(y.qkv, l * 3 * MC + ro * 3 * C);
        void* atty_l = md->A(y.atty, l * MC);
        void* atty = md->A(y.atty, l * MC + ro * C);
        float* lse = md->at<float>(y.lse) + (size_t)l * y.M * NH;
        void* res2 = md->A(y.res2, l * MC + ro * C);
        void* ln2 = md->A(y.ln2, l * MC + ro * C);
        float* ln2m = md->at<float>(y.ln2_mean) + (size_t)l * y.M + ro;
        float* ln2r = md->at<float>(y.ln2_rstd) + (size_t)l * y.M + ro;
        void* fch = md->A(y.fch, l * 4 * MC + ro * 4 * C);
        void* fchg = md->A(y.fch_gelu, l * 4 * MC + ro * 4 * C);
        void* res3 = md->A(y.res3, l * MC + ro * C);

        LAUNCH(md, GPT2_KC_LAYERNORM, 0, es * 2.0 * M * C + 8.0 * M,
               gk::layernorm_forward(s, ln1, ln1m, ln1r, resid, md->P(P_LN1W) + l * C,
                                     md->P(P_LN1B) + l * C, M, C, h));
        Mm a = mm(gk::GEMM_NT, gk::EPI_STORE, M, 3 * C, C, ln1, C,
                  (const char*)md->W(P_QKVW) + (size_t)l * 3 * C * C * y.es, C, qkv, 3 * C);
        a.bias = md->P(P_QKVB) + l * 3 * C;
        TRY(run_gemm(md, a));
        if (y.rope)
            LAUNCH(md, GPT2_KC_OTHER, 0, es * 4.0 * M * C,
                   gk::rope_apply(s, qkv, md->at<float>(y.rope_cs) + ro * hsz, B, T - r0, C, NH,
                                  1, h));
        {
            const double hs = hsz;
            const double rows = (double)T * (T + 1) / 2.0 - (double)r0 * (r0 + 1) / 2.0;
            const double flops = 4.0 * B * NH * hs * rows;
            LAUNCH(md, GPT2_KC_ATTENTION, flops, es * 4.0 * M * C + 4.0 * M * NH,
                   gk::attention_forward(s, atty_l, lse, qkv_l, B, T, C, NH, h, r0));
        }
        a = mm(gk::GEMM_NT, gk::EPI_RESID, M, C, C, atty, C,
               (const char*)md->W(P_ATTPROJW) + (size_t)l * C * C * y.es, C, res2, C);
        a.bias = md->P(P_ATTPROJB) + l * C;
        a.aux = resid;
        a.ldaux = C;
        TRY(run_gemm(md, a));
        LAUNCH(md, GPT2_KC_LAYERNORM, 0, es * 2.0 * M * C + 8.0 * M,
               gk::layernorm_forward(s, ln2, ln2m, ln2r, res2, md->P(P_LN2W) + l * C,
                                     md->P(P_LN2B) + l * C, M, C, h));
        a = mm(gk::GEMM_NT, gk::EPI_GELU, M, 4 * C, C, ln2, C,
               (const char*)md->W(P_FCW) + (size_t)l * 4 * C * C * y.es, C, fch, 4 * C);
        a.bias = md->P(P_FCB) + l * 4 * C;
        a.out2 = fchg;
        TRY(run_gemm(md, a));
        a = mm(gk::GEMM_NT, gk::EPI_RESID, M, C, 4 * C, fchg, 4 * C,
               (const char*)md->W(P_FCPROJW) + (size_t)l * C * 4 * C * y.es, 4 * C, res3, C);
        a.bias = md->P(P_FCPROJB) + l * C;
        a.aux = res2;
        a.ldaux = C;
        TRY(run_gemm(md, a));
    }
    const void* last = md->A(y.res3, (L - 1) * MC + ro * C);
    void* lnf = md->A(y.lnf, ro * C);
    LAUNCH(md, GPT2_KC_LAYERNORM, 0, es * 2.0 * M * C + 8.0 * M,
           gk::layernorm_forward(s, lnf, md->at<float>(y.lnf_mean) + ro,
                                 md->at<float>(y.lnf_rstd) + ro, last, md->P(P_LNFW),
                                 md->P(P_LNFB), M, C, h));
    void* logits = md->A(y.logits, ro * y.Vp);
    TRY(run_gemm(md, mm(gk::GEMM_NT, gk::EPI_STORE, M, V, C, lnf, C, md->W(P_WTE), C, logits,
                        y.Vp)));
    const bool train = mode == FWD_TRAIN;
    if (tgt) {
        float* losses = md->at<float>(y.losses);
        LAUNCH(md, GPT2_KC_SOFTMAX_CE, 0, es * (train ? 2.0 : 1.0) * M * (double)V + 8.0 * M,
               gk::softmax_ce(s, logits, losses, tgt, M, V, y.Vp, train ? 1.0f / M : 0.0f,
                              train && y.dt == DT_F16 ? md->lscale() : nullptr, md->flag(), h));
        LAUNCH(md, GPT2_KC_OTHER, 0, 4.0 * M, gk::mean_reduce(s, md->dloss(), losses, M));
    }
    if (train) {
        const int np2 = 1 << ceil_log2(M);
        LAUNCH(md, GPT2_KC_OTHER, 0, 4.0 * M + 4.0 * np2,
               gk::encoder_sort(s, md->at<uint32_t>(y.keys), tok, M, V, y.pos_bits, np2));
    }
    md->B = B;
    md->T = T;
    md->have_fwd = true;
    md->have_loss = tgt != nullptr;
    md->have_targets = train;
    md->logits_valid = !train;
    return GPT2_OK;
}

int read_loss(gpt2_model* md, float* mean_loss) {
    TRY(hip_check(hipMemcpyAsync(md->h_scal, md->at<char>(md->lay.scalars), 8,
                                 hipMemcpyDeviceToHost, md->stream),
                  "loss readback"));
    TRY(hip_check(hipStreamSynchronize(md->stream), "stream synchronize"));
    int flag;
    std::memcpy(&flag, md->h_scal + 1, 4);
    if (mean_loss) *mean_loss = md->have_loss ? md->h_scal[0] : NAN;
    if (flag & 1) return fail(GPT2_ERANGE, "a token id is outside [0, vocab_size)");
    if (flag & 2) return fail(GPT2_ERANGE, "a target id is outside [0, vocab_size)");
    return GPT2_OK;
}

int check_bt(gpt2_model* md, int B, int T) {
    if (B <= 0 || T <= 0 || B > md->lay.Bmax || T > md->lay.Tmax)
        return fail(GPT2_EINVAL, "B=%d T=%d outside the allocated 1..%d x 1..%d", B, T,
                    md->lay.Bmax, md->lay.Tmax);
    return GPT2_OK;
}

// ---- backward --------------------------------------------------------------

int backward_impl(gpt2_model* md) {
    const Layout& y = md->lay;
    const int L = y.L, C = y.C, NH = y.NH, V = y.V, B = md->B, T = md->T, M = B * T;
    const int h = y.dt;
    const size_t MC = (size_t)y.M * C;
    const size_t wes = y.es;  // bytes per weight element of the matmul copy
    const double es = (double)y.es;
    hipStream_t s = md->stream;
    void* dres = md->A(y.dres);
    void* dtmp = md->A(y.dtmp);
    void* dqkv = md->A(y.dqkv);
    void* dfch = md->A(y.dfch);
    float* lnpart = md->at<float>(y.ln_part);
    float* bpart = md->at<float>(y.bias_part);
    void* dlogits = md->A(y.logits);
    void* lnf = md->A(y.lnf);
    auto Wl = [&](int i, size_t elems) { return (const char*)md->W(i) + elems * wes; };

    // LM head (tied): dlnf = dlogits wte;  dwte += dlogits^T lnf
    TRY(run_gemm(md, mm(gk::GEMM_NN, gk::EPI_STORE, M, C, V, dlogits, y.Vp, md->W(P_WTE), C,
                        dtmp, C)));
    TRY(run_gemm(md, mm(gk::GEMM_TN, gk::EPI_ACCUM, V, C, M, dlogits, y.Vp, lnf, C,
                        md->G(P_WTE), C)));
    // Each layernorm backward also sums the residual-stream gradient it
    // leaves, over rows: that is the output gradient of the projection whose
    // result was added into the stream there, so the sum is that projection's
    // bias gradient.  After the final layernorm: the last MLP projection's.
    const void* last = md->A(y.res3, (L - 1) * MC);
    LAUNCH(md, GPT2_KC_LAYERNORM, 0, es * 3.0 * M * C + 8.0 * M,
           gk::layernorm_backward(s, dres, 0, md->G(P_LNFW), md->G(P_LNFB),
                                  md->G(P_FCPROJB) + (size_t)(L - 1) * C, lnpart, dtmp, last,
                                  md->P(P_LNFW), md->at<float>(y.lnf_mean),
                                  md->at<float>(y.lnf_rstd), M, C, h));
    for (int l = L - 1; l >= 0; l--) {
        const void* resid = l == 0 ? (const void*)md->A(y.encoded) : md->A(y.res3, (l - 1) * MC);
        const void* ln1 = md->A(y.ln1, l * MC);
        const float* ln1m = md->at<float>(y.ln1_mean) + (size_t)l * y.M;
        const float* ln1r = md->at<float>(y.ln1_rstd) + (size_t)l * y.M;
        const void* qkv = md->A(y.qkv, l * 3 * MC);
        const void* atty = md->A(y.atty, l * MC);
        const float* lse = md->at<float>(y.lse) + (size_t)l * y.M * NH;
        const void* res2 = md->A(y.res2, l * MC);
        const void* ln2 = md->A(y.ln2, l * MC);
        const float* ln2m = md->at<float>(y.ln2_mean) + (size_t)l * y.M;
        const float* ln2r = md->at<float>(y.ln2_rstd) + (size_t)l * y.M;
        const void* fch = md->A(y.fch, l * 4 * MC);
        const void* fchg = md->A(y.fch_gelu, l * 4 * MC);

        // MLP projection: dfch = (dres W) * gelu'(fch);  dW += dres^T gelu(fch).
        // The epilogue also sums dfch (the fc output gradient) over each
        // 64-row block: partial rows of the fc bias gradient.
        Mm a = mm(gk::GEMM_NN, gk::EPI_GELU_BWD, M, 4 * C, C, dres, C,
                  Wl(P_FCPROJW, (size_t)l * C * 4 * C), 4 * C, dfch, 4 * C);
        a.aux = fch;
        a.ldaux = 4 * C;
        a.colsum = bpart;
        TRY(run_gemm(md, a));
        TRY(run_gemm(md, mm(gk::GEMM_TN, gk::EPI_ACCUM, C, 4 * C, M, dres, C, fchg, 4 * C,
                            md->G(P_FCPROJW) + (size_t)l * C * 4 * C, 4 * C)));
        // (its bias gradient came from the layernorm backward that left dres)
        // MLP fc: dln2 = dfch W;  dW += dfch^T ln2
        TRY(run_gemm(md, mm(gk::GEMM_NN, gk::EPI_STORE, M, C, 4 * C, dfch, 4 * C,
                            Wl(P_FCW, (size_t)l * 4 * C * C), C, dtmp, C)));
        TRY(run_gemm(md, mm(gk::GEMM_TN, gk::EPI_ACCUM, 4 * C, C, M, dfch, 4 * C, ln2, C,
                            md->G(P_FCW) + (size_t)l * 4 * C * C, C)));
        LAUNCH(md, GPT2_KC_OTHER, 0, 4.0 * ((M + 63) / 64) * 4 * C,
               gk::colsum_add(s, md->G(P_FCB) + l * 4 * C, nullptr, nullptr, 4 * C, bpart,
                              (M + 63) / 64, 4 * C));
        // ln2; its output column sums are the attention projection's bias gradient
        LAUNCH(md, GPT2_KC_LAYERNORM, 0, es * 4.0 * M * C + 8.0 * M,
               gk::layernorm_backward(s, dres, 1, md->G(P_LN2W) + l * C, md->G(P_LN2B) + l * C,
                                      md->G(P_ATTPROJB) + (size_t)l * C, lnpart, dtmp, res2,
                                      md->P(P_LN2W) + l * C, ln2m, ln2r, M, C, h));
        // attention projection: datty = dres W;  dW += dres^T atty
        TRY(run_gemm(md, mm(gk::GEMM_NN, gk::EPI_STORE, M, C, C, dres, C,
                            Wl(P_ATTPROJW, (size_t)l * C * C), C, dtmp, C)));
        TRY(run_gemm(md, mm(gk::GEMM_TN, gk::EPI_ACCUM, C, C, M, dres, C, atty, C,
                            md->G(P_ATTPROJW) + (size_t)l * C * C, C)));
        {
            const double hs = C / NH;
            const double flops = 8.0 * B * NH * hs * (double)T * (T + 1) / 2.0;
            const double nb32 = (T + 31) / 32;  // dS^T blocks written, then read
            const double ds_bytes = y.ds_stride ? 8.0 * B * NH * nb32 * (nb32 + 1) / 2 * 1024 : 0;
            LAUNCH(md, GPT2_KC_ATTENTION, flops, es * 7.0 * M * C + 8.0 * M * NH + ds_bytes,
                   gk::attention_backward(s, dqkv, md->at<float>(y.attn_d), dtmp, qkv, atty, lse,
                                          B, T, C, NH, h,
                                          y.ds_stride ? md->at<float>(y.attn_ds) : nullptr,
                                          y.ds_stride));
        }
        if (y.rope)  // back through the rotation: dq, dk of the unrotated q, k
            LAUNCH(md, GPT2_KC_OTHER, 0, es * 4.0 * M * C,
                   gk::rope_apply(s, dqkv, md->at<float>(y.rope_cs), B, T, C, NH, -1, h));
        // QKV: dln1 = dqkv W;  dW += dqkv^T ln1
        TRY(run_gemm(md, mm(gk::GEMM_NN, gk::EPI_STORE, M, C, 3 * C, dqkv, 3 * C,
                            Wl(P_QKVW, (size_t)l * 3 * C * C), C, dtmp, C)));
        TRY(run_gemm(md, mm(gk::GEMM_TN, gk::EPI_ACCUM, 3 * C, C, M, dqkv, 3 * C, ln1, C,
                            md->G(P_QKVW) + (size_t)l * 3 * C * C, C)));
        LAUNCH(md, GPT2_KC_OTHER, 0, es * 3.0 * M * C,
               gk::bias_grad(s, md->G(P_QKVB) + l * 3 * C, bpart, dqkv, M, 3 * C, 3 * C, h));
        // ln1; its output is the gradient at the previous layer's output, whose
        // column sums are that layer's MLP-projection bias gradient
        LAUNCH(md, GPT2_KC_LAYERNORM, 0, es * 4.0 * M * C + 8.0 * M,
               gk::layernorm_backward(s, dres, 1, md->G(P_LN1W) + l * C, md->G(P_LN1B) + l * C,
                                      l > 0 ? md->G(P_FCPROJB) + (size_t)(l - 1) * C : nullptr,
                                      lnpart, dtmp, resid, md->P(P_LN1W) + l * C, ln1m, ln1r, M,
                                      C, h));
    }
    LAUNCH(md, GPT2_KC_OTHER, 0, es * M * C + 8.0 * M * C + 8.0 * T * C + 4.0 * M,
           gk::encoder_backward(s, md->G(P_WTE), y.rope ? nullptr : md->G(P_WPE),
                                md->at<float>(y.embed_part), dres,
                                md->at<uint32_t>(y.keys), B,
                                T, C, V, y.pos_bits, h));
    return GPT2_OK;
}

bool valid_model(gpt2_model* md) { return md != nullptr && md->base != nullptr; }

// ---- debug guard words ---------------------------------------------------------

// GPT2_GUARD_WORDS set (and not "0") at create puts a guard region after
// every sub-buffer of the arena.
bool guards_requested() {
    const char* e = std::getenv("GPT2_GUARD_WORDS");
    return e && *e && std::strcmp(e, "0") != 0;
}

int write_guards(gpt2_model* md) {
    std::vector<uint32_t> pat(gh::kGuardBytes / 4, gh::kGuardWord);
    for (const auto& r : md->lay.regions)
        TRY(hip_check(hipMemcpy(md->base + r.guard, pat.data(), gh::kGuardBytes,
                                hipMemcpyHostToDevice),
                      "guard write"));
    return GPT2_OK;
}

}  // namespace

// ============================================================================
// C ABI
// ============================================================================

extern "C" {

void gpt2_destroy(gpt2_model* md) {
    if (!md) return;
    if (md->stream != nullptr || md->base) hipStreamSynchronize(md->stream);
    for (hipEvent_t e : md->prof.ev) hipEventDestroy(e);
    if (md->stage_done) hipEventDestroy(md->stage_done);
    if (md->h_stage) hipHostFree(md->h_stage);
    if (md->h_scal) hipHostFree(md->h_scal);
    if (md->base) {
        if (md->custom_alloc)
            md->alloc.free(md->base, md->alloc.ctx);
        else
            hipFree(md->base);
    }
    delete md;
}

int gpt2_create(const gpt2_config* cfg, const gpt2_allocator* alloc, void* hip_stream,
                gpt2_model** out) {
    if (!out) return fail(GPT2_EINVAL, "out is NULL");
    *out = nullptr;
    TRY(check_config(cfg));
    if (alloc && (!alloc->alloc || !alloc->free))
        return fail(GPT2_EINVAL, "allocator needs both alloc and free");
    gpt2_model* md = new gpt2_model();
    md->cfg = *cfg;
    md->lay.build(cfg, gk::device_cu_count(), guards_requested());
    md->stream = (hipStream_t)hip_stream;
    int rc = GPT2_OK;
    if (alloc) {
        md->alloc = *alloc;
        md->custom_alloc = true;
        md->base = (char*)alloc->alloc(md->lay.total, alloc->ctx);
        if (!md->base) rc = fail(GPT2_ENOMEM, "allocator returned NULL for %zu bytes", md->lay.total);
    } else {
        hipError_t e = hipMalloc((void**)&md->base, md->lay.total);
        if (e != hipSuccess) {
            md->base = nullptr;
            rc = fail(e == hipErrorOutOfMemory ? GPT2_ENOMEM : GPT2_EDEVICE,
                      "hipMalloc(%zu): %s", md->lay.total, hipGetErrorString(e));
        }
    }
    if (rc == GPT2_OK && ((uintptr_t)md->base & 255))
        rc = fail(GPT2_EINVAL, "allocator returned memory not aligned to 256 bytes");
    if (rc == GPT2_OK)
        rc = hip_check(hipHostMalloc((void**)&md->h_stage, 2 * (size_t)md->lay.M * sizeof(int32_t)),
                       "hipHostMalloc");
    if (rc == GPT2_OK) rc = hip_check(hipHostMalloc((void**)&md->h_scal, 64), "hipHostMalloc");
    if (rc == GPT2_OK)
        rc = hip_check(hipEventCreateWithFlags(&md->stage_done, hipEventDisableTiming),
                       "hipEventCreate");
    if (rc == GPT2_OK) {
        const hipError_t e = gk::encoder_sort_prepare(md->lay.n_pow2);
        rc = hip_check(e, "encoder sort setup");
    }
    if (rc == GPT2_OK && md->lay.rope) {
        // (cos, sin) of t * 10000^(-2i/hs), computed in double
        const int half = md->lay.C / md->lay.NH / 2;
        std::vector<float> cs((size_t)md->lay.Tmax * half * 2);
        for (int t = 0; t < md->lay.Tmax; t++)
            for (int i = 0; i < half; i++) {
                const double a = t * std::pow(10000.0, -2.0 * i / (2.0 * half));
                cs[((size_t)t * half + i) * 2] = (float)std::cos(a);
                cs[((size_t)t * half + i) * 2 + 1] = (float)std::sin(a);
            }
        rc = hip_check(hipMemcpy(md->at<char>(md->lay.rope_cs), cs.data(), cs.size() * sizeof(float),
                                 hipMemcpyHostToDevice),
                       "rotary table upload");
    }
    if (rc == GPT2_OK) {
        // parameters, gradients and both moments start at zero
        const hipError_t e = gk::fill_zero(md->stream, md->at<float>(0),
                                           (int64_t)(md->lay.encoded / sizeof(float)));
        rc = hip_check(e, "zero arenas");
        if (rc == GPT2_OK) rc = hip_check(hipStreamSynchronize(md->stream), "synchronize");
    }
    if (rc == GPT2_OK && md->lay.dt == DT_F16) {
        const float s0 = 65536.0f;  // 2^16; halves on overflow, doubles after 2000 clean steps
        const int32_t st[4] = {0, 0, 0, 0};
        rc = hip_check(hipMemcpy(md->lscale(), &s0, 4, hipMemcpyHostToDevice), "scale init");
        if (rc == GPT2_OK)
            rc = hip_check(hipMemcpy(md->lgood(), st, 12, hipMemcpyHostToDevice), "scale init");
    }
    if (rc == GPT2_OK && md->lay.guards) rc = write_guards(md);
    if (rc != GPT2_OK) {
        const std::string msg = gpt2_last_error();
        gpt2_destroy(md);
        gpt2_set_error(rc, msg.c_str());
        return rc;
    }
    *out = md;
    return GPT2_OK;
}

int64_t gpt2_num_parameters(const gpt2_model* md) { return md ? md->lay.nparams : -1; }

int gpt2_param_tensor(const gpt2_model* md, int i, const char** name, int64_t* offset,
                      int64_t* numel) {
    if (!md) return fail(GPT2_EINVAL, "model is NULL");
    return gpt2_config_param_tensor(&md->cfg, i, name, offset, numel);
}

int gpt2_copy_params(gpt2_model* md, float* dst, const float* src) {
    if (!valid_model(md)) return fail(GPT2_EINVAL, "model is NULL");
    if ((dst == nullptr) == (src == nullptr))
        return fail(GPT2_EINVAL, "exactly one of host_dst and host_src must be non-NULL");
    const size_t bytes = md->lay.nparams * sizeof(float);
    TRY(hip_check(hipStreamSynchronize(md->stream), "synchronize"));
    if (dst)
        return hip_check(hipMemcpy(dst, md->P(0), bytes, hipMemcpyDeviceToHost), "copy params");
    TRY(hip_check(hipMemcpy(md->P(0), src, bytes, hipMemcpyHostToDevice), "copy params"));
    if (md->lay.half) {
        TRY(hip_check(gk::to_half(md->stream, md->at<uint16_t>(md->lay.shadow), md->P(0),
                                  md->lay.nparams, md->lay.dt),
                      "16-bit weight copy"));
        TRY(hip_check(hipStreamSynchronize(md->stream), "synchronize"));
    }
    return GPT2_OK;
}

int gpt2_copy_grads(gpt2_model* md, float* dst) {
    if (!valid_model(md) || !dst) return fail(GPT2_EINVAL, "NULL argument");
    TRY(hip_check(hipStreamSynchronize(md->stream), "synchronize"));
    if (md->lay.dt == DT_F16) {  // the arena holds scale * gradient
        float sc;
        TRY(hip_check(hipMemcpy(&sc, md->lscale(), 4, hipMemcpyDeviceToHost), "scale readback"));
        TRY(hip_check(hipMemcpy(dst, md->G(0), md->lay.nparams * sizeof(float),
                                hipMemcpyDeviceToHost),
                      "copy grads"));
        const float inv = 1.0f / sc;
        for (int64_t i = 0; i < md->lay.nparams; i++) dst[i] *= inv;
        return GPT2_OK;
    }
    return hip_check(hipMemcpy(dst, md->G(0), md->lay.nparams * sizeof(float),
                               hipMemcpyDeviceToHost),
                     "copy grads");
}

int gpt2_copy_opt_state(gpt2_model* md, float* hm, float* hv) {
    if (!valid_model(md)) return fail(GPT2_EINVAL, "model is NULL");
    TRY(hip_check(hipStreamSynchronize(md->stream), "synchronize"));
    const size_t bytes = md->lay.nparams * sizeof(float);
    if (hm) TRY(hip_check(hipMemcpy(hm, md->at<float>(md->lay.m), bytes, hipMemcpyDeviceToHost), "copy m"));
    if (hv) TRY(hip_check(hipMemcpy(hv, md->at<float>(md->lay.v), bytes, hipMemcpyDeviceToHost), "copy v"));
    return GPT2_OK;
}

// ---- checkpoint -----------------------------------------------------------
//
// File: a 32-byte header {"GPT2CKPT", version 2 (u32), precision (u32),
// nparams (i64), step (i64)}, the 16-byte loss-scale block {scale (f32),
// clean updates (i32), growth interval (i32), 0 (u32)}, then params, m and v
// as nparams little-endian fp32 each, in the arena order.  Version-1 files
// (no scale block) still load.  Streamed through one host buffer of at most
// 16M floats.

namespace {

int ckpt_stream(gpt2_model* md, FILE* f, bool save) {
    const int64_t n = md->lay.nparams;
    const size_t chunk = (size_t)std::min<int64_t>(n, (int64_t)1 << 24);
    std::vector<float> buf;
    try {
        buf.resize(chunk);
    } catch (...) {
        return fail(GPT2_ENOMEM, "checkpoint buffer");
    }
    float* arenas[3] = {md->P(0), md->at<float>(md->lay.m), md->at<float>(md->lay.v)};
    for (float* a : arenas)
        for (int64_t off = 0; off < n; off += (int64_t)chunk) {
            const size_t cnt = (size_t)std::min<int64_t>((int64_t)chunk, n - off);
            if (save) {
                TRY(hip_check(hipMemcpy(buf.data(), a + off, cnt * 4, hipMemcpyDeviceToHost),
                              "checkpoint read"));
                if (fwrite(buf.data(), 4, cnt, f) != cnt)
                    return fail(GPT2_EINVAL, "checkpoint write failed: %s", strerror(errno));
            } else {
                if (fread(buf.data(), 4, cnt, f) != cnt)
                    return fail(GPT2_EINVAL, "checkpoint is truncated");
                TRY(hip_check(hipMemcpy(a + off, buf.data(), cnt * 4, hipMemcpyHostToDevice),
                              "checkpoint write"));
            }
        }
    return GPT2_OK;
}

}  // namespace

int gpt2_save_checkpoint(gpt2_model* md, const char* path, int64_t step) {
    if (!valid_model(md) || !path) return fail(GPT2_EINVAL, "NULL argument");
    if (step < 0) return fail(GPT2_EINVAL, "step %lld < 0", (long long)step);
    TRY(hip_check(hipStreamSynchronize(md->stream), "synchronize"));
    FILE* f = fopen(path, "wb");
    if (!f) return fail(GPT2_EINVAL, "cannot open %s: %s", path, strerror(errno));
    gh::CkptHeader h;
    gh::ckpt_header_make(&h, md->cfg.precision, md->lay.nparams, step);
    gh::CkptScale sc{1.0f, 0, 0, 0u};
    if (md->lay.dt == DT_F16) {  // the dynamic loss-scale state is part of the training state
        TRY(hip_check(hipMemcpy(&sc.scale, md->lscale(), 4, hipMemcpyDeviceToHost), "scale read"));
        TRY(hip_check(hipMemcpy(&sc.good, md->lgood(), 4, hipMemcpyDeviceToHost), "scale read"));
        sc.growth_interval = md->growth_interval;
    }
    int rc = fwrite(&h, sizeof h, 1, f) == 1 && fwrite(&sc, sizeof sc, 1, f) == 1
                 ? ckpt_stream(md, f, true)
                 : fail(GPT2_EINVAL, "checkpoint write failed");
    if (fclose(f) != 0 && rc == GPT2_OK) rc = fail(GPT2_EINVAL, "checkpoint close failed");
    return rc;
}

int gpt2_load_checkpoint(gpt2_model* md, const char* path, int64_t* step) {
    if (!valid_model(md) || !path) return fail(GPT2_EINVAL, "NULL argument");
    FILE* f = fopen(path, "rb");
    if (!f) return fail(GPT2_EINVAL, "cannot open %s: %s", path, strerror(errno));
    gh::CkptHeader h{};
    gh::CkptScale sc{1.0f, 0, 0, 0u};
    const size_t got = fread(&h, 1, sizeof h, f);
    int rc = gh::ckpt_header_check(&h, got, md->lay.nparams, path);
    if (rc == GPT2_OK && h.version >= 2)
        rc = gh::ckpt_scale_check(&sc, fread(&sc, 1, sizeof sc, f), h.precision, path);
    if (rc == GPT2_OK) rc = hip_check(hipStreamSynchronize(md->stream), "synchronize");
    if (rc == GPT2_OK) rc = ckpt_stream(md, f, false);
    if (rc == GPT2_OK && fgetc(f) != EOF) rc = fail(GPT2_EINVAL, "checkpoint has trailing bytes");
    fclose(f);
    if (rc != GPT2_OK) return rc;
    if (md->lay.half) {  // the 16-bit weight copies follow the loaded weights
        TRY(hip_check(gk::to_half(md->stream, md->at<uint16_t>(md->lay.shadow), md->P(0),
                                  md->lay.nparams, md->lay.dt),
                      "16-bit weight copy"));
        TRY(hip_check(hipStreamSynchronize(md->stream), "synchronize"));
    }
    if (md->lay.dt == DT_F16 && h.version >= 2 && h.precision == (uint32_t)GPT2_F16_MIXED) {
        // resume the saved loss-scale schedule (an fp32 or bf16 file leaves
        // the fp16 model's current schedule as it is)
        const int32_t st[3] = {sc.good, 0, 0};  // good, found, skipped
        TRY(hip_check(hipMemcpy(md->lscale(), &sc.scale, 4, hipMemcpyHostToDevice),
                      "scale write"));
        TRY(hip_check(hipMemcpy(md->lgood(), st, 12, hipMemcpyHostToDevice), "scale write"));
        md->growth_interval = sc.growth_interval;
    }
    if (step) *step = h.step;
    return GPT2_OK;
}

int gpt2_copy_activation(gpt2_model* md, const char* name, int layer, float* dst,
                         int64_t* numel) {
    if (!valid_model(md) || !name) return fail(GPT2_EINVAL, "NULL argument");
    if (!md->have_fwd) return fail(GPT2_ESTATE, "no forward has run");
    const Layout& y = md->lay;
    const int64_t M = (int64_t)md->B * md->T, C = y.C;
    const size_t MC = (size_t)y.M * C;
    struct Item {
        const char* n;
        size_t off;
        size_t layer_stride;  // elements; 0 = not per layer
        int64_t width;        // per row of B*T
        bool act;             // activation storage type (else fp32 statistics)
    };
    const Item items[] = {
        {"encoded", y.encoded, 0, C, true},
        {"ln1", y.ln1, MC, C, true},
        {"ln1_mean", y.ln1_mean, (size_t)y.M, 1, false},
        {"ln1_rstd", y.ln1_rstd, (size_t)y.M, 1, false},
        {"qkv", y.qkv, 3 * MC, 3 * C, true},
        {"atty", y.atty, MC, C, true},
        {"att_lse", y.lse, (size_t)y.M * y.NH, y.NH, false},
        {"residual2", y.res2, MC, C, true},
        {"ln2", y.ln2, MC, C, true},
        {"ln2_mean", y.ln2_mean, (size_t)y.M, 1, false},
        {"ln2_rstd", y.ln2_rstd, (size_t)y.M, 1, false},
        {"fch", y.fch, 4 * MC, 4 * C, true},
        {"fch_gelu", y.fch_gelu, 4 * MC, 4 * C, true},
        {"residual3", y.res3, MC, C, true},
        {"lnf", y.lnf, 0, C, true},
        {"lnf_mean", y.lnf_mean, 0, 1, false},
        {"lnf_rstd", y.lnf_rstd, 0, 1, false},
        {"logits", y.logits, 0, y.V, true},
        {"losses", y.losses, 0, 1, false},
    };
    for (const Item& it : items) {
        if (std::strcmp(it.n, name)) continue;
        if (it.layer_stride && (layer < 0 || layer >= y.L))
            return fail(GPT2_EINVAL, "layer %d outside 0..%d", layer, y.L - 1);
        const int64_t n = M * it.width;
        if (numel) *numel = n;
        if (!dst) return GPT2_OK;
        TRY(hip_check(hipStreamSynchronize(md->stream), "synchronize"));
        const size_t es = it.act ? y.es : sizeof(float);
        const char* src = md->base + it.off + (it.layer_stride ? layer * it.layer_stride : 0) * es;
        const bool logits = std::strcmp(name, "logits") == 0;
        if (es == sizeof(float)) {
            if (logits)
                return hip_check(hipMemcpy2D(dst, y.V * sizeof(float), src, y.Vp * sizeof(float),
                                             y.V * sizeof(float), M, hipMemcpyDeviceToHost),
                                 "copy logits");
            return hip_check(hipMemcpy(dst, src, n * sizeof(float), hipMemcpyDeviceToHost),
                             "copy activation");
        }
        // 16-bit: copy the bits, widen on the host
        std::vector<uint16_t> tmp((size_t)n);
        if (logits)
            TRY(hip_check(hipMemcpy2D(tmp.data(), y.V * 2, src, y.Vp * 2, y.V * 2, M,
                                      hipMemcpyDeviceToHost),
                          "copy logits"));
        else
            TRY(hip_check(hipMemcpy(tmp.data(), src, n * 2, hipMemcpyDeviceToHost),
                          "copy activation"));
        for (int64_t i = 0; i < n; i++)
            dst[i] = y.dt == DT_F16 ? half_bits_to_float(tmp[(size_t)i])
                                    : bf16_bits_to_float(tmp[(size_t)i]);
        return GPT2_OK;
    }
    return fail(GPT2_EINVAL, "unknown activation name '%s'", name);
}

namespace {

// Checks host ids and queues their upload through the pinned staging buffer
// (waiting until the previous upload has left it); *dtok / *dtgt get the
// device copies (*dtgt = NULL without targets).
int stage_ids(gpt2_model* md, const int32_t* tokens, const int32_t* targets, int B, int T,
              int32_t** dtok, int32_t** dtgt) {
    TRY(check_bt(md, B, T));
    const int M = B * T, V = md->lay.V;
    for (int i = 0; i < M; i++)
        if (tokens[i] < 0 || tokens[i] >= V)
            return fail(GPT2_ERANGE, "token %d at position %d outside [0, %d)", tokens[i], i, V);
    if (targets)
        for (int i = 0; i < M; i++)
            if (targets[i] < 0 || targets[i] >= V)
                return fail(GPT2_ERANGE, "target %d at position %d outside [0, %d)", targets[i],
                            i, V);
    if (md->stage_pending) TRY(hip_check(hipEventSynchronize(md->stage_done), "stage wait"));
    std::memcpy(md->h_stage, tokens, M * sizeof(int32_t));
    if (targets) std::memcpy(md->h_stage + md->lay.M, targets, M * sizeof(int32_t));
    *dtok = md->at<int32_t>(md->lay.tokens);
    *dtgt = targets ? md->at<int32_t>(md->lay.targets) : nullptr;
    TRY(hip_check(hipMemcpyAsync(*dtok, md->h_stage, M * sizeof(int32_t), hipMemcpyHostToDevice,
                                 md->stream),
                  "token upload"));
    if (targets)
        TRY(hip_check(hipMemcpyAsync(*dtgt, md->h_stage + md->lay.M, M * sizeof(int32_t),
                                     hipMemcpyHostToDevice, md->stream),
                      "target upload"));
    TRY(hip_check(hipEventRecord(md->stage_done, md->stream), "event record"));
    md->stage_pending = true;
    return GPT2_OK;
}

}  // namespace

int gpt2_forward(gpt2_model* md, const int32_t* tokens, const int32_t* targets, int B, int T,
                 float* mean_loss) {
    if (!valid_model(md) || !tokens) return fail(GPT2_EINVAL, "NULL argument");
    int32_t *dtok, *dtgt;
    TRY(stage_ids(md, tokens, targets, B, T, &dtok, &dtgt));
    TRY(forward_impl(md, dtok, dtgt, B, T, targets ? FWD_TRAIN : FWD_INFER));
    if (mean_loss) return read_loss(md, mean_loss);
    return GPT2_OK;
}

int gpt2_evaluate(gpt2_model* md, const int32_t* tokens, const int32_t* targets, int B, int T,
                  float* mean_loss) {
    if (!valid_model(md) || !tokens || !targets || !mean_loss)
        return fail(GPT2_EINVAL, "NULL argument");
    int32_t *dtok, *dtgt;
    TRY(stage_ids(md, tokens, targets, B, T, &dtok, &dtgt));
    TRY(forward_impl(md, dtok, dtgt, B, T, FWD_EVAL));
    return read_loss(md, mean_loss);
}

int gpt2_forward_device(gpt2_model* md, const int32_t* tokens, const int32_t* targets, int B,
                        int T, float* mean_loss) {
    if (!valid_model(md) || !tokens) return fail(GPT2_EINVAL, "NULL argument");
    TRY(check_bt(md, B, T));
    TRY(forward_impl(md, tokens, targets, B, T, targets ? FWD_TRAIN : FWD_INFER));
    if (mean_loss) return read_loss(md, mean_loss);
    return GPT2_OK;
}

int gpt2_sample(gpt2_model* md, int b, int t, float coin, int32_t* token) {
    if (!valid_model(md) || !token) return fail(GPT2_EINVAL, "NULL argument");
    if (!md->have_fwd || !md->logits_valid)
        return fail(GPT2_ESTATE, "sampling needs a preceding forward without targets");
    if (b < 0 || b >= md->B || t < 0 || t >= md->T)
        return fail(GPT2_EINVAL, "position (%d, %d) outside the last forward's %d x %d", b, t,
                    md->B, md->T);
    if (!(coin >= 0.f && coin < 1.f)) return fail(GPT2_EINVAL, "coin must be in [0, 1)");
    const Layout& y = md->lay;
    const char* row = md->A(y.logits, ((size_t)b * md->T + t) * y.Vp);
    LAUNCH(md, GPT2_KC_SOFTMAX_CE, 0, y.es * (double)y.V * 2.0 + 4.0,
           gk::sample_row(md->stream, row, y.V, coin, md->drawn(), y.dt));
    TRY(hip_check(hipMemcpyAsync(md->h_scal + 2, md->drawn(), 4, hipMemcpyDeviceToHost,
                                 md->stream),
                  "token readback"));
    TRY(hip_check(hipStreamSynchronize(md->stream), "stream synchronize"));
    std::memcpy(token, md->h_scal + 2, 4);
    return GPT2_OK;
}

int gpt2_generate(gpt2_model* md, int32_t* tokens, int prompt_len, int n, const float* coins) {
    if (!valid_model(md) || !tokens || (!coins && n > prompt_len))
        return fail(GPT2_EINVAL, "NULL argument");
    if (prompt_len < 1 || n < prompt_len || n > md->lay.Tmax)
        return fail(GPT2_EINVAL, "prompt_len=%d n=%d outside 1 <= prompt_len <= n <= %d",
                    prompt_len, n, md->lay.Tmax);
    // The prompt's forward, then one new position per drawn token: the rows
    // of the earlier positions, kept in the activation arena, serve as the
    // key/value cache.
    for (int t = prompt_len; t < n; t++) {
        int32_t *dtok, *dtgt;
        TRY(stage_ids(md, tokens, nullptr, 1, t, &dtok, &dtgt));
        TRY(forward_impl(md, dtok, nullptr, 1, t, FWD_INFER, t == prompt_len ? 0 : t - 1));
        TRY(gpt2_sample(md, 0, t - 1, coins[t - prompt_len], tokens + t));
    }
    return GPT2_OK;
}

int gpt2_zero_grad(gpt2_model* md) {
    if (!valid_model(md)) return fail(GPT2_EINVAL, "model is NULL");
    LAUNCH(md, GPT2_KC_OTHER, 0, 4.0 * md->lay.nparams,
           gk::fill_zero(md->stream, md->G(0), md->lay.nparams));
    return GPT2_OK;
}

int gpt2_backward(gpt2_model* md) {
    if (!valid_model(md)) return fail(GPT2_EINVAL, "model is NULL");
    if (!md->have_fwd || !md->have_targets)
        return fail(GPT2_ESTATE, "backward needs a preceding forward with targets");
    TRY(backward_impl(md));
    md->have_targets = false;  // the logits gradient has been consumed
    return GPT2_OK;
}

int gpt2_update(gpt2_model* md, float lr, float beta1, float beta2, float eps,
                float weight_decay, int step) {
    if (!valid_model(md)) return fail(GPT2_EINVAL, "model is NULL");
    if (step < 1) return fail(GPT2_EINVAL, "step must be >= 1 (got %d)", step);
    if (!(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f))
        return fail(GPT2_EINVAL, "betas must be in [0, 1)");
    const float bc1 = (float)(1.0 - std::pow((double)beta1, (double)step));
    const float bc2 = (float)(1.0 - std::pow((double)beta2, (double)step));
    const int64_t n = md->lay.nparams;
    const bool scaled = md->lay.dt == DT_F16;
    if (scaled)  // a non-finite (overflowed) gradient skips the whole update
        LAUNCH(md, GPT2_KC_ADAMW, 0, 4.0 * n,
               gk::check_finite(md->stream, md->G(0), n, md->lfound()));
    LAUNCH(md, GPT2_KC_ADAMW, 0, (md->lay.half ? 30.0 : 28.0) * n,
           gk::adamw(md->stream, md->P(0), md->G(0), md->at<float>(md->lay.m),
                     md->at<float>(md->lay.v),
                     md->lay.half ? md->at<uint16_t>(md->lay.shadow) : nullptr, md->lay.dt, n,
                     lr, beta1, beta2, eps, weight_decay, bc1, bc2,
                     scaled ? md->lscale() : nullptr, scaled ? md->lfound() : nullptr));
    if (scaled)
        LAUNCH(md, GPT2_KC_OTHER, 0, 16.0,
               gk::loss_scale_update(md->stream, md->lscale(), md->lgood(), md->lfound(),
                                     md->lskipped(), md->growth_interval, 1.0f));
    return GPT2_OK;
}

int gpt2_set_loss_scale(gpt2_model* md, float scale, int growth_interval) {
    if (!valid_model(md)) return fail(GPT2_EINVAL, "model is NULL");
    if (md->lay.dt != DT_F16) return fail(GPT2_EINVAL, "loss scaling applies to the fp16 model");
    if (!(scale >= 1.0f && scale < INFINITY) || growth_interval < 1)
        return fail(GPT2_EINVAL, "scale must be finite and >= 1, growth_interval >= 1");
    const int32_t st[4] = {0, 0, 0, 0};
    TRY(hip_check(hipStreamSynchronize(md->stream), "synchronize"));
    TRY(hip_check(hipMemcpy(md->lscale(), &scale, 4, hipMemcpyHostToDevice), "scale upload"));
    TRY(hip_check(hipMemcpy(md->lgood(), st, 12, hipMemcpyHostToDevice), "scale state"));
    md->growth_interval = growth_interval;
    return GPT2_OK;
}

int gpt2_get_loss_scale(gpt2_model* md, float* scale, int* last_update_skipped) {
    if (!valid_model(md)) return fail(GPT2_EINVAL, "model is NULL");
    if (md->lay.dt != DT_F16) return fail(GPT2_EINVAL, "loss scaling applies to the fp16 model");
    TRY(hip_check(hipStreamSynchronize(md->stream), "synchronize"));
    float sc;
    int sk;
    TRY(hip_check(hipMemcpy(&sc, md->lscale(), 4, hipMemcpyDeviceToHost), "scale readback"));
    TRY(hip_check(hipMemcpy(&sk, md->lskipped(), 4, hipMemcpyDeviceToHost), "scale readback"));
    if (scale) *scale = sc;
    if (last_update_skipped) *last_update_skipped = sk;
    return GPT2_OK;
}

int gpt2_check_guards(gpt2_model* md) {
    if (!valid_model(md)) return fail(GPT2_EINVAL, "model is NULL");
    if (!md->lay.guards)
        return fail(GPT2_EINVAL, "the model was created without GPT2_GUARD_WORDS");
    TRY(hip_check(hipStreamSynchronize(md->stream), "synchronize"));
    std::vector<uint32_t> got(gh::kGuardBytes / 4);
    for (const auto& r : md->lay.regions) {
        TRY(hip_check(hipMemcpy(got.data(), md->base + r.guard, gh::kGuardBytes,
                                hipMemcpyDeviceToHost),
                      "guard read"));
        for (size_t i = 0; i < got.size(); i++)
            if (got[i] != gh::kGuardWord)
                return fail(GPT2_ECORRUPT,
                            "guard after '%s' (%zu bytes) overwritten at byte %zu: 0x%08x",
                            r.name, r.bytes, 4 * i, got[i]);
    }
    return GPT2_OK;
}

int gpt2_synchronize(gpt2_model* md) {
    if (!valid_model(md)) return fail(GPT2_EINVAL, "model is NULL");
    TRY(hip_check(hipStreamSynchronize(md->stream), "synchronize"));
    int flag = 0;
    TRY(hip_check(hipMemcpy(&flag, md->flag(), 4, hipMemcpyDeviceToHost), "flag readback"));
    if (flag & 1) return fail(GPT2_ERANGE, "a token id is outside [0, vocab_size)");
    if (flag & 2) return fail(GPT2_ERANGE, "a target id is outside [0, vocab_size)");
    return GPT2_OK;
}

int gpt2_profile(gpt2_model* md, int class_mask) {
    if (!valid_model(md)) return fail(GPT2_EINVAL, "model is NULL");
    if (class_mask & ~GPT2_PROFILE_ALL) return fail(GPT2_EINVAL, "class mask 0x%x", class_mask);
    Prof& p = md->prof;
    if (class_mask) {
        p.mask = class_mask;
        if (p.ev.empty()) {
            p.ev.resize(kEventPool);
            for (auto& e : p.ev) TRY(hip_check(hipEventCreate(&e), "hipEventCreate"));
        }
        prof_flush(md);
        for (int k = 0; k < GPT2_KC_COUNT; k++) p.ms[k] = p.fl[k] = p.by[k] = 0, p.n[k] = 0;
        p.on = true;
    } else {
        prof_flush(md);
        p.on = false;
    }
    return GPT2_OK;
}

int gpt2_profile_read(gpt2_model* md, int kc, double* total_ms, int64_t* launches,
                      double* flops, double* bytes) {
    if (!valid_model(md)) return fail(GPT2_EINVAL, "model is NULL");
    if (kc < 0 || kc >= GPT2_KC_COUNT) return fail(GPT2_EINVAL, "kernel class %d", kc);
    prof_flush(md);
    if (total_ms) *total_ms = md->prof.ms[kc];
    if (launches) *launches = md->prof.n[kc];
    if (flops) *flops = md->prof.fl[kc];
    if (bytes) *bytes = md->prof.by[kc];
    return GPT2_OK;
}

}  // extern "C"
