// Host-only parts of the library (see host.h).  No HIP: this file also builds
// with a plain C++ compiler for the host sanitizer checks.
#include "host.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "dtype.h"
#include "plan.h"

namespace {
thread_local std::string g_err;
}  // namespace

int gpt2_set_error(int code, const char* msg) {
    g_err = msg ? msg : "";
    return code;
}

namespace gh {

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

const char* const kParamNames[16] = {"wte",      "wpe",      "ln1w", "ln1b", "qkvw",    "qkvb",
                                     "attprojw", "attprojb", "ln2w", "ln2b", "fcw",     "fcb",
                                     "fcprojw",  "fcprojb",  "lnfw", "lnfb"};

void param_sizes(const gpt2_config* c, int64_t* s) {
    const int64_t L = c->num_layers, C = c->channels, V = c->vocab_size, T = c->max_seq_len;
    const int64_t P = c->rope ? 0 : T * C;  // the rotary model has no position table
    const int64_t v[16] = {V * C, P, L * C, L * C, L * 3 * C * C, L * 3 * C, L * C * C,
                           L * C, L * C, L * C, L * 4 * C * C, L * 4 * C, L * C * 4 * C,
                           L * C, C, C};
    for (int i = 0; i < 16; i++) s[i] = v[i];
}

int ceil_log2(int64_t n) {
    int b = 0;
    while ((int64_t(1) << b) < n) b++;
    return b;
}

int check_config(const gpt2_config* c) {
    if (!c) return fail(GPT2_EINVAL, "config is NULL");
    if (c->num_layers <= 0 || c->channels <= 0 || c->num_heads <= 0 || c->vocab_size <= 0 ||
        c->max_seq_len <= 0 || c->batch_size <= 0 || c->seq_len <= 0)
        return fail(GPT2_EINVAL, "every config field must be positive");
    if (c->channels % c->num_heads)
        return fail(GPT2_EINVAL, "channels (%d) must be a multiple of num_heads (%d)",
                    c->channels, c->num_heads);
    const int hs = c->channels / c->num_heads;
    if (hs != 16 && hs != 32 && hs != 64)
        return fail(GPT2_EINVAL, "head size %d not supported (16, 32 or 64)", hs);
    if (c->channels > 1024) return fail(GPT2_EINVAL, "channels > 1024 not supported");
    if (c->num_layers > 1024) return fail(GPT2_EINVAL, "num_layers > 1024 not supported");
    if (c->seq_len > c->max_seq_len)
        return fail(GPT2_EINVAL, "seq_len %d > max_seq_len %d", c->seq_len, c->max_seq_len);
    if (c->max_seq_len > 65536) return fail(GPT2_EINVAL, "max_seq_len > 65536 not supported");
    if ((int64_t)c->batch_size * c->seq_len > 32768)
        return fail(GPT2_EINVAL, "batch_size*seq_len > 32768 not supported");
    if (c->vocab_size > 65536) return fail(GPT2_EINVAL, "vocab_size > 65536 not supported");
    if (c->precision != GPT2_FP32 && c->precision != GPT2_BF16_MIXED &&
        c->precision != GPT2_F16_MIXED)
        return fail(GPT2_EINVAL, "unknown precision %d", c->precision);
    if (c->rope != 0 && c->rope != 1) return fail(GPT2_EINVAL, "rope must be 0 or 1");
    if (c->attn_recompute != 0 && c->attn_recompute != 1)
        return fail(GPT2_EINVAL, "attn_recompute must be 0 or 1");
    return GPT2_OK;
}

float bf16_bits_to_float(uint16_t h) {
    const uint32_t u = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// IEEE binary16: sign, 5-bit exponent (bias 15), 10-bit fraction; exponent 0
// holds zero and the subnormals (fraction * 2^-24), 31 holds inf and NaN.
float half_bits_to_float(uint16_t h) {
    const int sign = h >> 15, e = (h >> 10) & 31, f = h & 1023;
    float v;
    if (e == 0)
        v = std::ldexp((float)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = std::ldexp((float)(1024 + f), e - 25);
    return sign ? -v : v;
}

void Layout::build(const gpt2_config* c, int cus, bool with_guards) {
    guards = with_guards;
    regions.clear();
    dt = c->precision == GPT2_BF16_MIXED ? DT_BF16 : c->precision == GPT2_F16_MIXED ? DT_F16
                                                                                    : DT_F32;
    half = dt != DT_F32;
    rope = c->rope;
    es = half ? 2 : 4;
    L = c->num_layers;
    C = c->channels;
    NH = c->num_heads;
    V = c->vocab_size;
    Vp = (V + 63) / 64 * 64;
    maxT = c->max_seq_len;
    Bmax = c->batch_size;
    Tmax = c->seq_len;
    M = Bmax * Tmax;
    pos_bits = std::max(1, ceil_log2(M));
    n_pow2 = 1 << ceil_log2(M);
    param_sizes(c, psize);
    nparams = 0;
    for (int i = 0; i < 16; i++) {
        poff[i] = nparams;
        nparams += psize[i];
    }
    size_t off = 0;
    auto take = [&](const char* name, size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        size_t g = 0;
        if (guards) {
            g = off;
            off += kGuardBytes;
        }
        regions.push_back({name, o, bytes, g});
        return o;
    };
    const size_t f = sizeof(float);
    const size_t MC = (size_t)M * C;
    params = take("params", nparams * f);
    grads = take("grads", nparams * f);
    m = take("adam_m", nparams * f);
    v = take("adam_v", nparams * f);
    shadow = half ? take("weights_16bit", nparams * 2) : 0;
    encoded = take("encoded", MC * es);
    ln1 = take("ln1", L * MC * es);
    ln1_mean = take("ln1_mean", (size_t)L * M * f);
    ln1_rstd = take("ln1_rstd", (size_t)L * M * f);
    qkv = take("qkv", L * 3 * MC * es);
    atty = take("atty", L * MC * es);
    lse = take("att_lse", (size_t)L * M * NH * f);
    res2 = take("residual2", L * MC * es);
    ln2 = take("ln2", L * MC * es);
    ln2_mean = take("ln2_mean", (size_t)L * M * f);
    ln2_rstd = take("ln2_rstd", (size_t)L * M * f);
    fch = take("fch", L * 4 * MC * es);
    fch_gelu = take("fch_gelu", L * 4 * MC * es);
    res3 = take("residual3", L * MC * es);
    lnf = take("lnf", MC * es);
    lnf_mean = take("lnf_mean", (size_t)M * f);
    lnf_rstd = take("lnf_rstd", (size_t)M * f);
    logits = take("logits", (size_t)M * Vp * es);
    losses = take("losses", (size_t)M * f);
    dres = take("dresidual", MC * es);
    dtmp = take("dtmp", MC * es);
    dqkv = take("dqkv", 3 * MC * es);
    dfch = take("dfch", 4 * MC * es);
    attn_d = take("att_rowdot", (size_t)M * NH * f);
    ds_stride = 0;
    attn_ds = 0;
    if (!half && !c->attn_recompute &&
        (int64_t)Bmax * NH * gk::attn_ds_stride(Tmax, C / NH) * (int64_t)f <
            gk::kAttnDsMaxBytes) {
        ds_stride = gk::attn_ds_stride(Tmax, C / NH);
        attn_ds = take("att_dsT", (size_t)Bmax * NH * ds_stride * f);
    }
    ln_part = take("ln_partials", gk::layernorm_partials_floats(M, C) * f);
    bias_part = take("bias_partials", gk::bias_partials_floats(M, 4 * C) * f);
    embed_part = take("embed_partials", gk::embed_partials_floats(M, C) * f);
    // the largest split-K workspace over every matmul of the step
    gemm_ws_bytes = 0;
    auto need = [&](int op, int epi, int mm, int n, int k) {
        const size_t b = half ? gk::gemm_bf16_workspace_bytes(op, epi, mm, n, k, cus)
                              : gk::gemm_workspace_bytes(op, epi, mm, n, k, cus);
        gemm_ws_bytes = std::max(gemm_ws_bytes, b);
    };
    const int outs[4][2] = {{3 * C, C}, {C, C}, {4 * C, C}, {C, 4 * C}};
    for (auto& o : outs) need(gk::GEMM_TN, gk::EPI_ACCUM, o[0], o[1], M);
    need(gk::GEMM_TN, gk::EPI_ACCUM, V, C, M);
    for (int k : {C, 3 * C, 4 * C}) {
        need(gk::GEMM_NT, gk::EPI_RESID, M, C, k);
        need(gk::GEMM_NN, gk::EPI_STORE, M, C, k);
    }
    need(gk::GEMM_NT, gk::EPI_STORE, M, 3 * C, C);
    need(gk::GEMM_NN, gk::EPI_STORE, M, C, V);
    gemm_ws = take("gemm_workspace", gemm_ws_bytes);
    keys = take("sort_keys", (size_t)n_pow2 * sizeof(uint32_t));
    tokens = take("tokens", (size_t)M * sizeof(int32_t));
    targets = take("targets", (size_t)M * sizeof(int32_t));
    scalars = take("scalars", 256);
    rope_cs = rope ? take("rope_table", (size_t)Tmax * (C / NH / 2) * 2 * f) : 0;
    total = off;
}

namespace {
constexpr char kCkptMagic[8] = {'G', 'P', 'T', '2', 'C', 'K', 'P', 'T'};
}  // namespace

void ckpt_header_make(CkptHeader* h, int precision, int64_t nparams, int64_t step) {
    std::memset(h, 0, sizeof *h);
    std::memcpy(h->magic, kCkptMagic, 8);
    h->version = kCkptVersion;
    h->precision = (uint32_t)precision;
    h->nparams = nparams;
    h->step = step;
}

int ckpt_header_check(const CkptHeader* h, size_t got, int64_t nparams, const char* path) {
    if (got != sizeof *h || std::memcmp(h->magic, kCkptMagic, 8) != 0 ||
        (h->version != 1 && h->version != 2))
        return fail(GPT2_EINVAL, "%s is not a version-1 or -2 checkpoint", path);
    if (h->precision > (uint32_t)GPT2_F16_MIXED)
        return fail(GPT2_EINVAL, "%s: unknown precision %u", path, h->precision);
    if (h->step < 0) return fail(GPT2_EINVAL, "%s: negative step %lld", path, (long long)h->step);
    if (h->nparams != nparams)
        return fail(GPT2_EINVAL, "checkpoint holds %lld parameters, the model %lld",
                    (long long)h->nparams, (long long)nparams);
    return GPT2_OK;
}

int ckpt_scale_check(const CkptScale* s, size_t got, uint32_t precision, const char* path) {
    if (got != sizeof *s) return fail(GPT2_EINVAL, "%s: truncated loss-scale block", path);
    if (s->zero != 0) return fail(GPT2_EINVAL, "%s: malformed loss-scale block", path);
    if (precision == (uint32_t)GPT2_F16_MIXED &&
        (!(s->scale >= 1.0f && s->scale < INFINITY) || s->good < 0 || s->growth_interval < 1 ||
         s->good >= s->growth_interval))
        return fail(GPT2_EINVAL, "%s: invalid loss-scale state (scale %g, %d of %d)", path,
                    (double)s->scale, s->good, s->growth_interval);
    return GPT2_OK;
}

}  // namespace gh

// ---- host-only entry points of the C ABI ------------------------------------

extern "C" {

const char* gpt2_last_error(void) { return g_err.c_str(); }

int gpt2_validate_config(const gpt2_config* cfg) { return gh::check_config(cfg); }

int64_t gpt2_config_num_parameters(const gpt2_config* cfg) {
    if (gh::check_config(cfg) != GPT2_OK) return -1;
    int64_t s[16], n = 0;
    gh::param_sizes(cfg, s);
    for (int i = 0; i < 16; i++) n += s[i];
    return n;
}

int gpt2_config_param_tensor(const gpt2_config* cfg, int i, const char** name, int64_t* offset,
                             int64_t* numel) {
    const int rc = gh::check_config(cfg);
    if (rc != GPT2_OK) return rc;
    if (i < 0 || i >= 16) return gh::fail(GPT2_EINVAL, "parameter index %d outside 0..15", i);
    int64_t s[16], off = 0;
    gh::param_sizes(cfg, s);
    for (int k = 0; k < i; k++) off += s[k];
    if (name) *name = gh::kParamNames[i];
    if (offset) *offset = off;
    if (numel) *numel = s[i];
    return GPT2_OK;
}

int64_t gpt2_config_device_bytes(const gpt2_config* cfg) {
    if (gh::check_config(cfg) != GPT2_OK) return -1;
    gh::Layout y;
    y.build(cfg, gh::host_cu_count(), false);
    return (int64_t)y.total;
}

}  // extern "C"
