// Test infrastructure: drives the library's host-only code (host.cpp,
// plan.cpp, loader.cpp) without a GPU, for builds under AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_host_sanitize.py compiles it with
// g++ -fsanitize=address,undefined -fno-sanitize-recover=all).  It checks:
//   - config validation, every rejection branch included;
//   - the parameter layout (contiguous, summing to the count);
//   - the arena layout of many configs, with and without guard regions:
//     every sub-buffer 256-byte aligned, in order, non-overlapping, inside the
//     total, guards between buffers; split-K workspaces cover every plan;
//   - the bf16 / fp16 widening of every 16-bit pattern against the formats'
//     definitions;
//   - checkpoint headers, well-formed and malformed;
//   - the token-file loader on well-formed and malformed files.
// Prints "ok" and exits 0 on success; a failed check prints it and exits 1.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#include <cmath>
#include <string>
#include <vector>

#include "dtype.h"
#include "gpt2.h"
#include "host.h"
#include "plan.h"

int gh::host_cu_count() { return 256; }

static int failures = 0;
#define CHECK(cond)                                                         \
    do {                                                                    \
        if (!(cond)) {                                                      \
            printf("check failed at line %d: %s\n", __LINE__, #cond);       \
            failures++;                                                     \
        }                                                                   \
    } while (0)

static gpt2_config cfg(int L, int C, int NH, int V, int maxT, int B, int T, int prec = 0,
                       int rope = 0) {
    gpt2_config c;
    c.max_seq_len = maxT;
    c.vocab_size = V;
    c.num_layers = L;
    c.num_heads = NH;
    c.channels = C;
    c.batch_size = B;
    c.seq_len = T;
    c.precision = prec;
    c.rope = rope;
    c.attn_recompute = 0;
    return c;
}

static void test_configs() {
    gpt2_config ok = cfg(12, 768, 12, 50257, 1024, 16, 1024);
    CHECK(gpt2_validate_config(&ok) == GPT2_OK);
    CHECK(gpt2_config_num_parameters(&ok) == 124439808);
    CHECK(gpt2_validate_config(nullptr) == GPT2_EINVAL);
    const gpt2_config bad[] = {
        cfg(0, 64, 4, 512, 64, 2, 64),        cfg(2, 64, 5, 512, 64, 2, 64),
        cfg(2, 128, 1, 512, 64, 2, 64),       cfg(2, 2048, 32, 512, 64, 2, 64),
        cfg(2000, 64, 4, 512, 64, 2, 64),     cfg(2, 64, 4, 512, 64, 2, 65),
        cfg(2, 64, 4, 512, 70000, 2, 64),     cfg(2, 64, 4, 512, 1024, 64, 1024),
        cfg(2, 64, 4, 70000, 64, 2, 64),      cfg(2, 64, 4, 512, 64, 2, 64, 3),
        cfg(2, 64, 4, 512, 64, 2, 64, 0, 2),  cfg(2, 64, 4, -1, 64, 2, 64),
        cfg(2, 64, 4, 512, 64, -3, 64),
    };
    gpt2_config rc = cfg(2, 64, 4, 512, 64, 2, 64);
    rc.attn_recompute = 2;
    CHECK(gpt2_validate_config(&rc) == GPT2_EINVAL);
    for (const auto& c : bad) {
        CHECK(gpt2_validate_config(&c) == GPT2_EINVAL);
        CHECK(strlen(gpt2_last_error()) > 0);
        CHECK(gpt2_config_num_parameters(&c) == -1);
        CHECK(gpt2_config_device_bytes(&c) == -1);
    }
    // parameter tensors: contiguous, in arena order, summing to the count
    for (int rope = 0; rope < 2; rope++) {
        gpt2_config c = cfg(3, 96, 3, 1001, 80, 3, 77, 0, rope);
        int64_t off = 0;
        for (int i = 0; i < 16; i++) {
            const char* name = nullptr;
            int64_t o = -1, n = -1;
            CHECK(gpt2_config_param_tensor(&c, i, &name, &o, &n) == GPT2_OK);
            CHECK(name && strcmp(name, gh::kParamNames[i]) == 0);
            CHECK(o == off);
            CHECK(n >= 0);
            if (i == 1) CHECK(n == (rope ? 0 : 80 * 96));
            off += n;
        }
        CHECK(off == gpt2_config_num_parameters(&c));
        CHECK(gpt2_config_param_tensor(&c, 16, nullptr, nullptr, nullptr) == GPT2_EINVAL);
        CHECK(gpt2_config_param_tensor(&c, -1, nullptr, nullptr, nullptr) == GPT2_EINVAL);
    }
}

static void check_layout(const gpt2_config& c, bool guards) {
    gh::Layout y;
    y.build(&c, 256, guards);
    CHECK(!y.regions.empty());
    size_t end = 0;
    for (const auto& r : y.regions) {
        CHECK(r.off % 256 == 0);
        CHECK(r.off >= end);
        size_t stop = gh::align256(r.off + r.bytes);
        if (guards) {
            CHECK(r.guard == stop);
            CHECK(r.guard % 256 == 0);
            stop = r.guard + gh::kGuardBytes;
        } else {
            CHECK(r.guard == 0);
        }
        end = stop;
    }
    CHECK(end == y.total);
    CHECK(y.params == 0 && y.grads >= y.nparams * 4 && y.m > y.grads && y.v > y.m);
    CHECK((y.shadow != 0) == (c.precision != GPT2_FP32));
    CHECK((y.rope_cs != 0) == (c.rope != 0));
    // the dS workspace: fp32 models that keep dS and fit the cap
    const int64_t ds_bytes = (int64_t)y.Bmax * y.NH * gk::attn_ds_stride(y.Tmax, y.C / y.NH) * 4;
    const bool keep = !y.half && c.attn_recompute == 0 && ds_bytes < gk::kAttnDsMaxBytes;
    CHECK((y.ds_stride != 0) == keep);
    if (keep) {
        CHECK(y.ds_stride == gk::attn_ds_stride(y.Tmax, y.C / y.NH));
        for (int T = 1; T <= y.Tmax; T += 37)  // a shorter run fits the same slice
            CHECK(gk::attn_ds_stride(T, y.C / y.NH) <= y.ds_stride);
        bool found = false;
        for (const auto& r : y.regions)
            if (r.off == y.attn_ds) found = r.bytes == (size_t)ds_bytes;
        CHECK(found);
    }
    CHECK(y.n_pow2 >= y.M && y.n_pow2 < 2 * y.M + 2);
    CHECK((1 << y.pos_bits) >= y.M);
    // the workspace covers every split plan of the step's products
    const int M = y.M, C = y.C;
    const int shapes[][5] = {
        {gk::GEMM_TN, gk::EPI_ACCUM, 3 * C, C, M}, {gk::GEMM_TN, gk::EPI_ACCUM, C, C, M},
        {gk::GEMM_TN, gk::EPI_ACCUM, 4 * C, C, M}, {gk::GEMM_TN, gk::EPI_ACCUM, C, 4 * C, M},
        {gk::GEMM_TN, gk::EPI_ACCUM, y.V, C, M},   {gk::GEMM_NN, gk::EPI_STORE, M, C, y.V},
        {gk::GEMM_NN, gk::EPI_STORE, M, C, 4 * C}, {gk::GEMM_NT, gk::EPI_RESID, M, C, 4 * C},
    };
    for (const auto& s : shapes) {
        const size_t need = y.half ? gk::gemm_bf16_workspace_bytes(s[0], s[1], s[2], s[3], s[4], 256)
                                   : gk::gemm_workspace_bytes(s[0], s[1], s[2], s[3], s[4], 256);
        CHECK(need <= y.gemm_ws_bytes);
        if (!y.half) {
            const int sp = gk::gemm_choose_splits(s[0], s[1], s[2], s[3], s[4], 256);
            CHECK(sp >= 1);
            if (sp > 1) {
                const int chunk = gk::gemm_split_chunk(s[4], sp);
                CHECK(chunk % gk::kGemmSplitStep == 0);
                CHECK((int64_t)chunk * gk::cdiv(s[4], chunk) >= s[4]);
            }
        } else {
            const gk::PlanH p = gk::gemm16_plan(s[0], s[1], s[2], s[3], s[4], 8, 8, 256);
            CHECK(p.splits >= 1 && p.splits <= 32);
        }
    }
}

static void test_layouts() {
    for (int guards = 0; guards < 2; guards++)
        for (int prec = 0; prec < 3; prec++)
            for (int rope = 0; rope < 2; rope++) {
                check_layout(cfg(2, 64, 4, 512, 64, 2, 64, prec, rope), guards);
                check_layout(cfg(2, 96, 3, 1001, 80, 3, 77, prec, rope), guards);
                check_layout(cfg(2, 80, 5, 1001, 80, 3, 77, prec, rope), guards);
                check_layout(cfg(2, 64, 4, 512, 64, 512, 64, prec, rope), guards);
                check_layout(cfg(4, 256, 4, 8192, 256, 4, 256, prec, rope), guards);
                check_layout(cfg(12, 768, 12, 50257, 1024, 16, 1024, prec, rope), guards);
                check_layout(cfg(1, 16, 1, 1, 1, 1, 1, prec, rope), guards);
                // dS workspace past its cap (B1 T32768, 4 heads: 8.6 GB)
                check_layout(cfg(1, 64, 4, 512, 32768, 1, 32768, prec, rope), guards);
                gpt2_config r = cfg(2, 96, 3, 1001, 80, 3, 77, prec, rope);
                r.attn_recompute = 1;
                check_layout(r, guards);
            }
    // the byte count the ABI reports is the layout's, with guards off
    gpt2_config c = cfg(12, 768, 12, 50257, 1024, 16, 1024);
    gh::Layout y;
    y.build(&c, 256, false);
    CHECK(gpt2_config_device_bytes(&c) == (int64_t)y.total);
}

static void test_conversions() {
    for (uint32_t h = 0; h < 65536; h++) {
        const float b = gh::bf16_bits_to_float((uint16_t)h);
        uint32_t u;
        memcpy(&u, &b, 4);
        CHECK(u == h << 16);
        const float f = gh::half_bits_to_float((uint16_t)h);
        const int e = (h >> 10) & 31, m = h & 1023;
        const double mag = e == 0 ? std::ldexp((double)m, -24)
                                  : std::ldexp(1.0 + m / 1024.0, e - 15);
        if (e == 31) {
            CHECK(m ? std::isnan(f) : std::isinf(f));
        } else {
            CHECK((double)f == ((h >> 15) ? -mag : mag));
        }
    }
    CHECK(gh::half_bits_to_float(0x3C00) == 1.0f);
    CHECK(gh::half_bits_to_float(0x0001) == std::ldexp(1.0f, -24));
    CHECK(gh::half_bits_to_float(0xFBFF) == -65504.0f);
}

static void test_checkpoint_headers() {
    gh::CkptHeader h;
    gh::ckpt_header_make(&h, GPT2_BF16_MIXED, 124439808, 7);
    CHECK(gh::ckpt_header_check(&h, sizeof h, 124439808, "x") == GPT2_OK);
    CHECK(gh::ckpt_header_check(&h, sizeof h - 1, 124439808, "x") == GPT2_EINVAL);
    CHECK(gh::ckpt_header_check(&h, 0, 124439808, "x") == GPT2_EINVAL);
    CHECK(gh::ckpt_header_check(&h, sizeof h, 124439807, "x") == GPT2_EINVAL);
    gh::CkptHeader b = h;
    b.magic[3] = 'X';
    CHECK(gh::ckpt_header_check(&b, sizeof b, 124439808, "x") == GPT2_EINVAL);
    CHECK(h.version == 2);
    b = h;
    b.version = 1;
    CHECK(gh::ckpt_header_check(&b, sizeof b, 124439808, "x") == GPT2_OK);
    b.version = 3;
    CHECK(gh::ckpt_header_check(&b, sizeof b, 124439808, "x") == GPT2_EINVAL);
    // the loss-scale block
    const gh::CkptScale ok16 = {1024.0f, 1, 2, 0u}, ok32 = {1.0f, 0, 0, 0u};
    CHECK(gh::ckpt_scale_check(&ok16, sizeof ok16, GPT2_F16_MIXED, "x") == GPT2_OK);
    CHECK(gh::ckpt_scale_check(&ok32, sizeof ok32, GPT2_FP32, "x") == GPT2_OK);
    CHECK(gh::ckpt_scale_check(&ok32, sizeof ok32, GPT2_F16_MIXED, "x") == GPT2_EINVAL);
    CHECK(gh::ckpt_scale_check(&ok16, 15, GPT2_F16_MIXED, "x") == GPT2_EINVAL);
    const gh::CkptScale bad_s[] = {{0.5f, 0, 2, 0u}, {INFINITY, 0, 2, 0u}, {NAN, 0, 2, 0u},
                                   {4.0f, -1, 2, 0u}, {4.0f, 2, 2, 0u}, {4.0f, 0, 2, 9u}};
    for (const auto& x : bad_s) CHECK(gh::ckpt_scale_check(&x, sizeof x, GPT2_F16_MIXED, "x") == GPT2_EINVAL);
    b = h;
    b.precision = 9;
    CHECK(gh::ckpt_header_check(&b, sizeof b, 124439808, "x") == GPT2_EINVAL);
    b = h;
    b.step = -1;
    CHECK(gh::ckpt_header_check(&b, sizeof b, 124439808, "x") == GPT2_EINVAL);
    // arbitrary bytes never read past the header
    unsigned char junk[sizeof h];
    for (int t = 0; t < 1000; t++) {
        for (size_t i = 0; i < sizeof junk; i++) junk[i] = (unsigned char)(rand() & 255);
        gh::CkptHeader j;
        memcpy(&j, junk, sizeof j);
        (void)gh::ckpt_header_check(&j, sizeof j, 124439808, "junk");
    }
}

static std::string write_file(const char* dir, const char* name, const void* data, size_t n) {
    std::string p = std::string(dir) + "/" + name;
    FILE* f = fopen(p.c_str(), "wb");
    if (n) fwrite(data, 1, n, f);
    fclose(f);
    return p;
}

static void test_loader(const char* dir) {
    std::vector<int32_t> ids(1001);
    for (size_t i = 0; i < ids.size(); i++) ids[i] = (int32_t)(i * 7 % 50257);
    const std::string good = write_file(dir, "good.bin", ids.data(), ids.size() * 4);
    gpt2_loader* L = nullptr;
    CHECK(gpt2_loader_open(good.c_str(), 4, 25, &L) == GPT2_OK);
    CHECK(gpt2_loader_num_tokens(L) == 1001);
    CHECK(gpt2_loader_num_batches(L) == 10);
    std::vector<int32_t> tok(100), tgt(100);
    for (int b = 0; b < 25; b++) {  // wraps after 10 windows
        CHECK(gpt2_loader_next(L, tok.data(), tgt.data()) == GPT2_OK);
        const int start = (b % 10) * 100;
        for (int i = 0; i < 100; i++) {
            CHECK(tok[i] == ids[start + i]);
            CHECK(tgt[i] == ids[start + i + 1]);
        }
    }
    CHECK(gpt2_loader_reset(L) == GPT2_OK);
    CHECK(gpt2_loader_next(L, tok.data(), tgt.data()) == GPT2_OK && tok[0] == ids[0]);
    CHECK(gpt2_loader_next(L, nullptr, tgt.data()) == GPT2_EINVAL);
    gpt2_loader_close(L);
    gpt2_loader_close(nullptr);
    CHECK(gpt2_loader_num_tokens(nullptr) == -1 && gpt2_loader_num_batches(nullptr) == -1);
    CHECK(gpt2_loader_reset(nullptr) == GPT2_EINVAL);
    // malformed inputs
    const std::string odd = write_file(dir, "odd.bin", ids.data(), 4 * 100 + 3);
    const std::string tiny = write_file(dir, "tiny.bin", ids.data(), 4 * 100);
    const std::string empty = write_file(dir, "empty.bin", nullptr, 0);
    gpt2_loader* X = reinterpret_cast<gpt2_loader*>(0x1);
    CHECK(gpt2_loader_open(odd.c_str(), 2, 10, &X) == GPT2_EINVAL && X == nullptr);
    CHECK(gpt2_loader_open(tiny.c_str(), 4, 25, &X) == GPT2_EINVAL);  // 100 < 4*25+1
    CHECK(gpt2_loader_open(empty.c_str(), 1, 1, &X) == GPT2_EINVAL);
    CHECK(gpt2_loader_open((std::string(dir) + "/missing.bin").c_str(), 1, 1, &X) ==
          GPT2_EINVAL);
    CHECK(gpt2_loader_open(dir, 1, 1, &X) == GPT2_EINVAL && X == nullptr);  // a directory
    CHECK(gpt2_loader_open(good.c_str(), 0, 4, &X) == GPT2_EINVAL);
    CHECK(gpt2_loader_open(good.c_str(), 4, -1, &X) == GPT2_EINVAL);
    CHECK(gpt2_loader_open(good.c_str(), 1 << 16, 1 << 16, &X) == GPT2_EINVAL);
    CHECK(gpt2_loader_open(nullptr, 1, 1, &X) == GPT2_EINVAL);
    CHECK(gpt2_loader_open(good.c_str(), 1, 1, nullptr) == GPT2_EINVAL);
    // exactly one window: B*T + 1 ids
    const std::string one = write_file(dir, "one.bin", ids.data(), 4 * 101);
    CHECK(gpt2_loader_open(one.c_str(), 4, 25, &L) == GPT2_OK);
    CHECK(gpt2_loader_num_batches(L) == 1);
    for (int b = 0; b < 3; b++) CHECK(gpt2_loader_next(L, tok.data(), tgt.data()) == GPT2_OK);
    CHECK(tgt[99] == ids[100]);
    gpt2_loader_close(L);
    // a file that shrinks under an open loader: the read fails cleanly
    CHECK(gpt2_loader_open(good.c_str(), 4, 25, &L) == GPT2_OK);
    CHECK(truncate(good.c_str(), 4 * 50) == 0);
    CHECK(gpt2_loader_next(L, tok.data(), tgt.data()) == GPT2_EINVAL);
    gpt2_loader_close(L);
}

int main(int argc, char** argv) {
    const char* dir = argc > 1 ? argv[1] : ".";
    test_configs();
    test_layouts();
    test_conversions();
    test_checkpoint_headers();
    test_loader(dir);
    if (failures) {
        printf("%d checks failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
