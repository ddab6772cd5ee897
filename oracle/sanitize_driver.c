/* Test infrastructure: a standalone driver that runs the CPU oracle end to
 * end on small ragged models, for builds under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py compiles it with
 * gcc -fsanitize=address,undefined).  It includes the oracle's single source
 * file, so every static helper is covered too.  Exit status 0 means every
 * call returned and every loss was finite; the sanitizers abort on the first
 * finding. */
#include "gpt2_oracle.c"

#include <stdio.h>

static uint64_t lcg = 0x2545F4914F6CDD1DULL;
static double uniform01(void) {
    lcg = lcg * 6364136223846793005ULL + 1442695040888963407ULL;
    return (double)(lcg >> 11) / 9007199254740992.0;
}

static int run(int rope, int B, int T) {
    OracleConfig cfg = {16, 37, 2, 3, 24, rope}; /* maxT, V, L, NH, C, rope */
    OracleModel* M = oracle_create(&cfg, B, T);
    if (!M) return 1;
    real* p = oracle_params(M);
    for (int64_t i = 0; i < oracle_num_params(M); i++) p[i] = (real)(0.04 * (uniform01() - 0.5));
    int* tok = malloc(sizeof(int) * B * T);
    int* tgt = malloc(sizeof(int) * B * T);
    for (int i = 0; i < B * T; i++) {
        tok[i] = (int)(uniform01() * cfg.vocab_size) % cfg.vocab_size;
        tgt[i] = (int)(uniform01() * cfg.vocab_size) % cfg.vocab_size;
    }
    int bad = 0;
    for (int step = 1; step <= 2; step++) {
        const double loss = oracle_forward(M, tok, tgt);
        if (!isfinite(loss)) bad = 1;
        oracle_zero_grad(M);
        if (oracle_backward(M) != 0) bad = 1;
        oracle_update(M, 1e-3, 0.9, 0.999, 1e-8, 0.01, step);
        printf("rope=%d B=%d T=%d step %d loss %.6f\n", rope, B, T, step, loss);
    }
    if (!isnan(oracle_forward(M, tok, NULL))) bad = 1; /* no targets: NaN */
    oracle_destroy(M);
    free(tok);
    free(tgt);
    return bad;
}

static int run_generate(void) {
    OracleConfig cfg = {16, 37, 2, 3, 24, 0};
    OracleModel* M = oracle_create(&cfg, 1, 12);
    if (!M) return 1;
    real* p = oracle_params(M);
    for (int64_t i = 0; i < oracle_num_params(M); i++) p[i] = (real)(0.04 * (uniform01() - 0.5));
    int tokens[12] = {36};
    double coins[11];
    for (int i = 0; i < 11; i++) coins[i] = uniform01();
    const int rc = oracle_generate(M, tokens, 1, 12, coins);
    for (int i = 0; i < 12; i++)
        if (tokens[i] < 0 || tokens[i] >= cfg.vocab_size) return 1;
    oracle_destroy(M);
    double scale = 65536.0;
    int good = 0;
    oracle_loss_scale_step(&scale, &good, 1, 4, 1.0);
    oracle_loss_scale_step(&scale, &good, 0, 4, 1.0);
    return rc != 0;
}

int main(void) {
    int bad = 0;
    bad |= run(0, 2, 11);
    bad |= run(1, 3, 7);
    bad |= run(0, 1, 16);
    bad |= run_generate();
    printf(bad ? "FAILED\n" : "ok\n");
    return bad;
}
