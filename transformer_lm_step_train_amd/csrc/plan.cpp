// Launch plans of the matmuls and scratch sizes (see plan.h).  Host only.
#include "plan.h"

#include <algorithm>
#include <cmath>

namespace gk {

int gemm_split_chunk(int K, int splits) {
    const int c = cdiv(K, splits);
    return cdiv(c, kGemmSplitStep) * kGemmSplitStep;
}

// Split the reduction over K when the output tiles alone leave the chip
// idle: weight gradients of the C x C and 4C x C layers (K = B*T, few tiles,
// split so that the workgroups fill about two whole rounds), and long-K
// input-gradient products whose tile count falls between one and two rounds
// of resident workgroups (two splits make whole rounds).  The unit of a
// round is two workgroups per compute unit: the 16-step kernel can hold
// three, but plans sized for three split the weight gradients further and
// measured slower.
int gemm_choose_splits(int op, int epi, int M, int N, int K, int cus) {
    if ((N % 4) != 0) return 1;
    const int tiles = cdiv(M, kGemmTile) * cdiv(N, kGemmTile);
    const int slots = 2 * std::max(cus, 1);
    if (op == GEMM_TN) {
        if (epi != EPI_ACCUM && epi != EPI_STORE) return 1;
        // Many tiles and a long reduction (the LM-head weight gradient,
        // K = B*T): four splits of at least 4096 each measured 11% faster
        // than none (shorter reductions per tile, a fuller last round).
        if (tiles >= 2 * slots) return K >= 4 * 4096 ? 4 : 1;
        // Few tiles, long reduction (the per-layer weight gradients, K =
        // B*T): a split count that is a multiple of 8, so that each XCD
        // takes whole K chunks and the tiles resident on it share their
        // operand chunks through its L2 (split_remap in the kernel): 16, or
        // 32 when the tiles fill under an eighth of the resident slots.  At
        // B*T = 16384 this halves their fetched bytes (QKV 4.8 -> 2.0x the
        // operand bytes, attention projection 4.2 -> 1.3x, fc 4.3 -> 2.0x,
        // fc projection 3.4 -> 1.7x) at the same speed as the best
        // unaligned counts (standalone sweep: -1.8%, -1.0%, -1.3%, +0.7%).
        // Each split keeps at least 4 reduction steps.
        const int max_splits = K / (kGemmSplitStep * 4);
        const int aligned = std::min(tiles * 8 < slots ? 32 : 16, max_splits / 8 * 8);
        if (aligned >= 8) return aligned;
        // Otherwise the smallest split count that fills about two rounds of
        // resident workgroups with little idle tail.
        int best = 1;
        double best_eff = 0.0;
        for (int sp = 2; sp <= max_splits; sp++) {
            const int nz = cdiv(K, gemm_split_chunk(K, sp));
            const double x = (double)tiles * nz / slots;
            if (x > 4.0) break;
            const double eff = x / std::ceil(x);
            if (x >= 1.8 && eff >= 0.9) return sp;
            if (eff > best_eff + 0.02) {
                best_eff = eff;
                best = sp;
            }
        }
        return best;
    }
    // Forward products: never (the fc-proj forward, K = 3072, measured 3%
    // faster unsplit).  Input gradients with a very long K whose tiles fill
    // between one and two rounds (the LM-head dX, K = V): two splits.
    if (op == GEMM_NT || (epi != EPI_STORE && epi != EPI_RESID)) return 1;
    const bool whole_rounds = tiles > slots && tiles < 2 * slots && (2 * tiles) % slots == 0;
    return whole_rounds && K >= 8192 ? 2 : 1;
}

size_t gemm_workspace_bytes(int op, int epi, int M, int N, int K, int cus) {
    const int splits = gemm_choose_splits(op, epi, M, N, K, cus);
    if (splits <= 1) return 0;
    const int nz = cdiv(K, gemm_split_chunk(K, splits));
    return (size_t)nz * M * N * sizeof(float);
}

int gemm16_split_chunk(int K, int splits) {
    return cdiv(cdiv(K, splits), kGemm16Step) * kGemm16Step;
}

// Weight gradients (TN) and input gradients with a very long K (the LM head,
// K = V) take the 256x256 kernel with the split count that minimises (rounds
// of one-per-CU workgroups) x (reduction steps per workgroup) plus the cost
// of the partial sums, each split at least 4 steps; everything else takes
// the 128x128 kernels unsplit.
PlanH gemm16_plan(int op, int epi, int M, int N, int K, int64_t lda, int64_t ldb, int cus) {
    const bool big = (op == GEMM_TN || (op == GEMM_NN && K >= 16384)) && lda % 8 == 0 &&
                     ldb % 8 == 0;
    if (!big) return {false, 1};
    const bool can_split = (N % 4) == 0 && (epi == EPI_ACCUM || epi == EPI_STORE);
    const int tiles = cdiv(M, kGemm16BigTile) * cdiv(N, kGemm16BigTile);
    cus = std::max(cus, 1);
    const int max_splits = can_split ? std::min(32, std::max(1, K / (4 * kGemm16Step))) : 1;
    PlanH best{true, 1};
    double best_t = 1e300;
    for (int sp = 1; sp <= max_splits; sp++) {
        const int chunk = sp > 1 ? gemm16_split_chunk(K, sp) : K;
        const int nz = sp > 1 ? cdiv(K, chunk) : 1;
        if (nz != sp) continue;
        // Each split also writes an M x N fp32 partial that the sum kernel
        // reads back: at about 4 TB/s against about 3.4 us per 256x256x64
        // step, M*N/1.7e6 steps per split.
        const double t = std::ceil((double)tiles * nz / cus) * std::ceil((double)chunk / kGemm16Step) +
                         (sp > 1 ? sp * (double)M * N / 1.7e6 : 0.0);
        if (t < best_t) {
            best_t = t;
            best.splits = sp;
        }
    }
    return best;
}

size_t gemm_bf16_workspace_bytes(int op, int epi, int M, int N, int K, int cus) {
    // the workspace bound assumes the large-tile path is eligible
    const PlanH p = gemm16_plan(op, epi, M, N, K, 8, 8, cus);
    if (!p.big || p.splits <= 1) return 0;
    return (size_t)cdiv(K, gemm16_split_chunk(K, p.splits)) * M * N * sizeof(float);
}

// Upper bound of the backward's workgroup count over every row count up to
// N: at most 1024 (rows per workgroup grow past 4096 rows) and at most
// ceil(N/4).
size_t layernorm_partials_floats(int N, int C) {
    const int nb = std::min(1024, (N + 3) / 4);
    return (size_t)nb * 3 * C;
}

size_t bias_partials_floats(int M, int N) {
    return (size_t)((M + kBiasRows - 1) / kBiasRows) * N;
}

}  // namespace gk
