// Launch plans of the matmuls and the sizes of the step's scratch buffers:
// host-only arithmetic (no HIP), shared by the kernels' launchers and by the
// arena layout, and built on its own for the host sanitizer checks.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace gk {

// C[m,n] = sum_k A(m,k) B(k,n), row-major with leading dims:
//   NT: A(m,k) = A[m*lda + k], B(k,n) = B[n*ldb + k]   (Y = X W^T, forward)
//   NN: A(m,k) = A[m*lda + k], B(k,n) = B[k*ldb + n]   (dX = dY W)
//   TN: A(m,k) = A[k*lda + m], B(k,n) = B[k*ldb + n]   (dW = dY^T X)
enum GemmOp { GEMM_NT = 0, GEMM_NN = 1, GEMM_TN = 2 };

enum GemmEpi {
    EPI_STORE = 0,     // C = acc (+ bias[n])
    EPI_RESID = 1,     // C = acc + bias[n] + aux[m,n]           (residual add)
    EPI_GELU = 2,      // C = acc + bias[n];  out2 = gelu(C)
    EPI_GELU_BWD = 3,  // C = acc * gelu'(aux[m,n])
    EPI_ACCUM = 4,     // C += acc
};

inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// ---- fp32 matmul (128x128 output tiles; split chunks are whole multiples of
// every reduction step depth the kernel uses) --------------------------------
constexpr int kGemmTile = 128;
constexpr int kGemmSplitStep = 32;

// K per split for `splits` splits.
int gemm_split_chunk(int K, int splits);
// How many ways the reduction over K is split, for a device with `cus`
// compute units.
int gemm_choose_splits(int op, int epi, int M, int N, int K, int cus);
// Workspace bytes (split-K partial sums) the product needs; 0 if unsplit.
size_t gemm_workspace_bytes(int op, int epi, int M, int N, int K, int cus);

// ---- 16-bit matmul -----------------------------------------------------------
constexpr int kGemm16Step = 64;     // the reduction step of the split plan
constexpr int kGemm16BigTile = 256;  // output tile of the large-tile kernel
// Outputs at least this wide keep three reduction steps of loads in flight
// in the 32-deep-step forward and input-gradient products (two otherwise).
constexpr int kGemm16DeepPrefetchN = 16384;

// Which kernel (the 256x256 one: `big`) and how many K splits.
struct PlanH {
    bool big;
    int splits;
};
int gemm16_split_chunk(int K, int splits);
PlanH gemm16_plan(int op, int epi, int M, int N, int K, int64_t lda, int64_t ldb, int cus);
// Workspace bytes for the product when its operands allow the large tile.
size_t gemm_bf16_workspace_bytes(int op, int epi, int M, int N, int K, int cus);

// ---- other scratch -----------------------------------------------------------
// Partial rows of the layernorm backward's parameter sums (dgamma, dbeta and
// one bias) for N rows of C.
size_t layernorm_partials_floats(int N, int C);
// Rows summed by one bias-gradient workgroup, and the partial rows of M.
constexpr int kBiasRows = 64;
size_t bias_partials_floats(int M, int N);

// Keys per chunk of the embedding backward, and its two partial rows per
// chunk of M sorted keys.
constexpr int kEmbedChunk = 16;
inline size_t embed_partials_floats(int M, int C) {
    return (size_t)2 * cdiv(M, kEmbedChunk) * C;
}

// The attention backward's dS workspace, per (sequence, head) of T
// positions and head size hs: the 128 x 128 blocks of dS^T on or below the
// diagonal, then the keys in the dQ product's operand order (one 32-key
// block per 1024 floats and 32 head dimensions).  Kept only while the whole
// workspace stays under kAttnDsMaxBytes (so each (sequence, head) slice is
// addressable with 32-bit byte offsets).
constexpr int kAttnBlock = 128;
constexpr int64_t kAttnDsMaxBytes = (int64_t)2 << 30;
inline int64_t attn_ds_blocks_floats(int T) {
    const int64_t nb = cdiv(T, kAttnBlock);
    return nb * (nb + 1) / 2 * kAttnBlock * kAttnBlock;
}
inline int64_t attn_ds_stride(int T, int hs) {
    return attn_ds_blocks_floats(T) + (int64_t)cdiv(T, 32) * cdiv(hs, 32) * 1024;
}

}  // namespace gk
