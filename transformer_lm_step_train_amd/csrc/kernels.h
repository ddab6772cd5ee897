// Internal launchers of the gfx950 kernels.  Every launcher queues work on
// the given stream and returns the launch error (hipSuccess on success).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gk {

// ---- matmul ---------------------------------------------------------------
// C[m,n] = sum_k A(m,k) B(k,n), all fp32, row-major with leading dims:
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

struct GemmArgs {
    int op, epi;
    int M, N, K;
    const float* A;
    int64_t lda;
    const float* B;
    int64_t ldb;
    float* C;
    int64_t ldc;
    const float* bias;  // EPI_STORE (optional), EPI_RESID, EPI_GELU
    const float* aux;   // EPI_RESID, EPI_GELU_BWD
    int64_t ldaux;
    float* out2;        // EPI_GELU
};

// Workspace bytes a call may need for split-K partial sums.
size_t gemm_workspace_bytes(int op, int epi, int M, int N, int K);
hipError_t gemm(hipStream_t s, const GemmArgs& a, float* workspace,
                size_t workspace_bytes);

// ---- attention ------------------------------------------------------------
// qkv (B*T, 3C) rows [q | k | v], head h = channels [h*hs, (h+1)*hs).
// Forward writes out (B*T, C) and lse (B, NH, T) = log-sum-exp of each
// scaled score row; backward reads dout and writes dqkv (B*T, 3C), using
// dpre (B, NH, T) as scratch for rowsum(dout * out).
hipError_t attention_forward(hipStream_t s, float* out, float* lse,
                             const float* qkv, int B, int T, int C, int NH);
hipError_t attention_backward(hipStream_t s, float* dqkv, float* dpre,
                              const float* dout, const float* qkv,
                              const float* out, const float* lse, int B, int T,
                              int C, int NH);

// ---- layernorm ------------------------------------------------------------
hipError_t layernorm_forward(hipStream_t s, float* out, float* mean,
                             float* rstd, const float* inp, const float* w,
                             const float* b, int N, int C);
// dres (+)= dx;  dw += sum dy*xhat, db += sum dy (two deterministic stages,
// `partials` holds layernorm_partials_floats(N, C) floats).
size_t layernorm_partials_floats(int N, int C);
hipError_t layernorm_backward(hipStream_t s, float* dres, int accumulate,
                              float* dw, float* db, float* partials,
                              const float* dout, const float* inp,
                              const float* w, const float* mean,
                              const float* rstd, int N, int C);

// ---- fused softmax + cross-entropy -----------------------------------------
// logits (N, ldv) with V valid columns.  losses[n] = lse - logit[target];
// logits are overwritten by (softmax - onehot) * dscale, columns V..ldv-1 by
// 0.  A target outside [0, V) sets *flag |= 2 and zeroes that row.
hipError_t softmax_ce(hipStream_t s, float* logits, float* losses,
                      const int32_t* targets, int N, int V, int ldv,
                      float dscale, int* flag);
// out[0] = mean of x[0..n) (deterministic order)
hipError_t mean_reduce(hipStream_t s, float* out, const float* x, int n);

// ---- embedding -------------------------------------------------------------
// out[b,t] = wte[tok] + wpe[t]; a token outside [0, V) sets *flag |= 1 and
// gives a zero row.
hipError_t encoder_forward(hipStream_t s, float* out, const int32_t* tok,
                           const float* wte, const float* wpe, int B, int T,
                           int C, int V, int* flag);
// keys (n_pow2 uint32) sorted ascending: (token << pos_bits) | position.
// encoder_sort_prepare(n_pow2) must run once (per process) before sorts of
// up to n_pow2 keys: it raises the kernel's LDS limit.
hipError_t encoder_sort_prepare(int n_pow2);
hipError_t encoder_sort(hipStream_t s, uint32_t* keys, const int32_t* tok,
                        int n, int V, int pos_bits, int n_pow2);
// dwte[tok] += dx rows (summed in position order), dwpe[t] += sum_b dx.
hipError_t encoder_backward(hipStream_t s, float* dwte, float* dwpe,
                            const float* dx, const uint32_t* sorted_keys,
                            int B, int T, int C, int V, int pos_bits);

// ---- reductions and elementwise -------------------------------------------
// db[n] += sum_m dy[m*ld + n]; `partials` holds bias_partials_floats(M, N).
size_t bias_partials_floats(int M, int N);
hipError_t bias_grad(hipStream_t s, float* db, float* partials,
                     const float* dy, int M, int N, int64_t ld);
// out0[c] += sum_r part[r*ncols + c] for c < split, out1[c-split] likewise
// for c >= split; rows summed in a fixed order.
hipError_t colsum_add(hipStream_t s, float* out0, float* out1, int split, const float* part,
                      int nrows, int ncols);
hipError_t fill_zero(hipStream_t s, float* p, int64_t n);
hipError_t adamw(hipStream_t s, float* p, const float* g, float* m, float* v,
                 int64_t n, float lr, float b1, float b2, float eps, float wd,
                 float bc1, float bc2);

}  // namespace gk
