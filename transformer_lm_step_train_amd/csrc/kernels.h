// Internal launchers of the gfx950 kernels.  Every launcher queues work on
// the given stream and returns the launch error (hipSuccess on success).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "plan.h"

namespace gk {

// ---- launch-time events ---------------------------------------------------
// While the runtime times a group of launches it sets `start` and `stop`;
// every launch of the group then carries them in its own dispatch (the first
// launch the start event, each launch the stop event, so the last one
// stands), so timing adds no event packets between kernels.  One per host
// thread.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
    int launched = 0;
};
LaunchEvents& launch_events();  // runtime.cpp

// Every kernel of the library is launched through here.
template <class F, class... Args>
inline void launch(F kernel, dim3 grid, dim3 block, uint32_t shm, hipStream_t s, Args... args) {
    LaunchEvents& e = launch_events();
    hipExtLaunchKernelGGL(kernel, grid, block, shm, s, e.start, e.stop, 0, args...);
    e.start = nullptr;
    e.launched++;
}

// ---- matmul ---------------------------------------------------------------
// Operand layouts (GemmOp) and fused epilogues (GemmEpi) are in plan.h.
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
    // EPI_GELU_BWD, optional: colsum[(m / 64) * N + n] = the sum of the stored
    // C[m', n] over the 64 rows m' of that block (cdiv(M, 64) x N floats; the
    // product then runs without a K split).
    float* colsum;
};

// 16-bit variant (mixed precision): A and B are bf16 (f16 = 0) or fp16
// (f16 = 1) bits, accumulation fp32.  C is 16-bit (activations; EPI_STORE
// with out_f32 != 0 writes fp32) or fp32 (EPI_ACCUM: weight gradients).
// bias is fp32, aux and out2 are 16-bit like A.
struct GemmArgsH {
    int op, epi;
    int f16;
    int M, N, K;
    const uint16_t* A;
    int64_t lda;
    const uint16_t* B;
    int64_t ldb;
    void* C;
    int64_t ldc;
    int out_f32;
    const float* bias;
    const uint16_t* aux;
    int64_t ldaux;
    uint16_t* out2;
    float* colsum;  // as in GemmArgs, of C as stored (rounded to 16 bits)
};
hipError_t gemm_bf16(hipStream_t s, const GemmArgsH& a, float* workspace,
                     size_t workspace_bytes);

// The number of compute units the plans are made for (the current device's).
int device_cu_count();
hipError_t gemm(hipStream_t s, const GemmArgs& a, float* workspace,
                size_t workspace_bytes);

// ---- attention ------------------------------------------------------------
// qkv (B*T, 3C) rows [q | k | v], head h = channels [h*hs, (h+1)*hs).
// Forward writes out (B*T, C) and lse (B, NH, T) = log-sum-exp of each
// scaled score row; backward reads dout and writes dqkv (B*T, 3C), using
// dpre (B, NH, T) as scratch for rowsum(dout * out).
// Activations are stored per dt (DT_F32, DT_BF16, DT_F16); lse and D fp32.
// q_first: rows before it are left as they are (their keys and values are
// read, their outputs not recomputed: whole 128-row blocks before it are
// skipped, and rows of its own block are rewritten with the same values).
hipError_t attention_forward(hipStream_t s, void* out, float* lse, const void* qkv, int B,
                             int T, int C, int NH, int dt, int q_first = 0);
// ds_ws (optional, fp32 models): dS workspace of ds_stride floats per
// (sequence, head), ds_stride >= attn_ds_stride(T, C / NH) (plan.h); with it the
// backward keeps dS instead of recomputing the scores for dQ.
hipError_t attention_backward(hipStream_t s, void* dqkv, float* dpre, const void* dout,
                              const void* qkv, const void* out, const float* lse, int B,
                              int T, int C, int NH, int dt, float* ds_ws = nullptr,
                              int64_t ds_stride = 0);
// Mixed-precision attention on the 16-bit matrix cores (all tensors bf16 or
// fp16 bits per dt, lse and D fp32).
hipError_t attention_forward_half(hipStream_t s, uint16_t* out, float* lse, const uint16_t* qkv,
                                  int B, int T, int C, int NH, int dt, int q_first);
hipError_t attention_backward_half(hipStream_t s, uint16_t* dqkv, float* D,
                                   const uint16_t* dout, const uint16_t* qkv,
                                   const uint16_t* out, const float* lse, int B, int T, int C,
                                   int NH, int dt);

// ---- rotary position embedding ---------------------------------------------
// Rotates the q and k slices of qkv (B*T rows of 3C, stored per dt) in
// place, dir = +1 (forward) or -1 (inverse, the backward).  cs: (T_table,
// hs/2) float pairs (cos, sin) of t * 10000^(-2i/hs), T <= T_table.
hipError_t rope_apply(hipStream_t s, void* qkv, const float* cs, int B, int T, int C, int NH,
                      int dir, int dt);

// ---- layernorm ------------------------------------------------------------
// Activations (out, inp, dres, dout) are stored per dt (DT_F32, DT_BF16,
// DT_F16); mean, rstd, weights and their gradients are always fp32.
hipError_t layernorm_forward(hipStream_t s, void* out, float* mean, float* rstd,
                             const void* inp, const float* w, const float* b, int N, int C,
                             int dt);
// dres (+)= dx;  dw += sum dy*xhat, db += sum dy, and when dbias is not
// NULL dbias += the column sums of dres as stored after this call (two
// deterministic stages; `partials` holds layernorm_partials_floats(N, C)
// floats).
hipError_t layernorm_backward(hipStream_t s, void* dres, int accumulate, float* dw, float* db,
                              float* dbias, float* partials, const void* dout, const void* inp,
                              const float* w, const float* mean, const float* rstd, int N,
                              int C, int dt);

// ---- fused softmax + cross-entropy -----------------------------------------
// logits (N, ldv) with V valid columns.  losses[n] = lse - logit[target];
// logits are overwritten by (softmax - onehot) * dscale, columns V..ldv-1 by
// 0; dscale == 0 leaves the logits untouched (loss only).  A target outside [0, V) sets *flag |= 2 and zeroes that row.
// logits fp32, bf16 bits or fp16 per dt (the statistics are fp32).
// gscale (device, NULL = none): the loss scale of the fp16 model, which
// multiplies dscale.
hipError_t softmax_ce(hipStream_t s, void* logits, float* losses,
                      const int32_t* targets, int N, int V, int ldv,
                      float dscale, const float* gscale, int* flag, int dt);
// out[0] = mean of x[0..n) (deterministic order)
// One inverse-CDF draw (coin in [0, 1)) from softmax of one logits row of V
// values; writes the token to out (device).
hipError_t sample_row(hipStream_t s, const void* logits, int V, float coin, int32_t* out,
                      int dt);
hipError_t mean_reduce(hipStream_t s, float* out, const float* x, int n);

// ---- embedding -------------------------------------------------------------
// out[b,t] = wte[tok] + wpe[t]; a token outside [0, V) sets *flag |= 1 and
// gives a zero row.
hipError_t encoder_forward(hipStream_t s, void* out, const int32_t* tok,
                           const float* wte, const float* wpe, int B, int T,
                           int C, int V, int* flag, int dt);
// keys (n_pow2 uint32) sorted ascending: (token << pos_bits) | position.
// encoder_sort_prepare(n_pow2) must run once (per process) before sorts of
// up to n_pow2 keys: it raises the kernel's LDS limit.
hipError_t encoder_sort_prepare(int n_pow2);
hipError_t encoder_sort(hipStream_t s, uint32_t* keys, const int32_t* tok,
                        int n, int V, int pos_bits, int n_pow2);
// dwte[tok] += dx rows (chunks of sorted keys summed in position order, then
// the chunks of each run in order), dwpe[t] += sum_b dx.  ws holds
// embed_partials_floats(B*T, C) floats.
hipError_t encoder_backward(hipStream_t s, float* dwte, float* dwpe, float* ws,
                            const void* dx, const uint32_t* sorted_keys,
                            int B, int T, int C, int V, int pos_bits, int dt);

// ---- reductions and elementwise -------------------------------------------
// db[n] += sum_m dy[m*ld + n]; `partials` holds bias_partials_floats(M, N).
hipError_t bias_grad(hipStream_t s, float* db, float* partials,
                     const void* dy, int M, int N, int64_t ld, int dt);
// Column c of part (nrows x ncols) is summed over rows in a fixed order and
// added to out_k[c - k*split], k = c / split (k <= 2; out2 may be NULL when
// ncols <= 2*split, out1 when ncols <= split).
hipError_t colsum_add(hipStream_t s, float* out0, float* out1, float* out2, int split,
                      const float* part, int nrows, int ncols);
hipError_t fill_zero(hipStream_t s, float* p, int64_t n);
// shadow: optional 16-bit copy of the updated parameters (NULL = none) of
// storage type shadow_dt (DT_BF16 or DT_F16).  Loss scaling (fp16 model):
// gscale (device, NULL = none) divides the gradients; *skip != 0 (device,
// NULL = none) skips the whole sweep.
hipError_t adamw(hipStream_t s, float* p, const float* g, float* m, float* v, void* shadow,
                 int shadow_dt, int64_t n, float lr, float b1, float b2, float eps, float wd,
                 float bc1, float bc2, const float* gscale, const int* skip);
// out[i] = in[i] rounded to the 16-bit type dt (DT_BF16 or DT_F16).
hipError_t to_half(hipStream_t s, void* out, const float* in, int64_t n, int dt);
// *flag = 1 if any g[i] is inf or NaN (flag is only ever set).
hipError_t check_finite(hipStream_t s, const float* g, int64_t n, int* flag);
// One step of dynamic loss scaling (device state, one thread): a non-finite
// step halves *scale (not below min_scale) and sets *skipped; `interval`
// clean steps in a row double it; *found is cleared.
hipError_t loss_scale_update(hipStream_t s, float* scale, int* good, int* found, int* skipped,
                             int interval, float min_scale);

}  // namespace gk
