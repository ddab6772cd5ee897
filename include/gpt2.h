/*
 * gpt2.h -- C ABI of the MI355X (gfx950) GPT-2 training-step library.
 *
 * The library follows the problem statement of the llm.c articles:
 *   - all memory is allocated once, up front, as flat 1-D arenas (parameters,
 *     gradients, optimizer moments, activations) and never allocated or freed
 *     while training (yinghuohong.cn article "OpenAI创始大神手搓千行C代码训练GPT",
 *     section "脚动完成每一个层前向/反向流传"; ujoy.net article "徒手用 1000 行
 *     C 语言实现", section "用C语言实现LLM");
 *   - one training step is forward, zero-grad, backward and an Adam(W) update
 *     at lr 1e-4 (ujoy.net, section "训练过程");
 *   - the model is GPT-2 with the config fields that page prints (max_seq_len,
 *     vocab_size, num_layers, num_heads, channels).
 *
 * Conventions.  Every entry point returns 0 (GPT2_OK) or a negative status;
 * gpt2_last_error() then gives a message (thread-local, valid until the next
 * call on the same thread).  All device work is queued on the one HIP stream
 * given at create, in call order.  Host buffers are owned by the caller and
 * may be reused as soon as a call returns.  Device memory is owned by the
 * library: allocated in gpt2_create only, released in gpt2_destroy only.
 *
 * Layouts.  Parameters live in one fp32 arena of 16 tensors in this order:
 * wte (V,C), wpe (maxT,C), ln1w (L,C), ln1b (L,C), qkvw (L,3C,C), qkvb (L,3C),
 * attprojw (L,C,C), attprojb (L,C), ln2w (L,C), ln2b (L,C), fcw (L,4C,C),
 * fcb (L,4C), fcprojw (L,C,4C), fcprojb (L,C), lnfw (C), lnfb (C); linear
 * weights are (out, in) row-major and the LM head is wte itself (tied, no
 * bias).  Gradients and the two Adam moments use the same layout.  Token ids
 * are int32, row-major (B,T); targets likewise.
 */
#ifndef GPT2_H
#define GPT2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GPT2_API __attribute__((visibility("default")))

/* ---- status codes ------------------------------------------------------ */
#define GPT2_OK 0
#define GPT2_EINVAL (-1)  /* bad config, size, name or argument            */
#define GPT2_ERANGE (-2)  /* a token or target id outside [0, vocab_size)   */
#define GPT2_ESTATE (-3)  /* call out of order (backward before a forward
                             with targets)                                  */
#define GPT2_ENOMEM (-4)  /* the allocator returned NULL                    */
#define GPT2_EDEVICE (-5) /* a HIP runtime error (message has its string)   */
#define GPT2_ECORRUPT (-6) /* a debug guard word was overwritten            */

/* ---- precision --------------------------------------------------------- */
#define GPT2_FP32 0       /* everything fp32, fp32 matrix cores            */
#define GPT2_BF16_MIXED 1 /* bf16 activations and matmul inputs (fp32
                             accumulate); fp32 master weights, gradients,
                             Adam state, loss and softmax statistics      */
#define GPT2_F16_MIXED 2  /* as GPT2_BF16_MIXED with IEEE fp16 instead of
                             bf16, and dynamic loss scaling (below)       */

typedef struct gpt2_model gpt2_model; /* opaque */

/* Model shape plus the largest batch the arenas are sized for.  Limits:
 * channels % num_heads == 0 with head size 16, 32 or 64; channels <= 1024;
 * num_layers <= 1024; seq_len <= max_seq_len <= 65536; batch_size*seq_len <=
 * 32768; vocab_size <= 65536; rope and attn_recompute are 0 or 1.
 *
 * rope = 1 replaces the learned position table by a rotary position
 * embedding, the architectural extension the pages name (yinghuohong.cn,
 * section "脚动完成每一个层前向/反向流传": more layers such as RoPE for newer
 * architectures).  Reading (RoFormer, Su et al. 2021): the encoder output is
 * wte[token] alone, and in every layer the q and k slices of each head are
 * rotated after the QKV matmul: the channel pair (2i, 2i+1) of the row at
 * position t turns by t * 10000^(-2i/hs).  The wpe tensor then has 0
 * elements (the other 15 tensors keep their order). */
typedef struct {
    int32_t max_seq_len, vocab_size, num_layers, num_heads, channels;
    int32_t batch_size, seq_len; /* arena sizing, fixed at create */
    int32_t precision;           /* GPT2_FP32, GPT2_BF16_MIXED, GPT2_F16_MIXED */
    int32_t rope;                /* 0: learned position table wpe (GPT-2);
                                    1: rotary position embedding instead */
    int32_t attn_recompute;      /* 0: the fp32 attention backward keeps dS
                                    (and the keys in the dQ product's
                                    operand order) in a workspace of
                                    batch_size * num_heads * 4 * (128^2 *
                                    nb(nb+1)/2 + 1024 * ceil(seq_len/32) *
                                    ceil(hs/32)) bytes, nb = ceil(seq_len /
                                    128), when that is under 2 GiB (480 MiB
                                    for the 124M model at B16 T1024), and
                                    computes dQ from it; 1: no workspace,
                                    the dQ kernel recomputes the scores
                                    (slower).  Results agree to rounding;
                                    each is deterministic. */
} gpt2_config;

/* Optional device allocator.  alloc returns device memory of at least
 * `bytes` bytes, aligned to 256 bytes, or NULL; it is called exactly once,
 * from gpt2_create; free is called once from gpt2_destroy. */
typedef struct {
    void* (*alloc)(size_t bytes, void* ctx);
    void (*free)(void* ptr, void* ctx);
    void* ctx;
} gpt2_allocator;

/* ---- host-only queries (no device needed) -------------------------------*/

/* GPT2_OK if the config is within the limits above, else GPT2_EINVAL. */
GPT2_API int gpt2_validate_config(const gpt2_config* cfg);

/* Number of parameters (124,439,808 for the 124M shape), or -1 if invalid.
 * The count is printed by the C trainer (ujoy.net, section "训练过程"). */
GPT2_API int64_t gpt2_config_num_parameters(const gpt2_config* cfg);

/* Name, element offset and element count of parameter tensor i (0..15). */
GPT2_API int gpt2_config_param_tensor(const gpt2_config* cfg, int i, const char** name,
                             int64_t* offset, int64_t* numel);

/* Bytes of device memory gpt2_create will request for this config. */
GPT2_API int64_t gpt2_config_device_bytes(const gpt2_config* cfg);

/* ---- lifetime ---------------------------------------------------------- */

/* Validates cfg, allocates every arena in one allocation (through alloc, or
 * hipMalloc when alloc is NULL), zeroes parameters, gradients and moments,
 * and binds the model to hip_stream (a hipStream_t; NULL = the null stream).
 * On failure nothing is leaked and *out is NULL. */
GPT2_API int gpt2_create(const gpt2_config* cfg, const gpt2_allocator* alloc,
                void* hip_stream, gpt2_model** out);
GPT2_API void gpt2_destroy(gpt2_model* model);

GPT2_API int64_t gpt2_num_parameters(const gpt2_model* model);
GPT2_API int gpt2_param_tensor(const gpt2_model* model, int i, const char** name,
                      int64_t* offset, int64_t* numel);

/* ---- host <-> device copies (synchronous) -------------------------------*/

/* Exactly one of host_dst / host_src is non-NULL: read or write all
 * parameters (fp32, arena layout).  Writing also refreshes the bf16 weight
 * copies of the mixed-precision model. */
GPT2_API int gpt2_copy_params(gpt2_model* model, float* host_dst, const float* host_src);
GPT2_API int gpt2_copy_grads(gpt2_model* model, float* host_dst);
/* Either pointer may be NULL. */
GPT2_API int gpt2_copy_opt_state(gpt2_model* model, float* host_m, float* host_v);

/* ---- checkpoint ----------------------------------------------------------
 * Save and resume training state: the fp32 parameters, both AdamW moments,
 * the fp16 model's dynamic loss-scale state and the caller's step counter,
 * as one raw file: a 32-byte header {"GPT2CKPT", u32 version 2, u32
 * precision, i64 nparams, i64 step}, a 16-byte block {f32 loss scale, i32
 * clean updates in a row, i32 growth interval, u32 0} (1, 0, 0 for the fp32
 * and bf16 models), then params, m and v as nparams little-endian fp32 each,
 * in arena order.  Both calls wait for the stream and stream the arenas
 * through a host buffer of at most 64 MB.  Loading requires the same
 * parameter count (any precision: master weights are fp32 in every model),
 * refreshes the 16-bit weight copies, restores the loss-scale state when
 * both the file and the model are fp16 (otherwise the model keeps its own),
 * and returns the saved step in *step (may be NULL).  Version-1 files (the
 * 32-byte header directly followed by the arenas) load too.  Errors:
 * GPT2_EINVAL for a NULL model or path, step < 0, an unreadable or foreign
 * file, an unknown precision or an invalid loss-scale block, a
 * parameter-count mismatch (these leave the model untouched), or a
 * truncated or oversized file (found while streaming: the model is then
 * partly overwritten); GPT2_ENOMEM, GPT2_EDEVICE. */
GPT2_API int gpt2_save_checkpoint(gpt2_model* model, const char* path, int64_t step);
GPT2_API int gpt2_load_checkpoint(gpt2_model* model, const char* path, int64_t* step);

/* Copy one activation of the last forward to the host as fp32 (converted from
 * bf16 in the mixed-precision model).  Names: "encoded", "ln1", "ln1_mean",
 * "ln1_rstd", "qkv", "atty", "att_lse", "residual2", "ln2", "ln2_mean",
 * "ln2_rstd", "fch", "fch_gelu", "residual3", "lnf", "lnf_mean", "lnf_rstd",
 * "logits", "losses".  layer is used by the per-layer names and ignored by
 * the others.  Sizes are those of the last forward's (B,T): (B*T, width),
 * except att_lse (B, num_heads, T) and logits (B*T, vocab_size).  After a
 * forward with targets, "logits" holds d(mean loss)/d(logits) instead of the
 * logits (the loss kernel overwrites them in place).  With host_dst NULL only
 * *numel is set. */
GPT2_API int gpt2_copy_activation(gpt2_model* model, const char* name, int layer,
                         float* host_dst, int64_t* numel);

/* ---- the training step ------------------------------------------------- */

/* Forward pass on B <= batch_size sequences of T <= seq_len tokens.
 * tokens: host int32 (B,T), each in [0, vocab_size).  targets: host int32
 * (B,T) or NULL.  With targets, *mean_loss (if mean_loss is non-NULL) gets the
 * mean cross-entropy over the B*T positions (this waits for the stream) and
 * the state needed by gpt2_backward is kept; without targets the logits are
 * kept and *mean_loss is NaN.  Ids are checked on the host: GPT2_ERANGE. */
GPT2_API int gpt2_forward(gpt2_model* model, const int32_t* tokens,
                 const int32_t* targets, int B, int T, float* mean_loss);

/* As gpt2_forward, with tokens / targets already in device memory (the
 * caller keeps them alive until the stream has consumed them).  Ids are
 * checked on the device; a bad id zeroes its row, and the next call that
 * reads the loss (this one, if mean_loss is non-NULL) returns GPT2_ERANGE. */
GPT2_API int gpt2_forward_device(gpt2_model* model, const int32_t* tokens,
                        const int32_t* targets, int B, int T,
                        float* mean_loss);

/* Forward-only evaluation: the mean cross-entropy of B <= batch_size
 * sequences of T <= seq_len host ids against host targets (both (B,T)
 * int32, range-checked on the host: GPT2_ERANGE) into *mean_loss (waits for
 * the stream).  Unlike a training forward it writes no gradient over the
 * logits (the loss kernel only reads them) and keeps no backward state:
 * gpt2_backward afterwards returns GPT2_ESTATE, and the logits stay valid
 * for gpt2_sample.  The pages' loop prints such a "val loss" between
 * training steps (ujoy.net article "徒手用 1000 行 C 语言实现", section
 * "训练过程").  All arguments are required (GPT2_EINVAL if NULL). */
GPT2_API int gpt2_evaluate(gpt2_model* model, const int32_t* tokens, const int32_t* targets,
                           int B, int T, float* mean_loss);

/* One token drawn from the model's next-token distribution at position
 * (b, t) of the last forward, which must have been run without targets or
 * by gpt2_evaluate (a training forward replaces the logits by their
 * gradient): the softmax of
 * that logits row, sampled by the inverse CDF -- the smallest token v with
 * coin < sum_{u <= v} p_u (V - 1 if rounding leaves none).  coin is a
 * uniform draw in [0, 1) supplied by the caller, so callers own the random
 * stream.  The pages' training loop samples text from the model from a
 * leading token 50256 (ujoy.net article "徒手用 1000 行 C 语言实现", section
 * "训练过程": the "generated:" line); sampling from the softmax is the
 * plainest reading.  *token is written on the host; the call synchronizes.
 * Returns GPT2_OK, GPT2_EINVAL (NULL, position outside the last forward's
 * B x T, coin outside [0, 1)) or GPT2_ESTATE (no forward, or the last one
 * had targets). */
GPT2_API int gpt2_sample(gpt2_model* model, int b, int t, float coin, int32_t* token);

/* Autoregressive generation for one sequence: tokens[0 .. prompt_len) is the
 * prompt (host, ids in [0, V)); for t = prompt_len .. n-1 it runs a forward
 * of tokens[0 .. t) (B = 1, T = t, no targets) and writes
 * gpt2_sample(0, t-1, coins[t - prompt_len]) to tokens[t].  coins holds
 * n - prompt_len uniforms in [0, 1).  The first step runs the whole prompt;
 * every later step runs only the newest position, reading the keys and
 * values of the earlier positions from the activations the previous steps
 * left (a key/value cache in the arena), so the logits equal those of a
 * whole forward bit for bit.  Afterwards the activations are those of a
 * forward of tokens[0 .. n-1), except att_lse (scratch here).  Requires
 * 1 <= prompt_len
 * <= n <= seq_len of the config.  Errors as gpt2_forward / gpt2_sample; on
 * error tokens[prompt_len .. n) may be partly written. */
GPT2_API int gpt2_generate(gpt2_model* model, int32_t* tokens, int prompt_len, int n,
                           const float* coins);

/* Clears the parameter gradients (backward accumulates into them). */
GPT2_API int gpt2_zero_grad(gpt2_model* model);

/* Gradient of the mean loss of the last forward, added (+=) into the
 * parameter gradients.  GPT2_ESTATE if the last forward had no targets. */
GPT2_API int gpt2_backward(gpt2_model* model);

/* One AdamW step over the whole flat arena (1-based step, decoupled weight
 * decay applied to every parameter):
 *   m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
 *   p -= lr (m/(1-b1^step) / (sqrt(v/(1-b2^step)) + eps) + weight_decay p). */
GPT2_API int gpt2_update(gpt2_model* model, float lr, float beta1, float beta2,
                float eps, float weight_decay, int step);

/* ---- loss scaling (GPT2_F16_MIXED only) ----------------------------------
 * The pages name lower precision such as fp16 as an extension (yinghuohong.cn,
 * section "脚动完成每一个层前向/反向流传").  fp16's range is narrow, so the
 * fp16 model trains with dynamic loss scaling (Micikevicius et al. 2018, the
 * reading taken here): the loss gradient is multiplied by a scale S, so every
 * activation gradient and the accumulated parameter gradients hold S times
 * their value; gpt2_update first checks the gradients, skips the whole update
 * if any is inf or NaN and then halves S (not below 1), and otherwise divides
 * them by S, updates, and doubles S after growth_interval clean updates in a
 * row.  S starts at 2^16 with growth_interval 2000.  gpt2_copy_grads returns
 * gradients divided by the current S; the "logits" activation after a
 * forward with targets holds S times the logits gradient.  The update-step
 * number passed to gpt2_update is the caller's: a skipped update still
 * consumed its number unless the caller re-uses it. */

/* Sets S (finite, >= 1) and growth_interval (>= 1) and clears the count of
 * clean updates.  GPT2_EINVAL for other models or bad values. */
GPT2_API int gpt2_set_loss_scale(gpt2_model* model, float scale, int growth_interval);
/* Reads S and whether the last gpt2_update was skipped (waits for the
 * stream).  Either pointer may be NULL.  GPT2_EINVAL for other models. */
GPT2_API int gpt2_get_loss_scale(gpt2_model* model, float* scale, int* last_update_skipped);

/* ---- token files ---------------------------------------------------------
 * A token file is a raw stream of little-endian int32 GPT-2 token ids with no
 * header (ujoy.net article "徒手用 1000 行 C 语言实现", section "训练过程":
 * the .bin files the data preparation writes).  A loader cuts batches of B
 * sequences of T tokens from it: from a window of B*T + 1 consecutive ids,
 * tokens = ids [0, B*T) and targets = ids [1, B*T] (row-major (B, T) host
 * arrays; each sequence's targets are its tokens shifted by one).  Successive
 * batches advance by B*T ids; when fewer than B*T + 1 ids remain the
 * position returns to the start of the file.  The loader reads one window
 * per batch; it does not check ids against a vocabulary (gpt2_forward does).
 * Host only: no GPU call. */
typedef struct gpt2_loader gpt2_loader;

/* Opens path for batches of B x T.  Errors: GPT2_EINVAL (NULL, B or T <= 0,
 * B*T > 2^30, unreadable or not a regular file, size not a multiple of 4,
 * fewer than B*T + 1 ids),
 * GPT2_ENOMEM.  The loader owns the open file until gpt2_loader_close. */
GPT2_API int gpt2_loader_open(const char* path, int B, int T, gpt2_loader** out);
/* Ids in the file, and floor(ids / (B*T)) batches per pass (-1 if NULL). */
GPT2_API int64_t gpt2_loader_num_tokens(const gpt2_loader* loader);
GPT2_API int64_t gpt2_loader_num_batches(const gpt2_loader* loader);
/* Writes the next batch into caller-owned host arrays of B*T int32 each. */
GPT2_API int gpt2_loader_next(gpt2_loader* loader, int32_t* tokens, int32_t* targets);
/* Back to the first batch. */
GPT2_API int gpt2_loader_reset(gpt2_loader* loader);
GPT2_API void gpt2_loader_close(gpt2_loader* loader);

/* ---- loss without allocation ------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the loss
 * step that ends gpt2_forward / gpt2_evaluate, on caller-owned device
 * buffers, with no allocation of any kind.  The per-row losses go to a fixed
 * device array of the library (32768 floats, 128 KiB per device, held until
 * the process ends), so N <= 32768.  Every call on a device shares that
 * array: calls that overlap on one device (different streams or threads)
 * race and must be serialized by the caller.
 *
 * logits   device, N rows of ldv elements (fp32, or bf16 / fp16 bits for
 *          GPT2_BF16_MIXED / GPT2_F16_MIXED), V valid columns;
 *          V <= ldv <= 65536, ldv % 4 == 0, the buffer 16-byte aligned.
 * targets  device int32 (N), each in [0, V).
 * grad_scale 0: the logits are only read.  Otherwise they are overwritten by
 *          (softmax(row) - onehot(target)) * grad_scale and columns
 *          V..ldv-1 by 0 (gpt2_forward uses 1/N, the mean's gradient).
 * mean_loss device float: the mean over the rows of lse(row) - row[target].
 * flag     device int32: set to 0, then to 2 if some target is outside
 *          [0, V) (that row then counts 0 loss and gets a 0 gradient).
 * hip_stream the stream everything is queued on (NULL = null stream); the
 *          call does not wait for it.
 * Rows are the same kernels' rows as the model's, so the loss and gradient
 * equal the model's for the same logits, ldv and targets bit for bit.
 * Errors (nothing is launched): GPT2_EINVAL for NULL pointers, N outside
 * 1..32768, bad V / ldv, an unknown precision; GPT2_EDEVICE for a HIP error.
 */
GPT2_API int gpt2_cross_entropy_static(const void* logits, int64_t ldv, const int32_t* targets,
                                       int N, int V, int precision, float grad_scale,
                                       float* mean_loss, int32_t* flag, void* hip_stream);

/* Debug guard words.  With the environment variable GPT2_GUARD_WORDS set
 * (and not "0") when gpt2_create runs, every sub-buffer of the arena is
 * followed by 256 bytes of the word 0xC0DEFACE (the arena grows by 256 bytes
 * per sub-buffer).  The pages stress that in one flat allocation every
 * tensor offset has to line up by hand (yinghuohong.cn, section
 * "脚动完成每一个层前向/反向流传"); the guards catch a kernel that writes
 * past its buffer.  gpt2_check_guards waits for the stream and reads every
 * guard: GPT2_OK, GPT2_ECORRUPT naming the first buffer whose guard changed,
 * or GPT2_EINVAL if the model has no guards. */
GPT2_API int gpt2_check_guards(gpt2_model* model);

/* Waits for the model's stream; reports a pending device-side id error. */
GPT2_API int gpt2_synchronize(gpt2_model* model);

GPT2_API const char* gpt2_last_error(void);

/* ---- per-kernel timing (HIP events on the model's stream) ---------------*/

/* Kernel classes timed when profiling is on. */
#define GPT2_KC_GEMM 0      /* every matmul (forward, dX, dW, split-K sum) */
#define GPT2_KC_ATTENTION 1 /* attention forward and backward             */
#define GPT2_KC_LAYERNORM 2 /* layernorm forward and backward             */
#define GPT2_KC_SOFTMAX_CE 3
#define GPT2_KC_ADAMW 4
#define GPT2_KC_OTHER 5     /* encoder, bias sums, zero-grad, loss mean   */
#define GPT2_KC_COUNT 6

#define GPT2_PROFILE_ALL ((1 << GPT2_KC_COUNT) - 1)

/* class_mask != 0 clears the counters and from now on counts the launches
 * and algorithmic work of every class; the classes whose bit is set in
 * class_mask (bit k = class k; GPT2_PROFILE_ALL for all) are also timed.  A
 * timed call's first kernel dispatch carries a start event and its last one
 * a stop event (hipExtLaunchKernel), so timing adds no packets between
 * kernels, but each timed dispatch still costs about 3 us of issue time.
 * class_mask == 0 stops profiling.  Returns GPT2_EINVAL for bits past the
 * last class. */
GPT2_API int gpt2_profile(gpt2_model* model, int class_mask);

/* Totals since profiling was enabled for one kernel class: summed kernel
 * time (ms, waits for the stream; 0 for an untimed class), number of
 * launches, and the algorithmic work of those launches: floating-point
 * operations and HBM bytes. */
GPT2_API int gpt2_profile_read(gpt2_model* model, int kernel_class, double* total_ms,
                      int64_t* launches, double* flops, double* bytes);

#ifdef __cplusplus
}
#endif
#endif /* GPT2_H */
