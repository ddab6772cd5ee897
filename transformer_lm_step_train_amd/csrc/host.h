// Host-only parts of the library (no HIP): the thread's error message, config
// checks, the parameter layout, the byte layout of the one device allocation,
// the 16-bit conversions used by the copies to the host, and the checkpoint
// header.  The runtime builds on these; a sanitizer build drives them alone.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "../../include/gpt2.h"

// Sets the thread's last-error message; returns code.
int gpt2_set_error(int code, const char* msg);

namespace gh {

// printf-style gpt2_set_error.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Compute units the split plans are made for.  Defined by the runtime (the
// current device's count) and by host-only drivers.
int host_cu_count();

extern const char* const kParamNames[16];
enum { P_WTE, P_WPE, P_LN1W, P_LN1B, P_QKVW, P_QKVB, P_ATTPROJW, P_ATTPROJB,
       P_LN2W, P_LN2B, P_FCW, P_FCB, P_FCPROJW, P_FCPROJB, P_LNFW, P_LNFB };

// Element counts of the 16 parameter tensors in arena order.
void param_sizes(const gpt2_config* c, int64_t* s);
int ceil_log2(int64_t n);
// GPT2_OK, or GPT2_EINVAL with a message naming the violated limit.
int check_config(const gpt2_config* c);

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// bf16 is the top half of an fp32; IEEE binary16 widened exactly.
float bf16_bits_to_float(uint16_t h);
float half_bits_to_float(uint16_t h);

// Debug guard words: with guards on, every sub-buffer is followed by
// kGuardBytes of the pattern kGuardWord, which the runtime writes at create
// and checks on request.
constexpr size_t kGuardBytes = 256;
constexpr uint32_t kGuardWord = 0xC0DEFACEu;

// Byte offsets of every sub-buffer inside the one device allocation.
struct Layout {
    int L, C, NH, V, Vp, maxT, Bmax, Tmax, M, pos_bits, n_pow2;
    int dt;     // activation storage: DT_F32, DT_BF16 or DT_F16
    int half;   // 16-bit activations and a 16-bit copy of the matmul weights
    int rope;   // rotary position embedding instead of the wpe table
    size_t es;  // bytes per activation element
    int64_t nparams, poff[16], psize[16];
    size_t params, grads, m, v, shadow;
    size_t encoded, ln1, ln1_mean, ln1_rstd, qkv, atty, lse, res2, ln2, ln2_mean, ln2_rstd, fch,
        fch_gelu, res3, lnf, lnf_mean, lnf_rstd, logits, losses;
    size_t dres, dtmp, dqkv, dfch, attn_d, attn_ds, ln_part, bias_part, embed_part, gemm_ws, keys,
        tokens, targets, scalars, rope_cs;
    int64_t ds_stride;  // floats per (sequence, head) of attn_ds; 0: no dS workspace
    size_t gemm_ws_bytes, total;
    // Every sub-buffer in allocation order: name, offset, bytes and (with
    // guards) the offset of its guard region.
    struct Region {
        const char* name;
        size_t off, bytes, guard;
    };
    std::vector<Region> regions;
    bool guards = false;

    // cus: compute units the matmul split plans (and so the workspace) are
    // sized for.
    void build(const gpt2_config* c, int cus, bool with_guards);
};

// Checkpoint file: a 32-byte header (little-endian); in version 2 the
// 16-byte loss-scale state of the fp16 model follows; then params, m, v.
struct CkptHeader {
    char magic[8];
    uint32_t version, precision;
    int64_t nparams, step;
};
static_assert(sizeof(CkptHeader) == 32, "checkpoint header is 32 bytes");
struct CkptScale {
    float scale;              // the loss scale S (1 for the other models)
    int32_t good;             // clean updates in a row since S last changed
    int32_t growth_interval;  // clean updates that double S (0 for the others)
    uint32_t zero;
};
static_assert(sizeof(CkptScale) == 16, "checkpoint scale block is 16 bytes");
constexpr uint32_t kCkptVersion = 2;
void ckpt_header_make(CkptHeader* h, int precision, int64_t nparams, int64_t step);
// GPT2_OK if `got` bytes were read and they hold a version-1 or -2 header of
// a known precision for nparams parameters; else GPT2_EINVAL naming path.
int ckpt_header_check(const CkptHeader* h, size_t got, int64_t nparams, const char* path);
// GPT2_OK if `got` bytes were read and they hold a scale block that a model of
// the header's precision can resume from; else GPT2_EINVAL naming path.
int ckpt_scale_check(const CkptScale* s, size_t got, uint32_t precision, const char* path);

}  // namespace gh
