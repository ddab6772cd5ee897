"""Seeded synthetic inputs shared by the HIP path and by the tests' oracle.

This module holds no arithmetic of the training step: only the random number
generator and the recipes that turn it into weights and token ids.

Generator: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), used counter-style: draw i of a stream with
seed s is mix(s + (i+1) * 0x9E3779B97F4A7C15), so any slice can be produced
independently of the others.  Uniforms take the top 53 bits; normals come from
the Box-Muller transform of uniform pairs (2p, 2p+1); bounded integers use the
multiply-shift map (u32 * n) >> 32 (Lemire 2019).

Weights follow the GPT-2 initialisation: N(0, 0.02) for the embeddings and the
QKV / fc weights, N(0, 0.02/sqrt(2L)) for the two residual projections,
layernorm gain 1 and shift 0, every bias 0.
"""
import math

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

PARAM_SEED = 1337
TOKEN_SEED = 42
COIN_SEED = 7

PARAM_NAMES = ["wte", "wpe", "ln1w", "ln1b", "qkvw", "qkvb", "attprojw",
               "attprojb", "ln2w", "ln2b", "fcw", "fcb", "fcprojw", "fcprojb",
               "lnfw", "lnfb"]


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Draws start .. start+count-1 of the SplitMix64 stream `seed` (uint64)."""
    with np.errstate(over="ignore"):
        idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = np.uint64(seed % (1 << 64)) + idx * GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform01(seed: int, start: int, count: int) -> np.ndarray:
    """Uniform float64 in [0, 1) from the top 53 bits of each draw."""
    z = splitmix64(seed, start, count)
    return (z >> np.uint64(11)).astype(np.float64) * (1.0 / (1 << 53))


def normals(seed: int, start: int, count: int) -> np.ndarray:
    """Standard normals n[start .. start+count-1]; n[2p], n[2p+1] are the
    cosine and sine outputs of Box-Muller on uniforms (2p, 2p+1)."""
    if count == 0:
        return np.zeros(0)
    p0 = start // 2
    p1 = (start + count + 1) // 2
    u = uniform01(seed, 2 * p0, 2 * (p1 - p0)).reshape(-1, 2)
    r = np.sqrt(-2.0 * np.log1p(-u[:, 0]))  # 1 - u in (0, 1]
    th = 2.0 * math.pi * u[:, 1]
    out = np.empty((p1 - p0) * 2)
    out[0::2] = r * np.cos(th)
    out[1::2] = r * np.sin(th)
    off = start - 2 * p0
    return out[off:off + count]


def randint(seed: int, start: int, count: int, n: int) -> np.ndarray:
    """Integers uniform on [0, n) by multiply-shift of the top 32 bits."""
    z = splitmix64(seed, start, count) >> np.uint64(32)
    return ((z * np.uint64(n)) >> np.uint64(32)).astype(np.int32)


def param_sizes(L, C, V, maxT, rope=False):
    """Element count of each of the 16 parameter tensors, arena order (the
    rotary model has no position table: wpe has 0 elements)."""
    return {
        "wte": V * C, "wpe": 0 if rope else maxT * C, "ln1w": L * C, "ln1b": L * C,
        "qkvw": L * 3 * C * C, "qkvb": L * 3 * C, "attprojw": L * C * C,
        "attprojb": L * C, "ln2w": L * C, "ln2b": L * C, "fcw": L * 4 * C * C,
        "fcb": L * 4 * C, "fcprojw": L * C * 4 * C, "fcprojb": L * C,
        "lnfw": C, "lnfb": C,
    }


def init_params(L, C, V, maxT, seed=PARAM_SEED, dtype=np.float32,
                chunk=1 << 23, rope=False) -> np.ndarray:
    """The flat parameter arena, GPT-2 initialisation.  Element j of a
    normally-initialised tensor is normal number (arena offset of j)."""
    sizes = param_sizes(L, C, V, maxT, rope)
    total = sum(sizes.values())
    out = np.empty(total, dtype=dtype)
    resid_std = 0.02 / math.sqrt(2 * L)
    off = 0
    for name in PARAM_NAMES:
        n = sizes[name]
        if name in ("ln1w", "ln2w", "lnfw"):
            out[off:off + n] = 1
        elif name in ("wte", "wpe", "qkvw", "fcw", "attprojw", "fcprojw"):
            std = resid_std if name in ("attprojw", "fcprojw") else 0.02
            for s in range(0, n, chunk):
                e = min(n, s + chunk)
                out[off + s:off + e] = std * normals(seed, off + s, e - s)
        else:
            out[off:off + n] = 0
        off += n
    return out


def token_stream(B, T, V, seed=TOKEN_SEED):
    """tokens (B,T) and targets (B,T), targets = tokens shifted by one along
    one contiguous stream of B*T+1 uniform ids."""
    s = randint(seed, 0, B * T + 1, V)
    return s[:B * T].reshape(B, T).copy(), s[1:].reshape(B, T).copy()


def zipf_tokens(B, T, V, a=1.1, seed=TOKEN_SEED):
    """Ids with a Zipf(a) law over [0, V) (rank r has weight 1/(r+1)^a),
    by inverse CDF; many repeats, to stress the embedding scatter-add."""
    w = 1.0 / np.arange(1, V + 1, dtype=np.float64) ** a
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = uniform01(seed, 0, B * T + 1)
    s = np.minimum(np.searchsorted(cdf, u, side="right"), V - 1).astype(np.int32)
    return s[:B * T].reshape(B, T).copy(), s[1:].reshape(B, T).copy()


# The five workloads.  `steps` is how many consecutive training steps the
# workload runs on its one fixed batch.
def coins(count: int, seed: int = COIN_SEED) -> np.ndarray:
    """Uniform float32 draws in [0, 1) for sampling (float32 so that both
    sides see the same values)."""
    u = uniform01(seed, 0, count).astype(np.float32)
    return np.minimum(u, np.float32(1.0) - np.finfo(np.float32).epsneg)


CONFIGS = {
    "tiny": dict(L=2, C=64, NH=4, V=512, maxT=64, B=2, T=64, steps=1),
    "small": dict(L=4, C=256, NH=4, V=8192, maxT=256, B=4, T=256, steps=10),
    "gpt2_124m_b4t64": dict(L=12, C=768, NH=12, V=50257, maxT=1024, B=4, T=64,
                            steps=1),
    "gpt2_124m_b16t1024": dict(L=12, C=768, NH=12, V=50257, maxT=1024, B=16,
                               T=1024, steps=1),
    # ragged: odd vocab, odd T, non-power-of-two width; exercises every tail
    "ragged": dict(L=2, C=96, NH=3, V=1001, maxT=80, B=3, T=77, steps=1),
    # width 80 (head size 16): every matmul reduction length (80, 240, 320)
    # leaves a partial 32-deep step
    "ragged80": dict(L=2, C=80, NH=5, V=1001, maxT=80, B=3, T=77, steps=1),
    # rotary position embedding instead of the wpe table
    "tiny_rope": dict(L=2, C=64, NH=4, V=512, maxT=64, B=2, T=64, steps=1, rope=True),
    "ragged_rope": dict(L=2, C=96, NH=3, V=1001, maxT=80, B=3, T=77, steps=1, rope=True),
    # a vocabulary past 51200 columns (the widest softmax rows, up to 65536)
    "wide_vocab": dict(L=1, C=64, NH=4, V=60001, maxT=32, B=2, T=24, steps=1),
    # sequences past 1024 positions: nine 128-row query blocks, a ragged last
    "tiny_long": dict(L=2, C=64, NH=4, V=512, maxT=1152, B=1, T=1100, steps=1),
    # width 704 (3C = 2112 and 4C = 2816 outputs, reductions of 2112 and 2816)
    # with B*T = 231 rows: the 16-bit forward and input-gradient products of
    # the wide layers on ragged row and column tiles
    "ragged704": dict(L=1, C=704, NH=11, V=1001, maxT=80, B=3, T=77, steps=1),
}

ADAMW = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
