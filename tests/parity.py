"""Comparison helpers shared by the GPU parity tests.

Tolerance metric (max |a - r| / max |r| per tensor): loss rel 1e-5, logits,
their gradient and every parameter gradient 1e-3, parameters after one AdamW
step 1e-4.

Step 1 of Adam moves each element by lr * g / (|g| + eps), about lr whatever
the size of g.  Its derivative in g is lr * eps / (|g| + eps)^2, up to
lr / eps at g = 0, so a gradient error inside the tensor-wide tolerance
(1e-3 max |g|) can move an element whose own gradient is near zero by far
more than the parameter tolerance.  Such an element's update is not
determined by two correct fp32 implementations.  An element is counted as
undetermined when it misses the parameter tolerance AND either its gradient
differs by more than 1e-3 of its own size, or a gradient error at the
tensor-wide tolerance could move its update past the parameter tolerance.
Those elements are excluded, counted and capped; the update itself is
checked separately and exactly (the oracle's AdamW applied to the GPU's own
gradients).

One slice is undetermined by construction in the learned-position model:
the key bias (the middle C of each layer's 3C QKV bias).  It adds the same
q.b_k to every score of a softmax row, which the softmax ignores, so its
exact gradient is 0 and both sides hold rounding noise there.  (With rotary
embeddings the key bias is rotated by each key's position and its gradient
is not 0.)  It is checked to be noise (below the
gradient tolerance of the QKV bias) and left out of the parameter check and
of the capped count.
"""
import numpy as np

import oracle

PARAM_TOL = 1e-4
GRAD_TOL = 1e-3
# Largest share of the arena, key bias aside, whose step-1 update may be
# undetermined.  Seen at most 3.0e-5 (tiny and ragged configs, a handful of
# elements) and 3.4e-6 (124M at B=4 T=64); the tests print every count.
EXCLUDED_CAP = 1e-4


def rel(a, r):
    a = np.asarray(a, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if r.size == 0:  # the rotary model's empty wpe
        return 0.0
    return float(np.max(np.abs(a - r)) / max(np.max(np.abs(r)), 1e-30))


def split(flat, sizes):
    out, off = {}, 0
    for n in oracle.PARAM_NAMES:
        out[n] = flat[off:off + sizes[n]]
        off += sizes[n]
    return out


def key_bias_mask(qkvb_size, C):
    """True on the key-bias slice of the stacked (L, 3C) QKV bias."""
    m = np.zeros(qkvb_size, dtype=bool).reshape(-1, 3 * C)
    m[:, C:2 * C] = True
    return m.reshape(-1)


def check_params_after_step1(PG, PO, G, R, lr, eps=1e-8, tag="parity", rope=False):
    """PG/PO: per-tensor parameters after one step (GPU, reference); G/R:
    the gradients they were updated with.  Returns the excluded count (key
    bias aside)."""
    excluded = 0
    total = 0
    C = PO["lnfw"].size
    gq = np.abs(np.asarray(R["qkvb"], dtype=np.float64))
    kb = key_bias_mask(PO["qkvb"].size, C) & (not rope)
    noise = max(np.max(np.abs(np.asarray(G["qkvb"])[kb]), initial=0.0),
                np.max(gq[kb], initial=0.0))
    assert noise <= GRAD_TOL * gq.max(), (noise, gq.max())
    for n in oracle.PARAM_NAMES:
        po = np.asarray(PO[n], dtype=np.float64)
        total += po.size
        if po.size == 0:
            continue
        scale = max(float(np.max(np.abs(po))), 1e-30)
        bad = np.abs(np.asarray(PG[n], dtype=np.float64) - po) > PARAM_TOL * scale
        if n == "qkvb":
            total -= int(kb.sum())
            bad &= ~kb
        if not bad.any():
            continue
        g = np.asarray(G[n], dtype=np.float64)
        rr = np.asarray(R[n], dtype=np.float64)
        r = np.abs(rr)
        gtol = GRAD_TOL * max(float(r.max()), 1e-30)
        # the largest move of the update that a gradient error of gtol causes
        sensitive = lr * eps * gtol / (r + eps) ** 2 > PARAM_TOL * scale
        ill = (np.abs(g - rr) > GRAD_TOL * r) | sensitive
        excluded += int(np.sum(bad & ill))
        idx = np.flatnonzero(bad & ~ill)[:5]
        assert idx.size == 0, (n, [(int(i), float(g[i]), float(rr[i]),
                                    float(PG[n][i]), float(PO[n][i])) for i in idx])
    print(f"[{tag}] params: {excluded} of {total} elements "
          f"({excluded / max(total, 1):.2e}) with undetermined step-1 updates excluded "
          f"(key bias aside; its gradient noise {noise:.1e} of max {gq.max():.1e})",
          flush=True)
    assert excluded <= EXCLUDED_CAP * total, (excluded, total)
    return excluded
