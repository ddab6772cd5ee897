"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: numbers the
pages print, closed forms, invariants, library routines (numpy, scipy, torch
float64 autograd and optim.AdamW) and central finite differences on the
float64 build.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import OracleModel, lib, ptr
from transformer_lm_step_train_amd import synth

from torch_ref import step as torch_step

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(0)


def rel(a, r):
    a = np.asarray(a, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    return float(np.max(np.abs(a - r)) / max(np.max(np.abs(r)), 1e-300))


def make_model(name, precision="f32", params=None):
    c = synth.CONFIGS[name]
    rope = c.get("rope", False)
    m = OracleModel(c["L"], c["C"], c["NH"], c["V"], c["maxT"], c["B"], c["T"],
                    precision=precision, rope=rope)
    if params is None:
        params = synth.init_params(c["L"], c["C"], c["V"], c["maxT"], rope=rope)
    m.params[:] = params
    return m, c


# ---------------------------------------------------------------- printouts --

def test_page_printout_counts():
    g = json.load(open(os.path.join(GOLDEN, "gpt2_124m_printout.json")))
    cfg = g["config"]
    args = (cfg["num_layers"], cfg["channels"], cfg["num_heads"],
            cfg["vocab_size"], cfg["max_seq_len"])
    _, nparams = oracle.param_sizes(*args)
    assert nparams == g["num_parameters"]
    # B*T = 256 from the printed batch counts ...
    bt = [n for n in range(1, 4097)
          if g["train_tokens"] // n == g["train_num_batches"]
          and g["val_tokens"] // n == g["val_num_batches"]
          and g["val_tokens"] % n == 0]
    assert bt == [256]
    # ... and the activation count then singles out B=4, T=64
    hits = [(B, T) for T in range(1, 1025) for B in range(1, 65)
            if oracle.act_sizes(*args, B, T)[1] == g["num_activations"]]
    assert hits == [(4, 64)]


def test_param_counts_other_configs():
    # closed form V*C + maxT*C + L*(12 C^2 + 13 C) + 2 C
    for name, want in (("tiny", 136960), ("small", 5322240)):
        c = synth.CONFIGS[name]
        _, n = oracle.param_sizes(c["L"], c["C"], c["NH"], c["V"], c["maxT"])
        assert n == want
        L, C, V, T = c["L"], c["C"], c["V"], c["maxT"]
        assert n == V * C + T * C + L * (12 * C * C + 13 * C) + 2 * C
        assert n == sum(synth.param_sizes(L, C, V, T).values())


# ------------------------------------------------------------------ layers --

def test_encoder_bruteforce_and_zero_wte():
    L64 = lib("f64")
    B, T, C, V = 3, 5, 8, 11
    tok = rng.integers(0, V, (B, T)).astype(np.int32)
    wte = rng.standard_normal((V, C))
    wpe = rng.standard_normal((T, C))
    out = np.zeros((B, T, C))
    L64.oracle_encoder_forward(ptr(out), ptr(tok), ptr(wte), ptr(wpe), B, T, C)
    for b in range(B):
        for t in range(T):
            assert np.array_equal(out[b, t], wte[tok[b, t]] + wpe[t])
    L64.oracle_encoder_forward(ptr(out), ptr(tok), ptr(np.zeros_like(wte)),
                               ptr(wpe), B, T, C)
    assert np.array_equal(out, np.broadcast_to(wpe, (B, T, C)))
    # backward: per-row scatter with repeats == np.add.at
    tok[:] = 3  # every position collides
    tok[0, 0] = 7
    d = rng.standard_normal((B, T, C))
    dwte = np.zeros((V, C))
    dwpe = np.zeros((T, C))
    L64.oracle_encoder_backward(ptr(dwte), ptr(dwpe), ptr(d), ptr(tok), B, T, C)
    ref = np.zeros((V, C))
    np.add.at(ref, tok.reshape(-1), d.reshape(-1, C))
    assert np.allclose(dwte, ref, rtol=1e-14, atol=1e-14)
    assert np.allclose(dwpe, d.sum(0), rtol=1e-14, atol=1e-14)


def test_layernorm_moments_and_torch():
    L64 = lib("f64")
    N, C = 17, 48
    x = rng.standard_normal((N, C)) * 3 + 1.5
    w, b = np.ones(C), np.zeros(C)
    y, mu, rs = np.zeros((N, C)), np.zeros(N), np.zeros(N)
    L64.oracle_layernorm_forward(ptr(y), ptr(mu), ptr(rs), ptr(x), ptr(w),
                                 ptr(b), N, C)
    var = x.var(axis=1)
    assert np.allclose(y.mean(1), 0, atol=1e-13)
    assert np.allclose(y.var(1), var / (var + 1e-5), rtol=1e-12)
    # with an affine map, against torch's layer_norm and its autograd
    w = rng.standard_normal(C)
    b = rng.standard_normal(C)
    L64.oracle_layernorm_forward(ptr(y), ptr(mu), ptr(rs), ptr(x), ptr(w),
                                 ptr(b), N, C)
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    bt = torch.tensor(b, requires_grad=True)
    yt = torch.nn.functional.layer_norm(xt, (C,), wt, bt, eps=1e-5)
    assert rel(y, yt.detach().numpy()) < 1e-13
    dy = rng.standard_normal((N, C))
    yt.backward(torch.tensor(dy))
    dx, dw, db = np.zeros((N, C)), np.zeros(C), np.zeros(C)
    L64.oracle_layernorm_backward(ptr(dx), ptr(dw), ptr(db), ptr(dy), ptr(x),
                                  ptr(w), ptr(mu), ptr(rs), N, C)
    assert rel(dx, xt.grad.numpy()) < 1e-12
    assert rel(dw, wt.grad.numpy()) < 1e-12
    assert rel(db, bt.grad.numpy()) < 1e-12


def test_matmul_vs_numpy():
    L64 = lib("f64")
    N, C, OC = 13, 24, 40
    x = rng.standard_normal((N, C))
    w = rng.standard_normal((OC, C))
    b = rng.standard_normal(OC)
    y = np.zeros((N, OC))
    L64.oracle_matmul_forward(ptr(y), ptr(x), ptr(w), ptr(b), N, C, OC)
    assert rel(y, x @ w.T + b) < 1e-13
    L64.oracle_matmul_forward(ptr(y), ptr(x), ptr(w), None, N, C, OC)
    assert rel(y, x @ w.T) < 1e-13
    dy = rng.standard_normal((N, OC))
    dx = np.full((N, C), 0.5)
    dw = np.full((OC, C), -0.25)
    db = np.full(OC, 2.0)
    L64.oracle_matmul_backward(ptr(dx), ptr(dw), ptr(db), ptr(dy), ptr(x),
                               ptr(w), N, C, OC)
    assert rel(dx, 0.5 + dy @ w) < 1e-13          # accumulates
    assert rel(dw, -0.25 + dy.T @ x) < 1e-13
    assert rel(db, 2.0 + dy.sum(0)) < 1e-13


def _attention(B, T, C, NH, qkv):
    L64 = lib("f64")
    out = np.zeros((B, T, C))
    pre = np.zeros((B, NH, T, T))
    att = np.zeros((B, NH, T, T))
    L64.oracle_attention_forward(ptr(out), ptr(pre), ptr(att), ptr(qkv), B, T,
                                 C, NH)
    return out, pre, att


def test_attention_invariants_and_torch():
    B, T, C, NH = 2, 9, 24, 3
    hs = C // NH
    qkv = rng.standard_normal((B, T, 3 * C))
    out, pre, att = _attention(B, T, C, NH, qkv)
    v = qkv[:, :, 2 * C:]
    # row t=0 sees only key 0: output is v_0 exactly
    assert np.array_equal(out[:, 0], v[:, 0])
    # rows sum to one, nothing above the diagonal
    assert np.allclose(att.sum(-1), 1, atol=1e-14)
    assert np.all(att[..., np.triu_indices(T, 1)[0], np.triu_indices(T, 1)[1]] == 0)
    # T = 1: output equals v
    o1, _, _ = _attention(B, 1, C, NH, qkv[:, :1].copy())
    assert np.array_equal(o1, v[:, :1])
    # torch scaled_dot_product_attention (causal), forward and backward
    qkv_t = torch.tensor(qkv, requires_grad=True)
    q, k, vv = qkv_t.split(C, -1)
    sh = lambda z: z.reshape(B, T, NH, hs).transpose(1, 2)
    y = torch.nn.functional.scaled_dot_product_attention(sh(q), sh(k), sh(vv),
                                                         is_causal=True)
    y = y.transpose(1, 2).reshape(B, T, C)
    assert rel(out, y.detach().numpy()) < 1e-12
    dy = rng.standard_normal((B, T, C))
    y.backward(torch.tensor(dy))
    L64 = lib("f64")
    dqkv = np.zeros((B, T, 3 * C))
    dpre = np.zeros((B, NH, T, T))
    datt = np.zeros((B, NH, T, T))
    L64.oracle_attention_backward(ptr(dqkv), ptr(dpre), ptr(datt), ptr(dy),
                                  ptr(qkv), ptr(att), B, T, C, NH)
    assert rel(dqkv, qkv_t.grad.numpy()) < 1e-12


def test_gelu_closed_form_and_fd():
    L64 = lib("f64")
    x = np.concatenate([np.linspace(-6, 6, 1001), [0.0]])
    y = np.zeros_like(x)
    L64.oracle_gelu_forward(ptr(y), ptr(x), x.size)
    ref = torch.nn.functional.gelu(torch.tensor(x), approximate="tanh").numpy()
    assert rel(y, ref) < 1e-14
    assert y[-1] == 0.0
    d = np.zeros_like(x)
    L64.oracle_gelu_backward(ptr(d), ptr(x), ptr(np.ones_like(x)), x.size)
    assert d[-1] == 0.5
    h = 1e-6
    yp, ym = np.zeros_like(x), np.zeros_like(x)
    L64.oracle_gelu_forward(ptr(yp), ptr(x + h), x.size)
    L64.oracle_gelu_forward(ptr(ym), ptr(x - h), x.size)
    assert np.max(np.abs(d - (yp - ym) / (2 * h))) < 1e-8


def test_softmax_crossentropy():
    from scipy.special import log_softmax, softmax
    L64 = lib("f64")
    N, V = 7, 33
    z = rng.standard_normal((N, V)) * 4
    p = np.zeros((N, V))
    L64.oracle_softmax_forward(ptr(p), ptr(z), N, V)
    assert np.allclose(p.sum(1), 1, atol=1e-14)
    assert rel(p, softmax(z, axis=1)) < 1e-13
    tgt = rng.integers(0, V, N).astype(np.int32)
    loss = np.zeros(N)
    L64.oracle_crossentropy_forward(ptr(loss), ptr(p), ptr(tgt), N, V)
    assert rel(loss, -log_softmax(z, 1)[np.arange(N), tgt]) < 1e-12
    # uniform logits: loss = ln V
    L64.oracle_softmax_forward(ptr(p), ptr(np.zeros((N, V))), N, V)
    L64.oracle_crossentropy_forward(ptr(loss), ptr(p), ptr(tgt), N, V)
    assert np.allclose(loss, math.log(V), rtol=1e-14)
    dz = np.zeros((N, V))
    dl = np.full(N, 1.0 / N)
    L64.oracle_crossentropy_softmax_backward(ptr(dz), ptr(dl), ptr(p), ptr(tgt),
                                             N, V)
    onehot = np.eye(V)[tgt]
    assert np.allclose(dz, (1.0 / V - onehot) / N, atol=1e-16)


def test_adamw_first_step_closed_form_and_torch():
    L64 = lib("f64")
    n = 1000
    g = rng.standard_normal(n) * np.logspace(-9, 1, n)
    p = rng.standard_normal(n)
    p0 = p.copy()
    m, v = np.zeros(n), np.zeros(n)
    lr, eps = 1e-4, 1e-8
    L64.oracle_adamw(ptr(p), ptr(g), ptr(m), ptr(v), n, lr, 0.9, 0.999, eps, 0.0, 1)
    assert rel(p - p0, -lr * g / (np.abs(g) + eps)) < 1e-9
    # several steps with weight decay, against torch.optim.AdamW
    p = p0.copy()
    m, v = np.zeros(n), np.zeros(n)
    pt = torch.tensor(p0.copy(), requires_grad=True)
    opt = torch.optim.AdamW([pt], lr=1e-3, betas=(0.8, 0.95), eps=1e-6,
                            weight_decay=0.1)
    for s in range(1, 6):
        gs = rng.standard_normal(n)
        L64.oracle_adamw(ptr(p), ptr(gs), ptr(m), ptr(v), n, 1e-3, 0.8, 0.95,
                         1e-6, 0.1, s)
        pt.grad = torch.tensor(gs)
        opt.step()
    assert rel(p - p0, pt.detach().numpy() - p0) < 1e-10


# ------------------------------------------------------------- whole model --

def test_zero_wte_loss_is_lnV_and_dwte_closed_form():
    for name in ("tiny", "ragged"):
        params = None
        m, c = make_model(name, "f64")
        m.param("wte")[:] = 0
        tok, tgt = synth.token_stream(c["B"], c["T"], c["V"])
        loss = m.forward(tok, tgt)
        assert abs(loss - math.log(c["V"])) < 1e-12
        assert np.all(m.act("logits") == 0)
        m.zero_grad()
        m.backward()
        M, V, C = c["B"] * c["T"], c["V"], c["C"]
        for n in oracle.PARAM_NAMES:
            if n != "wte":
                assert np.all(m.grad(n) == 0), n
        lnf = m.act("lnf").reshape(M, C)
        onehot = np.eye(V)[tgt.reshape(-1)]
        want = (1.0 / V - onehot).T @ lnf / M
        assert rel(m.grad("wte").reshape(V, C), want) < 1e-12
        m.close()


@pytest.mark.parametrize("name", ["tiny", "ragged"])
def test_whole_step_vs_torch_autograd(name):
    """Loss, logits, all 16 gradients and the AdamW update against torch
    float64 autograd + optim.AdamW on the same weights and tokens."""
    m, c = make_model(name, "f64")
    p0 = m.params.copy()
    tok, tgt = synth.token_stream(c["B"], c["T"], c["V"])
    loss = m.forward(tok, tgt)
    m.zero_grad()
    m.backward()
    m.update(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=1)
    losses, logits, grads, p1 = torch_step(
        p0, tok, tgt, c["L"], c["C"], c["NH"], c["V"], c["maxT"], lr=1e-3,
        weight_decay=0.01)
    assert abs(loss - losses[0]) / losses[0] < 1e-13
    assert rel(m.act("logits"), logits.reshape(-1)) < 1e-12
    off = 0
    for n in oracle.PARAM_NAMES:
        sz = m.param_sizes[n]
        if n == "wpe":  # rows >= T get no gradient in either
            pass
        assert rel(m.grad(n), grads[off:off + sz]) < 1e-10, n
        off += sz
    assert rel(m.params - p0, p1 - p0) < 1e-9
    m.close()


@pytest.mark.parametrize("name", ["tiny", "tiny_rope"])
def test_finite_differences_f64(name):
    """Central differences (L(th+h) - L(th-h)) / 2h on the float64 build."""
    m, c = make_model(name, "f64")
    tok, tgt = synth.token_stream(c["B"], c["T"], c["V"])
    m.forward(tok, tgt)
    m.zero_grad()
    m.backward()
    g = m.grads.copy()
    sizes = m.param_sizes
    offs = np.cumsum([0] + [sizes[n] for n in oracle.PARAM_NAMES])
    idx = []
    r = np.random.default_rng(1)
    for i, n in enumerate(oracle.PARAM_NAMES):
        lo, hi = offs[i], offs[i + 1]
        if n in ("lnfw", "lnfb"):
            idx += list(range(lo, hi))
        else:
            if n == "wpe":  # only rows t < T are used (none in the rotary model)
                hi = lo + min(c["T"] * c["C"], hi - lo)
                if hi <= lo:
                    continue
            if n == "wte":  # bias the sample toward rows that occur as tokens
                rows = np.unique(tok.reshape(-1))[:8]
                idx += [lo + int(rr) * c["C"] + int(cc) for rr in rows
                        for cc in r.integers(0, c["C"], 2)]
            idx += list(r.integers(lo, hi, 14))
    assert len(idx) >= 200
    # h = 1e-5 balances truncation (~h^2) against cancellation (~1e-16/h);
    # the residual error is ~3e-10 absolute at this size.
    h = 1e-5
    bad = []
    for j in idx:
        old = m.params[j]
        m.params[j] = old + h
        lp = m.forward(tok, tgt)
        m.params[j] = old - h
        lm = m.forward(tok, tgt)
        m.params[j] = old
        fd = (lp - lm) / (2 * h)
        if abs(fd - g[j]) > 1e-5 * abs(g[j]) + 2e-9:
            bad.append((j, fd, g[j]))
    assert not bad, bad[:5]
    m.close()


def test_f32_build_matches_f64():
    params = None
    m32, c = make_model("tiny", "f32")
    m64, _ = make_model("tiny", "f64", params=m32.params.astype(np.float64))
    tok, tgt = synth.token_stream(c["B"], c["T"], c["V"])
    l32 = m32.forward(tok, tgt)
    l64 = m64.forward(tok, tgt)
    assert abs(l32 - l64) / l64 < 1e-5
    for mm in (m32, m64):
        mm.zero_grad()
        mm.backward()
    assert rel(m32.grads, m64.grads) < 1e-4
    m32.close()
    m64.close()


@pytest.mark.slow
def test_small_config_overfits_one_batch():
    """Ten AdamW steps on one fixed batch: the loss falls every step."""
    m, c = make_model("small", "f32")
    tok, tgt = synth.token_stream(c["B"], c["T"], c["V"])
    losses = []
    for s in range(1, c["steps"] + 1):
        losses.append(m.forward(tok, tgt))
        m.zero_grad()
        m.backward()
        m.update(step=s, **{k: v for k, v in synth.ADAMW.items()})
    assert all(b < a for a, b in zip(losses, losses[1:])), losses
    m.close()


def test_synth_generator_reference_values():
    # SplitMix64 with seed 0: the first outputs of the published generator
    z = synth.splitmix64(0, 0, 3)
    assert [int(x) for x in z] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                   0x06C45D188009454F]
    n = synth.normals(7, 0, 200000)
    assert abs(n.mean()) < 0.01 and abs(n.std() - 1) < 0.01
    assert np.array_equal(synth.normals(7, 1001, 5), n[1001:1006])
    t = synth.randint(3, 0, 100000, 50257)
    assert t.min() >= 0 and t.max() < 50257
    tok, tgt = synth.token_stream(2, 5, 100)
    assert np.array_equal(tok.reshape(-1)[1:], tgt.reshape(-1)[:-1])


# ---------------------------------------------------------------- sampling --

def _near_boundary(probs, coin, tol=1e-6):
    cdf = np.cumsum(np.asarray(probs, dtype=np.float64))
    return np.min(np.abs(cdf - coin * cdf[-1])) < tol * cdf[-1]


def test_sample_uniform_row_is_floor_coin_times_V():
    """Equal probabilities: the inverse-CDF draw is floor(coin * V)."""
    for V in (7, 512, 50257):
        probs = np.full(V, 1.0 / V, dtype=np.float32)
        for coin in synth.coins(200, seed=11):
            if _near_boundary(probs, coin):
                continue
            assert oracle.sample(probs, coin) == math.floor(float(coin) * V)


def test_sample_one_hot_and_edges():
    probs = np.zeros(100, dtype=np.float32)
    probs[37] = 1.0
    for coin in (0.0, 0.25, 0.999999):
        assert oracle.sample(probs, coin) == 37
    # coin 0 takes the first token with nonzero probability
    probs = np.zeros(10, dtype=np.float32)
    probs[[3, 8]] = 0.5
    assert oracle.sample(probs, 0.0) == 3
    assert oracle.sample(probs, 0.4999) == 3
    assert oracle.sample(probs, 0.5) == 8


def test_sample_matches_numpy_searchsorted():
    """Library routine: the first index whose cumulative sum exceeds
    coin * total (numpy cumsum + searchsorted, float64)."""
    r = np.random.default_rng(5)
    for V in (3, 97, 1001):
        for _ in range(20):
            probs = r.dirichlet(np.full(V, 0.3)).astype(np.float32)
            coin = float(r.random())
            if _near_boundary(probs, coin):
                continue
            cdf = np.cumsum(probs.astype(np.float64))
            want = int(np.searchsorted(cdf, coin * cdf[-1], side="right"))
            assert oracle.sample(probs, coin) == min(want, V - 1)


def test_sample_frequencies_follow_probabilities():
    probs = np.array([0.05, 0.1, 0.4, 0.15, 0.3], dtype=np.float32)
    n = 200000
    counts = np.bincount([oracle.sample(probs, c) for c in synth.coins(n, seed=3)],
                         minlength=5)
    sigma = np.sqrt(n * probs * (1 - probs))
    assert np.all(np.abs(counts - n * probs) < 5 * sigma), counts


def test_generate_with_zero_embeddings_is_floor_coin_times_V():
    """wte = 0 makes every logit exactly 0, so every draw is floor(coin * V);
    the prompt and the other weights do not matter."""
    c = synth.CONFIGS["tiny"]
    m = OracleModel(c["L"], c["C"], c["NH"], c["V"], c["maxT"], 1, c["maxT"])
    m.params[:] = synth.init_params(c["L"], c["C"], c["V"], c["maxT"])
    m.param("wte")[:] = 0
    n = c["maxT"]
    coins = synth.coins(n - 1)
    tok = m.generate([c["V"] - 1], n, coins)
    want = np.floor(coins.astype(np.float64) * c["V"]).astype(np.int64)
    assert tok[0] == c["V"] - 1
    assert np.array_equal(tok[1:], want)
    m.close()


def test_generate_is_causal_and_deterministic():
    """Each draw depends only on the prefix: generating n tokens, then n + 8
    with the same coins, agrees on the first n."""
    c = synth.CONFIGS["tiny"]
    params = synth.init_params(c["L"], c["C"], c["V"], c["maxT"])
    m = OracleModel(c["L"], c["C"], c["NH"], c["V"], c["maxT"], 1, c["maxT"])
    m.params[:] = params
    coins = synth.coins(c["maxT"])
    a = m.generate([5], 40, coins[:39])
    b = m.generate([5], 48, coins[:47])
    assert np.array_equal(a, b[:40])
    assert np.all((b >= 0) & (b < c["V"]))
    m.close()


def test_page_generation_shape():
    g = json.load(open(os.path.join(GOLDEN, "gpt2_124m_printout.json")))
    assert g["generated_length"] == 64 and g["generated_first_token"] == 50256
    assert g["generated_first_token"] == g["config"]["vocab_size"] - 1


# ------------------------------------------------------------------ rotary --

def _rope(qkv, B, T, C, NH, inverse=False, precision="f64"):
    lb = lib(precision)
    x = np.ascontiguousarray(qkv, dtype=lb.dtype).copy()
    fn = lb.oracle_rope_backward if inverse else lb.oracle_rope_forward
    fn(ptr(x), B, T, C, NH)
    return x


def test_rope_scores_depend_only_on_relative_position():
    """The defining property of the rotary embedding: with the same q and k
    vector at every position, q'_t . k'_s depends only on t - s, per head."""
    B, T, C, NH = 1, 40, 64, 4
    hs = C // NH
    r = np.random.default_rng(8)
    row = r.standard_normal(3 * C)
    qkv = np.tile(row, (B * T, 1))
    out = _rope(qkv, B, T, C, NH).reshape(T, 3 * C)
    for h in range(NH):
        q = out[:, h * hs:(h + 1) * hs]
        k = out[:, C + h * hs:C + (h + 1) * hs]
        S = q @ k.T
        for d in range(-T + 1, T):
            diag = np.diagonal(S, offset=d)
            assert np.max(np.abs(diag - diag[0])) < 1e-9 * max(1.0, np.abs(diag).max()), (h, d)
    # position 0 is the identity, v is untouched, pair norms are kept
    assert np.allclose(out[0], row, atol=1e-15)
    assert np.array_equal(out[:, 2 * C:], qkv[:, 2 * C:])
    pairs_in = qkv[:, :2 * C].reshape(T, -1, 2)
    pairs_out = out[:, :2 * C].reshape(T, -1, 2)
    assert np.allclose(np.hypot(*pairs_in.transpose(2, 0, 1)),
                       np.hypot(*pairs_out.transpose(2, 0, 1)), rtol=1e-13)


def test_rope_two_dim_head_turns_by_t_radians():
    """hs = 2: one pair per head with frequency 10000^0 = 1, so position t
    turns it by t radians (a closed form)."""
    B, T, C, NH = 2, 9, 4, 2
    r = np.random.default_rng(9)
    qkv = r.standard_normal((B * T, 3 * C))
    out = _rope(qkv, B, T, C, NH)
    for row in range(B * T):
        t = row % T
        for j in range(0, 2 * C, 2):
            x, y = qkv[row, j], qkv[row, j + 1]
            assert abs(out[row, j] - (x * math.cos(t) - y * math.sin(t))) < 1e-12
            assert abs(out[row, j + 1] - (x * math.sin(t) + y * math.cos(t))) < 1e-12


def test_rope_backward_is_the_adjoint():
    """<R u, w> = <u, R^T w>: the backward (inverse rotation) is the adjoint
    of the forward, so it is the gradient map; and R^T R = I."""
    B, T, C, NH = 2, 13, 96, 3
    r = np.random.default_rng(10)
    u = r.standard_normal((B * T, 3 * C))
    w = r.standard_normal((B * T, 3 * C))
    lhs = np.sum(_rope(u, B, T, C, NH) * w)
    rhs = np.sum(u * _rope(w, B, T, C, NH, inverse=True))
    assert abs(lhs - rhs) < 1e-10 * abs(lhs)
    assert np.allclose(_rope(_rope(u, B, T, C, NH), B, T, C, NH, inverse=True), u, atol=1e-13)


def test_rope_param_count():
    """The rotary model drops only the wpe table."""
    _, full = oracle.param_sizes(12, 768, 12, 50257, 1024)
    sizes, rope = oracle.param_sizes(12, 768, 12, 50257, 1024, rope=1)
    assert sizes["wpe"] == 0 and full - rope == 1024 * 768


# ------------------------------------------------------------ loss scaling --

def test_loss_scale_schedule_worked_example():
    """Hand-worked: start 2^16, interval 3.  Steps: clean, clean, clean
    (third clean step doubles), overflow (halves, skipped), clean, overflow,
    overflow, clean x3 (doubles)."""
    seq = [0, 0, 0, 1, 0, 1, 1, 0, 0, 0]
    got = oracle.loss_scale_schedule(65536.0, seq, 3)
    want = [(True, 65536.0), (True, 65536.0), (True, 131072.0), (False, 65536.0),
            (True, 65536.0), (False, 32768.0), (False, 16384.0), (True, 16384.0),
            (True, 16384.0), (True, 32768.0)]
    assert got == want


def test_loss_scale_floor_and_long_run():
    """The scale never drops below the floor; k overflows from S give
    max(S / 2^k, floor); n * interval clean steps multiply by 2^n."""
    got = oracle.loss_scale_schedule(8.0, [1] * 6, 5, min_scale=1.0)
    assert [s for _, s in got] == [4.0, 2.0, 1.0, 1.0, 1.0, 1.0]
    assert not any(a for a, _ in got)
    got = oracle.loss_scale_schedule(2.0 ** 10, [0] * 40, 8)
    assert got[-1] == (True, 2.0 ** 15) and all(a for a, _ in got)
