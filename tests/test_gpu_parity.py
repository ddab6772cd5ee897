"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Tolerances (max |a - r| / max |r| per tensor unless noted):
  loss rel 1e-5; logits, their gradient and every parameter gradient 1e-3;
  parameters after the AdamW step 1e-4; forward activations 1e-4.
Step-1 AdamW updates that a tolerated gradient error leaves undetermined are
excluded and counted by tests/parity.py; the update itself is checked exactly
by applying the oracle's AdamW to the GPU's own gradients.
"""
import math
import time

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from oracle import OracleModel, ptr
from transformer_lm_step_train_amd import synth

from parity import check_params_after_step1, rel, split

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


def gpt2():
    from transformer_lm_step_train_amd import gpt2 as g
    return g


class Pair:
    """A GPU model and an oracle model with identical weights."""

    def __init__(self, name, B=None, T=None, alloc_B=None, alloc_T=None, params=None,
                 attn_recompute=False):
        c = dict(synth.CONFIGS[name])
        self.c = c
        self.B = B or c["B"]
        self.T = T or c["T"]
        print(f"[parity] config={name} B={self.B} T={self.T} attn_recompute={attn_recompute}",
              flush=True)
        rope = c.get("rope", False)
        if params is None:
            params = synth.init_params(c["L"], c["C"], c["V"], c["maxT"], rope=rope)
        self.p0 = params
        g = gpt2()
        self.gpu = g.Model(c["L"], c["C"], c["NH"], c["V"], c["maxT"], alloc_B or self.B,
                           alloc_T or self.T, rope=rope, attn_recompute=attn_recompute)
        self.gpu.set_params(params)
        self.orc = OracleModel(c["L"], c["C"], c["NH"], c["V"], c["maxT"], self.B, self.T,
                               rope=rope)
        self.orc.params[:] = params
        self.sizes = self.orc.param_sizes

    def close(self):
        self.gpu.close()
        self.orc.close()


def lse_from_preatt(pre, B, NH, T):
    pre = pre.reshape(B, NH, T, T).astype(np.float64)
    mask = np.tril(np.ones((T, T), dtype=bool))
    z = np.where(mask, pre, -np.inf)
    mx = z.max(-1, keepdims=True)
    return (mx[..., 0] + np.log(np.exp(z - mx).sum(-1))).reshape(-1)


FWD_NAMES = ["ln1", "ln1_mean", "ln1_rstd", "qkv", "atty", "residual2", "ln2",
             "ln2_mean", "ln2_rstd", "fch", "fch_gelu", "residual3"]


@pytest.mark.parametrize("name", ["tiny", "ragged", "small", "tiny_rope", "ragged_rope"])
def test_forward_activations(name):
    P = Pair(name)
    c, B, T = P.c, P.B, P.T
    tok, tgt = synth.token_stream(B, T, c["V"])
    P.gpu.forward(tok)              # no targets: logits stay
    P.orc.forward(tok, tgt)
    M, L, NH = B * T, c["L"], c["NH"]
    assert rel(P.gpu.activation("encoded"), P.orc.act("encoded")) < 1e-6
    for n in FWD_NAMES:
        ref = P.orc.act(n).reshape(L, -1)
        for l in range(L):
            r = rel(P.gpu.activation(n, l), ref[l])
            assert r < 1e-4, (n, l, r)
    pre = P.orc.act("preatt").reshape(L, -1)
    for l in range(L):
        want = lse_from_preatt(pre[l], B, NH, T)
        got = P.gpu.activation("att_lse", l)
        assert np.max(np.abs(got - want)) < 1e-4 * max(1.0, np.max(np.abs(want)))
    for n in ("lnf", "lnf_mean", "lnf_rstd"):
        assert rel(P.gpu.activation(n), P.orc.act(n)) < 1e-4, n
    assert rel(P.gpu.activation("logits"), P.orc.act("logits")) < 1e-4
    P.close()


def check_step(P, tok, tgt, lr=1e-4, wd=0.0):
    c = P.c
    loss_g = P.gpu.forward(tok, tgt)
    loss_o = P.orc.forward(tok, tgt)
    assert abs(loss_g - loss_o) / abs(loss_o) < 1e-5, (loss_g, loss_o)
    assert rel(P.gpu.activation("losses"), P.orc.act("losses")) < 1e-5
    P.gpu.zero_grad()
    P.gpu.backward()
    P.orc.zero_grad()
    P.orc.backward()
    # d(loss)/d(logits), written by the fused softmax-CE over the logits
    assert rel(P.gpu.activation("logits"), P.orc.act_grad("logits")) < 1e-3
    gg = P.gpu.grads()
    go = P.orc.grads.copy()
    G, R = split(gg, P.sizes), split(go, P.sizes)
    for n in oracle.PARAM_NAMES:
        r = rel(G[n], R[n])
        assert r < 1e-3, (n, r)
    p_before = P.gpu.params()
    P.gpu.update(lr=lr, weight_decay=wd, step=1)
    P.orc.update(lr=lr, weight_decay=wd, step=1)
    pg = P.gpu.params()
    # the update alone: oracle AdamW applied to the GPU's own gradients
    L32 = oracle.lib("f32")
    p_chk = p_before.copy()
    m0 = np.zeros_like(p_chk)
    v0 = np.zeros_like(p_chk)
    L32.oracle_adamw(ptr(p_chk), ptr(gg), ptr(m0), ptr(v0), p_chk.size, lr, 0.9, 0.999,
                     1e-8, wd, 1)
    for n, (a, b) in {k: (split(pg, P.sizes)[k], split(p_chk, P.sizes)[k])
                      for k in oracle.PARAM_NAMES}.items():
        assert rel(a, b) < 1e-6, n
    mg, vg = P.gpu.opt_state()
    assert rel(mg, m0) < 1e-6 and rel(vg, v0) < 1e-6
    # the whole step against the oracle's own step, with the elements whose
    # step-1 update is undetermined counted and excluded (tests/parity.py)
    check_params_after_step1(split(pg, P.sizes), split(P.orc.params.copy(), P.sizes), G, R,
                             lr=lr, rope=bool(c.get("rope", False)))
    return loss_g


@pytest.mark.parametrize("name", ["tiny", "ragged", "small", "ragged80", "ragged704",
                                  "gpt2_124m_b4t64", "tiny_rope", "ragged_rope", "wide_vocab",
                                  "tiny_long"])
def test_one_training_step(name):
    P = Pair(name)
    tok, tgt = synth.token_stream(P.B, P.T, P.c["V"])
    check_step(P, tok, tgt)
    P.close()


@pytest.mark.parametrize("name", ["tiny", "ragged", "small", "ragged_rope", "tiny_long"])
def test_one_training_step_recomputing_attention(name):
    """The attention backward without the dS workspace (its dQ kernel
    recomputes the scores) against the oracle."""
    P = Pair(name, attn_recompute=True)
    tok, tgt = synth.token_stream(P.B, P.T, P.c["V"])
    check_step(P, tok, tgt)
    P.close()


@pytest.mark.parametrize("name,B,T", [("ragged", None, None), ("small", None, None),
                                      ("gpt2_124m_b4t64", None, None), ("tiny", 2, 300)])
def test_attention_backward_paths_agree(name, B, T):
    """The two attention backwards (dS kept, dS recomputed) compute the same
    sums in different orders: their gradients agree to a few roundoffs, and
    the dS path repeats bit for bit."""
    c = synth.CONFIGS[name]
    B, T = B or c["B"], T or c["T"]
    g = gpt2()
    params = synth.init_params(c["L"], c["C"], c["V"], max(c["maxT"], T))
    tok, tgt = synth.token_stream(B, T, c["V"])
    grads = {}
    for rec in (False, True):
        m = g.Model(c["L"], c["C"], c["NH"], c["V"], max(c["maxT"], T), B, T,
                    attn_recompute=rec)
        m.set_params(params)
        runs = []
        for _ in range(2):
            m.forward(tok, tgt)
            m.zero_grad()
            m.backward()
            runs.append(m.grads())
        assert np.array_equal(runs[0], runs[1]), rec
        grads[rec] = runs[0]
        m.close()
    sizes, _ = oracle.param_sizes(c["L"], c["C"], c["NH"], c["V"], max(c["maxT"], T))
    G, R = split(grads[False], sizes), split(grads[True], sizes)
    errs = {n: rel(G[n], R[n]) for n in oracle.PARAM_NAMES}
    print(f"[parity] {name} B={B} T={T} dS kept vs recomputed:",
          {k: f"{v:.1e}" for k, v in errs.items()}, flush=True)
    assert all(v < 2e-5 for v in errs.values()), errs


def test_weight_decay_step():
    P = Pair("ragged")
    tok, tgt = synth.token_stream(P.B, P.T, P.c["V"])
    check_step(P, tok, tgt, lr=1e-3, wd=0.1)
    P.close()


@pytest.mark.parametrize("name", ["tiny", "tiny_rope"])
def test_smaller_batch_than_allocated(name):
    P = Pair(name, B=1, T=37, alloc_B=2, alloc_T=64)
    tok, tgt = synth.token_stream(P.B, P.T, P.c["V"])
    check_step(P, tok, tgt)
    P.close()


@pytest.mark.parametrize("B,kind", [(256, "uniform"), (512, "uniform"), (256, "zipf")])
def test_large_batch_sort_variants(B, kind):
    """B*T = 16384 and 32768 positions on the tiny model: the embedding
    backward's key sort runs with 16 and 32 keys per thread (the latter fills
    the 160 KiB of LDS), and the weight gradients take their largest K
    splits.  Uniform ids repeat about B/8 times each; with Zipf(1.1) ids the
    most frequent one fills a run of thousands of positions across hundreds
    of the backward's 16-key chunks."""
    P = Pair("tiny", B=B, T=64)
    if kind == "zipf":
        tok, tgt = synth.zipf_tokens(P.B, P.T, P.c["V"])
    else:
        tok, tgt = synth.token_stream(P.B, P.T, P.c["V"])
    check_step(P, tok, tgt)
    P.close()


def test_sort_variant_below_allocation():
    """A model allocated for B*T = 32768 run at B*T = 6400 and 150: each run
    picks a smaller sort variant than the allocation's (8 keys and 1 key per
    thread), whose LDS limit must have been raised at create."""
    c = synth.CONFIGS["tiny"]
    params = synth.init_params(c["L"], c["C"], c["V"], c["maxT"])
    g = gpt2()
    m = g.Model(c["L"], c["C"], c["NH"], c["V"], c["maxT"], 512, 64)
    for B, T in ((100, 64), (3, 50)):
        print(f"[parity] tiny allocated 512x64, run B={B} T={T}", flush=True)
        m.set_params(params)
        o = OracleModel(c["L"], c["C"], c["NH"], c["V"], c["maxT"], B, T)
        o.params[:] = params
        tok, tgt = synth.token_stream(B, T, c["V"])
        lg = m.forward(tok, tgt)
        lo = o.forward(tok, tgt)
        assert abs(lg - lo) / lo < 1e-5, (lg, lo)
        m.zero_grad()
        m.backward()
        o.zero_grad()
        o.backward()
        G, R = split(m.grads(), o.param_sizes), split(o.grads.copy(), o.param_sizes)
        for n in oracle.PARAM_NAMES:
            assert rel(G[n], R[n]) < 1e-3, (B, T, n, rel(G[n], R[n]))
        o.close()
    m.close()


@pytest.mark.parametrize("kind", ["all_same", "zipf"])
def test_embedding_scatter_with_repeats(kind):
    P = Pair("ragged")
    B, T, V = P.B, P.T, P.c["V"]
    if kind == "all_same":
        tok = np.full((B, T), 7, dtype=np.int32)
        _, tgt = synth.token_stream(B, T, V)
    else:
        tok, tgt = synth.zipf_tokens(B, T, V)
    check_step(P, tok, tgt)
    P.close()


def test_small_ten_steps_overfit():
    P = Pair("small")
    tok, tgt = synth.token_stream(P.B, P.T, P.c["V"])
    lg, lo = [], []
    for s in range(1, 11):
        lg.append(P.gpu.step(tok, tgt, s, **synth.ADAMW))
        lo.append(P.orc.forward(tok, tgt))
        P.orc.zero_grad()
        P.orc.backward()
        P.orc.update(step=s, **synth.ADAMW)
    print("[parity] gpu losses", lg, flush=True)
    assert all(b < a for a, b in zip(lg, lg[1:])), lg
    for a, b in zip(lg, lo):
        assert abs(a - b) / b < 1e-4, (lg, lo)
    P.close()


@pytest.mark.parametrize("prec", ["fp32", "bf16", "fp16"])
def test_evaluate_loss_only(prec):
    """gpt2_evaluate: the same loss as a training forward (same kernels up to
    the loss), the logits left as an inference forward leaves them, no
    backward state, and sampling from its logits."""
    g = gpt2()
    c = synth.CONFIGS["ragged"]
    p = {"fp32": g.GPT2_FP32, "bf16": g.GPT2_BF16_MIXED, "fp16": g.GPT2_F16_MIXED}[prec]
    params = synth.init_params(c["L"], c["C"], c["V"], c["maxT"])
    m = g.Model(c["L"], c["C"], c["NH"], c["V"], c["maxT"], c["B"], c["T"], precision=p)
    m.set_params(params)
    tok, tgt = synth.token_stream(c["B"], c["T"], c["V"])
    le = m.evaluate(tok, tgt)
    z_eval = m.activation("logits")
    d_eval = m.sample(1, 40, 0.625)
    with pytest.raises(g.GPT2Error) as e:
        m.backward()
    assert e.value.code == g.GPT2_ESTATE
    m.forward(tok)
    assert np.array_equal(m.activation("logits"), z_eval)
    assert m.sample(1, 40, 0.625) == d_eval
    lt = m.forward(tok, tgt)
    assert le == lt, (le, lt)
    if prec == "fp32":
        o = OracleModel(c["L"], c["C"], c["NH"], c["V"], c["maxT"], c["B"], c["T"])
        o.params[:] = params
        lo = o.forward(tok, tgt)
        assert abs(le - lo) / lo < 1e-5
        o.close()
    m.zero_grad()
    m.backward()  # the training forward's state is intact
    m.close()


@pytest.mark.parametrize("name,prec,B", [("tiny", "fp32", 2), ("ragged", "bf16", 3),
                                         ("ragged80", "fp16", 3), ("ragged_rope", "fp32", 3),
                                         ("small", "fp32", 4), ("tiny", "bf16", 512)])
def test_guard_words_intact(name, prec, B, monkeypatch):
    """With GPT2_GUARD_WORDS every arena sub-buffer is followed by a guard
    region: two training steps, an evaluation, a smaller batch and a sample
    leave every guard intact, and the results equal an unguarded model's bit
    for bit."""
    g = gpt2()
    c = synth.CONFIGS[name]
    p = {"fp32": g.GPT2_FP32, "bf16": g.GPT2_BF16_MIXED, "fp16": g.GPT2_F16_MIXED}[prec]
    rope = c.get("rope", False)
    params = synth.init_params(c["L"], c["C"], c["V"], c["maxT"], rope=rope)
    tok, tgt = synth.token_stream(B, c["T"], c["V"])
    out = []
    for guards in ("1", "0"):
        monkeypatch.setenv("GPT2_GUARD_WORDS", guards)
        m = g.Model(c["L"], c["C"], c["NH"], c["V"], c["maxT"], B, c["T"], precision=p,
                    rope=rope)
        m.set_params(params)
        losses = [m.step(tok, tgt, s, **synth.ADAMW) for s in (1, 2)]
        losses.append(m.evaluate(tok[:1, :c["T"] // 2], tgt[:1, :c["T"] // 2]))
        losses.append(m.sample(0, 3, 0.5))
        if guards == "1":
            m.check_guards()
        else:
            with pytest.raises(g.GPT2Error) as e:
                m.check_guards()
            assert e.value.code == g.GPT2_EINVAL
        out.append((losses, m.params()))
        m.close()
    assert out[0][0] == out[1][0]
    assert np.array_equal(out[0][1], out[1][1])


def test_deterministic():
    c = synth.CONFIGS["small"]
    g = gpt2()
    params = synth.init_params(c["L"], c["C"], c["V"], c["maxT"])
    tok, tgt = synth.zipf_tokens(c["B"], c["T"], c["V"])
    outs = []
    for _ in range(2):
        m = g.Model(c["L"], c["C"], c["NH"], c["V"], c["maxT"], c["B"], c["T"])
        m.set_params(params)
        losses = [m.step(tok, tgt, s) for s in (1, 2)]
        outs.append((losses, m.grads(), m.params()))
        m.close()
    assert outs[0][0] == outs[1][0]
    assert np.array_equal(outs[0][1], outs[1][1])
    assert np.array_equal(outs[0][2], outs[1][2])


def test_error_paths():
    g = gpt2()
    c = synth.CONFIGS["tiny"]
    m = g.Model(c["L"], c["C"], c["NH"], c["V"], c["maxT"], c["B"], c["T"])
    m.set_params(synth.init_params(c["L"], c["C"], c["V"], c["maxT"]))
    tok, tgt = synth.token_stream(c["B"], c["T"], c["V"])
    with pytest.raises(g.GPT2Error) as e:
        m.backward()
    assert e.value.code == g.GPT2_ESTATE
    bad = tok.copy()
    bad[1, 3] = c["V"]
    with pytest.raises(g.GPT2Error) as e:
        m.forward(bad, tgt)
    assert e.value.code == g.GPT2_ERANGE
    with pytest.raises(g.GPT2Error) as e:
        m.forward(tok[:, :10].copy(), np.full((c["B"], 10), -1, dtype=np.int32))
    assert e.value.code == g.GPT2_ERANGE
    with pytest.raises(g.GPT2Error) as e:
        m.forward(np.zeros((c["B"] + 1, c["T"]), dtype=np.int32))
    assert e.value.code == g.GPT2_EINVAL
    # ids checked on the device
    dtok = torch.tensor(bad, dtype=torch.int32, device="cuda")
    dtgt = torch.tensor(tgt, dtype=torch.int32, device="cuda")
    with pytest.raises(g.GPT2Error) as e:
        m.forward_device(dtok, dtgt)
    assert e.value.code == g.GPT2_ERANGE
    # forward without targets: backward refuses
    m.forward(tok)
    with pytest.raises(g.GPT2Error) as e:
        m.backward()
    assert e.value.code == g.GPT2_ESTATE
    # the model still works after the errors
    l1 = m.forward(tok, tgt)
    l2 = m.forward_device(torch.tensor(tok, dtype=torch.int32, device="cuda"), dtgt)
    assert l1 == l2 and math.isfinite(l1)
    with pytest.raises(g.GPT2Error) as e:
        m.update(step=0)
    assert e.value.code == g.GPT2_EINVAL
    m.close()


def test_profile_class_mask():
    """Timed classes report kernel time; the others only count launches and
    algorithmic work, identical to the timed run's counts."""
    g = gpt2()
    c = synth.CONFIGS["tiny"]
    m = g.Model(c["L"], c["C"], c["NH"], c["V"], c["maxT"], c["B"], c["T"])
    m.set_params(synth.init_params(c["L"], c["C"], c["V"], c["maxT"]))
    tok, tgt = synth.token_stream(c["B"], c["T"], c["V"])

    def run(mask, step):
        g.gpt2_profile(m.h, mask)
        m.step(tok, tgt, step)
        m.synchronize()
        out = {n: g.gpt2_profile_read(m.h, i) for i, n in enumerate(g.KC_NAMES)}
        g.gpt2_profile(m.h, False)
        return out

    gemm_only = run(1 << g.KC_NAMES.index("gemm"), 1)
    every = run(True, 2)
    assert gemm_only["gemm"]["ms"] > 0 and gemm_only["gemm"]["launches"] > 0
    for n in g.KC_NAMES:
        assert every[n]["launches"] == gemm_only[n]["launches"] > 0, n
        assert every[n]["flops"] == gemm_only[n]["flops"], n
        assert every[n]["bytes"] == gemm_only[n]["bytes"], n
        assert every[n]["ms"] > 0, n
        if n != "gemm":
            assert gemm_only[n]["ms"] == 0.0, n
    with pytest.raises(g.GPT2Error) as e:
        g.gpt2_profile(m.h, 1 << len(g.KC_NAMES))
    assert e.value.code == g.GPT2_EINVAL
    m.close()
