"""Element-wise parity at the benchmark's shape: GPT-2 124M, B=16, T=1024, in
the launch configuration the benchmark times (one model allocated for the
whole batch, device-resident ids), fp32 and bf16 mixed precision.

The 16 sequences of a batch never interact: attention stays inside its own
row and every other layer works per position.  The batch loss is the mean of
the sequences' mean losses, so its gradient is the mean of their gradients.
The oracle therefore runs each sequence alone (B=1, T=1024) and the
reference gradient is the float64 mean of the 16 sequence gradients.  Each
sequence is one test case (about 11 s of oracle time on 16 cores).  It checks
that sequence's 1024 per-position losses and its whole 1024 x 50257 block of
logit gradients.  The batch tests then compare the loss, all 16 parameter
gradients, and the parameters after one AdamW step.

These shapes reach code paths no smaller case does:
  - the embedding key sort with 16 keys per thread;
  - the weight-gradient matmuls with K = 16384 and their K-split plans;
  - attention over eight 128-row query blocks at head size 64;
  - the 16-bit 256x256 matmul's split plan at K = 16384.

Tolerances: fp32 as everywhere (loss rel 1e-5; logit and parameter gradients
1e-3 max-abs-normalised; parameters 1e-4 after one step, with the
undetermined step-1 updates counted as in tests/parity.py).  bf16: the
stated loss bound rel 2e-2; gradients and logit gradients within a bound
derived from bf16 rounding (tests/test_gpu_bf16.py).
"""
import time

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from oracle import OracleModel, ptr
from transformer_lm_step_train_amd import synth

from parity import GRAD_TOL, check_params_after_step1, rel, split

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

CFG = synth.CONFIGS["gpt2_124m_b16t1024"]
B, T, V = CFG["B"], CFG["T"], CFG["V"]
LR = synth.ADAMW["lr"]
BF16_GRAD_BOUND = 15 * 2.0 ** -9  # 15 bf16 unit roundoffs, as in tests/test_gpu_bf16.py
BF16_LOSS_BOUND = 2e-2


def gpt2():
    from transformer_lm_step_train_amd import gpt2 as g
    return g


@pytest.fixture(scope="module")
def inputs():
    params = synth.init_params(CFG["L"], CFG["C"], V, CFG["maxT"])
    tok, tgt = synth.token_stream(B, T, V)
    return params, tok, tgt


def run_gpu(precision, params, tok, tgt):
    """One step of the batch on the GPU; everything the checks need, on the
    host."""
    g = gpt2()
    print(f"[full] gpu step, precision {precision}", flush=True)
    m = g.Model(CFG["L"], CFG["C"], CFG["NH"], V, CFG["maxT"], B, T, precision=precision)
    m.set_params(params)
    dtok = torch.tensor(tok, dtype=torch.int32, device="cuda")
    dtgt = torch.tensor(tgt, dtype=torch.int32, device="cuda")
    out = {"loss": m.forward_device(dtok, dtgt)}
    out["loss_repeat"] = m.forward_device(dtok, dtgt)
    out["losses"] = m.activation("losses").reshape(B, T)
    out["dlogits"] = m.activation("logits").reshape(B, T, V)
    m.zero_grad()
    m.backward()
    out["grads"] = m.grads()
    m.update(step=1, **synth.ADAMW)
    out["params1"] = m.params()
    out["loss_after"] = m.forward_device(dtok, dtgt)
    m.close()
    torch.cuda.synchronize()
    return out


@pytest.fixture(scope="module")
def gpu32(inputs):
    return run_gpu(gpt2().GPT2_FP32, *inputs)


@pytest.fixture(scope="module")
def gpu16(inputs):
    return run_gpu(gpt2().GPT2_BF16_MIXED, *inputs)


@pytest.fixture(scope="module")
def orc(inputs):
    """The oracle at B=1, T=1024 and the running sums over sequences."""
    params, _, _ = inputs
    o = OracleModel(CFG["L"], CFG["C"], CFG["NH"], V, CFG["maxT"], 1, T)
    state = {"model": o, "params": params, "gsum": np.zeros(o.num_params), "loss": {},
             "losses": {}, "checked": set()}
    yield state
    o.close()


def oracle_sequence(orc, inputs, b):
    """Forward and backward of sequence b alone; adds its gradient to the
    running sum once."""
    if b in orc["loss"]:
        return None
    _, tok, tgt = inputs
    o = orc["model"]
    o.params[:] = orc["params"]
    t0 = time.time()
    orc["loss"][b] = o.forward(tok[b:b + 1], tgt[b:b + 1])
    orc["losses"][b] = o.act("losses").copy()
    o.zero_grad()
    o.backward()
    orc["gsum"] += o.grads
    print(f"[full] oracle sequence {b}: loss {orc['loss'][b]:.6f}, {time.time() - t0:.1f} s",
          flush=True)
    # d(loss_b)/d(logits) of this sequence alone: the batch's is 1/B of it
    return o.act_grad("logits").reshape(T, V)


@pytest.mark.parametrize("b", range(B))
def test_sequence(b, inputs, gpu32, gpu16, orc):
    dl_ref = oracle_sequence(orc, inputs, b)
    lo, lpos = orc["loss"][b], orc["losses"][b]
    g32, g16 = gpu32["losses"][b], gpu16["losses"][b]
    assert abs(g32.mean() - lo) / lo < 1e-5, (g32.mean(), lo)
    assert rel(g32, lpos) < 1e-5
    assert abs(g16.mean() - lo) / lo < BF16_LOSS_BOUND, (g16.mean(), lo)
    if dl_ref is not None:  # full logit-gradient block (the batch's is 1/B of it)
        e32 = rel(gpu32["dlogits"][b] * B, dl_ref)
        e16 = rel(gpu16["dlogits"][b] * B, dl_ref)
        print(f"[full] sequence {b}: dlogits rel fp32 {e32:.2e} bf16 {e16:.2e}", flush=True)
        assert e32 < GRAD_TOL
        assert e16 < BF16_GRAD_BOUND


def reference_gradient(orc, inputs):
    for b in range(B):
        oracle_sequence(orc, inputs, b)
    return (orc["gsum"] / B).astype(np.float32)


def test_fp32_batch_step(inputs, gpu32, orc):
    params, _, _ = inputs
    R = reference_gradient(orc, inputs)
    lref = float(np.mean([orc["loss"][b] for b in range(B)]))
    r = abs(gpu32["loss"] - lref) / lref
    print(f"[full] fp32 loss {gpu32['loss']:.6f} oracle {lref:.6f} rel {r:.2e}", flush=True)
    assert r < 1e-5, (gpu32["loss"], lref)
    assert gpu32["loss_repeat"] == gpu32["loss"]
    assert gpu32["loss_after"] < gpu32["loss"]
    sizes = orc["model"].param_sizes
    G, RR = split(gpu32["grads"], sizes), split(R, sizes)
    errs = {n: rel(G[n], RR[n]) for n in oracle.PARAM_NAMES}
    print("[full] fp32 grad rel:", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert all(v < GRAD_TOL for v in errs.values()), errs
    # the oracle's AdamW step from the same weights with the reference gradient
    p_ref = params.copy()
    m0 = np.zeros_like(p_ref)
    v0 = np.zeros_like(p_ref)
    oracle.lib("f32").oracle_adamw(ptr(p_ref), ptr(R), ptr(m0), ptr(v0), p_ref.size, LR,
                                   synth.ADAMW["beta1"], synth.ADAMW["beta2"],
                                   synth.ADAMW["eps"], synth.ADAMW["weight_decay"], 1)
    check_params_after_step1(split(gpu32["params1"], sizes), split(p_ref, sizes), G, RR,
                             lr=LR, tag="full fp32")


def test_bf16_batch_step(inputs, gpu16, orc):
    R = reference_gradient(orc, inputs)
    lref = float(np.mean([orc["loss"][b] for b in range(B)]))
    r = abs(gpu16["loss"] - lref) / lref
    print(f"[full] bf16 loss {gpu16['loss']:.6f} oracle {lref:.6f} rel {r:.2e}", flush=True)
    assert r < BF16_LOSS_BOUND
    assert gpu16["loss_repeat"] == gpu16["loss"]
    assert gpu16["loss_after"] < gpu16["loss"]
    sizes = orc["model"].param_sizes
    G, RR = split(gpu16["grads"], sizes), split(R, sizes)
    errs = {n: rel(G[n], RR[n]) for n in oracle.PARAM_NAMES}
    print("[full] bf16 grad rel:", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert all(v < BF16_GRAD_BOUND for v in errs.values()), errs
    assert np.all(np.isfinite(gpu16["params1"]))


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_max_batch_equals_its_halves(prec, monkeypatch):
    """The largest batch the limits allow at T = 1024: B = 32, B*T = 32768
    (the 32-key embedding sort, the weight gradients split over K = 32768,
    a 960 MiB attention dS workspace), with guard words after every buffer.
    Sequences never interact, so the batch loss is the mean of the two
    16-sequence halves' losses and the batch gradient the mean of their
    gradients; the halves run on a second model allocated for B = 16.
    Tolerances: loss rel 1e-6 (same per-row losses, another summation
    order), gradients rel 1e-4 fp32 / the bf16 bound (sums over K split
    differently)."""
    g = gpt2()
    p = g.GPT2_FP32 if prec == "fp32" else g.GPT2_BF16_MIXED
    monkeypatch.setenv("GPT2_GUARD_WORDS", "1")
    params = synth.init_params(CFG["L"], CFG["C"], V, CFG["maxT"])
    tok, tgt = synth.token_stream(2 * B, T, V)
    print(f"[full] B=32 step, precision {prec}", flush=True)
    m = g.Model(CFG["L"], CFG["C"], CFG["NH"], V, CFG["maxT"], 2 * B, T, precision=p)
    m.set_params(params)
    dtok = torch.tensor(tok, dtype=torch.int32, device="cuda")
    dtgt = torch.tensor(tgt, dtype=torch.int32, device="cuda")
    loss = m.forward_device(dtok, dtgt)
    m.zero_grad()
    m.backward()
    G = m.grads().astype(np.float64)
    m.check_guards()
    m.close()
    m = g.Model(CFG["L"], CFG["C"], CFG["NH"], V, CFG["maxT"], B, T, precision=p)
    m.set_params(params)
    hl, hg = [], np.zeros_like(G)
    for h in range(2):
        hl.append(m.forward_device(dtok[h * B:(h + 1) * B].contiguous(),
                                   dtgt[h * B:(h + 1) * B].contiguous()))
        m.zero_grad()
        m.backward()
        hg += m.grads()
    m.check_guards()
    m.close()
    torch.cuda.synchronize()
    lref = (hl[0] + hl[1]) / 2
    print(f"[full] B=32 {prec} loss {loss:.7f}, halves {hl}", flush=True)
    assert abs(loss - lref) / lref < 1e-6, (loss, hl)
    sizes, _ = oracle.param_sizes(CFG["L"], CFG["C"], CFG["NH"], V, CFG["maxT"])
    GG, RR = split(G, sizes), split(hg / 2, sizes)
    errs = {n: rel(GG[n], RR[n]) for n in oracle.PARAM_NAMES}
    print(f"[full] B=32 {prec} grad rel to the halves:", {k: f"{v:.1e}" for k, v in errs.items()},
          flush=True)
    bound = 1e-4 if prec == "fp32" else BF16_GRAD_BOUND
    assert all(v < bound for v in errs.values()), errs
