"""The training loop of the pages on the C ABI: batches from token files,
forward / zero-grad / backward / AdamW per step, a validation loss and a
generated sample at fixed intervals (ujoy.net article "徒手用 1000 行 C 语言实现",
section "训练过程": the printed "val loss", "step N: train loss ... (took ...
ms)" and "generated: ..." lines).  The pages do not print their intervals;
they are arguments here.

Every number comes from the library: the batches from gpt2_loader_*, the
training losses from gpt2_forward, the validation losses from gpt2_evaluate
(no gradient, no backward state), the sample from gpt2_generate.  This module only
sequences the calls and formats the log.
"""
import time

import numpy as np

from . import gpt2, synth


def val_loss(model, loader, batches):
    """Mean of the per-batch mean losses over the first `batches` batches."""
    loader.reset()
    total = 0.0
    for _ in range(batches):
        tok, tgt = loader.next()
        total += model.evaluate(tok, tgt)
    return total / batches


def train(model, train_path, val_path, steps, B, T, *, val_every=20, val_batches=None,
          sample_every=20, gen_tokens=64, start_token=None, coin_seed=synth.COIN_SEED,
          lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, log=print):
    """Runs `steps` AdamW steps (numbered from 1 for the bias correction).

    Before step s (0-based) the validation loss is computed when s is a
    multiple of val_every, and a sample of gen_tokens tokens (from
    start_token, default V - 1, GPT-2's end-of-text id) is generated when
    s > 0 is a multiple of sample_every; both also run after the last step
    when their interval divides `steps`.  val_batches defaults to the val
    file's batch count.  The model must hold batches of B x T and
    sequences of gen_tokens.  Returns the history as a dict.
    """
    tl = gpt2.Loader(train_path, B, T)
    vl = gpt2.Loader(val_path, B, T)
    nval = vl.num_batches if val_batches is None else min(val_batches, vl.num_batches)
    V = model.V
    first = V - 1 if start_token is None else start_token
    hist = {"train": [], "val": [], "generated": [], "ms": []}
    draws = 0
    for s in range(steps + 1):
        if val_every and s % val_every == 0:
            v = val_loss(model, vl, nval)
            hist["val"].append((s, v))
            log(f"val loss {v:f}")
        if sample_every and s > 0 and s % sample_every == 0:
            coins = synth.coins(draws + gen_tokens - 1, seed=coin_seed)[draws:]
            draws += gen_tokens - 1
            toks = model.generate([first], gen_tokens, coins)
            hist["generated"].append((s, toks.tolist()))
            log("generated: " + " ".join(str(t) for t in toks.tolist()))
        if s == steps:
            break
        tok, tgt = tl.next()
        t0 = time.perf_counter()
        loss = model.forward(tok, tgt)
        model.zero_grad()
        model.backward()
        model.update(lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay,
                     step=s + 1)
        model.synchronize()
        ms = (time.perf_counter() - t0) * 1000.0
        hist["train"].append(loss)
        hist["ms"].append(ms)
        log(f"step {s}: train loss {loss:f} (took {ms:f} ms)")
    tl.close()
    vl.close()
    return hist


def write_tokens(path, ids):
    """Writes ids as a raw little-endian int32 token file."""
    np.ascontiguousarray(ids, dtype="<i4").tofile(path)


def main(argv=None):
    """python -m transformer_lm_step_train_amd.train --train T.bin --val V.bin
    [--steps 40] ...: the loop on GPT-2 124M (or --config) from the seeded
    GPT-2 initialisation (no pretrained weights are loaded)."""
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--train", required=True)
    ap.add_argument("--val", required=True)
    ap.add_argument("--config", default="gpt2_124m_b4t64", choices=sorted(synth.CONFIGS))
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--val-every", type=int, default=20)
    ap.add_argument("--val-batches", type=int, default=None)
    ap.add_argument("--sample-every", type=int, default=20)
    ap.add_argument("--gen-tokens", type=int, default=64)
    ap.add_argument("--precision", choices=["fp32", "bf16"], default="fp32")
    a = ap.parse_args(argv)
    c = synth.CONFIGS[a.config]
    m = gpt2.Model(c["L"], c["C"], c["NH"], c["V"], c["maxT"], c["B"], max(c["T"], a.gen_tokens),
                   precision=gpt2.GPT2_BF16_MIXED if a.precision == "bf16" else gpt2.GPT2_FP32)
    m.set_params(synth.init_params(c["L"], c["C"], c["V"], c["maxT"]))
    train(m, a.train, a.val, a.steps, c["B"], c["T"], val_every=a.val_every,
          val_batches=a.val_batches, sample_every=a.sample_every, gen_tokens=a.gen_tokens)
    m.close()


if __name__ == "__main__":
    main()
