"""Training throughput of one GPT-2 124M step (forward, backward, AdamW) on
one MI355X, B=16 sequences of T=1024 tokens, fp32.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints one JSON line.  The timed region covers exactly K training steps,
each = forward with the loss read back to the host + zero-grad + backward +
AdamW update, with token ids already resident in device memory; it is
bracketed by device synchronizations.  The matmul family's launch times come
from HIP events carried in the library's own dispatches on its stream during
the timed steps; the per-class breakdown from a second, fully instrumented
pass.  By default the line also carries `mixed_bf16`: the same measurement
of the bf16 mixed-precision model on the same batch.  The CPU-oracle
baseline is timed afterwards on a bounded sample (one sequence of the batch)
on the host cores.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "gpt2_124m_b16t1024"
MFMA_FP32_PEAK_TFLOPS = 157.3
MFMA_BF16_PEAK_TFLOPS = 2500.0
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--precision", choices=["fp32", "bf16", "fp16"], default="fp32",
                    help="fp32 (the headline workload), or the bf16 / fp16 mixed-precision "
                         "model")
    ap.add_argument("--tokens", choices=["uniform", "zipf"], default="uniform",
                    help="token ids: uniform (the workload), or Zipf(1.1) like real text "
                         "(many repeats of a few ids; for timing the embedding backward)")
    ap.add_argument("--no-mixed", action="store_true",
                    help="fp32 run only: no mixed_bf16 leg")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="no kernel events: no roofline object and no instrumented second pass")
    a = ap.parse_args()
    if a.steps < 1 or a.warmup < 0:
        ap.error("--steps must be at least 1 and --warmup at least 0")
    return a


def source_hash(precision="fp32"):
    """SHA-256 of a matmul family's sources (kernels, their helpers and the
    split plans, which decide the tile order): the fp32 or the 16-bit one."""
    h = hashlib.sha256()
    kern = "gemm.hip" if precision == "fp32" else "gemm_bf16.hip"
    for f in (kern, "common.h", "plan.cpp", "plan.h"):
        h.update(open(os.path.join(ROOT, "transformer_lm_step_train_amd", "csrc", f), "rb").read())
    return h.hexdigest()


TRAFFIC_FILES = {"fp32": "gemm_fp32_traffic.json", "bf16": "gemm_bf16_traffic.json"}


def measured_traffic(precision):
    """HBM bytes per matmul launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary of this precision's step, or None if the matmul
    sources have changed since the counters were taken (or for fp16, which
    they do not cover)."""
    name = TRAFFIC_FILES.get(precision)
    path = os.path.join(ROOT, "profiles", name) if name else None
    if not path or not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if source_hash(precision) != rec.get("source_sha256"):
        return None
    return round(rec["hbm_bytes_per_launch"])


def host_ram_gib():
    try:
        return round(os.sysconf("SC_PAGE_SIZE") * os.sysconf("SC_PHYS_PAGES") / 2**30, 1)
    except (ValueError, OSError):
        return None


def oracle_steps(o, tok, tgt, n):
    """n full training steps of the oracle; seconds per step."""
    times = []
    for s in range(1, n + 1):
        t0 = time.perf_counter()
        o.forward(tok, tgt)
        o.zero_grad()
        o.backward()
        o.update(step=s, lr=1e-4)
        times.append(time.perf_counter() - t0)
    return times


def cpu_baseline(c, params, tok, tgt):
    """The oracle (plain C, OpenMP over rows) timed as it is, on a bounded
    sample of the workload: one sequence of the batch (B=1, T=1024), 1
    warm-up step (first touch of its arenas) and 2 timed steps on every host
    core.  Its per-token work equals the full batch's (sequences are
    independent and every matmul is linear in the rows), so tokens/s carries
    over to B=16, which needs about 76 GB of host memory and 3 minutes per
    step.  A second leg runs the pages' own shape (124M, B=4, T=64) at 8
    threads, the setting of the pages' run, printed at 1.29-1.45 s per step
    on an M3 Max (ujoy.net, section "训练过程")."""
    import oracle as _o
    from oracle import OracleModel
    from transformer_lm_step_train_amd import synth
    cores = int(os.environ.get("OMP_NUM_THREADS") or len(os.sched_getaffinity(0)))
    lb = _o.lib("f32")
    lb.oracle_set_threads(cores)
    o = OracleModel(c["L"], c["C"], c["NH"], c["V"], c["maxT"], 1, c["T"])
    o.params[:] = params
    times = oracle_steps(o, tok[:1], tgt[:1], 3)
    o.close()
    dt = sum(times[1:]) / 2
    out = {"value": round(c["T"] / dt, 2), "unit": "tokens/s", "cores": cores,
           "kind": "oracle",
           "sample": f"B=1 T={c['T']} (one sequence of the B={c['B']} batch): 1 warm-up + 2 "
                     f"timed training steps (fwd+bwd+AdamW), {times[1]:.2f} / {times[2]:.2f} s "
                     f"(warm-up {times[0]:.2f} s); host RAM {host_ram_gib()} GiB",
           "threads_8": None}
    p4 = synth.CONFIGS["gpt2_124m_b4t64"]
    lb.oracle_set_threads(8)
    o = OracleModel(p4["L"], p4["C"], p4["NH"], p4["V"], p4["maxT"], p4["B"], p4["T"])
    o.params[:] = params
    t4, g4 = synth.token_stream(p4["B"], p4["T"], p4["V"])
    times = oracle_steps(o, t4, g4, 3)
    o.close()
    lb.oracle_set_threads(cores)
    s8 = sum(times[1:]) / 2
    out["threads_8"] = {"workload": "GPT-2 124M, B=4 T=64 (the pages' run)", "threads": 8,
                        "steps": "1 warm-up + 2 timed", "s_per_step": round(s8, 3),
                        "tokens_per_s": round(256 / s8, 1),
                        "page_m3max_s_per_step": [1.289, 1.452]}
    return out


def pages_shape_gpu(params):
    """The GPU step at the pages' run shape (124M, B=4, T=64, fp32)."""
    from transformer_lm_step_train_amd import gpt2, synth
    import torch
    p4 = synth.CONFIGS["gpt2_124m_b4t64"]
    m = gpt2.Model(p4["L"], p4["C"], p4["NH"], p4["V"], p4["maxT"], p4["B"], p4["T"])
    m.set_params(params)
    tok, tgt = synth.token_stream(p4["B"], p4["T"], p4["V"])
    dtok = torch.tensor(tok, dtype=torch.int32, device="cuda")
    dtgt = torch.tensor(tgt, dtype=torch.int32, device="cuda")
    def one(s):
        m.forward_device(dtok, dtgt)
        m.zero_grad()
        m.backward()
        m.update(step=s, lr=1e-4)
    for s in range(1, 6):
        one(s)
    m.synchronize()
    t0 = time.perf_counter()
    for s in range(6, 26):
        one(s)
    m.synchronize()
    ms = (time.perf_counter() - t0) / 20 * 1000.0
    m.close()
    return {"workload": "GPT-2 124M, B=4 T=64 (the pages' run), fp32", "ms_per_step": round(ms, 3),
            "tokens_per_s": round(256 / ms * 1000.0, 1)}


def run_leg(precision, args, params, tok, tgt):
    """Warm-up, K timed training steps, then K instrumented steps of one
    model on the batch; its throughput, step roofline and per-class times."""
    import torch
    from transformer_lm_step_train_amd import gpt2, synth
    c = synth.CONFIGS[WORKLOAD]
    B, T = c["B"], c["T"]
    half = precision in ("bf16", "fp16")
    prec = {"fp32": gpt2.GPT2_FP32, "bf16": gpt2.GPT2_BF16_MIXED,
            "fp16": gpt2.GPT2_F16_MIXED}[precision]
    m = gpt2.Model(c["L"], c["C"], c["NH"], c["V"], c["maxT"], B, T, precision=prec)
    m.set_params(params)
    dtok = torch.tensor(tok, dtype=torch.int32, device="cuda")
    dtgt = torch.tensor(tgt, dtype=torch.int32, device="cuda")
    adamw = dict(synth.ADAMW)

    step = 0
    losses = []
    marks = []

    def train_step():
        nonlocal step
        step += 1
        losses.append(m.forward_device(dtok, dtgt))
        marks.append(time.perf_counter())
        m.zero_grad()
        m.backward()
        m.update(step=step, **adamw)

    for _ in range(args.warmup):
        train_step()
    m.synchronize()
    marks.clear()
    # Inside the timed region only the matmul family (the roofline's kernel)
    # is timed; every class still counts its launches and algorithmic work.
    if not args.no_kernel_timing:
        gpt2.gpt2_profile(m.h, 1 << gpt2.KC_NAMES.index("gemm"))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        train_step()
    m.synchronize()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = 1000.0 * dt / args.steps
    tokens_per_s = B * T * args.steps / dt
    # The loss readback of step i+1 ends one full step after that of step i
    # (zero-grad, backward and AdamW of step i, forward of step i+1).
    per_step = np.diff(np.array(marks)) * 1000.0
    ms_median = float(np.median(per_step)) if len(per_step) else ms

    timed_losses = list(losses)
    kc, kci, inst_ms = {}, {}, None
    if not args.no_kernel_timing:
        for i, name in enumerate(gpt2.KC_NAMES):
            kc[name] = gpt2.gpt2_profile_read(m.h, i)
        gpt2.gpt2_profile(m.h, False)
        # A second pass of K steps with every launch timed, for the per-class
        # breakdown (each timed dispatch costs a few microseconds of issue).
        gpt2.gpt2_profile(m.h, True)
        ti = time.perf_counter()
        for _ in range(args.steps):
            train_step()
        m.synchronize()
        inst_ms = 1000.0 * (time.perf_counter() - ti) / args.steps
        for i, name in enumerate(gpt2.KC_NAMES):
            kci[name] = gpt2.gpt2_profile_read(m.h, i)
        gpt2.gpt2_profile(m.h, False)
    assert all(np.isfinite(losses)), losses
    m.close()

    roofline = None
    step_roof = None
    peak = MFMA_BF16_PEAK_TFLOPS if half else MFMA_FP32_PEAK_TFLOPS
    if kc:
        # Composite bound of the whole step: every kernel class at the larger
        # of its MFMA time and its HBM time for the algorithmic work.
        t_roof = sum(max(r["flops"] / (peak * 1e12), r["bytes"] / (HBM_PEAK_GBS * 1e9))
                     for r in kc.values()) / args.steps * 1000.0
        step_roof = {"t_roof_ms": round(t_roof, 3), "frac": round(t_roof / ms, 4),
                     "rule": "sum over kernel classes of max(FLOP/MFMA peak, bytes/HBM peak)"}
        g = kc["gemm"]
        n = max(g["launches"], 1)
        avg_s = g["ms"] / n / 1000.0
        achieved = (g["flops"] / n) / avg_s / 1e12 if avg_s > 0 else 0.0
        roofline = {"bound": "mfma", "achieved": round(achieved, 2),
                    "peak": peak, "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4), "traffic": measured_traffic(precision),
                    "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE+WRITE_SIZE)",
                    "algorithmic_bytes_per_launch": round(g["bytes"] / n),
                    "kernel": "gemm (all %s MFMA matmul launches of the step)" % precision,
                    "launches_per_step": n // args.steps,
                    "avg_launch_ms": round(g["ms"] / n, 4)}
        print(f"[{precision}] per-class kernel time per step (instrumented pass, "
              f"{inst_ms:.3f} ms per step):", file=sys.stderr)
        total = 0.0
        for name, r in kci.items():
            per = r["ms"] / args.steps
            total += per
            gbs = r["bytes"] / (r["ms"] / 1e3) / 1e9 if r["ms"] > 0 else 0.0
            tf = r["flops"] / (r["ms"] / 1e3) / 1e12 if r["ms"] > 0 else 0.0
            print(f"  {name:11s} {per:9.3f} ms  launches/step {r['launches'] // args.steps:4d}"
                  f"  {tf:7.2f} TFLOP/s  {gbs:8.1f} GB/s", file=sys.stderr)
        print(f"  {'sum':11s} {total:9.3f} ms of {inst_ms:.3f} ms per step", file=sys.stderr)
    return {
        "value": round(tokens_per_s, 1),
        "ms_per_step": round(ms, 3),
        "ms_per_step_median": round(ms_median, 3),
        "dtype": {"fp32": "f32", "bf16": "bf16", "fp16": "f16"}[precision],
        "workload": "GPT-2 124M training step, B=16 T=1024 "
                    + (f"{precision} mixed precision" if half else "fp32"),
        "roofline": roofline,
        "step_roofline": step_roof,
        "kernel_ms_per_step": {k: round(v["ms"] / args.steps, 3) for k, v in kci.items()},
        "kernel_timing": None if not kc else (
            "the timed region times the matmul family only (roofline); kernel_ms_per_step "
            f"comes from a second pass of {args.steps} steps with every launch timed, "
            f"{inst_ms:.3f} ms per step there"),
        "loss_first_last": [round(timed_losses[0], 5), round(timed_losses[-1], 5)],
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this library runs on one GPU "
              f"only (no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    from transformer_lm_step_train_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    c = synth.CONFIGS[WORKLOAD]
    B, T = c["B"], c["T"]
    params = synth.init_params(c["L"], c["C"], c["V"], c["maxT"])
    if args.tokens == "zipf":
        tok, tgt = synth.zipf_tokens(B, T, c["V"])
    else:
        tok, tgt = synth.token_stream(B, T, c["V"])
    half = args.precision in ("bf16", "fp16")
    head = run_leg(args.precision, args, params, tok, tgt)

    out = {
        "metric": "training tokens/sec (fwd+bwd+AdamW), GPT-2 124M B16 T1024 at 1 GPU"
                  + ("" if not half else f" ({args.precision} mixed precision)"),
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "ms_per_step_median": head["ms_per_step_median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": f"synthetic (seeded {args.tokens} int32 token ids, GPT-2 init N(0,0.02))",
        "config": {"workload": head["workload"],
                   "global_batch": B, "seq_len": T, "layers": c["L"], "channels": c["C"],
                   "heads": c["NH"], "vocab": c["V"], "parallelism": "single GPU"},
        "roofline": head["roofline"],
        "step_roofline": head["step_roofline"],
        "cpu_baseline": None,
        "kernel_ms_per_step": head["kernel_ms_per_step"],
        "kernel_timing": head["kernel_timing"],
        "loss_first_last": head["loss_first_last"],
    }
    if not half and not args.no_mixed:
        # the mixed-precision configuration of the same workload (bf16
        # activations and matmul operands, fp32 master weights and Adam state)
        out["mixed_bf16"] = run_leg("bf16", args, params, tok, tgt)
    if not args.no_cpu_baseline and not half:
        out["cpu_baseline"] = cpu_baseline(c, params, tok, tgt)
        out["pages_shape_gpu"] = pages_shape_gpu(params)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
