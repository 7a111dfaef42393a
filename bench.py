"""Benchmark: KV-cached GPT-2 124M (bf16) decode and prefill on one MI355X.

A step is one whole generation of the GPT-2 124M-shaped workload: prefill of
a 128-id prompt followed by 896 greedy KV-cached decode steps (batch 1), all
through the C ABI of libngpt.  ``value`` is decode throughput over the timed
steps (generated tokens / wall time, prefill included).  The 1024-id prefill
of the same shape is timed separately and reported as prefill tokens/s.

Inputs are synthetic (seeded N(0, 0.02) bf16 weights, uniform ids) and
resident in HBM before timing starts.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, published
DECODE_KERNEL = "decode_persistent_kernel"
# the decode kernel's sources and the file that picks its launch grid: the
# counter summary is valid only for exactly these
KERNEL_SOURCES = [os.path.join(ROOT, "gpt_decoder_amd", "csrc", f)
                  for f in ("k_persist.hip", "common.hpp", "kernels.hpp", "engine.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_persistent_gpt2_124m_b1_traffic.txt")


def decode_bytes_per_step(w, pos: int) -> int:
    """Algorithmic HBM bytes of one decode step at batch 1 whose new token
    sits at position ``pos``: every weight read once (bf16), LayerNorm
    weights, and the K/V rows 0..pos of every layer."""
    C, L, V = w.n_embd, w.n_layer, w.vocab_size
    weights = 2 * (12 * L * C * C + V * C)
    ln = 2 * (2 * L + 1) * C
    kv = 2 * L * C * 2 * (pos + 1)
    return weights + ln + kv


def kernel_sources_sha256() -> str:
    """SHA-256 over the decode kernel's sources, in a fixed order."""
    import hashlib
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        h.update(open(path, "rb").read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the decode kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel
    calibration), or None when that summary was taken on a different
    version of the kernel's sources."""
    try:
        fields = dict(line.split(":", 1) for line in open(TRAFFIC_FILE)
                      if ":" in line)
        src = kernel_sources_sha256()
        if fields.get("kernel_source_sha256", "").strip() != src:
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def copy_calibration(n_mib: int = 1024, reps: int = 5):
    """A plain device copy of n_mib MiB (read n, write n), for scaling the
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    x = torch.ones(n_mib * (1 << 20) // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": n_mib * (1 << 20),
                      "reps": reps}), flush=True)


def prefill_flops(w, T: int) -> int:
    """Algorithmic FLOPs of a T-token prefill at batch 1: the four linear
    layers on T rows, causal attention (lower triangle only) and lm_head on
    the last row."""
    C, L, V = w.n_embd, w.n_layer, w.vocab_size
    return 2 * T * 12 * L * C * C + L * 2 * C * T * (T + 1) + 2 * C * V


def cpu_baseline(w, W, ids, lens, steps: int):
    """The CPU oracle, as it stands, on a bounded sample of the workload:
    prefill the 128-id prompt, then ``steps`` greedy KV-cached decode steps;
    returns decode tokens/s and the BLAS thread count."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    o = oracle.OracleGPT(w, W, act_bf16=True)
    lg = o.prefill(ids, lens)
    t0 = time.perf_counter()
    for _ in range(steps):
        lg = o.decode([int(np.argmax(lg[0]))])
    dt = time.perf_counter() - t0
    return steps / dt, cores


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--prefill-reps", type=int, default=20)
    ap.add_argument("--cpu-steps", type=int, default=192,
                    help="decode steps of the CPU-oracle sample (0: skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain copy of known size (counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not "
              "supported (the path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return

    import torch
    import gpt_decoder_amd as ng
    import synth

    torch.cuda.set_device(0)
    w = synth.workload("gpt2_124m_b1")
    wp = synth.workload("gpt2_124m_prefill1024")
    W = synth.make_weights(w)
    ids, lens = synth.make_prompts(w)
    idsP, lensP = synth.make_prompts(wp)
    n_new = w.steps

    m = ng.model_from_workload(w, W, max_batch=1, max_prefill_tokens=1024)
    m.set_sampling(greedy=True)
    kv = m.new_kv(1)
    d_ids = torch.as_tensor(ids).cuda()
    d_idsP = torch.as_tensor(idsP).cuda()
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    stream = m.stream

    def generation(ev=None, kev=None):
        m.prefill(kv, d_ids, list(lens))
        if ev is not None:
            ev[0].record(stream)
        for s in range(n_new):
            # after the first step each greedy step is one launch of the
            # decode kernel on this stream: bracket those with events
            if kev is not None and s > 0:
                kev[s - 1][0].record(stream)
            m.decode_step(kv, nxt, None)
            if kev is not None and s > 0:
                kev[s - 1][1].record(stream)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        generation()
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True),
            torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    kevs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n_new - 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        generation(evs[k], kevs[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert m.device_status() == 0
    dec_ms = np.mean([a.elapsed_time(b) for a, b in evs])
    step_us = dec_ms * 1000.0 / n_new
    # dominant kernel: the one-launch decode step, launch by launch
    k_us = np.array([[a.elapsed_time(b) * 1000.0 for a, b in kk] for kk in kevs])
    kernel_us = float(k_us.mean())
    # its algorithmic bytes: step s + 1 of a generation puts its token at
    # position 128 + s + 1
    k_bytes = float(np.mean([decode_bytes_per_step(w, 128 + s) for s in range(1, n_new)]))
    dec_gbs = k_bytes / (kernel_us * 1e-6) / 1e9
    traffic = measured_traffic()

    # prefill: 1024-token prompt, same shape
    mp = ng.model_from_workload(wp, W, max_batch=1, max_prefill_tokens=1024)
    kvp = mp.new_kv(1)
    for _ in range(3):
        mp.prefill(kvp, d_idsP, list(lensP))
    torch.cuda.synchronize()
    pa, pb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pa.record(mp.stream)
    for _ in range(args.prefill_reps):
        mp.prefill(kvp, d_idsP, list(lensP))
    pb.record(mp.stream)
    torch.cuda.synchronize()
    pre_us = pa.elapsed_time(pb) * 1000.0 / args.prefill_reps
    pre_tflops = prefill_flops(wp, 1024) / (pre_us * 1e-6) / 1e12

    cpu = None
    if args.cpu_steps > 0:
        rate, cores = cpu_baseline(w, W, ids, lens, args.cpu_steps)
        cpu = {"value": round(rate, 3), "unit": "tokens/s", "cores": cores,
               "kind": "oracle",
               "sample": f"GPT-2 124M shape, batch 1: 128-id prefill then "
                         f"{args.cpu_steps} greedy KV-cached decode steps "
                         "(numpy fp64 oracle, bf16 activation rounding)"}

    value = args.steps * n_new / elapsed
    out = {
        "metric": "decode tokens/sec + prefill tokens/sec, GPT-2 124M bf16, "
                  "1 MI355X; % roofline",
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1000.0 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) bf16 weights, uniform ids)",
        "config": {"workload": "gpt2_124m_b1: GPT-2 124M shape (12L/12H/768, "
                               "vocab 50304, block 1024, no bias), batch 1, "
                               "128-id prompt + 896 greedy KV-cached decode "
                               "steps per step",
                   "global_batch": 1, "seq_len": 1024},
        "decode_us_per_token": round(step_us, 3),
        "prefill_tokens_per_s": round(1024 / (pre_us * 1e-6), 1),
        "prefill_us_1024": round(pre_us, 2),
        "prefill_mfma_frac": round(pre_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "kernel": DECODE_KERNEL,
                     "kernel_us": round(kernel_us, 2),
                     "algorithmic_bytes_per_launch": round(k_bytes)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
