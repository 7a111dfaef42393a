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
                  for f in ("k_persist.hip", "k_persist.hpp", "common.hpp")]
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
    return prefill_flops_rows(w, [T])


def prefill_flops_rows(w, lens) -> int:
    """Prefill FLOPs of prompts of the given lengths: linear layers on every
    row, causal attention of each prompt (2 C T(T+1) per layer: q k^T and
    p v over the lower triangle), lm_head on each prompt's last row."""
    C, L, V = w.n_embd, w.n_layer, w.vocab_size
    M = int(sum(lens))
    attn = sum(L * 2 * C * int(T) * (int(T) + 1) for T in lens)
    return 2 * M * 12 * L * C * C + attn + len(lens) * 2 * C * V


def eval_flops(w, T: int) -> int:
    """FLOPs of the evaluation forward over T positions: the prefill's
    linear layers and attention, and lm_head on every row."""
    C, L, V = w.n_embd, w.n_layer, w.vocab_size
    return 2 * T * 12 * L * C * C + L * 2 * C * T * (T + 1) + T * 2 * C * V


def step_weight_bytes(w) -> int:
    """Bytes of parameters one decode step reads once (16-bit): the four
    matrices of every block and the tied embedding, LayerNorm weights, and
    the biases of a model with biases."""
    C, L, V = w.n_embd, w.n_layer, w.vocab_size
    n = 12 * L * C * C + V * C + (2 * L + 1) * C
    if w.bias:
        n += L * 11 * C + C
    return 2 * n


def step_kv_bytes(w, positions) -> int:
    """K and V bytes one decode step reads: for each active row with its new
    token at position p, rows 0..p of every layer (16-bit)."""
    return sum(2 * w.n_layer * w.n_embd * 2 * (int(p) + 1) for p in positions)


def cpu_info():
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, os.cpu_count() or 1


def cpu_table(budget_s: float = 60.0):
    """The oracle timed on the host at 1 thread and at all BLAS threads on
    bounded samples of each workload: prefill tokens/s and decode tokens/s.
    Samples (per workload, at each thread count): the tiny character model
    in full (16-id prompt, 47 steps); the Shakespeare-char shape with its 8
    prompts and 8 decode steps; GPT-2 124M: the 128-id prompt and 16 steps,
    and the 1024-id prompt (prefill only); the batch-64 ragged workload on 2
    of its sequences (prefill + 4 steps); GPT-2 XL on 1 sequence of 128 ids
    (prefill + 2 steps, all threads only).  Rates of subsets are per token,
    extrapolated to the workload."""
    import oracle
    import synth
    from threadpoolctl import threadpool_limits, threadpool_info
    all_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    specs = [("char_4l128_fp32", 1, None, 47), ("char_6l384_bf16_b8", 8, None, 8),
             ("gpt2_124m_b1", 1, None, 16), ("gpt2_124m_prefill1024", 1, None, 0),
             ("gpt2_124m_bias_b64_ragged", 2, None, 4), ("gpt2_xl_b32", 1, 128, 2)]
    out = {}
    t_start = time.perf_counter()
    for name, nseq, plen, steps in specs:
        w = synth.workload(name)
        if w.n_layer > 12 and time.perf_counter() - t_start > budget_s:
            continue
        W = synth.make_weights(w)
        ids, lens = synth.make_prompts(w)
        ids, lens = ids[:nseq], lens[:nseq].copy()
        if plen:
            lens[:] = plen
            ids = ids[:, :plen]
        res = {}
        for threads in ((1, all_threads) if w.n_layer <= 12 else (all_threads,)):
            with threadpool_limits(threads):
                o = oracle.OracleGPT(w, W, act_bf16=(w.dtype == "bf16"))
                t0 = time.perf_counter()
                lg = o.prefill(ids, lens)
                tp = time.perf_counter() - t0
                t0 = time.perf_counter()
                for _ in range(steps):
                    lg = o.decode([int(np.argmax(r)) for r in lg])
                td = time.perf_counter() - t0
            res[f"threads_{threads}"] = {
                "prefill_tokens_per_s": round(float(np.sum(lens)) / tp, 2),
                "decode_tokens_per_s": round(nseq * steps / td, 2) if steps else None}
        res["sample"] = f"{nseq} sequence(s), prompt {int(lens[0])}{'+' if len(set(lens)) > 1 else ''} ids, {steps} decode steps"
        out[name] = res
    model, nproc = cpu_info()
    return {"cpu_model": model, "nproc": nproc, "blas_threads": all_threads,
            "kind": "oracle", "workloads": out}


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


def run_batched_workloads(torch, ng, synth):
    """The other workloads on the GPU, one generation each after a warm-up:
    the batch-64 ragged workload with biases (prefill of all prompts, then
    top-k 50 sampled decode until every row holds 1024 tokens), the GPT-2 XL
    shape at batch 32 (512-id prompts, 512 greedy steps), the
    Shakespeare-char shape at batch 8 (64-id prompts, 192 sampled steps),
    and the evaluation forward with labels over one 1024-id sequence.  The
    batch-64 workload runs twice: on a contiguous cache and on a paged one
    (64-position pages in a shuffled order).  Decode is reported against HBM
    (bytes the steps must read) and, for the large batches, MFMA (their
    matrix-product FLOPs); prefill against MFMA."""
    res = {}

    def ev():
        return torch.cuda.Event(enable_timing=True)

    runs = (("gpt2_124m_bias_b64_ragged", False), ("gpt2_124m_bias_b64_ragged", True),
            ("gpt2_xl_b32", False), ("char_6l384_bf16_b8", False))
    for name, paged in runs:
        w = synth.workload(name)
        W = synth.make_weights(w)
        ids, lens = synth.make_prompts(w)
        steps = synth.decode_steps(w, lens)
        uni = torch.as_tensor(synth.make_uniforms(w, steps)).cuda()
        m = ng.model_from_workload(w, W, max_prefill_tokens=int(lens.sum()))
        if w.greedy:
            m.set_sampling(greedy=True)
        else:
            m.set_sampling(temperature=w.temperature, top_k=w.top_k)
        if paged:
            nblk = (w.block_size + 63) // 64
            kv = m.new_kv(w.batch, num_pages=w.batch * nblk)
            order = np.random.default_rng(w.index).permutation(w.batch * nblk)
            for b in range(w.batch):
                m.kv_map(kv, b, 0, order[b * nblk:(b + 1) * nblk])
        else:
            kv = m.new_kv(w.batch)
        nxt = torch.empty(w.batch, dtype=torch.int32, device="cuda")
        d_ids = torch.as_tensor(ids).cuda()
        t = {}
        for rep in range(2):        # warm-up, then the timed generation
            a, b, c = ev(), ev(), ev()
            a.record(m.stream)
            m.prefill(kv, d_ids, list(lens))
            b.record(m.stream)
            for s in range(steps):
                m.decode_step(kv, nxt, uni[s])
            c.record(m.stream)
            torch.cuda.synchronize()
            t = {"prefill_ms": a.elapsed_time(b), "decode_ms": b.elapsed_time(c)}
        assert m.device_status() == 0
        m.close()
        del kv
        C, L, V = w.n_embd, w.n_layer, w.vocab_size
        limit = w.decode_to if w.decode_to else int(lens.max()) + steps
        new_tokens = int(sum(min(limit, int(l) + steps) - int(l) for l in lens))
        pos_bytes, flops = 0, 0
        for s in range(steps):
            act = [int(l) + s for l in lens if int(l) + s < limit]
            pos_bytes += step_weight_bytes(w) + step_kv_bytes(w, act)
            flops += len(act) * (2 * (12 * L * C * C + V * C)) + sum(4 * L * C * (p + 1) for p in act)
        dec_s = t["decode_ms"] / 1e3
        pre_flops = prefill_flops_rows(w, [int(l) for l in lens])
        r = {"workload": w.description + (", paged KV cache" if paged else ""),
             "prefill_tokens_per_s": round(float(lens.sum()) / (t["prefill_ms"] / 1e3), 1),
             "prefill_ms": round(t["prefill_ms"], 3),
             "prefill_mfma_frac": round(pre_flops / (t["prefill_ms"] / 1e3) / 1e12
                                        / MFMA_BF16_PEAK_TFLOPS, 4),
             "decode_tokens_per_s": round(new_tokens / dec_s, 1),
             "decode_us_per_step": round(t["decode_ms"] * 1e3 / steps, 2),
             "decode_steps": steps,
             "decode_hbm_frac": round(pos_bytes / dec_s / 1e9 / HBM_PEAK_GBS, 4),
             "decode_mfma_frac": round(flops / dec_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
        key = name + ("_paged" if paged else "")
        res[key] = r
        print(json.dumps({"batched": key, **r}), file=sys.stderr, flush=True)

    # evaluation forward with labels over 1024 positions
    wp = synth.workload("gpt2_124m_prefill1024")
    W = synth.make_weights(wp)
    ids, lens = synth.make_prompts(wp)
    m = ng.model_from_workload(wp, W, max_batch=1, max_prefill_tokens=1024)
    kv = m.new_kv(1)
    lg = torch.empty((1024, wp.vocab_size), dtype=torch.float32, device="cuda")
    for _ in range(2):
        m.eval_loss(kv, ids, list(lens), logits=lg)
    torch.cuda.synchronize()
    a, b = ev(), ev()
    reps = 10
    a.record(m.stream)
    for _ in range(reps):
        m.eval_loss(kv, ids, list(lens), logits=lg)
    b.record(m.stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    m.close()
    res["eval_1024"] = {"workload": "GPT-2 124M shape, one 1024-id sequence, logits at every "
                                    "position and the shifted cross-entropy",
                        "us": round(us, 2),
                        "tokens_per_s": round(1024 / (us * 1e-6), 1),
                        "mfma_frac": round(eval_flops(wp, 1024) / (us * 1e-6) / 1e12
                                           / MFMA_BF16_PEAK_TFLOPS, 4)}
    return res


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
    ap.add_argument("--no-batched", dest="batched", action="store_false",
                    help="skip the batched workloads (batch 8 / 64 / XL 32) and the eval forward")
    ap.add_argument("--cpu-table", type=float, default=60.0,
                    help="seconds budget of the CPU-oracle table (0: skip)")
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

    def generation(ev=None):
        m.prefill(kv, d_ids, list(lens))
        if ev is not None:
            ev[0].record(stream)
        for s in range(n_new):
            m.decode_step(kv, nxt, None)
            # after the first step (the graph with the sampler head node)
            # each greedy step is one launch of the decode kernel on this
            # stream, back to back: ev[1] .. ev[2] spans launches 2..n_new
            # (one event pair per launch would add its own gaps)
            if ev is not None and s == 0:
                ev[1].record(stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        generation()
    torch.cuda.synchronize()

    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        generation(evs[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert m.device_status() == 0
    dec_ms = np.mean([e[0].elapsed_time(e[2]) for e in evs])
    step_us = dec_ms * 1000.0 / n_new
    # dominant kernel: the one-launch decode step; its mean launch time over
    # launches 2..n_new of every timed generation (inter-launch gaps, if
    # any, counted in)
    kernel_us = float(np.mean([e[1].elapsed_time(e[2]) * 1000.0 / (n_new - 1) for e in evs]))
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

    extra = run_batched_workloads(torch, ng, synth) if args.batched else {}

    cpu = None
    if args.cpu_steps > 0:
        rate, cores = cpu_baseline(w, W, ids, lens, args.cpu_steps)
        model, nproc = cpu_info()
        cpu = {"value": round(rate, 3), "unit": "tokens/s", "cores": cores,
               "kind": "oracle", "nproc": nproc, "cpu_model": model,
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
    out.update(extra)
    if cpu is not None and args.cpu_table > 0:
        out["cpu_table"] = cpu_table(args.cpu_table)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
