"""Host checks of the figures bench.py reports: the algorithmic bytes of a
decode step (the HBM roofline's numerator), the FLOPs of a prefill (the MFMA
fraction's numerator) and the rule that ties the committed counter summary to
the decode kernel's sources.  No GPU."""
import os

import numpy as np

import bench
import synth


def _tiny_bf16():
    w = synth.Workload("tiny_bench", 5, 3, 2, 64, 32, 97, 97, False, "bf16",
                       batch=1, prompt_len=4)
    return w, synth.make_weights(w)


def test_decode_bytes_equal_a_count_of_what_one_step_reads():
    """One batch-1 decode step reads every matrix once (bf16), the LayerNorm
    scales, the tied wte once more as lm_head, and the K/V rows 0..pos of
    every layer.  Counted here from the weight tensors themselves."""
    w, W = _tiny_bf16()
    weights = W["wte"].size + W["lnf_w"].size
    for lw in W["layers"]:
        for name in ("ln1_w", "attn_w", "attnproj_w", "ln2_w", "fc_w", "mlpproj_w"):
            weights += lw[name].size
    for pos in (0, 5, w.block_size - 1):
        kv = w.n_layer * 2 * (pos + 1) * w.n_embd      # K and V rows, all heads
        assert bench.decode_bytes_per_step(w, pos) == 2 * (weights + kv)


def test_decode_bytes_of_the_benchmark_generation():
    """The bench divides by the mean over the 895 timed launches of a
    generation (new tokens at positions 129..1023) of the GPT-2 124M shape."""
    w = synth.workload("gpt2_124m_b1")
    mean = np.mean([bench.decode_bytes_per_step(w, 128 + s) for s in range(1, 896)])
    assert mean == 268445184
    # weights alone: 247.2 MB
    assert bench.decode_bytes_per_step(w, -1) == 2 * (12 * 12 * 768 ** 2 + 50304 * 768 + 25 * 768)


def test_prefill_flops_equal_a_loop_count():
    """Two FLOPs per multiply-add: the four linear layers on every row,
    q.k and p.v over each row's visible keys (causal), and lm_head on the
    last row only."""
    w, _ = _tiny_bf16()
    C, L, V, T = w.n_embd, w.n_layer, w.vocab_size, 9
    flops = 0
    for _ in range(L):
        flops += T * 2 * C * (3 * C + C + 4 * C + 4 * C)
        for t in range(T):
            flops += 2 * 2 * C * (t + 1)    # scores and weighted values, all heads
    flops += 2 * C * V
    assert bench.prefill_flops(w, T) == flops


def test_batched_counts_equal_loop_counts():
    """The batched workloads' numerators: a step reads every parameter once
    (with biases when the model has them) plus each active row's K/V rows;
    ragged prefill FLOPs sum each prompt's lower triangle; the evaluation
    forward adds lm_head on every row."""
    w = synth.Workload("tiny_bias", 6, 2, 2, 64, 32, 97, 97, True, "bf16", batch=3,
                       prompt_len=4)
    W = synth.make_weights(w)
    n = W["wte"].size + W["lnf_w"].size + W["lnf_b"].size
    for lw in W["layers"]:
        n += sum(t.size for t in lw.values() if t is not None)
    assert bench.step_weight_bytes(w) == 2 * n
    pos = [3, 7, 0]
    assert bench.step_kv_bytes(w, pos) == sum(2 * 2 * w.n_layer * w.n_embd * (p + 1) for p in pos)
    lens = [5, 9, 1]
    assert bench.prefill_flops_rows(w, lens) == (
        sum(bench.prefill_flops(w, T) for T in lens))
    C, L, V, T = w.n_embd, w.n_layer, w.vocab_size, 9
    assert bench.eval_flops(w, T) == bench.prefill_flops(w, T) + (T - 1) * 2 * C * V


def test_traffic_summary_is_used_only_for_the_current_kernel_sources(tmp_path, monkeypatch):
    good = tmp_path / "good.txt"
    good.write_text(f"kernel_source_sha256: {bench.kernel_sources_sha256()}\n"
                    "traffic_bytes_per_launch: 123456\n")
    stale = tmp_path / "stale.txt"
    stale.write_text("kernel_source_sha256: " + "0" * 64 + "\n"
                     "traffic_bytes_per_launch: 123456\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(good))
    assert bench.measured_traffic() == 123456
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(stale))
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic() is None


def test_committed_traffic_summary_matches_the_sources():
    """The summary under profiles/ was taken on exactly these sources."""
    assert os.path.exists(bench.TRAFFIC_FILE)
    assert bench.measured_traffic() is not None
