"""The fp16 model (IEEE float16 weights, KV cache and matrix-product
inputs; fp32 residual, statistics, softmax and logits) through the C ABI,
against the oracle's fp16 mode and its exact mode, at the fp16 bar (the
bf16 bar scaled by the ratio of unit roundoffs, see gpu_common)."""
import numpy as np
import pytest

import synth
from gpu_common import (TOL_F16, Timer, dev_i32, greedy_must_agree, log,
                        make_exact_oracle, make_model, make_oracle, max_abs,
                        need_gpu)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("L,H,C,bias", [(3, 4, 256, True), (2, 8, 256, False), (2, 6, 384, False)])
def test_fp16_ragged_prefill_feed_and_greedy(L, H, C, bias):
    torch = need_gpu()
    w = synth.Workload(f"f16_{L}_{H}_{C}", 44, L, H, C, 256, 300, 300, bias, "f16",
                       batch=3, prompt_len=8)
    W = synth.make_weights(w, gamma_std=0.1)
    rng = np.random.default_rng(10)
    ids = rng.integers(0, w.vocab_size, (3, 200)).astype(np.int32)
    lens = [7, 130, 200]
    m = make_model(w, W, max_batch=3, max_prefill_tokens=400)
    kv = m.new_kv(3)
    o, ox = make_oracle(w, W), make_exact_oracle(w, W)
    m.prefill(kv, ids, lens)
    got = [m.logits(3).cpu().numpy()]
    ref, rex = [o.prefill(ids, lens)], [ox.prefill(ids, lens)]
    for s in range(6):
        feed = rng.integers(0, w.vocab_size, 3).astype(np.int32)
        m.decode_feed(kv, dev_i32(feed))
        got.append(m.logits(3).cpu().numpy())
        ref.append(o.decode(feed))
        rex.append(ox.decode(feed))
    # greedy decode_step: every margin-qualified id is the oracle's argmax
    m.set_sampling(greedy=True)
    nxt = torch.empty(3, dtype=torch.int32, device="cuda")
    checked = 0
    for s in range(6):
        m.decode_step(kv, nxt, None)
        t = nxt.cpu().numpy()
        need = greedy_must_agree(ref[-1], TOL_F16)
        assert (t[need] == np.argmax(ref[-1], axis=1)[need]).all(), s
        checked += int(need.sum())
        got.append(m.logits(3).cpu().numpy())
        ref.append(o.decode(t))
        rex.append(ox.decode(t))
    e = max(max_abs(a, b) for a, b in zip(got, ref))
    ex = max(max_abs(a, b) for a, b in zip(got, rex))
    log(f"  fp16 L={L} H={H} C={C}: vs fp16-mode {e:.2e}, vs exact {ex:.2e}; greedy checked {checked}")
    assert e < TOL_F16
    assert ex < TOL_F16
    assert m.device_status() == 0
    m.close()


def test_fp16_gpt2_124m_prefill_1024_and_decode():
    """GPT-2 124M shape in fp16: the 1024-id prompt, then 8 fed decode
    steps at batch 1 (the graph path)."""
    need_gpu()
    base = synth.workload("gpt2_124m_prefill1024")
    w = synth.Workload("gpt2_124m_f16", base.index, 12, 12, 768, 1024, 50304, 50257, False,
                       "f16", batch=1, prompt_len=1000)
    W = synth.make_weights(w)
    ids, lens = synth.make_prompts(w)
    feed = synth.make_feed_tokens(w, 8)
    with Timer("  oracle, both modes"):
        o, ox = make_oracle(w, W), make_exact_oracle(w, W)
        ref = [o.prefill(ids, lens)] + [o.decode(feed[s]) for s in range(8)]
        rex = [ox.prefill(ids, lens)] + [ox.decode(feed[s]) for s in range(8)]
    m = make_model(w, W, max_batch=1, max_prefill_tokens=1024)
    kv = m.new_kv(1)
    m.prefill(kv, ids, list(lens))
    got = [m.logits(1).cpu().numpy()]
    for s in range(8):
        m.decode_feed(kv, dev_i32(feed[s]))
        got.append(m.logits(1).cpu().numpy())
    e = max(max_abs(a, b) for a, b in zip(got, ref))
    ex = max(max_abs(a, b) for a, b in zip(got, rex))
    log(f"  fp16 124M: vs fp16-mode {e:.2e}, vs exact {ex:.2e}")
    assert e < TOL_F16
    assert ex < TOL_F16
    m.close()


def test_fp16_eval_loss():
    need_gpu()
    w = synth.Workload("f16_eval", 45, 2, 4, 256, 128, 211, 211, True, "f16", batch=2,
                       prompt_len=8)
    W = synth.make_weights(w)
    ids = np.random.default_rng(11).integers(0, w.vocab_size, (2, 100)).astype(np.int32)
    lens = [100, 33]
    m = make_model(w, W, max_batch=2, max_prefill_tokens=200)
    kv = m.new_kv(2)
    lg, loss, mean = m.eval_loss(kv, ids, lens)
    lg, loss = lg.cpu().numpy(), loss.cpu().numpy()
    o = make_oracle(w, W)
    off, errs, all_l = 0, [], []
    for b, L in enumerate(lens):
        rl, rs = o.eval_losses(ids[b, :L])
        errs.append((max_abs(lg[off:off + L], rl), max_abs(loss[off:off + L - 1], rs)))
        all_l += rs.tolist()
        off += L
    md = abs(float(mean.item()) - float(np.mean(all_l)))
    log(f"  fp16 eval: logits {max(e[0] for e in errs):.2e}, losses {max(e[1] for e in errs):.2e}, "
        f"mean {md:.2e}")
    assert max(e[0] for e in errs) < TOL_F16
    assert max(e[1] for e in errs) < 2 * TOL_F16
    assert md < 2 * TOL_F16
    m.close()
