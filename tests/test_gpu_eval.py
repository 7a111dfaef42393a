"""The evaluation forward with labels (model-building chapter, section 4.6)
through ngpt_eval_loss, against the oracle: logits at every position, the
per-position cross-entropy against the next id (last position unscored) and
the mean.  The loss of a row moves by at most twice the row's largest logit
error (log-sum-exp moves by at most that error, the target logit by the
same), so losses and the mean are held to twice the logit bar."""
import numpy as np
import pytest

import synth
from gpu_common import (TOL_BF16, Timer, log, make_exact_oracle, make_model,
                        make_oracle, max_abs, need_gpu, tol_for)

pytestmark = pytest.mark.gpu


def check_eval(w, W, ids, lens, oracles):
    m = make_model(w, W, max_batch=len(lens), max_prefill_tokens=int(sum(lens)))
    kv = m.new_kv(len(lens))
    lg, loss, mean = m.eval_loss(kv, ids, lens)
    lg, loss, mean = lg.cpu().numpy(), loss.cpu().numpy(), float(mean.item())
    assert m.device_status() == 0
    m.close()
    tol = tol_for(w)
    out = []
    for o in oracles:
        off, all_l, errs_l, errs_s = 0, [], [], []
        for b, L in enumerate(lens):
            rl, rs = o.eval_losses(ids[b, :L])
            errs_l.append(max_abs(lg[off:off + L], rl))
            if L > 1:
                errs_s.append(max_abs(loss[off:off + L - 1], rs))
                all_l.extend(rs.tolist())
            assert loss[off + L - 1] == 0.0
            off += L
        want_mean = float(np.mean(all_l)) if all_l else 0.0
        out.append((max(errs_l), max(errs_s) if errs_s else 0.0, abs(mean - want_mean), want_mean))
        assert max(errs_l) < tol
        assert (max(errs_s) if errs_s else 0.0) < 2 * tol
        assert abs(mean - want_mean) < 2 * tol
    return out


@pytest.mark.parametrize("dtype,bias", [("f32", False), ("bf16", True)])
def test_eval_loss_small_ragged(dtype, bias):
    need_gpu()
    C = 128 if dtype == "f32" else 256
    w = synth.Workload(f"eval_{dtype}", 43, 3, 4, C, 128, 211, 211, bias, dtype,
                       batch=3, prompt_len=8)
    W = synth.make_weights(w, gamma_std=0.1)
    rng = np.random.default_rng(9)
    lens = [1, 37, 128]
    ids = rng.integers(0, w.vocab_size, (3, 128)).astype(np.int32)
    res = check_eval(w, W, ids, lens, [make_oracle(w, W)])
    log(f"  {dtype}: logits {res[0][0]:.2e}, losses {res[0][1]:.2e}, mean diff {res[0][2]:.2e} "
        f"(mean loss {res[0][3]:.4f})")


def test_eval_loss_gpt2_124m_1024():
    """One 1024-id sequence at the GPT-2 124M shape: every one of the 1024
    logits rows and 1023 losses, against both oracle modes."""
    need_gpu()
    w = synth.workload("gpt2_124m_prefill1024")
    W = synth.make_weights(w)
    ids, lens = synth.make_prompts(w)
    with Timer("  eval 1024 + oracle"):
        res = check_eval(w, W, ids, list(lens), [make_oracle(w, W), make_exact_oracle(w, W)])
    for name, r in zip(("bf16-mode", "exact"), res):
        log(f"  vs {name}: logits {r[0]:.2e}, losses {r[1]:.2e}, mean diff {r[2]:.2e} "
            f"(mean loss {r[3]:.4f})")
