"""Serving extensions of the KV-cached generate() loop, through the C ABI,
against the CPU oracle:

* chunked prefill into a live cache (ngpt_extend): several new tokens per
  row at once, with the causal mask offset by the past length;
* continuous batching (ngpt_prefill_slots, ngpt_retire): rows finish and new
  prompts take their place while the other rows keep decoding;
* generation past block_size (ngpt_slide): generate()'s crop to the last
  block_size tokens, each step re-running the window from position 0.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_common import (TOL_BF16, TOL_F32, dev_i32, log, make_model, max_abs,
                        need_gpu, tol_for)

pytestmark = pytest.mark.gpu


def small(dtype, L=2, H=4, C=256, Tb=256, V=300, bias=True, batch=3):
    return synth.Workload(f"serve_{dtype}_{L}_{H}_{C}_{Tb}_{batch}", 41, L, H, C, Tb,
                          V, V, bias, dtype, batch=batch, prompt_len=8)


def oracle_for(w, W):
    return oracle.OracleGPT(w, W, act_bf16=(w.dtype == "bf16"))


@pytest.mark.parametrize("dtype,H,C", [("bf16", 4, 256), ("bf16", 8, 256), ("f32", 4, 128)])
def test_extend_chunks_against_oracle(dtype, H, C):
    """Rows of a batch take chunks of 1..130 new tokens at pasts that are and
    are not multiples of the 64-key tile; logits after every chunk and after
    a few decode steps match the oracle's cached forward."""
    torch = need_gpu()
    w = small(dtype, H=H, C=C)
    W = synth.make_weights(w, gamma_std=0.1)
    rng = np.random.default_rng(5)
    toks = rng.integers(0, w.vocab_size, (3, 256)).astype(np.int32)
    m = make_model(w, W, max_batch=3, max_prefill_tokens=400)
    kv = m.new_kv(3)
    o = oracle_for(w, W)
    lens0 = [5, 64, 70]
    m.prefill(kv, toks[:, :70], lens0)
    ref = o.prefill(toks[:, :70], lens0)
    errs = [max_abs(m.logits(3).cpu().numpy(), ref)]
    have = list(lens0)
    plan = [  # (rows, counts)
        ([0, 2], [1, 59]),
        ([1], [130]),
        ([2, 0, 1], [64, 17, 3]),
        ([0], [100]),
    ]
    for rows, counts in plan:
        T = max(counts)
        ids = np.zeros((len(rows), T), np.int32)
        for i, (b, c) in enumerate(zip(rows, counts)):
            ids[i, :c] = toks[b, have[b]:have[b] + c]
        m.extend(kv, rows, ids, counts)
        got = m.logits(3).cpu().numpy()
        for b, c in zip(rows, counts):
            want = o.extend(b, toks[b, have[b]:have[b] + c])
            have[b] += c
            errs.append(max_abs(got[b], want))
    assert kv.lens.cpu().tolist() == have
    # decode continues from the extended caches
    for s in range(3):
        feed = rng.integers(0, w.vocab_size, 3).astype(np.int32)
        m.decode_feed(kv, dev_i32(feed))
        errs.append(max_abs(m.logits(3).cpu().numpy(), o.decode(feed)))
    log(f"  {dtype} H={H}: extend/decode max logit err {max(errs):.2e} (lens {have})")
    assert max(errs) < tol_for(w)
    assert m.device_status() == 0
    m.close()


def test_extend_batch1_long_past_key_split():
    """Batch 1, bf16: a 300-token prompt, then a 500-token chunk (the key
    split path with a past: up to 13 key tiles per query tile, in chunks of
    8) and a 1-token chunk at position 800."""
    need_gpu()
    w = small("bf16", L=2, H=4, C=256, Tb=1024, batch=1)
    W = synth.make_weights(w)
    rng = np.random.default_rng(6)
    toks = rng.integers(0, w.vocab_size, 801).astype(np.int32)
    m = make_model(w, W, max_batch=1, max_prefill_tokens=512)
    kv = m.new_kv(1)
    o = oracle_for(w, W)
    m.prefill(kv, toks[None, :300], [300])
    errs = [max_abs(m.logits(1).cpu().numpy()[0], o.prefill(toks[None, :300], [300])[0])]
    m.extend(kv, [0], toks[None, 300:800], [500])
    errs.append(max_abs(m.logits(1).cpu().numpy()[0], o.extend(0, toks[300:800])))
    m.extend(kv, [0], toks[None, 800:801], [1])
    errs.append(max_abs(m.logits(1).cpu().numpy()[0], o.extend(0, toks[800:801])))
    log(f"  batch-1 extend with key split: errs {['%.1e' % e for e in errs]}")
    assert max(errs) < TOL_BF16
    assert kv.lens.cpu().tolist() == [801]
    m.close()


def test_continuous_batching_admit_and_retire():
    """Four rows decode greedily; row 1 is retired mid-run and a new prompt
    is admitted into its place (and later row 3's), while the other rows
    keep their caches.  Every row's ids and logits follow the oracle of its
    own sequence."""
    torch = need_gpu()
    import gpt_decoder_amd as ng
    w = small("bf16", L=2, H=4, C=256, Tb=128, batch=4)
    W = synth.make_weights(w, gamma_std=0.1)
    rng = np.random.default_rng(7)
    m = make_model(w, W, max_batch=4, max_prefill_tokens=256)
    m.set_sampling(greedy=True)
    kv = m.new_kv(4)
    o = oracle_for(w, W)
    p0 = rng.integers(0, w.vocab_size, (4, 20)).astype(np.int32)
    m.prefill(kv, p0, [20, 11, 15, 9])
    ref = o.prefill(p0, [20, 11, 15, 9])
    nxt = torch.empty(4, dtype=torch.int32, device="cuda")
    errs, n_checked = [max_abs(m.logits(4).cpu().numpy(), ref)], 0
    active = [True] * 4
    for s in range(14):
        if s == 5:
            m.retire(kv, [1])
            active[1] = False
        if s == 7:
            newp = rng.integers(0, w.vocab_size, (1, 30)).astype(np.int32)
            m.prefill_slots(kv, [1], newp, [30])
            ref[1] = o.admit(1, newp[0])
            errs.append(max_abs(m.logits(4).cpu().numpy()[1], ref[1]))
            active[1] = True
        if s == 10:
            newp = rng.integers(0, w.vocab_size, (1, 3)).astype(np.int32)
            m.prefill_slots(kv, [3], newp, [3], [60])
            ref[3] = o.admit(3, newp[0])
        m.decode_step(kv, nxt, None)
        ids = nxt.cpu().numpy()
        for b in range(4):
            if not active[b]:
                assert ids[b] == -1, (s, b)
                continue
            gap = np.sort(ref[b])[-1] - np.sort(ref[b])[-2]
            if gap > 2 * TOL_BF16:
                assert ids[b] == int(np.argmax(ref[b])), (s, b)
                n_checked += 1
        lg = m.logits(4).cpu().numpy()
        new_ref = o.decode([int(i) if i >= 0 else 0 for i in ids], active=active)
        for b in range(4):
            if active[b]:
                ref[b] = new_ref[b]
                errs.append(max_abs(lg[b], ref[b]))
    lens = kv.lens.cpu().tolist()
    assert lens == [20 + 14, 30 + 7, 15 + 14, 3 + 4], lens
    log(f"  continuous batching: max logit err {max(errs):.2e}, greedy ids checked {n_checked}")
    assert max(errs) < TOL_BF16
    assert m.device_status() == ng.NGPT_OK
    m.close()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_generation_past_block_size(dtype):
    """generate() beyond block_size: once a row's cache is full, each step
    draws the next id from the current logits (ngpt_sample) and runs the
    window of the last block_size tokens again (ngpt_slide).  Greedy ids and
    logits follow the oracle's cropped forward: every margin-qualified id
    agrees, and for the fp32 model at least 95% of the ids qualify."""
    torch = need_gpu()
    Tb = 64
    w = synth.Workload(f"crop_{dtype}", 42, 2, 4, 128 if dtype == "f32" else 256, Tb, 97, 97,
                       False, dtype, batch=2, prompt_len=16)
    W = synth.make_weights(w)
    if dtype == "f32":
        # a larger tied embedding spreads the logits, so that nearly every
        # greedy id is decided beyond the fp32 tolerance (the bf16 model keeps
        # the plain init, at which the 2e-2 bar is stated)
        W["wte"] = W["wte"] * np.float32(8.0)
    rng = np.random.default_rng(8)
    prompts = rng.integers(0, w.vocab_size, (2, 16)).astype(np.int32)
    m = make_model(w, W, max_batch=2, max_prefill_tokens=2 * Tb)
    m.set_sampling(greedy=True)
    kv = m.new_kv(2)
    m.prefill(kv, prompts, [16, 16])
    o = oracle_for(w, W)
    seqs = [list(prompts[0]), list(prompts[1])]
    nxt = torch.empty(2, dtype=torch.int32, device="cuda")
    tol = tol_for(w)
    errs, checked, steps = [], 0, 30 + (Tb - 16)
    for s in range(steps):
        lg = m.logits(2).cpu().numpy()
        want = np.stack([o.window_logits(seqs[b]) for b in range(2)])
        errs.append(max_abs(lg, want))
        if kv.lens.cpu().tolist()[0] < Tb:
            m.decode_step(kv, nxt, None)
        else:
            m.sample(m.logits(2), out=nxt)
            m.slide(kv, [0, 1], nxt)
        ids = nxt.cpu().numpy()
        for b in range(2):
            gap = np.sort(want[b])[-1] - np.sort(want[b])[-2]
            if gap > 2 * tol:
                assert ids[b] == int(np.argmax(want[b])), (s, b)
                checked += 1
            seqs[b].append(int(ids[b]))
    errs.append(max_abs(m.logits(2).cpu().numpy(),
                        np.stack([o.window_logits(seqs[b]) for b in range(2)])))
    assert kv.lens.cpu().tolist() == [Tb, Tb]
    assert len(seqs[0]) == 16 + steps > Tb
    log(f"  {dtype}: {steps} steps, {steps - (Tb - 16)} past block_size; max logit err "
        f"{max(errs):.2e}; greedy ids checked {checked}/{2 * steps}")
    assert max(errs) < tol
    if dtype == "f32":
        assert checked >= 0.95 * 2 * steps
    assert m.device_status() == 0
    m.close()


def test_serving_calls_reject_bad_arguments():
    need_gpu()
    import gpt_decoder_amd as ng
    w = small("bf16", batch=2, Tb=64)
    W = synth.make_weights(w)
    m = make_model(w, W, max_batch=2, max_prefill_tokens=100)
    kv = m.new_kv(2)
    ids = np.zeros((2, 10), np.int32)
    m.prefill(kv, ids, [10, 10], [12, 64])
    cases = [
        (lambda: m.extend(kv, [0], ids[:1], [3]), ng.NGPT_E_CONTEXT),   # past limit 12
        (lambda: m.extend(kv, [2], ids[:1], [1]), ng.NGPT_E_RANGE),     # slot out of range
        (lambda: m.extend(kv, [1, 1], ids, [1, 1]), ng.NGPT_E_ARG),     # repeated slot
        (lambda: m.extend(kv, [1], ids[:1], [0]), ng.NGPT_E_RANGE),     # empty chunk
        (lambda: m.prefill_slots(kv, [0], np.full((1, 4), w.vocab_size, np.int32), [4]),
         ng.NGPT_E_RANGE),                                               # id = vocab
        (lambda: m.slide(kv, [1], dev_i32([0, 0])), ng.NGPT_E_ARG),     # row not full
        (lambda: m.extend(m.new_kv(2), [0], ids[:1], [1]), ng.NGPT_E_ARG),  # not the recorded kv
    ]
    for fn, code in cases:
        with pytest.raises(ng.NgptError) as ei:
            fn()
        assert ei.value.code == code
    m.extend(kv, [0], ids[:1], [2])
    assert kv.lens.cpu().tolist() == [12, 10]
    m.close()
