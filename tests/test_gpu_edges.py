"""GPU edge cases: degenerate lengths, limits, error paths forced from the
host, batch-size boundaries between kernel families, determinism, KV-cached
decode against a full recompute on the GPU, graph argument updates."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from gpu_common import (TOL_BF16, TOL_F32, check_cache_stage, dev_f64, dev_i32, draws_must_agree,
                        gpu_prefill, kv_layer_bits, make_exact_oracle,
                        log, make_model, make_oracle, max_abs, need_gpu, tol_for)

pytestmark = pytest.mark.gpu


def small(dtype="bf16", L=2, H=4, C=256, Tb=96, V=300, bias=True, batch=4):
    return synth.Workload(f"edge_{dtype}_{C}_{H}", 11, L, H, C, Tb, V, V, bias,
                          dtype, batch=batch, prompt_len=8)


@pytest.mark.parametrize("dtype,H,C", [("bf16", 4, 256), ("bf16", 4, 128),
                                       ("f32", 4, 128), ("f32", 2, 128)])
def test_ragged_prefill_decode_head_sizes(dtype, H, C):
    """hs = 64 and 32, bf16 and fp32, biases and non-unit LayerNorm weights,
    ragged lengths including a single-token prompt."""
    need_gpu()
    w = small(dtype, H=H, C=C)
    W = synth.make_weights(w, gamma_std=0.1)
    rng = np.random.default_rng(5)
    lens = np.array([1, 17, 64, 33], np.int32)
    ids = rng.integers(0, w.vocab_size, (4, 64)).astype(np.int32)
    o = make_oracle(w, W)
    ref = [o.prefill(ids, lens)]
    m = make_model(w, W)
    kv = m.new_kv(4)
    got = [gpu_prefill(m, kv, ids, lens)]
    for s in range(6):
        t = rng.integers(0, w.vocab_size, 4).astype(np.int32)
        m.decode_feed(kv, dev_i32(t))
        got.append(m.logits(4).cpu().numpy())
        ref.append(o.decode(t))
    errs = [max_abs(a, b) for a, b in zip(got, ref)]
    log(f"  {dtype} hs={C // H}: max err {max(errs):.2e}")
    assert max(errs) < tol_for(w)


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 8, 9, 65])
def test_batch_sizes_across_kernel_families(B):
    """Decode batches on both sides of the streaming/MFMA boundary give the
    oracle's logits and every row equals the same row run alone."""
    need_gpu()
    w = small("bf16", batch=B, L=1, Tb=64)
    W = synth.make_weights(w)
    rng = np.random.default_rng(B)
    lens = rng.integers(1, 30, B).astype(np.int32)
    ids = rng.integers(0, w.vocab_size, (B, 30)).astype(np.int32)
    o = make_oracle(w, W)
    ref = o.prefill(ids, lens)
    m = make_model(w, W, max_batch=max(B, 1))
    kv = m.new_kv(B)
    got = gpu_prefill(m, kv, ids, lens)
    t = rng.integers(0, w.vocab_size, B).astype(np.int32)
    m.decode_feed(kv, dev_i32(t))
    got2 = m.logits(B).cpu().numpy()
    ref2 = o.decode(t)
    assert max_abs(got, ref) < TOL_BF16 and max_abs(got2, ref2) < TOL_BF16


def test_zero_layer_model_closed_form():
    """n_layer = 0: logits = ln_f(wte[id] + wpe[pos]) wte^T."""
    need_gpu()
    w = dataclasses.replace(small("f32", bias=True), n_layer=0)
    W = synth.make_weights(w, gamma_std=0.1)
    ids = np.array([[3, 7, 250, 1]], np.int32)
    m = make_model(w, W, max_batch=1)
    kv = m.new_kv(1)
    got = gpu_prefill(m, kv, ids, [4])
    x = W["wte"][250].astype(np.float64) + W["wpe"][2]
    ids2 = np.array([[3, 7, 250]], np.int32)
    got3 = gpu_prefill(m, kv, ids2, [3])
    z = oracle.layer_norm(x, W["lnf_w"], W["lnf_b"])
    assert max_abs(got3[0], W["wte"].astype(np.float64) @ z) < TOL_F32
    assert max_abs(got[0], make_oracle(w, W).prefill(ids, [4])[0]) < TOL_F32


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_kv_decode_matches_gpu_full_recompute(dtype):
    """Logits after prefill(p) + k fed steps equal a prefill of the whole
    p+k sequence (within the path's tolerance)."""
    need_gpu()
    w = small(dtype, batch=2)
    W = synth.make_weights(w)
    rng = np.random.default_rng(9)
    seq = rng.integers(0, w.vocab_size, (2, 40)).astype(np.int32)
    m = make_model(w, W)
    kv = m.new_kv(2)
    gpu_prefill(m, kv, seq[:, :25], [25, 25])
    for s in range(25, 40):
        m.decode_feed(kv, dev_i32(seq[:, s]))
    dec = m.logits(2).cpu().numpy()
    kv2 = m.new_kv(2)
    full = gpu_prefill(m, kv2, seq, [40, 40])
    log(f"  {dtype}: decode vs recompute {max_abs(dec, full):.2e}")
    assert max_abs(dec, full) < tol_for(w)


def test_limits_inactive_rows_and_context_error():
    torch = need_gpu()
    import gpt_decoder_amd as ng
    w = small("bf16", batch=3, Tb=32)
    W = synth.make_weights(w)
    ids = np.random.default_rng(3).integers(0, w.vocab_size, (3, 32)).astype(np.int32)
    m = make_model(w, W)
    m.set_sampling(greedy=True)
    kv = m.new_kv(3)
    m.prefill(kv, dev_i32(ids), [30, 5, 32], [31, 7, 32])
    before = m.logits(3).cpu().numpy()
    nxt = torch.empty(3, dtype=torch.int32, device="cuda")
    m.decode_step(kv, nxt, None)
    ids1 = nxt.cpu().numpy()
    assert ids1[2] == -1 and ids1[0] >= 0 and ids1[1] >= 0
    after = m.logits(3).cpu().numpy()
    np.testing.assert_array_equal(after[2], before[2])   # untouched row
    m.decode_step(kv, nxt, None)
    ids2 = nxt.cpu().numpy()
    assert ids2[0] == -1 and ids2[1] >= 0 and ids2[2] == -1
    assert kv.lens.cpu().tolist() == [31, 7, 32]
    with pytest.raises(ng.NgptError) as ei:
        m.decode_step(kv, nxt, None)
    assert ei.value.code == ng.NGPT_E_CONTEXT
    assert m.device_status() == 0


def test_host_validation_errors():
    torch = need_gpu()
    import gpt_decoder_amd as ng
    w = small("bf16", batch=2, Tb=32)
    W = synth.make_weights(w)
    m = make_model(w, W, max_prefill_tokens=40)
    kv = m.new_kv(2)
    ids = np.zeros((2, 32), np.int32)
    cases = [
        (([0, 5], None), ng.NGPT_E_RANGE),       # empty prompt
        (([33, 5], None), ng.NGPT_E_RANGE),      # longer than block_size
        (([30, 20], None), ng.NGPT_E_SIZE),      # sum above max_prefill_tokens
        (([5, 5], [4, 32]), ng.NGPT_E_RANGE),    # limit below length
        (([5, 5], [5, 33]), ng.NGPT_E_RANGE),    # limit above block_size
    ]
    for (lens, limit), code in cases:
        with pytest.raises(ng.NgptError) as ei:
            m.prefill(kv, ids, lens, limit)
        assert ei.value.code == code, (lens, limit)
    with pytest.raises(ng.NgptError) as ei:      # B larger than the kv batch
        m.prefill(kv, np.zeros((3, 4), np.int32), [4, 4, 4])
    assert ei.value.code == ng.NGPT_E_ARG
    for bad_id in (-1, w.vocab_size):            # host ids checked before the copy
        bad = np.zeros((2, 32), np.int32)
        bad[1, 3] = bad_id
        with pytest.raises(ng.NgptError) as ei:
            m.prefill(kv, bad, [5, 5])
        assert ei.value.code == ng.NGPT_E_RANGE
    bad = np.zeros((2, 32), np.int32)
    bad[1, 7] = -5                               # past lens[1]: never read
    m.prefill(kv, bad, [5, 5])
    m.set_sampling(temperature=1.0, top_k=0, greedy=False)
    m.prefill(kv, ids, [4, 4])
    nxt = torch.empty(2, dtype=torch.int32, device="cuda")
    with pytest.raises(ng.NgptError) as ei:      # sampling needs uniforms
        m.decode_step(kv, nxt, None)
    assert ei.value.code == ng.NGPT_E_ARG
    with pytest.raises(ng.NgptError):
        m.set_sampling(temperature=0.0, top_k=0, greedy=False)
    other = m.new_kv(2)                          # not the cache of the last prefill
    with pytest.raises(ng.NgptError) as ei:
        m.decode_step(other, nxt, dev_f64([0.5, 0.5]))
    assert ei.value.code == ng.NGPT_E_ARG
    assert m.device_status() == ng.NGPT_OK


def test_out_of_range_ids_are_reported_not_faulted():
    need_gpu()
    import gpt_decoder_amd as ng
    w = small("bf16", batch=1)
    m = make_model(w, synth.make_weights(w))
    kv = m.new_kv(1)
    # device ids (ngpt_prefill_device) cannot be checked on the host: the
    # kernel uses id 0 and raises the flag
    m.prefill(kv, dev_i32([[1, 2, w.vocab_size + 5, 3]]), [4])
    assert m.device_status() == ng.NGPT_E_DEVICE
    assert m.device_status() == ng.NGPT_OK       # cleared
    m.decode_feed(kv, dev_i32([-1]))
    assert m.device_status() == ng.NGPT_E_DEVICE


def test_bitwise_determinism_and_graph_argument_updates():
    """Two identical runs give bitwise-identical logits and ids; changing the
    next_ids / uniforms buffers between steps (graph node update) and the
    sampling parameters (device-resident) behaves like fresh buffers."""
    torch = need_gpu()
    w = small("bf16", batch=4, Tb=64)
    W = synth.make_weights(w)
    ids = np.random.default_rng(2).integers(0, w.vocab_size, (4, 10)).astype(np.int32)
    uni = np.random.default_rng(4).random((12, 4))

    def run(switch_buffers):
        m = make_model(w, W)
        m.set_sampling(temperature=0.9, top_k=20)
        kv = m.new_kv(4)
        m.prefill(kv, dev_i32(ids), [10] * 4)
        bufs = [torch.empty(4, dtype=torch.int32, device="cuda") for _ in range(2)]
        ubufs = [dev_f64(uni[s]) for s in range(12)]
        out, lg = [], []
        for s in range(12):
            if s == 6:
                m.set_sampling(greedy=True)
            nb = bufs[s % 2] if switch_buffers else bufs[0]
            m.decode_step(kv, nb, ubufs[s])
            out.append(nb.cpu().numpy().copy())
            lg.append(m.logits(4).cpu().numpy())
        m.close()
        return np.array(out), np.array(lg)

    a_ids, a_lg = run(False)
    b_ids, b_lg = run(True)
    np.testing.assert_array_equal(a_ids, b_ids)
    np.testing.assert_array_equal(a_lg, b_lg)
    # from step 6 on the draws are greedy: each id is the argmax of the
    # previous step's logits
    for s in range(6, 12):
        np.testing.assert_array_equal(a_ids[s], np.argmax(a_lg[s - 1], axis=1))


def test_fused_greedy_step_matches_sampler_head_node():
    """At batch 1 (bf16, head size 64) a greedy step that follows a one-launch
    forward picks its id inside the launch, from the argmax candidates the
    previous launch left behind; with top_k = 1 the same choice is made by
    the sampler head node.  Ids, logits, lens and the whole KV cache must
    agree bit for bit over a run that mixes a prefill, greedy steps, feed
    steps, switched next_ids buffers and a second prefill (which makes the
    candidates stale, so the next step must go through the head node)."""
    torch = need_gpu()
    w = small("bf16", L=3, H=4, C=256, Tb=160, V=300, bias=False, batch=1)
    W = synth.make_weights(w, gamma_std=0.1)
    # a larger (still bf16-exact) tied embedding makes the greedy ids move
    # from step to step instead of settling on one token
    W["wte"] = W["wte"] * np.float32(16.0)
    rng = np.random.default_rng(17)
    p1 = rng.integers(0, w.vocab_size, (1, 40)).astype(np.int32)
    p2 = rng.integers(0, w.vocab_size, (1, 70)).astype(np.int32)
    feed = rng.integers(0, w.vocab_size, (40,)).astype(np.int32)
    uni = rng.random((40, 1))

    def run(greedy):
        m = make_model(w, W)
        if greedy:
            m.set_sampling(greedy=True)
        else:
            m.set_sampling(temperature=1.0, top_k=1)
        kv = m.new_kv(1)
        bufs = [torch.empty(1, dtype=torch.int32, device="cuda") for _ in range(2)]
        ub = [dev_f64(uni[s]) for s in range(40)]
        m.prefill(kv, dev_i32(p1), [40])
        ids, lg = [], []
        for s in range(40):
            if s % 5 == 2:   # a fed id: the next step picks from new logits
                m.decode_feed(kv, dev_i32(feed[s:s + 1]))
            if s == 25:
                m.prefill(kv, dev_i32(p2), [70])
            nb = bufs[s % 2]
            m.decode_step(kv, nb, ub[s])
            ids.append(int(nb.cpu().numpy()[0]))
            lg.append(m.logits(1).cpu().numpy()[0].copy())
        out = (np.array(ids), np.array(lg), int(kv.lens.cpu().numpy()[0]),
               kv.k.cpu().numpy().copy(), kv.v.cpu().numpy().copy())
        assert m.device_status() == 0
        m.close()
        return out

    g_ids, g_lg, g_len, g_k, g_v = run(True)
    s_ids, s_lg, s_len, s_k, s_v = run(False)
    log(f"  fused greedy ids {g_ids[:12]}..., final length {g_len}")
    assert len(set(g_ids.tolist())) > 5, "ids too uniform to test the choice"
    np.testing.assert_array_equal(g_ids, s_ids)
    np.testing.assert_array_equal(g_lg, s_lg)
    assert g_len == s_len == 70 + (40 - 25) + 3   # feeds at steps 27, 32, 37
    # cache layout [L][B][H][Tb][64] bf16; positions past the length were
    # never written (torch.empty)
    shp = (w.n_layer, 1, w.n_head, w.block_size, w.n_embd // w.n_head)
    for a_, b_ in ((g_k, s_k), (g_v, s_v)):
        a_ = a_.view(np.uint16).reshape(shp)[:, :, :, :g_len]
        b_ = b_.view(np.uint16).reshape(shp)[:, :, :, :g_len]
        np.testing.assert_array_equal(a_, b_)
    # each greedy id is the argmax of the logits before it (lowest id on ties)
    for s in range(1, 40):
        if s % 5 == 2 or s == 25:
            continue
        assert g_ids[s] == int(np.argmax(g_lg[s - 1]))


def test_greedy_row_without_finite_maximum_same_rule_in_both_paths():
    """A logits row with no finite maximum (here all NaN, from a NaN ln_f
    gain) gives id 0 and the invalid-input flag, both from the sampler head
    node (first step after a prefill) and from the one-launch kernel's own
    greedy pick (later steps)."""
    torch = need_gpu()
    import gpt_decoder_amd as ng
    w = small("bf16", L=2, H=4, C=256, Tb=64, V=300, bias=False, batch=1)
    W = synth.make_weights(w)
    W["lnf_w"] = np.full_like(W["lnf_w"], np.nan)
    m = make_model(w, W)
    m.set_sampling(greedy=True)
    kv = m.new_kv(1)
    gpu_prefill(m, kv, np.arange(8, dtype=np.int32)[None], [8])
    assert np.isnan(m.logits(1).cpu().numpy()).all()
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    got = []
    for s in range(4):
        m.decode_step(kv, nxt, None)
        got.append(int(nxt.item()))
        assert m.device_status() == ng.NGPT_E_DEVICE, s
    assert got == [0, 0, 0, 0]
    assert kv.lens.cpu().tolist() == [12]
    m.close()


@pytest.mark.parametrize("L,H,C,Tb,plen,steps,bias", [
    (2, 1, 64, 512, 300, 6, False),     # one head; three attention items per head
    (1, 8, 512, 1024, 1000, 6, False),  # eight items per head near the block end
    (3, 12, 768, 1024, 1015, 8, False),  # GPT-2 width, positions up to 1022
    (2, 4, 256, 64, 10, 40, False),     # short block, decoded up to its limit
    (2, 12, 768, 256, 140, 12, True),   # GPT-2 width with LayerNorm and Linear biases
])
def test_one_launch_decode_shapes_against_oracle(L, H, C, Tb, plen, steps, bias):
    """Batch-1 bf16 decode with hs 64 runs as one launch per token.  Its
    work split depends on the shape and the position (row pairs per
    workgroup, attention items per head and their XCD placement, record
    merging, over-read slack at the end of each exchange buffer).  Fed
    steps and then greedy steps (which fold the argmax into the launch)
    are checked against the oracle's KV-cached decode of the same ids."""
    torch = need_gpu()
    V = 500
    w = synth.Workload(f"persist_{L}_{H}_{C}_{Tb}_{int(bias)}", 11, L, H, C, Tb, V, V, bias,
                       "bf16", batch=1, prompt_len=plen)
    W = synth.make_weights(w, gamma_std=0.1)
    rng = np.random.default_rng(C + Tb)
    ids = rng.integers(0, V, (1, plen)).astype(np.int32)
    feed = rng.integers(0, V, (steps,)).astype(np.int32)
    m = make_model(w, W)
    m.set_sampling(greedy=True)
    kv = m.new_kv(1)
    o = oracle.OracleGPT(w, W, act_bf16=True)
    worst = max_abs(gpu_prefill(m, kv, ids, [plen]), o.prefill(ids, [plen]))
    n_feed = min(steps, Tb - plen) // 2
    for s in range(n_feed):
        m.decode_feed(kv, dev_i32(feed[s:s + 1]))
        worst = max(worst, max_abs(m.logits(1).cpu().numpy(), o.decode([int(feed[s])])))
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    prev = m.logits(1).cpu().numpy()
    for s in range(n_feed, min(steps, Tb - plen)):
        m.decode_step(kv, nxt, None)
        tok = int(nxt.cpu().numpy()[0])
        assert tok == int(np.argmax(prev[0]))
        prev = m.logits(1).cpu().numpy()
        worst = max(worst, max_abs(prev, o.decode([tok])))
    assert m.device_status() == 0
    assert int(kv.lens.cpu().numpy()[0]) == plen + min(steps, Tb - plen)
    log(f"  L={L} H={H} C={C} Tb={Tb} p0={plen} bias={bias}: max logit err {worst:.2e}")
    assert worst < TOL_BF16
    m.close()


@pytest.mark.gpu
@pytest.mark.parametrize("B", [1, 3])
def test_fp32_rows_wider_than_the_streaming_kernel(B):
    """fp32 model with n_embd = 1280: the MLP projection's K = 5120 is wider
    than one streaming (GEMV) launch covers for fp32 (16 chunks of 256), so
    these small-batch rows take the tiled kernel.  Ragged prefill and fed
    decode steps match the oracle at the fp32 bar."""
    need_gpu()
    V = 65
    w = synth.Workload("fp32_wide_1280", 12, 1, 20, 1280, 16, V, V, False, "f32",
                       batch=B, prompt_len=6)
    W = synth.make_weights(w)
    rng = np.random.default_rng(1280 + B)
    ids = rng.integers(0, V, (B, 6)).astype(np.int32)
    lens = [6 - b for b in range(B)]
    m = make_model(w, W)
    m.set_sampling(greedy=True)
    kv = m.new_kv(B)
    o = oracle.OracleGPT(w, W, act_bf16=False)
    worst = max_abs(gpu_prefill(m, kv, ids, lens), o.prefill(ids, lens))
    for s in range(4):
        tok = rng.integers(0, V, (B,)).astype(np.int32)
        m.decode_feed(kv, dev_i32(tok))
        worst = max(worst, max_abs(m.logits(B).cpu().numpy(), o.decode([int(t) for t in tok])))
    assert m.device_status() == 0
    log(f"  fp32 C=1280 B={B}: max logit err {worst:.2e}")
    assert worst < TOL_F32
    m.close()


@pytest.mark.gpu
def test_one_launch_decode_wait_timeout_is_reported_and_recovered():
    """Every wait of the one-launch decode kernel is bounded.  With the limit
    set to one pass the waits give up: the launches still end, the timeout
    is reported (ahead of the id error the timed-out greedy pick raises), and
    once the limit is restored and the prompt prefilled again, decoding
    matches the oracle."""
    torch = need_gpu()
    import gpt_decoder_amd as ng
    V = 500
    w = synth.Workload("timeout_2_4_256", 13, 2, 4, 256, 64, V, V, False, "bf16",
                       batch=1, prompt_len=8)
    W = synth.make_weights(w)
    ids = np.random.default_rng(99).integers(0, V, (1, 8)).astype(np.int32)
    m = make_model(w, W)
    m.set_sampling(greedy=True)
    kv = m.new_kv(1)
    gpu_prefill(m, kv, ids, [8])
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    m.set_wait_limit(1)
    m.decode_step(kv, nxt, None)   # graph: sampler node + one-launch forward
    m.decode_step(kv, nxt, None)   # one launch with the greedy pick folded in
    assert m.device_status() == ng.NGPT_E_TIMEOUT
    assert m.device_status() == 0  # the flags were cleared
    m.set_wait_limit(0)
    o = oracle.OracleGPT(w, W, act_bf16=True)
    worst = max_abs(gpu_prefill(m, kv, ids, [8]), o.prefill(ids, [8]))
    prev = m.logits(1).cpu().numpy()
    for _ in range(6):
        m.decode_step(kv, nxt, None)
        tok = int(nxt.cpu().numpy()[0])
        assert tok == int(np.argmax(prev[0]))
        prev = m.logits(1).cpu().numpy()
        worst = max(worst, max_abs(prev, o.decode([tok])))
    assert m.device_status() == 0
    log(f"  after the timeout: max logit err {worst:.2e}")
    assert worst < TOL_BF16
    m.close()


@pytest.mark.gpu
def test_one_launch_decode_sampled_batch1():
    """Batch-1 sampled decode (temperature 0.9, top-k 40) runs the sampler
    node and the one-launch forward as one captured graph.  Every drawn id
    equals the sampler's own pick on the same logits and uniform
    (bit-exact), draws that the oracle's logits decide beyond doubt agree
    with the oracle, and the new logits match the oracle's decode of the
    drawn id."""
    torch = need_gpu()
    V, T, K, n = 500, 0.9, 40, 30
    w = synth.Workload("sampled_b1_2l768", 17, 2, 12, 768, 128, V, V, False, "bf16",
                       batch=1, prompt_len=20)
    W = synth.make_weights(w)
    ids = np.random.default_rng(5).integers(0, V, (1, 20)).astype(np.int32)
    uni = np.random.default_rng(6).random((n, 1))
    m = make_model(w, W)
    m.set_sampling(temperature=T, top_k=K)
    kv = m.new_kv(1)
    o = oracle.OracleGPT(w, W, act_bf16=True)
    ref_lg = o.prefill(ids, [20])
    got_lg = gpu_prefill(m, kv, ids, [20])
    worst = max_abs(got_lg, ref_lg)
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    need_n = 0
    for s in range(n):
        u = dev_f64(uni[s])
        want = m.sample(torch.from_numpy(got_lg.astype(np.float32)).cuda(), u).cpu().numpy()
        ref_ids, _, marg = oracle.sample_rows(ref_lg.astype(np.float32), uni[s], T, K, False)
        need = draws_must_agree(ref_lg, got_lg, marg, T, K)
        m.decode_step(kv, nxt, u)
        tok = nxt.cpu().numpy()
        assert np.array_equal(tok, want), f"step {s}: graph draw differs from the sampler's"
        assert np.array_equal(tok[need], ref_ids[need]), f"step {s}: draw differs from the oracle's"
        need_n += int(need.sum())
        ref_lg = o.decode([int(tok[0])])
        got_lg = m.logits(1).cpu().numpy()
        worst = max(worst, max_abs(got_lg, ref_lg))
    assert m.device_status() == 0
    log(f"  batch-1 sampled: max logit err {worst:.2e}; draws beyond doubt {need_n}/{n}")
    assert worst < TOL_BF16
    m.close()


@pytest.mark.gpu
@pytest.mark.parametrize("H,C", [(8, 256), (4, 256)])
def test_prefill_key_split_head_sizes(H, C):
    """A long batch-1 prompt splits the keys of its later query tiles into
    chunks whose (max, sum, output) records a second kernel merges in chunk
    order; both head sizes (32 and 64) against the oracle's prefill."""
    need_gpu()
    V, T = 300, 970    # 16 key tiles: the last query tiles take 2 chunks of 8
    w = synth.Workload(f"split_{H}_{C}", 19, 2, H, C, 1024, V, V, False, "bf16",
                       batch=1, prompt_len=T)
    W = synth.make_weights(w)
    ids = np.random.default_rng(H).integers(0, V, (1, T)).astype(np.int32)
    m = make_model(w, W)
    kv = m.new_kv(1)
    o = oracle.OracleGPT(w, W, act_bf16=True)
    err = max_abs(gpu_prefill(m, kv, ids, [T]), o.prefill(ids, [T]))
    assert m.device_status() == 0
    log(f"  hs={C // H}: {T}-token prefill, max logit err {err:.2e}")
    assert err < TOL_BF16
    m.close()


@pytest.mark.gpu
def test_one_launch_decode_stops_at_the_sequence_limit():
    """Batch 1 through the one-launch kernel (the first step behind the
    sampler node, then fused greedy steps): a prefill limit of prompt + 3
    allows exactly three steps, the fourth returns NGPT_E_CONTEXT, and the
    tokens and logits of the three match the oracle."""
    torch = need_gpu()
    import gpt_decoder_amd as ng
    V = 400
    w = synth.Workload("limit_b1_2l256", 23, 2, 4, 256, 64, V, V, False, "bf16",
                       batch=1, prompt_len=12)
    W = synth.make_weights(w)
    ids = np.random.default_rng(23).integers(0, V, (1, 12)).astype(np.int32)
    m = make_model(w, W)
    m.set_sampling(greedy=True)
    kv = m.new_kv(1)
    o = oracle.OracleGPT(w, W, act_bf16=True)
    m.prefill(kv, dev_i32(ids), [12], [15])
    ref = o.prefill(ids, [12])
    worst = max_abs(m.logits(1).cpu().numpy(), ref)
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        m.decode_step(kv, nxt, None)
        tok = int(nxt.cpu().numpy()[0])
        assert tok == int(np.argmax(ref[0]))
        ref = o.decode([tok])
        worst = max(worst, max_abs(m.logits(1).cpu().numpy(), ref))
    assert kv.lens.cpu().tolist() == [15]
    with pytest.raises(ng.NgptError) as ei:
        m.decode_step(kv, nxt, None)
    assert ei.value.code == ng.NGPT_E_CONTEXT
    assert kv.lens.cpu().tolist() == [15]
    assert m.device_status() == 0
    assert worst < TOL_BF16
    m.close()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_eight_wavefront_tiles_mid_size_prefill(dtype):
    """A packed prefill of about 2000 rows at n_embd 768 runs c_attn and c_fc
    through the eight-wavefront 128x128 tiles (more than one round of them,
    fewer than 4096 rows), with a ragged last row tile: (bf16) every row's
    layer-0 K and V against the oracle's first-block steps, and the
    last-position logits of every sequence against both oracle modes."""
    need_gpu()
    w = synth.Workload(f"edge_tiles_768_{dtype}", 12, 1, 12, 768, 512, 300, 300, True, dtype,
                       batch=4, prompt_len=8)
    W = synth.make_weights(w, gamma_std=0.1)
    rng = np.random.default_rng(77)
    lens = np.array([512, 512, 511, 500], np.int32)          # 2035 rows
    ids = rng.integers(0, w.vocab_size, (4, 512)).astype(np.int32)
    m = make_model(w, W, max_prefill_tokens=int(lens.sum()))
    kv = m.new_kv(4)
    got = gpu_prefill(m, kv, ids, lens)
    lw = W["layers"][0]
    C, hs = w.n_embd, w.n_embd // w.n_head
    kb, vb = kv_layer_bits(kv, w, 0, "k"), kv_layer_bits(kv, w, 0, "v")
    worst = 0.0
    for b in range(4 if dtype == "bf16" else 0):
        L0 = int(lens[b])
        x0 = W["wte"][ids[b, :L0]].astype(np.float64) + W["wpe"][:L0]
        h = oracle.round_bf16(oracle.layer_norm(x0, lw["ln1_w"], lw["ln1_b"]))
        qkv = oracle.linear(h, lw["attn_w"], lw["attn_b"])
        for which, bits in (("k", kb), ("v", vb)):
            off = C if which == "k" else 2 * C
            want = oracle.round_bf16(qkv[:, off:off + C]).reshape(L0, w.n_head, hs).transpose(1, 0, 2)
            _, err = check_cache_stage(bits[b][:, :L0], want)
            worst = max(worst, err)
    ref = make_oracle(w, W).prefill(ids, lens)
    ref_exact = make_exact_oracle(w, W).prefill(ids, lens)
    e1, e2 = max_abs(got, ref), max_abs(got, ref_exact)
    log(f"  2035-row {dtype} prefill: layer-0 K/V largest abs diff {worst:.2e}; logits "
        f"{e1:.2e} ({dtype} mode) / {e2:.2e} (exact)")
    assert e1 < tol_for(w) and e2 < tol_for(w)
    assert m.device_status() == 0
