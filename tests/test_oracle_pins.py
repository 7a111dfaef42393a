"""Pins for the CPU oracle: every check here compares the oracle with
something other than itself -- a closed form, a textbook value, a library
routine written by others (torch), a brute force over a tiny case, a value
printed on the pages, or an invariant the definition implies.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth
from oracle.gpt import OracleGPT, causal_attention, layer_norm, gelu, linear
from oracle.sampler import sample_row, sample_rows, topk_keep_set

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


def small_cfg(L=2, H=4, C=64, Tb=32, V=97, bias=False, dtype="f32"):
    return synth.Workload("test_small", 9, L, H, C, Tb, V, V, bias, dtype,
                          batch=2, prompt_len=8, steps=4)


# --------------------------------------------------------------------------
# bfloat16 rounding
# --------------------------------------------------------------------------

def test_round_bf16_matches_torch_conversion():
    x = rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))
    # exact float32 midpoints between neighbouring bf16 values (ties)
    mids = (rng.integers(0, 0x7F80, 2000).astype(np.uint32) << 16) | 0x8000
    mids[::2] |= np.uint32(0x80000000)   # negative ties too
    x = np.concatenate([x, mids.view(np.float32).astype(np.float64)])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle.round_bf16(x), want)


def test_round_fp16_matches_torch_conversion():
    x = np.concatenate([rng.standard_normal(20000) * 3, rng.standard_normal(2000) * 1e-5,
                        np.array([0.0, -0.0, 1.0, 65504.0, 2.0 ** -24])])
    want = torch.from_numpy(x).to(torch.float32).to(torch.float16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_fp16(x), want)
    # ties to even: 1 + 2^-11 lies halfway between 1 and 1 + 2^-10
    assert oracle.round_fp16(np.array([1 + 2.0 ** -11]))[0] == 1.0
    assert oracle.round_fp16(np.array([1 + 3 * 2.0 ** -11]))[0] == 1 + 2 * 2.0 ** -10


def test_round_bf16_ties_to_even_examples():
    # 1 + 2^-8 lies halfway between bf16 1.0 and 1 + 2^-7: even is 1.0
    assert oracle.round_bf16(np.array([1.0 + 2**-8]))[0] == 1.0
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even)
    assert oracle.round_bf16(np.array([1.0 + 3 * 2**-8]))[0] == 1.0 + 2**-6
    assert oracle.round_bf16(np.array([-2.5]))[0] == -2.5


# --------------------------------------------------------------------------
# LayerNorm
# --------------------------------------------------------------------------

@pytest.mark.parametrize("with_bias", [False, True])
def test_layer_norm_vs_torch(with_bias):
    x = rng.standard_normal((7, 96)) * 3 + 1.5
    w = 1 + 0.1 * rng.standard_normal(96)
    b = 0.1 * rng.standard_normal(96) if with_bias else None
    want = F.layer_norm(torch.from_numpy(x), (96,), torch.from_numpy(w),
                        None if b is None else torch.from_numpy(b), 1e-5).numpy()
    np.testing.assert_allclose(layer_norm(x, w, b), want, rtol=0, atol=1e-12)


def test_layer_norm_closed_forms():
    # constant row: (x - mean) = 0 so the output is exactly the bias
    b = rng.standard_normal(16)
    out = layer_norm(np.full((1, 16), 3.25), np.ones(16), b)
    np.testing.assert_array_equal(out[0], b)
    # two-element row [a, -a]: mean 0, population variance a^2
    a = 0.7
    out = layer_norm(np.array([[a, -a]]), np.ones(2), None)
    np.testing.assert_allclose(out[0], [a / math.sqrt(a * a + 1e-5),
                                        -a / math.sqrt(a * a + 1e-5)], rtol=1e-15)


def test_layer_norm_none_bias_equals_zero_bias():
    """Serving page, section 1: a None bias and a zero bias give numerically
    identical forwards."""
    x = rng.standard_normal((5, 64))
    w = 1 + 0.1 * rng.standard_normal(64)
    np.testing.assert_array_equal(layer_norm(x, w, None),
                                  layer_norm(x, w, np.zeros(64)))


def test_layer_norm_statistics():
    x = rng.standard_normal((4, 768)) * 5 - 2
    y = layer_norm(x, np.ones(768), None)
    np.testing.assert_allclose(y.mean(-1), 0, atol=1e-13)
    var = x.var(-1)
    np.testing.assert_allclose(y.var(-1), var / (var + 1e-5), rtol=1e-12)


# --------------------------------------------------------------------------
# GELU
# --------------------------------------------------------------------------

def test_gelu_textbook_values():
    # Phi(1) and Phi(-1), the standard normal CDF (textbook constants)
    np.testing.assert_allclose(gelu(np.array([1.0]))[0], 0.8413447460685429,
                               rtol=1e-15)
    np.testing.assert_allclose(gelu(np.array([-1.0]))[0], -0.15865525393145707,
                               rtol=1e-14)
    assert gelu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(gelu(np.array([10.0]))[0], 10.0, rtol=1e-15)
    assert abs(gelu(np.array([-10.0]))[0]) < 1e-20


def test_gelu_vs_torch_erf_form():
    z = rng.standard_normal(5000) * 4
    want = F.gelu(torch.from_numpy(z), approximate="none").numpy()
    np.testing.assert_allclose(gelu(z), want, rtol=1e-14, atol=1e-15)
    # the tanh approximation is measurably different: guards the variant
    tanh = F.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    assert np.max(np.abs(gelu(z) - tanh)) > 1e-4


# --------------------------------------------------------------------------
# Linear and softmax
# --------------------------------------------------------------------------

def test_linear_brute_force_and_torch():
    x = rng.standard_normal((3, 5))
    w = rng.standard_normal((4, 5))
    b = rng.standard_normal(4)
    brute = np.array([[sum(x[r, k] * w[n, k] for k in range(5)) + b[n]
                       for n in range(4)] for r in range(3)])
    np.testing.assert_allclose(linear(x, w, b), brute, rtol=1e-14)
    want = F.linear(torch.from_numpy(x), torch.from_numpy(w),
                    torch.from_numpy(b)).numpy()
    np.testing.assert_allclose(linear(x, w, b), want, rtol=1e-14)
    # weight layout is [out, in]: the transposed layout gives another result
    assert linear(x, w, None).shape == (3, 4)


def test_softmax_rows_properties():
    s = rng.standard_normal((6, 50)) * 10
    s[:, 30:] = -np.inf
    p = oracle.softmax_rows(s)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=1e-14)
    assert np.all(p[:, 30:] == 0)
    np.testing.assert_allclose(oracle.softmax_rows(s + 123.0), p, rtol=1e-12)
    want = torch.softmax(torch.from_numpy(s), -1).numpy()
    np.testing.assert_allclose(p, want, rtol=1e-12, atol=1e-300)


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def test_attention_single_position_returns_v():
    C, H = 32, 4
    q, k, v = (rng.standard_normal((1, C)) for _ in range(3))
    np.testing.assert_array_equal(causal_attention(q, k, v, H, 0), v)


def test_attention_zero_query_is_prefix_mean():
    C, H, T = 32, 4, 9
    q = np.zeros((T, C))
    k, v = rng.standard_normal((T, C)), rng.standard_normal((T, C))
    y = causal_attention(q, k, v, H, 0)
    want = np.cumsum(v, 0) / np.arange(1, T + 1)[:, None]
    np.testing.assert_allclose(y, want, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("hs", [32, 64])
def test_attention_vs_torch_sdpa(hs):
    H, T = 3, 17
    C = H * hs
    q, k, v = (rng.standard_normal((T, C)) for _ in range(3))
    y = causal_attention(q, k, v, H, 0)
    qt, kt, vt = (torch.from_numpy(a).view(T, H, hs).transpose(0, 1)
                  for a in (q, k, v))
    want = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    want = want.transpose(0, 1).reshape(T, C).numpy()
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-13)


def test_attention_cached_rows_equal_full():
    """A new row against the cache equals the same row of the full causal
    attention (serving page, KV-cache section)."""
    C, H, T = 48, 3, 12
    q, k, v = (rng.standard_normal((T, C)) for _ in range(3))
    full = causal_attention(q, k, v, H, 0)
    for t in (0, 5, T - 1):
        one = causal_attention(q[t:t + 1], k[:t + 1], v[:t + 1], H, t)
        np.testing.assert_allclose(one, full[t:t + 1], rtol=1e-13, atol=1e-15)
    # several new rows with an offset mask (chunk after a past of 4)
    part = causal_attention(q[4:9], k[:9], v[:9], H, 4)
    np.testing.assert_allclose(part, full[4:9], rtol=1e-13, atol=1e-15)


def test_attention_mask_matches_page_diagram():
    """The visible keys of each query equal the worked 4-position example of
    the model-building chapter, section 4.5."""
    want = {}
    with open(os.path.join(GOLDEN, "causal_mask_4pos.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            t, keys = line.split(":")
            want[int(t)] = [int(x) for x in keys.split()]
    T, C, H = 4, 8, 1
    q, k, v = (rng.standard_normal((T, C)) for _ in range(3))
    _, probs = causal_attention(q, k, v, H, 0, return_probs=True)
    for t in range(T):
        assert list(np.nonzero(probs[0][t])[0]) == want[t]
        np.testing.assert_allclose(probs[0][t].sum(), 1.0, rtol=1e-15)


# --------------------------------------------------------------------------
# A second, independent model built from torch modules (third opinion)
# --------------------------------------------------------------------------

BF16_POINTS = ("h1", "q", "k", "v", "y", "h2", "f", "z")


def torch_fp16(a):
    """Round a float64 tensor through torch's float32 and float16
    conversions, back to float64."""
    return a.to(torch.float32).to(torch.float16).to(torch.float64)


def torch_bf16(a):
    """Round a float64 tensor through torch's own float32 and bfloat16
    conversions (round to nearest even), back to float64."""
    return a.to(torch.float32).to(torch.bfloat16).to(torch.float64)


def torch_reference_logits(cfg, w, ids, cast_points=(), cast=None):
    """All-position logits of one sequence, written with torch.nn.functional
    from the page fragments: embedding sum, pre-LN blocks with SDPA
    (is_causal=True), exact GELU, tied bias-free head.

    ``cast_points`` names the tensors that are rounded to bfloat16 with
    torch's conversion where a bf16 data path stores them: the two
    LayerNorm outputs of a block (h1, h2), q, k, v, the attention output y,
    the GELU output f and the final LayerNorm output z.  "x" (the residual
    stream after each add, which a bf16 data path keeps in fp32) exists only
    to show that rounding it is detected.
    """
    t = lambda a: None if a is None else torch.from_numpy(np.asarray(a, np.float64))
    cp = set(cast_points)
    cast = cast or torch_bf16
    r = lambda name, a: cast(a) if name in cp else a
    C, H = cfg.n_embd, cfg.n_head
    ids_t = torch.as_tensor(np.asarray(ids), dtype=torch.long)
    T = len(ids)
    x = F.embedding(ids_t, t(w["wte"])) + F.embedding(torch.arange(T), t(w["wpe"]))
    for lw in w["layers"]:
        h = r("h1", F.layer_norm(x, (C,), t(lw["ln1_w"]), t(lw["ln1_b"]), 1e-5))
        q, k, v = F.linear(h, t(lw["attn_w"]), t(lw["attn_b"])).split(C, dim=1)
        q, k, v = r("q", q), r("k", k), r("v", v)
        q, k, v = (a.reshape(T, H, C // H).transpose(0, 1) for a in (q, k, v))
        y = F.scaled_dot_product_attention(q, k, v, is_causal=True)
        y = r("y", y.transpose(0, 1).reshape(T, C))
        x = r("x", x + F.linear(y, t(lw["attnproj_w"]), t(lw["attnproj_b"])))
        h = r("h2", F.layer_norm(x, (C,), t(lw["ln2_w"]), t(lw["ln2_b"]), 1e-5))
        f = r("f", F.gelu(F.linear(h, t(lw["fc_w"]), t(lw["fc_b"]))))
        x = r("x", x + F.linear(f, t(lw["mlpproj_w"]), t(lw["mlpproj_b"])))
    z = r("z", F.layer_norm(x, (C,), t(w["lnf_w"]), t(w["lnf_b"]), 1e-5))
    return F.linear(z, t(w["wte"])).numpy()


@pytest.mark.parametrize("bias,gamma", [(False, 0.0), (True, 0.1)])
def test_model_vs_torch_reference(bias, gamma):
    cfg = small_cfg(bias=bias)
    w = synth.make_weights(cfg, gamma_std=gamma)
    ids = rng.integers(0, cfg.vocab_size, 20)
    o = OracleGPT(cfg, w)
    mine = o.full_logits(ids, positions=list(range(20)))
    want = torch_reference_logits(cfg, w, ids)
    np.testing.assert_allclose(mine, want, rtol=0, atol=1e-11)


def test_model_tiny_char_vs_torch_reference():
    cfg = synth.workload("char_4l128_fp32")
    w = synth.make_weights(cfg)
    ids, lens = synth.make_prompts(cfg)
    o = OracleGPT(cfg, w)
    mine = o.prefill(ids, lens)
    want = torch_reference_logits(cfg, w, ids[0, :lens[0]])[-1]
    np.testing.assert_allclose(mine[0], want, rtol=0, atol=1e-11)


def test_model_zero_layers_closed_form():
    """With no blocks the model is ln_f(wte[id] + wpe[pos]) @ wte.T."""
    cfg = small_cfg(L=0)
    w = synth.make_weights(cfg, gamma_std=0.1, bias=True)
    ids = [3, 50, 7]
    o = OracleGPT(cfg, w)
    got = o.full_logits(ids, positions=[0, 1, 2])
    for p, i in enumerate(ids):
        x = w["wte"][i].astype(np.float64) + w["wpe"][p]
        mu = x.mean()
        sd = math.sqrt(((x - mu) ** 2).mean() + 1e-5)
        z = (x - mu) / sd * w["lnf_w"] + w["lnf_b"]
        np.testing.assert_allclose(got[p], w["wte"].astype(np.float64) @ z,
                                   rtol=1e-12, atol=1e-14)


def test_kv_decode_equals_full_recompute():
    """KV-cached decode (one new token per step) gives the logits of a
    full-prefix recompute at every step (serving page, KV-cache section)."""
    cfg = synth.workload("char_4l128_fp32")
    w = synth.make_weights(cfg)
    prompt = list(rng.integers(0, 65, 6))
    o = OracleGPT(cfg, w)
    toks, logits = o.generate_greedy(prompt, 10)
    seq = prompt + toks
    full = OracleGPT(cfg, w).full_logits(seq[:-1], positions=list(range(5, 15)))
    np.testing.assert_allclose(np.array(logits), full, rtol=0, atol=1e-12)


def test_extend_in_chunks_equals_full_recompute():
    """Prefill of a prefix, then chunks of several new tokens at a time (the
    causal mask offset by the past length), give the full-prefix forward's
    logits at each chunk's last position."""
    cfg = small_cfg(L=3, Tb=64, bias=True)
    w = synth.make_weights(cfg, gamma_std=0.1)
    ids = rng.integers(0, cfg.vocab_size, 50)
    o = OracleGPT(cfg, w)
    o.admit(0, ids[:7])
    cuts = [7, 8, 21, 40, 50]
    full = OracleGPT(cfg, w).full_logits(ids, positions=[c - 1 for c in cuts[1:]])
    for (a, b), want in zip(zip(cuts[:-1], cuts[1:]), full):
        np.testing.assert_allclose(o.extend(0, ids[a:b]), want, rtol=0, atol=1e-12)
    assert o.lengths() == [50]


def test_admit_restarts_one_sequence_only():
    cfg = small_cfg(L=2, Tb=32)
    w = synth.make_weights(cfg)
    ids = rng.integers(0, cfg.vocab_size, (2, 12)).astype(np.int32)
    o = OracleGPT(cfg, w)
    o.prefill(ids, [12, 12])
    o.decode([3, 4])
    fresh = o.admit(1, [5, 6, 7])
    np.testing.assert_allclose(fresh, OracleGPT(cfg, w).full_logits([5, 6, 7])[0],
                               rtol=0, atol=1e-12)
    assert o.lengths() == [13, 3]
    got = o.decode([9, 9])
    want0 = OracleGPT(cfg, w).full_logits(list(ids[0]) + [3, 9])[0]
    np.testing.assert_allclose(got[0], want0, rtol=0, atol=1e-12)


def test_window_logits_is_the_crop_of_the_last_block():
    cfg = small_cfg(L=2, Tb=16)
    w = synth.make_weights(cfg)
    toks = list(rng.integers(0, cfg.vocab_size, 40))
    o = OracleGPT(cfg, w)
    np.testing.assert_array_equal(o.window_logits(toks), o.full_logits(toks[-16:])[0])
    np.testing.assert_array_equal(o.window_logits(toks[:10]), o.full_logits(toks[:10])[0])


def test_cross_entropy_vs_torch_and_closed_forms():
    lg = rng.standard_normal((30, 50)) * 4
    tg = rng.integers(0, 50, 30)
    want = F.cross_entropy(torch.from_numpy(lg), torch.from_numpy(tg), reduction="none").numpy()
    np.testing.assert_allclose(oracle.cross_entropy_rows(lg, tg), want, rtol=0, atol=1e-12)
    # equal logits: log(V); one dominant logit on the target: ~0
    np.testing.assert_allclose(oracle.cross_entropy_rows(np.zeros((1, 65)), np.array([7])),
                               [math.log(65)], rtol=1e-15)
    big = np.zeros((1, 10)); big[0, 3] = 60.0
    assert 0 <= oracle.cross_entropy_rows(big, np.array([3]))[0] < 1e-24
    # large offsets do not overflow (the maximum is taken out)
    np.testing.assert_allclose(oracle.cross_entropy_rows(lg + 1e4, tg), want, atol=1e-9)


def test_eval_losses_shift_labels_by_one():
    """Position t is scored against ids[t+1] with the logits of position t
    (model-building chapter, section 4.6: logits drop the last position,
    labels drop the first); brute force over the positions."""
    cfg = small_cfg(L=2, Tb=32, bias=True)
    w = synth.make_weights(cfg)
    ids = list(rng.integers(0, cfg.vocab_size, 12))
    o = OracleGPT(cfg, w)
    lg, loss = o.eval_losses(ids)
    assert lg.shape == (12, cfg.vocab_size) and loss.shape == (11,)
    for t in range(11):
        p = np.exp(lg[t] - lg[t].max())
        p /= p.sum()
        np.testing.assert_allclose(loss[t], -math.log(p[ids[t + 1]]), rtol=1e-12)
    np.testing.assert_allclose(lg[5], o.full_logits(ids[:6])[0], rtol=0, atol=1e-12)


def test_batch_rows_are_independent_and_ragged():
    cfg = small_cfg(bias=True)
    w = synth.make_weights(cfg)
    ids = rng.integers(0, cfg.vocab_size, (3, 9)).astype(np.int32)
    lens = [9, 2, 5]
    o = OracleGPT(cfg, w)
    lg = o.prefill(ids, lens)
    for b in range(3):
        alone = OracleGPT(cfg, w).full_logits(ids[b, :lens[b]])
        np.testing.assert_allclose(lg[b], alone[0], rtol=0, atol=1e-12)
    # decode with one inactive row leaves its cache untouched
    out = o.decode([1, 2, 3], active=[True, False, True])
    assert np.all(np.isnan(out[1])) and o.lengths() == [10, 2, 6]


def test_causal_outputs_ignore_future_tokens():
    cfg = small_cfg(bias=True)
    w = synth.make_weights(cfg, gamma_std=0.1)
    ids = rng.integers(0, cfg.vocab_size, 12)
    ids2 = ids.copy()
    ids2[7:] = rng.integers(0, cfg.vocab_size, 5)
    o = OracleGPT(cfg, w)
    a = o.hidden_states(ids)
    b = o.hidden_states(ids2)
    for xa, xb in zip(a, b):
        np.testing.assert_array_equal(xa[:7], xb[:7])
        assert not np.array_equal(xa[7:], xb[7:])


def test_model_none_bias_equals_zero_bias():
    cfg = small_cfg()
    w = synth.make_weights(cfg)
    wz = synth.make_weights(cfg)
    C = cfg.n_embd
    wz["lnf_b"] = np.zeros(C, np.float32)
    for lw in wz["layers"]:
        for name, n in [("ln1_b", C), ("ln2_b", C), ("attn_b", 3 * C),
                        ("attnproj_b", C), ("fc_b", 4 * C), ("mlpproj_b", C)]:
            lw[name] = np.zeros(n, np.float32)
    ids = rng.integers(0, cfg.vocab_size, 10)
    np.testing.assert_array_equal(OracleGPT(cfg, w).full_logits(ids),
                                  OracleGPT(cfg, wz).full_logits(ids))


def test_weight_tying_head_reads_wte():
    """lm_head is wte (architecture analysis, section 4.1): changing one wte
    row that the input does not use changes exactly that logit, by the dot
    product of the change with ln_f(x)."""
    cfg = small_cfg()
    w = synth.make_weights(cfg)
    ids = [1, 2, 3, 4]
    base = OracleGPT(cfg, w).full_logits(ids)[0]
    w2 = synth.make_weights(cfg)
    delta = rng.standard_normal(cfg.n_embd).astype(np.float32) * 0.01
    w2["wte"][40] += delta
    got = OracleGPT(cfg, w2).full_logits(ids)[0]
    changed = np.nonzero(got != base)[0]
    assert list(changed) == [40]
    o = OracleGPT(cfg, w)
    x = o.hidden_states(ids)[-1][-1]
    z = layer_norm(x, w["lnf_w"], w["lnf_b"])
    np.testing.assert_allclose(got[40] - base[40],
                               (w2["wte"][40].astype(np.float64) - w["wte"][40]) @ z,
                               rtol=1e-9)


def test_bf16_mode_rounds_cache_and_stays_close():
    cfg = small_cfg()
    w = synth.make_weights(cfg)
    ids = rng.integers(0, cfg.vocab_size, (1, 10)).astype(np.int32)
    ob = OracleGPT(cfg, w, act_bf16=True)
    lb = ob.prefill(ids, [10])
    kc = ob.caches[0].k[1]
    np.testing.assert_array_equal(oracle.round_bf16(kc), kc)
    le = OracleGPT(cfg, w).prefill(ids, [10])
    err = np.max(np.abs(lb - le))
    assert 0 < err < 2e-2


@pytest.mark.parametrize("bias,gamma", [(False, 0.0), (True, 0.1)])
def test_bf16_mode_matches_torch_model_with_bf16_casts(bias, gamma):
    """The bf16 mode equals an independent torch model that rounds h1, q,
    k, v, y, h2, f and z through torch.bfloat16 and nothing else (3 blocks,
    with and without biases, every position)."""
    cfg = small_cfg(L=3, bias=bias)
    w = synth.make_weights(cfg, gamma_std=gamma)
    ids = rng.integers(0, cfg.vocab_size, 24)
    mine = OracleGPT(cfg, w, act_bf16=True).full_logits(ids, positions=list(range(24)))
    want = torch_reference_logits(cfg, w, ids, cast_points=BF16_POINTS)
    np.testing.assert_allclose(mine, want, rtol=0, atol=1e-9)


def test_fp16_mode_matches_torch_model_with_fp16_casts():
    """The fp16 mode equals the independent torch model rounding the same
    tensors through torch.float16 (fp16 weights, 3 blocks with biases)."""
    cfg = small_cfg(L=3, bias=True, dtype="f16")
    w = synth.make_weights(cfg, gamma_std=0.1)
    ids = rng.integers(0, cfg.vocab_size, 24)
    mine = OracleGPT(cfg, w, act_fp16=True).full_logits(ids, positions=list(range(24)))
    want = torch_reference_logits(cfg, w, ids, cast_points=BF16_POINTS, cast=torch_fp16)
    np.testing.assert_allclose(mine, want, rtol=0, atol=1e-9)
    # and it is not the bf16 mode
    other = OracleGPT(cfg, w, act_bf16=True).full_logits(ids, positions=list(range(24)))
    assert np.max(np.abs(other - mine)) > 1e-4


@pytest.mark.parametrize("dropped", BF16_POINTS + ("+x",))
def test_bf16_pin_detects_each_rounding_point(dropped):
    """The comparison above is sensitive to every rounding point: the torch
    model without any one of them (or with the residual stream rounded too)
    misses the bf16 mode by far more than the 1e-9 bar."""
    cfg = small_cfg(L=3, bias=True)
    w = synth.make_weights(cfg, gamma_std=0.1)
    ids = rng.integers(0, cfg.vocab_size, 24)
    mine = OracleGPT(cfg, w, act_bf16=True).full_logits(ids, positions=list(range(24)))
    pts = [p for p in BF16_POINTS if p != dropped] + (["x"] if dropped == "+x" else [])
    other = torch_reference_logits(cfg, w, ids, cast_points=pts)
    assert np.max(np.abs(mine - other)) > 1e-6


# --------------------------------------------------------------------------
# Parameter count (model-building chapter, sections 4.3 and 4.5)
# --------------------------------------------------------------------------

def test_parameter_counts():
    with open(os.path.join(GOLDEN, "param_counts.json")) as f:
        g = json.load(f)
    ex = g["tying_saving_example"]
    # the page: tying saves vocab x n_embd, "about 19M" for 50257 x 384
    saving = ex["vocab"] * ex["n_embd"]
    assert round(saving / 1e6) == ex["saving_millions_approx"]
    for name, wl in synth.WORKLOADS.items():
        if wl.n_layer > 12:
            continue   # keep the CPU suite small; closed form checked below
        w = synth.make_weights(wl)
        n = oracle.count_parameters(w)
        assert n == oracle.param_count_closed_form(
            wl.n_layer, wl.n_embd, wl.vocab_size, wl.block_size, wl.bias), name
        est = oracle.param_count_page_estimate(wl.n_layer, wl.n_embd,
                                               wl.vocab_size)
        assert abs(n - est) / n < 0.012, name
    # GPT-2 124M (untied head would add 50304 x 768)
    assert oracle.param_count_closed_form(12, 768, 50304, 1024, False) == 124373760
    xl = oracle.param_count_closed_form(48, 1600, 50304, 1024, False)
    assert abs(xl - oracle.param_count_page_estimate(48, 1600, 50304)) / xl < 0.012


# --------------------------------------------------------------------------
# Sampler (serving page, section 2)
# --------------------------------------------------------------------------

def test_topk_keep_set_brute_force_with_ties():
    for trial in range(200):
        V = int(rng.integers(1, 40))
        s = rng.integers(-5, 5, V).astype(np.float32)   # many ties
        k = int(rng.integers(0, 50))
        keep = topk_keep_set(s, k)
        if k == 0 or k >= V:
            assert keep.all()
            continue
        # brute force: the k-th largest value by full descending sort
        kth = sorted(s.tolist(), reverse=True)[k - 1]
        assert [bool(x) for x in keep] == [x >= kth for x in s.tolist()]
        assert keep.sum() >= k


def test_topk_one_keeps_the_maxima():
    s = np.array([1.0, 3.0, 2.0, 3.0], np.float32)
    assert list(np.nonzero(topk_keep_set(s, 1))[0]) == [1, 3]


def test_sampler_matches_definition_probabilities():
    """Sweeping u over a fine grid reproduces the probabilities the
    definition gives: scaled logits s = l / T, the kept set = values not
    below the k-th largest (found here by a full descending sort),
    probability exp(s_i - max) normalised over the kept set, zero outside."""
    V, k, T = 12, 5, 0.8
    lg = rng.standard_normal(V).astype(np.float32) * 2
    s = lg.astype(np.float64) / T
    kth = sorted(s.tolist(), reverse=True)[min(k, V) - 1]
    kept = np.array([x >= kth for x in s.tolist()])
    e = np.where(kept, np.exp(s - s.max()), 0.0)
    p = e / e.sum()
    N = 200000
    counts = np.zeros(V)
    for i in range(N):
        counts[sample_row(lg, (i + 0.5) / N, T, k, False)[0]] += 1
    np.testing.assert_allclose(counts / N, p, atol=2e-5)


def test_sampler_edges_and_greedy():
    lg = np.array([0.5, 2.0, -1.0, 2.0, 1.0], np.float32)
    # u = 0 -> first kept id; u just below 1 -> last kept id
    assert sample_row(lg, 0.0, 1.0, 0, False)[0] == 0
    assert sample_row(lg, 1 - 2**-53, 1.0, 0, False)[0] == 4
    assert sample_row(lg, 0.0, 1.0, 2, False)[0] == 1
    assert sample_row(lg, 1 - 2**-53, 1.0, 2, False)[0] == 3
    # greedy: argmax, lowest id among ties
    assert sample_row(lg, 0.3, 1.0, 0, True)[0] == 1
    # top_k larger than the vocabulary keeps everything (min(top_k, V))
    _, keep, _ = sample_row(lg, 0.3, 1.0, 200, False)
    assert keep.all()
    # a very low temperature concentrates the draw on the maxima
    ids, _, _ = sample_rows(np.tile(lg, (64, 1)), np.linspace(0, 0.999, 64),
                            1e-4, 0, False)
    assert set(ids.tolist()) <= {1, 3}


def test_sampler_temperature_is_float32_division():
    lg = rng.standard_normal(1000).astype(np.float32)
    T = 0.7
    _, keep, _ = sample_row(lg, 0.5, T, 10, False)
    s = (torch.from_numpy(lg) / torch.tensor(T, dtype=torch.float32)).numpy()
    kth = np.sort(s)[::-1][9]
    np.testing.assert_array_equal(keep, s >= kth)
