"""Helpers shared by the GPU parity tests (not a test module).

Everything that reaches the GPU goes through the C ABI via the ctypes
binding; the expected values come from the CPU oracle run on the same seeded
inputs from ``synth``.
"""
from __future__ import annotations

import sys
import time

import numpy as np
import pytest

import oracle
import synth

TOL_F32 = 1e-4     # max-abs logit error, fp32 data path
TOL_BF16 = 2e-2    # max-abs logit error, bf16 data path
# fp16 data path: the bf16 bar scaled by the ratio of the two formats' unit
# roundoffs, 2^-11 / 2^-8 (the errors come from rounding activations to the
# 16-bit format, and fp16 keeps three more significand bits)
TOL_F16 = TOL_BF16 * 2.0 ** -3


def log(*a):
    print("[gpu-test]", *a, flush=True, file=sys.stderr)


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this environment")
    return torch


def tol_for(w) -> float:
    return {"f32": TOL_F32, "f16": TOL_F16}.get(w.dtype, TOL_BF16)


def make_oracle(w, weights):
    """The oracle in the precision mode of the workload's data path (bf16
    rounding at the bf16 storage points for bf16 workloads)."""
    return oracle.OracleGPT(w, weights, act_bf16=(w.dtype == "bf16"),
                            act_fp16=(w.dtype == "f16"))


def make_exact_oracle(w, weights):
    """The oracle evaluating the model exactly as defined (no activation
    rounding): the bf16 path is held to the same bar against it."""
    return oracle.OracleGPT(w, weights, act_bf16=False)


def kv_layer_bits(kv, w, layer, which="k"):
    """The GPU cache of one layer as bf16 bit patterns [B][H][Tb][hs]."""
    t = kv.k if which == "k" else kv.v
    a = t.cpu().numpy().view(np.uint16)
    shp = (w.n_layer, kv.batch, w.n_head, w.block_size, w.n_embd // w.n_head)
    return a[:int(np.prod(shp))].reshape(shp)[layer]


def bf16_ulp_distance(bits, values):
    """Distance in bf16 ulps between bf16 bit patterns and bf16-exact float
    values (ordered-integer difference, so +0 and -0 are 1 apart at most)."""
    vb = (np.asarray(values, np.float32).view(np.uint32) >> 16).astype(np.int64)
    gb = np.asarray(bits).astype(np.int64)

    def ordered(b):
        return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + b)
    return np.abs(ordered(gb) - ordered(vb))


def make_model(w, weights, *, max_batch=None, max_prefill_tokens=None):
    import gpt_decoder_amd as ng
    return ng.model_from_workload(w, weights, max_batch=max_batch,
                                  max_prefill_tokens=max_prefill_tokens)


def dev_i32(a):
    import torch
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def dev_f64(a):
    import torch
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.float64)).cuda()


def gpu_prefill(model, kv, ids, lens, limit=None):
    """Prefill through ngpt_prefill with host ids (checked by the library)."""
    model.prefill(kv, np.ascontiguousarray(ids, dtype=np.int32), list(lens), limit)
    return model.logits(len(lens)).cpu().numpy().astype(np.float64)


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


class Timer:
    def __init__(self, what):
        self.what = what

    def __enter__(self):
        self.t = time.time()
        return self

    def __exit__(self, *exc):
        log(f"{self.what}: {time.time() - self.t:.2f}s")


def draws_must_agree(ref_logits, got_logits, margins, temperature, top_k):
    """Which draws are decided beyond doubt by both sides' logits.

    With logit errors at most d per row, each scaled logit moves by at most
    delta = d/T and each weight exp(s_i - m) by a factor within
    exp(+-delta) (the common max cancels in the ratios).  A normalised
    running sum F = c_i/S then moves by at most
    F(1-F)(exp(2 delta) - 1) <= (exp(2 delta) - 1)/4.  A draw whose oracle
    margin exceeds twice that bound must agree.  With a top-k filter the
    k-th and (k+1)-th scaled logits must also be more than 2 delta apart, so
    that both sides keep the same set.
    """
    ref = np.asarray(ref_logits, np.float64)
    got = np.asarray(got_logits, np.float64)
    delta = np.max(np.abs(ref - got), axis=1) / temperature
    need = margins > 0.5 * (np.exp(2.0 * delta) - 1.0)
    if top_k and top_k < ref.shape[1]:
        s = np.sort(ref / temperature, axis=1)[:, ::-1]
        gap = s[:, top_k - 1] - s[:, top_k]
        need &= gap > 2.0 * delta
    return need


def greedy_must_agree(ref_logits, tol):
    """Rows whose oracle top-1 / top-2 gap exceeds twice the tolerance."""
    s = np.sort(np.asarray(ref_logits, np.float64), axis=1)
    return (s[:, -1] - s[:, -2]) > 2.0 * tol


def check_cache_stage(bits, want):
    """Compare GPU cache entries (bf16 bits) with the oracle's bf16 values.

    Every entry must lie within one bf16 ulp of the oracle's, or within
    8e-3 absolute: a LayerNorm output that rounds the other way at a bf16 tie
    (|h| up to ~5, ulp 2^-5) moves a K/V entry by up to |W| * ulp(h) ~ 3e-3,
    which is many ulps for an entry near zero.  At most 1% of entries may be
    beyond one ulp.  A wrong row, head, position or dimension moves entries
    by ~|K| ~ 0.5.  Returns (fraction beyond one ulp, largest absolute
    difference)."""
    gv = (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    d = bf16_ulp_distance(bits, want)
    err = np.abs(gv - want)
    frac = float((d > 1).mean())
    assert ((d <= 1) | (err <= 8e-3)).all(), f"max abs diff {err.max():.3e}"
    assert frac <= 0.01, f"{frac:.3e} of entries beyond one ulp"
    return frac, float(err.max())
