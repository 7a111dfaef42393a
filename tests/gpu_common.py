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


def log(*a):
    print("[gpu-test]", *a, flush=True, file=sys.stderr)


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this environment")
    return torch


def tol_for(w) -> float:
    return TOL_F32 if w.dtype == "f32" else TOL_BF16


def make_oracle(w, weights):
    return oracle.OracleGPT(w, weights, act_bf16=(w.dtype == "bf16"))


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
    model.prefill(kv, dev_i32(ids), list(lens), limit)
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
