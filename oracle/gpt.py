"""Oracle GPT-2 forward with a KV cache (TEST INFRASTRUCTURE ONLY).

Plain numpy, float64 by default.  Each function follows one definition on
the pages; see the package docstring for the page list.

Precision modes.  ``act_bf16=False`` evaluates the model exactly as defined
(in the compute dtype) on the given weights.  ``act_bf16=True`` additionally
rounds to bfloat16 (``act_fp16=True``: to IEEE float16, the fp16 model of
the SDK guide's mixed-precision section) the tensors that a 16-bit data path
stores in 16 bits: the
LayerNorm outputs that feed a matrix product, q/k/v (the KV cache and the q
scratch), the attention output that feeds c_proj, the GELU output that feeds
the MLP projection, and the final LayerNorm output that feeds lm_head.  The
residual stream, attention scores/probabilities and logits stay in the
compute dtype.  Which tensors are stored in bf16 is a reading of the bf16
data path, not something the pages fix; the rounding itself is IEEE-style
round-to-nearest-even from float32, written out below.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

import numpy as np
from scipy.special import erf as _erf


# ---------------------------------------------------------------------------
# Elementary operations
# ---------------------------------------------------------------------------

def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 value (ties to even), returned as float64.

    bfloat16 keeps the top 16 bits of an IEEE float32 (1 sign, 8 exponent,
    7 mantissa bits).  The value is first rounded to float32 (as a float32
    producer would hold it), then the low 16 bits are rounded away with
    ties going to the value whose bit 16 is zero.  NaN and inf are not
    expected here and are not special-cased.
    """
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16) << np.uint64(16)
    return (u.astype(np.uint32)).view(np.float32).astype(np.float64)


def round_fp16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest IEEE binary16 value (ties to even), returned as
    float64, after first rounding to float32 (as a float32 producer holds
    it).  numpy's float32 -> float16 conversion is that rounding."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float64)


def layer_norm(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray],
               eps: float = 1e-5) -> np.ndarray:
    """LayerNorm over the last axis with an optional bias.

    Serving page, section 1: ``F.layer_norm(input, weight.shape, weight,
    bias, 1e-5)`` with ``bias=None`` when the model has no biases.  That is
    (x - mean) / sqrt(var + eps) * weight (+ bias), with the population
    variance (divide by C) and eps inside the square root.
    """
    mu = x.mean(axis=-1, keepdims=True)
    d = x - mu
    var = (d * d).mean(axis=-1, keepdims=True)
    y = d / np.sqrt(var + eps) * w
    if b is not None:
        y = y + b
    return y


def gelu(z: np.ndarray) -> np.ndarray:
    """GELU, exact form: z * Phi(z) = z/2 * (1 + erf(z / sqrt 2)).

    The pages name the activation "GELU" (architecture analysis page,
    section 4.1: Linear -> GELU -> Linear) with no approximation flag;
    ``nn.GELU()``'s default is this erf form.
    """
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def linear(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray]) -> np.ndarray:
    """``nn.Linear``: x @ w.T (+ b), with w stored [out_features, in_features]."""
    y = x @ w.T
    if b is not None:
        y = y + b
    return y


def cross_entropy_rows(logits: np.ndarray, targets: np.ndarray) -> np.ndarray:
    """Cross-entropy of each row of logits against its target id:
    log(sum_j exp(l_j)) - l_target, the log-sum-exp taken around the row
    maximum.  (Model-building chapter "第 4 章 模型构建", section 4.6: the loss
    is CrossEntropyLoss over the logits and labels.)"""
    m = np.max(logits, axis=-1, keepdims=True)
    lse = m[:, 0] + np.log(np.sum(np.exp(logits - m), axis=-1))
    return lse - logits[np.arange(len(targets)), targets]


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Softmax over the last axis, max-subtracted; -inf entries give 0."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                     n_head: int, past_len: int,
                     return_probs: bool = False):
    """Multi-head causal self-attention for new rows against a cache.

    ``q`` is [n, C] for the n new positions past_len .. past_len+n-1; ``k``
    and ``v`` are [past_len + n, C] (the cache followed by the new rows).
    Head j is the column slice [j*hs, (j+1)*hs).  Scores are q kᵀ times
    1/sqrt(hs); key u is visible to the query at position t iff u <= t (the
    lower-triangular mask of the model-building chapter, section 4.5, and the
    masked_fill with -inf of the SDK guide's manual path); softmax; times v.
    With past_len == 0 this is the ``is_causal=True`` prefill; with n == 1 it
    is the KV-cached decode step, where the single query sees every cached
    key and itself (serving page, KV-cache section).
    """
    n, C = q.shape
    T = k.shape[0]
    assert T == past_len + n
    hs = C // n_head
    scale = 1.0 / math.sqrt(hs)
    t_pos = past_len + np.arange(n)[:, None]
    u_pos = np.arange(T)[None, :]
    masked = u_pos > t_pos
    y = np.empty((n, C), dtype=q.dtype)
    probs = []
    for j in range(n_head):
        sl = slice(j * hs, (j + 1) * hs)
        s = (q[:, sl] @ k[:, sl].T) * scale
        s = np.where(masked, -np.inf, s)
        p = softmax_rows(s)
        y[:, sl] = p @ v[:, sl]
        if return_probs:
            probs.append(p)
    if return_probs:
        return y, probs
    return y


# ---------------------------------------------------------------------------
# Parameter counting (model-building chapter, section 4.3)
# ---------------------------------------------------------------------------

def count_parameters(weights: dict) -> int:
    """Number of distinct trainable values: the sum of tensor sizes.

    lm_head has no tensor of its own (it is wte, architecture analysis page,
    section 4.1), so the tied matrix is counted once.  Absent biases count 0.
    """
    n = 0
    for key in ("wte", "wpe", "lnf_w", "lnf_b"):
        if weights.get(key) is not None:
            n += weights[key].size
    for layer in weights["layers"]:
        for t in layer.values():
            if t is not None:
                n += t.size
    return n


def param_count_closed_form(n_layer: int, n_embd: int, vocab: int,
                            block_size: int, bias: bool) -> int:
    """Exact parameter count of the tied model.

    Per layer: c_attn 3C^2, c_proj C^2, MLP 4C^2 + 4C^2, two LayerNorm
    weights 2C; with biases add 3C + C + 4C + C + 2C = 11C.  Embeddings:
    wte V*C (shared with lm_head), wpe Tb*C; final LayerNorm C (+ C bias).
    """
    C, L = n_embd, n_layer
    per_layer = 12 * C * C + 2 * C + (11 * C if bias else 0)
    return L * per_layer + vocab * C + block_size * C + C + (C if bias else 0)


def param_count_page_estimate(n_layer: int, n_embd: int, vocab: int) -> int:
    """The approximation of the model-building chapter, section 4.3:
    12 * n_layer * n_embd^2 + vocab * n_embd (tied embedding counted once)."""
    return 12 * n_layer * n_embd * n_embd + vocab * n_embd


# ---------------------------------------------------------------------------
# The model
# ---------------------------------------------------------------------------

class _SeqCache:
    """Per-sequence KV cache: for each layer, K and V as [T, C] arrays
    (all heads side by side; head j is columns [j*hs, (j+1)*hs))."""

    def __init__(self, n_layer: int, C: int, dtype):
        self.k = [np.zeros((0, C), dtype) for _ in range(n_layer)]
        self.v = [np.zeros((0, C), dtype) for _ in range(n_layer)]
        self.length = 0


class OracleGPT:
    """nanoGPT GPT-2 forward used by ``generate()``, with a KV cache.

    ``weights`` is the dict produced by ``synth.make_weights`` (float32
    arrays, nn.Linear layout).  The forward of the new rows of one sequence
    at positions p0 .. p0+n-1 is (SDK guide "模型架构解析"; architecture
    analysis section 4.1; model-building chapter section 4.5):

        x = wte[ids] + wpe[positions]
        for each block:  x = x + c_proj(attn(ln_1(x)))
                         x = x + mlp_proj(GELU(c_fc(ln_2(x))))
        logits = ln_f(x_last) @ wte.T            (tied, no bias, last row)
    """

    def __init__(self, cfg, weights: dict, *, act_bf16: bool = False,
                 act_fp16: bool = False, compute_dtype=np.float64):
        self.L = cfg.n_layer
        self.H = cfg.n_head
        self.C = cfg.n_embd
        self.Tb = cfg.block_size
        self.V = cfg.vocab_size
        assert self.C % self.H == 0
        assert not (act_bf16 and act_fp16)
        self.act_bf16 = act_bf16
        self.act_fp16 = act_fp16
        self.dt = compute_dtype

        def cv(a):
            return None if a is None else np.asarray(a, dtype=self.dt)

        self.wte = cv(weights["wte"])
        self.wpe = cv(weights["wpe"])
        self.lnf_w = cv(weights["lnf_w"])
        self.lnf_b = cv(weights["lnf_b"])
        self.layers = [{k: cv(t) for k, t in layer.items()}
                       for layer in weights["layers"]]
        assert len(self.layers) == self.L
        self.caches: List[_SeqCache] = []

    # -- precision helper --------------------------------------------------
    def _act(self, a: np.ndarray) -> np.ndarray:
        if self.act_bf16:
            return round_bf16(a).astype(self.dt)
        if self.act_fp16:
            return round_fp16(a).astype(self.dt)
        return a

    # -- one block of new rows for one sequence ----------------------------
    def _forward_rows(self, ids: np.ndarray, cache: _SeqCache,
                      collect: Optional[dict] = None) -> np.ndarray:
        """Run the new rows ``ids`` (positions cache.length ..) through every
        block, appending their K/V to ``cache``; returns the final residual
        stream [n, C] (before ln_f)."""
        p0 = cache.length
        n = len(ids)
        assert p0 + n <= self.Tb, "positions beyond block_size are undefined"
        assert all(0 <= int(i) < self.V for i in ids)
        x = self.wte[np.asarray(ids)] + self.wpe[p0:p0 + n]
        C = self.C
        for l, w in enumerate(self.layers):
            h = self._act(layer_norm(x, w["ln1_w"], w["ln1_b"]))
            qkv = linear(h, w["attn_w"], w["attn_b"])
            q = self._act(qkv[:, 0:C])
            k = self._act(qkv[:, C:2 * C])
            v = self._act(qkv[:, 2 * C:3 * C])
            cache.k[l] = np.concatenate([cache.k[l], k], axis=0)
            cache.v[l] = np.concatenate([cache.v[l], v], axis=0)
            y = causal_attention(q, cache.k[l], cache.v[l], self.H, p0)
            y = self._act(y)
            x = x + linear(y, w["attnproj_w"], w["attnproj_b"])
            h2 = self._act(layer_norm(x, w["ln2_w"], w["ln2_b"]))
            f = self._act(gelu(linear(h2, w["fc_w"], w["fc_b"])))
            x = x + linear(f, w["mlpproj_w"], w["mlpproj_b"])
            if collect is not None:
                collect.setdefault("x", []).append(x.copy())
        cache.length = p0 + n
        return x

    def _head(self, x_rows: np.ndarray) -> np.ndarray:
        """ln_f then the tied, bias-free lm_head on the given rows."""
        z = self._act(layer_norm(x_rows, self.lnf_w, self.lnf_b))
        return z @ self.wte.T

    # -- public API mirroring the library's calls ---------------------------
    def prefill(self, ids: np.ndarray, lens: Sequence[int]) -> np.ndarray:
        """Process each sequence's prompt ``ids[b, :lens[b]]`` from an empty
        cache; returns the logits [B, V] at each sequence's last position."""
        B = len(lens)
        self.caches = [_SeqCache(self.L, self.C, self.dt) for _ in range(B)]
        out = np.empty((B, self.V), dtype=self.dt)
        for b in range(B):
            x = self._forward_rows(ids[b, :lens[b]], self.caches[b])
            out[b] = self._head(x[-1:])[0]
        return out

    def decode(self, tokens: Sequence[int],
               active: Optional[Sequence[bool]] = None) -> np.ndarray:
        """Feed one new token per sequence (KV-cached step); returns the new
        last-position logits [B, V].  Rows with ``active[b]`` false are left
        untouched and get NaN logits."""
        B = len(self.caches)
        out = np.full((B, self.V), np.nan, dtype=self.dt)
        for b in range(B):
            if active is not None and not active[b]:
                continue
            x = self._forward_rows(np.asarray([tokens[b]]), self.caches[b])
            out[b] = self._head(x)[0]
        return out

    def admit(self, slot: int, ids: Sequence[int]) -> np.ndarray:
        """Start sequence ``slot`` over from an empty cache with prompt
        ``ids`` (the other sequences keep their caches); returns the logits
        [V] at the prompt's last position.  Continuous batching: a finished
        sequence's place is reused (serving page, section "HF 在哪些情况下
        实际上会更好")."""
        while len(self.caches) <= slot:
            self.caches.append(_SeqCache(self.L, self.C, self.dt))
        self.caches[slot] = _SeqCache(self.L, self.C, self.dt)
        x = self._forward_rows(np.asarray(ids), self.caches[slot])
        return self._head(x[-1:])[0]

    def extend(self, slot: int, ids: Sequence[int]) -> np.ndarray:
        """Append the tokens ``ids`` to sequence ``slot``'s cache in one
        forward (a chunk of new rows with a past); returns the logits [V] at
        the last new position.  The new rows see the whole past and each
        other causally: ``causal_attention`` with past_len = the cache
        length (serving page, KV-cache section, extended to several new
        tokens)."""
        x = self._forward_rows(np.asarray(ids), self.caches[slot])
        return self._head(x[-1:])[0]

    def lengths(self) -> List[int]:
        return [c.length for c in self.caches]

    def full_logits(self, ids: Sequence[int],
                    positions: Optional[Sequence[int]] = None) -> np.ndarray:
        """Full-prefix recompute for one sequence (no cache reuse): run all of
        ``ids`` from an empty cache and return the logits at ``positions``
        (default: the last one), shape [len(positions), V]."""
        cache = _SeqCache(self.L, self.C, self.dt)
        x = self._forward_rows(np.asarray(ids), cache)
        if positions is None:
            positions = [len(ids) - 1]
        return self._head(x[np.asarray(positions)])

    def hidden_states(self, ids: Sequence[int]) -> List[np.ndarray]:
        """Residual stream after every block for one sequence (testing aid)."""
        cache = _SeqCache(self.L, self.C, self.dt)
        col: dict = {}
        self._forward_rows(np.asarray(ids), cache, collect=col)
        return col.get("x", [])

    def eval_losses(self, ids: Sequence[int]):
        """The forward with labels of the model-building chapter, section
        4.6, for one sequence: logits at every position; the last position
        is dropped and the labels (the ids themselves) are shifted by one, so
        position t is scored against ids[t + 1].  Returns (logits [T, V],
        per-position losses [T - 1])."""
        ids = list(ids)
        lg = self.full_logits(ids, positions=list(range(len(ids))))
        return lg, cross_entropy_rows(lg[:-1], np.asarray(ids[1:], dtype=np.int64))

    def window_logits(self, tokens: Sequence[int]) -> np.ndarray:
        """generate()'s crop (serving page, section 2): the logits [V] of
        the last position of the last block_size tokens, run from position
        0 with no cache."""
        return self.full_logits(list(tokens)[-self.Tb:])[0]

    def generate_greedy(self, prompt: Sequence[int], steps: int):
        """KV-cached greedy generation for one sequence: returns the new
        tokens and the logits before each choice (the choice is the argmax,
        lowest id on ties)."""
        lg = self.prefill(np.asarray([prompt]), [len(prompt)])[0]
        toks, logits = [], []
        for _ in range(steps):
            t = int(np.argmax(lg))
            toks.append(t)
            logits.append(lg)
            lg = self.decode([t])[0]
        return toks, logits
