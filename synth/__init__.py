"""Seeded synthetic inputs for the GPT-2 decoder workloads.

This module only draws random numbers and lays them out.  It holds none of
the model's arithmetic: no LayerNorm, no matrix product, no attention, no
sampling.  Both the CPU oracle (``oracle/``) and the HIP path
(``gpt_decoder_amd``) consume what it returns, so it is the one piece of
code the two sides share.

Workload shapes follow the pages:

* the GPTConfig dataclass of the nanoGPT SDK guide (page "极速上手nanoGPT",
  section "模型架构解析"/GPTConfig): block_size 1024, vocab_size 50304
  (50257 padded to a multiple of 64), 12 layers, 12 heads, n_embd 768;
* the Shakespeare-char quick-start models of the same page (section
  "快速开始"): 6 layers/6 heads/384 wide with a 256 context on a GPU,
  4 layers/4 heads/128 wide with a 64 context on a CPU;
* gpt2-xl, one of the four pretrained sizes named in the architecture
  analysis page ("nanoGPT 架构分析", section 4.1), at 48 layers, 25 heads,
  1600 wide.

Initialisation follows the pages: N(0, 0.02) weights (framework guide page
"LLM研究框架选择指南", FAQ section), LayerNorm weight = ones and bias = zeros
or absent (serving page "原生 nanoGPT 模型服务首选", section 1, LayerNorm
fragment), and the residual projections scaled by 1/sqrt(2 n_layer)
(architecture analysis page, section 4.1) for the tiny character model.

Token ids stand in for text: they are uniform over the real vocabulary
(65 characters or 50257 BPE ids).  The datasets and trained checkpoints the
pages train on are not used.

Generator recipe: numpy ``default_rng([seed, tensor_index])`` per tensor;
``standard_normal * std`` in float64, rounded to float32, then to bfloat16
(round to nearest even, done by torch's dtype conversion) for bf16
workloads.  Seeds for workload i: weights 1000+i, prompts 2000+i,
uniforms 3000+i, teacher-forcing tokens 4000+i.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "make_weights", "make_prompts",
    "make_uniforms", "make_feed_tokens", "make_logits", "param_names",
    "LAYER_TENSORS",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int                 # seed offset
    n_layer: int
    n_head: int
    n_embd: int
    block_size: int
    vocab_size: int            # padded vocabulary (logit width)
    vocab_real: int            # ids drawn from [0, vocab_real)
    bias: bool
    dtype: str                 # "f32", "bf16" or "f16"
    batch: int
    prompt_len: int            # fixed prompt length (0 => ragged, see lens)
    prompt_len_lo: int = 0     # ragged prompt lengths uniform in [lo, hi]
    prompt_len_hi: int = 0
    decode_to: int = 0         # each sequence is decoded to this total length
    steps: int = 0             # decode steps (new tokens) for fixed prompts
    temperature: float = 1.0
    top_k: int = 0             # 0 => no top-k filter
    greedy: bool = True
    scaled_proj_init: bool = False
    description: str = ""

    @property
    def head_dim(self) -> int:
        return self.n_embd // self.n_head

    @property
    def ragged(self) -> bool:
        return self.prompt_len == 0


WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    Workload("char_4l128_fp32", 1, 4, 4, 128, 64, 65, 65, False, "f32",
             batch=1, prompt_len=16, steps=48, greedy=True,
             scaled_proj_init=True,
             description="tiny character GPT, fp32, batch 1, 16-id prompt, "
                         "48 greedy KV-cached steps"),
    Workload("char_6l384_bf16_b8", 2, 6, 6, 384, 256, 65, 65, False, "bf16",
             batch=8, prompt_len=64, steps=192, temperature=0.8, top_k=200,
             greedy=False,
             description="Shakespeare-char-shaped GPT, bf16, batch 8, 64-id "
                         "prompts, 192 sampled steps (T=0.8, top_k=200)"),
    Workload("gpt2_124m_b1", 3, 12, 12, 768, 1024, 50304, 50257, False, "bf16",
             batch=1, prompt_len=128, steps=896, greedy=True,
             description="GPT-2 124M shape, bf16, batch 1, 128-id prompt, "
                         "896 greedy KV-cached steps"),
    Workload("gpt2_124m_bias_b64_ragged", 4, 12, 12, 768, 1024, 50304, 50257,
             True, "bf16", batch=64, prompt_len=0, prompt_len_lo=32,
             prompt_len_hi=512, decode_to=1024, temperature=1.0, top_k=50,
             greedy=False,
             description="GPT-2 124M shape with biases, bf16, batch 64, "
                         "prompt lengths uniform in [32,512], each decoded "
                         "to 1024 tokens (T=1.0, top_k=50)"),
    Workload("gpt2_xl_b32", 5, 48, 25, 1600, 1024, 50304, 50257, False, "bf16",
             batch=32, prompt_len=512, steps=512, greedy=True,
             description="GPT-2 XL shape, bf16, batch 32, 512-id prompts, "
                         "512 greedy KV-cached steps"),
    Workload("gpt2_124m_prefill1024", 6, 12, 12, 768, 1024, 50304, 50257,
             False, "bf16", batch=1, prompt_len=1024, steps=0, greedy=True,
             description="GPT-2 124M shape, bf16, batch 1, one 1024-id "
                         "prompt (prefill only)"),
]}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


# Fixed per-layer tensor order; the index of a tensor in the generator is
# its position in this enumeration whether or not it is drawn, so that the
# bias=False and bias=True variants of one shape share their weights.
LAYER_TENSORS = ["attn_w", "attn_b", "attnproj_w", "attnproj_b", "fc_w",
                 "fc_b", "mlpproj_w", "mlpproj_b", "ln1_b", "ln2_b",
                 "ln1_w", "ln2_w"]


def param_names(n_layer: int) -> List[str]:
    names = ["wte", "wpe"]
    for l in range(n_layer):
        names += [f"h{l}.{t}" for t in LAYER_TENSORS]
    names += ["lnf_b", "lnf_w"]
    return names


def _to_bf16_values(a32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 (round to nearest even) -> float32, via torch."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _to_f16_values(a32: np.ndarray) -> np.ndarray:
    """float32 -> float16 (round to nearest even) -> float32, via torch."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a32))
    return t.to(torch.float16).to(torch.float32).numpy()


def _to_storage(a32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return _to_bf16_values(a32)
    if dtype == "f16":
        return _to_f16_values(a32)
    return a32


def _draw(seed: int, index: int, shape, std: float, dtype: str) -> np.ndarray:
    rng = np.random.default_rng([seed, index])
    a = (rng.standard_normal(shape) * std).astype(np.float32)
    return _to_storage(a, dtype)


def make_weights(w: Workload, *, seed: Optional[int] = None,
                 gamma_std: float = 0.0, bias: Optional[bool] = None,
                 n_layer: Optional[int] = None) -> dict:
    """Weights of workload ``w`` as float32 numpy arrays.

    Layout is nanoGPT's ``nn.Linear`` layout, [out_features, in_features]
    row-major; ``attn_w`` is [3C, C] with the q rows first, then k, then v.
    For bf16 workloads every value is exactly representable in bfloat16.
    For f16 workloads every value is exactly representable in IEEE float16.
    ``gamma_std > 0`` draws LayerNorm weights 1 + N(0, gamma_std) instead of
    ones (a test-only variant that exercises the scale path).  Biases are
    ``None`` when the workload has no biases.
    """
    seed = 1000 + w.index if seed is None else seed
    has_bias = w.bias if bias is None else bias
    L = w.n_layer if n_layer is None else n_layer
    C, V, Tb, dt = w.n_embd, w.vocab_size, w.block_size, w.dtype
    proj_std = 0.02 / math.sqrt(2 * w.n_layer) if w.scaled_proj_init else 0.02
    names = param_names(L)
    idx = {n: i for i, n in enumerate(names)}

    def ln_w(name):
        if gamma_std > 0:
            g = 1.0 + _draw(seed, idx[name], (C,), gamma_std, "f32")
            return _to_storage(g, dt)
        return np.ones((C,), np.float32)

    def maybe_bias(name, n):
        return _draw(seed, idx[name], (n,), 0.02, dt) if has_bias else None

    out = {
        "wte": _draw(seed, idx["wte"], (V, C), 0.02, dt),
        "wpe": _draw(seed, idx["wpe"], (Tb, C), 0.02, dt),
        "layers": [],
        "lnf_w": ln_w("lnf_w"),
        "lnf_b": maybe_bias("lnf_b", C),
    }
    for l in range(L):
        p = f"h{l}."
        out["layers"].append({
            "ln1_w": ln_w(p + "ln1_w"),
            "ln1_b": maybe_bias(p + "ln1_b", C),
            "attn_w": _draw(seed, idx[p + "attn_w"], (3 * C, C), 0.02, dt),
            "attn_b": maybe_bias(p + "attn_b", 3 * C),
            "attnproj_w": _draw(seed, idx[p + "attnproj_w"], (C, C),
                                proj_std, dt),
            "attnproj_b": maybe_bias(p + "attnproj_b", C),
            "ln2_w": ln_w(p + "ln2_w"),
            "ln2_b": maybe_bias(p + "ln2_b", C),
            "fc_w": _draw(seed, idx[p + "fc_w"], (4 * C, C), 0.02, dt),
            "fc_b": maybe_bias(p + "fc_b", 4 * C),
            "mlpproj_w": _draw(seed, idx[p + "mlpproj_w"], (C, 4 * C),
                               proj_std, dt),
            "mlpproj_b": maybe_bias(p + "mlpproj_b", C),
        })
    return out


def make_prompts(w: Workload, *, seed: Optional[int] = None,
                 batch: Optional[int] = None):
    """Right-padded prompt ids ``[B, Tmax]`` (int32) and lengths ``[B]``.

    Fixed-length workloads draw ``prompt_len`` ids per row; ragged ones first
    draw each row's length uniformly in [lo, hi], then the ids.  Entries past
    a row's length are 0 and must never be read.
    """
    seed = 2000 + w.index if seed is None else seed
    B = w.batch if batch is None else batch
    rng = np.random.default_rng(seed)
    if w.ragged:
        lens = rng.integers(w.prompt_len_lo, w.prompt_len_hi + 1, size=B)
    else:
        lens = np.full(B, w.prompt_len)
    tmax = int(lens.max())
    ids = rng.integers(0, w.vocab_real, size=(B, tmax))
    for b in range(B):
        ids[b, lens[b]:] = 0
    return ids.astype(np.int32), lens.astype(np.int32)


def decode_steps(w: Workload, lens: np.ndarray) -> int:
    """Number of decode steps the workload runs after prefill."""
    if w.decode_to:
        return int(w.decode_to - lens.min())
    return w.steps


def make_uniforms(w: Workload, steps: int, batch: Optional[int] = None, *,
                  seed: Optional[int] = None) -> np.ndarray:
    """Per-step uniform draws ``[steps, B]`` in [0, 1) as float64."""
    seed = 3000 + w.index if seed is None else seed
    B = w.batch if batch is None else batch
    return np.random.default_rng(seed).random((steps, B))


def make_feed_tokens(w: Workload, steps: int, batch: Optional[int] = None, *,
                     seed: Optional[int] = None) -> np.ndarray:
    """Teacher-forcing token stream ``[steps, B]`` (int32), uniform ids."""
    seed = 4000 + w.index if seed is None else seed
    B = w.batch if batch is None else batch
    rng = np.random.default_rng(seed)
    return rng.integers(0, w.vocab_real, size=(steps, B)).astype(np.int32)


def make_logits(B: int, V: int, *, seed: int, scale: float = 3.0,
                ties: int = 0) -> np.ndarray:
    """Synthetic float32 logits ``[B, V]`` for sampler tests.

    ``ties > 0`` copies a few values so that equal logits occur, including
    at the top of each row.
    """
    rng = np.random.default_rng(seed)
    lg = (rng.standard_normal((B, V)) * scale).astype(np.float32)
    if ties:
        for b in range(B):
            src = rng.integers(0, V, size=ties)
            dst = rng.integers(0, V, size=ties)
            lg[b, dst] = lg[b, src]
            top = int(np.argmax(lg[b]))
            lg[b, rng.integers(0, V, size=2)] = lg[b, top]
    return lg
