"""ctypes binding of libngpt (the C ABI in include/ngpt.h).

Argument marshalling only: every step of the forward pass and the sampler
runs in the library's HIP kernels.  PyTorch provides device memory (weights,
KV cache, ids, uniforms, outputs) and the stream.  There is no CPU fallback:
importing this module without the built library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libngpt.so")

NGPT_OK = 0
NGPT_E_ARG = -1
NGPT_E_CONFIG = -2
NGPT_E_RANGE = -3
NGPT_E_SIZE = -4
NGPT_E_CONTEXT = -5
NGPT_E_HIP = -6
NGPT_E_DEVICE = -7
NGPT_E_TIMEOUT = -8
NGPT_E_PAGE = -9
NGPT_PAGE_TOKENS = 64
NGPT_F32 = 0
NGPT_BF16 = 1
NGPT_F16 = 2
NGPT_MAX_BATCH = 256


class NgptError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_status_name(code)} ({code}): {msg}")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layer", "n_head", "n_embd", "block_size", "vocab_size", "bias",
        "dtype", "max_batch", "max_prefill_tokens")]


_LAYER_FIELDS = ("ln1_w", "ln1_b", "attn_w", "attn_b", "attnproj_w",
                 "attnproj_b", "ln2_w", "ln2_b", "fc_w", "fc_b", "mlpproj_w",
                 "mlpproj_b")


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _LAYER_FIELDS]


class Weights(ctypes.Structure):
    _fields_ = [("wte", ctypes.c_void_p), ("wpe", ctypes.c_void_p),
                ("lnf_w", ctypes.c_void_p), ("lnf_b", ctypes.c_void_p),
                ("layers", ctypes.POINTER(LayerWeights))]


class KV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("lens", ctypes.c_void_p), ("limit", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("block_table", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libngpt.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m "
            "gpt_decoder_amd.build` (there is no fallback path)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.ngpt_kv_bytes.argtypes = [ctypes.POINTER(Config), i32]
    L.ngpt_kv_bytes.restype = sz
    L.ngpt_kv_pool_bytes.argtypes = [ctypes.POINTER(Config), i32]
    L.ngpt_kv_pool_bytes.restype = sz
    L.ngpt_kv_map.argtypes = [vp, ctypes.POINTER(KV), i32, i32, i32, vp]
    L.ngpt_workspace_bytes.argtypes = [ctypes.POINTER(Config)]
    L.ngpt_workspace_bytes.restype = sz
    L.ngpt_check_config.argtypes = [ctypes.POINTER(Config)]
    L.ngpt_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights),
                              vp, sz, vp, ctypes.POINTER(vp)]
    L.ngpt_destroy.argtypes = [vp]
    L.ngpt_set_sampling.argtypes = [vp, ctypes.c_float, i32, i32]
    L.ngpt_prefill.argtypes = [vp, ctypes.POINTER(KV), vp,
                               ctypes.POINTER(i32), ctypes.POINTER(i32), i32,
                               i32]
    L.ngpt_prefill_device.argtypes = [vp, ctypes.POINTER(KV), vp,
                                      ctypes.POINTER(i32), ctypes.POINTER(i32),
                                      i32, i32]
    L.ngpt_prefill_slots.argtypes = [vp, ctypes.POINTER(KV), vp, vp,
                                     ctypes.POINTER(i32), ctypes.POINTER(i32),
                                     i32, i32]
    L.ngpt_extend.argtypes = [vp, ctypes.POINTER(KV), vp, vp, vp, i32, i32]
    L.ngpt_eval_loss.argtypes = [vp, ctypes.POINTER(KV), vp, ctypes.POINTER(i32),
                                 i32, i32, vp, vp, vp]
    L.ngpt_retire.argtypes = [vp, ctypes.POINTER(KV), vp, i32]
    L.ngpt_slide.argtypes = [vp, ctypes.POINTER(KV), vp, i32, vp]
    L.ngpt_decode_step.argtypes = [vp, ctypes.POINTER(KV), vp, vp]
    L.ngpt_decode_feed.argtypes = [vp, ctypes.POINTER(KV), vp]
    L.ngpt_sample.argtypes = [vp, vp, i32, i32, vp, vp]
    L.ngpt_logits.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(i32)]
    L.ngpt_copy_logits.argtypes = [vp, vp, i32, i32]
    L.ngpt_device_status.argtypes = [vp, vp]
    L.ngpt_set_wait_limit.argtypes = [vp, i32]
    L.ngpt_last_error.argtypes = [vp]
    L.ngpt_last_error.restype = ctypes.c_char_p
    L.ngpt_status_string.argtypes = [ctypes.c_int]
    L.ngpt_status_string.restype = ctypes.c_char_p
    for name in ("ngpt_check_config", "ngpt_create", "ngpt_destroy",
                 "ngpt_set_sampling", "ngpt_prefill", "ngpt_prefill_device",
                 "ngpt_prefill_slots", "ngpt_extend", "ngpt_retire", "ngpt_slide",
                 "ngpt_eval_loss",
                 "ngpt_decode_step",
                 "ngpt_decode_feed", "ngpt_sample", "ngpt_logits",
                 "ngpt_copy_logits", "ngpt_device_status", "ngpt_set_wait_limit"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _status_name(code: int) -> str:
    try:
        return lib().ngpt_status_string(code).decode()
    except Exception:
        return str(code)


def make_config(n_layer, n_head, n_embd, block_size, vocab_size, bias, dtype,
                max_batch, max_prefill_tokens) -> Config:
    d = {"f32": NGPT_F32, "bf16": NGPT_BF16, "f16": NGPT_F16}.get(dtype, dtype)
    return Config(n_layer, n_head, n_embd, block_size, vocab_size, int(bias),
                  d, max_batch, max_prefill_tokens)


def kv_bytes(cfg: Config, batch: int) -> int:
    return int(lib().ngpt_kv_bytes(ctypes.byref(cfg), batch))


def kv_pool_bytes(cfg: Config, num_pages: int) -> int:
    return int(lib().ngpt_kv_pool_bytes(ctypes.byref(cfg), num_pages))


def workspace_bytes(cfg: Config) -> int:
    return int(lib().ngpt_workspace_bytes(ctypes.byref(cfg)))


def check_config(cfg: Config) -> int:
    return int(lib().ngpt_check_config(ctypes.byref(cfg)))


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


class KVCache:
    """Caller-owned KV cache plus lens/limit.

    Contiguous (``num_pages`` None): K and V [L][B][H][Tb][hs].  Paged: K and
    V pools [L][num_pages][H][64][hs] and a block table [B][ceil(Tb/64)] of
    page ids, every block unmapped (-1) until mapped with Model.kv_map."""

    def __init__(self, cfg: Config, batch: int, device="cuda", num_pages=None):
        import torch
        paged = num_pages is not None
        nbytes = kv_pool_bytes(cfg, num_pages) if paged else kv_bytes(cfg, batch)
        if nbytes == 0 and cfg.n_layer > 0:
            raise NgptError(NGPT_E_CONFIG, "invalid config for the KV cache")
        n = max(nbytes, 16)
        self.k = torch.empty(n, dtype=torch.uint8, device=device)
        self.v = torch.empty(n, dtype=torch.uint8, device=device)
        self.lens = torch.zeros(batch, dtype=torch.int32, device=device)
        self.limit = torch.zeros(batch, dtype=torch.int32, device=device)
        self.batch = batch
        self.num_pages = num_pages
        self.nblk = (cfg.block_size + NGPT_PAGE_TOKENS - 1) // NGPT_PAGE_TOKENS
        self.table = (torch.full((batch, self.nblk), -1, dtype=torch.int32, device=device)
                      if paged else None)
        self.struct = KV(_ptr(self.k), _ptr(self.v), _ptr(self.lens),
                         _ptr(self.limit), batch, int(num_pages or 0), _ptr(self.table))


class Model:
    """A libngpt model handle bound to one stream.

    ``weights`` is a dict in nn.Linear layout (see ``synth.make_weights``):
    numpy or torch arrays; they are uploaded once to the device in the model
    dtype and kept alive here for the handle's lifetime.
    """

    def __init__(self, *, n_layer, n_head, n_embd, block_size, vocab_size,
                 bias, dtype, weights, max_batch, max_prefill_tokens,
                 device="cuda", stream=None, static_workspace=False):
        import torch
        self.torch = torch
        self.device = torch.device(device)
        self.cfg = make_config(n_layer, n_head, n_embd, block_size, vocab_size,
                               bias, dtype, max_batch, max_prefill_tokens)
        self.vocab = vocab_size
        tdt = {NGPT_BF16: torch.bfloat16, NGPT_F16: torch.float16}.get(self.cfg.dtype,
                                                                       torch.float32)
        keep = []

        def up(a):
            if a is None:
                return None
            t = torch.as_tensor(np.asarray(a) if not torch.is_tensor(a) else a)
            t = t.to(device=self.device, dtype=tdt).contiguous()
            keep.append(t)
            return t

        layers = (LayerWeights * max(1, n_layer))()
        for l, lw in enumerate(weights["layers"]):
            for f in _LAYER_FIELDS:
                setattr(layers[l], f, _ptr(up(lw[f])))
        self._weights = Weights(_ptr(up(weights["wte"])),
                                _ptr(up(weights["wpe"])),
                                _ptr(up(weights["lnf_w"])),
                                _ptr(up(weights["lnf_b"])), layers)
        self._layers = layers
        self._keep = keep
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        self.stream = stream
        self._status = torch.zeros(1, dtype=torch.int32, device=self.device)
        h = ctypes.c_void_p()
        if static_workspace:
            # the library's fixed per-device workspace: no allocation at all
            self.workspace = None
            fn = lib().ngpt_create_static
            fn.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights),
                           ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
            fn.restype = ctypes.c_int
            rc = fn(ctypes.byref(self.cfg), ctypes.byref(self._weights),
                    ctypes.c_void_p(stream.cuda_stream), ctypes.byref(h))
        else:
            # caller-owned workspace (torch's allocations are 256-byte aligned)
            nws = workspace_bytes(self.cfg)
            if nws == 0:
                raise NgptError(NGPT_E_CONFIG, "invalid config")
            self.workspace = torch.empty(nws, dtype=torch.uint8, device=self.device)
            rc = lib().ngpt_create(ctypes.byref(self.cfg),
                                   ctypes.byref(self._weights),
                                   _ptr(self.workspace), nws,
                                   ctypes.c_void_p(stream.cuda_stream),
                                   ctypes.byref(h))
        if rc != NGPT_OK:
            raise NgptError(rc, lib().ngpt_last_error(None).decode())
        self.h = h

    # -- helpers -----------------------------------------------------------
    def _check(self, rc):
        if rc != NGPT_OK:
            raise NgptError(rc, lib().ngpt_last_error(self.h).decode())

    def new_kv(self, batch: int, num_pages=None) -> KVCache:
        return KVCache(self.cfg, batch, self.device, num_pages)

    # -- the C calls ---------------------------------------------------------
    def set_sampling(self, temperature=1.0, top_k=0, greedy=False):
        self._check(lib().ngpt_set_sampling(self.h, float(temperature),
                                            int(top_k), int(bool(greedy))))

    def prefill(self, kv: KVCache, ids, lens: Sequence[int],
                limit: Optional[Sequence[int]] = None):
        """``ids``: int32 [B, Tmax], host (numpy; checked by the library) or
        device (torch, ngpt_prefill_device); ``lens``/``limit``: host ints."""
        B, Tmax = ids.shape
        lens_a = (ctypes.c_int32 * B)(*[int(x) for x in lens])
        lim_a = None if limit is None else (ctypes.c_int32 * B)(
            *[int(x) for x in limit])
        if self.torch.is_tensor(ids) and ids.is_cuda:
            assert ids.dtype == self.torch.int32 and ids.is_contiguous()
            self._check(lib().ngpt_prefill_device(
                self.h, ctypes.byref(kv.struct), _ptr(ids), lens_a, lim_a, B,
                Tmax))
            return
        a = np.ascontiguousarray(np.asarray(ids), dtype=np.int32)
        self._check(lib().ngpt_prefill(
            self.h, ctypes.byref(kv.struct),
            a.ctypes.data_as(ctypes.c_void_p), lens_a, lim_a, B, Tmax))

    @staticmethod
    def _host_i32(a):
        return np.ascontiguousarray(np.asarray(a), dtype=np.int32)

    def prefill_slots(self, kv: KVCache, slots, ids, lens, limit=None):
        """Admit prompts (host ids [n, Tmax]) into kv rows ``slots``."""
        sl = self._host_i32(slots)
        a = self._host_i32(ids)
        n, Tmax = a.shape
        lens_a = (ctypes.c_int32 * n)(*[int(x) for x in lens])
        lim_a = None if limit is None else (ctypes.c_int32 * n)(
            *[int(x) for x in limit])
        self._check(lib().ngpt_prefill_slots(
            self.h, ctypes.byref(kv.struct), sl.ctypes.data_as(ctypes.c_void_p),
            a.ctypes.data_as(ctypes.c_void_p), lens_a, lim_a, n, Tmax))

    def extend(self, kv: KVCache, slots, ids, counts):
        """Append counts[b] tokens (host ids [n, Tmax]) to live rows."""
        sl, a, c = self._host_i32(slots), self._host_i32(ids), self._host_i32(counts)
        n, Tmax = a.shape
        self._check(lib().ngpt_extend(
            self.h, ctypes.byref(kv.struct), sl.ctypes.data_as(ctypes.c_void_p),
            a.ctypes.data_as(ctypes.c_void_p), c.ctypes.data_as(ctypes.c_void_p),
            n, Tmax))

    def eval_loss(self, kv: KVCache, ids, lens, logits=None):
        """Forward with labels over every position (host ids [B, Tmax]).
        Returns (logits [sum(lens), V], losses [sum(lens)], mean [1]), all
        device fp32; ``logits`` may be given to reuse a buffer."""
        a = self._host_i32(ids)
        B, Tmax = a.shape
        M = int(sum(int(x) for x in lens))
        t = self.torch
        if logits is None:
            logits = t.empty((M, self.vocab), dtype=t.float32, device=self.device)
        losses = t.empty(M, dtype=t.float32, device=self.device)
        mean = t.empty(1, dtype=t.float32, device=self.device)
        lens_a = (ctypes.c_int32 * B)(*[int(x) for x in lens])
        self._check(lib().ngpt_eval_loss(
            self.h, ctypes.byref(kv.struct), a.ctypes.data_as(ctypes.c_void_p),
            lens_a, B, Tmax, _ptr(logits), _ptr(losses), _ptr(mean)))
        return logits, losses, mean

    def kv_map(self, kv: KVCache, slot: int, first_block: int, pages):
        """Map blocks first_block.. of row ``slot`` of a paged cache to the
        host page ids ``pages`` (-1 unmaps)."""
        pg = self._host_i32(pages)
        self._check(lib().ngpt_kv_map(self.h, ctypes.byref(kv.struct), int(slot),
                                      int(first_block), len(pg),
                                      pg.ctypes.data_as(ctypes.c_void_p)))

    def retire(self, kv: KVCache, slots):
        sl = self._host_i32(slots)
        self._check(lib().ngpt_retire(self.h, ctypes.byref(kv.struct),
                                      sl.ctypes.data_as(ctypes.c_void_p), len(sl)))

    def slide(self, kv: KVCache, slots, next_ids):
        """Crop full rows to their last block_size - 1 tokens plus
        next_ids[row] (device int32 [batch]) and run that window."""
        sl = self._host_i32(slots)
        assert next_ids.dtype == self.torch.int32 and next_ids.is_cuda
        self._check(lib().ngpt_slide(self.h, ctypes.byref(kv.struct),
                                     sl.ctypes.data_as(ctypes.c_void_p), len(sl),
                                     _ptr(next_ids)))

    def decode_step(self, kv: KVCache, next_ids, uniforms):
        """``next_ids``: device int32 [batch] (out); ``uniforms``: device
        float64 [batch]."""
        assert next_ids.dtype == self.torch.int32
        assert uniforms is None or uniforms.dtype == self.torch.float64
        self._check(lib().ngpt_decode_step(self.h, ctypes.byref(kv.struct),
                                           _ptr(next_ids), _ptr(uniforms)))

    def decode_feed(self, kv: KVCache, ids):
        assert ids.dtype == self.torch.int32
        self._check(lib().ngpt_decode_feed(self.h, ctypes.byref(kv.struct),
                                           _ptr(ids)))

    def sample(self, logits, uniforms=None, out=None):
        """Sampler alone on device fp32 logits [B, ld]; returns int32 [B]."""
        B, ld = logits.shape
        assert logits.dtype == self.torch.float32 and logits.is_contiguous()
        if out is None:
            out = self.torch.empty(B, dtype=self.torch.int32,
                                   device=self.device)
        self._check(lib().ngpt_sample(self.h, _ptr(logits), ld, B,
                                      _ptr(uniforms), _ptr(out)))
        return out

    def logits(self, B: int, out=None):
        """Copy of the first B logits rows (device fp32 [B, vocab])."""
        if out is None:
            out = self.torch.empty((B, self.vocab), dtype=self.torch.float32,
                                   device=self.device)
        self._check(lib().ngpt_copy_logits(self.h, _ptr(out), out.shape[1], B))
        return out

    def logits_ptr(self):
        p, ld = ctypes.c_void_p(), ctypes.c_int32()
        self._check(lib().ngpt_logits(self.h, ctypes.byref(p), ctypes.byref(ld)))
        return p.value, ld.value

    def set_wait_limit(self, passes: int = 0):
        """Poll passes before a one-launch decode wait gives up (0: default)."""
        self._check(lib().ngpt_set_wait_limit(self.h, int(passes)))

    def device_status(self) -> int:
        """Kernel-side status since the last call (the library enqueues the
        read; this waits for it)."""
        self._check(lib().ngpt_device_status(self.h, _ptr(self._status)))
        return int(self._status.item())

    def close(self):
        if getattr(self, "h", None):
            rc = lib().ngpt_destroy(self.h)
            self.h = None
            if rc != NGPT_OK:
                raise NgptError(rc, lib().ngpt_last_error(None).decode())

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def model_from_workload(w, weights, *, max_batch=None, max_prefill_tokens=None,
                        device="cuda", stream=None, static_workspace=False) -> Model:
    """Model for a ``synth.Workload``-like shape description."""
    mb = max_batch or w.batch
    mpt = max_prefill_tokens or mb * w.block_size
    return Model(n_layer=len(weights["layers"]), n_head=w.n_head,
                 n_embd=w.n_embd, block_size=w.block_size,
                 vocab_size=w.vocab_size, bias=weights["lnf_b"] is not None,
                 dtype=w.dtype, weights=weights, max_batch=mb,
                 max_prefill_tokens=mpt, device=device, stream=stream,
                 static_workspace=static_workspace)
