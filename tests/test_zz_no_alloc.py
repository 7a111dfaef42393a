"""ngpt_create_static: a model whose workspace is the library's fixed
per-device array, for callers that cannot allocate device memory.  Its
results must equal those of a model over a caller-owned workspace, bit for
bit (the kernels are the same), on two creations in a row, the second with a
smaller model and a shorter input; the array is shared, so a second live
static model on the device is refused, and a config too large for the array
is refused."""
import ctypes

import numpy as np
import pytest

import synth
from gpu_common import log, need_gpu

pytestmark = pytest.mark.gpu


def _run(m, w, ids, lens, steps):
    import torch
    m.set_sampling(greedy=True)
    kv = m.new_kv(w.batch)
    m.prefill(kv, ids, list(lens))
    lg = [m.logits(w.batch).cpu().numpy()]
    toks = []
    nxt = torch.empty(w.batch, dtype=torch.int32, device="cuda")
    for _ in range(steps):
        m.decode_step(kv, nxt, None)
        toks.append(nxt.cpu().numpy().copy())
        lg.append(m.logits(w.batch).cpu().numpy())
    # the cache entries written (positions past a row's length were never
    # written: the buffer comes from torch.empty)
    hs = w.n_embd // w.n_head
    shp = (w.n_layer, w.batch, w.n_head, w.block_size, hs)
    k = kv.k.cpu().numpy().view(np.uint16)[:int(np.prod(shp))].reshape(shp)
    n = kv.lens.cpu().numpy()
    k = np.concatenate([k[:, b, :, :n[b]].ravel() for b in range(w.batch)])
    st = m.device_status()
    return np.array(toks), np.array(lg), k, st


def test_static_workspace_model_matches_caller_workspace_model():
    need_gpu()
    import gpt_decoder_amd as ng
    cases = [
        # (workload, prompt length, decode steps): the second is smaller
        (synth.Workload("static_a", 31, 3, 4, 256, 128, 400, 400, True, "bf16",
                        batch=2, prompt_len=40), 40, 12),
        (synth.Workload("static_b", 32, 2, 4, 256, 64, 300, 300, False, "bf16",
                        batch=1, prompt_len=9), 9, 6),
    ]
    for w, plen, steps in cases:
        W = synth.make_weights(w)
        ids, lens = synth.make_prompts(w)
        log(f"{w.name}: static workspace vs caller workspace, {steps} steps")
        ref = ng.model_from_workload(w, W)
        a = _run(ref, w, ids, lens, steps)
        ref.close()
        ms = ng.model_from_workload(w, W, static_workspace=True)
        # one static model per device at a time
        with pytest.raises(ng.NgptError) as ei:
            ng.model_from_workload(w, W, static_workspace=True)
        assert ei.value.code == ng.NGPT_E_ARG
        b = _run(ms, w, ids, lens, steps)
        ms.close()
        np.testing.assert_array_equal(a[0], b[0])    # ids
        np.testing.assert_array_equal(a[1], b[1])    # logits, every step
        np.testing.assert_array_equal(a[2], b[2])    # KV cache entries written
        assert a[3] == b[3] == ng.NGPT_OK
    # a config whose workspace exceeds the array
    big = synth.workload("gpt2_xl_b32")
    cfg = ng.make_config(big.n_layer, big.n_head, big.n_embd, big.block_size,
                         big.vocab_size, big.bias, big.dtype, 32, 32 * 512)
    assert ng.workspace_bytes(cfg) > 64 << 20
    lib = ng.lib()
    fn = lib.ngpt_create_static
    fn.argtypes = [ctypes.POINTER(ng.Config), ctypes.POINTER(ng.binding.Weights), ctypes.c_void_p,
                   ctypes.POINTER(ctypes.c_void_p)]
    layers = (ng.binding.LayerWeights * big.n_layer)()
    for l in range(big.n_layer):
        for f in ng.binding._LAYER_FIELDS:
            setattr(layers[l], f, 0 if f.endswith("_b") else 4096)
    wt = ng.binding.Weights(4096, 4096, 4096, 0, layers)
    out = ctypes.c_void_p()
    assert fn(ctypes.byref(cfg), ctypes.byref(wt), None, ctypes.byref(out)) == ng.NGPT_E_SIZE
    assert out.value is None
