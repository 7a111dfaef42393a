"""Host-only checks of the C ABI: the library loads, exports every function
that include/ngpt.h declares, and its pure host functions (sizes, config
validation, argument checks that precede any device work) behave as the
header documents.  No kernel runs here."""
import ctypes
import os
import re

import pytest

import gpt_decoder_amd as ng
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    with open(os.path.join(ROOT, "include", "ngpt.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ngpt_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = ng.lib()
    names = header_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n


def cfg_of(w, **kw):
    d = dict(n_layer=w.n_layer, n_head=w.n_head, n_embd=w.n_embd,
             block_size=w.block_size, vocab_size=w.vocab_size, bias=w.bias,
             dtype=w.dtype, max_batch=w.batch, max_prefill_tokens=w.batch * w.block_size)
    d.update(kw)
    return ng.make_config(**d)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_kv_bytes_matches_layout(name):
    w = synth.workload(name)
    cfg = cfg_of(w)
    es = 4 if w.dtype == "f32" else 2
    want = w.n_layer * w.batch * w.n_head * w.block_size * w.head_dim * es
    assert ng.kv_bytes(cfg, w.batch) == want
    assert ng.check_config(cfg) == ng.NGPT_OK


def test_kv_pool_bytes_is_pages_of_64_positions():
    # a paged pool of P pages holds P * 64 positions of every layer and head
    w = synth.workload("gpt2_124m_bias_b64_ragged")
    cfg = cfg_of(w)
    assert ng.NGPT_PAGE_TOKENS == 64
    assert ng.kv_pool_bytes(cfg, 1) == 12 * 64 * 768 * 2
    assert ng.kv_pool_bytes(cfg, 16) == ng.kv_bytes(cfg, 1)   # 16 pages = 1024 positions
    assert ng.kv_pool_bytes(cfg, 0) == 0
    bad = cfg_of(w, n_head=5)
    assert ng.kv_pool_bytes(bad, 4) == 0


def test_kv_bytes_known_values():
    # GPT-2 124M, bf16, one sequence: 12 layers x 1024 positions x 768 x 2 B
    w = synth.workload("gpt2_124m_b1")
    assert ng.kv_bytes(cfg_of(w), 1) == 12 * 1024 * 768 * 2 == 18874368
    assert ng.kv_bytes(cfg_of(w), 0) == 0


@pytest.mark.parametrize("change,code", [
    (dict(n_head=5), ng.NGPT_E_CONFIG),            # 768 % 5 != 0
    (dict(n_head=6), ng.NGPT_E_CONFIG),            # head_dim 128 unsupported
    (dict(n_head=24), ng.NGPT_E_CONFIG),           # head_dim 32 ok but 768/24=32 -> fine? see below
    (dict(dtype=7), ng.NGPT_E_CONFIG),
    (dict(block_size=0), ng.NGPT_E_CONFIG),
    (dict(block_size=8192), ng.NGPT_E_CONFIG),
    (dict(vocab_size=0), ng.NGPT_E_CONFIG),
    (dict(max_batch=0), ng.NGPT_E_CONFIG),
    (dict(max_batch=257), ng.NGPT_E_CONFIG),
    (dict(max_prefill_tokens=0), ng.NGPT_E_CONFIG),
    (dict(n_layer=-1), ng.NGPT_E_CONFIG),
    (dict(bias=2), ng.NGPT_E_CONFIG),
    (dict(n_embd=96, n_head=3), ng.NGPT_E_CONFIG),  # bf16 needs n_embd % 64
    # 32-bit buffer offsets: each matrix and activation buffer below 2 GiB
    (dict(vocab_size=1 << 20, n_embd=1024, n_head=16), ng.NGPT_E_CONFIG),
    (dict(max_prefill_tokens=1 << 20), ng.NGPT_E_CONFIG),
])
def test_config_validation(change, code):
    w = synth.workload("gpt2_124m_b1")
    cfg = cfg_of(w, **change)
    if change == dict(n_head=24):   # 768 / 24 = 32 is a supported head size
        assert ng.check_config(cfg) == ng.NGPT_OK
        return
    assert ng.check_config(cfg) == code
    assert ng.kv_bytes(cfg, 1) == 0


def test_workspace_bytes_covers_the_activation_buffers():
    """The workspace holds at least the fp32 residual, the bf16 LayerNorm /
    q / attention-output rows, the MLP activation and the fp32 logits of the
    config's row bounds; it grows with max_prefill_tokens and max_batch, and
    an invalid config gives 0."""
    w = synth.workload("gpt2_124m_b1")
    cfg = cfg_of(w, max_batch=1, max_prefill_tokens=1024)
    n = ng.workspace_bytes(cfg)
    C, V, M = 768, 50304, 1024
    floor = M * C * 4 + 3 * M * C * 2 + M * 4 * C * 2 + V * 4
    assert floor <= n < floor + (40 << 20)
    assert ng.workspace_bytes(cfg_of(w, max_batch=1, max_prefill_tokens=2048)) > n
    assert ng.workspace_bytes(cfg_of(w, max_batch=8, max_prefill_tokens=1024)) > n
    assert ng.workspace_bytes(cfg_of(w, n_head=5)) == 0
    assert n % 256 == 0


def test_zero_layer_config_is_valid():
    w = synth.workload("char_4l128_fp32")
    assert ng.check_config(cfg_of(w, n_layer=0)) == ng.NGPT_OK


def test_create_rejects_bad_arguments_before_any_device_work():
    lib = ng.lib()
    w = synth.workload("char_4l128_fp32")
    cfg = cfg_of(w)
    out = ctypes.c_void_p(1)
    # NULL weights
    rc = lib.ngpt_create(ctypes.byref(cfg), None, 4096, 1 << 30, None, ctypes.byref(out))
    assert rc == ng.NGPT_E_ARG and out.value is None
    # a bias pointer on a bias-free model
    layers = (ng.binding.LayerWeights * w.n_layer)()
    for l in range(w.n_layer):
        for f in ng.binding._LAYER_FIELDS:
            setattr(layers[l], f, 0 if f.endswith("_b") else 4096)
    wt = ng.binding.Weights(4096, 4096, 4096, 4096, layers)
    rc = lib.ngpt_create(ctypes.byref(cfg), ctypes.byref(wt), 4096, 1 << 30, None, ctypes.byref(out))
    assert rc == ng.NGPT_E_ARG
    assert b"lnf_b" in lib.ngpt_last_error(None)
    # misaligned weight pointer
    wt = ng.binding.Weights(4096 + 2, 4096, 4096, 0, layers)
    rc = lib.ngpt_create(ctypes.byref(cfg), ctypes.byref(wt), 4096, 1 << 30, None, ctypes.byref(out))
    assert rc == ng.NGPT_E_ARG
    # misaligned lnf_w (the LayerNorm kernels read parameters 4 at a time)
    wt = ng.binding.Weights(4096, 4096, 4096 + 4, 0, layers)
    rc = lib.ngpt_create(ctypes.byref(cfg), ctypes.byref(wt), 4096, 1 << 30, None, ctypes.byref(out))
    assert rc == ng.NGPT_E_ARG and b"aligned" in lib.ngpt_last_error(None)
    # misaligned bias pointer on a model with biases
    bcfg = cfg_of(w, bias=1)
    blayers = (ng.binding.LayerWeights * w.n_layer)()
    for l in range(w.n_layer):
        for f in ng.binding._LAYER_FIELDS:
            setattr(blayers[l], f, 4096)
    blayers[2].fc_b = 4096 + 8
    wt = ng.binding.Weights(4096, 4096, 4096, 4096, blayers)
    rc = lib.ngpt_create(ctypes.byref(bcfg), ctypes.byref(wt), 4096, 1 << 30, None, ctypes.byref(out))
    assert rc == ng.NGPT_E_ARG and b"aligned" in lib.ngpt_last_error(None)
    # missing layer weight
    layers[1].fc_w = 0
    wt = ng.binding.Weights(4096, 4096, 4096, 0, layers)
    rc = lib.ngpt_create(ctypes.byref(cfg), ctypes.byref(wt), 4096, 1 << 30, None, ctypes.byref(out))
    assert rc == ng.NGPT_E_ARG
    # invalid config
    bad = cfg_of(w, n_head=3)
    rc = lib.ngpt_create(ctypes.byref(bad), ctypes.byref(wt), 4096, 1 << 30, None, ctypes.byref(out))
    assert rc == ng.NGPT_E_CONFIG
    # the caller-owned workspace: NULL, misaligned, too small
    layers[1].fc_w = 4096
    wt = ng.binding.Weights(4096, 4096, 4096, 0, layers)
    need = ng.workspace_bytes(cfg)
    for ws, nbytes, code in ((0, need, ng.NGPT_E_ARG), (4096 + 16, need, ng.NGPT_E_ARG),
                             (4096, need - 1, ng.NGPT_E_SIZE)):
        rc = lib.ngpt_create(ctypes.byref(cfg), ctypes.byref(wt), ws, nbytes, None,
                             ctypes.byref(out))
        assert rc == code and out.value is None, (ws, nbytes)
        assert b"workspace" in lib.ngpt_last_error(None)


def test_null_handle_calls_fail_cleanly():
    lib = ng.lib()
    assert lib.ngpt_destroy(None) == ng.NGPT_E_ARG
    assert lib.ngpt_set_sampling(None, 1.0, 0, 1) == ng.NGPT_E_ARG
    assert lib.ngpt_prefill(None, None, None, None, None, 1, 1) == ng.NGPT_E_ARG
    assert lib.ngpt_prefill_device(None, None, None, None, None, 1, 1) == ng.NGPT_E_ARG
    assert lib.ngpt_device_status(None, None) == ng.NGPT_E_ARG
    assert lib.ngpt_decode_step(None, None, None, None) == ng.NGPT_E_ARG
    assert lib.ngpt_decode_feed(None, None, None) == ng.NGPT_E_ARG
    assert lib.ngpt_sample(None, None, 1, 1, None, None) == ng.NGPT_E_ARG
    assert lib.ngpt_status_string(-5) == b"NGPT_E_CONTEXT"
    assert lib.ngpt_status_string(ng.NGPT_E_TIMEOUT) == b"NGPT_E_TIMEOUT"
    assert lib.ngpt_set_wait_limit(None, 1) == ng.NGPT_E_ARG
