"""MI355X-native GPT-2 decoder (nanoGPT generate() forward with a KV cache).

The compute lives in ``libngpt.so`` (hand-written HIP kernels for gfx950,
C ABI in ``include/ngpt.h``); this package is its ctypes binding plus the
in-tree build script.
"""
from .binding import (workspace_bytes, Config, KVCache, Model, NgptError, check_config,
                      kv_bytes, kv_pool_bytes, lib, make_config, model_from_workload,
                      LIB_PATH, NGPT_OK, NGPT_E_ARG, NGPT_E_CONFIG,
                      NGPT_E_RANGE, NGPT_E_SIZE, NGPT_E_CONTEXT, NGPT_E_HIP,
                      NGPT_E_DEVICE, NGPT_E_TIMEOUT, NGPT_E_PAGE, NGPT_F32, NGPT_BF16,
                      NGPT_F16, NGPT_MAX_BATCH, NGPT_PAGE_TOKENS)

__all__ = [
    "Config", "KVCache", "Model", "NgptError", "check_config", "kv_bytes", "kv_pool_bytes",
    "lib", "make_config", "model_from_workload", "LIB_PATH", "NGPT_OK",
    "NGPT_E_ARG", "NGPT_E_CONFIG", "NGPT_E_RANGE", "NGPT_E_SIZE",
    "NGPT_E_CONTEXT", "NGPT_E_HIP", "NGPT_E_DEVICE", "NGPT_E_TIMEOUT", "NGPT_E_PAGE",
    "NGPT_F32", "NGPT_BF16", "NGPT_F16", "NGPT_MAX_BATCH", "NGPT_PAGE_TOKENS",
]
