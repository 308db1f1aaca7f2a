"""ctypes view of libdspark.so (include/dspark.h).  Loading does not touch the
GPU; a missing library raises ImportError so that nothing can silently fall
back to another implementation."""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdspark.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_WORKSPACE = -2
ERR_UNSUPPORTED = -3
ERR_HIP = -4
F32 = 0
BF16 = 1
HEAD_GATED = 1
HEAD_RNN = 2
STATUS_BAD_ANCHOR = 1
STATUS_BAD_TOKEN = 2
STATUS_BAD_OFFSETS = 4
STATUS_BAD_LABEL = 8
STATUS_WAIT_TIMEOUT = 16
NOALLOC_SCRATCH_BYTES = 4 << 20  # DSPARK_NOALLOC_SCRATCH_BYTES

_p = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t
_u64 = ctypes.c_uint64

SIGNATURES = {
    "dspark_version": (_i, []),
    "dspark_last_error": (ctypes.c_char_p, []),
    "dspark_block_attention_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "dspark_block_attention": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                    _i, _i, _i, _i, _i, _i, _i, _i, _f, _i,
                                    _p, _sz, _p, _p]),
    "dspark_markov_sample_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "dspark_markov_sample": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _u64,
                                  _p, _sz, _p, _p]),
    "dspark_markov_sample_noalloc": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _u64, _p, _p]),
    "dspark_accept_rate_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "dspark_accept_rate": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _sz, _p, _p]),
    "dspark_set_wait_limit": (None, [ctypes.c_uint32]),
    "dspark_eval_mask": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _p, _p]),
    "dspark_markov_block_logits_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "dspark_markov_block_logits": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _f, _p, _sz, _p, _p]),
    "dspark_l1_loss_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "dspark_l1_loss": (_i, [_p, _p, _p, _f, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p, _sz, _p]),
    "dspark_markov_head_sample_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "dspark_markov_head_sample": (_i, [_i, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _u64,
                                       _p, _sz, _p, _p]),
    "dspark_markov_head_block_logits_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "dspark_markov_head_block_logits": (_i, [_i, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f,
                                             _p, _sz, _p, _p]),
    "dspark_verify_workspace_bytes": (_sz, [_i, _i]),
    "dspark_verify": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _f, _u64, _p, _sz, _p, _p]),
    "dspark_confidence_schedule": (_i, [_p, _i, _p, _f, _p, _i, _p, _p, _i, _i, _p, _p, _p, _p, _p,
                                        _i, _i, _i, _i, _p, _p]),
}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python semi_autoregressive_block_amd/build.py` "
            "(the HIP library is required; there is no fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib
