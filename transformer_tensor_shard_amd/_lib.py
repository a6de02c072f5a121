"""ctypes binding of libtp.so (the C ABI declared in include/tp.h).

Argument marshalling only: tensors become device pointers, dtypes become
tp_dtype codes, streams become hipStream_t handles.  Every step of the path
runs in libtp.so; there is no other implementation to fall back to, and a
missing library is an error.

torch is imported before the library is loaded so that libtp.so binds to the
HIP runtime torch already mapped (both name it libamdhip64.so.7): the streams
and memory torch hands over are then valid inside the library.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must be loaded first: see the module docstring)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtp.so")

(TP_OK, TP_ERR_NULL, TP_ERR_SHAPE, TP_ERR_DTYPE, TP_ERR_ALIGN, TP_ERR_WORKSPACE, TP_ERR_LAUNCH,
 TP_ERR_SCRATCH) = range(8)
TP_F32, TP_BF16 = 0, 1
TP_EPI_NONE, TP_EPI_GELU, TP_EPI_GELU_BWD, TP_EPI_GELU_SAVE = 0, 1, 2, 3

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_sz = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/tp.h one to one
SIGNATURES = {
    "tp_status_string": (ctypes.c_char_p, [_int]),
    "tp_abi_version": (_int, []),
    "tp_mlp_shard_workspace": (_sz, [_i64, _i64, _int]),
    "tp_mlp_shard": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64, _i64, _int, _int, _vp]),
    "tp_mlp_shard_noalloc": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _vp]),
    "tp_attn_shard_workspace": (_sz, [_i64, _i64, _i64, _i64]),
    "tp_attn_shard": (_int, [_vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64, _i64, _i64, _i64, _int,
                             _int, _vp]),
    "tp_partial_sum": (_int, [_vp, _int, _vp, _int, _int, _i64, _i64, _vp, _vp, _int, _vp]),
    "tp_block_shard_workspace": (_sz, [_i64, _i64, _i64, _i64, _i64, _i64, _int]),
    "tp_block_shard": (_int, [_vp, _vp, _int, _vp, _vp, _vp, _vp, _vp, ctypes.c_float,
                              ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                              ctypes.POINTER(_vp), _int, _vp, _sz, _i64, _i64, _i64, _i64, _i64,
                              _i64, _vp]),
    "tp_block_shard_timed": (_int, [_vp, _vp, _int, _vp, _vp, _vp, _vp, _vp, ctypes.c_float,
                                    ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                    ctypes.POINTER(_vp), _int, _vp, _sz, _i64, _i64, _i64, _i64,
                                    _i64, _i64, _vp, _vp, _vp]),
    "tp_linear": (_int, [_vp, _i64, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _int, _int, _int,
                         _vp]),
    "tp_linear_batched": (_int, [ctypes.POINTER(_vp), _i64, ctypes.POINTER(_vp), _i64,
                                 ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i64, _int, _i64, _i64,
                                 _i64, _int, _int, _int, _vp]),
    "tp_attention_core": (_int, [_vp, _i64, _vp, _i64, _i64, _i64, _i64, _int, _vp]),
    "tp_attention_kv_split_workspace": (_sz, [_i64, _i64, _i64, _i64, _int]),
    "tp_attention_kv_split": (_int, [_vp, _i64, _vp, _i64, _i64, _i64, _i64, _i64, _int, _int,
                                      _vp, _sz, _vp]),
    "tp_layernorm": (_int, [_vp, _int, _vp, _vp, _vp, ctypes.c_float, _i64, _i64, _vp]),
    "tp_probe_mfma": (_int, [_vp, _int, _int, _vp]),
    "tp_gemm_tile_cols": (_int, [_int, _int, _int, _int, ctypes.POINTER(_i64),
                                 ctypes.POINTER(_i64), _i64]),
    "tp_matmul": (_int, [_vp, _i64, _int, _vp, _i64, _int, _vp, _vp, _i64, _vp, _i64, _i64, _i64,
                         _i64, _int, _int, _vp]),
    "tp_matmul_grouped": (_int, [ctypes.POINTER(_vp), ctypes.POINTER(_i64), _int,
                                 ctypes.POINTER(_vp), ctypes.POINTER(_i64), _int,
                                 ctypes.POINTER(_vp), ctypes.POINTER(_i64), ctypes.POINTER(_i64),
                                 ctypes.POINTER(_i64), _int, _i64, _int, _vp, _sz, _vp]),
    "tp_vocab_embedding_shard": (_int, [_vp, _i64, _vp, _i64, _i64, _i64, _vp, _int, _vp]),
    "tp_vocab_ce_shard_workspace": (_sz, [_i64, _i64]),
    "tp_vocab_ce_shard": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _sz, _vp]),
    "tp_vocab_ce_combine": (_int, [_vp, _int, _i64, _vp, _vp, _vp]),
    "tp_vocab_parallel_ce_workspace": (_sz, [_i64, _i64, _int]),
    "tp_vocab_parallel_ce": (_int, [_vp, ctypes.POINTER(_vp), _int, _vp, _i64, _i64, _i64, _vp,
                                    _vp, _vp, _sz, _vp]),
    "tp_mlp_shard_train_fwd": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int,
                                      _vp]),
    "tp_mlp_shard_backward_workspace": (_sz, [_i64, _i64]),
    "tp_attention_core_train": (_int, [_vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _int, _vp]),
    "tp_attention_core_backward": (_int, [_vp, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                          _i64, _int, _vp]),
    "tp_attn_shard_train_fwd": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                       _i64, _int, _int, _vp]),
    "tp_attn_shard_backward_workspace": (_sz, [_i64, _i64, _i64, _i64]),
    "tp_attn_shard_backward": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                      _i64, _i64, _i64, _i64, _i64, _int, _int, _vp]),
    "tp_mlp_shard_backward": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                     _i64, _i64, _i64, _int, _vp]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libtp.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it first (python -m transformer_tensor_shard_amd.build "
            "or __graft_entry__.build()); there is no non-HIP fallback")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
