"""ctypes binding of libtpmlp (the C ABI declared in include/tpmlp.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libtpmlp.so.  torch tensors supply device pointers and shapes; the stream is
torch's current HIP stream unless one is given.  There is no fallback: if the
library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtpmlp.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m sequence_transformer_gemms_amd.build` "
        "(there is no CPU fallback)")

lib = ctypes.CDLL(LIB_PATH)

# ---- enums (mirror include/tpmlp.h)
F32, BF16, FP8_E4M3, FP8_E5M2 = 0, 1, 2, 3
ACT_NONE, ACT_RELU, ACT_GELU_ERF, ACT_GELU_TANH, ACT_SILU = 0, 1, 2, 3, 4
EPI_FWD, EPI_DACT, EPI_GATED, EPI_DGATED = 0, 1, 2, 3
OK, EINVAL, EUNSUPPORTED, EHIP, ETIMEOUT, EWORKSPACE = 0, -1, -2, -3, -4, -5
(OP_SEQ_CHUNK_GEMM, OP_MLP_FWD, OP_MLP_BWD, OP_GATED_MLP_FWD, OP_GATED_MLP_BWD, OP_MX_MLP_FWD,
 OP_FP8_DELAYED_MLP_FWD, OP_MLP_BWD_FP8, OP_CAST_FP8, OP_LINEAR_BWD) = 0, 1, 2, 3, 4, 5, 6, 7, 8, 9
MAX_CHUNKS = 256

_i64, _i32, _u32, _vp, _sz = ctypes.c_int64, ctypes.c_int, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_size_t

lib.seq_chunk_gemm.restype = _i32
lib.seq_chunk_gemm.argtypes = [_i64, _i64, _i64,
                               _vp, _i64, _i32, _i32, _vp,
                               _vp, _i64, _i32, _i32, _vp,
                               _vp, _i64, _i32,
                               _i32, _i32, _vp, _i64, _vp,
                               _i32, _vp, _vp, _u32,
                               _vp, _sz, _vp]
lib.seq_chunk_gemm_noalloc.restype = _i32
lib.seq_chunk_gemm_noalloc.argtypes = [_i64, _i64, _i64,
                                       _vp, _i64, _i32, _i32, _vp,
                                       _vp, _i64, _i32, _i32, _vp,
                                       _vp, _i64, _i32,
                                       _i32, _i32, _vp, _i64, _vp,
                                       _i32, _vp, _vp]
lib.tp_mlp_fwd.restype = _i32
lib.tp_mlp_fwd.argtypes = [_i64, _i64, _i64, _i32, _i32,
                           _vp, _vp, _vp,
                           _i32, _vp, _i32,
                           _vp, _vp, _vp, _vp,
                           _i32, _vp, _vp, _u32,
                           _vp, _vp,
                           _vp, _sz, _vp]
lib.tp_mlp_bwd.restype = _i32
lib.tp_mlp_bwd.argtypes = [_i64, _i64, _i64, _i32, _i32,
                           _vp, _vp, _vp,
                           _vp, _vp, _vp,
                           _i32, _i32,
                           _vp, _vp, _vp, _i32,
                           _i32, _vp, _vp, _u32,
                           _vp, _sz, _vp]
lib.tp_linear_bwd.restype = _i32
lib.tp_linear_bwd.argtypes = [_i64, _i64, _i64,
                              _vp, _vp, _vp, _i32,
                              _vp, _vp, _i32,
                              _vp, _sz, _vp]
lib.tp_gated_mlp_fwd.restype = _i32
lib.tp_gated_mlp_fwd.argtypes = [_i64, _i64, _i64, _i32, _i32,
                                 _vp, _vp, _vp, _i32, _i32,
                                 _vp, _vp, _vp,
                                 _i32, _vp, _vp, _u32,
                                 _vp, _vp,
                                 _vp, _sz, _vp]
lib.tp_gated_mlp_bwd.restype = _i32
lib.tp_gated_mlp_bwd.argtypes = [_i64, _i64, _i64, _i32, _i32,
                                 _vp, _vp, _vp,
                                 _vp, _vp, _vp, _i32, _i32,
                                 _vp, _vp, _vp, _i32,
                                 _i32, _vp, _vp, _u32,
                                 _vp, _sz, _vp]
lib.tpm_mx_scales_bytes.restype = _sz
lib.tpm_mx_scales_bytes.argtypes = [_i64, _i64]
lib.tpm_mx_swizzle_scales.restype = _i32
lib.tpm_mx_swizzle_scales.argtypes = [_i64, _i64, _vp, _i64, _vp, _vp]
lib.seq_chunk_gemm_mx.restype = _i32
lib.seq_chunk_gemm_mx.argtypes = [_i64, _i64, _i64,
                                  _vp, _i64, _vp,
                                  _vp, _i64, _vp,
                                  _vp, _i64, _i32, _vp,
                                  _i32, _vp, _i64,
                                  _i32, _vp, _vp, _u32,
                                  _vp, _sz, _vp]
lib.tp_mlp_fwd_mx.restype = _i32
lib.tp_mlp_fwd_mx.argtypes = [_i64, _i64, _i64, _i32, _i32,
                              _vp, _vp, _vp, _vp,
                              _vp, _vp, _i32,
                              _vp, _vp, _vp, _vp,
                              _i32, _vp, _vp, _u32,
                              _vp, _vp,
                              _vp, _sz, _vp]
lib.tp_mlp_fwd_delayed.restype = _i32
lib.tp_mlp_fwd_delayed.argtypes = [_i64, _i64, _i64, _i32, _i32,
                                   _vp, _vp, _vp, _vp,
                                   _vp, _vp, _i32,
                                   _vp, _vp, _vp,
                                   _i32, _vp, _vp, _u32,
                                   _vp, _vp,
                                   _vp, _sz, _vp]
lib.tpm_fp8_delayed_scale.restype = _i32
lib.tpm_fp8_delayed_scale.argtypes = [_vp, _i32, _vp, _vp]
lib.tpm_cast_fp8.restype = _i32
lib.tpm_cast_fp8.argtypes = [_i64, _i64, _vp, _i64, _i32, _vp, _i64, _vp, _i64, _vp, _vp, _sz, _vp]
lib.tp_mlp_bwd_fp8.restype = _i32
lib.tp_mlp_bwd_fp8.argtypes = [_i64, _i64, _i64, _i32, _i32,
                               _vp, _vp, _vp, _vp,
                               _vp, _vp, _vp, _i32, _vp, _i32,
                               _vp, _vp, _vp, _i32,
                               _i32, _vp, _vp, _u32,
                               _vp, _sz, _vp]
lib.partial_reduce_seqshard.restype = _i32
lib.partial_reduce_seqshard.argtypes = [_i32, _i64, _i64, _i32,
                                        _vp, _i64, _i64, _i32,
                                        _vp, _i64, _i32, _vp]
lib.tpm_workspace_bytes.restype = _sz
lib.tpm_workspace_bytes.argtypes = [_i32, _i64, _i64, _i64, _i32, _i32, _i32]
lib.tpm_signal_chunk.restype = _i32
lib.tpm_signal_chunk.argtypes = [_vp, _vp, _u32]
lib.tpm_write_chunks.restype = _i32
lib.tpm_write_chunks.argtypes = [_vp, _vp, _i64, _i32, _vp, _vp, _vp, _u32, _vp, _vp]
lib.tpm_poll_device_error.restype = _i32
lib.tpm_poll_device_error.argtypes = [_vp]
lib.tpm_set_wait_limit.restype = _i32
lib.tpm_set_wait_limit.argtypes = [_u32]
lib.tpm_last_error.restype = ctypes.c_char_p
lib.tpm_last_error.argtypes = []
lib.tpm_version.restype = ctypes.c_char_p
lib.tpm_version.argtypes = []

EXPORTS = ["seq_chunk_gemm", "seq_chunk_gemm_noalloc", "tp_mlp_fwd", "tp_mlp_bwd", "tp_linear_bwd", "tp_gated_mlp_fwd", "tp_gated_mlp_bwd",
           "seq_chunk_gemm_mx", "tp_mlp_fwd_mx", "tpm_mx_scales_bytes", "tpm_mx_swizzle_scales",
           "tp_mlp_fwd_delayed", "tpm_fp8_delayed_scale", "tpm_cast_fp8", "tp_mlp_bwd_fp8",
           "partial_reduce_seqshard",
           "tpm_workspace_bytes", "tpm_signal_chunk", "tpm_write_chunks", "tpm_poll_device_error",
           "tpm_set_wait_limit", "tpm_last_error", "tpm_version"]


class TpmError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"tpmlp error {code}: {msg}")
        self.code = code


def last_error() -> str:
    return lib.tpm_last_error().decode()


def check(rc: int) -> int:
    if rc != OK:
        raise TpmError(rc, last_error())
    return rc


def int_array(values):
    """Host int32 array for order arguments (or None)."""
    if values is None:
        return None
    arr = (ctypes.c_int32 * len(values))(*[int(v) for v in values])
    return arr
