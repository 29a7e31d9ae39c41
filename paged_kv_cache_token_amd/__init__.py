"""libqkprep for MI355X: the fused pre-attention prepare pass (Q/K RMSNorm +
RoPE + FP8 quantisation + paged KV append, and the MLA latent concat) as
hand-written HIP kernels for gfx950 behind a C ABI (include/qkprep.h).

This package holds the HIP sources (``csrc/``), the in-tree build
(``build.py``) and the ctypes binding (``binding.py``).  PyTorch only
provides device memory and streams.
"""
from .binding import (  # noqa: F401
    ADDR_PAGED, ADDR_SLOT, BF16, FP8_E4M3, KV_SCALE_GROUP, KV_SCALE_STATIC, KV_SCALE_TOKEN, NORM_GEMMA, NORM_NONE, NORM_RMS, QSCALE_REQ_HEAD_PADDED,
    QSCALE_TOKEN_HEAD, Q_BF16, STORE_KEEP, STORE_STREAM, Q_FP8_DYNAMIC, Q_FP8_STATIC, ROPE_INTERLEAVED, ROPE_NEOX, LIB_PATH,
    MlaParams, NormRopeAppendParams, QkprepError, call_mla_concat_rope_append, call_norm_rope_append,
    lib, mla_params, norm_rope_append_params, qkprep_abi_version, qkprep_mla_concat_rope_append,
    qkprep_norm_rope_append, qkprep_status_string,
)
