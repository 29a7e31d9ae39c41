"""ctypes binding of libqkprep (include/qkprep.h).

Argument marshalling only: tensors become device pointers and element
strides, enum names become integers, and the call goes straight to the C
entry point of the same name on torch's current HIP stream.  Every step of
the prepare pass runs in the library's kernels; there is no fallback.  If
``libqkprep.so`` has not been built the import fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqkprep.so")

QKPREP_OK = 0
_STATUS = {0: "QKPREP_OK", 1: "QKPREP_E_NULL", 2: "QKPREP_E_SHAPE", 3: "QKPREP_E_UNSUPPORTED",
           4: "QKPREP_E_ALIGN", 5: "QKPREP_E_RANGE", 6: "QKPREP_E_LAUNCH", 7: "QKPREP_E_VERSION"}

BF16, FP8_E4M3 = 0, 1
NORM_NONE, NORM_RMS, NORM_GEMMA = 0, 1, 2
ROPE_NEOX, ROPE_INTERLEAVED = 0, 1
Q_BF16, Q_FP8_DYNAMIC, Q_FP8_STATIC = 0, 1, 2
KV_SCALE_STATIC, KV_SCALE_TOKEN, KV_SCALE_GROUP = 0, 1, 2
QSCALE_TOKEN_HEAD, QSCALE_REQ_HEAD_PADDED = 0, 1
STORE_STREAM, STORE_KEEP = 0, 1
ADDR_PAGED, ADDR_SLOT = 0, 1

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float


class NormRopeAppendParams(ctypes.Structure):
    """Mirror of qkprep_norm_rope_append_params (field order and types)."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("num_tokens", _i32), ("num_q_heads", _i32), ("num_kv_heads", _i32),
        ("head_dim", _i32), ("rotary_dim", _i32),
        ("qkv", _vp), ("qkv_row_stride", _i64),
        ("norm", _i32), ("eps", _f32), ("q_norm_weight", _vp), ("k_norm_weight", _vp),
        ("rope", _i32), ("cos_sin_cache", _vp), ("cos_sin_rows", _i64), ("positions", _vp),
        ("addressing", _i32), ("num_requests", _i32), ("q_indptr", _vp), ("seq_lens", _vp),
        ("page_table", _vp), ("max_pages_per_request", _i32), ("slot_mapping", _vp),
        ("k_cache", _vp), ("v_cache", _vp), ("kv_dtype", _i32), ("num_pages", _i32), ("page_size", _i32),
        ("k_page_stride", _i64), ("v_page_stride", _i64), ("k_scale", _vp), ("v_scale", _vp),
        ("zero_tail", _i32),
        ("q_out", _vp), ("q_out_row_stride", _i64), ("q_mode", _i32), ("q_scale", _vp),
        ("q_scale_layout", _i32), ("max_seqlen", _i32), ("q_scale_inv", _vp), ("upper_max", _f32),
        ("k_out", _vp), ("k_out_row_stride", _i64),
        ("flags", _vp),
        ("out_k", _vp), ("out_v", _vp), ("out_kv_row_stride", _i64),
        ("kv_scale_mode", _i32), ("kv_group_size", _i32), ("k_scale_out", _vp), ("v_scale_out", _vp),
        ("store_policy", _i32),
    ]


class MlaParams(ctypes.Structure):
    """Mirror of qkprep_mla_params."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("num_tokens", _i32), ("num_q_heads", _i32), ("nope_dim", _i32), ("rope_dim", _i32),
        ("kv_lora_rank", _i32),
        ("q", _vp), ("q_token_stride", _i64), ("q_head_stride", _i64),
        ("kv_c", _vp), ("kv_c_stride", _i64), ("k_pe", _vp), ("k_pe_stride", _i64),
        ("rope", _i32), ("cos_sin_cache", _vp), ("cos_sin_rows", _i64), ("positions", _vp),
        ("slot_mapping", _vp),
        ("kv_cache", _vp), ("kv_dtype", _i32), ("num_blocks", _i64), ("block_size", _i32),
        ("block_stride", _i64), ("kv_scale", _vp),
        ("q_mode", _i32), ("q_out", _vp), ("q_out_token_stride", _i64), ("q_out_head_stride", _i64),
        ("q_scale", _vp), ("q_scale_inv", _vp), ("upper_max", ctypes.c_float),
        ("store_policy", _i32),
    ]


class QkprepError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        msg = _lib().qkprep_status_string(status).decode()
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libqkprep.so is not built ({LIB_PATH}); run __graft_entry__.build() "
                              "or python -m paged_kv_cache_token_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        L.qkprep_norm_rope_append.restype = ctypes.c_int
        L.qkprep_norm_rope_append.argtypes = [ctypes.POINTER(NormRopeAppendParams), ctypes.c_void_p]
        L.qkprep_mla_concat_rope_append.restype = ctypes.c_int
        L.qkprep_mla_concat_rope_append.argtypes = [ctypes.POINTER(MlaParams), ctypes.c_void_p]
        L.qkprep_status_string.restype = ctypes.c_char_p
        L.qkprep_status_string.argtypes = [ctypes.c_int]
        L.qkprep_abi_version.restype = ctypes.c_int
        L.qkprep_abi_version.argtypes = []
        _LIB = L
    return _LIB


def lib():
    """The loaded libqkprep (ctypes.CDLL)."""
    return _lib()


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def qkprep_abi_version() -> int:
    return _lib().qkprep_abi_version()


def qkprep_status_string(status: int) -> str:
    return _lib().qkprep_status_string(status).decode()


def call_norm_rope_append(params: NormRopeAppendParams, stream=None) -> int:
    """Call the C entry point with a filled struct; returns the status code."""
    params.struct_size = ctypes.sizeof(NormRopeAppendParams)
    return _lib().qkprep_norm_rope_append(ctypes.byref(params), _stream(stream))


def call_mla_concat_rope_append(params: MlaParams, stream=None) -> int:
    params.struct_size = ctypes.sizeof(MlaParams)
    return _lib().qkprep_mla_concat_rope_append(ctypes.byref(params), _stream(stream))


def norm_rope_append_params(*, qkv, num_q_heads, num_kv_heads, head_dim, cos_sin_cache, positions,
                            k_cache, v_cache, q_out, norm=NORM_RMS, eps=1e-6, q_norm_weight=None,
                            k_norm_weight=None, rope=ROPE_NEOX, addressing=ADDR_PAGED, q_indptr=None,
                            seq_lens=None, page_table=None, slot_mapping=None, kv_dtype=BF16,
                            page_size=None, num_pages=None, k_page_stride=None, v_page_stride=None,
                            k_scale=None, v_scale=None, zero_tail=1, q_out_row_stride=None, q_mode=Q_BF16,
                            q_scale=None, q_scale_layout=QSCALE_TOKEN_HEAD, max_seqlen=0, q_scale_inv=None,
                            upper_max=448.0, k_out=None, k_out_row_stride=None, flags=None,
                            num_tokens=None, qkv_row_stride=None, num_requests=None,
                            rotary_dim=None, out_k=None, out_v=None, out_kv_row_stride=None,
                            kv_scale_mode=KV_SCALE_STATIC, kv_group_size=0, k_scale_out=None,
                            v_scale_out=None, store_policy=STORE_STREAM) -> NormRopeAppendParams:
    """Fill the params struct from tensors (shapes/strides read from them when not given).

    The struct holds raw device pointers; it also keeps a reference to every
    tensor it points into, so the memory stays allocated as long as the
    struct is alive (a temporary passed here would otherwise be freed and its
    memory handed to the next allocation)."""
    p = NormRopeAppendParams()
    p._tensors = tuple(t for t in (qkv, cos_sin_cache, positions, k_cache, v_cache, q_out, q_norm_weight,
                                   k_norm_weight, q_indptr, seq_lens, page_table, slot_mapping, k_scale, v_scale,
                                   q_scale, q_scale_inv, k_out, flags, out_k, out_v, k_scale_out, v_scale_out)
                       if t is not None)
    p.num_tokens = qkv.shape[0] if num_tokens is None else num_tokens
    p.num_q_heads, p.num_kv_heads, p.head_dim = num_q_heads, num_kv_heads, head_dim
    p.rotary_dim = head_dim if rotary_dim is None else rotary_dim
    p.qkv = _ptr(qkv)
    p.qkv_row_stride = qkv.stride(0) if qkv_row_stride is None else qkv_row_stride
    p.norm, p.eps = norm, eps
    p.q_norm_weight, p.k_norm_weight = _ptr(q_norm_weight), _ptr(k_norm_weight)
    p.rope = rope
    p.cos_sin_cache = _ptr(cos_sin_cache)
    p.cos_sin_rows = cos_sin_cache.shape[0] if cos_sin_cache is not None else 0
    p.positions = _ptr(positions)
    p.addressing = addressing
    if addressing == ADDR_PAGED:
        p.num_requests = (seq_lens.shape[0] if seq_lens is not None else 0) if num_requests is None else num_requests
        p.q_indptr, p.seq_lens, p.page_table = _ptr(q_indptr), _ptr(seq_lens), _ptr(page_table)
        p.max_pages_per_request = page_table.shape[1] if page_table is not None else 0
    p.slot_mapping = _ptr(slot_mapping)
    p.k_cache, p.v_cache = _ptr(k_cache), _ptr(v_cache)
    p.kv_dtype = kv_dtype
    p.num_pages = (k_cache.shape[0] if k_cache is not None else 0) if num_pages is None else num_pages
    p.page_size = (k_cache.shape[1] if k_cache is not None else 0) if page_size is None else page_size
    p.k_page_stride = (k_cache.stride(0) if k_cache is not None else 0) if k_page_stride is None else k_page_stride
    p.v_page_stride = (v_cache.stride(0) if v_cache is not None else 0) if v_page_stride is None else v_page_stride
    p.k_scale, p.v_scale = _ptr(k_scale), _ptr(v_scale)
    p.zero_tail = zero_tail
    p.q_out = _ptr(q_out)
    p.q_out_row_stride = q_out.stride(0) if q_out_row_stride is None else q_out_row_stride
    p.q_mode = q_mode
    p.q_scale = _ptr(q_scale)
    p.q_scale_layout = q_scale_layout
    p.max_seqlen = max_seqlen
    p.q_scale_inv = _ptr(q_scale_inv)
    p.upper_max = upper_max
    p.k_out = _ptr(k_out)
    if k_out is not None:
        p.k_out_row_stride = k_out.stride(0) if k_out_row_stride is None else k_out_row_stride
    p.flags = _ptr(flags)
    p.out_k, p.out_v = _ptr(out_k), _ptr(out_v)
    if out_k is not None:
        p.out_kv_row_stride = out_k.stride(0) if out_kv_row_stride is None else out_kv_row_stride
    p.kv_scale_mode, p.kv_group_size = kv_scale_mode, kv_group_size
    p.k_scale_out, p.v_scale_out = _ptr(k_scale_out), _ptr(v_scale_out)
    p.store_policy = store_policy
    return p


def qkprep_norm_rope_append(stream=None, **kw) -> None:
    """Fused Q/K RMSNorm + RoPE + (FP8) quant + paged KV append (one launch).

    Keyword arguments are the fields of qkprep_norm_rope_append_params given
    as tensors / ints (see include/qkprep.h); raises QkprepError on a
    non-OK status.
    """
    st = call_norm_rope_append(norm_rope_append_params(**kw), stream)
    if st != QKPREP_OK:
        raise QkprepError(st)


def mla_params(*, q, kv_c, k_pe, cos_sin_cache, positions, slot_mapping, kv_cache, num_q_heads,
               nope_dim=128, rope_dim=64, kv_lora_rank=512, rope=ROPE_INTERLEAVED, kv_dtype=FP8_E4M3,
               kv_scale=None, num_tokens=None, q_token_stride=None, q_head_stride=None, q_mode=Q_BF16,
               q_out=None, q_out_token_stride=None, q_out_head_stride=None, q_scale=None, q_scale_inv=None,
               upper_max=448.0, store_policy=STORE_STREAM) -> MlaParams:
    """Fill the MLA params struct from tensors; like norm_rope_append_params,
    the struct keeps a reference to every tensor it points into."""
    p = MlaParams()
    p._tensors = tuple(t for t in (q, kv_c, k_pe, cos_sin_cache, positions, slot_mapping, kv_cache, kv_scale,
                                   q_out, q_scale, q_scale_inv) if t is not None)
    p.num_tokens = q.shape[0] if num_tokens is None else num_tokens
    p.num_q_heads, p.nope_dim, p.rope_dim, p.kv_lora_rank = num_q_heads, nope_dim, rope_dim, kv_lora_rank
    p.q = _ptr(q)
    p.q_token_stride = q.stride(0) if q_token_stride is None else q_token_stride
    p.q_head_stride = q.stride(1) if q_head_stride is None else q_head_stride
    p.kv_c, p.kv_c_stride = _ptr(kv_c), kv_c.stride(0)
    p.k_pe, p.k_pe_stride = _ptr(k_pe), k_pe.stride(0)
    p.rope = rope
    p.cos_sin_cache, p.cos_sin_rows = _ptr(cos_sin_cache), cos_sin_cache.shape[0]
    p.positions, p.slot_mapping = _ptr(positions), _ptr(slot_mapping)
    p.kv_cache, p.kv_dtype = _ptr(kv_cache), kv_dtype
    p.num_blocks, p.block_size, p.block_stride = kv_cache.shape[0], kv_cache.shape[1], kv_cache.stride(0)
    p.kv_scale = _ptr(kv_scale)
    p.q_mode = q_mode
    p.q_out = _ptr(q_out)
    if q_out is not None:
        p.q_out_token_stride = q_out.stride(0) if q_out_token_stride is None else q_out_token_stride
        p.q_out_head_stride = q_out.stride(1) if q_out_head_stride is None else q_out_head_stride
    p.q_scale, p.q_scale_inv, p.upper_max = _ptr(q_scale), _ptr(q_scale_inv), upper_max
    p.store_policy = store_policy
    return p


def qkprep_mla_concat_rope_append(stream=None, **kw) -> None:
    """MLA: RoPE on q's rope slice in place (or [q_nope | RoPE(q_rope)] as E4M3
    into q_out) + [kv_c | RoPE(k_pe)] into the latent cache."""
    st = call_mla_concat_rope_append(mla_params(**kw), stream)
    if st != QKPREP_OK:
        raise QkprepError(st)
