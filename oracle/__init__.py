"""CPU oracle for the pre-attention prepare pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (``libqkprep`` and its
binding in ``paged_kv_cache_token_amd``) never imports, loads or calls it.

The arithmetic lives in ``qkprep_oracle.c`` (plain single-threaded C99, fp64,
one rounding at the end); this module only builds it with gcc and marshals
numpy arrays through ctypes.  It shares no code with the HIP library.

Every function of the oracle is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` against closed forms, invariants, library
conversions and brute-force enumeration; the pages print no worked numeric
example (see the header of ``qkprep_oracle.c`` for the passages followed).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qkprep_oracle.c")
_LIB = os.path.join(_HERE, "libqkprep_oracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no FP contraction, strict IEEE)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
            "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm",
        ])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        L.oracle_bf16_to_f64.restype = ctypes.c_double
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_e4m3_to_f64.restype = ctypes.c_double
        L.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        L.oracle_f64_to_e4m3.restype = ctypes.c_uint8
        L.oracle_f64_to_e4m3.argtypes = [ctypes.c_double]
        L.oracle_f32_to_bf16_n.restype = None
        L.oracle_f32_to_bf16_n.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        L.oracle_f64_to_e4m3_n.restype = None
        L.oracle_f64_to_e4m3_n.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        L.oracle_rmsnorm.restype = None
        L.oracle_rmsnorm.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                     ctypes.c_double, ctypes.c_void_p]
        L.oracle_rope.restype = None
        L.oracle_rope.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_rope_partial.restype = None
        L.oracle_rope_partial.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_q_scale.restype = ctypes.c_float
        L.oracle_q_scale.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_double]
        L.oracle_norm_rope_append.restype = ctypes.c_int
        L.oracle_norm_rope_append.argtypes = [ctypes.c_void_p]
        L.oracle_mla_concat_rope_append.restype = ctypes.c_int
        L.oracle_mla_concat_rope_append.argtypes = [ctypes.c_void_p]
        _lib = L
    return _lib


# ----------------------------------------------------------------------------
# converters and step functions
# ----------------------------------------------------------------------------

def _ptr(a: np.ndarray | None) -> int | None:
    if a is None:
        return None
    return a.ctypes.data


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits (RNE), elementwise."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_f32_to_bf16_n(_ptr(x), _ptr(out), x.size)
    return out


def f64_to_e4m3(x: np.ndarray) -> np.ndarray:
    """fp64 -> E4M3 code (RN satfinite), elementwise."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().oracle_f64_to_e4m3_n(_ptr(x), _ptr(out), x.size)
    return out


def e4m3_to_f64(code: int) -> float:
    return lib().oracle_e4m3_to_f64(int(code))


def bf16_to_f64(bits: int) -> float:
    return lib().oracle_bf16_to_f64(int(bits))


def rmsnorm(x: np.ndarray, w: np.ndarray | None, norm: int, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    D = x.size
    w = np.ones(D, np.float32) if w is None else np.ascontiguousarray(w, dtype=np.float32)
    y = np.empty(D, np.float64)
    lib().oracle_rmsnorm(_ptr(x), D, _ptr(w), norm, float(eps), _ptr(y))
    return y


def rope(y: np.ndarray, rope_style: int, c: np.ndarray, s: np.ndarray, rot: int | None = None) -> np.ndarray:
    """RoPE of one head row; ``rot`` rotated dims (default: the whole row)."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    c = np.ascontiguousarray(c, dtype=np.float64)
    s = np.ascontiguousarray(s, dtype=np.float64)
    o = np.empty_like(y)
    if rot is None:
        lib().oracle_rope(_ptr(y), y.size, rope_style, _ptr(c), _ptr(s), _ptr(o))
    else:
        lib().oracle_rope_partial(_ptr(y), y.size, int(rot), rope_style, _ptr(c), _ptr(s), _ptr(o))
    return o


def q_scale(v32: np.ndarray, upper_max: float) -> float:
    v32 = np.ascontiguousarray(v32, dtype=np.float32)
    return lib().oracle_q_scale(_ptr(v32), v32.size, float(upper_max))


# ----------------------------------------------------------------------------
# fused pass
# ----------------------------------------------------------------------------

class _NraArgs(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
        ("rot", ctypes.c_int32),
        ("qkv", ctypes.c_void_p), ("qkv_row_stride", ctypes.c_int64),
        ("norm", ctypes.c_int32), ("eps", ctypes.c_float),
        ("q_w", ctypes.c_void_p), ("k_w", ctypes.c_void_p),
        ("rope", ctypes.c_int32), ("cos_sin", ctypes.c_void_p), ("cs_rows", ctypes.c_int64),
        ("positions", ctypes.c_void_p),
        ("addressing", ctypes.c_int32), ("B", ctypes.c_int32),
        ("q_indptr", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p), ("page_table", ctypes.c_void_p),
        ("maxp", ctypes.c_int32), ("slot_mapping", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("kv_fp8", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("k_page_stride", ctypes.c_int64), ("v_page_stride", ctypes.c_int64),
        ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float), ("zero_tail", ctypes.c_int32),
        ("q_out", ctypes.c_void_p), ("q_out_row_stride", ctypes.c_int64), ("q_mode", ctypes.c_int32),
        ("q_scale", ctypes.c_void_p), ("q_scale_padded", ctypes.c_int32), ("max_seqlen", ctypes.c_int32),
        ("q_scale_inv", ctypes.c_float), ("upper_max", ctypes.c_float),
        ("k_out", ctypes.c_void_p), ("k_out_row_stride", ctypes.c_int64),
        ("flags", ctypes.c_void_p),
        ("out_k", ctypes.c_void_p), ("out_v", ctypes.c_void_p), ("out_kv_row_stride", ctypes.c_int64),
        ("kv_scale_mode", ctypes.c_int32), ("kv_group_size", ctypes.c_int32),
        ("k_scale_out", ctypes.c_void_p), ("v_scale_out", ctypes.c_void_p),
    ]


class _MlaArgs(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("nope_dim", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32), ("kv_lora_rank", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("q_token_stride", ctypes.c_int64), ("q_head_stride", ctypes.c_int64),
        ("kv_c", ctypes.c_void_p), ("kv_c_stride", ctypes.c_int64),
        ("k_pe", ctypes.c_void_p), ("k_pe_stride", ctypes.c_int64),
        ("rope", ctypes.c_int32), ("cos_sin", ctypes.c_void_p), ("cs_rows", ctypes.c_int64),
        ("positions", ctypes.c_void_p), ("slot_mapping", ctypes.c_void_p),
        ("kv_cache", ctypes.c_void_p), ("kv_fp8", ctypes.c_int32), ("num_blocks", ctypes.c_int64),
        ("block_size", ctypes.c_int32), ("block_stride", ctypes.c_int64), ("kv_scale", ctypes.c_float),
        ("q_mode", ctypes.c_int32), ("q_out", ctypes.c_void_p), ("q_out_token_stride", ctypes.c_int64),
        ("q_out_head_stride", ctypes.c_int64), ("q_scale", ctypes.c_void_p), ("q_scale_inv", ctypes.c_float),
        ("upper_max", ctypes.c_float),
    ]


def _need(a: np.ndarray, dtype) -> np.ndarray:
    if a.dtype != dtype or not a.flags["C_CONTIGUOUS"]:
        raise TypeError(f"oracle expects a C-contiguous {np.dtype(dtype)} array, got {a.dtype}")
    return a


@dataclass
class NraResult:
    q_out: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    q_scale: np.ndarray | None
    flags: np.ndarray | None
    qkv: np.ndarray


def norm_rope_append(inp, out) -> NraResult:
    """Run the oracle on host copies.

    ``inp`` is a workloads.NraInputs (inputs + scalars); ``out`` holds the
    output buffers as numpy arrays (``q_out``, ``k_cache``, ``v_cache``,
    ``q_scale``, ``flags``, ``qkv``), which are updated in place.  For the
    in-place variant (``inp.q_in_place``) ``q_out`` is ``qkv`` itself.
    """
    qkv = _need(out["qkv"], np.uint16)
    k_cache = _need(out["k_cache"], np.uint8 if inp.kv_fp8 else np.uint16)
    v_cache = _need(out["v_cache"], np.uint8 if inp.kv_fp8 else np.uint16)
    D = inp.D
    a = _NraArgs()
    a.T, a.Hq, a.Hkv, a.D, a.rot = inp.T, inp.Hq, inp.Hkv, D, inp.rot
    a.qkv = _ptr(qkv)
    a.qkv_row_stride = inp.qkv_row_stride
    a.norm = inp.norm
    a.eps = inp.eps
    a.q_w = _ptr(_need(inp.q_norm_weight, np.float32))
    a.k_w = _ptr(_need(inp.k_norm_weight, np.float32))
    a.rope = inp.rope
    a.cos_sin = _ptr(_need(inp.cos_sin, np.float32))
    a.cs_rows = inp.cos_sin.shape[0]
    a.positions = _ptr(_need(inp.positions, np.int64))
    a.addressing = inp.addressing
    a.B = inp.B
    if inp.addressing == 0:
        a.q_indptr = _ptr(_need(inp.q_indptr, np.int32))
        a.seq_lens = _ptr(_need(inp.seq_lens, np.int32))
        a.page_table = _ptr(_need(inp.page_table, np.int32))
        a.maxp = inp.page_table.shape[1]
    else:
        a.slot_mapping = _ptr(_need(inp.slot_mapping, np.int64))
    a.k_cache = _ptr(k_cache)
    a.v_cache = _ptr(v_cache)
    a.kv_fp8 = 1 if inp.kv_fp8 else 0
    a.num_pages = inp.num_pages
    a.page_size = inp.page_size
    a.k_page_stride = inp.page_size * inp.Hkv * D
    a.v_page_stride = inp.page_size * inp.Hkv * D
    a.k_scale = inp.k_scale
    a.v_scale = inp.v_scale
    a.zero_tail = 1 if inp.zero_tail else 0
    if inp.q_in_place:
        a.q_out = _ptr(qkv)
        a.q_out_row_stride = inp.qkv_row_stride
    else:
        q_out = _need(out["q_out"], np.uint8 if inp.q_mode else np.uint16)
        a.q_out = _ptr(q_out)
        a.q_out_row_stride = inp.Hq * D
    a.q_mode = inp.q_mode
    if inp.q_mode == 1:
        a.q_scale = _ptr(_need(out["q_scale"], np.float32))
    a.q_scale_padded = 1 if inp.q_scale_padded else 0
    a.max_seqlen = inp.max_seqlen
    a.q_scale_inv = inp.q_scale_inv
    a.upper_max = inp.upper_max
    if inp.k_in_place:
        a.k_out = qkv.ctypes.data + inp.Hq * D * 2
        a.k_out_row_stride = inp.qkv_row_stride
    if out.get("flags") is not None:
        a.flags = _ptr(_need(out["flags"], np.int32))
    kdt = np.uint8 if inp.kv_fp8 else np.uint16
    if inp.kv_redirect:
        a.out_k = _ptr(_need(out["out_k"], kdt))
        a.out_v = _ptr(_need(out["out_v"], kdt))
        a.out_kv_row_stride = inp.Hkv * D
    a.kv_scale_mode = inp.kv_scale_mode
    a.kv_group_size = inp.kv_group_size
    if inp.kv_scale_mode:
        a.k_scale_out = _ptr(_need(out["k_scale_out"], np.float32))
        a.v_scale_out = _ptr(_need(out["v_scale_out"], np.float32))
    rc = lib().oracle_norm_rope_append(ctypes.byref(a))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")
    return NraResult(q_out=qkv if inp.q_in_place else out["q_out"], k_cache=k_cache, v_cache=v_cache,
                     q_scale=out.get("q_scale"), flags=out.get("flags"), qkv=qkv)


def mla_concat_rope_append(inp, out) -> None:
    """Run the MLA oracle; ``out`` holds ``q`` (updated in place in the bf16
    Q mode), ``kv_cache`` and, in the FP8 Q modes, ``q_out`` (and ``q_scale``
    for the dynamic one)."""
    q = _need(out["q"], np.uint16)
    cache = _need(out["kv_cache"], np.uint8 if inp.kv_fp8 else np.uint16)
    a = _MlaArgs()
    a.T, a.H, a.nope_dim, a.rope_dim, a.kv_lora_rank = inp.T, inp.H, inp.nope_dim, inp.rope_dim, inp.kv_lora_rank
    a.q = _ptr(q)
    a.q_token_stride = inp.H * (inp.nope_dim + inp.rope_dim)
    a.q_head_stride = inp.nope_dim + inp.rope_dim
    a.kv_c = _ptr(_need(inp.kv_c, np.uint16))
    a.kv_c_stride = inp.kv_lora_rank
    a.k_pe = _ptr(_need(inp.k_pe, np.uint16))
    a.k_pe_stride = inp.rope_dim
    a.rope = inp.rope
    a.cos_sin = _ptr(_need(inp.cos_sin, np.float32))
    a.cs_rows = inp.cos_sin.shape[0]
    a.positions = _ptr(_need(inp.positions, np.int64))
    a.slot_mapping = _ptr(_need(inp.slot_mapping, np.int64))
    a.kv_cache = _ptr(cache)
    a.kv_fp8 = 1 if inp.kv_fp8 else 0
    a.num_blocks = inp.num_blocks
    a.block_size = inp.block_size
    a.block_stride = inp.block_size * (inp.kv_lora_rank + inp.rope_dim)
    a.kv_scale = inp.kv_scale
    a.q_mode = inp.q_mode
    if inp.q_mode != 0:
        q_out = _need(out["q_out"], np.uint8)
        a.q_out = _ptr(q_out)
        a.q_out_token_stride = inp.H * (inp.nope_dim + inp.rope_dim)
        a.q_out_head_stride = inp.nope_dim + inp.rope_dim
        a.q_scale_inv = inp.q_scale_inv
        a.upper_max = inp.upper_max
        if inp.q_mode == 1:
            a.q_scale = _ptr(_need(out["q_scale"], np.float32))
    rc = lib().oracle_mla_concat_rope_append(ctypes.byref(a))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")
