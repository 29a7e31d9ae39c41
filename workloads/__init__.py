"""Seeded synthetic inputs for the prepare pass (shared by the tests, the
bench and the smoke check).

This module only draws inputs: it holds none of the method's arithmetic.
It never imports the HIP binding or the oracle.  Every array is numpy on the
host; bf16 tensors are carried as raw ``uint16`` bit patterns and FP8 caches
as ``uint8`` codes.  bf16 values are drawn in fp64 and rounded to bf16 with
torch's conversion (a library routine).

Shapes and distributions follow the five configurations the prepare pass is
measured on (tiny decode, B=256 decode, ragged FP8 prefill, strided D=256
Gemma path, MLA concat) -- see ``CONFIGS``; each constructor's docstring
states its recipe.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64/fp32 values to bf16 (torch's RNE conversion); return bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Values rounded to bf16, returned as fp32."""
    return bf16_bits_to_f32(to_bf16_bits(x))


def cos_sin_table(rows: int, rot_dim: int, theta: float) -> np.ndarray:
    """fp32 [rows, rot_dim]: row p = [cos(p f_0..f_{R/2-1}) | sin(...)],
    f_i = theta^(-2i/R), evaluated in fp64 and rounded once to fp32."""
    half = rot_dim // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / rot_dim)
    ang = np.arange(rows, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def sentinel_bytes(rng: np.random.Generator, nbytes: int) -> np.ndarray:
    return rng.integers(0, 256, size=nbytes, dtype=np.uint8)


# ----------------------------------------------------------------------------
# norm + rope + append
# ----------------------------------------------------------------------------

Q_BF16, Q_FP8_DYNAMIC, Q_FP8_STATIC = 0, 1, 2
KV_SCALE_STATIC, KV_SCALE_TOKEN, KV_SCALE_GROUP = 0, 1, 2
NORM_NONE, NORM_RMS, NORM_GEMMA = 0, 1, 2
ROPE_NEOX, ROPE_INTERLEAVED = 0, 1
ADDR_PAGED, ADDR_SLOT = 0, 1


@dataclass
class NraInputs:
    """One call of the norm-rope-append pass with its initial output buffers."""
    name: str
    T: int
    Hq: int
    Hkv: int
    D: int
    B: int
    qkv: np.ndarray                 # uint16 [T, qkv_row_stride] (bf16 bits, padding included)
    qkv_row_stride: int             # elements
    norm: int
    eps: float
    q_norm_weight: np.ndarray       # fp32 [D]
    k_norm_weight: np.ndarray       # fp32 [D]
    rope: int
    cos_sin: np.ndarray             # fp32 [rows, rot]
    positions: np.ndarray           # int64 [T]
    addressing: int
    q_indptr: np.ndarray | None     # int32 [B+1]
    seq_lens: np.ndarray | None     # int32 [B]
    page_table: np.ndarray | None   # int32 [B, maxp]
    slot_mapping: np.ndarray | None  # int64 [T]
    kv_fp8: bool
    num_pages: int
    page_size: int
    k_scale: float
    v_scale: float
    zero_tail: bool
    q_mode: int
    q_in_place: bool
    k_in_place: bool
    q_scale_padded: bool
    max_seqlen: int
    q_scale_inv: float
    upper_max: float
    # initial contents of the outputs (sentinels); None = allocate on device
    k_cache0: np.ndarray | None
    v_cache0: np.ndarray | None
    q_out0: np.ndarray | None
    q_scale0: np.ndarray | None
    flags0: np.ndarray | None
    cache_seed: int = 0
    meta: dict = field(default_factory=dict)
    rotary_dim: int | None = None   # rotated dims per head (None: the whole head)
    # K/V redirect to caller rows out_k / out_v [T, Hkv, D] (no cache write, no tail clear)
    kv_redirect: bool = False
    out_k0: np.ndarray | None = None
    out_v0: np.ndarray | None = None
    # FP8 K/V scales: KV_SCALE_STATIC, KV_SCALE_TOKEN (per token and kv head), KV_SCALE_GROUP
    kv_scale_mode: int = 0
    kv_group_size: int = 0
    k_scale_out0: np.ndarray | None = None   # fp32 [cache rows or T, Hkv, D / group]
    v_scale_out0: np.ndarray | None = None
    # cache policy of the library's row stores (0 streaming, 1 keep); no effect on values
    store_policy: int = 0

    @property
    def R(self) -> int:
        return self.Hq + 2 * self.Hkv

    @property
    def rot(self) -> int:
        return self.D if self.rotary_dim is None else self.rotary_dim

    @property
    def kv_group(self) -> int:
        return self.kv_group_size if self.kv_scale_mode == KV_SCALE_GROUP else self.D

    @property
    def kv_elt(self) -> int:
        return 1 if self.kv_fp8 else 2

    @property
    def q_elt(self) -> int:
        return 1 if self.q_mode != Q_BF16 else 2

    @property
    def cache_shape(self):
        return (self.num_pages, self.page_size, self.Hkv, self.D)

    @property
    def q_scale_shape(self):
        if self.q_mode != Q_FP8_DYNAMIC:
            return (0,)
        if self.q_scale_padded:
            P = (self.max_seqlen + 127) // 128 * 128
            return (self.B, self.Hq, P)
        return (self.T, self.Hq)

    def touched_pages(self) -> np.ndarray:
        """Sorted physical pages this call may write (appended rows and cleared tails)."""
        if self.addressing == ADDR_SLOT:
            s = self.slot_mapping
            s = s[(s >= 0) & (s < self.num_pages * self.page_size)]
            return np.unique(s // self.page_size).astype(np.int64)
        pages = []
        for b in range(self.B):
            ql = int(self.q_indptr[b + 1] - self.q_indptr[b])
            sl = int(self.seq_lens[b])
            lo = sl - ql
            if self.zero_tail and not self.kv_redirect and ql == 0 and sl > 0:
                lo = sl - 1
            if sl > lo:
                pages.append(self.page_table[b, lo // self.page_size:(sl - 1) // self.page_size + 1])
        if not pages:
            return np.zeros(0, np.int64)
        return np.unique(np.concatenate(pages)).astype(np.int64)

    def algorithmic_bytes(self) -> dict:
        """Bytes the pass must move: qkv read (Q, K, V heads), norm weights,
        cos/sin rows, Q write (+ q_scale), K/V append, tail zeros, K write-back."""
        T, D, Hq, Hkv = self.T, self.D, self.Hq, self.Hkv
        tail_rows = 0
        if self.addressing == ADDR_PAGED and self.zero_tail:
            for b in range(self.B):
                sl = int(self.seq_lens[b])
                if sl > 0:
                    tail_rows += self.page_size - 1 - (sl - 1) % self.page_size
        if self.kv_redirect:
            tail_rows = 0
        ng = D // self.kv_group if self.kv_scale_mode else 0
        d = {
            "kv_scales": (T + tail_rows) * 2 * Hkv * ng * 4,
            "qkv_read": T * self.R * D * 2,
            "norm_weights": (2 * D * 4) if self.norm != NORM_NONE else 0,
            "cos_sin": T * self.rot * 4,
            "q_write": T * Hq * D * self.q_elt,
            "q_scale": T * Hq * 4 if self.q_mode == Q_FP8_DYNAMIC else 0,
            "kv_append": T * 2 * Hkv * D * self.kv_elt,
            "tail_zero": tail_rows * 2 * Hkv * D * self.kv_elt,
            "k_writeback": T * Hkv * D * 2 if self.k_in_place else 0,
        }
        d["total"] = sum(d.values())
        return d


def nra_case(*, name="custom", seed, q_lens, prior_lens, Hq, Hkv, D, page_size,
             qkv_sigma=1.0, row_pad=0, norm=NORM_RMS, eps=1e-6, rope=ROPE_NEOX, theta=1e6,
             cs_rows=None, kv_fp8=False, q_mode=Q_BF16, q_scale_padded=False, max_seqlen=0,
             upper_max=448.0, q_scale_inv=1.0, k_scale=1.0, v_scale=1.0, zero_tail=True,
             q_in_place=False, k_in_place=False, addressing=ADDR_PAGED, spare_pages=None,
             maxp=None, host_caches=True, positions=None, rotary_dim=None, kv_redirect=False,
             kv_scale_mode=KV_SCALE_STATIC, kv_group_size=0) -> NraInputs:
    """Draw one norm-rope-append call.

    Request b appends ``q_lens[b]`` tokens after ``prior_lens[b]`` cached
    ones; ``seq_lens = prior + q_len`` (the length after the append) and the
    position of token j of request b is ``prior_b + j``.  Pages of each
    request are a seeded random permutation of the pool; page-table columns a
    request does not own hold -1.
    """
    rng = np.random.default_rng(seed)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    prior_lens = np.asarray(prior_lens, dtype=np.int64)
    B = len(q_lens)
    T = int(q_lens.sum())
    R = Hq + 2 * Hkv
    stride = R * D + row_pad
    # qkv
    vals = rng.standard_normal((T, R * D)) * qkv_sigma
    qkv = np.empty((T, stride), np.uint16)
    qkv[:, :R * D] = to_bf16_bits(vals)
    if row_pad:
        qkv[:, R * D:] = rng.integers(0, 1 << 16, size=(T, row_pad), dtype=np.uint16)
    # norm weights (bf16-representable values held in fp32)
    if norm == NORM_GEMMA:
        qw = bf16_round(0.1 * rng.standard_normal(D))
        kw = bf16_round(0.1 * rng.standard_normal(D))
    else:
        qw = bf16_round(1.0 + 0.1 * rng.standard_normal(D))
        kw = bf16_round(1.0 + 0.1 * rng.standard_normal(D))
    seq_lens = prior_lens + q_lens
    if positions is None:
        positions = np.concatenate([prior_lens[b] + np.arange(q_lens[b]) for b in range(B)]) \
            if T else np.zeros(0, np.int64)
    positions = np.asarray(positions, dtype=np.int64)
    if cs_rows is None:
        cs_rows = int(max(int(seq_lens.max()) if B else 1, 1))
    rot = D if rotary_dim is None else int(rotary_dim)
    cos_sin = cos_sin_table(cs_rows, rot, theta) if rot else np.zeros((cs_rows, 0), np.float32)
    q_indptr = np.zeros(B + 1, np.int32)
    q_indptr[1:] = np.cumsum(q_lens)
    need = (seq_lens + page_size - 1) // page_size
    if maxp is None:
        maxp = int(max(int(need.max()) if B else 1, 1))
    used = int(need.sum())
    if spare_pages is None:
        spare_pages = max(4, used // 8)
    num_pages = used + spare_pages
    perm = rng.permutation(num_pages).astype(np.int32)
    page_table = np.full((B, maxp), -1, np.int32)
    k = 0
    for b in range(B):
        page_table[b, :need[b]] = perm[k:k + need[b]]
        k += need[b]
    slot_mapping = None
    if addressing == ADDR_SLOT:
        cap = num_pages * page_size
        slot_mapping = rng.permutation(cap)[:T].astype(np.int64)
    kv_elt = 1 if kv_fp8 else 2
    cache_bytes = num_pages * page_size * Hkv * D * kv_elt
    cache_dtype = np.uint8 if kv_fp8 else np.uint16
    cache_seed = int(rng.integers(0, 2**31))
    if host_caches:
        crng = np.random.default_rng(cache_seed)
        k_cache0 = sentinel_bytes(crng, cache_bytes).view(cache_dtype).reshape(num_pages, page_size, Hkv, D)
        v_cache0 = sentinel_bytes(crng, cache_bytes).view(cache_dtype).reshape(num_pages, page_size, Hkv, D)
    else:
        k_cache0 = v_cache0 = None
    q_elt = 1 if q_mode != Q_BF16 else 2
    q_out0 = None
    if not q_in_place:
        q_out0 = sentinel_bytes(rng, T * Hq * D * q_elt).view(np.uint8 if q_elt == 1 else np.uint16)
        q_out0 = q_out0.reshape(T, Hq, D)
    q_scale0 = None
    if q_mode == Q_FP8_DYNAMIC:
        if q_scale_padded:
            P = (max_seqlen + 127) // 128 * 128
            shape = (B, Hq, P)
        else:
            shape = (T, Hq)
        q_scale0 = sentinel_bytes(rng, int(np.prod(shape)) * 4).view(np.float32).reshape(shape)
    flags0 = np.full((B, Hkv), 0x5A5A5A5A, np.int32) if addressing == ADDR_PAGED else None
    out_k0 = out_v0 = None
    if kv_redirect:
        out_k0 = sentinel_bytes(rng, T * Hkv * D * kv_elt).view(cache_dtype).reshape(T, Hkv, D)
        out_v0 = sentinel_bytes(rng, T * Hkv * D * kv_elt).view(cache_dtype).reshape(T, Hkv, D)
    k_scale_out0 = v_scale_out0 = None
    if kv_scale_mode != KV_SCALE_STATIC:
        g = kv_group_size if kv_scale_mode == KV_SCALE_GROUP else D
        rows = T if kv_redirect else num_pages * page_size
        k_scale_out0 = sentinel_bytes(rng, rows * Hkv * (D // g) * 4).view(np.float32).reshape(rows, Hkv, D // g)
        v_scale_out0 = sentinel_bytes(rng, rows * Hkv * (D // g) * 4).view(np.float32).reshape(rows, Hkv, D // g)
    return NraInputs(
        name=name, T=T, Hq=Hq, Hkv=Hkv, D=D, B=B, qkv=qkv, qkv_row_stride=stride,
        norm=norm, eps=eps, q_norm_weight=qw.astype(np.float32), k_norm_weight=kw.astype(np.float32),
        rope=rope, cos_sin=cos_sin, positions=positions, addressing=addressing,
        q_indptr=q_indptr if addressing == ADDR_PAGED else None,
        seq_lens=seq_lens.astype(np.int32) if addressing == ADDR_PAGED else None,
        page_table=page_table if addressing == ADDR_PAGED else None,
        slot_mapping=slot_mapping, kv_fp8=kv_fp8, num_pages=num_pages, page_size=page_size,
        k_scale=k_scale, v_scale=v_scale, zero_tail=zero_tail and addressing == ADDR_PAGED,
        q_mode=q_mode, q_in_place=q_in_place, k_in_place=k_in_place,
        q_scale_padded=q_scale_padded, max_seqlen=max_seqlen, q_scale_inv=q_scale_inv,
        upper_max=upper_max, k_cache0=k_cache0, v_cache0=v_cache0, q_out0=q_out0,
        q_scale0=q_scale0, flags0=flags0, cache_seed=cache_seed,
        meta={"seed": seed, "q_lens": q_lens.tolist() if B <= 64 else None},
        rotary_dim=rot, kv_redirect=kv_redirect, out_k0=out_k0, out_v0=out_v0,
        kv_scale_mode=kv_scale_mode, kv_group_size=kv_group_size if kv_scale_mode == KV_SCALE_GROUP else 0,
        k_scale_out0=k_scale_out0, v_scale_out0=v_scale_out0,
    )


# ----------------------------------------------------------------------------
# MLA concat + rope
# ----------------------------------------------------------------------------


@dataclass
class MlaInputs:
    name: str
    T: int
    H: int
    nope_dim: int
    rope_dim: int
    kv_lora_rank: int
    q: np.ndarray            # uint16 [T, H, nope + rope]
    kv_c: np.ndarray         # uint16 [T, kv_lora_rank]
    k_pe: np.ndarray         # uint16 [T, rope_dim]
    rope: int
    cos_sin: np.ndarray      # fp32 [rows, rope_dim]
    positions: np.ndarray    # int64 [T]
    slot_mapping: np.ndarray  # int64 [T]
    kv_fp8: bool
    num_blocks: int
    block_size: int
    kv_scale: float
    kv_cache0: np.ndarray    # uint8/uint16 [num_blocks, block_size, kv_lora_rank + rope_dim]
    meta: dict = field(default_factory=dict)
    q_mode: int = Q_BF16     # Q_BF16: RoPE in place in q; FP8 modes: E4M3 q_out, q read-only
    q_scale_inv: float = 1.0
    upper_max: float = 448.0
    q_out0: np.ndarray | None = None    # uint8 [T, H, nope + rope] (FP8 Q modes)
    q_scale0: np.ndarray | None = None  # fp32 [T] (dynamic)
    store_policy: int = 0               # cache policy of the library's row stores; no effect on values

    @property
    def row_elems(self) -> int:
        return self.kv_lora_rank + self.rope_dim

    def algorithmic_bytes(self) -> dict:
        T, H, R, K = self.T, self.H, self.rope_dim, self.kv_lora_rank
        elt = 1 if self.kv_fp8 else 2
        n_written = int(((self.slot_mapping >= 0) &
                         (self.slot_mapping < self.num_blocks * self.block_size)).sum())
        if self.q_mode != Q_BF16:
            W = self.nope_dim + R
            d = {
                "q_read": T * H * W * 2,
                "q_write": T * H * W,
                "q_scale": T * 4 if self.q_mode == Q_FP8_DYNAMIC else 0,
            }
        else:
            d = {
                "q_rope_read": T * H * R * 2,
                "q_rope_write": T * H * R * 2,
            }
        d.update({
            "kv_c_read": T * K * 2,
            "k_pe_read": T * R * 2,
            "cos_sin": T * R * 4,
            "cache_write": n_written * (K + R) * elt,
        })
        d["total"] = sum(d.values())
        return d


def mla_case(*, name="custom", seed, T, H=128, nope_dim=128, rope_dim=64, kv_lora_rank=512,
             rope=ROPE_INTERLEAVED, theta=1e4, cs_rows=16384, num_blocks=128, block_size=64,
             kv_fp8=True, kv_scale=0.02, negative_slots=0, positions=None, q_mode=Q_BF16,
             q_scale_inv=1.0, upper_max=448.0) -> MlaInputs:
    rng = np.random.default_rng(seed)
    q = to_bf16_bits(rng.standard_normal((T, H, nope_dim + rope_dim)))
    kv_c = to_bf16_bits(rng.standard_normal((T, kv_lora_rank)))
    k_pe = to_bf16_bits(rng.standard_normal((T, rope_dim)))
    if positions is None:
        positions = rng.integers(0, cs_rows, size=T, dtype=np.int64)
    cos_sin = cos_sin_table(cs_rows, rope_dim, theta)
    cap = num_blocks * block_size
    slots = rng.permutation(cap)[:T].astype(np.int64)
    if negative_slots:
        slots[rng.choice(T, size=negative_slots, replace=False)] = -1
    elt = 1 if kv_fp8 else 2
    nbytes = num_blocks * block_size * (kv_lora_rank + rope_dim) * elt
    cache0 = sentinel_bytes(rng, nbytes).view(np.uint8 if kv_fp8 else np.uint16)
    cache0 = cache0.reshape(num_blocks, block_size, kv_lora_rank + rope_dim)
    q_out0 = q_scale0 = None
    if q_mode != Q_BF16:
        q_out0 = sentinel_bytes(rng, T * H * (nope_dim + rope_dim)).reshape(T, H, nope_dim + rope_dim)
        if q_mode == Q_FP8_DYNAMIC:
            q_scale0 = sentinel_bytes(rng, T * 4).view(np.float32).copy()
    return MlaInputs(name=name, T=T, H=H, nope_dim=nope_dim, rope_dim=rope_dim,
                     kv_lora_rank=kv_lora_rank, q=q, kv_c=kv_c, k_pe=k_pe, rope=rope,
                     cos_sin=cos_sin, positions=np.asarray(positions, np.int64), slot_mapping=slots,
                     kv_fp8=kv_fp8, num_blocks=num_blocks, block_size=block_size,
                     kv_scale=kv_scale, kv_cache0=cache0, meta={"seed": seed}, q_mode=q_mode,
                     q_scale_inv=q_scale_inv, upper_max=upper_max, q_out0=q_out0, q_scale0=q_scale0)


# ----------------------------------------------------------------------------
# the five measured configurations
# ----------------------------------------------------------------------------


def c1_tiny_decode(seed=1001, **kw):
    """16 requests x 1 new token, Hq/Hkv/D 8/1/128, bf16 everywhere, page 16,
    prior lengths U[1, 2048], table [4096, 128], theta 1e6."""
    rng = np.random.default_rng(seed)
    prior = rng.integers(1, 2049, size=16)
    args = dict(name="c1_tiny_decode", seed=seed + 7, q_lens=np.ones(16, np.int64), prior_lens=prior,
                Hq=8, Hkv=1, D=128, page_size=16, norm=NORM_RMS, theta=1e6, cs_rows=4096)
    args.update(kw)
    return nra_case(**args)


def c2_decode_b256(seed=1002, **kw):
    """Qwen3-8B-like decode: 256 requests x 1 token, 32/8/128, bf16, page 16,
    prior lengths U[1, 32768], table [40960, 128], theta 1e6."""
    rng = np.random.default_rng(seed)
    prior = rng.integers(1, 32769, size=256)
    args = dict(name="c2_decode_b256", seed=seed + 7, q_lens=np.ones(256, np.int64), prior_lens=prior,
                Hq=32, Hkv=8, D=128, page_size=16, norm=NORM_RMS, theta=1e6, cs_rows=40960,
                spare_pages=64, host_caches=False)
    args.update(kw)
    return nra_case(**args)


def c3_prefill_fp8(seed=1003, empty_request=None, **kw):
    """Ragged FP8 prefill: 8 requests, lengths U[1, 4096] (fresh prefill),
    64/8/128, qkv sigma 2, FP8 E4M3 caches page 64, dynamic per-token-head Q
    scale in the padded [B, Hq, 4096] layout, upper_max 448,
    k_scale = v_scale = 0.05, tails zeroed, table [40960, 128], theta 1e6."""
    rng = np.random.default_rng(seed)
    q_lens = np.asarray(kw.pop("q_lens")) if "q_lens" in kw else rng.integers(1, 4097, size=8)
    if empty_request is not None:
        q_lens[empty_request] = 0
    args = dict(name="c3_prefill_fp8", seed=seed + 7, q_lens=q_lens, prior_lens=np.zeros(len(q_lens), np.int64),
                Hq=64, Hkv=8, D=128, page_size=64, qkv_sigma=2.0, norm=NORM_RMS, theta=1e6,
                cs_rows=40960, kv_fp8=True, q_mode=Q_FP8_DYNAMIC, q_scale_padded=True,
                max_seqlen=4096, upper_max=448.0, k_scale=0.05, v_scale=0.05, maxp=64)
    args.update(kw)
    return nra_case(**args)


def sixteen_k_lengths(seed=1013, B=8, total=16384, hi=4096):
    """B request lengths in [1, hi] that sum to exactly `total`: a seeded
    random composition (B - 1 distinct cut points drawn uniformly from
    [1, total), redrawn until every part lies in [1, hi])."""
    rng = np.random.default_rng(seed)
    while True:
        cuts = np.sort(rng.choice(np.arange(1, total), size=B - 1, replace=False))
        lens = np.diff(np.concatenate([[0], cuts, [total]])).astype(np.int64)
        if lens.min() >= 1 and lens.max() <= hi:
            return lens


def c3_prefill_fp8_16k(seed=1013, **kw):
    """The ragged FP8 prefill at exactly 16 384 tokens: the C3 shapes and
    encodings with 8 request lengths in [1, 4096] summing to 16 384."""
    args = dict(name="c3_prefill_fp8_16k", seed=seed, q_lens=sixteen_k_lengths(seed))
    args.update(kw)
    return c3_prefill_fp8(**args)


def c4_strided_d256(seed=1004, **kw):
    """Strided head_dim 256: 4 requests x 2048 tokens, 16/4/256, rows padded
    by 64 bf16 elements, Gemma RMSNorm (1 + w), w ~ 0.1 N(0,1), theta 1e7,
    table [8192, 256], bf16 caches page 32, Q and K written back in place."""
    rng = np.random.default_rng(seed)
    prior = rng.integers(0, 2048, size=4)
    args = dict(name="c4_strided_d256", seed=seed + 7, q_lens=np.full(4, 2048, np.int64), prior_lens=prior,
                Hq=16, Hkv=4, D=256, page_size=32, row_pad=64, norm=NORM_GEMMA, theta=1e7,
                cs_rows=8192, q_in_place=True, k_in_place=True, maxp=128)
    args.update(kw)
    return nra_case(**args)


def c5_mla(seed=1005, **kw):
    """DeepSeek-like MLA: T = 4096, q [T, 128, 192] with interleaved RoPE on
    the last 64 dims, kv_c [T, 512], k_pe [T, 64], theta 1e4, positions
    U[0, 16384), FP8 E4M3 cache [128, 64, 576], scale 0.02, distinct slots."""
    args = dict(name="c5_mla", seed=seed, T=4096)
    args.update(kw)
    return mla_case(**args)


CONFIGS = {
    "c1": c1_tiny_decode,
    "c2": c2_decode_b256,
    "c3": c3_prefill_fp8,
    "c4": c4_strided_d256,
    "c5": c5_mla,
}


# ----------------------------------------------------------------------------
# the rows the FlashInfer PR (fused QK RMSNorm + NeoX RoPE + FP8 E4M3 quantize
# + NHD paged-KV append) measures in its Performance section
# ----------------------------------------------------------------------------

# name -> (kind, requests, tokens per request, (Hq, Hkv), Q policy, page size,
#          printed bytes in MB).  Every row has D = 128, bf16 qkv, E4M3 Q and
# E4M3 caches, norm policy 2; Q policy 1 is the dynamic per-token-head scale.
PAGES_ROWS = {
    "P_decode_64x8_q1_n2": ("decode", 32, 1, (64, 8), 1, 64, 5.136),
    "P_prefill_64x8_q1_n2": ("prefill", 8, 16, (64, 8), 1, 64, 4.817),
    "P_decode_8x1_q1_n2": ("decode", 32, 1, (8, 1), 1, 64, 0.656),
    "E_prefill_64x8_q128": ("prefill", 4, 128, (64, 8), 1, 64, 16.122),
    "X_decode_64x8_B1_q1_n2": ("decode", 1, 1, (64, 8), 1, 64, 0.161),
    "X_decode_64x8_B128_q1_n2": ("decode", 128, 1, (64, 8), 1, 64, 20.546),
    "X_decode_64x8_B256_q1_n2": ("decode", 256, 1, (64, 8), 1, 64, 41.091),
    "X_decode_8x1_B256_q1_n2": ("decode", 256, 1, (8, 1), 1, 64, 5.251),
    "X_prefill_64x8_B1_Q1024_q1_n2": ("prefill", 1, 1024, (64, 8), 1, 64, 32.244),
    "X_prefill_8x1_B1_Q1024_q1_n2": ("prefill", 1, 1024, (8, 1), 1, 64, 4.489),
}


def pages_row(name, seed=2001, prior_pages=64, **kw):
    """One of the FlashInfer PR's measured rows, rebuilt from its name.

    Decode rows: each request appends one token after a prior length that is
    a multiple of the page size (U[0, prior_pages) pages), so the token lands in row 0
    of a fresh page and the rest of that page is tail; Q scales token-major
    [T, Hq].  Prefill rows: fresh requests (prior 0) of equal length, Q
    scales in the padded [B, Hq, round_up(q_len, 128)] layout with
    max_seqlen = q_len.  qkv ~ N(0, 1); norm policy 2 read as the (1 + w)
    weighting; k_scale = v_scale = 0.05; upper_max 448; theta 1e6, table
    [8192, 128].  The byte model of these rows (qkv read, E4M3 Q and its
    scales, cos/sin rows, K/V append, tail rows; no norm weights) then gives
    the printed megabytes."""
    kind, B, q, (hq, hkv), qpol, ps, _ = PAGES_ROWS[name]
    rng = np.random.default_rng(seed)
    if kind == "decode":
        prior = ps * rng.integers(0, prior_pages, size=B)
    else:
        prior = np.zeros(B, np.int64)
    args = dict(name=name, seed=seed + 7, q_lens=np.full(B, q, np.int64), prior_lens=prior,
                Hq=hq, Hkv=hkv, D=128, page_size=ps, norm=NORM_GEMMA, theta=1e6, cs_rows=8192,
                kv_fp8=True, q_mode=Q_FP8_DYNAMIC if qpol == 1 else Q_FP8_STATIC,
                q_scale_padded=kind == "prefill", max_seqlen=q if kind == "prefill" else 0,
                upper_max=448.0, q_scale_inv=2.0, k_scale=0.05, v_scale=0.05)
    args.update(kw)
    return nra_case(**args)
