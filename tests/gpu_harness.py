"""GPU-side test plumbing: upload seeded inputs with guard bytes, call the
C ABI through the binding, download outputs, and compare them with the
oracle under the stated tolerances.

Tolerances (GPU vs oracle):
- bit-exact: flags, placement, tail zeros, every byte the call must not
  write, bf16 V copies, the V columns and row padding of an in-place qkv;
- bf16 Q / K / MLA q_rope / k_pe: <= 2 bf16 ulp on the monotone ordinal
  line (+0 and -0 equal); where the oracle's value is below 2^-8 in
  magnitude, an absolute difference <= 2^-16 is also accepted (fp32
  cancellation in a*c - b*s leaves ~2^-20 absolute error while the bf16
  ulp vanishes near zero; at 2^-8 and above that error is under 1/16 ulp);
- E4M3 payloads: <= 1 code on the monotone ordinal line;
- q_scale: relative 1e-5.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import paged_kv_cache_token_amd as qp
import workloads as W

GUARD = 256
GUARD_BYTE = 0xA5

DEV = "cuda"


# ----------------------------------------------------------------------------
# guarded device buffers
# ----------------------------------------------------------------------------

class Guarded:
    """A device tensor with GUARD bytes of a known pattern on both sides."""

    def __init__(self, nbytes: int, dtype: torch.dtype, shape, init: np.ndarray | None = None,
                 fill_seed: int | None = None):
        self.nbytes = nbytes
        self.raw = torch.full((nbytes + 2 * GUARD,), GUARD_BYTE, dtype=torch.uint8, device=DEV)
        body = self.raw[GUARD:GUARD + nbytes]
        if init is not None:
            body.copy_(torch.from_numpy(np.ascontiguousarray(init).view(np.uint8).reshape(-1)).to(DEV))
        elif fill_seed is not None:
            g = torch.Generator(device=DEV)
            g.manual_seed(fill_seed)
            body.random_(0, 256, generator=g)
        self.t = body.view(dtype).view(shape)

    def guards_intact(self) -> bool:
        head = self.raw[:GUARD]
        tail = self.raw[GUARD + self.nbytes:]
        return bool((head == GUARD_BYTE).all().item() and (tail == GUARD_BYTE).all().item())


def _np_to_dev(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).view(dtype)


def _scalar(x: float) -> torch.Tensor:
    return torch.tensor([x], dtype=torch.float32, device=DEV)


# ----------------------------------------------------------------------------
# norm-rope-append
# ----------------------------------------------------------------------------

class DeviceNra:
    """Device copies of one call's inputs and guarded outputs."""

    def __init__(self, inp: W.NraInputs):
        self.inp = inp
        D, T = inp.D, inp.T
        self.qkv = Guarded(inp.qkv.nbytes, torch.int16, inp.qkv.shape, init=inp.qkv)
        self.q_w = _np_to_dev(inp.q_norm_weight, torch.float32)
        self.k_w = _np_to_dev(inp.k_norm_weight, torch.float32)
        self.cos_sin = _np_to_dev(inp.cos_sin, torch.float32)
        self.positions = _np_to_dev(inp.positions, torch.int64)
        if inp.addressing == W.ADDR_PAGED:
            self.q_indptr = _np_to_dev(inp.q_indptr, torch.int32)
            self.seq_lens = _np_to_dev(inp.seq_lens, torch.int32)
            self.page_table = _np_to_dev(inp.page_table, torch.int32)
            self.slot_mapping = None
        else:
            self.q_indptr = self.seq_lens = self.page_table = None
            self.slot_mapping = _np_to_dev(inp.slot_mapping, torch.int64)
        cdt = torch.uint8 if inp.kv_fp8 else torch.int16
        cbytes = int(np.prod(inp.cache_shape)) * inp.kv_elt
        if inp.k_cache0 is not None:
            self.k_cache = Guarded(cbytes, cdt, inp.cache_shape, init=inp.k_cache0)
            self.v_cache = Guarded(cbytes, cdt, inp.cache_shape, init=inp.v_cache0)
        else:
            self.k_cache = Guarded(cbytes, cdt, inp.cache_shape, fill_seed=inp.cache_seed)
            self.v_cache = Guarded(cbytes, cdt, inp.cache_shape, fill_seed=inp.cache_seed + 1)
        if inp.q_in_place:
            self.q_out = None
        else:
            qdt = torch.int16 if inp.q_mode == W.Q_BF16 else torch.uint8
            self.q_out = Guarded(inp.q_out0.nbytes, qdt, inp.q_out0.shape, init=inp.q_out0)
        self.q_scale = None
        if inp.q_scale0 is not None:
            self.q_scale = Guarded(inp.q_scale0.nbytes, torch.float32, inp.q_scale0.shape, init=inp.q_scale0)
        self.flags = None
        if inp.flags0 is not None and inp.flags0.size:
            self.flags = Guarded(inp.flags0.nbytes, torch.int32, inp.flags0.shape, init=inp.flags0)
        self.k_scale = _scalar(inp.k_scale)
        self.v_scale = _scalar(inp.v_scale)
        self.q_scale_inv = _scalar(inp.q_scale_inv)
        self.out_k = self.out_v = self.k_scale_out = self.v_scale_out = None
        if inp.kv_redirect:
            self.out_k = Guarded(inp.out_k0.nbytes, cdt, inp.out_k0.shape, init=inp.out_k0)
            self.out_v = Guarded(inp.out_v0.nbytes, cdt, inp.out_v0.shape, init=inp.out_v0)
        if inp.kv_scale_mode:
            sh = inp.k_scale_out0.shape
            self.k_scale_out = Guarded(inp.k_scale_out0.nbytes, torch.float32, sh, init=inp.k_scale_out0)
            self.v_scale_out = Guarded(inp.v_scale_out0.nbytes, torch.float32, sh, init=inp.v_scale_out0)

    def kwargs(self) -> dict:
        inp = self.inp
        D, Hq, Hkv = inp.D, inp.Hq, inp.Hkv
        qkv = self.qkv.t
        if inp.q_in_place:
            q_out, q_stride = qkv, inp.qkv_row_stride
        else:
            q_out, q_stride = self.q_out.t, Hq * D
        k_out = None
        if inp.k_in_place:
            k_out = qkv.view(-1)[Hq * D:].as_strided((inp.T, Hkv * D), (inp.qkv_row_stride, 1))
        return dict(
            qkv=qkv, num_tokens=inp.T, qkv_row_stride=inp.qkv_row_stride, num_q_heads=Hq,
            num_kv_heads=Hkv, head_dim=D, norm=inp.norm, eps=inp.eps, q_norm_weight=self.q_w,
            k_norm_weight=self.k_w, rope=inp.rope, cos_sin_cache=self.cos_sin, positions=self.positions,
            addressing=inp.addressing, q_indptr=self.q_indptr, seq_lens=self.seq_lens,
            page_table=self.page_table, num_requests=inp.B if inp.addressing == W.ADDR_PAGED else 0,
            slot_mapping=self.slot_mapping, k_cache=self.k_cache.t, v_cache=self.v_cache.t,
            kv_dtype=qp.FP8_E4M3 if inp.kv_fp8 else qp.BF16, k_scale=self.k_scale, v_scale=self.v_scale,
            zero_tail=1 if inp.zero_tail else 0, q_out=q_out, q_out_row_stride=q_stride,
            q_mode=inp.q_mode, q_scale=None if self.q_scale is None else self.q_scale.t,
            q_scale_layout=qp.QSCALE_REQ_HEAD_PADDED if inp.q_scale_padded else qp.QSCALE_TOKEN_HEAD,
            max_seqlen=inp.max_seqlen, q_scale_inv=self.q_scale_inv, upper_max=inp.upper_max,
            k_out=k_out, k_out_row_stride=inp.qkv_row_stride,
            flags=None if self.flags is None else self.flags.t, rotary_dim=inp.rot,
            out_k=None if self.out_k is None else self.out_k.t,
            out_v=None if self.out_v is None else self.out_v.t,
            kv_scale_mode=inp.kv_scale_mode, kv_group_size=inp.kv_group_size,
            k_scale_out=None if self.k_scale_out is None else self.k_scale_out.t,
            v_scale_out=None if self.v_scale_out is None else self.v_scale_out.t,
            store_policy=inp.store_policy,
        )

    def run(self, stream=None):
        qp.qkprep_norm_rope_append(stream=stream, **self.kwargs())

    def guards_intact(self) -> bool:
        bufs = [self.qkv, self.k_cache, self.v_cache, self.q_out, self.q_scale, self.flags, self.out_k,
                self.out_v, self.k_scale_out, self.v_scale_out]
        return all(b.guards_intact() for b in bufs if b is not None)

    def host_outputs(self, pages: np.ndarray | None = None) -> dict:
        """Outputs as numpy; caches restricted to `pages` when given."""
        inp = self.inp
        cdt = np.uint8 if inp.kv_fp8 else np.uint16

        def cache(g):
            t = g.t if pages is None else g.t[torch.from_numpy(pages).to(DEV)]
            return t.cpu().numpy().view(cdt)

        out = {
            "qkv": self.qkv.t.cpu().numpy().view(np.uint16),
            "k_cache": cache(self.k_cache),
            "v_cache": cache(self.v_cache),
            "q_out": None if self.q_out is None else
            self.q_out.t.cpu().numpy().view(np.uint16 if inp.q_mode == W.Q_BF16 else np.uint8),
            "q_scale": None if self.q_scale is None else self.q_scale.t.cpu().numpy(),
            "flags": None if self.flags is None else self.flags.t.cpu().numpy(),
        }
        for name in ("out_k", "out_v"):
            g = getattr(self, name)
            out[name] = None if g is None else g.t.cpu().numpy().view(cdt)
        for name in ("k_scale_out", "v_scale_out"):
            g = getattr(self, name)
            out[name] = None if g is None else g.t.cpu().numpy()
        return out


def oracle_outputs(inp: W.NraInputs) -> dict:
    out = {
        "qkv": inp.qkv.copy(),
        "k_cache": inp.k_cache0.copy(),
        "v_cache": inp.v_cache0.copy(),
        "q_out": None if inp.q_in_place else inp.q_out0.copy(),
        "q_scale": None if inp.q_scale0 is None else inp.q_scale0.copy(),
        "flags": None if inp.flags0 is None else inp.flags0.copy(),
    }
    for name in ("out_k0", "out_v0", "k_scale_out0", "v_scale_out0"):
        a = getattr(inp, name)
        out[name[:-1]] = None if a is None else a.copy()
    oracle.norm_rope_append(inp, out)
    return out


def compact_inputs(inp: W.NraInputs, k_before: np.ndarray, v_before: np.ndarray, pages: np.ndarray):
    """The same call on a pool that holds only `pages` (relabelled 0..n-1);
    the prepare pass is equivariant under page relabelling."""
    import copy
    c = copy.copy(inp)
    remap = np.full(inp.num_pages, -1, np.int64)
    remap[pages] = np.arange(len(pages))
    if inp.addressing == W.ADDR_PAGED:
        pt = inp.page_table.astype(np.int64)
        c.page_table = np.where(pt >= 0, remap[np.clip(pt, 0, None)], -1).astype(np.int32)
    else:
        s = inp.slot_mapping
        ok = (s >= 0) & (s < inp.num_pages * inp.page_size)
        c.slot_mapping = np.where(ok, remap[np.clip(s // inp.page_size, 0, inp.num_pages - 1)] * inp.page_size
                                  + s % inp.page_size, -1).astype(np.int64)
    c.num_pages = len(pages)
    c.k_cache0, c.v_cache0 = k_before, v_before
    return c


# ----------------------------------------------------------------------------
# comparisons
# ----------------------------------------------------------------------------

def bf16_ord(b: np.ndarray) -> np.ndarray:
    b = b.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def e4m3_ord(c: np.ndarray) -> np.ndarray:
    c = c.astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def check_bf16(got: np.ndarray, ref: np.ndarray, what: str, stats: dict):
    got = got.view(np.uint16)
    ref = ref.view(np.uint16)
    d = np.abs(bf16_ord(got) - bf16_ord(ref))
    vg = W.bf16_bits_to_f32(got).astype(np.float64)
    vr = W.bf16_bits_to_f32(ref).astype(np.float64)
    bad = (d > 2) & ~((np.abs(vr) < 2.0 ** -8) & (np.abs(vg - vr) <= 2.0 ** -16))
    stats[what] = {"n": int(got.size), "exact": float((d == 0).mean()) if got.size else 1.0,
                   "max_ulp": int(d.max()) if got.size else 0}
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} bf16 values beyond 2 ulp; first at {tuple(i)}: "
                             f"gpu {vg[tuple(i)]!r} oracle {vr[tuple(i)]!r}")


# Shares of values equal to the oracle's that full-size runs must reach: the
# tolerances above admit a systematic in-tolerance drift (an eps or rsqrt
# error, a cos/sin row off by one on near-zero outputs); these floors do not.
EXACT_FLOOR_BF16 = 0.999
EXACT_FLOOR_E4M3 = 0.99


def assert_exact_floors(stats: dict):
    """Every bf16 / E4M3 comparison in `stats` reached its exact-match floor."""
    for what, st in stats.items():
        if "max_ulp" in st and st["n"]:
            assert st["exact"] >= EXACT_FLOOR_BF16, f"{what}: exact {st['exact']:.6f} < {EXACT_FLOOR_BF16}"
        if "max_code" in st and st["n"]:
            assert st["exact"] >= EXACT_FLOOR_E4M3, f"{what}: exact {st['exact']:.6f} < {EXACT_FLOOR_E4M3}"


def check_e4m3(got: np.ndarray, ref: np.ndarray, what: str, stats: dict):
    got = got.view(np.uint8)
    ref = ref.view(np.uint8)
    assert not ((got & 0x7F) == 0x7F).any(), f"{what}: NaN code from the GPU"
    d = np.abs(e4m3_ord(got) - e4m3_ord(ref))
    stats[what] = {"n": int(got.size), "exact": float((d == 0).mean()) if got.size else 1.0,
                   "max_code": int(d.max()) if got.size else 0}
    if (d > 1).any():
        i = np.argwhere(d > 1)[0]
        raise AssertionError(f"{what}: {int((d > 1).sum())} E4M3 codes off by >1; first at {tuple(i)}: "
                             f"gpu {got[tuple(i)]:#x} oracle {ref[tuple(i)]:#x}")


def check_exact(got: np.ndarray, ref: np.ndarray, what: str):
    g = np.ascontiguousarray(got).view(np.uint8)
    r = np.ascontiguousarray(ref).view(np.uint8)
    if not np.array_equal(g, r):
        n = int((g != r).sum())
        i = int(np.argmax(g != r))
        raise AssertionError(f"{what}: {n} bytes differ (first at byte {i})")


def written_cells(inp: W.NraInputs, pages_index=None):
    """(token, page, row) of every token the call appends (valid position and
    slot); page numbers relabelled through `pages_index` when given."""
    out = []
    if inp.kv_redirect:
        return out
    rows = inp.cos_sin.shape[0]
    for t in range(inp.T):
        pos = int(inp.positions[t])
        if inp.rot > 0 and (pos < 0 or pos >= rows):
            continue
        if inp.addressing == W.ADDR_PAGED:
            b = int(np.searchsorted(inp.q_indptr, t, side="right") - 1)
            ql = int(inp.q_indptr[b + 1] - inp.q_indptr[b])
            L = int(inp.seq_lens[b]) - ql + (t - int(inp.q_indptr[b]))
            p = int(inp.page_table[b, L // inp.page_size])
            r = L % inp.page_size
        else:
            s = int(inp.slot_mapping[t])
            if s < 0 or s >= inp.num_pages * inp.page_size:
                continue
            p, r = divmod(s, inp.page_size)
        out.append((t, p, r))
    return out


def compare_nra(inp: W.NraInputs, gpu: dict, ref: dict) -> dict:
    """Compare every output under the tolerances of the module docstring."""
    stats = {}
    D, Hq, Hkv = inp.D, inp.Hq, inp.Hkv
    if ref["flags"] is not None:
        check_exact(gpu["flags"], ref["flags"], "flags")
    invalid = ref["flags"] is not None and ref["flags"].size and (ref["flags"] == -1).all()
    rows = inp.cos_sin.shape[0]
    live = np.array([inp.rot == 0 or 0 <= int(p) < rows for p in inp.positions], bool) if inp.T \
        else np.zeros(0, bool)
    if invalid:
        live[:] = False
    # caches: token rows with tolerance, every other byte exact
    kg, kr = gpu["k_cache"].copy(), ref["k_cache"].copy()
    vg, vr = gpu["v_cache"].copy(), ref["v_cache"].copy()
    cells = [] if invalid else written_cells(inp)
    if cells:
        ps = np.array([c[1] for c in cells])
        rs = np.array([c[2] for c in cells])
        if inp.kv_fp8:
            check_e4m3(kg[ps, rs], kr[ps, rs], "k_cache rows", stats)
            check_e4m3(vg[ps, rs], vr[ps, rs], "v_cache rows", stats)
        else:
            check_bf16(kg[ps, rs], kr[ps, rs], "k_cache rows", stats)
            check_exact(vg[ps, rs], vr[ps, rs], "v_cache rows (bf16 copy)")
        kg[ps, rs] = 0
        kr[ps, rs] = 0
        vg[ps, rs] = 0
        vr[ps, rs] = 0
    check_exact(kg, kr, "k_cache outside appended rows")
    check_exact(vg, vr, "v_cache outside appended rows")
    # Q
    if inp.q_in_place:
        qg = gpu["qkv"][:, :Hq * D].reshape(inp.T, Hq, D)
        qr = ref["qkv"][:, :Hq * D].reshape(inp.T, Hq, D)
    else:
        qg, qr = gpu["q_out"], ref["q_out"]
    if live.any():
        if inp.q_mode == W.Q_BF16:
            check_bf16(qg[live], qr[live], "q", stats)
        else:
            check_e4m3(qg[live], qr[live], "q", stats)
    check_exact(qg[~live], qr[~live], "q rows not written")
    # qkv: K columns (in place) with tolerance, everything else exact
    gq, rq = gpu["qkv"].copy(), ref["qkv"].copy()
    if inp.q_in_place:
        gq[:, :Hq * D] = 0
        rq[:, :Hq * D] = 0
    if inp.k_in_place:
        ks = slice(Hq * D, (Hq + Hkv) * D)
        if live.any():
            check_bf16(gq[live][:, ks], rq[live][:, ks], "k written back", stats)
        gq[live, ks] = 0
        rq[live, ks] = 0
    check_exact(gq, rq, "qkv (V, padding and unwritten columns)")
    # q_scale
    if ref["q_scale"] is not None:
        check_scales(gpu["q_scale"], ref["q_scale"], inp.q_scale0, "q_scale", stats)
    # redirected K/V rows
    if inp.kv_redirect:
        for name in ("out_k", "out_v"):
            g, r = gpu[name], ref[name]
            if live.any():
                if inp.kv_fp8:
                    check_e4m3(g[live], r[live], name, stats)
                elif name == "out_k":
                    check_bf16(g[live], r[live], name, stats)
                else:
                    check_exact(g[live], r[live], "out_v (bf16 copy)")
            check_exact(g[~live], r[~live], f"{name} rows not written")
    if inp.kv_scale_mode:
        check_scales(gpu["k_scale_out"], ref["k_scale_out"], inp.k_scale_out0, "k_scale_out", stats)
        check_scales(gpu["v_scale_out"], ref["v_scale_out"], inp.v_scale_out0, "v_scale_out", stats)
    return stats


def check_scales(got: np.ndarray, ref: np.ndarray, before: np.ndarray, what: str, stats: dict):
    """fp32 scales: entries the oracle wrote within relative 1e-5 (zeros of
    cleared rows exactly), every other entry byte-identical."""
    g, r, b = got.reshape(-1), ref.reshape(-1), before.reshape(-1)
    written = r.view(np.uint32) != b.view(np.uint32)
    nz = written & (r != 0)
    if nz.any():
        rel = np.abs(g[nz].astype(np.float64) - r[nz]) / np.abs(r[nz].astype(np.float64))
        stats[what] = {"n": int(nz.sum()), "max_rel": float(rel.max())}
        assert rel.max() <= 1e-5, f"{what} relative error {rel.max()}"
    check_exact(g[~nz], r[~nz], f"{what} entries not written or zeroed")


# ----------------------------------------------------------------------------
# MLA
# ----------------------------------------------------------------------------

class DeviceMla:
    def __init__(self, inp: W.MlaInputs):
        self.inp = inp
        self.q = Guarded(inp.q.nbytes, torch.int16, inp.q.shape, init=inp.q)
        self.kv_c = _np_to_dev(inp.kv_c, torch.int16)
        self.k_pe = Guarded(inp.k_pe.nbytes, torch.int16, inp.k_pe.shape, init=inp.k_pe)
        self.cos_sin = _np_to_dev(inp.cos_sin, torch.float32)
        self.positions = _np_to_dev(inp.positions, torch.int64)
        self.slots = _np_to_dev(inp.slot_mapping, torch.int64)
        cdt = torch.uint8 if inp.kv_fp8 else torch.int16
        self.cache = Guarded(inp.kv_cache0.nbytes, cdt, inp.kv_cache0.shape, init=inp.kv_cache0)
        self.kv_scale = _scalar(inp.kv_scale)
        self.q_out = self.q_scale = None
        if inp.q_out0 is not None:
            self.q_out = Guarded(inp.q_out0.nbytes, torch.uint8, inp.q_out0.shape, init=inp.q_out0)
        if inp.q_scale0 is not None:
            self.q_scale = Guarded(inp.q_scale0.nbytes, torch.float32, inp.q_scale0.shape, init=inp.q_scale0)
        self.q_scale_inv = _scalar(inp.q_scale_inv)

    def kwargs(self) -> dict:
        inp = self.inp
        return dict(
            q=self.q.t, kv_c=self.kv_c, k_pe=self.k_pe.t, cos_sin_cache=self.cos_sin,
            positions=self.positions, slot_mapping=self.slots, kv_cache=self.cache.t, num_q_heads=inp.H,
            nope_dim=inp.nope_dim, rope_dim=inp.rope_dim, kv_lora_rank=inp.kv_lora_rank, rope=inp.rope,
            kv_dtype=qp.FP8_E4M3 if inp.kv_fp8 else qp.BF16, kv_scale=self.kv_scale, q_mode=inp.q_mode,
            q_out=None if self.q_out is None else self.q_out.t,
            q_scale=None if self.q_scale is None else self.q_scale.t, q_scale_inv=self.q_scale_inv,
            upper_max=inp.upper_max, store_policy=inp.store_policy)

    def run(self, stream=None):
        qp.qkprep_mla_concat_rope_append(stream=stream, **self.kwargs())

    def guards_intact(self):
        bufs = [self.q, self.cache, self.k_pe, self.q_out, self.q_scale]
        return all(b.guards_intact() for b in bufs if b is not None)

    def host_outputs(self):
        cdt = np.uint8 if self.inp.kv_fp8 else np.uint16
        out = {"q": self.q.t.cpu().numpy().view(np.uint16), "kv_cache": self.cache.t.cpu().numpy().view(cdt),
               "k_pe": self.k_pe.t.cpu().numpy().view(np.uint16)}
        if self.q_out is not None:
            out["q_out"] = self.q_out.t.cpu().numpy().view(np.uint8)
        if self.q_scale is not None:
            out["q_scale"] = self.q_scale.t.cpu().numpy().view(np.float32)
        return out


def oracle_mla(inp: W.MlaInputs) -> dict:
    out = {"q": inp.q.copy(), "kv_cache": inp.kv_cache0.copy(),
           "q_out": None if inp.q_out0 is None else inp.q_out0.copy(),
           "q_scale": None if inp.q_scale0 is None else inp.q_scale0.copy()}
    oracle.mla_concat_rope_append(inp, out)
    return out


def compare_mla(inp: W.MlaInputs, gpu: dict, ref: dict) -> dict:
    stats = {}
    nope, R, K = inp.nope_dim, inp.rope_dim, inp.kv_lora_rank
    rows = inp.cos_sin.shape[0]
    live = (inp.positions >= 0) & (inp.positions < rows)
    check_exact(gpu["k_pe"], inp.k_pe, "k_pe (read only)")
    if inp.q_mode == W.Q_BF16:
        check_exact(gpu["q"][:, :, :nope], ref["q"][:, :, :nope], "q_nope")
        if live.any():
            check_bf16(gpu["q"][live][:, :, nope:nope + R], ref["q"][live][:, :, nope:nope + R], "q_rope", stats)
        check_exact(gpu["q"][~live], ref["q"][~live], "q of suppressed tokens")
    else:
        check_exact(gpu["q"], inp.q, "q (read only in the FP8 Q modes)")
        if live.any():
            check_e4m3(gpu["q_out"][live], ref["q_out"][live], "q_out codes", stats)
        check_exact(gpu["q_out"][~live], ref["q_out"][~live], "q_out of suppressed tokens")
        if inp.q_mode == W.Q_FP8_DYNAMIC:
            sg, sr = gpu["q_scale"], ref["q_scale"]
            if live.any():
                rel = np.abs(sg[live].astype(np.float64) - sr[live]) / np.abs(sr[live].astype(np.float64))
                stats["q_scale"] = {"n": int(live.sum()), "max_rel": float(rel.max())}
                assert rel.max() <= 1e-5, f"q_scale relative error {rel.max()}"
            check_exact(sg[~live], sr[~live], "q_scale of suppressed tokens")
    cap = inp.num_blocks * inp.block_size
    s = inp.slot_mapping
    ok = live & (s >= 0) & (s < cap)
    cg = gpu["kv_cache"].reshape(cap, K + R).copy()
    cr = ref["kv_cache"].reshape(cap, K + R).copy()
    idx = s[ok]
    if idx.size:
        if inp.kv_fp8:
            check_e4m3(cg[idx], cr[idx], "latent cache rows", stats)
        else:
            check_exact(cg[idx][:, :K], cr[idx][:, :K], "latent kv_c (bf16 copy)")
            check_bf16(cg[idx][:, K:], cr[idx][:, K:], "latent rope part", stats)
        cg[idx] = 0
        cr[idx] = 0
    check_exact(cg, cr, "latent cache outside written rows")
    return stats
