"""End-to-end pins of the oracle's fused pass on tiny inputs.

- placement: a hand-worked fixture (tests/golden/placement_example.json) and
  an independent brute-force enumeration over every cache cell;
- validation: hand-built malformed metadata -> all flags -1, no byte written;
- quantisation: FP8 payloads decode back to the fp32 value within half an
  E4M3 step; the head maximum encodes to upper_max; q_scale layouts;
- slot addressing and the MLA concat.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _copy(a):
    return None if a is None else a.copy()


def run_oracle(inp: W.NraInputs):
    out = {
        "qkv": inp.qkv.copy(),
        "k_cache": inp.k_cache0.copy(),
        "v_cache": inp.v_cache0.copy(),
        "q_out": None if inp.q_in_place else inp.q_out0.copy(),
        "q_scale": _copy(inp.q_scale0),
        "flags": _copy(inp.flags0),
        "out_k": _copy(inp.out_k0),
        "out_v": _copy(inp.out_v0),
        "k_scale_out": _copy(inp.k_scale_out0),
        "v_scale_out": _copy(inp.v_scale_out0),
    }
    oracle.norm_rope_append(inp, out)
    return out


def _small(**kw):
    args = dict(seed=5, q_lens=[3, 2, 0, 0], prior_lens=[3, 0, 4, 5], Hq=2, Hkv=1, D=128, page_size=4)
    args.update(kw)
    return W.nra_case(**args)


# ----------------------------------------------------------------------------
# placement
# ----------------------------------------------------------------------------

def test_placement_matches_hand_worked_fixture():
    g = json.load(open(os.path.join(GOLDEN, "placement_example.json")))
    inp = _small(norm=W.NORM_NONE)
    inp.page_table = np.array(g["page_table"], np.int32)
    inp.num_pages = g["num_pages"]
    shape = (g["num_pages"], g["page_size"], g["Hkv"], g["D"])
    rng = np.random.default_rng(0)
    inp.k_cache0 = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    inp.v_cache0 = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    assert inp.q_indptr.tolist() == g["q_indptr"] and inp.seq_lens.tolist() == g["seq_lens"]
    assert inp.positions.tolist() == g["expected_positions"]
    # the contract's derived position r + seq_lens[b] - q_indptr[b+1]
    derived = []
    for b in range(inp.B):
        for r in range(inp.q_indptr[b], inp.q_indptr[b + 1]):
            derived.append(r + inp.seq_lens[b] - inp.q_indptr[b + 1])
    assert derived == g["expected_positions"]
    out = run_oracle(inp)
    Hq, Hkv, D = inp.Hq, inp.Hkv, inp.D
    for t, (p, r) in enumerate(g["expected_token_cells"]):
        vrow = inp.qkv[t, (Hq + Hkv) * D:(Hq + 2 * Hkv) * D]
        assert np.array_equal(out["v_cache"][p, r].ravel(), vrow)
    for p, r in g["expected_tail_cells"]:
        assert not out["k_cache"][p, r].any() and not out["v_cache"][p, r].any()
    written = {tuple(c) for c in g["expected_token_cells"]} | {tuple(c) for c in g["expected_tail_cells"]}
    for p in range(g["num_pages"]):
        for r in range(g["page_size"]):
            if (p, r) not in written:
                assert np.array_equal(out["k_cache"][p, r], inp.k_cache0[p, r])
                assert np.array_equal(out["v_cache"][p, r], inp.v_cache0[p, r])
    assert out["flags"].ravel().tolist() == g["expected_flags"]


def _brute_force_owner(inp: W.NraInputs):
    """For every cache cell: which (request, logical row) owns it -- found by
    scanning each request's page list, not by the forward formula."""
    owner = {}
    for b in range(inp.B):
        sl = int(inp.seq_lens[b])
        npages = -(-sl // inp.page_size)
        for k in range(npages):
            p = int(inp.page_table[b, k])
            for r in range(inp.page_size):
                owner[(p, r)] = (b, k * inp.page_size + r)
    return owner


@pytest.mark.parametrize("seed,ps,zero_tail", [(1, 4, True), (2, 16, True), (3, 8, False), (4, 1, True)])
def test_placement_brute_force(seed, ps, zero_tail):
    rng = np.random.default_rng(seed)
    B = 7
    q_lens = rng.integers(0, 9, size=B)
    q_lens[2] = 0
    prior = rng.integers(0, 30, size=B)
    inp = W.nra_case(seed=seed, q_lens=q_lens, prior_lens=prior, Hq=2, Hkv=2, D=128, page_size=ps,
                     norm=W.NORM_RMS, zero_tail=zero_tail)
    out = run_oracle(inp)
    assert (out["flags"] == 0).all()
    owner = _brute_force_owner(inp)
    Hq, Hkv, D = inp.Hq, inp.Hkv, inp.D
    n_tok = n_tail = 0
    for p in range(inp.num_pages):
        for r in range(ps):
            before_k, before_v = inp.k_cache0[p, r], inp.v_cache0[p, r]
            after_k, after_v = out["k_cache"][p, r], out["v_cache"][p, r]
            if (p, r) not in owner:
                assert np.array_equal(after_k, before_k) and np.array_equal(after_v, before_v)
                continue
            b, L = owner[(p, r)]
            sl = int(inp.seq_lens[b])
            ql = int(q_lens[b])
            if sl - ql <= L < sl:
                t = int(inp.q_indptr[b]) + L - (sl - ql)
                vrow = inp.qkv[t, (Hq + Hkv) * D:(Hq + 2 * Hkv) * D]
                assert np.array_equal(after_v.ravel(), vrow)
                assert not np.array_equal(after_k, before_k)
                n_tok += 1
            elif L >= sl and zero_tail and sl > 0 and L // ps == (sl - 1) // ps:
                assert not after_k.any() and not after_v.any()
                n_tail += 1
            else:
                assert np.array_equal(after_k, before_k) and np.array_equal(after_v, before_v)
    assert n_tok == inp.T
    if zero_tail and ps > 1:
        assert n_tail > 0


# ----------------------------------------------------------------------------
# validation
# ----------------------------------------------------------------------------

def _mutations():
    return {
        "first_nonzero": lambda i: i.q_indptr.__setitem__(0, 1),
        "non_monotone": lambda i: i.q_indptr.__setitem__(2, i.q_indptr[1] - 1),
        "last_short": lambda i: i.q_indptr.__setitem__(-1, i.T - 1),
        "last_long": lambda i: i.q_indptr.__setitem__(-1, i.T + 1),
        "seq_len_below_q_len": lambda i: i.seq_lens.__setitem__(0, 2),
        "too_many_pages": lambda i: i.seq_lens.__setitem__(1, i.page_table.shape[1] * i.page_size + 1),
        "page_id_negative": lambda i: i.page_table.__setitem__((0, (int(i.seq_lens[0]) - 1) // i.page_size), -1),
        "page_id_past_pool": lambda i: i.page_table.__setitem__((1, 0), i.num_pages),
    }


@pytest.mark.parametrize("name", list(_mutations()))
def test_malformed_metadata_writes_only_minus_one_flags(name):
    inp = _small(q_mode=W.Q_FP8_DYNAMIC, q_scale_padded=True, max_seqlen=8, kv_fp8=True,
                 k_scale=0.05, v_scale=0.05)
    _mutations()[name](inp)
    out = run_oracle(inp)
    assert (out["flags"] == -1).all()
    assert np.array_equal(out["k_cache"], inp.k_cache0)
    assert np.array_equal(out["v_cache"], inp.v_cache0)
    assert np.array_equal(out["q_out"], inp.q_out0)
    assert np.array_equal(out["q_scale"].view(np.uint32), inp.q_scale0.view(np.uint32))
    assert np.array_equal(out["qkv"], inp.qkv)


def test_request_above_max_seqlen_is_invalid_only_for_padded_scales():
    inp = _small(q_mode=W.Q_FP8_DYNAMIC, q_scale_padded=True, max_seqlen=2, kv_fp8=True)
    out = run_oracle(inp)
    assert (out["flags"] == -1).all() and np.array_equal(out["q_out"], inp.q_out0)
    inp = _small(q_mode=W.Q_FP8_DYNAMIC, q_scale_padded=False, max_seqlen=2, kv_fp8=True)
    out = run_oracle(inp)
    assert (out["flags"] == 0).all()


def test_out_of_range_position_suppresses_only_that_token():
    inp = _small(norm=W.NORM_RMS)
    inp.positions = inp.positions.copy()
    inp.positions[1] = inp.cos_sin.shape[0]    # past the table
    inp.positions[3] = -1
    out = run_oracle(inp)
    assert (out["flags"] == 0).all()
    for t in range(inp.T):
        same = np.array_equal(out["q_out"][t], inp.q_out0[t])
        assert same == (t in (1, 3))


# ----------------------------------------------------------------------------
# quantisation
# ----------------------------------------------------------------------------

def _decode_e4m3(codes):
    lut = np.array([oracle.e4m3_to_f64(c) for c in range(256)])
    return lut[codes]


@pytest.mark.parametrize("upper_max", [448.0, 240.0])
def test_dynamic_q_scale_and_payloads(upper_max):
    inp = _small(q_mode=W.Q_FP8_DYNAMIC, q_scale_padded=False, upper_max=upper_max, kv_fp8=True,
                 k_scale=0.05, v_scale=0.05, qkv_sigma=2.0)
    out = run_oracle(inp)
    top = oracle.f64_to_e4m3(np.array([upper_max]))[0]
    q = out["q_out"]
    s = out["q_scale"]
    for t in range(inp.T):
        for h in range(inp.Hq):
            codes = q[t, h]
            mags = codes & 0x7F
            # the head maximum encodes to +-upper_max, nothing exceeds it
            assert mags.max() == top
            assert (mags <= top).all()
            # dequantised payload approximates the bf16-rounded result (norm +
            # rope only ever moves a value by < 1 bf16 ulp from its fp32 form)
            deq = _decode_e4m3(codes) * float(s[t, h])
            assert np.all(np.isfinite(deq))
    # the bf16 variant of the same call gives the rotated values; the FP8
    # payload must be the nearest E4M3 code of value / scale within one step
    inp_b = _small(q_mode=W.Q_BF16, qkv_sigma=2.0)
    outb = run_oracle(inp_b)
    vals = W.bf16_bits_to_f32(outb["q_out"]).astype(np.float64)
    for t in range(inp.T):
        for h in range(inp.Hq):
            amax = np.abs(vals[t, h]).max()
            assert abs(float(s[t, h]) - amax / upper_max) <= 1e-2 * amax / upper_max
            deq = _decode_e4m3(q[t, h]) * float(s[t, h])
            step = np.maximum(np.abs(vals[t, h]) / 8, 2**-9 * float(s[t, h]))
            assert np.all(np.abs(deq - vals[t, h]) <= step + 1e-2 * np.abs(vals[t, h]))


def test_padded_q_scale_layout_is_indexed_by_position_in_request():
    inp = _small(q_mode=W.Q_FP8_DYNAMIC, q_scale_padded=True, max_seqlen=129, kv_fp8=True,
                 k_scale=0.05, v_scale=0.05)
    out_p = run_oracle(inp)
    inp_t = _small(q_mode=W.Q_FP8_DYNAMIC, q_scale_padded=False, kv_fp8=True, k_scale=0.05, v_scale=0.05)
    out_t = run_oracle(inp_t)
    P = 256
    assert out_p["q_scale"].shape == (inp.B, inp.Hq, P)
    touched = np.zeros(out_p["q_scale"].shape, bool)
    for b in range(inp.B):
        for j in range(int(inp.q_indptr[b + 1] - inp.q_indptr[b])):
            t = int(inp.q_indptr[b]) + j
            assert np.array_equal(out_p["q_scale"][b, :, j], out_t["q_scale"][t])
            touched[b, :, j] = True
    # padding entries are never written
    assert np.array_equal(out_p["q_scale"][~touched].view(np.uint32), inp.q_scale0[~touched].view(np.uint32))
    assert np.array_equal(out_p["q_out"], out_t["q_out"])


def test_static_q_and_kv_scales():
    inp = _small(q_mode=W.Q_FP8_STATIC, q_scale_inv=4.0, kv_fp8=True, k_scale=0.25, v_scale=0.5,
                 norm=W.NORM_NONE)
    inp.positions = np.zeros(inp.T, np.int64)       # identity rotation
    out = run_oracle(inp)
    Hq, Hkv, D = inp.Hq, inp.Hkv, inp.D
    x = W.bf16_bits_to_f32(inp.qkv).astype(np.float64)
    # identity rotation + no norm: Q payload = E4M3(x * 4), V payload = E4M3(x / 0.5)
    assert np.array_equal(out["q_out"].reshape(inp.T, -1), oracle.f64_to_e4m3(x[:, :Hq * D] * 4.0))
    t = 0
    b = 0
    L = int(inp.seq_lens[b] - (inp.q_indptr[b + 1] - inp.q_indptr[b]))
    p = inp.page_table[b, L // inp.page_size]
    r = L % inp.page_size
    vx = x[t, (Hq + Hkv) * D:(Hq + 2 * Hkv) * D]
    kx = x[t, Hq * D:(Hq + Hkv) * D]
    assert np.array_equal(out["v_cache"][p, r].ravel(), oracle.f64_to_e4m3(vx / 0.5))
    assert np.array_equal(out["k_cache"][p, r].ravel(), oracle.f64_to_e4m3(kx / 0.25))


def test_bf16_identity_path_is_bit_exact_copy():
    inp = _small(q_mode=W.Q_BF16, norm=W.NORM_NONE)
    inp.positions = np.zeros(inp.T, np.int64)
    out = run_oracle(inp)
    Hq, D = inp.Hq, inp.D
    assert np.array_equal(out["q_out"].reshape(inp.T, -1), inp.qkv[:, :Hq * D])


def test_one_hot_head_reads_cos_then_sin_half_of_the_table_row():
    inp = _small(q_mode=W.Q_BF16, norm=W.NORM_NONE)
    qkv = np.zeros_like(inp.qkv)
    i = 9
    qkv[:, i] = 0x3F80            # 1.0 at dim i of Q head 0
    inp.qkv = qkv
    out = run_oracle(inp)
    for t in range(inp.T):
        pos = inp.positions[t]
        c, s = inp.cos_sin[pos, i], inp.cos_sin[pos, inp.D // 2 + i]
        got = W.bf16_bits_to_f32(out["q_out"][t, 0])
        assert got[i] == W.bf16_round(np.array([c]))[0]
        assert got[i + inp.D // 2] == W.bf16_round(np.array([s]))[0]


@pytest.mark.parametrize("R", [64, 32])
def test_partial_rotary_passes_the_nope_dims_through(R):
    """rotary_dim R < D: with no norm and bf16 outputs, dims [R, D) of every
    Q and K head are the input bits and dims [0, R) are the RoPE of the
    R-dim prefix with the table row of R floats."""
    inp = _small(q_mode=W.Q_BF16, norm=W.NORM_NONE, rotary_dim=R, kv_fp8=False)
    assert inp.cos_sin.shape[1] == R
    out = run_oracle(inp)
    Hq, D = inp.Hq, inp.D
    for t in range(inp.T):
        pos = inp.positions[t]
        c, s = inp.cos_sin[pos, :R // 2], inp.cos_sin[pos, R // 2:]
        for h in range(Hq):
            src = inp.qkv[t, h * D:(h + 1) * D]
            got = out["q_out"][t, h]
            assert np.array_equal(got[R:], src[R:])
            x = W.bf16_bits_to_f32(src).astype(np.float64)
            o = oracle.rope(x[:R], inp.rope, c, s)
            assert np.array_equal(got[:R], W.to_bf16_bits(o.astype(np.float32)))


def test_no_rotary_dims_copy_q_and_k_and_ignore_positions():
    """rotary_dim 0 (a NoPE layer): no norm + bf16 makes Q and the K cache
    rows bit copies of the input, and positions outside any table suppress
    nothing."""
    inp = _small(q_mode=W.Q_BF16, norm=W.NORM_NONE, rotary_dim=0, kv_fp8=False)
    inp.positions = np.full(inp.T, -7, np.int64)
    out = run_oracle(inp)
    Hq, Hkv, D = inp.Hq, inp.Hkv, inp.D
    assert np.array_equal(out["q_out"].reshape(inp.T, -1), inp.qkv[:, :Hq * D])
    kv_changed = ~np.all(out["k_cache"] == inp.k_cache0, axis=(2, 3))
    assert kv_changed.sum() > 0
    t = 0
    for b in range(inp.B):
        ql = int(inp.q_indptr[b + 1] - inp.q_indptr[b])
        for j in range(ql):
            L = int(inp.seq_lens[b]) - ql + j
            page = inp.page_table[b, L // inp.page_size]
            assert np.array_equal(out["k_cache"][page, L % inp.page_size].reshape(-1),
                                  inp.qkv[t, Hq * D:(Hq + Hkv) * D])
            t += 1


def test_head_dim_64_matches_per_head_composition():
    """D = 64 heads (the GPT-OSS row of the vLLM issue's model table): each
    Q head equals rmsnorm -> rope -> bf16 of the pinned step functions."""
    inp = _small(D=64, Hq=4, Hkv=2, q_mode=W.Q_BF16, norm=W.NORM_RMS)
    out = run_oracle(inp)
    D = 64
    for t in range(inp.T):
        pos = inp.positions[t]
        c, s = inp.cos_sin[pos, :D // 2], inp.cos_sin[pos, D // 2:]
        for h in range(inp.Hq):
            x = W.bf16_bits_to_f32(inp.qkv[t, h * D:(h + 1) * D]).astype(np.float64)
            y = oracle.rmsnorm(x, inp.q_norm_weight, W.NORM_RMS, inp.eps)
            o = oracle.rope(y, inp.rope, c, s)
            assert np.array_equal(out["q_out"][t, h], W.to_bf16_bits(o.astype(np.float32)))


def test_in_place_q_and_k_leave_v_and_padding_untouched():
    inp = _small(row_pad=64, q_in_place=True, k_in_place=True, norm=W.NORM_GEMMA)
    out = run_oracle(inp)
    Hq, Hkv, D = inp.Hq, inp.Hkv, inp.D
    assert np.array_equal(out["qkv"][:, (Hq + Hkv) * D:], inp.qkv[:, (Hq + Hkv) * D:])
    # Q and K columns equal the out-of-place result
    ref = _small(row_pad=64, norm=W.NORM_GEMMA)
    out_ref = run_oracle(ref)
    assert np.array_equal(out["qkv"][:, :Hq * D], out_ref["q_out"].reshape(inp.T, -1))
    assert np.array_equal(out["k_cache"], out_ref["k_cache"])
    assert np.array_equal(out["v_cache"], out_ref["v_cache"])


def test_slot_addressing_matches_paged_when_slots_are_the_paged_cells():
    inp = _small(norm=W.NORM_RMS, zero_tail=False)
    out_paged = run_oracle(inp)
    slots = []
    for b in range(inp.B):
        ql = int(inp.q_indptr[b + 1] - inp.q_indptr[b])
        for j in range(ql):
            L = int(inp.seq_lens[b]) - ql + j
            slots.append(int(inp.page_table[b, L // inp.page_size]) * inp.page_size + L % inp.page_size)
    inp.addressing = W.ADDR_SLOT
    inp.slot_mapping = np.array(slots, np.int64)
    inp.slot_mapping[0] = -1                  # padding token: Q written, K/V skipped
    out_slot = run_oracle(inp)
    assert np.array_equal(out_slot["q_out"], out_paged["q_out"])
    p0, r0 = divmod(slots[0], inp.page_size)
    kc = out_paged["k_cache"].copy()
    vc = out_paged["v_cache"].copy()
    kc[p0, r0] = inp.k_cache0[p0, r0]
    vc[p0, r0] = inp.v_cache0[p0, r0]
    assert np.array_equal(out_slot["k_cache"], kc)
    assert np.array_equal(out_slot["v_cache"], vc)


# ----------------------------------------------------------------------------
# MLA
# ----------------------------------------------------------------------------

def run_mla(inp: W.MlaInputs):
    out = {"q": inp.q.copy(), "kv_cache": inp.kv_cache0.copy()}
    oracle.mla_concat_rope_append(inp, out)
    return out


@pytest.mark.parametrize("fp8", [True, False])
def test_mla_concat_layout_and_values(fp8):
    inp = W.mla_case(seed=3, T=9, H=4, num_blocks=4, block_size=8, kv_fp8=fp8, negative_slots=2)
    out = run_mla(inp)
    K, R, nope = inp.kv_lora_rank, inp.rope_dim, inp.nope_dim
    # q_nope untouched; each head's rope slice is the interleaved rotation of
    # that head's own slice by the token's own angles, written as bf16 (numpy
    # complex multiplication of the pairs (2i, 2i+1) by cos + i sin, in fp64)
    assert np.array_equal(out["q"][:, :, :nope], inp.q[:, :, :nope])
    for t in range(inp.T):
        pos = inp.positions[t]
        e = inp.cos_sin[pos, :R // 2].astype(np.float64) + 1j * inp.cos_sin[pos, R // 2:].astype(np.float64)
        for h in range(inp.H):
            x = W.bf16_bits_to_f32(inp.q[t, h, nope:]).astype(np.float64)
            z = (x[0::2] + 1j * x[1::2]) * e
            o = np.empty(R)
            o[0::2], o[1::2] = z.real, z.imag
            assert np.array_equal(out["q"][t, h, nope:], W.to_bf16_bits(o.astype(np.float32))), (t, h)
    written = set()
    for t in range(inp.T):
        s = int(inp.slot_mapping[t])
        if s < 0:
            continue
        row = out["kv_cache"][s // inp.block_size, s % inp.block_size]
        written.add(s)
        kc = W.bf16_bits_to_f32(inp.kv_c[t]).astype(np.float64)
        if fp8:
            assert np.array_equal(row[:K], oracle.f64_to_e4m3(kc / np.float64(np.float32(0.02))))
        else:
            assert np.array_equal(row[:K], inp.kv_c[t])
        # the rope part equals the roped k_pe, which RoPE on q uses identically:
        # treat k_pe as a q head and compare
        x = W.bf16_bits_to_f32(inp.k_pe[t]).astype(np.float64)
        pos = inp.positions[t]
        c = inp.cos_sin[pos, :R // 2].astype(np.float64)
        sn = inp.cos_sin[pos, R // 2:].astype(np.float64)
        o = oracle.rope(x, 1, c, sn).astype(np.float32)
        if fp8:
            assert np.array_equal(row[K:], oracle.f64_to_e4m3(o.astype(np.float64) / np.float64(np.float32(0.02))))
        else:
            assert np.array_equal(row[K:], oracle.f32_to_bf16(o))
    # all other rows keep their bytes
    flat = out["kv_cache"].reshape(-1, K + R)
    flat0 = inp.kv_cache0.reshape(-1, K + R)
    for s in range(flat.shape[0]):
        if s not in written:
            assert np.array_equal(flat[s], flat0[s])


# ----------------------------------------------------------------------------
# MLA Q quantisation (FP8 q_out; the vLLM issue's static per-tensor and
# dynamic per-token question, the FlashInfer MLA RoPE + quantize kernel)
# ----------------------------------------------------------------------------

def run_mla_q8(inp: W.MlaInputs):
    out = {"q": inp.q.copy(), "kv_cache": inp.kv_cache0.copy(), "q_out": inp.q_out0.copy(),
           "q_scale": None if inp.q_scale0 is None else inp.q_scale0.copy()}
    oracle.mla_concat_rope_append(inp, out)
    return out


def _e4m3_grid_bits(rng, shape, lo_exp=-5, hi_exp=7):
    """bf16 bits of random normal E4M3 values 2^e * (1 + m/8), e in [lo, hi]."""
    e = rng.integers(lo_exp, hi_exp + 1, size=shape)
    m = rng.integers(0, 8, size=shape)
    sgn = np.where(rng.random(shape) < 0.5, -1.0, 1.0)
    v = sgn * np.ldexp(1.0 + m / 8.0, e)
    return W.to_bf16_bits(v)


@pytest.mark.parametrize("q_scale_inv", [1.0, 0.5])
def test_mla_static_fp8_q_of_grid_values_at_position_zero(q_scale_inv):
    """At position 0 RoPE is the identity (cos 1, sin 0), so with inputs on
    the E4M3 grid and a power-of-two static scale every code is exact: the
    nope dims pass through, the rope dims too, and q stays untouched."""
    inp = W.mla_case(seed=8, T=5, H=3, num_blocks=2, block_size=8, positions=np.zeros(5, np.int64),
                     q_mode=W.Q_FP8_STATIC, q_scale_inv=q_scale_inv)
    rng = np.random.default_rng(80)
    inp.q = _e4m3_grid_bits(rng, inp.q.shape)
    out = run_mla_q8(inp)
    assert np.array_equal(out["q"], inp.q)
    x = W.bf16_bits_to_f32(inp.q).astype(np.float64) * q_scale_inv
    lut = np.array([oracle.e4m3_to_f64(c) for c in range(256)])
    assert np.array_equal(lut[out["q_out"]], x)


def test_mla_dynamic_fp8_q_scale_spans_all_heads_of_a_token():
    """One scale per token over every head: token 0 has a single 10.0 in head
    2 and values <= 1 elsewhere, so s = fp32(10 / 448) for the whole token;
    10.0 encodes to 448 (0x7E) and the other heads' codes use the same s."""
    T, H = 3, 4
    inp = W.mla_case(seed=9, T=T, H=H, num_blocks=2, block_size=8, positions=np.zeros(T, np.int64),
                     q_mode=W.Q_FP8_DYNAMIC)
    rng = np.random.default_rng(90)
    vals = rng.uniform(-1.0, 1.0, size=inp.q.shape)
    vals[0, 2, 17] = 10.0
    vals[1] = 0.0                                  # all-zero token
    inp.q = W.to_bf16_bits(vals)
    out = run_mla_q8(inp)
    s0 = out["q_scale"][0]
    assert s0 == np.float32(10.0 / 448.0)
    assert out["q_out"][0, 2, 17] == 0x7E
    x0 = W.bf16_bits_to_f32(inp.q[0]).astype(np.float64)
    assert np.array_equal(out["q_out"][0], oracle.f64_to_e4m3(x0 / np.float64(s0)))
    assert out["q_scale"][1] == np.float32(1e-6 / 448.0)
    assert not out["q_out"][1].any()
    # no code above the top of the range
    lut = np.array([abs(oracle.e4m3_to_f64(c)) if c not in (0x7F, 0xFF) else np.inf for c in range(256)])
    assert lut[out["q_out"]].max() <= 448.0


def test_mla_fp8_q_suppressed_token_writes_nothing():
    inp = W.mla_case(seed=10, T=6, H=2, num_blocks=2, block_size=8, q_mode=W.Q_FP8_DYNAMIC)
    inp.positions = inp.positions.copy()
    inp.positions[4] = -1
    out = run_mla_q8(inp)
    assert np.array_equal(out["q_out"][4], inp.q_out0[4])
    assert out["q_scale"][4].tobytes() == inp.q_scale0[4].tobytes()
    assert not np.array_equal(out["q_out"][3], inp.q_out0[3])
    assert np.array_equal(out["q"], inp.q)


def test_mla_static_fp8_q_rotates_only_the_rope_slice():
    """At non-zero positions the nope dims of E4M3-grid inputs still pass
    through exactly (scale 1), and the rope dims are E4M3 of the pinned RoPE
    of that slice rounded to fp32."""
    inp = W.mla_case(seed=11, T=4, H=3, num_blocks=2, block_size=8, q_mode=W.Q_FP8_STATIC, rope=W.ROPE_NEOX)
    rng = np.random.default_rng(110)
    inp.q = _e4m3_grid_bits(rng, inp.q.shape)
    out = run_mla_q8(inp)
    N, R = inp.nope_dim, inp.rope_dim
    lut = np.array([oracle.e4m3_to_f64(c) for c in range(256)])
    x = W.bf16_bits_to_f32(inp.q).astype(np.float64)
    assert np.array_equal(lut[out["q_out"][:, :, :N]], x[:, :, :N])
    for t in range(inp.T):
        pos = inp.positions[t]
        c, s = inp.cos_sin[pos, :R // 2], inp.cos_sin[pos, R // 2:]
        for h in range(inp.H):
            o = oracle.rope(x[t, h, N:], W.ROPE_NEOX, c, s).astype(np.float32)
            assert np.array_equal(out["q_out"][t, h, N:], oracle.f64_to_e4m3(o.astype(np.float64)))



# ----------------------------------------------------------------------------
# K/V redirect and dynamic K/V scales
# ----------------------------------------------------------------------------

def _cell(inp, t):
    b = int(np.searchsorted(inp.q_indptr, t, side="right") - 1)
    ql = int(inp.q_indptr[b + 1] - inp.q_indptr[b])
    L = int(inp.seq_lens[b]) - ql + (t - int(inp.q_indptr[b]))
    return int(inp.page_table[b, L // inp.page_size]), L % inp.page_size


@pytest.mark.parametrize("kv_fp8,mode", [(True, W.KV_SCALE_STATIC), (False, W.KV_SCALE_STATIC),
                                         (True, W.KV_SCALE_TOKEN), (True, W.KV_SCALE_GROUP)])
def test_redirected_kv_rows_equal_the_cache_rows_and_leave_the_caches_alone(kv_fp8, mode):
    """FlashInfer "Contract" (caller-owned out_k / out_v) and its review (no
    tail clear when K/V are redirected): row t of out_k / out_v holds what the
    plain call writes at token t's cache cell, with the same scales; the
    caches keep every byte; flags and Q are unchanged."""
    kw = dict(kv_fp8=kv_fp8, k_scale=0.05, v_scale=0.07, kv_scale_mode=mode, kv_group_size=32,
              q_mode=W.Q_FP8_DYNAMIC)
    plain = _small(**kw)
    red = _small(kv_redirect=True, **kw)
    op, orr = run_oracle(plain), run_oracle(red)
    assert np.array_equal(orr["k_cache"], red.k_cache0) and np.array_equal(orr["v_cache"], red.v_cache0)
    assert np.array_equal(op["q_out"], orr["q_out"]) and np.array_equal(op["flags"], orr["flags"])
    for t in range(plain.T):
        page, row = _cell(plain, t)
        assert np.array_equal(orr["out_k"][t], op["k_cache"][page, row])
        assert np.array_equal(orr["out_v"][t], op["v_cache"][page, row])
        if mode != W.KV_SCALE_STATIC:
            crow = page * plain.page_size + row
            assert np.array_equal(orr["k_scale_out"][t], op["k_scale_out"][crow])
            assert np.array_equal(orr["v_scale_out"][t], op["v_scale_out"][crow])


@pytest.mark.parametrize("mutation", ["page_id_negative", "page_id_past_pool"])
def test_redirect_reads_and_checks_no_page_id(mutation):
    """Page ids are checked for the pages a call writes (the FlashInfer
    contract's validation guards the pool; its review: nothing is written
    into the caches when K/V are redirected).  A redirected call writes no
    page, so an out-of-pool page id leaves it valid with the same outputs,
    while the same table makes the paged call invalid.  The other metadata
    checks still apply under redirect."""
    kw = dict(kv_fp8=True, k_scale=0.05, v_scale=0.07, q_mode=W.Q_FP8_DYNAMIC)
    ok = run_oracle(_small(kv_redirect=True, **kw))
    red = _small(kv_redirect=True, **kw)
    _mutations()[mutation](red)
    got = run_oracle(red)
    assert (got["flags"] == 0).all()
    for k in ("q_out", "out_k", "out_v", "k_cache", "v_cache"):
        assert np.array_equal(got[k], ok[k]), k
    plain = _small(**kw)
    _mutations()[mutation](plain)
    assert (run_oracle(plain)["flags"] == -1).all()
    bad_len = _small(kv_redirect=True, **kw)
    _mutations()["seq_len_below_q_len"](bad_len)
    out = run_oracle(bad_len)
    assert (out["flags"] == -1).all() and np.array_equal(out["out_k"], bad_len.out_k0)


def test_token_kv_scales_closed_forms():
    """Dynamic per-(token, kv head) K/V scales, s = max(amax, 1e-6) / 448 of
    the encoded row: with no norm at position 0 (identity rotation) a K row
    whose largest magnitude is 10 gets s = fp32(10/448) and that element
    encodes to 448 (0x7E); an all-zero V row gets fp32(1e-6/448) and zero codes."""
    inp = _small(kv_fp8=True, kv_scale_mode=W.KV_SCALE_TOKEN, norm=W.NORM_NONE, Hkv=1)
    inp.positions = np.zeros(inp.T, np.int64)
    qkv = inp.qkv.copy()
    Hq, D = inp.Hq, inp.D
    rng = np.random.default_rng(12)
    qkv[:, Hq * D:(Hq + 1) * D] = W.to_bf16_bits(rng.uniform(-1, 1, size=(inp.T, D)))
    qkv[0, Hq * D + 5] = W.to_bf16_bits(np.array([-10.0]))[0]
    qkv[:, (Hq + 1) * D:(Hq + 2) * D] = 0
    inp.qkv = qkv
    out = run_oracle(inp)
    page, row = _cell(inp, 0)
    crow = page * inp.page_size + row
    assert out["k_scale_out"][crow, 0, 0] == np.float32(10.0 / 448.0)
    assert out["k_cache"][page, row, 0, 5] == 0xFE           # -448
    assert out["v_scale_out"][crow, 0, 0] == np.float32(1e-6 / 448.0)
    assert not out["v_cache"][page, row].any()
    for t in range(inp.T):
        page, row = _cell(inp, t)
        crow = page * inp.page_size + row
        x = W.bf16_bits_to_f32(inp.qkv[t, Hq * D:(Hq + 1) * D]).astype(np.float64)
        s = out["k_scale_out"][crow, 0, 0]
        assert s == np.float32(np.abs(x).max() / 448.0)
        assert np.array_equal(out["k_cache"][page, row, 0], oracle.f64_to_e4m3(x / np.float64(s)))


def test_group_kv_scales_follow_each_group_and_reduce_to_token_mode():
    """Per-group scales (groups of 32 dims): group k of a V row with largest
    magnitude 2^k gets s_k = fp32(2^k / 448); a group size equal to the head
    dim gives exactly the per-token result."""
    inp = _small(kv_fp8=True, kv_scale_mode=W.KV_SCALE_GROUP, kv_group_size=32, Hkv=1)
    qkv = inp.qkv.copy()
    Hq, D = inp.Hq, inp.D
    rng = np.random.default_rng(13)
    v = rng.uniform(-0.5, 0.5, size=(inp.T, D))
    for k in range(D // 32):
        v[:, 32 * k + 3] = 2.0 ** k
    qkv[:, (Hq + 1) * D:(Hq + 2) * D] = W.to_bf16_bits(v)
    inp.qkv = qkv
    out = run_oracle(inp)
    for t in range(inp.T):
        page, row = _cell(inp, t)
        crow = page * inp.page_size + row
        for k in range(D // 32):
            assert out["v_scale_out"][crow, 0, k] == np.float32(2.0 ** k / 448.0)
            assert out["v_cache"][page, row, 0, 32 * k + 3] == 0x7E
    tok = _small(kv_fp8=True, kv_scale_mode=W.KV_SCALE_TOKEN, Hkv=1)
    grp = _small(kv_fp8=True, kv_scale_mode=W.KV_SCALE_GROUP, kv_group_size=D, Hkv=1)
    ot, og = run_oracle(tok), run_oracle(grp)
    for key in ("k_cache", "v_cache", "k_scale_out", "v_scale_out"):
        assert np.array_equal(ot[key], og[key]), key


def test_tail_clear_zeroes_the_dynamic_scales_of_cleared_rows():
    inp = _small(kv_fp8=True, kv_scale_mode=W.KV_SCALE_TOKEN)
    out = run_oracle(inp)
    ps = inp.page_size
    for b in range(inp.B):
        sl = int(inp.seq_lens[b])
        if sl <= 0:
            continue
        last = (sl - 1) % ps
        page = int(inp.page_table[b, (sl - 1) // ps])
        for r in range(last + 1, ps):
            assert not out["k_scale_out"][page * ps + r].any()
            assert not out["v_scale_out"][page * ps + r].any()
            assert not out["k_cache"][page, r].any()
