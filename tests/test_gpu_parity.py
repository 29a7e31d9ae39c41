"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Every case draws seeded inputs, runs libqkprep on the GPU and the oracle on
host copies of the same inputs, and compares every output byte under the
tolerances stated in tests/gpu_harness.py.  Guard bytes around every device
buffer must survive each call.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_token_amd as qp
import workloads as W
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def run_and_compare(inp: W.NraInputs) -> dict:
    dev = H.DeviceNra(inp)
    dev.run()
    torch.cuda.synchronize()
    assert dev.guards_intact(), "guard bytes around a device buffer changed"
    gpu = dev.host_outputs()
    ref = H.oracle_outputs(inp)
    return H.compare_nra(inp, gpu, ref)


# ----------------------------------------------------------------------------
# the five configurations at full size
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["c1", "c3", "c3_16k", "c4"])
def test_config_full_size(name):
    inp = W.c3_prefill_fp8_16k() if name == "c3_16k" else W.CONFIGS[name]()
    if name == "c3_16k":
        assert inp.T == 16384 and inp.B == 8 and 1 <= np.diff(inp.q_indptr).min() \
            and np.diff(inp.q_indptr).max() <= 4096
    stats = run_and_compare(inp)
    H.assert_exact_floors(stats)
    print(name, inp.T, stats, flush=True)


@pytest.mark.parametrize("page_size", [16, 1])
def test_prefill_16k_small_pages(page_size):
    """The 16 384-token FP8 prefill at page 16 (1 032 pages) and page 1
    (16 384 pages): the validation reads and checks every page id the call
    writes in every workgroup; placement, tails and values as at page 64."""
    inp = W.c3_prefill_fp8_16k(page_size=page_size, maxp=4096 // page_size)
    stats = run_and_compare(inp)
    H.assert_exact_floors(stats)
    print(page_size, stats, flush=True)


_POLICY_CASES = {
    "prefill_fp8_dyn_padded": lambda: W.c3_prefill_fp8(q_lens=np.array([300, 0, 77, 1025]), name="p"),
    "decode_bf16": lambda: W.nra_case(seed=71, q_lens=np.ones(40, np.int64),
                                      prior_lens=np.random.default_rng(71).integers(0, 500, 40),
                                      Hq=32, Hkv=8, D=128, page_size=16),
    "d64_static_partial": lambda: W.nra_case(seed=72, q_lens=[33, 70, 5], prior_lens=[0, 12, 90], Hq=8, Hkv=2,
                                             D=64, page_size=16, kv_fp8=True, k_scale=0.05, v_scale=0.05,
                                             q_mode=W.Q_FP8_STATIC, q_scale_inv=2.0, rotary_dim=32),
    "d256_partial_rotary_fp8kv": lambda: W.nra_case(seed=73, q_lens=[40, 9], prior_lens=[3, 100], Hq=4, Hkv=2,
                                               D=256, page_size=32, kv_fp8=True, k_scale=0.05,
                                               v_scale=0.05, rotary_dim=96),
    "redirect_token_scales": lambda: W.nra_case(seed=74, q_lens=[50, 13], prior_lens=[0, 7], Hq=8, Hkv=2,
                                                D=128, page_size=16, kv_fp8=True, kv_redirect=True,
                                                kv_scale_mode=W.KV_SCALE_TOKEN, q_mode=W.Q_FP8_DYNAMIC),
}


@pytest.mark.parametrize("case", list(_POLICY_CASES))
def test_store_policies_write_the_same_bytes(case):
    """QKPREP_STORE_KEEP (ordinary row stores) and the default streaming
    stores run different kernel instances; both match the oracle and each
    other byte for byte."""
    outs = []
    for policy in (qp.STORE_STREAM, qp.STORE_KEEP):
        inp = _POLICY_CASES[case]()
        inp.store_policy = policy
        dev = H.DeviceNra(inp)
        dev.run()
        torch.cuda.synchronize()
        assert dev.guards_intact()
        gpu = dev.host_outputs()
        H.compare_nra(inp, gpu, H.oracle_outputs(inp))
        outs.append(gpu)
    for k in outs[0]:
        if outs[0][k] is not None:
            H.check_exact(outs[0][k], outs[1][k], f"{k}: streaming vs keep")


@pytest.mark.parametrize("q_mode", [W.Q_BF16, W.Q_FP8_DYNAMIC, W.Q_FP8_STATIC])
def test_mla_store_policies_write_the_same_bytes(q_mode):
    outs = []
    for policy in (qp.STORE_STREAM, qp.STORE_KEEP):
        inp = W.mla_case(seed=81 + q_mode, T=77, H=24, num_blocks=8, block_size=16, negative_slots=2,
                         q_mode=q_mode, q_scale_inv=0.5)
        inp.store_policy = policy
        dev = H.DeviceMla(inp)
        dev.run()
        torch.cuda.synchronize()
        assert dev.guards_intact()
        gpu = dev.host_outputs()
        H.compare_mla(inp, gpu, H.oracle_mla(inp))
        outs.append(gpu)
    for k in outs[0]:
        H.check_exact(outs[0][k], outs[1][k], f"{k}: streaming vs keep")


def test_checks_fire_on_planted_corruption():
    """Negative controls of the checker itself: after a valid call that
    passes, a guard byte flipped with a plain torch write (no kernel) fails
    guards_intact(), and a byte flipped in a page the call never writes
    fails the byte-exact comparison of the untouched cache bytes."""
    inp = W.nra_case(seed=61, q_lens=[5, 9], prior_lens=[2, 30], Hq=8, Hkv=2, D=128, page_size=16)
    dev = H.DeviceNra(inp)
    dev.run()
    torch.cuda.synchronize()
    assert dev.guards_intact()
    ref = H.oracle_outputs(inp)
    H.compare_nra(inp, dev.host_outputs(), ref)
    dev.k_cache.raw[H.GUARD - 1] ^= 0xFF            # the byte just before the cache
    assert not dev.guards_intact()
    dev.k_cache.raw[H.GUARD - 1] ^= 0xFF
    dev.v_cache.raw[-1] ^= 0x01                     # the last guard byte after the V cache
    assert not dev.guards_intact()
    dev.v_cache.raw[-1] ^= 0x01
    assert dev.guards_intact()
    untouched = np.setdiff1d(np.arange(inp.num_pages), inp.touched_pages())
    p = int(untouched[len(untouched) // 2])
    dev.v_cache.t.view(inp.num_pages, -1)[p, 77] ^= 0x0100
    with pytest.raises(AssertionError, match="v_cache outside appended rows"):
        H.compare_nra(inp, dev.host_outputs(), ref)
    dev.v_cache.t.view(inp.num_pages, -1)[p, 77] ^= 0x0100
    H.compare_nra(inp, dev.host_outputs(), ref)


@pytest.mark.parametrize("mutation", ["page_id_negative", "page_id_past_pool"])
def test_redirect_reads_and_checks_no_page_id(mutation):
    """With K/V redirected the call writes no page, so page ids are neither
    read nor checked: an out-of-pool id leaves the call valid, with the
    oracle's outputs; the other metadata checks still apply (see the
    malformed-metadata cases)."""
    q, prior = _ragged(93, B=5, max_q=30, max_prior=100)
    q[0] = 4
    inp = W.nra_case(seed=93, q_lens=q, prior_lens=prior, Hq=8, Hkv=2, D=128, page_size=16, kv_fp8=True,
                     k_scale=0.05, v_scale=0.05, q_mode=W.Q_FP8_DYNAMIC, kv_redirect=True)
    if mutation == "page_id_negative":
        inp.page_table[0, (int(inp.seq_lens[0]) - 1) // inp.page_size] = -1
    else:
        inp.page_table[2, 0] = inp.num_pages
    stats = run_and_compare(inp)
    assert (H.oracle_outputs(inp)["flags"] == 0).all()
    print(stats, flush=True)


def test_c3_with_an_empty_request():
    inp = W.c3_prefill_fp8(empty_request=3)
    assert inp.q_indptr[4] == inp.q_indptr[3]
    stats = run_and_compare(inp)
    print(stats, flush=True)


@pytest.mark.parametrize("name", ["X_decode_64x8_B256_q1_n2", "X_decode_8x1_B256_q1_n2", "E_prefill_64x8_q128",
                                  "P_prefill_64x8_q1_n2", "X_prefill_64x8_B1_Q1024_q1_n2"])
def test_pages_measured_rows(name):
    """The FlashInfer PR's measured rows as rebuilt for the benchmark (decode
    tokens in row 0 of a fresh page, token-major Q scales; prefill requests
    with padded Q scales and max_seqlen = q_len), on a smaller page pool."""
    print(run_and_compare(W.pages_row(name, prior_pages=4)), flush=True)


def test_c2_full_pool():
    """B=256 decode over the full ~262k-page pool (17 GB of bf16 cache): the
    touched pages are compared with the oracle run on a pool relabelled to
    those pages; every other page must be byte-identical to its snapshot."""
    inp = W.c2_decode_b256()
    dev = H.DeviceNra(inp)
    pages = inp.touched_pages()
    pidx = torch.from_numpy(pages).to(H.DEV)
    k_before = dev.k_cache.t[pidx].cpu().numpy().view(np.uint16)
    v_before = dev.v_cache.t[pidx].cpu().numpy().view(np.uint16)
    k_snap = dev.k_cache.t.clone()
    v_snap = dev.v_cache.t.clone()
    dev.run()
    torch.cuda.synchronize()
    assert dev.guards_intact()
    untouched = torch.ones(inp.num_pages, dtype=torch.bool, device=H.DEV)
    untouched[pidx] = False
    assert torch.equal(dev.k_cache.t[untouched], k_snap[untouched])
    assert torch.equal(dev.v_cache.t[untouched], v_snap[untouched])
    del k_snap, v_snap
    gpu = dev.host_outputs(pages=pages)
    cinp = H.compact_inputs(inp, k_before, v_before, pages)
    ref = H.oracle_outputs(cinp)
    stats = H.compare_nra(cinp, gpu, ref)
    H.assert_exact_floors(stats)
    print(stats, flush=True)


def test_c5_mla_full_size():
    inp = W.c5_mla()
    dev = H.DeviceMla(inp)
    dev.run()
    torch.cuda.synchronize()
    assert dev.guards_intact()
    stats = H.compare_mla(inp, dev.host_outputs(), H.oracle_mla(inp))
    H.assert_exact_floors(stats)
    print(stats, flush=True)


@pytest.mark.parametrize("q_mode", [W.Q_BF16, W.Q_FP8_DYNAMIC])
def test_mla_long_call_at_the_grid_limits(q_mode):
    """140 000 tokens of one head: the bf16-query launch wants 35 000
    workgroups of 8 items and is capped at 32 768 (so each takes 8 or 9
    items and the range split works near its 31-bit bound); the E4M3-query
    launch loops each workgroup over about 45 tokens.  Every output against
    the oracle."""
    inp = W.mla_case(seed=730, T=140_000, H=1, num_blocks=2200, block_size=64, q_mode=q_mode, negative_slots=3)
    dev = H.DeviceMla(inp)
    dev.run()
    torch.cuda.synchronize()
    assert dev.guards_intact()
    stats = H.compare_mla(inp, dev.host_outputs(), H.oracle_mla(inp))
    H.assert_exact_floors(stats)


# ----------------------------------------------------------------------------
# variants on small shapes (several tiles and a ragged tail)
# ----------------------------------------------------------------------------

def _ragged(seed, B=6, max_q=40, max_prior=300):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, max_q, size=B)
    q[1] = 0
    prior = rng.integers(0, max_prior, size=B)
    return q, prior


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("norm", [W.NORM_NONE, W.NORM_RMS, W.NORM_GEMMA])
@pytest.mark.parametrize("q_mode", [W.Q_BF16, W.Q_FP8_DYNAMIC, W.Q_FP8_STATIC])
@pytest.mark.parametrize("kv_fp8", [False, True])
def test_variant_matrix(D, norm, q_mode, kv_fp8):
    q, prior = _ragged(D + 10 * norm + 3 * q_mode + int(kv_fp8))
    inp = W.nra_case(seed=int(q.sum()), q_lens=q, prior_lens=prior, Hq=8, Hkv=2, D=D, page_size=16,
                     norm=norm, q_mode=q_mode, kv_fp8=kv_fp8, k_scale=0.07, v_scale=0.11,
                     q_scale_inv=3.5, qkv_sigma=2.0)
    run_and_compare(inp)


@pytest.mark.parametrize("rope", [W.ROPE_NEOX, W.ROPE_INTERLEAVED])
@pytest.mark.parametrize("heads", [(8, 1), (64, 8), (2, 2), (12, 4)])
@pytest.mark.parametrize("ps", [1, 4, 64])
def test_heads_pages_rope(rope, heads, ps):
    q, prior = _ragged(heads[0] + ps + rope, B=5, max_q=20, max_prior=200)
    inp = W.nra_case(seed=7 + ps, q_lens=q, prior_lens=prior, Hq=heads[0], Hkv=heads[1], D=128, page_size=ps,
                     rope=rope, q_mode=W.Q_FP8_DYNAMIC, kv_fp8=True, k_scale=0.05, v_scale=0.05)
    run_and_compare(inp)


# rotated dims R < D: R/16 rope lanes per head row, the rest pass through;
# R/2 a multiple of 16 pairs the rope lanes for 16-byte FP8 stores, other R
# store 8-byte halves; R = 0 reads no positions
@pytest.mark.parametrize("D,R", [(128, 64), (128, 32), (128, 96), (128, 48), (128, 16), (128, 0),
                                 (128, 80), (128, 112),
                                 (256, 128), (256, 80), (256, 64), (256, 112), (256, 16),
                                 (256, 160), (256, 144), (256, 240), (64, 32), (64, 16), (64, 48), (64, 0)])
@pytest.mark.parametrize("arm", ["fp8", "bf16"])
def test_partial_rotary(D, R, arm):
    q, prior = _ragged(D + R, B=5, max_q=30, max_prior=200)
    fp8 = arm == "fp8"
    inp = W.nra_case(seed=D * 7 + R, q_lens=q, prior_lens=prior, Hq=8, Hkv=2, D=D, page_size=16,
                     rotary_dim=R, rope=W.ROPE_NEOX if fp8 else W.ROPE_INTERLEAVED,
                     norm=W.NORM_RMS if fp8 else W.NORM_GEMMA,
                     q_mode=W.Q_FP8_DYNAMIC if fp8 else W.Q_BF16, kv_fp8=fp8, k_scale=0.05, v_scale=0.05,
                     k_in_place=not fp8, q_in_place=not fp8, row_pad=0 if fp8 else 64)
    if R == 0:
        inp.positions = inp.positions.copy()
        inp.positions[:3] = -9          # not read without rotated dims
    run_and_compare(inp)


@pytest.mark.parametrize("D", [128, 64])
def test_nope_layer_with_group_kv_scales(D):
    """No rotated dims (a NoPE layer) takes the whole-head lane layout, so
    per-group K/V scales smaller than the head are supported there too."""
    q, prior = _ragged(D + 3, B=5, max_q=30, max_prior=200)
    inp = W.nra_case(seed=D + 3, q_lens=q, prior_lens=prior, Hq=8, Hkv=2, D=D, page_size=16, rotary_dim=0,
                     kv_fp8=True, kv_scale_mode=W.KV_SCALE_GROUP, kv_group_size=32, q_mode=W.Q_FP8_DYNAMIC)
    inp.positions = inp.positions.copy()
    inp.positions[:2] = -5          # not read without rotated dims
    run_and_compare(inp)


def test_nope_layer_full_size_prefill():
    """The 15k-token FP8 prefill of a NoPE layer (rotary_dim = 0)."""
    stats = run_and_compare(W.c3_prefill_fp8(rotary_dim=0))
    H.assert_exact_floors(stats)
    print(stats, flush=True)


@pytest.mark.parametrize("D,R", [(128, 64), (128, 32), (256, 64), (128, 96), (256, 192), (64, 32)])
def test_partial_rotary_full_size_prefill(D, R):
    """The 15k-token FP8 prefill with partial rotary: round-robin spans, and
    the mirrored loads that read whole lines (all lanes trade up to half the
    head; beyond it only the outer lanes of each row do)."""
    stats = run_and_compare(W.c3_prefill_fp8(D=D, rotary_dim=R))
    H.assert_exact_floors(stats)
    print(stats, flush=True)


# K/V redirect to caller rows (caches untouched, no tail clear) and dynamic
# FP8 K/V scales per (token, kv head) or per group of dims
@pytest.mark.parametrize("addressing", [W.ADDR_PAGED, W.ADDR_SLOT])
@pytest.mark.parametrize("kv", ["bf16", "fp8", "fp8_token", "fp8_group32"])
def test_kv_redirect(addressing, kv):
    q, prior = _ragged(91 + addressing, B=5, max_q=40, max_prior=200)
    mode = {"bf16": 0, "fp8": 0, "fp8_token": W.KV_SCALE_TOKEN, "fp8_group32": W.KV_SCALE_GROUP}[kv]
    inp = W.nra_case(seed=91, q_lens=q, prior_lens=prior, Hq=8, Hkv=2, D=128, page_size=16,
                     addressing=addressing, kv_fp8=kv != "bf16", k_scale=0.05, v_scale=0.05,
                     q_mode=W.Q_FP8_DYNAMIC, kv_redirect=True, kv_scale_mode=mode, kv_group_size=32)
    inp.positions = inp.positions.copy()
    inp.positions[2] = -3
    run_and_compare(inp)


@pytest.mark.parametrize("D,mode,g", [(128, W.KV_SCALE_TOKEN, 0), (128, W.KV_SCALE_GROUP, 8),
                                      (128, W.KV_SCALE_GROUP, 16), (128, W.KV_SCALE_GROUP, 32),
                                      (128, W.KV_SCALE_GROUP, 64), (128, W.KV_SCALE_GROUP, 128),
                                      (256, W.KV_SCALE_GROUP, 128), (256, W.KV_SCALE_TOKEN, 0),
                                      (64, W.KV_SCALE_GROUP, 32), (64, W.KV_SCALE_TOKEN, 0)])
@pytest.mark.parametrize("addressing", [W.ADDR_PAGED, W.ADDR_SLOT])
def test_dynamic_kv_scales(D, mode, g, addressing):
    q, prior = _ragged(D + g + addressing, B=6, max_q=35, max_prior=150)
    inp = W.nra_case(seed=D + g, q_lens=q, prior_lens=prior, Hq=8, Hkv=2, D=D, page_size=16,
                     addressing=addressing, kv_fp8=True, kv_scale_mode=mode, kv_group_size=g,
                     q_mode=W.Q_FP8_STATIC, q_scale_inv=2.0, norm=W.NORM_GEMMA, qkv_sigma=3.0)
    run_and_compare(inp)


@pytest.mark.parametrize("D,R", [(128, 64), (128, 0), (128, 96), (128, 112), (64, 32), (256, 192)])
def test_token_kv_scales_with_partial_rotary(D, R):
    """Per-token K/V scales (an amax over the whole K row) with every
    rotary load layout: mirrored halves, the outer-lane trade above half the
    head, and paired rows of 64-dim heads."""
    q, prior = _ragged(R + D + 5, B=4, max_q=30, max_prior=100)
    inp = W.nra_case(seed=R + D + 5, q_lens=q, prior_lens=prior, Hq=4, Hkv=4, D=D, page_size=8,
                     rotary_dim=R, kv_fp8=True, kv_scale_mode=W.KV_SCALE_TOKEN)
    run_and_compare(inp)


@pytest.mark.parametrize("D,R", [(128, 96), (64, 48), (256, 208)])
@pytest.mark.parametrize("q_mode", [W.Q_FP8_STATIC, W.Q_BF16])
def test_wide_partial_rotary_other_q_modes(D, R, q_mode):
    """Rotary above half the head (and 64-dim partial rotary) with static
    E4M3 Q and bf16 Q, interleaved pairs, Gemma weights, K written back in
    place for the bf16 arm."""
    q, prior = _ragged(R + D + 11, B=5, max_q=25, max_prior=150)
    bf = q_mode == W.Q_BF16
    inp = W.nra_case(seed=R + D + 11, q_lens=q, prior_lens=prior, Hq=8, Hkv=2, D=D, page_size=16,
                     rotary_dim=R, rope=W.ROPE_INTERLEAVED, norm=W.NORM_GEMMA, q_mode=q_mode, q_scale_inv=2.0,
                     kv_fp8=not bf, k_scale=0.05, v_scale=0.05, q_in_place=bf, k_in_place=bf)
    run_and_compare(inp)


def test_c3_with_per_token_kv_scales():
    """The ragged 15k-token FP8 prefill with dynamic per-(token, kv head)
    K/V scales instead of the static ones (page-64 cache, tails cleared)."""
    inp = W.c3_prefill_fp8(kv_scale_mode=W.KV_SCALE_TOKEN)
    print(run_and_compare(inp), flush=True)


def test_head_dim_64_gqa_8_to_1():
    """64 Q heads over 8 KV heads of 64 dims (the GPT-OSS row of the vLLM
    issue's model table), FP8 Q with padded scales and E4M3 caches."""
    q, prior = _ragged(64, B=6, max_q=70, max_prior=500)
    inp = W.nra_case(seed=64, q_lens=q, prior_lens=prior, Hq=64, Hkv=8, D=64, page_size=16,
                     q_mode=W.Q_FP8_DYNAMIC, q_scale_padded=True, max_seqlen=128, kv_fp8=True,
                     k_scale=0.05, v_scale=0.05)
    run_and_compare(inp)


@pytest.mark.parametrize("hq,hkv,q_mode,kv_fp8,rope", [
    (3, 1, W.Q_BF16, False, W.ROPE_NEOX),          # 5 rows: the last row pair has one row past the end
    (7, 1, W.Q_FP8_DYNAMIC, True, W.ROPE_NEOX),    # 9 rows
    (5, 5, W.Q_FP8_STATIC, True, W.ROPE_INTERLEAVED),   # 15 rows, interleaved pairs
    (24, 8, W.Q_FP8_DYNAMIC, False, W.ROPE_NEOX),  # 40 rows: chunks of 16 rows end mid-token
])
def test_head_dim_64_row_pairs(hq, hkv, q_mode, kv_fp8, rope):
    """64-dim heads are loaded as pairs of whole 128-byte rows and exchanged
    between lanes: row counts that leave a pair half past the last row, and
    chunks that end inside a token, against the oracle."""
    q, prior = _ragged(640 + hq, B=5, max_q=90, max_prior=300)
    inp = W.nra_case(seed=640 + hq, q_lens=q, prior_lens=prior, Hq=hq, Hkv=hkv, D=64, page_size=16,
                     rope=rope, q_mode=q_mode, kv_fp8=kv_fp8, k_scale=0.05, v_scale=0.05)
    run_and_compare(inp)


def test_head_dim_64_long_call_row_pairs():
    """A 64-dim call long enough for round-robin spans (about 10k tokens),
    token-major Q scales."""
    q = np.array([3000, 2500, 2000, 2700], dtype=np.int64)
    inp = W.nra_case(seed=6464, q_lens=q, prior_lens=np.zeros(4, np.int64), Hq=16, Hkv=2, D=64, page_size=32,
                     q_mode=W.Q_FP8_DYNAMIC, kv_fp8=True, k_scale=0.05, v_scale=0.05)
    run_and_compare(inp)


@pytest.mark.parametrize("qlen", [127, 128, 129])
def test_dynamic_scale_padding_edge(qlen):
    """4 requests x Q tokens with max_seqlen = Q: the padded q_scale row is
    round_up(Q, 128) long and entries past Q are never written."""
    inp = W.nra_case(seed=qlen, q_lens=[qlen] * 4, prior_lens=[0, 5, 64, 300], Hq=8, Hkv=1, D=128,
                     page_size=16, norm=W.NORM_GEMMA, q_mode=W.Q_FP8_DYNAMIC, q_scale_padded=True,
                     max_seqlen=qlen, kv_fp8=True, k_scale=0.05, v_scale=0.05)
    run_and_compare(inp)


def test_upper_max_240():
    q, prior = _ragged(240)
    inp = W.nra_case(seed=240, q_lens=q, prior_lens=prior, Hq=8, Hkv=1, D=128, page_size=16,
                     q_mode=W.Q_FP8_DYNAMIC, upper_max=240.0, kv_fp8=True, k_scale=0.05, v_scale=0.05)
    run_and_compare(inp)


@pytest.mark.parametrize("D", [128, 256])
def test_strided_in_place(D):
    q, prior = _ragged(D + 1)
    inp = W.nra_case(seed=3, q_lens=q, prior_lens=prior, Hq=4, Hkv=2, D=D, page_size=8, row_pad=64,
                     norm=W.NORM_GEMMA, q_in_place=True, k_in_place=True)
    run_and_compare(inp)


@pytest.mark.parametrize("kv_fp8", [False, True])
def test_slot_addressing(kv_fp8):
    q, prior = _ragged(17)
    inp = W.nra_case(seed=17, q_lens=q, prior_lens=prior, Hq=8, Hkv=2, D=128, page_size=16,
                     addressing=W.ADDR_SLOT, kv_fp8=kv_fp8, q_mode=W.Q_FP8_DYNAMIC, k_scale=0.05,
                     v_scale=0.05)
    inp.slot_mapping = inp.slot_mapping.copy()
    inp.slot_mapping[[0, 5]] = -1                                   # padding tokens
    inp.slot_mapping[7] = inp.num_pages * inp.page_size + 3         # past the pool: skipped
    run_and_compare(inp)


@pytest.mark.parametrize("D,R", [(128, 128), (128, 96), (128, 32), (64, 32)])
def test_long_call_with_slot_addressing(D, R):
    """Over 8 tokens per resident workgroup the kernel deals 4-token spans
    round-robin instead of one contiguous range per workgroup: slot
    addressing, per-token-head Q scales, padding slots and suppressed
    positions on that path, with the whole-head and the partial-rotary load
    layouts."""
    q_lens = np.array([3001, 2999, 3100, 17], np.int64)
    inp = W.nra_case(seed=23 + R, q_lens=q_lens, prior_lens=np.array([5, 0, 64, 900]), Hq=8, Hkv=2, D=D,
                     page_size=16, addressing=W.ADDR_SLOT, q_mode=W.Q_FP8_DYNAMIC, kv_fp8=True,
                     k_scale=0.05, v_scale=0.05, rope=W.ROPE_INTERLEAVED, rotary_dim=R)
    assert inp.T >= 8 * 1024
    inp.slot_mapping = inp.slot_mapping.copy()
    inp.slot_mapping[[0, 4097, inp.T - 1]] = -1
    inp.positions = inp.positions.copy()
    inp.positions[[3, 5000]] = [-1, inp.cos_sin.shape[0] + 2]
    run_and_compare(inp)


def test_decode_mrope_positions_use_the_first_axis():
    """Decode with multimodal RoPE (SGLang PR, Qwen3 dispatch: decode mRoPE
    positions repeat one position on all three axes, so the first axis is
    exact): passing row 0 of a [3, T] int64 positions tensor gives the same
    bytes as the 1-D positions."""
    inp = W.nra_case(seed=33, q_lens=np.ones(48, np.int64), prior_lens=np.arange(48) * 37 + 5, Hq=16,
                     Hkv=2, D=128, page_size=16, q_mode=W.Q_FP8_DYNAMIC, kv_fp8=True, k_scale=0.05,
                     v_scale=0.05)
    plain = H.DeviceNra(inp)
    plain.run()
    mrope = H.DeviceNra(inp)
    pos3 = plain.positions.unsqueeze(0).repeat(3, 1).contiguous()
    kw = mrope.kwargs()
    kw["positions"] = pos3[0]
    qp.qkprep_norm_rope_append(**kw)
    torch.cuda.synchronize()
    a, b = plain.host_outputs(), mrope.host_outputs()
    for k in ("q_out", "q_scale", "k_cache", "v_cache", "flags"):
        assert np.array_equal(a[k], b[k]), k
    H.compare_nra(inp, b, H.oracle_outputs(inp))


def test_out_of_range_positions_suppress_tokens():
    q, prior = _ragged(21)
    inp = W.nra_case(seed=21, q_lens=q, prior_lens=prior, Hq=8, Hkv=2, D=128, page_size=16)
    inp.positions = inp.positions.copy()
    inp.positions[[2, 9]] = [-5, inp.cos_sin.shape[0]]
    run_and_compare(inp)


def test_only_empty_requests():
    inp = W.nra_case(seed=4, q_lens=[0, 0, 0], prior_lens=[5, 0, 33], Hq=8, Hkv=2, D=128, page_size=16)
    assert inp.T == 0
    run_and_compare(inp)


def test_empty_call_launches_nothing():
    inp = W.nra_case(seed=4, q_lens=[], prior_lens=[], Hq=8, Hkv=2, D=128, page_size=16)
    dev = H.DeviceNra(inp)
    dev.run()
    torch.cuda.synchronize()
    assert dev.guards_intact()


@pytest.mark.parametrize("mutation", ["first_nonzero", "non_monotone", "last_short", "seq_len_below_q_len",
                                      "too_many_pages", "page_id_negative", "page_id_past_pool",
                                      "above_max_seqlen"])
@pytest.mark.parametrize("shape", ["ragged", "short"])
def test_malformed_metadata(mutation, shape):
    """Each malformed input rejects the whole call: on a ragged batch (full
    validation path) and on a batch of 1-2-token requests, which writes at
    most two pages per request (short validation path)."""
    if shape == "ragged":
        q, prior = _ragged(31)
        q[0] = 5
    else:
        q = np.array([2, 1, 2, 1, 1, 2, 1, 1, 2, 1, 1, 1], np.int64)
        prior = np.random.default_rng(32).integers(0, 100, size=len(q))
    inp = W.nra_case(seed=31, q_lens=q, prior_lens=prior, Hq=8, Hkv=2, D=128, page_size=16,
                     q_mode=W.Q_FP8_DYNAMIC, q_scale_padded=True, max_seqlen=64, kv_fp8=True,
                     k_scale=0.05, v_scale=0.05)
    if mutation == "first_nonzero":
        inp.q_indptr[0] = 1
    elif mutation == "non_monotone":
        inp.q_indptr[2] = inp.q_indptr[1] - 1
    elif mutation == "last_short":
        inp.q_indptr[-1] = inp.T - 1
    elif mutation == "seq_len_below_q_len":
        inp.seq_lens[0] = int(q[0]) - 1
    elif mutation == "too_many_pages":
        inp.seq_lens[3] = inp.page_table.shape[1] * inp.page_size + 1
    elif mutation == "page_id_negative":
        inp.page_table[0, (int(inp.seq_lens[0]) - 1) // inp.page_size] = -1
    elif mutation == "page_id_past_pool":
        inp.page_table[2, (int(inp.seq_lens[2]) - 1) // inp.page_size] = inp.num_pages
    elif mutation == "above_max_seqlen":
        inp.max_seqlen = int(q.max()) - 1
    dev = H.DeviceNra(inp)
    dev.run()
    torch.cuda.synchronize()
    assert dev.guards_intact()
    gpu = dev.host_outputs()
    assert (gpu["flags"] == -1).all()
    H.check_exact(gpu["k_cache"], inp.k_cache0, "k_cache")
    H.check_exact(gpu["v_cache"], inp.v_cache0, "v_cache")
    H.check_exact(gpu["q_out"], inp.q_out0, "q_out")
    H.check_exact(gpu["q_scale"], inp.q_scale0, "q_scale")
    H.check_exact(gpu["qkv"], inp.qkv, "qkv")
    ref = H.oracle_outputs(inp)
    assert (ref["flags"] == -1).all()


@pytest.mark.parametrize("b", [5, 550])
@pytest.mark.parametrize("which", [0, 1, 2])
def test_out_of_pool_page_in_each_check_path(b, which):
    """600 requests writing 3-4 pages each (more than the 512 requests whose
    metadata the prologue holds in registers, more pages than the 256 page
    slots): a page id past the pool as a request's 1st, 2nd or 3rd written
    page, for a request below and one above 512, must reject the whole call."""
    B = 600
    q = np.full(B, 12, dtype=np.int64)
    prior = np.arange(B, dtype=np.int64) % 4
    inp = W.nra_case(seed=600 + b + which, q_lens=q, prior_lens=prior, Hq=8, Hkv=1, D=128, page_size=4,
                     maxp=8)
    first = int(prior[b]) // 4
    inp.page_table[b, first + which] = inp.num_pages + 1
    dev = H.DeviceNra(inp)
    dev.run()
    torch.cuda.synchronize()
    assert dev.guards_intact()
    gpu = dev.host_outputs()
    assert (gpu["flags"] == -1).all()
    H.check_exact(gpu["k_cache"], inp.k_cache0, "k_cache")
    H.check_exact(gpu["v_cache"], inp.v_cache0, "v_cache")
    assert (H.oracle_outputs(inp)["flags"] == -1).all()


@pytest.mark.parametrize("b,which,long_req", [(0, 0, None), (70, 1, None), (255, 1, None), (130, 0, 131),
                                               (200, 1, 3)])
def test_out_of_pool_page_short_validation_path(b, which, long_req):
    """256 requests writing two pages each (2 tokens across a page boundary)
    take the short validation path, where each thread checks its own
    request's page ids; one request writing three or more pages sends the
    call down the full path.  A page id past the pool as a request's 1st or
    2nd written page rejects the whole call in both."""
    B = 256
    q = np.full(B, 2, dtype=np.int64)
    prior = 4 * (np.arange(B, dtype=np.int64) % 5) + 3
    if long_req is not None:
        q[long_req] = 9
    inp = W.nra_case(seed=700 + b + which, q_lens=q, prior_lens=prior, Hq=8, Hkv=1, D=128, page_size=4, maxp=8)
    first = int(prior[b]) // 4
    inp.page_table[b, first + which] = inp.num_pages + 1
    dev = H.DeviceNra(inp)
    dev.run()
    torch.cuda.synchronize()
    assert dev.guards_intact()
    gpu = dev.host_outputs()
    assert (gpu["flags"] == -1).all()
    H.check_exact(gpu["k_cache"], inp.k_cache0, "k_cache")
    H.check_exact(gpu["v_cache"], inp.v_cache0, "v_cache")
    assert (H.oracle_outputs(inp)["flags"] == -1).all()


@pytest.mark.parametrize("q_mode,kv_fp8", [(W.Q_BF16, False), (W.Q_FP8_DYNAMIC, True), (W.Q_FP8_STATIC, True)])
@pytest.mark.parametrize("bad", [None, 0, 255])
def test_decodes_that_clear_tails_after_the_rows(q_mode, kv_fp8, bad):
    """Decodes of 256 or more requests with at least 4 head-row chunks per
    token (32/8/128 heads: 6) clear the page tails after the token rows.
    Valid calls match the oracle (tails zeroed, rows, flags); a page id past
    the pool in request 0 or 255 rejects the whole call and writes nothing."""
    B = 256
    rng = np.random.default_rng(720)
    prior = rng.integers(0, 60, B)
    inp = W.nra_case(seed=721, q_lens=np.ones(B, dtype=np.int64), prior_lens=prior, Hq=32, Hkv=8, D=128,
                     page_size=16, maxp=8, q_mode=q_mode, kv_fp8=kv_fp8, k_scale=0.05 if kv_fp8 else 1.0,
                     v_scale=0.05 if kv_fp8 else 1.0, q_scale_inv=4.0 if q_mode == W.Q_FP8_STATIC else 1.0)
    if bad is None:
        run_and_compare(inp)
        return
    inp.page_table[bad, int(prior[bad]) // 16] = inp.num_pages + 3
    dev = H.DeviceNra(inp)
    dev.run()
    torch.cuda.synchronize()
    assert dev.guards_intact()
    gpu = dev.host_outputs()
    assert (gpu["flags"] == -1).all()
    H.check_exact(gpu["k_cache"], inp.k_cache0, "k_cache")
    H.check_exact(gpu["v_cache"], inp.v_cache0, "v_cache")
    assert (H.oracle_outputs(inp)["flags"] == -1).all()


@pytest.mark.parametrize("long_req", [None, 0, 255])
def test_short_and_full_validation_paths_agree_on_valid_calls(long_req):
    """The same 256 two-page requests, valid, with and without one request
    long enough to force the full validation path: outputs match the oracle."""
    B = 256
    q = np.full(B, 2, dtype=np.int64)
    prior = 4 * (np.arange(B, dtype=np.int64) % 5) + 3
    if long_req is not None:
        q[long_req] = 9
    run_and_compare(W.nra_case(seed=710, q_lens=q, prior_lens=prior, Hq=8, Hkv=1, D=128, page_size=4, maxp=8))


@pytest.mark.parametrize("bad_tail", [False, True])
def test_short_validation_path_with_empty_requests(bad_tail):
    """A decode batch (short validation path) where some requests append
    nothing: an empty request with cached rows still has its last page's
    tail cleared, so that page is checked too; one past the pool rejects
    the call.  Requests with no rows at all touch no page."""
    B = 40
    q = np.ones(B, dtype=np.int64)
    q[[3, 17, 30]] = 0
    prior = (np.arange(B, dtype=np.int64) * 7) % 50
    prior[30] = 0                      # empty and no cached rows
    inp = W.nra_case(seed=720 + bad_tail, q_lens=q, prior_lens=prior, Hq=8, Hkv=2, D=128, page_size=16, maxp=8)
    if not bad_tail:
        run_and_compare(inp)
        return
    sl = int(prior[17])
    inp.page_table[17, (sl - 1) // 16] = inp.num_pages + 3
    dev = H.DeviceNra(inp)
    dev.run()
    torch.cuda.synchronize()
    assert dev.guards_intact()
    gpu = dev.host_outputs()
    assert (gpu["flags"] == -1).all()
    H.check_exact(gpu["k_cache"], inp.k_cache0, "k_cache")
    H.check_exact(gpu["v_cache"], inp.v_cache0, "v_cache")
    assert (H.oracle_outputs(inp)["flags"] == -1).all()


def test_many_requests_cross_page_ragged():
    rng = np.random.default_rng(99)
    B = 300
    q = rng.integers(0, 6, size=B)
    prior = rng.integers(0, 100, size=B)
    inp = W.nra_case(seed=99, q_lens=q, prior_lens=prior, Hq=16, Hkv=4, D=128, page_size=4,
                     kv_fp8=True, k_scale=0.05, v_scale=0.05, q_mode=W.Q_FP8_STATIC, q_scale_inv=2.0)
    run_and_compare(inp)


def test_maximum_request_count():
    """B = 4096 (the most the kernel stages): request metadata beyond the
    first 512 entries, page slots beyond the first 256, more requests than
    workgroups for the tail clears."""
    rng = np.random.default_rng(4096)
    B = 4096
    q = rng.integers(0, 3, size=B)
    prior = rng.integers(0, 50, size=B)
    inp = W.nra_case(seed=4096, q_lens=q, prior_lens=prior, Hq=8, Hkv=1, D=128, page_size=16)
    run_and_compare(inp)


def test_maximum_request_count_with_one_bad_request():
    rng = np.random.default_rng(4097)
    B = 4096
    q = rng.integers(1, 3, size=B)
    prior = rng.integers(0, 50, size=B)
    inp = W.nra_case(seed=4097, q_lens=q, prior_lens=prior, Hq=8, Hkv=1, D=128, page_size=16)
    inp.seq_lens = inp.seq_lens.copy()
    inp.seq_lens[4000] = 0                      # below its q_len: the whole call is invalid
    stats = run_and_compare(inp)
    assert stats == {} or "q" not in stats


def test_requests_spread_tails_with_scattered_page_slots():
    """100 requests (page slots found by scatter) and more workgroups than
    requests (each page-64 tail split across workgroups)."""
    rng = np.random.default_rng(100)
    q = rng.integers(20, 60, size=100)
    q[[3, 50]] = 0
    prior = rng.integers(0, 300, size=100)
    inp = W.nra_case(seed=100, q_lens=q, prior_lens=prior, Hq=8, Hkv=2, D=128, page_size=64,
                     kv_fp8=True, k_scale=0.05, v_scale=0.05, q_mode=W.Q_FP8_DYNAMIC, q_scale_padded=True,
                     max_seqlen=64)
    run_and_compare(inp)


# ----------------------------------------------------------------------------
# MLA variants
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("fp8", [True, False])
@pytest.mark.parametrize("rope", [W.ROPE_INTERLEAVED, W.ROPE_NEOX])
@pytest.mark.parametrize("H_", [128, 16, 20, 7, 1])   # odd H: the last head pair has one head past H
def test_mla_variants(fp8, rope, H_):
    inp = W.mla_case(seed=H_ + rope, T=77, H=H_, num_blocks=8, block_size=16, kv_fp8=fp8, rope=rope,
                     negative_slots=3)
    inp.positions = inp.positions.copy()
    inp.positions[5] = -1
    dev = H.DeviceMla(inp)
    dev.run()
    torch.cuda.synchronize()
    assert dev.guards_intact()
    H.compare_mla(inp, dev.host_outputs(), H.oracle_mla(inp))


def _run_mla(inp):
    dev = H.DeviceMla(inp)
    dev.run()
    torch.cuda.synchronize()
    assert dev.guards_intact()
    return H.compare_mla(inp, dev.host_outputs(), H.oracle_mla(inp))


@pytest.mark.parametrize("q_mode", [W.Q_FP8_DYNAMIC, W.Q_FP8_STATIC])
def test_mla_fp8_q_full_size(q_mode):
    """The 4096-token, 128-head MLA workload with Q quantised into an E4M3
    q_out: one dynamic scale per token over all heads, or a static scale."""
    inp = W.c5_mla(q_mode=q_mode, q_scale_inv=0.75)
    stats = _run_mla(inp)
    H.assert_exact_floors(stats)
    print(stats, flush=True)


# nope_dim multiple of 32 up to 128 (odd nope-vector counts store 8-byte
# pieces), head counts below, at and above a 64-head round, both caches
@pytest.mark.parametrize("q_mode", [W.Q_FP8_DYNAMIC, W.Q_FP8_STATIC])
@pytest.mark.parametrize("H_,nope", [(128, 128), (16, 64), (20, 96), (100, 32), (3, 0), (64, 128), (7, 64),
                                     (1, 128)])
@pytest.mark.parametrize("fp8", [True, False])
def test_mla_fp8_q_variants(q_mode, H_, nope, fp8):
    inp = W.mla_case(seed=H_ + nope + q_mode, T=61, H=H_, nope_dim=nope, num_blocks=8, block_size=16,
                     kv_fp8=fp8, rope=W.ROPE_NEOX if H_ % 2 else W.ROPE_INTERLEAVED, negative_slots=3,
                     q_mode=q_mode, q_scale_inv=2.0, upper_max=448.0 if fp8 else 240.0)
    inp.positions = inp.positions.copy()
    inp.positions[[0, 7]] = [-1, inp.cos_sin.shape[0]]
    _run_mla(inp)


def test_mla_static_fp8_q_more_than_two_rounds_of_heads():
    # 200 heads: the static mode walks 64-head rounds two at a time
    inp = W.mla_case(seed=200, T=19, H=200, num_blocks=4, block_size=16, q_mode=W.Q_FP8_STATIC,
                     q_scale_inv=1.5)
    _run_mla(inp)


# ----------------------------------------------------------------------------
# determinism, idempotency, graph capture
# ----------------------------------------------------------------------------

def _snapshot(dev: H.DeviceNra):
    return [b.raw.clone() for b in (dev.qkv, dev.k_cache, dev.v_cache, dev.q_out, dev.q_scale, dev.flags)
            if b is not None]


def _restore(dev: H.DeviceNra, snap):
    for b, s in zip([b for b in (dev.qkv, dev.k_cache, dev.v_cache, dev.q_out, dev.q_scale, dev.flags)
                     if b is not None], snap):
        b.raw.copy_(s)


def test_deterministic_and_idempotent():
    q, prior = _ragged(55)
    inp = W.nra_case(seed=55, q_lens=q, prior_lens=prior, Hq=8, Hkv=2, D=128, page_size=16,
                     q_mode=W.Q_FP8_DYNAMIC, kv_fp8=True, k_scale=0.05, v_scale=0.05)
    dev = H.DeviceNra(inp)
    before = _snapshot(dev)
    dev.run()
    first = _snapshot(dev)
    dev.run()                       # a repeated call rewrites the same bytes
    second = _snapshot(dev)
    _restore(dev, before)
    dev.run()
    third = _snapshot(dev)
    for a, b, c in zip(first, second, third):
        assert torch.equal(a, b) and torch.equal(a, c)


def test_graph_capture_replays_match_eager():
    q, prior = _ragged(77)
    inp = W.nra_case(seed=77, q_lens=q, prior_lens=prior, Hq=8, Hkv=2, D=128, page_size=16,
                     q_mode=W.Q_FP8_DYNAMIC, q_scale_padded=True, max_seqlen=64, kv_fp8=True,
                     k_scale=0.05, v_scale=0.05)
    dev = H.DeviceNra(inp)
    before = _snapshot(dev)
    dev.run()
    torch.cuda.synchronize()
    eager = _snapshot(dev)
    _restore(dev, before)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            dev.run()
    torch.cuda.synchronize()
    for rep in range(3):
        _restore(dev, before)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(dev)
        for a, b in zip(eager, got):
            assert torch.equal(a, b), f"replay {rep} differs from eager"


@pytest.mark.parametrize("maxp_pad", [0, 1])
@pytest.mark.parametrize("where", ["first", "middle", "last", "before_first", "after_last"])
def test_page_ids_read_as_vectors(where, maxp_pad):
    """A few requests writing many pages each, with prior lengths that put
    the first written column at every offset inside a 16-byte vector: with a
    page-table row length that is a multiple of 4 the ids are read as
    vectors, otherwise one by one.  A bad id in the first, a middle or the
    last written column of a request rejects the call; a bad id in the
    column just before the first written one or just after the last (read in
    the same vector, not written) leaves it valid."""
    q = np.array([37, 5, 0, 61, 19, 44], dtype=np.int64)
    prior = np.array([3, 6, 9, 2, 0, 13], dtype=np.int64)
    ps = 2
    need = (q + prior + ps - 1) // ps
    maxp = int(-(-int(need.max() + 2) // 4) * 4) + maxp_pad
    assert (maxp % 4 == 0) == (maxp_pad == 0)
    inp = W.nra_case(seed=881, q_lens=q, prior_lens=prior, Hq=8, Hkv=1, D=128, page_size=ps, maxp=maxp,
                     kv_fp8=True, k_scale=0.05, v_scale=0.05, q_mode=W.Q_FP8_DYNAMIC)
    b = 3
    sl, ql = int(inp.seq_lens[b]), int(q[b])
    lo, hi = (sl - ql) // ps, (sl - 1) // ps
    assert lo % 4 == 1 and hi - lo > 8 and hi + 1 < maxp
    col = {"first": lo, "middle": (lo + hi) // 2, "last": hi, "before_first": lo - 1, "after_last": hi + 1}[where]
    inp.page_table[b, col] = inp.num_pages + 2
    if where in ("before_first", "after_last"):
        stats = run_and_compare(inp)
        assert (H.oracle_outputs(inp)["flags"] == 0).all()
        print(stats, flush=True)
        return
    dev = H.DeviceNra(inp)
    dev.run()
    torch.cuda.synchronize()
    assert dev.guards_intact()
    gpu = dev.host_outputs()
    assert (gpu["flags"] == -1).all()
    H.check_exact(gpu["k_cache"], inp.k_cache0, "k_cache")
    H.check_exact(gpu["v_cache"], inp.v_cache0, "v_cache")
    H.check_exact(gpu["q_out"], inp.q_out0, "q_out")
    assert (H.oracle_outputs(inp)["flags"] == -1).all()


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_every_written_page_is_checked(seed):
    """Corrupt one randomly chosen page id among those the call writes (many
    requests, several pages each, so the flattened page checks span several
    waves): the call must be rejected.  Then corrupt an id the call does not
    touch: the call must go through."""
    rng = np.random.default_rng(seed)
    B = 300
    q = rng.integers(0, 40, size=B)
    prior = rng.integers(0, 200, size=B)
    base = W.nra_case(seed=seed, q_lens=q, prior_lens=prior, Hq=8, Hkv=1, D=128, page_size=4, maxp=100)
    for trial in range(6):
        inp = W.nra_case(seed=seed, q_lens=q, prior_lens=prior, Hq=8, Hkv=1, D=128, page_size=4, maxp=100)
        b = int(rng.integers(0, B))
        sl, ql = int(inp.seq_lens[b]), int(q[b])
        lo = sl - ql if ql > 0 else sl - 1
        if sl <= 0 or sl <= lo:
            continue
        k = int(rng.integers(lo // 4, (sl - 1) // 4 + 1))
        inp.page_table[b, k] = inp.num_pages + int(rng.integers(0, 5))
        dev = H.DeviceNra(inp)
        dev.run()
        torch.cuda.synchronize()
        gpu = dev.host_outputs()
        assert (gpu["flags"] == -1).all(), (b, k)
        H.check_exact(gpu["k_cache"], inp.k_cache0, "k_cache")
    # an untouched page-table entry may hold anything
    inp = base
    b = int(np.argmax(inp.seq_lens > 8))
    inp.page_table[b, 0] = -7 if (int(inp.seq_lens[b]) - int(q[b])) >= 4 else inp.page_table[b, 0]
    run_and_compare(inp)
