"""The byte accounting behind every reported GB/s figure (CPU only).

``workloads.*.algorithmic_bytes()`` is the numerator of every bandwidth in
the benchmark.  It is checked here against the per-token closed forms of
the traffic each call must move (qkv head rows read, norm weights, the
token's cos/sin row, Q and its scale written, K/V appended, tail rows
zeroed), and its tail-row count against the rows the oracle actually
rewrites, found by comparing the caches before and after the oracle runs.
"""
import os
import sys

import numpy as np
import pytest

import oracle
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (percentile helper only; nothing here touches a GPU)


def _tail_rows_by_formula(inp):
    rows = 0
    for b in range(inp.B):
        sl = int(inp.seq_lens[b])
        if sl > 0:
            rows += inp.page_size - 1 - (sl - 1) % inp.page_size
    return rows


@pytest.mark.parametrize("name,per_token", [
    # qkv rows read + cos/sin row + Q written (+ its fp32 scale) + K and V appended
    ("c1", 10 * 256 + 512 + 8 * 256 + 2 * 256),
    ("c2", 48 * 256 + 512 + 32 * 256 + 16 * 256),
    ("c3", 80 * 256 + 512 + 64 * 128 + 64 * 4 + 16 * 128),
    # Q and K written back in place (bf16): 16 + 4 rows of 512 B
    ("c4", 24 * 512 + 1024 + 16 * 512 + 8 * 512 + 4 * 512),
])
def test_norm_rope_append_bytes_per_token(name, per_token):
    inp = W.CONFIGS[name](**({} if name == "c5" else {"host_caches": False}))
    d = inp.algorithmic_bytes()
    weights = 2 * inp.D * 4
    tails = _tail_rows_by_formula(inp) * 2 * inp.Hkv * inp.D * (1 if inp.kv_fp8 else 2)
    assert d["total"] == inp.T * per_token + weights + tails
    assert d["tail_zero"] == tails


def test_variant_bytes():
    c3 = W.c3_prefill_fp8(host_caches=False)
    base = c3.algorithmic_bytes()
    # rotary over 64 of 128 dims reads half a cos/sin row; rotary 0 reads none
    assert W.c3_prefill_fp8(rotary_dim=64, host_caches=False).algorithmic_bytes()["total"] == base["total"] - c3.T * 256
    assert W.c3_prefill_fp8(rotary_dim=0, host_caches=False).algorithmic_bytes()["total"] == base["total"] - c3.T * 512
    assert W.c3_prefill_fp8(rotary_dim=96, host_caches=False).algorithmic_bytes()["total"] == base["total"] - c3.T * 128
    # K/V redirect: no tail rows
    red = W.c3_prefill_fp8(kv_redirect=True, host_caches=False).algorithmic_bytes()
    assert red["tail_zero"] == 0 and red["total"] == base["total"] - base["tail_zero"]
    # per-token K/V scales: one fp32 per (row, kv head) for K and V, tail rows included
    tok = W.c3_prefill_fp8(kv_scale_mode=W.KV_SCALE_TOKEN, host_caches=False).algorithmic_bytes()
    tail_rows = _tail_rows_by_formula(c3)
    assert tok["kv_scales"] == (c3.T + tail_rows) * 2 * 8 * 4
    # no tail clear on the decode
    c2 = W.c2_decode_b256()
    c2n = W.c2_decode_b256(zero_tail=False)
    assert c2n.algorithmic_bytes()["total"] == c2.algorithmic_bytes()["total"] - c2.algorithmic_bytes()["tail_zero"]
    assert c2n.algorithmic_bytes()["total"] == 256 * (48 * 256 + 512 + 32 * 256 + 16 * 256) + 2 * 128 * 4


def test_mla_bytes_per_token():
    c5 = W.c5_mla()
    assert c5.algorithmic_bytes()["total"] == c5.T * (2 * 128 * 64 * 2 + 512 * 2 + 64 * 2 + 64 * 4 + 576)
    q8 = W.c5_mla(q_mode=W.Q_FP8_DYNAMIC)
    # whole head rows read (bf16) and written (E4M3), plus one scale per token
    assert q8.algorithmic_bytes()["total"] == q8.T * (128 * 192 * 2 + 128 * 192 + 4 + 512 * 2 + 64 * 2 + 64 * 4 + 576)


@pytest.mark.parametrize("seed,page_size,kv_fp8", [(21, 16, False), (22, 8, True), (23, 32, False)])
def test_tail_rows_match_the_rows_the_oracle_rewrites(seed, page_size, kv_fp8):
    """Rows of the caches the oracle changes = one per appended token + the
    counted tail rows (the caches start as random bytes, so a rewritten
    row differs from its start with overwhelming probability)."""
    rng = np.random.default_rng(seed)
    B = 12
    q = rng.integers(0, 9, size=B)
    prior = rng.integers(0, 3 * page_size, size=B)
    inp = W.nra_case(seed=seed, q_lens=q, prior_lens=prior, Hq=4, Hkv=2, D=64, page_size=page_size,
                     kv_fp8=kv_fp8, k_scale=0.5, v_scale=0.5)
    out = {"qkv": inp.qkv.copy(), "k_cache": inp.k_cache0.copy(), "v_cache": inp.v_cache0.copy(),
           "q_out": inp.q_out0.copy(), "q_scale": None, "flags": inp.flags0.copy()}
    oracle.norm_rope_append(inp, out)
    assert (out["flags"] == 0).all()
    elt_rows = inp.k_cache0.reshape(inp.k_cache0.shape[0] * page_size, -1)
    new_rows = out["k_cache"].reshape(elt_rows.shape)
    changed = int((elt_rows != new_rows).any(axis=1).sum())
    d = inp.algorithmic_bytes()
    row_bytes = inp.Hkv * inp.D * (1 if kv_fp8 else 2)
    assert changed == inp.T + d["tail_zero"] // (2 * row_bytes)
    assert d["kv_append"] == inp.T * 2 * row_bytes


def test_percentile_helper():
    v = [float(x) for x in range(1, 11)]
    assert bench.percentile(v, 0.5) == 5.5
    assert bench.percentile(v, 0.0) == 1.0 and bench.percentile(v, 1.0) == 10.0
    assert bench.percentile(v, 0.1) == pytest.approx(1.9)
    assert bench.percentile([3.0], 0.9) == 3.0
    assert bench.percentile([], 0.5) is None


@pytest.mark.parametrize("name", list(W.PAGES_ROWS))
def test_pages_rows_reproduce_the_printed_bytes(name):
    """The FlashInfer PR's performance tables print each row's bytes (MB,
    1e6 B, without the norm weights); the rows rebuilt from their names move
    exactly that many, so the timings set beside them are for the same
    traffic."""
    inp = W.pages_row(name, host_caches=False)
    d = inp.algorithmic_bytes()
    assert round((d["total"] - d["norm_weights"]) / 1e6, 3) == W.PAGES_ROWS[name][-1]
    assert d["norm_weights"] == 2 * 128 * 4
