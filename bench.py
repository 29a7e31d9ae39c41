#!/usr/bin/env python3
"""Throughput of the fused prepare pass on one MI355X.

One step = one pass of the whole norm-rope-append path over one batch of
each workload the headline metric names:
  * decode, B = 256 requests x 1 token, Hq/Hkv/D 32/8/128, bf16 Q and bf16
    paged cache (page 16) over the full ~262k-page pool, tails cleared;
  * ragged FP8 prefill, 8 requests (~15k tokens), 64/8/128, dynamic
    per-token-head Q scales, E4M3 cache (page 64), tails cleared.
Inputs are seeded and synthetic and already resident in HBM when the timed
region starts.  `value` is the step's algorithmic bytes (qkv read + norm
weights + cos/sin rows + Q write incl. q_scale + cache write incl. tail
zeros) divided by the measured step time, in GB/s (1e9 B/s).

The timed region holds only the K steps' launches (no event markers
between them: on this GPU each marker delays the next kernel by a few
microseconds).  Also reported: tokens/s; each kernel's duration from HIP
events on its launch stream around runs of back-to-back launches of that
kernel (the roofline of the dominant kernel, the prefill launch, uses it);
the same launches timed one at a time after a clean 512 MiB read flush of
L2 and the 256 MB Infinity Cache; and the CPU oracle timed on the host on
the same step.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
       python bench.py --suite      (every configuration and variant, one by one)
       python bench.py --pages-rows (the FlashInfer PR's measured rows, beside its figures)
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of MI355X peak) + tokens/s, decode B=256 and prefill 16k tok"
HBM_PEAK_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--roofline-launches", type=int, default=20)
    ap.add_argument("--kernel-launches", type=int, default=20,
                    help="back-to-back launches per run when timing each kernel alone")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-roofline", action="store_true")
    ap.add_argument("--only", choices=["decode", "prefill", "mla"], default=None,
                    help="time one workload alone (profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 256 MiB copy (counter calibration) and exit")
    ap.add_argument("--suite", action="store_true",
                    help="time every workload (the five configurations and the variant rows) one by one "
                         "and print one JSON object; no headline line")
    ap.add_argument("--suite-only", default=None, help="comma-separated subset of the suite's workloads")
    ap.add_argument("--suite-launches", type=int, default=200,
                    help="clean-cache launches per session (three sessions) of each suite workload")
    ap.add_argument("--pages-rows", action="store_true",
                    help="time the FlashInfer PR's measured rows, rebuilt, after a cache flush each, and "
                         "print them beside that PR's B200 / H100 latencies (context only)")
    return ap.parse_args()


# Latencies in us that the FlashInfer PR (fused QK RMSNorm + NeoX RoPE + FP8
# E4M3 quantize + NHD paged-KV append) prints for these rows in its
# Performance section: B200 (sm_100a) and H100 80GB (sm_90a), each the median
# of a call's kernel activity with a cold L2.  Other hardware: context only.
PAGES_ROW_US = {
    "P_decode_64x8_q1_n2": (3.78, 4.22),
    "P_prefill_64x8_q1_n2": (4.29, 5.22),
    "P_decode_8x1_q1_n2": (3.26, 3.07),
    "E_prefill_64x8_q128": (10.75, 11.81),
    "X_decode_64x8_B1_q1_n2": (3.20, 2.91),
    "X_decode_64x8_B128_q1_n2": (8.00, 10.46),
    "X_decode_64x8_B256_q1_n2": (12.19, 18.98),
    "X_decode_8x1_B256_q1_n2": (4.42, 4.93),
    "X_prefill_64x8_B1_Q1024_q1_n2": (17.54, 20.22),
    "X_prefill_8x1_B1_Q1024_q1_n2": (4.45, 5.19),
}


def run_pages_rows(args, dev):
    """Each of the PR's rows, rebuilt: 20 warm-up launches, then three
    sessions of --suite-launches launches, each after a clean 512 MiB read
    flush (HIP events around each launch)."""
    import torch
    import workloads as W
    stream = torch.cuda.current_stream()
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    table = {}
    for name in W.PAGES_ROWS:
        log(f"pages row: {name}")
        inp = W.pages_row(name, host_caches=False)
        c = Call(inp, dev)
        for _ in range(20):
            c.launch()
        torch.cuda.synchronize()
        sessions = []
        for _ in range(3):
            cold = []
            for _ in range(args.suite_launches):
                flush.sum()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                c.launch()
                e1.record(stream)
                torch.cuda.synchronize()
                cold.append(e0.elapsed_time(e1) * 1e3)
            sessions.append(sorted(cold))
        allc = sorted(x for ses in sessions for x in ses)
        med = percentile(allc, 0.5)
        model = c.bytes - inp.algorithmic_bytes()["norm_weights"]
        b200, h100 = PAGES_ROW_US[name]
        table[name] = {"tokens": inp.T, "bytes_MB": round(model / 1e6, 3),
                       "clean_cache_median_us": round(med, 2),
                       "clean_cache_p10_us": round(percentile(allc, 0.1), 2),
                       "clean_cache_p90_us": round(percentile(allc, 0.9), 2),
                       "clean_cache_session_medians_us": [round(percentile(ses, 0.5), 2) for ses in sessions],
                       "TBps": round(model / med / 1e6, 3),
                       "pages_B200_us": b200, "pages_H100_us": h100}
        log(f"  {table[name]}")
        del c
        torch.cuda.empty_cache()
    print(json.dumps({"pages_rows": table, "launches_per_row": 3 * args.suite_launches}), flush=True)


def suite_workloads():
    """Name -> (constructor, kind) of every timed workload: the five
    configurations, then the variants (partial rotary, 64-dim heads, MLA
    with E4M3 Q, dynamic K/V scales, K/V redirect) at the prefill and MLA
    shapes."""
    import workloads as W
    return {
        "c1_tiny_decode": (W.c1_tiny_decode, "nra"),
        "c2_decode_b256": (W.c2_decode_b256, "nra"),
        "c2_decode_b256_no_tail_clear": (lambda: W.c2_decode_b256(zero_tail=False), "nra"),
        "c3_prefill_fp8": (W.c3_prefill_fp8, "nra"),
        "c4_strided_d256": (W.c4_strided_d256, "nra"),
        "c5_mla": (W.c5_mla, "mla"),
        "prefill_d64_gqa_64_8": (lambda: W.c3_prefill_fp8(D=64, name="prefill_d64"), "nra"),
        "prefill_rotary_64_of_128": (lambda: W.c3_prefill_fp8(rotary_dim=64, name="prefill_r64"), "nra"),
        "prefill_nope_layer": (lambda: W.c3_prefill_fp8(rotary_dim=0, name="prefill_r0"), "nra"),
        "prefill_rotary_96_of_128": (lambda: W.c3_prefill_fp8(rotary_dim=96, name="prefill_r96"), "nra"),
        "prefill_d64_rotary_32_of_64": (lambda: W.c3_prefill_fp8(D=64, rotary_dim=32, name="prefill_d64_r32"), "nra"),
        "c5_mla_q_fp8_dynamic": (lambda: W.c5_mla(q_mode=W.Q_FP8_DYNAMIC), "mla"),
        "c5_mla_q_fp8_static": (lambda: W.c5_mla(q_mode=W.Q_FP8_STATIC), "mla"),
        "prefill_kv_token_scales": (lambda: W.c3_prefill_fp8(kv_scale_mode=W.KV_SCALE_TOKEN), "nra"),
        "prefill_kv_group64_scales": (lambda: W.c3_prefill_fp8(kv_scale_mode=W.KV_SCALE_GROUP,
                                                               kv_group_size=64), "nra"),
        "prefill_kv_redirect": (lambda: W.c3_prefill_fp8(kv_redirect=True), "nra"),
        "decode_b256_kv_redirect": (lambda: W.c2_decode_b256(kv_redirect=True), "nra"),
    }


def percentile(sorted_vals, q):
    """q-quantile (0..1) of an ascending list, by linear interpolation."""
    if not sorted_vals:
        return None
    x = q * (len(sorted_vals) - 1)
    i = int(x)
    j = min(i + 1, len(sorted_vals) - 1)
    return sorted_vals[i] + (sorted_vals[j] - sorted_vals[i]) * (x - i)


def run_suite(args, dev):
    """Each workload alone: 20 warm-up launches; three runs of 20
    back-to-back launches (events on the launch stream around each run);
    then three sessions of --suite-launches launches, each after a clean
    512 MiB read flush of L2 and the Infinity Cache (events around each
    launch): median, p10 and p90 over all of them and each session's median."""
    import torch
    table = {}
    names = list(suite_workloads())
    if args.suite_only:
        names = [n for n in args.suite_only.split(",") if n]
    stream = torch.cuda.current_stream()
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    n_clean = args.suite_launches
    for name in names:
        make, kind = suite_workloads()[name]
        log(f"suite: {name}")
        inp = make()
        c = MlaCall(inp, dev) if kind == "mla" else Call(inp, dev)
        for _ in range(20):
            c.launch()
        torch.cuda.synchronize()
        runs = []
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(20):
                c.launch()
            e1.record(stream)
            torch.cuda.synchronize()
            runs.append(e0.elapsed_time(e1) * 1e3 / 20)
        sessions = []
        for _ in range(3):
            cold = []
            for _ in range(n_clean):
                flush.sum()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                c.launch()
                e1.record(stream)
                torch.cuda.synchronize()
                cold.append(e0.elapsed_time(e1) * 1e3)
            sessions.append(sorted(cold))
        allc = sorted(x for ses in sessions for x in ses)
        avg = sorted(runs)[1]
        med = percentile(allc, 0.5)
        table[name] = {"tokens": inp.T, "algorithmic_bytes": c.bytes, "avg_us": round(avg, 2),
                       "back_to_back_runs_us": [round(r, 2) for r in runs],
                       "clean_cache_median_us": round(med, 2),
                       "clean_cache_p10_us": round(percentile(allc, 0.1), 2),
                       "clean_cache_p90_us": round(percentile(allc, 0.9), 2),
                       "clean_cache_session_medians_us": [round(percentile(ses, 0.5), 2) for ses in sessions],
                       "clean_cache_launches": len(allc),
                       "GBps": round(c.bytes / (avg * 1e-6) / 1e9, 1),
                       "clean_cache_GBps": round(c.bytes / (med * 1e-6) / 1e9, 1),
                       "clean_cache_pct_of_peak": round(100 * c.bytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 1),
                       "Mtok_per_s_clean": round(inp.T / med, 2)}
        log(f"  {table[name]}")
        del c
        torch.cuda.empty_cache()
    print(json.dumps({"suite": table, "peak_GBps": HBM_PEAK_GBS}), flush=True)


class Call:
    """Device-resident inputs and outputs of one norm-rope-append call."""

    def __init__(self, inp, dev):
        import numpy as np
        import torch
        import paged_kv_cache_token_amd as qp
        import workloads as W
        self.inp = inp

        def up(a, dt):
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev).view(dt)

        def seeded(nbytes, seed, dt, shape):
            g = torch.Generator(device=dev)
            g.manual_seed(seed)
            return torch.empty(nbytes, dtype=torch.uint8, device=dev).random_(0, 256, generator=g).view(dt).view(shape)

        cdt = torch.uint8 if inp.kv_fp8 else torch.int16
        cbytes = int(np.prod(inp.cache_shape)) * inp.kv_elt
        self.qkv = up(inp.qkv, torch.int16)
        self.k_cache = seeded(cbytes, inp.cache_seed, cdt, inp.cache_shape)
        self.v_cache = seeded(cbytes, inp.cache_seed + 1, cdt, inp.cache_shape)
        qdt = torch.int16 if inp.q_mode == W.Q_BF16 else torch.uint8
        self.q_out = self.qkv if inp.q_in_place else up(inp.q_out0, qdt)
        k_out = None
        if inp.k_in_place:
            k_out = self.qkv.view(-1)[inp.Hq * inp.D:].as_strided((inp.T, inp.Hkv * inp.D),
                                                                  (inp.qkv_row_stride, 1))
        self.q_scale = None if inp.q_scale0 is None else up(inp.q_scale0, torch.float32)
        self.flags = up(inp.flags0, torch.int32)
        redirect = {}
        if inp.kv_redirect:
            redirect = dict(out_k=up(inp.out_k0, cdt), out_v=up(inp.out_v0, cdt))
        scales = {}
        if inp.kv_scale_mode:
            scales = dict(k_scale_out=up(inp.k_scale_out0, torch.float32),
                          v_scale_out=up(inp.v_scale_out0, torch.float32))
        self.extra = dict(redirect, **scales)
        sc = lambda x: torch.tensor([x], dtype=torch.float32, device=dev)  # noqa: E731
        self.kw = dict(
            qkv=self.qkv, num_q_heads=inp.Hq, num_kv_heads=inp.Hkv, head_dim=inp.D, norm=inp.norm,
            eps=inp.eps, q_norm_weight=up(inp.q_norm_weight, torch.float32),
            k_norm_weight=up(inp.k_norm_weight, torch.float32), rope=inp.rope,
            cos_sin_cache=up(inp.cos_sin, torch.float32), positions=up(inp.positions, torch.int64),
            q_indptr=up(inp.q_indptr, torch.int32), seq_lens=up(inp.seq_lens, torch.int32),
            page_table=up(inp.page_table, torch.int32), k_cache=self.k_cache, v_cache=self.v_cache,
            kv_dtype=qp.FP8_E4M3 if inp.kv_fp8 else qp.BF16, k_scale=sc(inp.k_scale), v_scale=sc(inp.v_scale),
            zero_tail=1 if inp.zero_tail else 0, q_out=self.q_out, q_out_row_stride=inp.qkv_row_stride if inp.q_in_place else inp.Hq * inp.D,
            q_mode=inp.q_mode, k_out=k_out, k_out_row_stride=inp.qkv_row_stride, qkv_row_stride=inp.qkv_row_stride,
            q_scale_inv=sc(inp.q_scale_inv), num_tokens=inp.T,
            q_scale=self.q_scale,
            q_scale_layout=qp.QSCALE_REQ_HEAD_PADDED if inp.q_scale_padded else qp.QSCALE_TOKEN_HEAD,
            max_seqlen=inp.max_seqlen, upper_max=inp.upper_max, flags=self.flags, rotary_dim=inp.rot,
            kv_scale_mode=inp.kv_scale_mode, kv_group_size=inp.kv_group_size, **self.extra)
        self.params = qp.norm_rope_append_params(**self.kw)
        self.params.struct_size = ctypes.sizeof(self.params)
        self._ref = ctypes.byref(self.params)
        self._fn = qp.lib().qkprep_norm_rope_append
        self._stream = torch.cuda.current_stream().cuda_stream
        self.bytes = inp.algorithmic_bytes()["total"]

    def launch(self):
        st = self._fn(self._ref, self._stream)
        if st != 0:
            import paged_kv_cache_token_amd as qp
            raise qp.QkprepError(st)


class MlaCall:
    def __init__(self, inp, dev):
        import numpy as np
        import torch
        import paged_kv_cache_token_amd as qp
        self.inp = inp

        def up(a, dt):
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev).view(dt)
        self.q = up(inp.q, torch.int16)
        self.cache = up(inp.kv_cache0, torch.uint8)
        sc = lambda x: torch.tensor([x], dtype=torch.float32, device=dev)  # noqa: E731
        self.q_out = None if inp.q_out0 is None else up(inp.q_out0, torch.uint8)
        self.q_scale = None if inp.q_scale0 is None else up(inp.q_scale0, torch.float32)
        # (the params struct keeps every tensor below alive)
        self.params = qp.mla_params(
            q=self.q, kv_c=up(inp.kv_c, torch.int16), k_pe=up(inp.k_pe, torch.int16),
            cos_sin_cache=up(inp.cos_sin, torch.float32), positions=up(inp.positions, torch.int64),
            slot_mapping=up(inp.slot_mapping, torch.int64), kv_cache=self.cache, num_q_heads=inp.H,
            nope_dim=inp.nope_dim, kv_scale=sc(inp.kv_scale), q_mode=inp.q_mode, q_out=self.q_out,
            q_scale=self.q_scale, q_scale_inv=sc(inp.q_scale_inv), upper_max=inp.upper_max)
        self.params.struct_size = ctypes.sizeof(self.params)
        self._ref = ctypes.byref(self.params)
        self._fn = qp.lib().qkprep_mla_concat_rope_append
        self._stream = torch.cuda.current_stream().cuda_stream
        self.bytes = inp.algorithmic_bytes()["total"]

    def launch(self):
        st = self._fn(self._ref, self._stream)
        if st != 0:
            import paged_kv_cache_token_amd as qp
            raise qp.QkprepError(st)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("nra_kernel.hip", "qkprep_device.h", "qkprep_internal.h", "qkprep_api.hip"):
        with open(os.path.join(ROOT, "paged_kv_cache_token_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel_hash: str):
    """HBM bytes per launch of the prefill kernel from the committed rocprofv3
    counter summary, valid only for the kernel source it was taken on."""
    path = os.path.join(ROOT, "profiles", "nra_prefill_fp8_c3_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_hash") != kernel_hash:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_cpu():
    """CPU model name and logical core count of the host."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count()


def cpu_baseline(c2, c3):
    """The oracle (single-threaded C, fp64) on the same step: the decode call
    on its touched pages and the full prefill call.  The step is timed three
    times (once if a run takes over 10 s) and the median reported."""
    runs = []
    while True:
        t, nbytes, ntok = cpu_step(c2, c3)
        runs.append(t)
        if len(runs) == 3 or t > 10.0:
            break
    t_total = sorted(runs)[len(runs) // 2]
    model, ncpu = host_cpu()
    return {"value": round(nbytes / t_total / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "tokens_per_s": round(ntok / t_total, 1), "seconds": round(t_total, 3),
            "runs_s": [round(r, 3) for r in runs], "host_cpu": model, "host_logical_cores": ncpu,
            "sample": "one full step (decode B=256 on its touched pages + the ragged FP8 prefill call), "
                      "single-threaded C oracle in fp64, median of the runs"}


def cpu_step(c2, c3):
    import numpy as np
    import oracle
    t_total = 0.0
    nbytes = 0
    ntok = 0
    for call in (c2, c3):
        inp = call.inp
        if inp.k_cache0 is None:
            # decode pool is 17 GB: run the oracle on the touched pages only
            import copy
            import torch
            pages = inp.touched_pages()
            pidx = torch.from_numpy(pages).to(call.k_cache.device)
            k0 = call.k_cache[pidx].cpu().numpy().view(np.uint16)
            v0 = call.v_cache[pidx].cpu().numpy().view(np.uint16)
            c = copy.copy(inp)
            remap = np.full(inp.num_pages, -1, np.int64)
            remap[pages] = np.arange(len(pages))
            pt = inp.page_table.astype(np.int64)
            c.page_table = np.where(pt >= 0, remap[np.clip(pt, 0, None)], -1).astype(np.int32)
            c.num_pages = len(pages)
            c.k_cache0, c.v_cache0 = k0, v0
            inp = c
        out = {"qkv": inp.qkv.copy(), "k_cache": inp.k_cache0.copy(), "v_cache": inp.v_cache0.copy(),
               "q_out": inp.q_out0.copy(), "q_scale": None if inp.q_scale0 is None else inp.q_scale0.copy(),
               "flags": inp.flags0.copy()}
        t0 = time.perf_counter()
        oracle.norm_rope_append(inp, out)
        t_total += time.perf_counter() - t0
        nbytes += call.bytes
        ntok += inp.T
    return t_total, nbytes, ntok


def copy_calibration(dev):
    """A plain copy of known size (256 MiB), for scaling the FETCH_SIZE /
    WRITE_SIZE counters: run under rocprofv3 --pmc, each dispatch must read
    and write 262144 KiB."""
    import torch
    n = 256 << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    for _ in range(3):
        flush.sum()
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "dispatches": 3}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch
    import workloads as W
    import paged_kv_cache_token_amd as qp  # noqa: F401  (fails loudly if libqkprep.so is missing)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        copy_calibration(dev)
        return
    if args.suite:
        run_suite(args, dev)
        return
    if args.pages_rows:
        run_pages_rows(args, dev)
        return

    log("generating decode B=256")
    c2 = Call(W.c2_decode_b256(), dev)
    log("generating ragged FP8 prefill")
    c3 = Call(W.c3_prefill_fp8(), dev)
    calls = {"decode": c2, "prefill": c3}
    if args.only == "mla":
        calls = {"mla": MlaCall(W.c5_mla(), dev)}
    elif args.only:
        calls = {args.only: calls[args.only]}
    names = list(calls)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        for c in calls.values():
            c.launch()
    torch.cuda.synchronize()
    # the timed region: K whole steps, launches only (an event marker between
    # launches would itself put a gap of a few microseconds before the next
    # kernel), bracketed by synchronisations and one event pair
    log(f"timing {args.steps} steps")
    e_start = torch.cuda.Event(enable_timing=True)
    e_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record(stream)
    for k in range(args.steps):
        for name in names:
            calls[name].launch()
    e_stop.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    ms_events = e_start.elapsed_time(e_stop) / args.steps
    step_bytes = sum(c.bytes for c in calls.values())
    step_tokens = sum(c.inp.T for c in calls.values())
    value = step_bytes / (ms * 1e-3) / 1e9

    # per-kernel duration: HIP events on the launch stream around a run of
    # back-to-back launches of that kernel (no marker between them)
    breakdown = {}
    for name in names:
        c = calls[name]
        runs = []
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.kernel_launches):
                c.launch()
            e1.record(stream)
            torch.cuda.synchronize()
            runs.append(e0.elapsed_time(e1) * 1e3 / args.kernel_launches)
        avg = sorted(runs)[1]
        breakdown[name] = {"tokens": c.inp.T, "algorithmic_bytes": c.bytes, "avg_us": round(avg, 2),
                           "runs_us": [round(r, 2) for r in runs],
                           "GBps": round(c.bytes / (avg * 1e-6) / 1e9, 1),
                           "Mtok_per_s": round(c.inp.T / avg, 2)}
    # the same launches one at a time after a clean flush (512 MiB read)
    if not args.no_roofline:
        flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        for name in names:
            c = calls[name]
            durs = []
            for _ in range(args.roofline_launches):
                flush.sum()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                c.launch()
                e1.record(stream)
                torch.cuda.synchronize()
                durs.append(e0.elapsed_time(e1) * 1e3)
            durs.sort()
            med = percentile(durs, 0.5)
            breakdown[name]["clean_cache_median_us"] = round(med, 2)
            breakdown[name]["clean_cache_p10_us"] = round(percentile(durs, 0.1), 2)
            breakdown[name]["clean_cache_p90_us"] = round(percentile(durs, 0.9), 2)
            breakdown[name]["clean_cache_GBps"] = round(c.bytes / (med * 1e-6) / 1e9, 1)
        del flush
    dominant = max(names, key=lambda n: breakdown[n]["avg_us"])
    log(f"step {ms:.4f} ms, {value:.1f} GB/s; {breakdown}")

    b = breakdown[dominant]
    khash = kernel_source_hash()
    traffic = recorded_traffic(khash) if dominant == "prefill" else None
    roofline = {"bound": "hbm", "kernel": dominant, "achieved": b["GBps"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(b["GBps"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": b["algorithmic_bytes"], "avg_launch_us": b["avg_us"],
                "kernel_source_hash": khash}

    cpu = None
    if not args.no_cpu_baseline and args.only is None:
        log("timing the CPU oracle on the same step")
        cpu = cpu_baseline(c2, c3)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "ms_per_step_events": round(ms_events, 5),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "tokens_per_s": round(step_tokens / (ms * 1e-3), 1),
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "config": {"workload": "decode B=256 (32/8/128 bf16, page 16, full pool) + ragged FP8 prefill "
                               f"(8 req, T={c3.inp.T}, 64/8/128, page 64)",
                   "step_tokens": step_tokens, "step_algorithmic_bytes": step_bytes, "calls": names},
        "roofline": roofline, "cpu_baseline": cpu, "breakdown": breakdown,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
