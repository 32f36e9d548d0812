#!/usr/bin/env python3
"""Decode-step benchmark of the MLA latent-KV library on one MI355X.

One step = the five calls of one MLA decode layer on the full-shape workload
(hidden 5120, n_h 128, d_h 128, d_c 512, d_R 64, bf16 cache and weights; 64
sequences at context 4096, 4 KV splits): absorb_q -> append_latent ->
decode_attention -> merge_lse -> absorb_out.  Inputs are seeded synthetic data
resident in HBM before timing; two independent copies of weights and cache
alternate between steps so no step re-reads the previous step's bytes from
the 256 MB last-level cache.

Prints one JSON line: decoded tokens/s (value), latent-cache GB/s, the HBM
roofline of the attention kernel measured with HIP events on the launch
stream, and the fp64 CPU oracle timed on a bounded sample on the host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="full",
                   help="full | lite | long | full-cq (query compression) | full-fp8 (FP8 latent "
                        "pool) | full-pre (chunked prefill: 4 x 256 prompt tokens at context "
                        "4096) (one layer each)")
    p.add_argument("--splits", type=int, default=0, help="KV splits (0 = workload default)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="budget of the oracle timing on the host (0 disables it)")
    p.add_argument("--attention-only", action="store_true",
                   help="time only the attention call (for profiling)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain 1 GiB device copy (calibrates HBM byte counters)")
    return p.parse_args()


def attention_kernel(w) -> str:
    """Name of the attention kernel that runs for workload `w`."""
    return "k_attn_f8mma_h128" if w.cache == "fp8" else "k_attn_mfma_h128"


def attention_traffic(kernel: str, workload: str):
    """HBM bytes per attention launch of `kernel` on `workload` (4 splits) from the
    committed rocprofv3 counter runs (FETCH_SIZE and WRITE_SIZE scaled by a
    plain-copy calibration), or None when there are none or the kernel source
    changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    try:
        rec = json.load(open(path))
        src = open(os.path.join(ROOT, rec["kernel_source"]), "rb").read()
    except (OSError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != rec.get("kernel_source_sha256"):
        return None
    return rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]


def cpu_baseline(w, seconds: float):
    """fp64 oracle (non-absorbed definition) on whole sequences of the same
    workload until `seconds` of host time are spent; tokens/s = sequences/s.
    Prefill workloads: the step's prompt tokens of sequence 0, one by one."""
    if w.chunk:
        return cpu_baseline_prefill(w, seconds)
    import numpy as np

    import oracle as O
    from mla_latent_kv_dkv_amd import inputs as I
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = len(os.sched_getaffinity(0))
    lens = I.seq_lengths(w)
    bt, _ = I.page_table(w, lens)
    wt = {n: I.to_f64(w, I.weight_values(w, n, 0)) for n in w.weight_names}
    cq = dict(w_dq=wt["w_dq"], w_uq=wt["w_uq"]) if w.d_cq else {}
    done, spent, b = 0, 0.0, 0
    while spent < seconds and b < w.batch:
        L = int(lens[b])
        fp8 = w.cache == "fp8"
        rows = I.pool_rows(w, bt, b, L, f32=fp8).astype(np.float64) if fp8 else I.to_f64(
            w, I.pool_rows(w, bt, b, L))
        h = I.to_f64(w, I.tensor_values(w, "h_dec", None, 1.0, 0, start=b * w.hidden,
                                         count=w.hidden))
        t = time.perf_counter()
        rows[L - 1] = O.latent_rows(h[None], wt["w_dkv"], wt["w_kr"], [L - 1], w.rope_base)[0]
        if fp8:     # the cache as the FP8 pool holds it
            rows = np.stack([O.fp8_dequantize_row(*O.fp8_quantize_row(r, w.d_latent)) for r in rows])
        O.mla_decode_step(h, rows, wt.get("w_q"), wt["w_qr"], wt["w_uk"], wt["w_uv"], wt["w_o"],
                          L - 1, w.n_heads, w.d_head, w.d_latent, w.d_rope, w.rope_base, **cq)
        spent += time.perf_counter() - t
        done += 1
        b += 1
    return {"value": done / spent, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {w.batch} sequences (context {int(lens[0])}), non-absorbed "
                      f"fp64 definition" + (" on the FP8-quantized cache" if w.cache == "fp8" else "")
                      + f", {spent:.1f} s of host time"}


def cpu_baseline_prefill(w, seconds: float):
    import numpy as np

    import oracle as O
    from mla_latent_kv_dkv_amd import inputs as I
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = len(os.sched_getaffinity(0))
    lens = I.seq_lengths(w)
    bt, _ = I.page_table(w, lens)
    wt = {n: I.to_f64(w, I.weight_values(w, n, 0)) for n in w.weight_names}
    L = int(lens[0])
    P = L - w.chunk
    rows = I.to_f64(w, I.pool_rows(w, bt, 0, L))
    h = I.to_f64(w, I.tensor_values(w, "h_dec", None, 1.0, 0, start=0, count=w.chunk * w.hidden))
    h = h.reshape(w.chunk, w.hidden)
    done, spent = 0, 0.0
    t = time.perf_counter()
    rows[P:] = O.latent_rows(h, wt["w_dkv"], wt["w_kr"], np.arange(P, L), w.rope_base)
    spent += time.perf_counter() - t
    while spent < seconds and done < w.chunk:
        t = time.perf_counter()
        O.mla_decode_step(h[done], rows[:P + done + 1], wt["w_q"], wt["w_qr"], wt["w_uk"],
                          wt["w_uv"], wt["w_o"], P + done, w.n_heads, w.d_head, w.d_latent,
                          w.d_rope, w.rope_base)
        spent += time.perf_counter() - t
        done += 1
    return {"value": done / spent, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {w.chunk} prompt tokens of sequence 0 (positions {P}..), "
                      f"non-absorbed fp64 definition, {spent:.1f} s of host time"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch
    if args.copy_calibration:
        a = torch.ones(1 << 29, dtype=torch.int16, device="cuda")   # 1 GiB
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": 2 * a.numel() * a.element_size(),
                          "read_bytes": a.numel() * a.element_size(),
                          "write_bytes": b.numel() * b.element_size()}), flush=True)
        return

    import mla_latent_kv_dkv_amd as M
    from mla_latent_kv_dkv_amd import inputs as I
    from mla_latent_kv_dkv_amd.harness import DeviceWorkload
    M.load()
    w = I.WORKLOADS[args.workload]
    S = args.splits or w.num_splits
    sets = [DeviceWorkload(w, layer=l, num_splits=S) for l in (0, 1)]
    torch.cuda.synchronize()
    lens = sets[0].lens
    nq = sets[0].nq                      # the step's tokens (decode: one per sequence)
    attended = (sets[0].q_pos_host.astype(np.int64) + 1).sum()   # cached rows read per launch
    # bytes of one cached row: d_c + d_R values in dtype, or (FP8 pool) d_c codes,
    # d_R bf16 and one fp32 scale
    row_bytes = (w.d_latent + 2 * w.d_rope + 4) if w.cache == "fp8" else w.row * w.elem_bytes
    cache_bytes = int(attended) * row_bytes
    attn_flop = 2 * w.n_heads * int(attended) * (2 * w.d_latent + w.d_rope)
    stream = torch.cuda.current_stream()

    def one(i, ev=None):
        dw = sets[i & 1]
        if args.attention_only:
            dw.attention()
            return
        dw.query_and_append()
        if ev is not None:
            ev[0].record(stream)
        dw.attention()
        if ev is not None:
            ev[1].record(stream)
        dw.merge()
        dw.absorb_out()

    for i in range(args.warmup):
        one(i)
    torch.cuda.synchronize()
    # timed region 1: whole steps
    t0 = time.perf_counter()
    for i in range(args.steps):
        one(i)
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps
    # timed region 2: the attention kernel alone, HIP events on its launch stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        if args.attention_only:
            evs[i][0].record(stream)
            one(i)
            evs[i][1].record(stream)
        else:
            one(i, evs[i])
    torch.cuda.synchronize()
    attn_s = sum(a.elapsed_time(b) for a, b in evs) / args.steps / 1e3
    assert M.mla_device_error() == 0

    B = w.batch
    achieved = cache_bytes / attn_s / 1e9
    tflops = attn_flop / attn_s / 1e12
    if w.chunk:     # prefill: the attention is a dense contraction; its bound is the MFMA rate
        roofline = {"bound": "mfma", "achieved": tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": tflops / BF16_PEAK_TFLOPS, "traffic": None,
                    "kernel": f"{attention_kernel(w)} (mla_prefill_attention)",
                    "algorithmic_flop_per_launch": attn_flop}
    else:
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBPS,
                    "traffic": attention_traffic(attention_kernel(w), w.name) if S == 4 else None,
                    "kernel": attention_kernel(w) + (" (mla_decode_attention_fp8)" if w.cache == "fp8"
                                                     else " (mla_decode_attention)"),
                    "algorithmic_bytes_per_launch": cache_bytes}
    line = {
        "metric": ("MLA chunked-prefill prompt tokens/s, n_h=128 d_c=512 1 GPU" if w.chunk else
                   "MLA decode tokens/s + latent-cache GB/s (% roofline), n_h=128 d_c=512 1 GPU"),
        "value": nq / step_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded, counter-based generator; random-init weights)",
        "config": {"workload": f"{w.name}: one MLA decode layer, hidden {w.hidden}, n_h {w.n_heads}, "
                               f"d_h {w.d_head}, d_c {w.d_latent}, d_R {w.d_rope}, batch {B}, "
                               f"context {int(lens.max())}, {S} KV splits, 64-token pages"
                               + (f", query compression d_c' {w.d_cq}" if w.d_cq else "")
                               + (", FP8 latent pool (e4m3 c^KV + row scale, bf16 k^R)"
                                  if w.cache == "fp8" else "")
                               + (f", prefill of the last {w.chunk} positions of every sequence "
                                  f"({nq} prompt tokens per step)" if w.chunk else ""),
                   "batch": B, "context": int(lens.max()), "num_splits": S},
        "latent_cache_GBps": achieved,
        "attention_us": attn_s * 1e6,
        "attention_mfma_tflops": tflops,
        "attention_mfma_frac": tflops / BF16_PEAK_TFLOPS,
        "roofline": roofline,
    }
    if args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
