#!/usr/bin/env python3
"""Benchmark of the exact tiled attention hot path on one MI355X.

One step = one pass of both halves of the hot path over resident synthetic
inputs:
  * attn_fwd on the causal GQA prefill workload (B=1, 12 query heads sharing
    2 K/V heads, T=8192, d=128, bf16, scale 1/sqrt(128)), and
  * attn_paged_decode on the paged-KV decode workload (64 sequences, one
    query token each, 12/2 heads, d=128, bf16, 16-token blocks, lengths
    uniform in [512, 8192], blocks placed by a seeded permutation).

`value` is the prefill's attention-forward throughput in TFLOP/s
(algorithmic flops 4*d*Hq*T(T+1)/2 over the average kernel time measured
with HIP events on the launch stream); the decode's GB/s (algorithmic bytes
over its average time) is reported beside it.  The steps either side of
decode are timed after the main loop, on the same 64-sequence cache: the
chunked prefill of 256 new rows per sequence (attn_paged_prefill) and the
append of those rows' keys and values (attn_kv_append); and the backward
pass (attn_bwd) of the prefill workload; and the memory-bound fusions of a
decoder layer of the same attention shape (8192 tokens, width 1536,
intermediate 8960): residual add + RMSNorm and the SwiGLU activation.
Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]

With `--configs NAME[,NAME...]` (or `--configs all`) it instead times
attn_fwd alone on each named dense workload (the ViT-B/16 shapes, the GQA and
the long MHA causal prefills) and prints one JSON line per workload: TFLOP/s
against the MFMA peak of its dtype and algorithmic GB/s against the HBM peak.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s & % bf16 MFMA peak; paged decode GB/s & % HBM peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 (matrix and vector alike)


def prefill_flops(cfg) -> float:
    pairs = cfg.N * (cfg.N + 1) / 2 if cfg.causal else cfg.N * cfg.N
    return 4.0 * cfg.d * cfg.B * cfg.Hq * pairs


def prefill_bytes(cfg) -> float:
    es = 2 if cfg.dtype == "bf16" else 4
    q = cfg.B * cfg.Hq * cfg.N * cfg.d * es
    kv = cfg.B * cfg.Hkv * cfg.N * cfg.d * es
    return q + 2 * kv + q + cfg.B * cfg.Hq * cfg.N * 4


def decode_bytes(p, cfg) -> float:
    """K and V of every cached position read once per kv head, plus q, o,
    lse, the used block-table entries and the lengths."""
    ctx = p["ctx_lens"].numpy().astype(np.int64)
    kv = int(ctx.sum()) * cfg.Hkv * cfg.d * 2 * 2
    qo = 2 * cfg.S * cfg.Hq * cfg.d * 2
    table = int(((ctx + cfg.block_size - 1) // cfg.block_size).sum()) * 4
    return kv + qo + cfg.S * cfg.Hq * 4 + table + cfg.S * 4


def decode_flops(p, cfg) -> float:
    return 4.0 * cfg.Hq * cfg.d * float(p["ctx_lens"].numpy().astype(np.int64).sum())


def chunked_flops(p, cfg) -> float:
    """Row t of a sequence with n new rows and length L attends L - n + t + 1 keys."""
    ctx = p["ctx_lens"].numpy().astype(np.int64)
    n = p["new_lens"].numpy().astype(np.int64)
    pairs = float((n * (ctx - n) + n * (n + 1) // 2).sum())
    return 4.0 * cfg.Hq * cfg.d * pairs


def chunked_bytes(p, cfg) -> float:
    """K and V of every cached position once per kv head, the new rows' q,
    o and lse, the used table entries, the lengths and the row offsets."""
    ctx = p["ctx_lens"].numpy().astype(np.int64)
    T = int(p["starts"][-1])
    kv = int(ctx.sum()) * cfg.Hkv * cfg.d * 2 * 2
    table = int(((ctx + cfg.block_size - 1) // cfg.block_size).sum()) * 4
    return kv + 2 * T * cfg.Hq * cfg.d * 2 + T * cfg.Hq * 4 + table + cfg.S * 4 + (cfg.S + 1) * 4


def append_bytes(p, cfg) -> float:
    """The new rows' K and V read once and written once, plus the lengths,
    row offsets and the table entries they land in."""
    T = int(p["starts"][-1])
    rows = 2 * T * cfg.Hkv * cfg.d * 2
    ctx = p["ctx_lens"].numpy().astype(np.int64)
    n = p["new_lens"].numpy().astype(np.int64)
    blocks = int(((ctx + cfg.block_size - 1) // cfg.block_size
                  - (ctx - n) // cfg.block_size).sum())
    return 2 * rows + cfg.S * 4 + (cfg.S + 1) * 4 + blocks * 4


def profiled_traffic(profile: str, sources) -> float | None:
    """HBM bytes per launch recorded in profiles/<profile>.md (FETCH_SIZE and
    WRITE_SIZE counter passes, scaled by the same counters' reading on a plain
    streaming kernel of known size), or None when that summary is missing or
    was taken on kernel sources other than the current ones."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile + ".md")
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in sources:
        src = os.path.join(ROOT, "exact_tiled_self_amd", "csrc", f)
        if not os.path.exists(src):
            return None
        h.update(open(src, "rb").read())
    traffic, digest = None, None
    for line in open(path):
        if line.startswith("traffic_bytes_per_launch:"):
            traffic = float(line.split(":")[1])
        elif line.startswith("source_sha256_16:"):
            digest = line.split(":")[1].split()[0]
    return traffic if digest == h.hexdigest()[:16] else None


def host_cores() -> int:
    return len(os.sched_getaffinity(0))


# Worker threads for the oracle: the host cores this process may use, capped
# at 16, the CPU share a one-GPU machine gives a job (its affinity mask can show
# the whole machine).
CPU_WORKER_CAP = 16


def cpu_workers(requested: int = 0) -> int:
    return requested or min(CPU_WORKER_CAP, host_cores())


def cpu_baseline(cfg, q, k, v, workers, min_seconds=10.0, max_reps=100, heads=None):
    """The fp64 oracle, as it stands, on a dense workload's host copy.

    The sample is the whole forward pass, or the query heads `heads` of it
    (every row of each: the oracle's cost per head is the same for all heads),
    repeated until about `min_seconds` have elapsed; the rate is the sample's
    algorithmic flops over its time.
    """
    from oracle import exact as OA
    if heads is not None:
        G = cfg.Hq // cfg.Hkv
        kvh = sorted({h // G for h in heads})
        q = q[:, list(heads)]
        k, v = k[:, kvh], v[:, kvh]
        if len(kvh) * G != len(heads):
            raise ValueError("a head sample must be whole GQA groups")
    qn, kn, vn = (t.to("cpu").double().numpy() for t in (q, k, v))
    times = []
    while len(times) < max_reps and sum(times) < min_seconds:
        t0 = time.perf_counter()
        OA.attention(qn, kn, vn, cfg.scale, cfg.causal, workers=workers)
        times.append(time.perf_counter() - t0)
    dt = float(np.mean(times))
    nh = cfg.Hq if heads is None else len(heads)
    flops = prefill_flops(cfg) * nh / cfg.Hq
    what = (f"the full {cfg.name} forward" if heads is None
            else f"query heads {list(heads)} (all {cfg.N} rows each) of the {cfg.name} forward")
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": workers,
            "host_cores": host_cores(), "worker_cap": CPU_WORKER_CAP,
            "kind": "oracle", "seconds_per_pass": round(dt, 4), "passes": len(times),
            "sample": f"{what} (B={cfg.B}, Hq={cfg.Hq}, Hkv={cfg.Hkv}, N={cfg.N}, d={cfg.d}, "
                      f"{'causal' if cfg.causal else 'non-causal'}, {cfg.dtype}), float64 numpy oracle "
                      f"on {workers} threads"}


def plain_copy(torch, dev, mib):
    """A plain streaming kernel of known size (reads and writes `mib` MiB once
    each): torch's elementwise negation, not the runtime's blit copy."""
    src = torch.ones((mib << 20) // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def dense_kernel_name(cfg) -> str:
    if cfg.dtype == "f32":
        if cfg.d == 64:
            return f"prefill_f32_mfma16_kernel<{'causal' if cfg.causal else 'non-causal'}>"
        return f"prefill_f32_kernel<{cfg.d}, {'causal' if cfg.causal else 'non-causal'}>"
    if cfg.d == 128 and cfg.causal:
        return f"prefill_sp_kernel<{cfg.d}, causal>"
    if cfg.d == 64 and cfg.N <= 208 and cfg.B * cfg.Hq >= 256:
        return (f"prefill_short_kernel<{'causal' if cfg.causal else 'non-causal'}, "
                f"{'pipelined' if cfg.N > 192 else 'staged whole'}>")
    return (f"prefill_bf16_kernel<{cfg.d}, {'causal' if cfg.causal else 'non-causal'}, "
            f"{32 if cfg.d == 64 else 64}-key tiles>")


# The committed rocprofv3 summary of each dense workload (profiles/<name>.md)
# and the sources its digest covers.
DENSE_PROFILES = {
    "vit_b16_fp32": ("prefill_f32_d64_vit_b16_b1_n196", ["prefill_f32.hip", "common.h", "internal.h"]),
    "vit_b16_bf16": ("prefill_bf16_d64_vit_b16_b64_n196",
                     ["prefill_bf16.hip", "prefill_tile.h", "common.h", "internal.h"]),
    "vit_b16_bf16_n577": ("prefill_bf16_d64_vit_b16_b64_n577",
                          ["prefill_bf16.hip", "prefill_tile.h", "common.h", "internal.h"]),
    "gqa_causal_t8192": ("prefill_bf16_d128_causal_gqa_t8192",
                         ["prefill_bf16.hip", "prefill_tile.h", "common.h", "internal.h"]),
    "mha_causal_t32768": ("prefill_bf16_d128_causal_mha_t32768",
                          ["prefill_bf16.hip", "prefill_tile.h", "common.h", "internal.h"]),
}


def time_dense(torch, dev, stream, cfg, steps, warmup):
    """attn_fwd alone on one dense workload, inputs resident: HIP events on
    the launch stream around every call.  Returns the timing record."""
    from exact_tiled_self_amd import attn_fwd
    from exact_tiled_self_amd.inputs import dense_inputs

    q, k, v = (t.to(dev) for t in dense_inputs(cfg))
    o = torch.empty_like(q)
    lse = torch.empty(cfg.B, cfg.Hq, cfg.N, dtype=torch.float32, device=dev)

    def fwd():
        attn_fwd(q, k, v, scale=cfg.scale, causal=cfg.causal, o=o, lse=lse, stream=stream)

    for _ in range(warmup):
        fwd()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    e[0].record(stream)
    for i in range(steps):
        fwd()
        e[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = [e[i].elapsed_time(e[i + 1]) for i in range(steps)]
    del q, k, v, o, lse
    avg_s = float(np.mean(ms)) / 1e3
    fl, by = prefill_flops(cfg), prefill_bytes(cfg)
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    tf, gb = fl / avg_s / 1e12, by / avg_s / 1e9
    # the roof of this workload: its dtype's matrix peak, or the HBM peak times
    # its arithmetic intensity when that is lower
    roof = min(peak, fl / by * PEAK_HBM_GBPS / 1e3)
    return {
        "workload": cfg.name, "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "N": cfg.N, "d": cfg.d,
        "dtype": cfg.dtype, "causal": cfg.causal, "steps": steps, "warmup": warmup,
        "avg_us": round(avg_s * 1e6, 2), "median_us": round(float(np.median(ms)) * 1e3, 2),
        "min_us": round(min(ms) * 1e3, 2),
        "TFLOP/s": round(tf, 2), "frac_mfma": round(tf / peak, 4), "mfma_peak_TFLOP/s": peak,
        "GB/s": round(gb, 1), "frac_hbm": round(gb / PEAK_HBM_GBPS, 4),
        "roof_TFLOP/s": round(roof, 1), "roof_bound": "mfma" if roof == peak else "hbm",
        "frac_roof": round(tf / roof, 4),
        "flops": fl, "algorithmic_bytes": int(by), "kernel": dense_kernel_name(cfg),
        # HBM bytes per launch counted by rocprofv3 (FETCH_SIZE + WRITE_SIZE,
        # calibrated) in the committed profile; null if its sources changed
        "traffic": (profiled_traffic(*DENSE_PROFILES[cfg.name]) if cfg.name in DENSE_PROFILES else None)}


def run_configs(names, steps, warmup, copy_mib=0):
    """attn_fwd alone on each named dense workload; one JSON line per workload."""
    import torch
    from exact_tiled_self_amd.inputs import DENSE_CONFIGS

    if names == ["all"]:
        names = list(DENSE_CONFIGS)
    unknown = [n for n in names if n not in DENSE_CONFIGS]
    if unknown:
        raise SystemExit(f"unknown workload(s) {unknown}; known: {sorted(DENSE_CONFIGS)}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    if copy_mib > 0:
        plain_copy(torch, dev, copy_mib)
    for name in names:
        print(json.dumps(time_dense(torch, dev, stream, DENSE_CONFIGS[name], steps, warmup)), flush=True)
    return 0


def profile_figures(profile: str, sources, kernel: str):
    """Counter figures recorded in profiles/<profile>.md for one kernel:
    HBM traffic per launch, MFMA busy fraction and the sustained shader clock
    (GRBM_GUI_ACTIVE per XCD over the kernel-trace average), or None where
    missing or taken on other sources than the current ones."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile + ".md")
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in sources:
        src = os.path.join(ROOT, "exact_tiled_self_amd", "csrc", f)
        if not os.path.exists(src):
            return None
        h.update(open(src, "rb").read())
    text = open(path).read()
    digest = None
    for line in text.splitlines():
        if line.startswith("source_sha256_16:"):
            digest = line.split(":")[1].split()[0]
    if digest != h.hexdigest()[:16]:
        return None
    vals, avg_ns = {}, None
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 5 and cells[0] == kernel and cells[1].isdigit():
            avg_ns = float(cells[2])
        elif len(cells) == 3 and cells[0] == kernel:
            try:
                vals[cells[1].split(" ")[0]] = float(cells[2])
            except ValueError:
                pass
    out = {"traffic": profiled_traffic(profile, sources)}
    if avg_ns and "GRBM_GUI_ACTIVE" in vals:
        cyc = vals["GRBM_GUI_ACTIVE"] / 8.0           # per XCD
        out["trace_avg_us"] = round(avg_ns / 1e3, 2)
        # GRBM_GUI_ACTIVE also counts the busy time around each dispatch, so
        # cycles over the trace time only estimate the clock for long kernels
        if avg_ns >= 1e5:
            out["sclk_under_load_mhz"] = round(cyc / avg_ns * 1e3, 0)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in vals:
            out["mfma_busy"] = round(vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * 1024), 4)
    return out


def consistency_checks(pre_prof, dec_prof, pre_flops, pre_seconds, dec_bytes):
    """The measurement's own checks: the decode's counted HBM bytes must be
    within 25 % of its algorithmic bytes (no re-reads, nothing skipped), and
    the prefill's MFMA busy fraction must be at least what the event-timed
    flops need at the clock the profile saw (a kernel cannot do its flops in
    fewer matrix-core cycles than they take) and not far above it (wasted
    matrix work).  A check whose counters are stale is reported as null."""
    out = {}
    tr = dec_prof.get("traffic") if dec_prof else None
    out["decode_traffic_vs_algorithmic"] = (
        {"ok": None, "why": "no profile of the current decode sources"} if tr is None else
        {"ok": abs(tr / dec_bytes - 1.0) <= 0.25, "ratio": round(tr / dec_bytes, 4), "limit": 0.25})
    if pre_prof and "mfma_busy" in pre_prof:
        mhz = pre_prof["sclk_under_load_mhz"]
        # bf16 32x32x16 MFMA: 1024 flops per cycle per SIMD, 1024 SIMDs
        need = pre_flops / pre_seconds / (1024.0 * 1024.0 * mhz * 1e6)
        busy = pre_prof["mfma_busy"]
        out["prefill_mfma_busy_vs_events"] = {
            "ok": 0.85 * need <= busy <= 1.6 * need, "mfma_busy": busy,
            "needed_at_profiled_clock": round(need, 4), "sclk_mhz": mhz}
    else:
        out["prefill_mfma_busy_vs_events"] = {"ok": None, "why": "no profile of the current prefill sources"}
    return out


def read_clocks():
    """sclk / mclk lines of `rocm-smi --showclocks` (run as a child process right
    after the timed loop), or None when the tool is unavailable."""
    import subprocess
    try:
        out = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True,
                             timeout=20).stdout
    except Exception:
        return None
    lines = [ln.strip() for ln in out.splitlines() if "sclk" in ln or "mclk" in ln]
    return lines[:4] or None


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-workers", type=int, default=0)
    ap.add_argument("--no-clocks", action="store_true",
                    help="skip the rocm-smi clock readout (a child process; under a counter "
                         "profiler every process initialises the GPU)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before timing "
                         "(calibrates the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing each dense workload alone (profiling runs of the bench kernels)")
    ap.add_argument("--configs", default=None,
                    help="comma-separated dense workloads (or 'all'): time attn_fwd alone on each "
                         "and print one JSON line per workload instead of the bench line")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        return 2

    if args.configs:
        return run_configs(args.configs.split(","), args.steps, args.warmup, args.copy_mib)

    import torch
    from exact_tiled_self_amd import attn_fwd, attn_paged_decode, attn_paged_decode_workspace_size
    from exact_tiled_self_amd import attn_bwd, attn_bwd_workspace_size, attn_kv_append, attn_paged_prefill
    from exact_tiled_self_amd import attn_add_rmsnorm, attn_swiglu
    from exact_tiled_self_amd import _lib
    from exact_tiled_self_amd.inputs import (CHUNK_NEW, DENSE_CONFIGS, PAGED_CONFIG, chunked_inputs,
                                             dense_inputs)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pcfg = DENSE_CONFIGS["gqa_causal_t8192"]
    dcfg = PAGED_CONFIG
    q, k, v = dense_inputs(pcfg)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty(pcfg.B, pcfg.Hq, pcfg.N, dtype=torch.float32, device=dev)
    p = chunked_inputs(dcfg, new_lens=CHUNK_NEW)       # the decode cache plus a chunk per sequence
    pd = {kk: (vv.to(dev) if isinstance(vv, torch.Tensor) else vv) for kk, vv in p.items()}
    od = torch.empty_like(pd["q"])
    lsed = torch.empty(dcfg.S, dcfg.Hq, dtype=torch.float32, device=dev)
    ws = torch.empty(attn_paged_decode_workspace_size(dcfg.S, dcfg.Hq, dcfg.d, p["max_blocks"], 16),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def prefill():
        attn_fwd(qd, kd, vd, scale=pcfg.scale, causal=True, o=o, lse=lse, stream=stream)

    def decode():
        attn_paged_decode(pd["q"], pd["k_cache"], pd["v_cache"], pd["block_table"], pd["ctx_lens"],
                          16, dcfg.scale, o=od, lse=lsed, workspace=ws, stream=stream)

    if args.copy_mib > 0:
        plain_copy(torch, dev, args.copy_mib)

    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        prefill()
        ev[i][1].record(stream)
        decode()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(K)]
    dec_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(K)]
    step_ms = ev[0][0].elapsed_time(ev[K - 1][2]) / K

    # decode with the 256 MB last-level cache flushed before every call: a
    # read-only sweep of 1 GiB (a write sweep would leave dirty lines whose
    # write-back the timed call would pay for)
    flush = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
    fl_ms = []
    for _ in range(max(20, K // 2)):
        flush.amax()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        decode()
        e1.record(stream)
        torch.cuda.synchronize()
        fl_ms.append(e0.elapsed_time(e1))
    del flush

    # the decode step replayed from a HIP graph of 8 calls (no per-call launch)
    from exact_tiled_self_amd.graph import DecodeGraph
    dg = DecodeGraph(pd["q"], pd["k_cache"], pd["v_cache"], pd["block_table"], pd["ctx_lens"], 16,
                     dcfg.scale, calls=8)
    g_ms = []
    for _ in range(12):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dg.replay()
        e1.record()
        torch.cuda.synchronize()
        g_ms.append(e0.elapsed_time(e1) / 8)
    del dg

    # the steps either side of decode, on the same cache: chunked prefill of
    # CHUNK_NEW rows per sequence, and the append of those rows' K/V into a
    # copy of the cache (the append rewrites the slots it targets)
    oc = torch.empty_like(pd["q_new"])
    lsec = torch.empty(pd["q_new"].shape[:2], dtype=torch.float32, device=dev)
    kc2, vc2 = pd["k_cache"].clone(), pd["v_cache"].clone()

    def chunked():
        attn_paged_prefill(pd["q_new"], pd["k_cache"], pd["v_cache"], pd["block_table"], pd["ctx_lens"],
                           pd["starts"], 16, dcfg.scale, max_new=p["max_new"], o=oc, lse=lsec,
                           stream=stream)

    def append():
        attn_kv_append(pd["k_new"], pd["v_new"], kc2, vc2, pd["block_table"], pd["ctx_lens"],
                       pd["starts"], 16, max_new=p["max_new"], stream=stream)

    def timed(fn, reps):
        for _ in range(2):
            fn()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        e[0].record(stream)
        for i in range(reps):
            fn()
            e[i + 1].record(stream)
        torch.cuda.synchronize()
        return [e[i].elapsed_time(e[i + 1]) for i in range(reps)]

    ch_ms = timed(chunked, K)
    ap_ms = timed(append, K)
    del kc2, vc2

    # the backward pass of the prefill workload (upstream gradient N(0,1), seed 100)
    g_np = np.random.default_rng(100).standard_normal((pcfg.B, pcfg.Hq, pcfg.N, pcfg.d), dtype=np.float32)
    dod = torch.from_numpy(g_np).to(torch.bfloat16).to(dev)
    dqd, dkd, dvd = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    bws = torch.empty(attn_bwd_workspace_size(pcfg.B, pcfg.Hq, pcfg.Hkv, pcfg.N, pcfg.d), dtype=torch.uint8,
                      device=dev)

    def backward():
        attn_bwd(qd, kd, vd, o, lse, dod, scale=pcfg.scale, causal=True, dq=dqd, dk=dkd, dv=dvd,
                 workspace=bws, stream=stream)

    bw_ms = timed(backward, max(10, K // 5))

    # decoder-layer fusions: 8192 tokens, residual width 1536, intermediate 8960
    T_L, D_L, F_L = 8192, 1536, 8960
    frng = np.random.default_rng(200)
    fx = torch.from_numpy(frng.standard_normal((T_L, D_L), dtype=np.float32)).to(torch.bfloat16).to(dev)
    fr = torch.from_numpy(frng.standard_normal((T_L, D_L), dtype=np.float32)).to(torch.bfloat16).to(dev)
    fw = torch.from_numpy(1 + 0.1 * frng.standard_normal(D_L).astype(np.float32)).to(torch.bfloat16).to(dev)
    fgu = torch.from_numpy(frng.standard_normal((T_L, 2 * F_L), dtype=np.float32)).to(torch.bfloat16).to(dev)
    fo, fro, fa = torch.empty_like(fx), torch.empty_like(fx), torch.empty((T_L, F_L), dtype=torch.bfloat16, device=dev)
    rms_ms = timed(lambda: attn_add_rmsnorm(fx, fr, fw, 1e-6, out=fo, residual_out=fro, stream=stream), K)
    swi_ms = timed(lambda: attn_swiglu(fgu, out=fa, stream=stream), K)

    # parity spot check on the benchmarked buffers (sampled rows / sequences)
    from oracle import exact as OA
    rows = np.array([0, 1, 4095, 8190, 8191])
    qn, kn, vn = (t.double().numpy() for t in (q, k, v))
    errs = []
    for h in (0, 5, 6, 11):
        ro, rl = OA.attention_rows(qn, kn, vn, pcfg.scale, True, 0, h, rows)
        errs.append(float(np.abs(o[0, h, torch.as_tensor(rows)].double().cpu().numpy() - ro).max()))
    sub = np.array([0, 31, 63])
    ro, rl = OA.paged_decode(p["q"][sub].double().numpy(), p["k_cache"].float().numpy(),
                             p["v_cache"].float().numpy(), p["block_table"].numpy()[sub],
                             p["ctx_lens"].numpy()[sub], 16, dcfg.scale)
    derr = float(np.abs(od[torch.as_tensor(sub)].double().cpu().numpy() - ro).max())
    st = p["starts"].numpy().astype(np.int64)
    cs = int(p["ctx_lens"].numpy().argmax())
    ro, rl = OA.paged_prefill(p["q_new"][st[cs]:st[cs + 1]].double().numpy(), p["k_cache"].float().numpy(),
                              p["v_cache"].float().numpy(), p["block_table"].numpy()[cs:cs + 1],
                              p["ctx_lens"].numpy()[cs:cs + 1], [0, st[cs + 1] - st[cs]], 16, dcfg.scale)
    cerr = float(np.abs(oc[st[cs]:st[cs + 1]].double().cpu().numpy() - ro).max())
    # backward: dq rows sampled against the oracle's per-head gradients of one head pair
    from oracle import backward as OB
    hs = [0, 6]
    bq = OB.attention_bwd(qn[:, hs], kn, vn, dod[:, hs].double().cpu().numpy(), pcfg.scale, True)[0]
    berr = float(np.abs(dqd[:, hs].double().cpu().numpy() - bq).max() / max(1.0, np.abs(bq).max()))

    # every dense workload alone (attn_fwd on resident inputs, events around
    # each call): the ViT-B/16 shapes, the GQA prefill and the long MHA prefill
    cfg_stats = {}
    for name, cfg in ({} if args.no_configs else DENSE_CONFIGS).items():
        reps = K if cfg.N * cfg.N * cfg.B * cfg.Hq < 2e9 else max(10, K // 5)
        cfg_stats[name] = time_dense(torch, dev, stream, cfg, reps, args.warmup)

    clocks = None if args.no_clocks else read_clocks()

    pf = prefill_flops(pcfg)
    pre_avg = float(np.mean(pre_ms))
    tflops = pf / (pre_avg * 1e-3) / 1e12
    db = decode_bytes(p, dcfg)
    dec_avg = float(np.mean(dec_ms))
    gbps = db / (dec_avg * 1e-3) / 1e9
    fl_avg = float(np.mean(fl_ms))
    cf, cb = chunked_flops(p, dcfg), chunked_bytes(p, dcfg)
    ch_avg, ap_avg = float(np.mean(ch_ms)), float(np.mean(ap_ms))
    ab = append_bytes(p, dcfg)
    bw_avg = float(np.mean(bw_ms))
    bf = 2.5 * pf                       # five products (S recomputed, dP, dV, dK, dQ) against two
    rms_bytes = 4 * T_L * D_L * 2 + D_L * 2          # x, residual read; out, residual written; weight
    swi_bytes = 3 * T_L * F_L * 2                    # gate, up read; out written
    rms_avg, swi_avg = float(np.mean(rms_ms)), float(np.mean(swi_ms))

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "gqa_causal_t8192 prefill + paged_decode_s64 decode",
            "prefill": {"B": pcfg.B, "Hq": pcfg.Hq, "Hkv": pcfg.Hkv, "T": pcfg.N, "d": pcfg.d,
                        "causal": True, "dtype": "bf16", "input": "0.5*N(0,1), seed 2"},
            "decode": {"S": dcfg.S, "Hq": dcfg.Hq, "Hkv": dcfg.Hkv, "d": dcfg.d, "block_size": 16,
                       "ctx": "uniform [512, 8192], seed 4", "sum_ctx": int(p["ctx_lens"].sum()),
                       "num_blocks": p["num_blocks"]},
        },
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": profiled_traffic("prefill_bf16_d128_causal_gqa_t8192",
                                                 ["prefill_bf16.hip", "prefill_tile.h", "common.h",
                                                  "internal.h"]),
                     "algorithmic_bytes": prefill_bytes(pcfg),
                     "kernel": "prefill_sp_kernel<128, causal>",
                     "per_launch": {"flops": pf, "avg_us": round(pre_avg * 1e3, 2),
                                    "median_us": round(float(np.median(pre_ms)) * 1e3, 2),
                                    "min_us": round(min(pre_ms) * 1e3, 2)}},
        "decode": {"value": round(gbps, 1), "unit": "GB/s", "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4),
                   "avg_us": round(dec_avg * 1e3, 2), "median_us": round(float(np.median(dec_ms)) * 1e3, 2),
                   "min_us": round(min(dec_ms) * 1e3, 2),
                   "bytes": db, "flops": decode_flops(p, dcfg),
                   "flushed_avg_us": round(fl_avg * 1e3, 2),
                   "flushed_median_us": round(float(np.median(fl_ms)) * 1e3, 2),
                   "flushed_GBps": round(db / (fl_avg * 1e-3) / 1e9, 1),
                   "graph_replay_median_us": round(float(np.median(g_ms)) * 1e3, 2),
                   "kernels": "decode_split_kernel<128, 0> + decode_merge_kernel<128, 0>",
                   "traffic": profiled_traffic("paged_decode_bf16_d128_s64",
                                               ["decode_paged.hip", "common.h", "internal.h"])},
        "chunked_prefill": {
            "workload": f"paged_decode_s64 cache, {CHUNK_NEW} new rows per sequence (T={int(st[-1])})",
            "value": round(cf / (ch_avg * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "frac_mfma": round(cf / (ch_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "avg_us": round(ch_avg * 1e3, 2), "median_us": round(float(np.median(ch_ms)) * 1e3, 2),
            "min_us": round(min(ch_ms) * 1e3, 2), "flops": cf, "algorithmic_bytes": cb,
            "kernel": "prefill_paged_kernel<128>",
            "traffic": profiled_traffic("chunked_prefill_bf16_d128_s64_c256",
                                        ["prefill_paged.hip", "prefill_tile.h", "common.h", "internal.h"])},
        "kv_append": {
            "workload": f"{CHUNK_NEW} new rows per sequence into the paged_decode_s64 cache",
            "value": round(ab / (ap_avg * 1e-3) / 1e9, 1), "unit": "GB/s",
            "frac_hbm": round(ab / (ap_avg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "avg_us": round(ap_avg * 1e3, 2), "median_us": round(float(np.median(ap_ms)) * 1e3, 2),
            "min_us": round(min(ap_ms) * 1e3, 2), "bytes": ab, "kernel": "kv_append_kernel",
            "traffic": profiled_traffic("kv_append_bf16_d128_s64_c256",
                                        ["kv_append.hip", "common.h", "internal.h"])},
        "backward": {
            "workload": "gqa_causal_t8192 (dout N(0,1), seed 100)",
            "value": round(bf / (bw_avg * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "frac_mfma": round(bf / (bw_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "avg_us": round(bw_avg * 1e3, 2), "median_us": round(float(np.median(bw_ms)) * 1e3, 2),
            "min_us": round(min(bw_ms) * 1e3, 2), "flops": bf,
            "kernels": "bwd_prep + bwd_dq + bwd_kvf (dK and dV) + bwd_reduce",
            "traffic": profiled_traffic("backward_bf16_d128_causal_gqa_t8192",
                                        ["backward_bf16.hip", "prefill_tile.h", "common.h", "internal.h"])},
        "fusion": {
            "workload": f"decoder layer, {T_L} tokens, width {D_L}, intermediate {F_L}, bf16",
            "add_rmsnorm": {"value": round(rms_bytes / (rms_avg * 1e-3) / 1e9, 1), "unit": "GB/s",
                            "frac_hbm": round(rms_bytes / (rms_avg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                            "avg_us": round(rms_avg * 1e3, 2),
                            "median_us": round(float(np.median(rms_ms)) * 1e3, 2), "bytes": rms_bytes,
                            "kernel": "add_rmsnorm_kernel<4>"},
            "swiglu": {"value": round(swi_bytes / (swi_avg * 1e-3) / 1e9, 1), "unit": "GB/s",
                       "frac_hbm": round(swi_bytes / (swi_avg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                       "avg_us": round(swi_avg * 1e3, 2), "median_us": round(float(np.median(swi_ms)) * 1e3, 2),
                       "bytes": swi_bytes, "kernel": "swiglu_kernel"},
            "traffic": profiled_traffic("fusion_bf16_t8192_d1536_f8960", ["fusion.hip", "common.h", "internal.h"])},
        "parity": {"prefill_sampled_max_abs": max(errs), "decode_sampled_max_abs": derr,
                   "chunked_prefill_sampled_max_abs": cerr, "tolerance": 2e-2,
                   "backward_dq_heads_0_6_rel_max": berr, "backward_tolerance_rel": 2e-2},
        "wall_s_timed": round(wall, 3),
        "clocks_after_timing": clocks,
        "library": _lib.library_path(),
    }
    # counter figures of the committed profiles (null where the kernel
    # sources changed since they were taken), and the consistency checks
    # between them and the event timings
    dec_prof = profile_figures("paged_decode_bf16_d128_s64", ["decode_paged.hip", "common.h", "internal.h"],
                               "decode_split_kernel<128, 0>")
    pre_prof = profile_figures("prefill_bf16_d128_causal_gqa_t8192",
                               ["prefill_bf16.hip", "prefill_tile.h", "common.h", "internal.h"],
                               "prefill_sp_kernel<128, true>")
    out["roofline"]["profile"] = pre_prof
    out["checks"] = consistency_checks(pre_prof, dec_prof, pf, pre_avg * 1e-3, db)
    for name, ck in out["checks"].items():
        if ck.get("ok") is False:
            print(f"bench.py: CONSISTENCY CHECK FAILED: {name}: {ck}", file=sys.stderr, flush=True)
    out["configs"] = cfg_stats

    if not args.no_cpu_baseline:
        workers = cpu_workers(args.cpu_workers)
        out["cpu_baseline"] = cpu_baseline(pcfg, q, k, v, workers)
        per = {}
        for name, cfg in DENSE_CONFIGS.items():
            if name == pcfg.name:
                per[name] = out["cpu_baseline"]
                continue
            qc, kc, vc = dense_inputs(cfg)
            # the 32768-token prefill: one GQA group of heads (one head) of it
            heads = list(range(cfg.Hq // cfg.Hkv)) if cfg.N > 16384 else None
            per[name] = cpu_baseline(cfg, qc, kc, vc, workers, min_seconds=2.0, heads=heads)
            del qc, kc, vc
        out["cpu_baseline_per_config"] = per
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
