#!/usr/bin/env python3
"""Benchmark of the MiMo-V2.6-Flash attention hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  1. sliding-window + sink prefill, B=4 x T=8192, 64 q / 8 KV heads, window 128
  2. global causal prefill, B=1 x T=32768, 64 q / 4 KV heads
  3. mixed decode step: ring append of the new token for 64 sliding and 16
     global sequences, then sliding decode (ring of 128) and global split-K
     decode (KV lengths ~ U[32768, 131072]).
Inputs are resident in HBM before the timed region.  The reported value is the
step's algorithmic attention FLOPs (2*(192+128)*64 per visible query-key pair)
over the measured step time.  Per-launch durations are taken with HIP events
on the stream the kernels are launched on (torch's current stream).

After the step, the default run also measures, each in `phases` with its own
figures: the on-box peaks (a bf16 MFMA loop on N(0,1) operands and on ones, a
1 GiB HBM copy and read; `peaks`), the sliding-window prefill B=1 x T=512 with
the Infinity Cache flushed before each call, and the 524288-token global
prefill in 8 query chunks of 65536 (one warmup and two timed passes, with its
own roofline object; --no-long skips it), and the sliding-window + sink backward
of the B=4 x T=8192 prefill (--no-backward skips it).  Every kernel figure is given as a
fraction of the vendor peaks (2.5 PFLOP/s bf16, 8 TB/s) and of the measured ones.

--workload long_prefill instead times the 524288-token global prefill run as 8
query chunks of 65536, each against its full causal prefix.

--workload spec_decode times multi-query decode (speculative verification) at
the mixed-decode sizes: 64 sliding sequences (ring of 128 + n_q - 1) and 16
global sequences, with n_q = 4 (EAGLE) and n_q = 8 (DFlash) draft tokens.

--workload paged_decode times decode over paged caches (128-slot blocks in
shuffled pools) at the mixed-decode sizes: the 16 global sequences with bf16
and with fp8 e4m3 pools, and the 64 sliding sequences with fp8 pools.

--workload backward times the sliding-window + sink backward (dq, dk, dv, d sink)
of the B=4 x T=8192 prefill, from the forward's output and LSE.

--workload serving_chunks times packed (THD) serving chunks of 8192 tokens:
four sliding-window chunks that continue sequences at positions 8192, 65536,
131072 and 262144 (each with the 127 keys before it) and four global chunks
after prefixes of 0, 8192, 24576 and 57344 tokens, one packed call each.

The fp64 oracle is timed on a bounded sample of the same workload on the host
cores (rank 0, N=1) as a CPU baseline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention prefill TFLOP/s (% bf16 MFMA peak); decode HBM GB/s (% peak)"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
FLOP_PER_PAIR_HEAD = 2 * (192 + 128)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------ algorithmic counts

def swa_pairs(T: int, W: int) -> int:
    """Visible (query, key) pairs of one sequence of T tokens, window W."""
    full = max(0, T - W + 1) * W
    early = sum(min(t + 1, W) for t in range(min(T, W - 1)))
    return full + early


def causal_pairs(q_lo: int, q_hi: int) -> int:
    """Pairs of queries at positions q_lo..q_hi-1 over all earlier keys."""
    return (q_hi * (q_hi + 1) - q_lo * (q_lo + 1)) // 2


def prefill_bytes(B, Tq, Tk, hq, hkv, sinks: bool) -> int:
    return sum(prefill_rw(B, Tq, Tk, hq, hkv, sinks))


def prefill_rw(B, Tq, Tk, hq, hkv, sinks: bool):
    """Algorithmic (read, written) bytes of a prefill: q, k, v (and sinks) in, out out."""
    return (B * (Tq * hq * 192 * 2 + Tk * hkv * (192 + 128) * 2) + (hq * 4 if sinks else 0),
            B * Tq * hq * 128 * 2)


# ------------------------------------------------------------ HBM traffic from the committed profile

_PREFILL_SOURCES = ["global_attention_sinks_amd/csrc/prefill.hip", "global_attention_sinks_amd/csrc/common.hpp",
                    "global_attention_sinks_amd/csrc/kernels.hpp"]
_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "hot_path_step_hbm_traffic.md")


def profiled_traffic(workload_label: str):
    """Bytes one launch moved to and from HBM, as the committed FETCH_SIZE / WRITE_SIZE
    profile recorded them (already scaled by the copy calibration), or None when the
    profile is missing or the kernel source changed since it was taken."""
    import hashlib
    import re
    if not os.path.exists(_TRAFFIC_PROFILE):
        return None
    text = open(_TRAFFIC_PROFILE).read()
    h = hashlib.sha256()
    for f in _PREFILL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    m = re.search(r"prefill sha256\[:16\] ([0-9a-f]{16})", text)
    if not m or m.group(1) != h.hexdigest()[:16]:
        return None
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip("|").split("|")]
        if len(cells) == 6 and cells[1] == workload_label:
            return (float(cells[4]) + float(cells[5])) * 1e9
    return None


_BACKWARD_SOURCES = ["global_attention_sinks_amd/csrc/backward.hip"]
_BACKWARD_PROFILE = os.path.join(ROOT, "profiles", "backward_swa_b4_t8192_pmc_counters.md")


def profiled_backward_traffic():
    """Bytes one backward call moved to and from HBM (all its kernels), summed from the
    committed FETCH_SIZE / WRITE_SIZE profile (already scaled by the copy calibration), or
    None when the profile is missing or the backward source changed since it was taken."""
    import hashlib
    import re
    if not os.path.exists(_BACKWARD_PROFILE):
        return None
    text = open(_BACKWARD_PROFILE).read()
    h = hashlib.sha256()
    for f in _BACKWARD_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    m = re.search(r"backward sha256\[:16\] ([0-9a-f]{16})", text)
    if not m or m.group(1) != h.hexdigest()[:16]:
        return None
    total, found = 0.0, False
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip("|").split("|")]
        if len(cells) == 6 and cells[0].startswith("bwd_"):
            total += (float(cells[3]) + float(cells[4])) * 1e9
            found = True
    return total if found else None


# ------------------------------------------------------------ workloads

def _dev_bf16(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def setup_layer_step(torch, gen, Bd):
    def dev_bf16(bits):
        return _dev_bf16(torch, bits)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")

    ph = {}
    # 1. sliding-window prefill
    log("setup: sliding-window prefill B=4 T=8192")
    d = gen.prefill_inputs(4, 8192, 64, 8, seed=1001, with_sinks=True)
    ph["swa_prefill"] = dict(
        cfg=Bd.swa_cfg(), q=dev_bf16(d["q"]), k=dev_bf16(d["k"]), v=dev_bf16(d["v"]),
        sinks=dev(d["sinks"]), out=torch.empty((4, 8192, 64, 128), dtype=torch.bfloat16, device="cuda"),
        flops=FLOP_PER_PAIR_HEAD * 64 * 4 * swa_pairs(8192, 128),
        bytes=prefill_bytes(4, 8192, 8192, 64, 8, True), host=d)
    # 2. global prefill
    log("setup: global prefill B=1 T=32768")
    d = gen.prefill_inputs(1, 32768, 64, 4, seed=1002, with_sinks=False)
    ph["global_prefill"] = dict(
        cfg=Bd.global_cfg(), q=dev_bf16(d["q"]), k=dev_bf16(d["k"]), v=dev_bf16(d["v"]),
        out=torch.empty((1, 32768, 64, 128), dtype=torch.bfloat16, device="cuda"),
        ws=torch.empty(Bd.mimo_attn_prefill_workspace_size(Bd.global_cfg(), 1, 32768), dtype=torch.uint8,
                       device="cuda"),
        flops=FLOP_PER_PAIR_HEAD * 64 * causal_pairs(0, 32768),
        bytes=prefill_bytes(1, 32768, 32768, 64, 4, False), host=d)
    # 3. mixed decode
    log("setup: mixed decode (64 sliding seqs, ring 128; 16 global seqs, cap 131072)")
    sw = gen.decode_inputs(64, 128, 64, 8, seed=1003, window=128, pos_lo=128, pos_hi=131072, with_sinks=True)
    gl = gen.decode_inputs(16, 131072, 64, 4, seed=2003, window=0, pos_lo=32768, pos_hi=131072,
                           with_sinks=False)
    ap_s = gen.append_inputs(64, 8, seed=3003, pos_lo=0, pos_hi=1)
    ap_g = gen.append_inputs(16, 4, seed=4003, pos_lo=0, pos_hi=1)
    dec = {}
    for name, dd, ap, cfg, cap in (("swa", sw, ap_s, Bd.swa_cfg(), 128),
                                   ("global", gl, ap_g, Bd.global_cfg(), 131072)):
        S = dd["q"].shape[0]
        ws_n = Bd.mimo_attn_decode_workspace_size(cfg, S, cap)
        L = np.minimum(dd["pos"] + 1, 128 if name == "swa" else dd["pos"] + 1)
        hkv = cfg.num_kv_heads
        dec[name] = dict(
            cfg=cfg, q=dev_bf16(dd["q"]), pos=dev(dd["pos"]), kc=dev_bf16(dd["k_cache"]),
            vc=dev_bf16(dd["v_cache"]), sinks=None if dd["sinks"] is None else dev(dd["sinks"]),
            out=torch.empty((S, 64, 128), dtype=torch.bfloat16, device="cuda"),
            ws=torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda"),
            k_new=dev_bf16(ap["k"]), v_new=dev_bf16(ap["v"]),
            flops=FLOP_PER_PAIR_HEAD * 64 * int(L.sum()),
            bytes=int(L.sum()) * hkv * 320 * 2 + S * 64 * (192 + 128) * 2 + S * 8 + (64 * 4 if dd["sinks"] is not None else 0),
            append_bytes=S * hkv * (192 * 2 + 320) * 2 + S * 8, host=dd)
    ph["decode"] = dec
    return ph


def run_layer_step(ph, Bd, ev=None):
    """Enqueue one step; ev maps a launch name to (start, end) events to record."""
    def rec(name, fn):
        if ev is not None:
            ev[name][0].record()
        fn()
        if ev is not None:
            ev[name][1].record()

    s = ph["swa_prefill"]
    rec("swa_prefill", lambda: Bd.mimo_attn_prefill_swa(s["cfg"], s["q"], s["k"], s["v"], s["sinks"], s["out"]))
    g = ph["global_prefill"]
    rec("global_prefill", lambda: Bd.mimo_attn_prefill_global(g["cfg"], g["q"], g["k"], g["v"], g["out"],
                                                                ws=g["ws"]))
    for name in ("swa", "global"):
        d = ph["decode"][name]
        rec(f"append_{name}", lambda d=d: Bd.mimo_kv_ring_append(d["cfg"], d["k_new"], d["v_new"], d["pos"],
                                                                  d["kc"], d["vc"]))
    for name in ("swa", "global"):
        d = ph["decode"][name]
        rec(f"decode_{name}", lambda d=d: Bd.mimo_attn_decode(d["cfg"], d["q"], d["pos"], d["kc"], d["vc"],
                                                               d["sinks"], d["out"], ws=d["ws"]))


# ------------------------------------------------------------ on-box peaks

def _event_ms(torch, fn, reps):
    """Median over reps of fn's time between HIP events recorded on torch's
    current stream (the stream the kernels are launched on)."""
    pairs = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        pairs.append((a, b))
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in pairs]))


def measure_peaks(torch, Bd):
    """What a plain bf16 MFMA loop (on N(0,1) operands, like attention's, and on
    ones) and plain HBM streams (a 1 GiB copy, a 1 GiB read) reach on this card."""
    waves = Bd.load_peaks().mimo_peak_mfma_waves()
    sink = torch.empty(waves, dtype=torch.float32, device="cuda")
    gen_ = torch.Generator(device="cuda")
    gen_.manual_seed(7)
    rnd = torch.randn(1 << 22, generator=gen_, device="cuda").to(torch.bfloat16)
    ones = torch.ones(1 << 22, dtype=torch.bfloat16, device="cuda")
    # ~2.5 ms launches back to back for about a second, so the clock settles where
    # sustained MFMA work holds it (the attention calls run 18 ms to seconds); the
    # median of the second half of the launches
    iters, reps = 1000, 400
    flops = Bd.peak_mfma_flops(iters)
    res = {"mfma_loop": f"{waves} waves x {iters * 64} MFMA 32x32x16 bf16 per launch, 8 chains, operands "
                        f"changing every MFMA; {reps} launches back to back, median of the last {reps // 2}"}
    for name, ops in (("randn", rnd), ("ones", ones)):
        pairs = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            Bd.peak_mfma_bf16(ops, iters, sink)
            b.record()
            pairs.append((a, b))
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in pairs[reps // 2:]]))
        res[f"mfma_bf16_{name}_tflops"] = flops / (ms * 1e-3) / 1e12
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    Bd.peak_copy(src, dst)
    res["hbm_copy_gbs"] = 2 * n / (_event_ms(torch, lambda: Bd.peak_copy(src, dst), 10) * 1e-3) / 1e9
    Bd.peak_read(src, out)
    res["hbm_read_gbs"] = n / (_event_ms(torch, lambda: Bd.peak_read(src, out), 10) * 1e-3) / 1e9
    Bd.peak_write(dst, 3)
    res["hbm_write_gbs"] = n / (_event_ms(torch, lambda: Bd.peak_write(dst, 3), 10) * 1e-3) / 1e9
    del src, dst
    return res


def mixed_ceiling_ms(peaks, read_bytes, write_bytes):
    """Time the measured streams would need for a kernel's algorithmic reads and
    writes: read bytes at the read rate plus written bytes at the write rate."""
    return (read_bytes / peaks["hbm_read_gbs"] + write_bytes / peaks["hbm_write_gbs"]) / 1e6


# ------------------------------------------------------------ the two workloads outside the step

def bench_swa_small(torch, gen, Bd, peaks, reps=10):
    """Sliding-window + sink prefill B=1 x T=512 (64 q / 8 KV heads): it fits in
    the 256 MB Infinity Cache, so a 512 MiB buffer is written between reps (untimed)
    and every rep reads its inputs from HBM."""
    d = gen.prefill_inputs(1, 512, 64, 8, seed=1000, with_sinks=True)
    cfg = Bd.swa_cfg()
    q, k, v = _dev_bf16(torch, d["q"]), _dev_bf16(torch, d["k"]), _dev_bf16(torch, d["v"])
    sinks = torch.from_numpy(d["sinks"]).to("cuda")
    out = torch.empty((1, 512, 64, 128), dtype=torch.bfloat16, device="cuda")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    flops = FLOP_PER_PAIR_HEAD * 64 * swa_pairs(512, 128)
    nbytes = prefill_bytes(1, 512, 512, 64, 8, True)
    ts = []
    for i in range(reps + 2):
        flush.fill_(i & 255)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        Bd.mimo_attn_prefill_swa(cfg, q, k, v, sinks, out)
        b.record()
        ts.append((a, b))
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ts[2:]]))
    tfl, gbs = flops / (ms * 1e-3) / 1e12, nbytes / (ms * 1e-3) / 1e9
    return {"ms": ms, "tflops": tfl, "gbs": gbs, "frac_mfma_peak": tfl / PEAK_BF16_TFLOPS,
            "frac_hbm_peak": gbs / PEAK_HBM_GBS,
            "frac_measured_hbm_mix": (mixed_ceiling_ms(peaks, *prefill_rw(1, 512, 512, 64, 8, True)) / ms
                                      if peaks else None),
            "note": f"median of {reps} calls, Infinity Cache flushed before each; launch-latency bound "
                    f"({flops / 1e9:.2f} GFLOP, {nbytes / 1e6:.1f} MB)"}


def bench_long_prefill(torch, gen, Bd, peaks, warmup=1, steps=2):
    """Global causal prefill of 524288 tokens in 8 query chunks of 65536, each
    against its whole prefix, one tile-image workspace for all chunks; q is drawn
    and uploaded chunk by chunk."""
    T, C = 524288, 65536
    n_chunks = T // C
    cfg = Bd.global_cfg()
    kv = gen.global_prefill_chunk(T, 64, 4, seed=1004, t_lo=T, t_hi=T)
    k, v = _dev_bf16(torch, kv["k"]), _dev_bf16(torch, kv["v"])
    del kv
    q = torch.empty((1, T, 64, 192), dtype=torch.bfloat16, device="cuda")
    for c in range(n_chunks):
        q[:, c * C:(c + 1) * C] = _dev_bf16(torch, gen.global_prefill_chunk(T, 64, 4, seed=1004, t_lo=c * C,
                                                                             t_hi=(c + 1) * C, kv=False)["q"])
    out = torch.empty((1, T, 64, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(Bd.mimo_attn_prefill_workspace_size(cfg, 1, T), dtype=torch.uint8, device="cuda")

    def chunk(c):
        Bd.mimo_attn_prefill_global(cfg, q[:, c * C:(c + 1) * C], k[:, :(c + 1) * C], v[:, :(c + 1) * C],
                                    out[:, c * C:(c + 1) * C], q_pos0=c * C, ws=ws)

    for _ in range(warmup):
        for c in range(n_chunks):
            chunk(c)
    torch.cuda.synchronize()
    evs = []
    for i in range(steps):
        row = []
        for c in range(n_chunks):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            chunk(c)
            b.record()
            row.append((a, b))
        evs.append(row)
        torch.cuda.synchronize()
        log(f"long prefill step {i} done")
    chunk_ms = [float(np.mean([r[c][0].elapsed_time(r[c][1]) for r in evs])) for c in range(n_chunks)]
    ms = float(sum(chunk_ms))
    flops = FLOP_PER_PAIR_HEAD * 64 * causal_pairs(0, T)
    nbytes = prefill_bytes(1, T, T, 64, 4, False)
    tfl = flops / (ms * 1e-3) / 1e12
    del q, k, v, out, ws
    return {"ms": ms, "tflops": tfl, "gbs": nbytes / (ms * 1e-3) / 1e9, "frac_mfma_peak": tfl / PEAK_BF16_TFLOPS,
            "chunks_ms": chunk_ms,
            "roofline": {"bound": "mfma", "kernel": "prefill_image_kernel (8 global causal chunks; their K/V image "
                                                    "passes are inside the timed calls)",
                         "achieved": tfl, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": tfl / PEAK_BF16_TFLOPS,
                         "frac_measured_mfma_randn": tfl / peaks["mfma_bf16_randn_tflops"] if peaks else None,
                         "traffic": profiled_traffic("long prefill T524288 (8 chunks)"),
                         "algorithmic_flops": flops, "algorithmic_bytes": nbytes}}


# ------------------------------------------------------------ CPU baseline

def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_layer_step(ph, budget_s: float, gen):
    """Time the fp64 oracle on the host cores: the sliding prefill (B4 x T8192) and
    the mixed decode (all 64 + 16 sequences) in full; the global prefill (T32768,
    ~22 TFLOP of fp64 work, hours on a CPU) on query rows sampled to take about
    half of budget_s, extrapolated by their visible-pair count; and the 512-token
    sliding prefill in full, reported on its own."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    per = {}

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    # config 1 (not part of the step), in full
    d1 = gen.prefill_inputs(1, 512, 64, 8, seed=1000, with_sinks=True)
    t1 = timed(lambda: oracle.prefill_swa(d1["q"], d1["k"], d1["v"], d1["sinks"], window=128, base=1e4,
                                          n_threads=threads))
    f1 = FLOP_PER_PAIR_HEAD * 64 * swa_pairs(512, 128)
    per["swa_prefill_b1_t512"] = {"s": t1, "tflops": f1 / t1 / 1e12, "kind": "full"}
    # sliding prefill, in full
    d = ph["swa_prefill"]["host"]
    t_swa = timed(lambda: oracle.prefill_swa(d["q"], d["k"], d["v"], d["sinks"], window=128, base=1e4,
                                             n_threads=threads))
    per["swa_prefill_b4_t8192"] = {"s": t_swa, "tflops": ph["swa_prefill"]["flops"] / t_swa / 1e12, "kind": "full"}
    # mixed decode, every sequence
    t_dec = 0.0
    for name, window, base in (("swa", 128, 1e4), ("global", 0, 1e7)):
        dd = ph["decode"][name]["host"]
        t = timed(lambda: oracle.decode(dd["q"], dd["pos"], dd["k_cache"], dd["v_cache"], sinks=dd["sinks"],
                                        window=window, base=base, n_threads=threads))
        per[f"decode_{name}"] = {"s": t, "tflops": ph["decode"][name]["flops"] / t / 1e12, "kind": "full"}
        t_dec += t
    # global prefill: a pilot, then rows sized to about half the budget
    g = ph["global_prefill"]["host"]
    rng = np.random.default_rng(0)

    def glob_rows(n):
        rows = np.unique(np.concatenate([[0, 32767], rng.integers(0, 32768, n)]))
        return timed(lambda: oracle.prefill_global(g["q"], g["k"], g["v"], base=1e7, rows=rows,
                                                   n_threads=threads)), rows
    tp, _ = glob_rows(16)
    dt, rows = glob_rows(int(min(32768, max(16, 16 * (budget_s / 2) / max(tp, 1e-3)))))
    sample_flops = FLOP_PER_PAIR_HEAD * 64 * int(sum(int(r) + 1 for r in rows))
    t_glob = dt * ph["global_prefill"]["flops"] / sample_flops
    per["global_prefill_t32768"] = {"s": t_glob, "tflops": ph["global_prefill"]["flops"] / t_glob / 1e12,
                                    "kind": f"extrapolated from {len(rows)} rows ({dt:.1f} s)"}
    step_flops = ph["swa_prefill"]["flops"] + ph["global_prefill"]["flops"] + sum(
        ph["decode"][n]["flops"] for n in ("swa", "global"))
    step_s = t_swa + t_dec + t_glob
    return {"value": step_flops / step_s / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "logical_cpus": os.cpu_count(),
            "sample": f"sliding prefill B4xT8192 and mixed decode (64 + 16 sequences) in full; global prefill "
                      f"T32768 on {len(rows)} sampled rows, extrapolated by visible pairs; "
                      f"{t1 + t_swa + t_dec + dt:.1f} s of fp64 oracle time",
            "step_s": step_s, "per_config": per}


# ------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", choices=["layer_step", "long_prefill", "serving_chunks", "spec_decode", "paged_decode",
                                            "backward"], default="layer_step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the on-box peak loops (profiling passes); fractions of them are then omitted")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the 524288-token prefill phase of the default run")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward phase of the default run")
    ap.add_argument("--cpu-budget", type=float, default=40.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run three 1 GiB device-to-device copies (a known-size reference "
                         "for the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: this build has no multi-GPU path (each GPU would run "
              "its own shard of heads or sequences with no communication); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from global_attention_sinks_amd import binding as Bd
    from global_attention_sinks_amd import inputs as gen
    Bd.load_library()   # fails loudly if the HIP library is not built
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("copy calibration: 3 x 1 GiB device-to-device copies done")

    if args.workload == "long_prefill":
        return main_long_prefill(args, torch, gen, Bd)
    if args.workload == "serving_chunks":
        return main_serving_chunks(args, torch, gen, Bd)
    if args.workload == "spec_decode":
        return main_spec_decode(args, torch, gen, Bd)
    if args.workload == "paged_decode":
        return main_paged_decode(args, torch, gen, Bd)
    if args.workload == "backward":
        return main_backward(args, torch, gen, Bd)

    ph = setup_layer_step(torch, gen, Bd)
    names = ["swa_prefill", "global_prefill", "append_swa", "append_global", "decode_swa", "decode_global"]
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        run_layer_step(ph, Bd)
    torch.cuda.synchronize()
    evs = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names}
           for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_layer_step(ph, Bd, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {n: float(np.mean([e[n][0].elapsed_time(e[n][1]) for e in evs])) for n in names}
    ms_step = wall * 1e3 / args.steps

    s, g = ph["swa_prefill"], ph["global_prefill"]
    ds, dg = ph["decode"]["swa"], ph["decode"]["global"]
    step_flops = s["flops"] + g["flops"] + ds["flops"] + dg["flops"]
    value = step_flops / (ms_step * 1e-3) / 1e12

    def tf(f, t):
        return f / (t * 1e-3) / 1e12

    def gbs(b, t):
        return b / (t * 1e-3) / 1e9

    phases = {
        "swa_prefill_b4_t8192": {"ms": ms["swa_prefill"], "tflops": tf(s["flops"], ms["swa_prefill"]),
                                 "gbs": gbs(s["bytes"], ms["swa_prefill"])},
        "global_prefill_t32768": {"ms": ms["global_prefill"], "tflops": tf(g["flops"], ms["global_prefill"]),
                                  "gbs": gbs(g["bytes"], ms["global_prefill"])},
        "ring_append_80seqs": {"ms": ms["append_swa"] + ms["append_global"]},
        "decode_swa_64seqs": {"ms": ms["decode_swa"], "gbs": gbs(ds["bytes"], ms["decode_swa"]),
                              "tflops": tf(ds["flops"], ms["decode_swa"])},
        "decode_global_16seqs": {"ms": ms["decode_global"], "gbs": gbs(dg["bytes"], ms["decode_global"]),
                                 "tflops": tf(dg["flops"], ms["decode_global"])},
    }
    for p in phases.values():
        if "tflops" in p:
            p["frac_mfma_peak"] = p["tflops"] / PEAK_BF16_TFLOPS
        if "gbs" in p:
            p["frac_hbm_peak"] = p["gbs"] / PEAK_HBM_GBS
    mixed_ms = ms["append_swa"] + ms["append_global"] + ms["decode_swa"] + ms["decode_global"]
    mixed_bytes = ds["bytes"] + dg["bytes"] + ds["append_bytes"] + dg["append_bytes"]
    phases["mixed_decode_step"] = {"ms": mixed_ms, "gbs": gbs(mixed_bytes, mixed_ms),
                                   "frac_hbm_peak": gbs(mixed_bytes, mixed_ms) / PEAK_HBM_GBS}
    # (read, written) algorithmic bytes of each phase, for the measured mixed-stream ceiling
    def dec_rw(d, S):
        w = S * 64 * 128 * 2
        return d["bytes"] - w, w
    def app_rw(d, S, hkv):
        w = S * hkv * 320 * 2
        return d["append_bytes"] - w, w
    rw = {"swa_prefill_b4_t8192": prefill_rw(4, 8192, 8192, 64, 8, True),
          "global_prefill_t32768": prefill_rw(1, 32768, 32768, 64, 4, False),
          "decode_swa_64seqs": dec_rw(ds, 64), "decode_global_16seqs": dec_rw(dg, 16)}
    rw["mixed_decode_step"] = tuple(a + b + c + e for a, b, c, e in zip(
        rw["decode_swa_64seqs"], rw["decode_global_16seqs"], app_rw(ds, 64, 8), app_rw(dg, 16, 4)))

    peaks = None
    if not args.no_peaks:
        log("on-box peaks: bf16 MFMA loop, HBM copy and read")
        peaks = measure_peaks(torch, Bd)
    for name, p in (phases.items() if peaks else ()):
        if "tflops" in p:
            p["frac_measured_mfma_randn"] = p["tflops"] / peaks["mfma_bf16_randn_tflops"]
        if name in rw:
            # the time the measured read and write streams need for the phase's bytes, over its time
            p["frac_measured_hbm_mix"] = mixed_ceiling_ms(peaks, *rw[name]) / p["ms"]
    log("sliding-window prefill B=1 T=512 (cache flushed between calls)")
    phases["swa_prefill_b1_t512"] = bench_swa_small(torch, gen, Bd, peaks)
    if not args.no_long:
        log("long global prefill T=524288 in 8 chunks of 65536")
        phases["global_prefill_t524288_8chunks"] = bench_long_prefill(torch, gen, Bd, peaks)
    if not args.no_backward:
        log("sliding-window + sink backward B=4 T=8192")
        phases["swa_backward_b4_t8192"] = bench_backward(torch, gen, Bd, 2, 10, src=ph["swa_prefill"])

    achieved = tf(g["flops"], ms["global_prefill"])
    roofline = {"bound": "mfma", "kernel": "prefill_image_kernel (global causal, T=32768; its K/V image pass "
                                           "is inside the timed call)",
                "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": profiled_traffic("global prefill T32768"),
                "measured_peak": peaks["mfma_bf16_randn_tflops"] if peaks else None,
                "frac_measured_peak": achieved / peaks["mfma_bf16_randn_tflops"] if peaks else None,
                "algorithmic_flops": g["flops"], "algorithmic_bytes": g["bytes"]}

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the fp64 oracle")
        cpu = cpu_baseline_layer_step(ph, args.cpu_budget, gen)

    out = {"metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic: seeded N(0,1) bf16 q/k/v and caches, N(0,1) fp32 sinks",
           "config": {"workload": "mimo_layer_step = swa_prefill_b4_t8192 + global_prefill_t32768 + "
                                  "mixed_decode_64swa_16global (append + decode)",
                      "step_gflop": step_flops / 1e9},
           "roofline": roofline, "cpu_baseline": cpu, "peaks": peaks, "phases": phases}
    print(json.dumps(out))


def main_long_prefill(args, torch, gen, Bd):
    log("on-box peaks")
    peaks = measure_peaks(torch, Bd)
    log("setup: long global prefill T=524288 (k/v whole, q chunk by chunk)")
    r = bench_long_prefill(torch, gen, Bd, peaks, warmup=args.warmup, steps=args.steps)
    flops = r["roofline"]["algorithmic_flops"]
    out_j = {"metric": METRIC, "value": r["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
             "warmup": args.warmup, "ms_per_step": r["ms"], "higher_is_better": True, "scaling": "weak",
             "vs_baseline": None, "dtype": "bf16", "data": "synthetic: seeded N(0,1) bf16 q/k/v",
             "config": {"workload": "global_prefill_t524288 in 8 query chunks of 65536 against the full prefix",
                        "step_gflop": flops / 1e9},
             "roofline": r["roofline"], "cpu_baseline": None, "peaks": peaks, "chunks_ms": r["chunks_ms"]}
    print(json.dumps(out_j))


def main_serving_chunks(args, torch, gen, Bd):
    def dev_bf16(bits):
        return _dev_bf16(torch, bits)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")

    C = 8192
    packs = {}
    log("setup: packed sliding chunks (4 x 8192, 127 earlier keys each)")
    starts = [8192, 65536, 131072, 262144]
    d = gen.varlen_inputs([C] * 4, [C + 127] * 4, 64, 8, seed=1005, with_sinks=True,
                          k_pos0=[st - 127 for st in starts])
    packs["sliding"] = dict(cfg=Bd.swa_cfg(), d=d, flops=FLOP_PER_PAIR_HEAD * 64 * 4 * C * 128)
    log("setup: packed global chunks (4 x 8192 after prefixes 0, 8192, 24576, 57344)")
    prefix = [0, 8192, 24576, 57344]
    d = gen.varlen_inputs([C] * 4, [C + p for p in prefix], 64, 4, seed=1006, with_sinks=False)
    packs["global"] = dict(cfg=Bd.global_cfg(), d=d,
                           flops=FLOP_PER_PAIR_HEAD * 64 * sum(causal_pairs(p, p + C) for p in prefix))
    for pk in packs.values():
        d = pk["d"]
        hkv = pk["cfg"].num_kv_heads
        pk.update(q=dev_bf16(d["q"]), k=dev_bf16(d["k"]), v=dev_bf16(d["v"]), cu_q=dev(d["cu_q"]),
                  cu_k=dev(d["cu_k"]), kpos=None if d["k_pos0"] is None else dev(d["k_pos0"]),
                  sinks=None if d["sinks"] is None else dev(d["sinks"]),
                  out=torch.empty((4 * C, 64, 128), dtype=torch.bfloat16, device="cuda"),
                  bytes=4 * C * 64 * (192 + 128) * 2 + int(d["cu_k"][-1]) * hkv * (192 + 128) * 2)
        n = Bd.mimo_attn_prefill_workspace_size(pk["cfg"], 4, int(d["cu_k"][-1]))
        pk["ws"] = torch.empty(n, dtype=torch.uint8, device="cuda") if n else False
        del pk["d"]
    names = list(packs)

    def step(ev=None):
        for n in names:
            pk = packs[n]
            if ev is not None:
                ev[n][0].record()
            Bd.mimo_attn_prefill_varlen(pk["cfg"], pk["q"], pk["k"], pk["v"], pk["sinks"], pk["cu_q"], pk["cu_k"],
                                        C, pk["out"], k_pos0=pk["kpos"], ws=pk["ws"])
            if ev is not None:
                ev[n][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names}
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    ms = {n: float(np.mean([e[n][0].elapsed_time(e[n][1]) for e in evs])) for n in names}
    flops = sum(pk["flops"] for pk in packs.values())
    value = flops / (ms_step * 1e-3) / 1e12
    phases = {}
    for n, pk in packs.items():
        t = ms[n] * 1e-3
        phases[f"{n}_chunks_4x8192"] = {"ms": ms[n], "tflops": pk["flops"] / t / 1e12, "gbs": pk["bytes"] / t / 1e9,
                                        "frac_mfma_peak": pk["flops"] / t / 1e12 / PEAK_BF16_TFLOPS,
                                        "frac_hbm_peak": pk["bytes"] / t / 1e9 / PEAK_HBM_GBS}
    g = phases["global_chunks_4x8192"]
    out_j = {"metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
             "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
             "vs_baseline": None, "dtype": "bf16", "data": "synthetic: seeded N(0,1) bf16 q/k/v, N(0,1) fp32 sinks",
             "config": {"workload": "serving_chunks = packed sliding chunks 4x8192 (continuing at 8K..256K) + "
                                    "packed global chunks 4x8192 (prefixes 0..57344)"},
             "roofline": {"bound": "mfma", "kernel": "prefill_image_kernel (packed global chunks)", "achieved": g["tflops"],
                          "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": g["frac_mfma_peak"],
                          "traffic": None},
             "cpu_baseline": None, "phases": phases}
    print(json.dumps(out_j))


def main_spec_decode(args, torch, gen, Bd):
    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")

    cases = {}
    for nq in (4, 8):
        for name, S, hkv, window, seed in (("swa", 64, 8, 128, 1003), ("global", 16, 4, 0, 2003)):
            rng = np.random.Generator(np.random.PCG64(seed))
            if window:
                pos = rng.integers(128, 131072, size=S)
                cap = window + nq - 1
            else:
                pos = rng.integers(32768, 131072, size=S, endpoint=True) - 1
                cap = 131072
            log(f"setup: multi-query decode {name} S={S} n_q={nq} cap={cap}")
            d = gen.decode_multi_inputs(S, nq, cap, 64, hkv, seed=seed, window=window, pos=pos,
                                        with_sinks=window > 0)
            cfg = Bd.swa_cfg() if window else Bd.global_cfg()
            # keys any draft token sees, and the visible (query, key) pairs
            if window:
                seen = np.minimum(pos + 1, window + nq - 1)
                pairs = sum(min(max(int(p) - (nq - 1 - i) + 1, 0), window) for p in pos for i in range(nq))
            else:
                seen = pos + 1
                pairs = sum(max(int(p) - (nq - 1 - i) + 1, 0) for p in pos for i in range(nq))
            cases[f"{name}_nq{nq}"] = dict(
                cfg=cfg, q=_dev_bf16(torch, d["q"]), pos=dev(d["pos"]), kc=_dev_bf16(torch, d["k_cache"]),
                vc=_dev_bf16(torch, d["v_cache"]), sinks=None if d["sinks"] is None else dev(d["sinks"]),
                out=torch.empty((S, nq, 64, 128), dtype=torch.bfloat16, device="cuda"),
                ws=torch.empty(Bd.mimo_attn_decode_multi_workspace_size(cfg, S, nq, cap), dtype=torch.uint8,
                               device="cuda"),
                bytes=int(seen.sum()) * hkv * 320 * 2 + S * nq * 64 * (192 + 128) * 2,
                flops=FLOP_PER_PAIR_HEAD * 64 * pairs)
            del d
    names = list(cases)

    def step(ev=None):
        for n in names:
            c = cases[n]
            if ev is not None:
                ev[n][0].record()
            Bd.mimo_attn_decode_multi(c["cfg"], c["q"], c["pos"], c["kc"], c["vc"], c["sinks"], c["out"], ws=c["ws"])
            if ev is not None:
                ev[n][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names}
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    ms = {n: float(np.mean([e[n][0].elapsed_time(e[n][1]) for e in evs])) for n in names}
    phases = {}
    for n, c in cases.items():
        t = ms[n] * 1e-3
        phases[n] = {"ms": ms[n], "gbs": c["bytes"] / t / 1e9, "frac_hbm_peak": c["bytes"] / t / 1e9 / PEAK_HBM_GBS,
                     "tflops": c["flops"] / t / 1e12}
    total_bytes = sum(c["bytes"] for c in cases.values())
    value = total_bytes / (ms_step * 1e-3) / 1e9
    g = phases["global_nq8"]
    out_j = {"metric": METRIC, "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
             "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
             "vs_baseline": None, "dtype": "bf16", "data": "synthetic: seeded N(0,1) bf16 q and caches, N(0,1) fp32 sinks",
             "config": {"workload": "spec_decode = multi-query decode, 64 sliding + 16 global sequences, "
                                    "n_q = 4 and n_q = 8"},
             "roofline": {"bound": "hbm", "kernel": "decode_partial_kernel (global, 8 draft tokens)",
                          "achieved": g["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": g["frac_hbm_peak"],
                          "traffic": None},
             "cpu_baseline": None, "phases": phases}
    print(json.dumps(out_j))


def main_paged_decode(args, torch, gen, Bd):
    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")

    cases = {}
    for name, S, hkv, window, seed, kv in (("global_bf16", 16, 4, 0, 2003, "bf16"),
                                           ("global_fp8", 16, 4, 0, 2003, "fp8"),
                                           ("swa_fp8", 64, 8, 128, 1003, "fp8")):
        rng = np.random.Generator(np.random.PCG64(seed))
        if window:
            pos = rng.integers(128, 131072, size=S)
        else:
            pos = rng.integers(32768, 131072, size=S, endpoint=True) - 1
        log(f"setup: paged decode {name} S={S}")
        d = gen.paged_decode_inputs(S, 1, 128, 64, hkv, seed=seed, window=window, pos=pos, with_sinks=window > 0,
                                    kv_dtype=kv, k_scale=0.02, v_scale=0.03)
        cfg = Bd.swa_cfg() if window else Bd.global_cfg()
        seen = np.minimum(pos + 1, window) if window else pos + 1
        elem = 1 if kv == "fp8" else 2
        pool = (lambda a: dev(a)) if kv == "fp8" else (lambda a: _dev_bf16(torch, a))
        cases[name] = dict(
            cfg=cfg, q=_dev_bf16(torch, d["q"]), pos=dev(d["pos"]), kp=pool(d["k_pool"]), vp=pool(d["v_pool"]),
            table=dev(d["table"]), sinks=None if d["sinks"] is None else dev(d["sinks"]),
            out=torch.empty((S, 1, 64, 128), dtype=torch.bfloat16, device="cuda"),
            ws=torch.empty(Bd.mimo_attn_decode_multi_workspace_size(cfg, S, 1, 0), dtype=torch.uint8, device="cuda"),
            bytes=int(seen.sum()) * hkv * 320 * elem + S * 64 * (192 + 128) * 2,
            bf16_bytes=int(seen.sum()) * hkv * 320 * 2 + S * 64 * (192 + 128) * 2)
        del d
    names = list(cases)

    def step(ev=None):
        for n in names:
            c = cases[n]
            if ev is not None:
                ev[n][0].record()
            Bd.mimo_attn_decode_paged(c["cfg"], c["q"], c["pos"], c["kp"], c["vp"], c["table"], c["sinks"], c["out"],
                                      ws=c["ws"], k_scale=0.02, v_scale=0.03)
            if ev is not None:
                ev[n][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names}
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    ms = {n: float(np.mean([e[n][0].elapsed_time(e[n][1]) for e in evs])) for n in names}
    phases = {}
    for n, c in cases.items():
        t = ms[n] * 1e-3
        phases[n] = {"ms": ms[n], "gbs": c["bytes"] / t / 1e9, "frac_hbm_peak": c["bytes"] / t / 1e9 / PEAK_HBM_GBS,
                     "bf16_equivalent_gbs": c["bf16_bytes"] / t / 1e9}
    value = sum(c["bytes"] for c in cases.values()) / (ms_step * 1e-3) / 1e9
    g = phases["global_fp8"]
    out_j = {"metric": METRIC, "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
             "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
             "vs_baseline": None, "dtype": "bf16 compute; bf16 and fp8 e4m3 KV",
             "data": "synthetic: seeded N(0,1) bf16 q, N(0,1) KV as bf16 or e4m3 codes of x / scale",
             "config": {"workload": "paged_decode = 16 global sequences (bf16 and fp8 pools) + 64 sliding "
                                    "sequences (fp8 pools), 128-slot blocks"},
             "roofline": {"bound": "hbm", "kernel": "decode_partial_kernel (paged fp8, global)",
                          "achieved": g["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": g["frac_hbm_peak"],
                          "traffic": None},
             "cpu_baseline": None, "phases": phases}
    print(json.dumps(out_j))


def bench_backward(torch, gen, Bd, warmup, steps, src=None):
    """The sliding-window + sink backward at B=4, T=8192 (one call = k rotation, dq, d sink, dk/dv),
    timed with events on the current stream.  src: the layer step's sliding-prefill inputs on the
    device (the same seeded draw), reused when given."""
    B, T = 4, 8192
    cfg = Bd.swa_cfg()
    if src is None:
        log("setup: sliding-window prefill B=4 T=8192, forward once for its output and LSE")
        d = gen.prefill_inputs(B, T, 64, 8, seed=1001, with_sinks=True)
        q, k, v = _dev_bf16(torch, d["q"]), _dev_bf16(torch, d["k"]), _dev_bf16(torch, d["v"])
        sinks = torch.from_numpy(d["sinks"]).to("cuda")
        del d
    else:
        q, k, v, sinks = src["q"], src["k"], src["v"], src["sinks"]
    dout = _dev_bf16(torch, gen.normal_bf16(np.random.SeedSequence(1012), (B, T, 64, 128)))
    out = torch.empty((B, T, 64, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, 64, T), dtype=torch.float32, device="cuda")
    Bd.mimo_attn_prefill_swa(cfg, q, k, v, sinks, out, lse=lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dsinks = torch.empty(64, dtype=torch.float32, device="cuda")
    ws = torch.empty(Bd.mimo_attn_backward_workspace_size(cfg, B, T), dtype=torch.uint8, device="cuda")

    def step():
        Bd.mimo_attn_prefill_backward(cfg, q, k, v, sinks, out, lse, dout, dq, dk, dv, dsinks, ws=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    s_ev.record()
    for _ in range(steps):
        step()
    e_ev.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_ev = s_ev.elapsed_time(e_ev) / steps
    pairs = B * swa_pairs(T, 128)
    # one recompute of S, then dP, dV, dK, dQ: 2 * (3 * 192 + 2 * 128) FLOP per visible pair and head
    flops = 2 * (3 * 192 + 2 * 128) * 64 * pairs
    # read q, out, dO and write dq per (token, query head); read k, v and write dk, dv per (token, KV head);
    # read the LSE
    nbytes = B * T * (64 * (192 + 128 + 128 + 192) * 2 + 8 * (192 + 128) * 2 * 2) + B * 64 * T * 4
    tflops = flops / (ms_ev * 1e-3) / 1e12
    gbs = nbytes / (ms_ev * 1e-3) / 1e9
    return {"ms": ms_ev, "ms_wall": wall * 1e3 / steps, "tflops": tflops, "gbs": gbs,
            "frac_hbm_peak": gbs / PEAK_HBM_GBS, "frac_mfma_peak": tflops / PEAK_BF16_TFLOPS,
            "algorithmic_flops": flops, "algorithmic_bytes": nbytes, "traffic": profiled_backward_traffic()}


def main_backward(args, torch, gen, Bd):
    r = bench_backward(torch, gen, Bd, args.warmup, args.steps)
    ms_step = r["ms_wall"]
    out_j = {"metric": METRIC, "value": r["algorithmic_flops"] / (ms_step * 1e-3) / 1e12, "unit": "TFLOP/s",
             "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
             "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
             "data": "synthetic: seeded N(0,1) bf16 q/k/v/dO, N(0,1) fp32 sinks",
             "config": {"workload": "swa_backward_b4_t8192 (dq, dk, dv, d sink from the forward's output and LSE)"},
             "roofline": {"bound": "hbm", "kernel": "bwd_krot + bwd_dq + bwd_sink + bwd_dkdv (one call)",
                          "achieved": r["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": r["frac_hbm_peak"],
                          "traffic": r["traffic"], "algorithmic_flops": r["algorithmic_flops"],
                          "algorithmic_bytes": r["algorithmic_bytes"], "tflops": r["tflops"],
                          "frac_mfma_peak": r["frac_mfma_peak"]},
             "cpu_baseline": None, "ms_per_call_events": r["ms"]}
    print(json.dumps(out_j))


if __name__ == "__main__":
    main()
