"""Benchmark of the fused attention forward (libmfa) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-decode] [--no-decode-len] [--no-decode-masked] [--no-softcap-window]
                    [--no-single-head]
                    [--no-packed] [--no-bias-dropout] [--no-backward]
                    [--no-cpu-baseline]

A step is one mfa_fwd call over one batch of synthetic input already resident
in HBM: the whole forward (tile ranges, Q/K/V staging, Q.K^T, soft-cap and
masks, online softmax, P.V, normalisation and LSE) for the workload.  The
default workload is the causal GQA prefill (B=4, L=2048, Hq=32, Hkv=8,
D=128, bf16); FLOPs count 4*D per visible (query, key) pair and query head.
The long-cache decode (B=64, Lk=32768, Hq=32, Hkv=8, D=128, bf16; split over
keys plus combine) is timed in the same run and reported under "decode" in
HBM GB/s of compulsory traffic, and so is the decode over a device-held length
(mfa_decode_len: 4 draft rows per batch on the same cache, full and half-full)
under "decode_len", and the decode over a cache whose valid keys a device mask
marks (mfa_decode_masked: all valid, valid keys with holes, and all valid with
a 4096-key window) under "decode_masked".  "softcap_window" times the causal sliding-window prefill
with soft-cap 50 (B=2, L=16384, Hq=16, Hkv=4, D=128, bf16, window 4096, 5 % of
keys masked, inputs of standard deviation 2) in visible-pair TFLOP/s.
"single_head_fp32" times the single-head causal fp32 workload (B=1, L=128,
D=64) in microseconds per call.
"packed_encoder" times the bidirectional encoder workload
(B=8, L=8192, H=12, D=64, fp16, window 128, tail padding) twice: padded with a
key mask through mfa_fwd, and packed without its padding through
mfa_packed_qkv_fwd.  "bias_mfma" times the causal GQA prefill with a
[1, 1, L, L] float32 additive mask (the MFMA kernel), "bias_dropout" the same
with dropout 0.1 and "dropout" dropout 0.1 alone (the MFMA kernel as well).  "backward" times mfa_bwd (dQ, dK, dV) on
the causal GQA prefill shape, and "backward_bias_dropout" the same with the mask
and dropout 0.1.

Calls take a caller-owned workspace (the allocation-free forms); the headline
is also timed through mfa_fwd's stream-ordered pool ("ms_per_step_pool").
Rank 0 prints one JSON line.  "roofline" describes the dominant kernel: its
average duration comes from HIP events that libmfa records on the launch
stream immediately around that kernel in every timed call
(mfa_set_kernel_events), and "traffic" is read from the committed rocprofv3
counter summary in profiles/ (null when the kernel sources changed since).
"warmup" is the requested count; "warmup_steps_run" the calls actually run
before timing, which continue until --warmup-ms has passed.
"cpu_baseline" times the fp64 CPU oracle on a bounded row sample of the same
workload on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (visible pairs) prefill + decode HBM GB/s, 1×MI355X"
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "transformer_mfa_fwd_amd", "csrc")


# ---------------------------------------------------------------------------
# work accounting
# ---------------------------------------------------------------------------

def visible_pairs(w, key_mask_cpu) -> int:
    """Visible (query row, key) pairs summed over batches and query heads,
    from the key-range bounds and prefix sums of the key mask."""
    i = np.arange(w.Lq, dtype=np.int64)
    aq = i + w.q_offset
    if w.causal:
        hi = aq.copy()
        lo = aq - w.window + 1 if w.window > 0 else np.zeros_like(aq)
    elif w.window > 0:
        lo, hi = aq - w.window // 2, aq + w.window // 2
    else:
        lo, hi = np.zeros_like(aq), np.full_like(aq, w.Lk - 1)
    lo = np.clip(lo, 0, None)
    hi = np.clip(hi, None, w.Lk - 1)
    total = 0
    for b in range(w.B):
        if key_mask_cpu is None:
            cnt = np.clip(hi - lo + 1, 0, None)
        else:
            keep = (key_mask_cpu[b].numpy() > 0.5).astype(np.int64)
            pre = np.concatenate([[0], np.cumsum(keep)])
            cnt = np.where(hi >= lo, pre[np.clip(hi + 1, 0, w.Lk)] - pre[np.clip(lo, 0, w.Lk)], 0)
        total += int(cnt.sum())
    return total * w.Hq


def algorithmic_bytes(w, q) -> int:
    """Compulsory HBM traffic: read Q, K, V (and the mask), write O and LSE."""
    es = q.element_size()
    n = (w.B * w.Lq * w.Hq * w.D * 2 + w.B * w.Lk * w.Hkv * w.D * 2) * es + w.B * w.Hq * w.Lq * 4
    if w.mask is not None:
        n += w.B * w.Lk * 4
    return n


def kernel_source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


PREFILL_SOURCES = ["kernels_mfma.hip", "mfa_device.h", "mfa_internal.h"]
DECODE_SOURCES = ["kernels_decode.hip", "mfa_device.h", "mfa_internal.h"]


def measured_traffic(name: str, sources) -> tuple:
    """Per-launch HBM bytes from the committed counter summary, if it was taken
    on the current kernel sources; else (None, reason)."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None, "no counter summary"
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash(sources):
        return None, "kernel changed since counters were taken"
    return rec.get("traffic_bytes_per_launch"), rec.get("note", "")


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------

def timed(fn, steps: int, warmup: int, warmup_ms: float = 0.0) -> dict:
    """Run fn() W times untimed (continued until warmup_ms has passed too: the
    GPU clocks take a few hundred milliseconds of load to settle), then K
    timed times back to back with nothing between the calls (wall clock, and
    HIP events around the whole loop), then K more with HIP events on the
    launch stream around each call and, attached by libmfa to its main
    kernel's dispatch (mfa_set_kernel_events), around that kernel.  Returns
    wall ms per call, GPU ms per call of the plain loop, the per-call
    events' averages and the number of warm-up calls run."""
    import torch
    import transformer_mfa_fwd_amd as mfa

    n_warm = 0
    t_w = time.perf_counter()
    while n_warm < warmup or (time.perf_counter() - t_w) * 1e3 < warmup_ms:
        fn()
        n_warm += 1
        if n_warm % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    # plain loop: the throughput a caller sees
    s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    s0.record(stream)
    for _ in range(steps):
        fn()
    e0.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    gpu_ms = s0.elapsed_time(e0) / steps

    # instrumented loop: each call and its main kernel
    def events():
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:         # created on first record
            a.record(stream)
            b.record(stream)
        return ev
    call_ev, kern_ev = events(), events()
    torch.cuda.synchronize()
    for (cs, ce), (ks, ke) in zip(call_ev, kern_ev):
        mfa.set_kernel_events(ks, ke)
        cs.record(stream)
        fn()
        ce.record(stream)
    torch.cuda.synchronize()
    mfa.set_kernel_events(None, None)
    kern = [a.elapsed_time(b) for a, b in kern_ev]
    return dict(wall_ms=wall_ms, gpu_ms=gpu_ms, call_ms=float(np.mean([a.elapsed_time(b) for a, b in call_ev])),
                kernel_ms=float(np.mean(kern)), kernel_ms_min=float(np.min(kern)), warmup_run=n_warm)


def time_workload(w, steps: int, warmup: int, seed: int = 0, warmup_ms: float = 0.0, pool: bool = False):
    """mfa_fwd on workload w with a caller-owned workspace (mfa_fwd_ws, the
    allocation-free form) or, with ``pool``, from the library's pool."""
    import torch
    import transformer_mfa_fwd_amd as mfa
    from transformer_mfa_fwd_amd import workloads as wl

    q, k, v, m = wl.make_inputs(w, "cuda", seed)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Lq), dtype=torch.float32, device=q.device)
    nbytes = mfa.workspace_size(w.B, w.Lq, w.Lk, w.Hq, w.Hkv, w.D, q.dtype)
    ws = None if pool or nbytes == 0 else torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    kw = dict(causal=w.causal, window=w.window, q_offset=w.q_offset, softcap=w.softcap,
              key_mask=m, scale=w.scale, out=out, lse=lse, workspace=ws)
    r = timed(lambda: mfa.fwd(q, k, v, **kw), steps, warmup, warmup_ms)
    r.update(path=mfa.plan(w.B, w.Lq, w.Lk, w.Hq, w.Hkv, w.D, q.dtype)[0],
             pairs=visible_pairs(w, None if m is None else m.cpu()), bytes=algorithmic_bytes(w, q))
    del ws, out, lse
    return r, (q, k, v, m)


def time_decode_len(w, lens_cpu, steps: int, warmup: int, warmup_ms: float = 0.0, seed: int = 0):
    """mfa_decode_len on workload w (Lq = draft rows R, Lk = capacity) with the
    given per-batch lengths, timed like time_workload.  Algorithmic bytes: Q and
    O, the LSE, the lengths and the K and V rows below each length."""
    import torch
    import transformer_mfa_fwd_amd as mfa
    from transformer_mfa_fwd_amd import workloads as wl

    q, k, v, _ = wl.make_inputs(w, "cuda", seed)
    d_len = lens_cpu.to("cuda")
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Lq), dtype=torch.float32, device=q.device)
    nbytes = mfa.decode_len_workspace_size(w.B, w.Lq, w.Lk, w.Hq, w.Hkv, w.D, q.dtype)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    r = timed(lambda: mfa.decode_len(q, k, v, d_len, out=out, lse=lse, workspace=ws), steps, warmup, warmup_ms)
    el = q.element_size()
    valid = int(lens_cpu.clamp(0, w.Lk).sum())
    r["bytes"] = (2 * q.numel() * el + lse.numel() * 4 + w.B * 4 + 2 * valid * w.Hkv * w.D * el)
    r["valid_keys"] = valid
    del q, k, v, out, lse, ws
    torch.cuda.empty_cache()
    return r


def time_decode_masked(w, mask_cpu, window: int, steps: int, warmup: int, warmup_ms: float = 0.0, seed: int = 0):
    """mfa_decode_masked on workload w (one query row per batch, Lk = capacity)
    with the given [B, Lk] validity mask.  Algorithmic bytes: Q, O, the LSE,
    the mask and the K and V rows of the used keys (valid, and inside the
    window when there is one): the rows the kernel must read, and the only
    ones it reads."""
    import torch
    import transformer_mfa_fwd_amd as mfa
    from transformer_mfa_fwd_amd import workloads as wl

    q, k, v, _ = wl.make_inputs(w, "cuda", seed)
    d_mask = mask_cpu.to("cuda")
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, 1), dtype=torch.float32, device=q.device)
    nbytes = mfa.decode_masked_workspace_size(w.B, w.Lk, w.Hq, w.Hkv, w.D, q.dtype)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    r = timed(lambda: mfa.decode_masked(q, k, v, d_mask, window=window, out=out, lse=lse, workspace=ws),
              steps, warmup, warmup_ms)
    el = q.element_size()
    used_keys = 0
    for b in range(w.B):
        valid = np.nonzero(mask_cpu[b].numpy() > 0.5)[0]
        if valid.size == 0:
            continue
        used = valid[valid > valid[-1] - window] if window > 0 else valid
        used_keys += used.size
    r["bytes"] = 2 * q.numel() * el + lse.numel() * 4 + mask_cpu.numel() * 4 + 2 * used_keys * w.Hkv * w.D * el
    del q, k, v, out, lse, ws, d_mask
    torch.cuda.empty_cache()
    return r


def time_calls(fn, steps: int, warmup: int, warmup_ms: float = 0.0):
    """(wall ms per call, main-kernel ms per call) of fn()."""
    r = timed(fn, steps, warmup, warmup_ms)
    return r["wall_ms"], r["kernel_ms"]


def packed_encoder(steps: int, warmup: int, warmup_ms: float):
    """The padded encoder workload against its packed form, which carries no
    padding rows (so it also drops the padding rows' pairs)."""
    import torch
    import transformer_mfa_fwd_amd as mfa
    from transformer_mfa_fwd_amd import workloads as wl

    w = wl.BIDIR_WINDOW_ENCODER_FP16
    res = {"workload": w.name, "unit": "TFLOP/s"}
    q, k, v, m = wl.make_inputs(w, "cuda")
    pairs = visible_pairs(w, m.cpu())
    out = torch.empty_like(q)
    wall, kern = time_calls(lambda: mfa.fwd(q, k, v, causal=False, window=w.window, key_mask=m,
                                            out=out, return_lse=False), steps, warmup, warmup_ms)
    # compulsory bytes of the call (no LSE is written): Q, K, V, the mask, O
    pbytes = (2 * w.B * w.Lq * w.Hq * w.D + 2 * w.B * w.Lk * w.Hkv * w.D) * q.element_size() + w.B * w.Lk * 4
    res["padded"] = {"api": "mfa_fwd + key mask", "rows": w.B * w.Lq, "ms_per_step": round(wall, 5),
                     "kernel_ms_avg": round(kern, 5),
                     "visible_pairs": pairs, "value": round(4.0 * w.D * pairs / (wall * 1e-3) / 1e12, 2),
                     "algorithmic_bytes": pbytes, "hbm_gbs": round(pbytes / (kern * 1e-3) / 1e9, 1),
                     "hbm_frac": round(pbytes / (kern * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del q, k, v, m, out
    torch.cuda.empty_cache()
    lengths = wl.encoder_packing_lengths(w)
    qkv, sb = wl.make_packed_qkv(lengths, w.Hq, w.D, w.dtype, "cuda")
    out = torch.empty((qkv.shape[0], w.Hq * w.D), dtype=qkv.dtype, device="cuda")
    wall, kern = time_calls(lambda: mfa.packed_qkv_fwd(qkv, sb, w.Hq, window=w.window, out=out,
                                                       return_lse=False), steps, warmup, warmup_ms)
    half = w.window // 2
    # the padded form also counts its padding rows' pairs with valid keys near the boundary
    ppairs = w.Hq * sum(sum(min(n - 1, r + half) - max(0, r - half) + 1 for r in range(n)) for n in lengths)
    # compulsory bytes: the fused QKV rows, the sequence bounds, O
    kbytes = (qkv.numel() + out.numel()) * qkv.element_size() + sb.numel() * sb.element_size()
    res["packed"] = {"api": "mfa_packed_qkv_fwd", "rows": int(qkv.shape[0]), "ms_per_step": round(wall, 5),
                     "kernel_ms_avg": round(kern, 5),
                     "visible_pairs": ppairs, "value": round(4.0 * w.D * ppairs / (wall * 1e-3) / 1e12, 2),
                     "algorithmic_bytes": kbytes, "hbm_gbs": round(kbytes / (kern * 1e-3) / 1e9, 1),
                     "hbm_frac": round(kbytes / (kern * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del qkv, sb, out
    torch.cuda.empty_cache()
    return res


def single_head_fp32(steps: int, warmup: int, warmup_ms: float):
    """The single-head causal fp32 workload (B=1, L=128, D=64): bound by launch
    latency, so it is reported in microseconds per call."""
    import torch
    from transformer_mfa_fwd_amd import workloads as wl

    w = wl.SINGLE_HEAD_CAUSAL_FP32
    r, t = time_workload(w, steps, warmup, warmup_ms=warmup_ms)
    del t
    torch.cuda.empty_cache()
    return {"workload": w.name, "path": r["path"], "unit": "us per call",
            "us_per_call_wall": round(r["wall_ms"] * 1e3, 2), "us_per_call_kernel": round(r["kernel_ms"] * 1e3, 2),
            "visible_pairs": r["pairs"]}


def softcap_window(steps: int, warmup: int, warmup_ms: float):
    """The causal sliding-window GQA prefill with soft-cap and a sparse key mask
    (MFMA kernel, soft-capped and masked instantiation)."""
    import torch
    from transformer_mfa_fwd_amd import workloads as wl

    w = wl.CAUSAL_WINDOW_SOFTCAP_BF16
    r, t = time_workload(w, steps, warmup, warmup_ms=warmup_ms)
    del t
    torch.cuda.empty_cache()
    flops = 4.0 * w.D * r["pairs"]
    kern = r["kernel_ms"]
    return {"workload": w.name, "path": r["path"], "unit": "TFLOP/s", "input_std": w.std,
            "ms_per_step": round(r["wall_ms"], 5), "kernel_ms_avg": round(kern, 5),
            "visible_pairs": r["pairs"], "value": round(flops / (r["wall_ms"] * 1e-3) / 1e12, 2),
            "roofline": {"bound": "mfma", "achieved": round(flops / (kern * 1e-3) / 1e12, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(flops / (kern * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "algorithmic_flops_per_launch": flops}}


def bias_mfma(steps: int, warmup: int, warmup_ms: float):
    """The prefill shape with a [1, 1, L, L] additive mask and no dropout: the
    MFMA kernel's BIAS instantiation."""
    import torch
    import transformer_mfa_fwd_amd as mfa
    from transformer_mfa_fwd_amd import workloads as wl

    w = wl.GQA_CAUSAL_PREFILL_BF16
    q, k, v, _ = wl.make_inputs(w, "cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    bias = torch.randn((1, 1, w.Lq, w.Lk), generator=g, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Lq), dtype=torch.float32, device="cuda")
    wall, kern = time_calls(lambda: mfa.fwd(q, k, v, causal=True, bias=bias, out=out, lse=lse), steps, warmup,
                            warmup_ms)
    pairs = visible_pairs(w, None)
    res = {"workload": w.name, "api": "mfa_fwd_bias_dropout", "bias_shape": [1, 1, w.Lq, w.Lk], "dropout_p": 0.0,
           "path": "mfma", "unit": "TFLOP/s", "ms_per_step": round(wall, 5), "kernel_ms_avg": round(kern, 5),
           "value": round(4.0 * w.D * pairs / (wall * 1e-3) / 1e12, 2)}
    del q, k, v, bias, out, lse
    torch.cuda.empty_cache()
    return res


def bias_dropout(steps: int, warmup: int, warmup_ms: float, with_bias: bool = True):
    """The prefill shape with dropout 0.1, with or without a [1, 1, L, L]
    additive mask: the MFMA kernel's DROP instantiations."""
    import torch
    import transformer_mfa_fwd_amd as mfa
    from transformer_mfa_fwd_amd import workloads as wl

    w = wl.GQA_CAUSAL_PREFILL_BF16
    q, k, v, _ = wl.make_inputs(w, "cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    bias = torch.randn((1, 1, w.Lq, w.Lk), generator=g, device="cuda") if with_bias else None
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Lq), dtype=torch.float32, device="cuda")
    wall, kern = time_calls(lambda: mfa.fwd(q, k, v, causal=True, bias=bias, dropout_p=0.1, seed=5,
                                            out=out, lse=lse), steps, warmup, warmup_ms)
    pairs = visible_pairs(w, None)
    res = {"workload": w.name, "api": "mfa_fwd_bias_dropout",
           "bias_shape": [1, 1, w.Lq, w.Lk] if with_bias else None,
           "dropout_p": 0.1, "path": "mfma", "unit": "TFLOP/s", "ms_per_step": round(wall, 5),
           "kernel_ms_avg": round(kern, 5), "value": round(4.0 * w.D * pairs / (wall * 1e-3) / 1e12, 2)}
    del q, k, v, bias, out, lse
    torch.cuda.empty_cache()
    return res


def backward(steps: int, warmup: int, warmup_ms: float, extras: bool = False):
    """mfa_bwd on the prefill shape; with ``extras`` the forward and backward
    carry a [1, 1, L, L] additive mask and dropout 0.1."""
    import torch
    import transformer_mfa_fwd_amd as mfa
    from transformer_mfa_fwd_amd import workloads as wl

    w = wl.GQA_CAUSAL_PREFILL_BF16
    q, k, v, _ = wl.make_inputs(w, "cuda")
    kw = dict(causal=True)
    if extras:
        g = torch.Generator(device="cuda")
        g.manual_seed(1)
        kw.update(bias=torch.randn((1, 1, w.Lq, w.Lk), generator=g, device="cuda"), dropout_p=0.1, seed=5)
    out, lse = mfa.fwd(q, k, v, **kw)
    dout = torch.randn(q.shape, device="cuda").to(q.dtype)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    r = timed(lambda: mfa.bwd(q, k, v, out, dout, lse, dq=dq, dk=dk, dv=dv, **kw), steps, warmup, warmup_ms)
    wall, kern = r["wall_ms"], r["call_ms"]     # the backward's three kernels
    pairs = visible_pairs(w, None)
    res = {"workload": w.name, "api": "mfa_bwd", "path": "mfma", "unit": "TFLOP/s",
           "flops_per_pair": 10 * w.D, "ms_per_step": round(wall, 5), "kernel_ms_avg": round(kern, 5),
           "value": round(10.0 * w.D * pairs / (wall * 1e-3) / 1e12, 2)}
    if extras:
        res.update(bias_shape=[1, 1, w.Lq, w.Lk], dropout_p=0.1)
    del q, k, v, out, lse, dout, dq, dk, dv, kw
    torch.cuda.empty_cache()
    return res


def cpu_baseline(w, tensors, target_s: float = 12.0, seed: int = 0):
    """Time the fp64 oracle on a seeded sample of query rows of the workload."""
    from oracle import default_oracle
    q, k, v, m = tensors
    orc = default_oracle()
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    qc, kc, vc = (t.float().cpu() for t in (q, k, v))
    mc = None if m is None else m.cpu()
    rng = np.random.default_rng(seed)
    b, h, i = np.meshgrid(np.arange(w.B), np.arange(w.Hq), np.arange(w.Lq), indexing="ij")
    rows = np.stack([b.ravel(), h.ravel(), i.ravel()], 1)[rng.permutation(w.B * w.Hq * w.Lq)]
    kw = dict(scale=w.scale, causal=w.causal, window=w.window, q_offset=w.q_offset,
              softcap=w.softcap, key_mask=mc, nthreads=cores)
    # calibrate on a small prefix, then size the sample for ~target_s seconds
    n_cal = min(len(rows), 64 * cores)
    t0 = time.perf_counter()
    _, _, nv = orc.rows(qc, kc, vc, rows[:n_cal], **kw)
    dt = max(time.perf_counter() - t0, 1e-6)
    n = int(min(len(rows), max(n_cal, n_cal * target_s / dt)))
    sample = rows[:n]
    t0 = time.perf_counter()
    _, _, nv = orc.rows(qc, kc, vc, sample, **kw)
    dt = time.perf_counter() - t0
    pairs = int(nv.sum())
    total_pairs = visible_pairs(w, mc)
    return {"value": 4.0 * w.D * pairs / dt / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "pairs_per_s": round(pairs / dt),
            "full_workload_s_extrapolated": round(total_pairs / (pairs / dt), 2),
            "sample": f"{n} of {len(rows)} query rows (seeded shuffle), {pairs} visible pairs, "
                      f"{dt:.1f} s, fp64 C oracle with {cores} threads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-ms", type=float, default=300.0,
                    help="keep warming up until this much time has passed (clock ramp)")
    ap.add_argument("--workload", default="gqa_causal_prefill_bf16")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-decode-len", action="store_true")
    ap.add_argument("--no-decode-masked", action="store_true")
    ap.add_argument("--no-softcap-window", action="store_true")
    ap.add_argument("--no-single-head", action="store_true")
    ap.add_argument("--no-packed", action="store_true")
    ap.add_argument("--no-bias-dropout", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB --steps times (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: libmfa has no multi-GPU path "
              "(every call runs on one device); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from transformer_mfa_fwd_amd import workloads as wl

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n * 4, "launches": args.steps}))
        return

    match = [x for x in wl.ALL if x.name.startswith(args.workload)]
    if not match:
        raise SystemExit(f"unknown workload {args.workload}; choose from {[x.name for x in wl.ALL]}")
    w = match[0]

    res, tensors = time_workload(w, args.steps, args.warmup, warmup_ms=args.warmup_ms)
    flops = 4.0 * w.D * res["pairs"]
    tflops_wall = flops / (res["wall_ms"] * 1e-3) / 1e12
    kern_ms = res["kernel_ms"]
    is_prefill = res["path"] in ("mfma", "generic")
    traffic, tnote = measured_traffic(f"{'prefill' if is_prefill else 'decode'}_{w.name}.counters.json",
                                      PREFILL_SOURCES if is_prefill else DECODE_SOURCES)
    # a prefill whose flops per compulsory byte fall below the ridge point
    # (peak flops / peak bandwidth) is bound by HBM, not by the matrix cores
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if is_prefill and flops / res["bytes"] >= ridge:
        roof = {"bound": "mfma", "achieved": round(flops / (kern_ms * 1e-3) / 1e12, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(res["bytes"] / (kern_ms * 1e-3) / 1e9, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = traffic
    roof["kernel"] = {"mfma": "v16_prepass_kernel + prefill_kernel" if w.dtype == "bf16" else "prefill_kernel",
                      "generic": "generic_fwd_kernel",
                      "split_decode": "decode_split_kernel + decode_combine_kernel"}[res["path"]]
    roof["kernel_ms_avg"] = round(kern_ms, 5)
    roof["algorithmic_flops_per_launch"] = flops
    roof["algorithmic_bytes_per_launch"] = res["bytes"]
    if traffic is None:
        roof["traffic_note"] = tnote

    line = {
        "metric": METRIC,
        "value": round(tflops_wall if is_prefill else res["bytes"] / (res["wall_ms"] * 1e-3) / 1e9, 2),
        "unit": "TFLOP/s" if is_prefill else "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "warmup_steps_run": res["warmup_run"], "warmup_ms": args.warmup_ms,
        "ms_per_step": round(res["wall_ms"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Lq": w.Lq, "Lk": w.Lk, "Hq": w.Hq, "Hkv": w.Hkv,
                   "D": w.D, "causal": w.causal, "window": w.window, "softcap": w.softcap,
                   "key_mask": w.mask, "path": res["path"], "visible_pairs": res["pairs"],
                   "api": "mfa_fwd_ws (caller-owned workspace)"},
        "roofline": roof,
        # GPU time per call of the plain loop; and, from the instrumented
        # loop, the whole call (events around it) less the main kernel (for
        # bf16 the V conversion plus the prefill): key-mask packing, launch
        # gaps and the event markers themselves
        "gpu_ms_per_step": round(res["gpu_ms"], 5),
        "call_ms_avg": round(res["call_ms"], 5),
        "outside_main_kernel_ms": round(res["call_ms"] - kern_ms, 5),
    }
    # the same calls with the workspace from the library's stream-ordered pool (mfa_fwd)
    del tensors
    torch.cuda.empty_cache()
    rp, tensors = time_workload(w, args.steps, args.warmup, warmup_ms=50.0, pool=True)
    line["ms_per_step_pool"] = round(rp["wall_ms"], 5)

    if not args.no_decode and w is not wl.LONG_CACHE_DECODE_BF16:
        del tensors
        torch.cuda.empty_cache()
        wd = wl.LONG_CACHE_DECODE_BF16
        rd, td = time_workload(wd, max(10, args.steps // 2), max(3, args.warmup // 2),
                               warmup_ms=args.warmup_ms)
        dtraffic, dnote = measured_traffic(f"decode_{wd.name}.counters.json", DECODE_SOURCES)
        dk = rd["kernel_ms"]
        line["decode"] = {
            "workload": wd.name, "path": rd["path"], "unit": "GB/s",
            "value": round(rd["bytes"] / (rd["wall_ms"] * 1e-3) / 1e9, 1),
            "ms_per_step": round(rd["wall_ms"], 5),
            "roofline": {"bound": "hbm", "achieved": round(rd["bytes"] / (dk * 1e-3) / 1e9, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(rd["bytes"] / (dk * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "traffic": dtraffic, "kernel_ms_avg": round(dk, 5),
                         "algorithmic_bytes_per_launch": rd["bytes"]},
        }
        if dtraffic is None:
            line["decode"]["roofline"]["traffic_note"] = dnote
        del td
        torch.cuda.empty_cache()
        tensors = None

    if not args.no_decode_len:
        del tensors
        torch.cuda.empty_cache()
        tensors = None
        wl_len = wl.DEVICE_LENGTH_DECODE_BF16
        dl = {"workload": wl_len.name, "api": "mfa_decode_len", "unit": "GB/s", "R": wl_len.Lq,
              "capacity": wl_len.Lk, "peak": PEAK_HBM_GBS}
        for tag, fill in (("full", 1.0), ("half", 0.5)):
            lens = torch.full((wl_len.B,), int(wl_len.Lk * fill), dtype=torch.int32)
            r = time_decode_len(wl_len, lens, max(10, args.steps // 2), max(3, args.warmup // 2),
                                warmup_ms=args.warmup_ms)
            dl[tag] = {"lengths": int(lens[0]), "value": round(r["bytes"] / (r["wall_ms"] * 1e-3) / 1e9, 1),
                       "ms_per_step": round(r["wall_ms"], 5), "kernel_ms_avg": round(r["kernel_ms"], 5),
                       "achieved": round(r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9, 1),
                       "frac": round(r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                       "algorithmic_bytes_per_launch": r["bytes"]}
        line["decode_len"] = dl

    if not args.no_decode_masked:
        tensors = None
        torch.cuda.empty_cache()
        wm = wl.LONG_CACHE_DECODE_BF16
        dm = {"workload": wm.name, "api": "mfa_decode_masked", "unit": "GB/s", "capacity": wm.Lk,
              "peak": PEAK_HBM_GBS,
              "bytes_note": "Q, O, LSE, the mask and the K/V rows of the used keys"}
        full = torch.ones((wm.B, wm.Lk))
        holes = wl.make_cache_masks(wm.B, wm.Lk, seed=3, edges=False)
        for tag, mask, window in (("full", full, 0), ("holes", holes, 0), ("window4096", full, 4096)):
            r = time_decode_masked(wm, mask, window, max(10, args.steps // 2), max(3, args.warmup // 2),
                                   warmup_ms=args.warmup_ms)
            dm[tag] = {"window": window, "valid_keys": int((mask > 0.5).sum()),
                       "value": round(r["bytes"] / (r["wall_ms"] * 1e-3) / 1e9, 1),
                       "ms_per_step": round(r["wall_ms"], 5), "kernel_ms_avg": round(r["kernel_ms"], 5),
                       "achieved": round(r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9, 1),
                       "frac": round(r["bytes"] / (r["kernel_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                       "algorithmic_bytes_per_launch": r["bytes"]}
        line["decode_masked"] = dm

    if not args.no_single_head and w is not wl.SINGLE_HEAD_CAUSAL_FP32:
        line["single_head_fp32"] = single_head_fp32(max(20, args.steps), max(5, args.warmup), 50.0)

    if not args.no_softcap_window and w is not wl.CAUSAL_WINDOW_SOFTCAP_BF16:
        tensors = None
        torch.cuda.empty_cache()
        line["softcap_window"] = softcap_window(max(10, args.steps // 2), max(3, args.warmup // 2),
                                                args.warmup_ms)

    if not args.no_packed:
        tensors = None
        torch.cuda.empty_cache()
        line["packed_encoder"] = packed_encoder(max(10, args.steps // 2), max(3, args.warmup // 2),
                                                args.warmup_ms)

    if not args.no_bias_dropout:
        tensors = None
        torch.cuda.empty_cache()
        line["bias_mfma"] = bias_mfma(max(10, args.steps // 2), max(3, args.warmup // 2), args.warmup_ms)
        line["bias_dropout"] = bias_dropout(max(10, args.steps // 2), max(3, args.warmup // 2), args.warmup_ms)
        line["dropout"] = bias_dropout(max(10, args.steps // 2), max(3, args.warmup // 2), args.warmup_ms,
                                       with_bias=False)

    if not args.no_backward:
        tensors = None
        torch.cuda.empty_cache()
        line["backward"] = backward(5, 2, args.warmup_ms)
        line["backward_bias_dropout"] = backward(5, 2, args.warmup_ms, extras=True)

    if not args.no_cpu_baseline:
        if tensors is None:
            _, tensors = time_workload(w, 1, 0)
        line["cpu_baseline"] = cpu_baseline(w, tensors)

    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
