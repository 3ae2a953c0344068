"""Helpers for the GPU parity tests: row sampling, tolerances and comparison
of libmfa output against the fp64 oracle."""
from __future__ import annotations

import math
import os

import numpy as np
import torch

from transformer_mfa_fwd_amd.workloads import Workload

# Tolerances on max-abs error against the fp64 oracle.
TOL_O = {"f32": 1e-4, "f16": 1e-2, "bf16": 1e-2}
TOL_LSE = 1e-3
MANT_BITS = {"f32": 23, "f16": 10, "bf16": 7}

ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of the output dtype at |x|: the rounding
    the output store itself must add, on top of the kernel's own error."""
    if dtype == "f32":
        return np.zeros_like(x)
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 1e-30)))
    if dtype == "f16":
        e = np.maximum(e, -14)
    return 0.5 * np.exp2(e - MANT_BITS[dtype])


def sample_rows(w: Workload, n_random: int = 16, seed: int = 1234):
    """(b, hq, i) rows to check: fixed rows at tile and window edges plus
    seeded random rows, for every (b, hq)."""
    L = w.Lq
    fixed = {0, 1, 2, 63, 64, 65, 127, 128, 129, 255, 256, L // 2 - 1, L // 2, L - 2, L - 1}
    if w.window > 0:
        fixed |= {w.window - 2, w.window - 1, w.window, w.window + 1, L - w.window, L - w.window // 2}
    rng = np.random.default_rng(seed)
    rows = []
    bs = range(w.B)
    for b in bs:
        extra = set()
        if w.mask == "pad_tail":
            extra = {"pad"}
        for h in range(w.Hq):
            rs = {i for i in fixed if 0 <= i < L}
            rs |= set(rng.integers(0, L, n_random).tolist())
            for i in sorted(rs):
                rows.append((b, h, i))
    return np.array(rows, dtype=np.int64).reshape(-1, 3)


def pad_boundary_rows(mask_cpu: torch.Tensor, w: Workload):
    """Rows around each batch's padding boundary (first masked key)."""
    rows = []
    for b in range(w.B):
        valid = int(mask_cpu[b].sum().item())
        for d in (-66, -65, -64, -63, -1, 0, 1, 63, 64, 65):
            i = valid + d
            if 0 <= i < w.Lq:
                for h in range(w.Hq):
                    rows.append((b, h, i))
    return np.array(rows, dtype=np.int64).reshape(-1, 3)


def gather_rows(out: torch.Tensor, lse: torch.Tensor, rows: np.ndarray):
    """GPU output at the given (b, hq, i) rows as float64 numpy arrays."""
    idx = torch.from_numpy(rows).to(out.device)
    o = out[idx[:, 0], idx[:, 2], idx[:, 1], :].double().cpu().numpy()
    l = None if lse is None else lse[idx[:, 0], idx[:, 1], idx[:, 2]].double().cpu().numpy()
    return o, l


def compare(dtype: str, o_gpu, l_gpu, o_ref, l_ref, what: str = "", o_scale: float = 1.0):
    """Assert the tolerances; returns (max O error, max LSE error).  o_scale
    multiplies the O tolerance: with dropout p the weights are formed (and
    rounded) before the factor 1 / (1 - p), so their error grows with it."""
    o_gpu = np.asarray(o_gpu, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    err = np.abs(o_gpu - o_ref)
    tol = TOL_O[dtype] * o_scale
    excess = err - (tol + half_ulp(o_ref, dtype))
    worst = int(np.argmax(excess)) if excess.size else 0
    assert excess.size == 0 or excess.flat[worst] <= 0, (
        f"{what}: |O - O_ref| = {err.flat[worst]:.3e} at flat index {worst} exceeds "
        f"{tol:.1e} + half-ulp (max abs err {err.max():.3e})")
    lerr = 0.0
    if l_gpu is not None:
        l_gpu = np.asarray(l_gpu, np.float64)
        l_ref = np.asarray(l_ref, np.float64)
        inf_ref = np.isneginf(l_ref)
        assert np.array_equal(np.isneginf(l_gpu), inf_ref), f"{what}: -inf LSE rows differ"
        fin = ~inf_ref
        if fin.any():
            lerr = float(np.max(np.abs(l_gpu[fin] - l_ref[fin])))
            assert lerr <= TOL_LSE, f"{what}: LSE error {lerr:.3e} > {TOL_LSE}"
        assert np.all(o_gpu[inf_ref] == 0.0), f"{what}: empty rows must be exactly 0"
    return float(err.max()) if err.size else 0.0, lerr


# Gradient tolerance: fp32 arithmetic throughout (1e-4); 16-bit inputs also
# round P and dS to the operand type and feed the backward libmfa's own
# rounded O (1e-2).
TOL_G = {"f32": 1e-4, "f16": 1e-2, "bf16": 1e-2}


def compare_grad(name: str, got, ref, dtype: str, what: str = "", dropout_p: float = 0.0):
    """Each gradient row (the D values of one query, key or value vector)
    within TOL_G * max(1, max |g_ref| over that row) / (1 - dropout_p) + half
    an ulp of the stored element.

    The bound is per row rather than per element: an element is a sum over
    many rows or keys whose terms can be much larger than their sum, and the
    operand rounding errs relative to the terms, not to the sum (a measured
    bf16 dV element of -0.057 built from terms near 1 is off by 0.014).  A
    whole wrong row or key block still fails.  Kept weights carry the factor
    1 / (1 - p) before they are rounded, so every term's rounding error grows
    with it, as for the forward's O under dropout.  Returns the max abs
    error."""
    got = got.double().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{what} {name}: non-finite gradient"
    err = np.abs(got - ref)
    row_scale = np.maximum(1.0, np.abs(ref).max(axis=-1, keepdims=True)) if ref.size else ref
    bound = TOL_G[dtype] * row_scale / (1.0 - dropout_p) + half_ulp(ref, dtype)
    worst = int(np.argmax(err - bound)) if err.size else 0
    assert err.size == 0 or err.flat[worst] <= bound.flat[worst], (
        f"{what} {name}: |g - g_ref| = {err.flat[worst]:.3e} > {bound.flat[worst]:.3e} at flat index "
        f"{worst} (g_ref {ref.flat[worst]:.3e}; max abs err {err.max():.3e})")
    return float(err.max()) if err.size else 0.0
