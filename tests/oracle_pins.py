"""Pins for the fp64 oracle: checks against facts other than the oracle itself.

Each ``pin_*`` function takes a loaded ``oracle.Oracle`` and raises
AssertionError when the oracle disagrees with what the pages or the
mathematics fix.  The checks use independent formulations: the window rules as
other functions on the pages state them, torch's float64 attention (a library
special case), a dense NumPy/SciPy formulation, closed forms (Q = 0, V = 1,
V = I, single visible key) and invariants (GQA head grouping, decode as the
last prefill row, mask tail as a shorter key axis, window limits, perturbation
of invisible keys).  ``ALL_PINS`` lists them for the mutation test.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch
from scipy.special import logsumexp

TIGHT = 1e-12
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(rng, shape, std=1.0):
    return (rng.standard_normal(shape) * std).astype(np.float32)


# ---------------------------------------------------------------------------
# independent statements of the visibility rule
# ---------------------------------------------------------------------------

def vis_causal_p1(aq, j, w):
    """ferrotensor attention.rs, AttentionOptions: a key is visible when it is
    not after the query and, with a window, closer than ``w`` positions."""
    return j <= aq and (w <= 0 or abs(aq - j) < w)


def vis_causal_p4(i, j, w):
    """forge attention.metal forward kernel (no offset): keys from
    i+1-w (when i+1 > w and w > 0) up to i."""
    jmax = i
    jmin = i + 1 - w if (w > 0 and i + 1 > w) else 0
    return jmin <= j <= jmax


def vis_bidir_packed(aq, j, w):
    """brotensor flash_attention.h, packed-QKV forward: with a window, keys
    within window/2 (integer halving) of the row; without one, every key."""
    return w <= 0 or abs(aq - j) <= w // 2


def dense_visibility(Lq, Lk, causal, window, q_offset, mask_b=None):
    """[Lq, Lk] boolean visibility from the statements above."""
    vis = np.zeros((Lq, Lk), bool)
    for i in range(Lq):
        aq = i + q_offset
        for j in range(Lk):
            ok = vis_causal_p1(aq, j, window) if causal else vis_bidir_packed(aq, j, window)
            if mask_b is not None and not (mask_b[j] > 0.5):
                ok = False
            vis[i, j] = ok
    return vis


# ---------------------------------------------------------------------------
# dense formulation (full score matrix, additive -inf mask, SciPy logsumexp)
# ---------------------------------------------------------------------------

def dense_reference(q, k, v, *, scale, causal, window, q_offset, softcap=0.0, key_mask=None):
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    kr = np.repeat(k, g, axis=2)          # head h uses kv head h // g
    vr = np.repeat(v, g, axis=2)
    O = np.zeros((B, Lq, Hq, D))
    L = np.zeros((B, Hq, Lq))
    for b in range(B):
        vis = dense_visibility(Lq, Lk, causal, window, q_offset,
                               None if key_mask is None else np.asarray(key_mask)[b])
        for h in range(Hq):
            s = scale * (q[b, :, h, :] @ kr[b, :, h, :].T)
            if softcap > 0:
                s = softcap * np.tanh(s / softcap)
            s = np.where(vis, s, -np.inf)
            lse = logsumexp(s, axis=1)
            empty = ~vis.any(1)
            lse[empty] = -np.inf
            p = np.where(vis, np.exp(s - np.where(empty, 0.0, lse)[:, None]), 0.0)
            O[b, :, h, :] = p @ vr[b, :, h, :]
            L[b, h, :] = lse
    return O, L


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), f"{what}: finiteness differs"
    assert np.array_equal(a[~fin], b[~fin]), f"{what}: infinities differ"
    if fin.any():
        err = np.max(np.abs(a[fin] - b[fin]))
        assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_range_causal_matches_ferrotensor_rule(orc):
    for Lk in range(1, 26):
        for aq in range(Lk):
            for w in range(-1, Lk + 3):
                lo, hi = orc.key_range(aq, Lk, True, w)
                got = {j for j in range(Lk) if lo <= j <= hi}
                want = {j for j in range(Lk) if vis_causal_p1(aq, j, w)}
                assert got == want, ("causal range", Lk, aq, w, got, want)


def pin_range_causal_matches_forge_rule(orc):
    for T in range(1, 26):
        for i in range(T):
            for w in range(0, T + 3):
                lo, hi = orc.key_range(i, T, True, w)
                got = {j for j in range(T) if lo <= j <= hi}
                want = {j for j in range(T) if vis_causal_p4(i, j, w)}
                assert got == want, ("forge causal range", T, i, w)


def pin_range_bidirectional_matches_packed_rule(orc):
    for Lk in range(1, 26):
        for aq in range(Lk):
            for w in range(-1, 2 * Lk + 3):
                lo, hi = orc.key_range(aq, Lk, False, w)
                got = {j for j in range(Lk) if lo <= j <= hi}
                want = {j for j in range(Lk) if vis_bidir_packed(aq, j, w)}
                assert got == want, ("bidirectional range", Lk, aq, w)


def pin_golden_visibility_tables(orc):
    """Hand-worked visibility tables under tests/golden (see the file)."""
    path = os.path.join(GOLDEN, "visibility_tables.txt")
    cases = _parse_tables(path)
    assert len(cases) >= 4
    for hdr, table in cases:
        B, Lq, Lk = 1, hdr["Lq"], hdr["Lk"]
        mask = None
        if "masked" in hdr:
            mask = np.ones((1, Lk), np.float32)
            mask[0, hdr["masked"]] = 0.0
        counts, _ = orc.visible_counts(B, Lq, Lk, causal=hdr["causal"], window=hdr["window"],
                                       q_offset=hdr["q_offset"], key_mask=mask)
        # V = I and Q = 0 reveal the exact visible set of each row
        D = max(Lk, 1)
        q = np.zeros((1, Lq, 1, D), np.float32)
        k = np.zeros((1, Lk, 1, D), np.float32)
        v = np.eye(Lk, D, dtype=np.float32).reshape(1, Lk, 1, D)
        O, _, _ = orc.full(q, k, v, scale=1.0, causal=hdr["causal"], window=hdr["window"],
                           q_offset=hdr["q_offset"], key_mask=mask)
        for i, keys in table.items():
            assert counts[0, i] == len(keys), (hdr, i, counts[0, i], keys)
            got = set(np.nonzero(O[0, i, 0, :Lk] > 0)[0].tolist())
            assert got == set(keys), (hdr, i, got, keys)


def _parse_tables(path):
    cases, hdr, table = [], None, None
    with open(path) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("case"):
                if hdr is not None:
                    cases.append((hdr, table))
                hdr, table = {}, {}
                for tok in line.split()[1:]:
                    key, val = tok.split("=")
                    if key == "causal":
                        hdr[key] = val == "1"
                    elif key == "masked":
                        hdr[key] = [int(x) for x in val.split(",") if x]
                    else:
                        hdr[key] = int(val)
                continue
            row, keys = line.split(":")
            table[int(row)] = [int(x) for x in keys.split()]
    if hdr is not None:
        cases.append((hdr, table))
    return cases


def pin_visible_counts_match_predicates(orc):
    rng = _rng(1)
    for causal in (True, False):
        for window in (-1, 0, 1, 2, 5, 8, 40):
            B, Lq, Lk = 3, 7, 19
            for q_offset in (0, 5, Lk - Lq):
                mask = (rng.random((B, Lk)) > 0.3).astype(np.float32)
                counts, total = orc.visible_counts(B, Lq, Lk, causal=causal, window=window,
                                                   q_offset=q_offset, key_mask=mask)
                want = np.stack([dense_visibility(Lq, Lk, causal, window, q_offset, mask[b]).sum(1)
                                 for b in range(B)])
                assert np.array_equal(counts, want), (causal, window, q_offset)
                assert total == int(want.sum())


def pin_matches_torch_sdpa_float64(orc):
    """No window, mask or soft-cap and Hq = Hkv: torch's float64 math-path
    attention is the same definition."""
    rng = _rng(2)
    for (B, Lq, Lk, H, D, causal) in [(2, 9, 9, 3, 16, True), (1, 13, 13, 2, 8, False),
                                      (2, 5, 11, 2, 8, False), (1, 4, 10, 3, 8, True)]:
        q, k, v = _rand(rng, (B, Lq, H, D)), _rand(rng, (B, Lk, H, D)), _rand(rng, (B, Lk, H, D))
        scale = 1.0 / math.sqrt(D) * 1.3
        O, L, _ = orc.full(q, k, v, scale=scale, causal=causal, window=0, q_offset=Lk - Lq)
        tq, tk, tv = (torch.from_numpy(x).double().permute(0, 2, 1, 3) for x in (q, k, v))
        if causal:
            # queries sit at the last Lq positions of the key axis
            allowed = torch.ones(Lq, Lk, dtype=torch.bool).tril(diagonal=Lk - Lq)
        else:
            allowed = torch.ones(Lq, Lk, dtype=torch.bool)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=allowed,
                                                               scale=scale)
        _close(O, ref.permute(0, 2, 1, 3).numpy(), TIGHT, "sdpa O")
        s = (tq @ tk.transpose(-1, -2)) * scale
        s = s.masked_fill(~allowed, float("-inf"))
        _close(L, torch.logsumexp(s, dim=-1).numpy(), TIGHT, "sdpa LSE")


def pin_matches_dense_bruteforce(orc):
    rng = _rng(3)
    cases = [
        dict(B=2, Lq=12, Lk=12, Hq=4, Hkv=2, D=8, causal=True, window=5, softcap=0.0, mask=True),
        dict(B=1, Lq=10, Lk=10, Hq=3, Hkv=1, D=16, causal=False, window=6, softcap=0.0, mask=True),
        dict(B=2, Lq=3, Lk=14, Hq=4, Hkv=4, D=8, causal=True, window=0, softcap=1.5, mask=False),
        dict(B=1, Lq=6, Lk=15, Hq=2, Hkv=1, D=8, causal=False, window=7, softcap=2.0, mask=True),
        dict(B=2, Lq=8, Lk=8, Hq=2, Hkv=2, D=8, causal=True, window=3, softcap=0.7, mask=True),
    ]
    for c in cases:
        B, Lq, Lk, Hq, Hkv, D = c["B"], c["Lq"], c["Lk"], c["Hq"], c["Hkv"], c["D"]
        q, k, v = _rand(rng, (B, Lq, Hq, D), 2.0), _rand(rng, (B, Lk, Hkv, D), 2.0), _rand(rng, (B, Lk, Hkv, D))
        mask = (rng.random((B, Lk)) > 0.25).astype(np.float32) if c["mask"] else None
        kw = dict(scale=0.4, causal=c["causal"], window=c["window"], q_offset=Lk - Lq,
                  softcap=c["softcap"], key_mask=mask)
        O, L, _ = orc.full(q, k, v, **kw)
        Od, Ld = dense_reference(q, k, v, **kw)
        _close(O, Od, TIGHT, f"dense O {c}")
        _close(L, Ld, TIGHT, f"dense LSE {c}")


def pin_zero_query_closed_form(orc):
    """Q = 0 makes every visible score 0 (soft-capped or not): each row is the
    plain mean of its visible V rows and LSE = ln(count)."""
    rng = _rng(4)
    for causal, window, softcap in [(True, 0, 0.0), (True, 4, 3.0), (False, 6, 0.0), (False, 0, 1.0)]:
        B, Lq, Lk, Hq, Hkv, D = 2, 7, 11, 4, 2, 8
        q = np.zeros((B, Lq, Hq, D), np.float32)
        k, v = _rand(rng, (B, Lk, Hkv, D)), _rand(rng, (B, Lk, Hkv, D))
        mask = (rng.random((B, Lk)) > 0.3).astype(np.float32)
        O, L, n = orc.full(q, k, v, scale=0.5, causal=causal, window=window, q_offset=Lk - Lq,
                           softcap=softcap, key_mask=mask)
        for b in range(B):
            vis = dense_visibility(Lq, Lk, causal, window, Lk - Lq, mask[b])
            for h in range(Hq):
                for i in range(Lq):
                    cnt = int(vis[i].sum())
                    assert n[b, h, i] == cnt
                    if cnt == 0:
                        assert np.all(O[b, i, h] == 0) and L[b, h, i] == -np.inf
                        continue
                    mean = v[b, vis[i], h // (Hq // Hkv), :].astype(np.float64).mean(0)
                    assert np.max(np.abs(O[b, i, h] - mean)) <= TIGHT
                    assert abs(L[b, h, i] - math.log(cnt)) <= TIGHT


def pin_rows_sum_to_one(orc):
    """V = 1 everywhere: O = sum_j P_ij must be 1 for every non-empty row."""
    rng = _rng(5)
    B, Lq, Lk, Hq, Hkv, D = 2, 9, 9, 2, 1, 8
    q, k = _rand(rng, (B, Lq, Hq, D), 3.0), _rand(rng, (B, Lk, Hkv, D), 3.0)
    v = np.ones((B, Lk, Hkv, D), np.float32)
    for causal, window in [(True, 0), (False, 4), (True, 3)]:
        O, _, n = orc.full(q, k, v, scale=1.0, causal=causal, window=window, q_offset=0)
        assert np.all(n > 0)
        assert np.max(np.abs(O - 1.0)) <= TIGHT


def pin_single_visible_key(orc):
    """A causal window of one key: row i sees only key i, so O_i = V_i and
    LSE_i is that single (scaled) score."""
    rng = _rng(6)
    B, L, H, D = 2, 6, 2, 8
    q, k, v = _rand(rng, (B, L, H, D)), _rand(rng, (B, L, H, D)), _rand(rng, (B, L, H, D))
    O, Lse, n = orc.full(q, k, v, scale=0.25, causal=True, window=1, q_offset=0)
    assert np.all(n == 1)
    _close(O, v.astype(np.float64), 0.0, "single key O")
    s = 0.25 * np.einsum("blhd,blhd->bhl", q.astype(np.float64), k.astype(np.float64))
    _close(Lse, s, TIGHT, "single key LSE")


def pin_gqa_equals_mha_on_repeated_kv(orc):
    rng = _rng(7)
    B, Lq, Lk, Hq, Hkv, D = 2, 6, 9, 6, 2, 8
    q, k, v = _rand(rng, (B, Lq, Hq, D)), _rand(rng, (B, Lk, Hkv, D)), _rand(rng, (B, Lk, Hkv, D))
    kw = dict(scale=0.3, causal=True, window=4, q_offset=Lk - Lq)
    Og, Lg, _ = orc.full(q, k, v, **kw)
    g = Hq // Hkv
    kt = torch.from_numpy(k).repeat_interleave(g, dim=2).numpy()
    vt = torch.from_numpy(v).repeat_interleave(g, dim=2).numpy()
    Om, Lm, _ = orc.full(q, kt, vt, **kw)
    _close(Og, Om, 0.0, "GQA vs MHA O")
    _close(Lg, Lm, 0.0, "GQA vs MHA LSE")


def pin_window_limits(orc):
    """window <= 0 is the unwindowed form; a causal window of at least Lk
    keys, or a bidirectional one of at least 2*Lk, changes nothing."""
    rng = _rng(8)
    B, L, H, D = 1, 10, 2, 8
    q, k, v = _rand(rng, (B, L, H, D)), _rand(rng, (B, L, H, D)), _rand(rng, (B, L, H, D))
    for causal, big in [(True, L), (True, L + 5), (False, 2 * L), (False, 2 * L + 3)]:
        base = orc.full(q, k, v, scale=0.5, causal=causal, window=0, q_offset=0)
        for w in (-3, -1, big):
            other = orc.full(q, k, v, scale=0.5, causal=causal, window=w, q_offset=0)
            _close(other[0], base[0], 0.0, f"window {w}")
            _close(other[1], base[1], 0.0, f"window {w}")


def pin_decode_rows_are_prefill_rows(orc):
    """A query block at the end of the key axis (q_offset = Lk - Lq) equals the
    same rows of the full causal prefill; Lq = 1 is the last row."""
    rng = _rng(9)
    B, L, Hq, Hkv, D = 2, 12, 4, 2, 8
    q, k, v = _rand(rng, (B, L, Hq, D)), _rand(rng, (B, L, Hkv, D)), _rand(rng, (B, L, Hkv, D))
    for window in (0, 5):
        Op, Lp, _ = orc.full(q, k, v, scale=0.35, causal=True, window=window, q_offset=0)
        for Lq in (1, 3):
            Od, Ld, _ = orc.full(q[:, L - Lq:], k, v, scale=0.35, causal=True, window=window,
                                 q_offset=L - Lq)
            _close(Od, Op[:, L - Lq:], 0.0, "decode O")
            _close(Ld, Lp[:, :, L - Lq:], 0.0, "decode LSE")


def pin_mask_tail_is_shorter_key_axis(orc):
    rng = _rng(10)
    B, Lq, Lk, H, D, V = 1, 5, 14, 2, 8, 9
    q, k, v = _rand(rng, (B, Lq, H, D)), _rand(rng, (B, Lk, H, D)), _rand(rng, (B, Lk, H, D))
    mask = np.ones((B, Lk), np.float32)
    mask[:, V:] = 0.0
    Om, Lm, _ = orc.full(q, k, v, scale=0.5, causal=False, window=0, q_offset=0, key_mask=mask)
    Os, Ls, _ = orc.full(q, k[:, :V], v[:, :V], scale=0.5, causal=False, window=0, q_offset=0)
    _close(Om, Os, 0.0, "mask tail O")
    _close(Lm, Ls, 0.0, "mask tail LSE")
    ones = np.ones((B, Lk), np.float32)
    Oa, La, _ = orc.full(q, k, v, scale=0.5, causal=True, window=4, q_offset=3, key_mask=ones)
    On, Ln, _ = orc.full(q, k, v, scale=0.5, causal=True, window=4, q_offset=3)
    _close(Oa, On, 0.0, "all-ones mask O")
    _close(La, Ln, 0.0, "all-ones mask LSE")


def pin_softcap_limits(orc):
    """A huge cap is the uncapped score to within its cubic term; a small cap
    c bounds every score by c, so LSE lies within [ln n - c, ln n + c]."""
    rng = _rng(11)
    B, L, H, D = 1, 8, 2, 8
    q, k, v = _rand(rng, (B, L, H, D), 2.0), _rand(rng, (B, L, H, D), 2.0), _rand(rng, (B, L, H, D))
    O0, L0, _ = orc.full(q, k, v, scale=0.5, causal=True, q_offset=0)
    Ob, Lb, _ = orc.full(q, k, v, scale=0.5, causal=True, q_offset=0, softcap=1e6)
    _close(Ob, O0, 1e-9, "huge cap O")
    _close(Lb, L0, 1e-9, "huge cap LSE")
    c = 0.25
    Oc, Lc, n = orc.full(q, k, v, scale=0.5, causal=True, q_offset=0, softcap=c)
    lnn = np.log(n.astype(np.float64))
    assert np.all(Lc <= lnn + c + TIGHT) and np.all(Lc >= lnn - c - TIGHT)
    # capped scores sit in (-c, c), so each weight is within e^{+-2c} of uniform
    Oz, _, _ = orc.full(np.zeros_like(q), k, v, scale=0.5, causal=True, q_offset=0, softcap=c)
    assert np.max(np.abs(Oc - Oz)) <= (math.exp(2 * c) - 1) * np.max(np.abs(v)) + TIGHT


def pin_invisible_keys_have_no_influence(orc):
    """Keys a row cannot see may hold anything finite without changing it."""
    rng = _rng(12)
    B, L, Hq, Hkv, D = 1, 16, 2, 1, 8
    q, k, v = _rand(rng, (B, L, Hq, D)), _rand(rng, (B, L, Hkv, D)), _rand(rng, (B, L, Hkv, D))
    mask = np.ones((B, L), np.float32)
    mask[0, [3, 11]] = 0.0
    kw = dict(scale=0.5, causal=True, window=5, q_offset=0, key_mask=mask)
    O, Lse, _ = orc.full(q, k, v, **kw)
    k2, v2 = k.copy(), v.copy()
    k2[0, [3, 11]] = 1e4
    v2[0, [3, 11]] = -1e4
    O2, L2, _ = orc.full(q, k2, v2, **kw)
    _close(O2, O, 0.0, "masked keys perturbed")
    _close(L2, Lse, 0.0, "masked keys perturbed LSE")
    # rows 0..7 cannot see keys 8.. (causal) -- perturb those too
    k3, v3 = k.copy(), v.copy()
    k3[0, 8:] = -1e4
    v3[0, 8:] = 1e4
    O3, L3, _ = orc.full(q, k3, v3, **kw)
    _close(O3[:, :8], O[:, :8], 0.0, "future keys perturbed")
    _close(L3[:, :, :8], Lse[:, :, :8], 0.0, "future keys perturbed LSE")


def pin_empty_rows(orc):
    """Rows with no visible key: O = 0 and LSE = -inf (reading for a case the
    pages leave open; brotensor's decode_len writes zeros for length 0)."""
    rng = _rng(13)
    B, L, H, D = 2, 5, 1, 8
    q, k, v = _rand(rng, (B, L, H, D)), _rand(rng, (B, L, H, D)), _rand(rng, (B, L, H, D))
    mask = np.zeros((B, L), np.float32)
    mask[1, 4] = 1.0
    O, Lse, n = orc.full(q, k, v, scale=0.5, causal=False, window=0, q_offset=0, key_mask=mask)
    assert np.all(n[0] == 0) and np.all(O[0] == 0) and np.all(Lse[0] == -np.inf)
    assert np.all(n[1] == 1)
    _close(O[1], np.broadcast_to(v[1, 4], (L, H, D)).astype(np.float64), 0.0, "one key")


# ---------------------------------------------------------------------------
# decode over a device-held length (R query rows per batch)
# ---------------------------------------------------------------------------

def decode_len_visibility(R, Lmax, n):
    """[R, Lmax] visibility as brotensor flash_attention.h states it for
    flash_attention_decode_len: row r sees the first n - R + 1 + r keys."""
    vis = np.zeros((R, Lmax), bool)
    for r in range(R):
        vis[r, :max(0, min(Lmax, n - R + 1 + r))] = True
    return vis


def dense_decode_len(q, k, v, lens, *, scale, softcap=0.0):
    """Full score matrix over the whole capacity with the count-form mask."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    B, R, Hq, D = q.shape
    Lmax, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    O = np.zeros((B, R, Hq, D))
    L = np.zeros((B, Hq, R))
    for b in range(B):
        vis = decode_len_visibility(R, Lmax, min(max(int(lens[b]), 0), Lmax))
        for h in range(Hq):
            s = scale * (q[b, :, h, :] @ k[b, :, h // g, :].T)
            if softcap > 0:
                s = softcap * np.tanh(s / softcap)
            s = np.where(vis, s, -np.inf)
            empty = ~vis.any(1)
            lse = np.where(empty, -np.inf, logsumexp(np.where(empty[:, None], 0.0, s), axis=1))
            p = np.where(vis, np.exp(s - np.where(empty, 0.0, lse)[:, None]), 0.0)
            O[b, :, h, :] = p @ v[b, :, h // g, :]
            L[b, h, :] = lse
    return O, L


def pin_decode_len_matches_dense(orc):
    """Against the dense count-form formulation, lengths 0 .. Lmax, R up to 4."""
    rng = _rng(14)
    for R, Hq, Hkv, softcap in [(1, 4, 2, 0.0), (3, 4, 1, 0.0), (4, 2, 2, 1.5)]:
        B, Lmax, D = 7, 13, 8
        lens = np.array([0, 1, R - 1, R, 6, 12, 13])
        q, k, v = _rand(rng, (B, R, Hq, D), 2.0), _rand(rng, (B, Lmax, Hkv, D), 2.0), _rand(rng, (B, Lmax, Hkv, D))
        O, L, n = orc.decode_len(q, k, v, lens, scale=0.45, softcap=softcap)
        Od, Ld = dense_decode_len(q, k, v, lens, scale=0.45, softcap=softcap)
        _close(O, Od, TIGHT, f"decode_len O R={R}")
        _close(L, Ld, TIGHT, f"decode_len LSE R={R}")
        for b in range(B):
            cnt = decode_len_visibility(R, Lmax, int(lens[b])).sum(1)
            assert np.array_equal(n[b], np.broadcast_to(cnt, (Hq, R))), (b, n[b], cnt)


def pin_decode_len_zero_query_closed_form(orc):
    """Q = 0: row r of a batch with length n is the mean of V rows
    0 .. n - R + r, LSE = ln(n - R + 1 + r); a row with no key (n = 0, or
    n < R for the first rows) is O = 0, LSE = -inf."""
    rng = _rng(15)
    B, R, Hq, Hkv, Lmax, D = 5, 3, 4, 2, 10, 8
    lens = np.array([0, 2, 3, 7, 10])
    q = np.zeros((B, R, Hq, D), np.float32)
    k, v = _rand(rng, (B, Lmax, Hkv, D)), _rand(rng, (B, Lmax, Hkv, D))
    O, L, _ = orc.decode_len(q, k, v, lens, scale=0.7, softcap=2.0)
    for b in range(B):
        for h in range(Hq):
            for r in range(R):
                cnt = int(lens[b]) - R + 1 + r
                if cnt <= 0:
                    assert np.all(O[b, r, h] == 0) and L[b, h, r] == -np.inf, (b, h, r)
                    continue
                mean = v[b, :cnt, h // (Hq // Hkv), :].astype(np.float64).mean(0)
                assert np.max(np.abs(O[b, r, h] - mean)) <= TIGHT
                assert abs(L[b, h, r] - math.log(cnt)) <= TIGHT


def pin_decode_len_ignores_rows_past_length(orc):
    """Cache rows at or past the length may hold anything finite."""
    rng = _rng(16)
    B, R, Hq, Hkv, Lmax, D = 3, 2, 2, 1, 12, 8
    lens = np.array([5, 9, 12])
    q, k, v = _rand(rng, (B, R, Hq, D)), _rand(rng, (B, Lmax, Hkv, D)), _rand(rng, (B, Lmax, Hkv, D))
    O, L, _ = orc.decode_len(q, k, v, lens, scale=0.5)
    k2, v2 = k.copy(), v.copy()
    for b in range(B):
        k2[b, lens[b]:] = 1e4
        v2[b, lens[b]:] = -1e4
    O2, L2, _ = orc.decode_len(q, k2, v2, lens, scale=0.5)
    _close(O2, O, 0.0, "decode_len past-length rows perturbed")
    _close(L2, L, 0.0, "decode_len past-length rows perturbed LSE")


# ---------------------------------------------------------------------------
# single-query decode over a fixed-capacity cache with a key mask
# ---------------------------------------------------------------------------

def decode_masked_visibility(mask_b, window):
    """[Lmax] kept keys as brotensor flash_attention.h states them for
    flash_attention_decode_masked: the query's position p is the last valid
    key (mask value > 0.5); a key is kept when it is valid and, with
    window > 0, lies after p - window."""
    valid = np.asarray(mask_b, np.float64) > 0.5
    if not valid.any():
        return valid
    p = int(np.max(np.nonzero(valid)[0]))
    j = np.arange(valid.size)
    return valid & ((j > p - window) if window > 0 else True)


def dense_decode_masked(q, k, v, mask, *, scale, window, softcap=0.0):
    """Full score row over the whole capacity with the literal kept set."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    B, _, Hq, D = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    O = np.zeros((B, 1, Hq, D))
    L = np.full((B, Hq, 1), -np.inf)
    for b in range(B):
        vis = decode_masked_visibility(mask[b], window)
        if not vis.any():
            continue
        for h in range(Hq):
            s = scale * (k[b, :, h // g, :] @ q[b, 0, h, :])
            if softcap > 0:
                s = softcap * np.tanh(s / softcap)
            s = np.where(vis, s, -np.inf)
            lse = logsumexp(s)
            O[b, 0, h, :] = np.exp(s - lse) @ v[b, :, h // g, :]
            L[b, h, 0] = lse
    return O, L


def _decode_masks(rng, B, Lmax):
    """Prefix masks, masks with holes, single valid keys at either end, and a
    batch with no valid key."""
    m = np.zeros((B, Lmax), np.float32)
    m[0, :Lmax // 2] = 1.0                                # prefix
    m[1] = (rng.random(Lmax) < 0.6).astype(np.float32)    # holes
    m[2, 0] = 1.0                                         # only key 0
    m[3, Lmax - 1] = 1.0                                  # only the last key
    m[4] = 1.0                                            # full capacity
    m[5, 3:Lmax - 4] = (rng.random(Lmax - 7) < 0.3)       # holes, last valid key inside
    m[5, Lmax - 5] = 0.9                                  # above 0.5: valid
    m[5, Lmax - 4:] = 0.5                                 # not above 0.5: invalid
    # m[6] stays all zero: no valid key
    return m


def pin_decode_masked_matches_dense(orc):
    """Against the dense formulation with the literal kept set: windows off,
    negative, 1, short and longer than the valid span; GQA; soft-cap."""
    rng = _rng(31)
    B, Lmax, D = 7, 23, 8
    for Hq, Hkv, window, softcap in [(4, 2, 0, 0.0), (4, 1, -3, 0.0), (2, 2, 1, 0.0), (4, 2, 3, 2.0),
                                     (6, 3, 7, 0.0), (2, 1, 100, 5.0)]:
        q = _rand(rng, (B, 1, Hq, D), 2.0)
        k, v = _rand(rng, (B, Lmax, Hkv, D), 2.0), _rand(rng, (B, Lmax, Hkv, D))
        m = _decode_masks(rng, B, Lmax)
        O, L, n = orc.decode_masked(q, k, v, m, scale=0.4, window=window, softcap=softcap)
        Od, Ld = dense_decode_masked(q, k, v, m, scale=0.4, window=window, softcap=softcap)
        _close(O, Od, TIGHT, f"decode_masked O w={window}")
        _close(L, Ld, TIGHT, f"decode_masked LSE w={window}")
        for b in range(B):
            cnt = int(decode_masked_visibility(m[b], window).sum())
            assert np.all(n[b] == cnt), (b, n[b], cnt)


def pin_decode_masked_prefix_equals_decode_at_valid_length(orc):
    """mask = [1] * n + [0] * (Lmax - n) gives exactly (bit for bit) the
    plain single-query decode over the first n keys, with or without a
    window, as the page states for this function."""
    rng = _rng(32)
    Lmax, Hq, Hkv, D = 40, 4, 2, 8
    for n in (1, 2, 17, 39, 40):
        for window, softcap in ((0, 0.0), (5, 0.0), (12, 3.0)):
            q = _rand(rng, (1, 1, Hq, D), 2.0)
            k, v = _rand(rng, (1, Lmax, Hkv, D)), _rand(rng, (1, Lmax, Hkv, D))
            m = np.zeros((1, Lmax), np.float32)
            m[0, :n] = 1.0
            O, L, _ = orc.decode_masked(q, k, v, m, scale=0.3, window=window, softcap=softcap)
            Od, Ld, _ = orc.full(q, k[:, :n], v[:, :n], scale=0.3, causal=True, window=window, q_offset=n - 1,
                                 softcap=softcap)
            assert np.array_equal(O, Od) and np.array_equal(L, Ld), (n, window)


def pin_decode_masked_zero_query_closed_form(orc):
    """Q = 0: the output is the mean of the kept V rows and LSE = ln(count),
    with the kept set from the literal rule; no valid key: O = 0,
    LSE = -inf."""
    rng = _rng(33)
    B, Lmax, Hq, Hkv, D = 7, 19, 4, 2, 8
    q = np.zeros((B, 1, Hq, D), np.float32)
    k, v = _rand(rng, (B, Lmax, Hkv, D)), _rand(rng, (B, Lmax, Hkv, D))
    m = _decode_masks(rng, B, Lmax)
    for window in (0, 1, 4):
        O, L, _ = orc.decode_masked(q, k, v, m, scale=0.9, window=window, softcap=1.5)
        for b in range(B):
            vis = decode_masked_visibility(m[b], window)
            for h in range(Hq):
                if not vis.any():
                    assert np.all(O[b, 0, h] == 0) and L[b, h, 0] == -np.inf
                    continue
                mean = v[b, vis, h // (Hq // Hkv), :].astype(np.float64).mean(0)
                assert np.max(np.abs(O[b, 0, h] - mean)) <= TIGHT, (b, h, window)
                assert abs(L[b, h, 0] - math.log(int(vis.sum()))) <= TIGHT


# ---------------------------------------------------------------------------
# sequences packed back to back in one fused QKV tensor
# ---------------------------------------------------------------------------

def packed_bounds(lengths):
    rows, s = [], 0
    for n in lengths:
        rows += [(s, s + n)] * n
        s += n
    return np.array(rows, np.int64).reshape(-1, 2)


def packed_visibility(sb, window):
    """[L, L] visibility as brotensor flash_attention.h states it for the
    packed-QKV forward: row r sees key j of its own sequence
    [sb[r,0], sb[r,1]), and with a window only when |r - j| <= window/2."""
    L = sb.shape[0]
    vis = np.zeros((L, L), bool)
    for r in range(L):
        for j in range(L):
            vis[r, j] = sb[r, 0] <= j < sb[r, 1] and (window <= 0 or abs(r - j) <= window // 2)
    return vis


def dense_packed(qkv, sb, H, *, scale, window, softcap=0.0):
    x = np.asarray(qkv, np.float64)
    L = x.shape[0]
    D = x.shape[1] // (3 * H)
    vis = packed_visibility(sb, window)
    O = np.zeros((L, H, D))
    LSE = np.zeros((H, L))
    for h in range(H):
        q = x[:, h * D:(h + 1) * D]
        k = x[:, (H + h) * D:(H + h + 1) * D]
        v = x[:, (2 * H + h) * D:(2 * H + h + 1) * D]
        s = scale * (q @ k.T)
        if softcap > 0:
            s = softcap * np.tanh(s / softcap)
        s = np.where(vis, s, -np.inf)
        lse = logsumexp(s, axis=1)
        O[:, h, :] = np.exp(s - lse[:, None]) @ v
        LSE[h] = lse
    return O, LSE


def pin_packed_matches_dense(orc):
    """Against the full packed score matrix with the pages' row rule."""
    rng = _rng(17)
    for lengths, H, window, softcap in [([5, 1, 9, 3], 2, 0, 0.0), ([7, 8], 1, 4, 0.0),
                                        ([1, 1, 12], 3, 5, 2.0), ([16], 2, 6, 0.0)]:
        D = 8
        L = sum(lengths)
        qkv = _rand(rng, (L, 3 * H * D), 2.0)
        sb = packed_bounds(lengths)
        O, LSE, N = orc.packed_qkv(qkv, sb, H, scale=0.4, window=window, softcap=softcap)
        Od, Ld = dense_packed(qkv, sb, H, scale=0.4, window=window, softcap=softcap)
        _close(O, Od, TIGHT, f"packed O {lengths}")
        _close(LSE, Ld, TIGHT, f"packed LSE {lengths}")
        assert np.array_equal(N, np.broadcast_to(packed_visibility(sb, window).sum(1), (H, L)))


def pin_packed_zero_query_closed_form(orc):
    """Q = 0: each row is the mean of the V rows of its sequence inside the
    window, LSE = ln(count)."""
    rng = _rng(18)
    lengths, H, D, window = [4, 10, 1, 6], 2, 8, 6
    L = sum(lengths)
    qkv = _rand(rng, (L, 3 * H * D))
    qkv[:, :H * D] = 0.0
    sb = packed_bounds(lengths)
    O, LSE, _ = orc.packed_qkv(qkv, sb, H, scale=0.9, window=window)
    for r in range(L):
        js = [j for j in range(sb[r, 0], sb[r, 1]) if abs(r - j) <= window // 2]
        for h in range(H):
            v = qkv[js, (2 * H + h) * D:(2 * H + h + 1) * D].astype(np.float64)
            assert np.max(np.abs(O[r, h] - v.mean(0))) <= TIGHT
            assert abs(LSE[h, r] - math.log(len(js))) <= TIGHT


def pin_packed_sequences_are_independent(orc):
    """Changing one sequence's rows (any of Q, K, V) leaves the others exactly
    unchanged."""
    rng = _rng(19)
    lengths, H, D = [6, 9, 5], 2, 8
    L = sum(lengths)
    qkv = _rand(rng, (L, 3 * H * D))
    sb = packed_bounds(lengths)
    O, LSE, _ = orc.packed_qkv(qkv, sb, H, scale=0.5, window=0)
    qkv2 = qkv.copy()
    qkv2[6:15] = 1e3
    O2, L2, _ = orc.packed_qkv(qkv2, sb, H, scale=0.5, window=0)
    keep = np.r_[0:6, 15:20]
    _close(O2[keep], O[keep], 0.0, "other sequences perturbed")
    _close(L2[:, keep], LSE[:, keep], 0.0, "other sequences perturbed LSE")


# ---------------------------------------------------------------------------
# separate query and key packings with prefix sums (varlen)
# ---------------------------------------------------------------------------

def varlen_visibility(cq, ck, causal, window):
    """[Tq, Tk] visibility as brotensor flash_attention.h states it for
    flash_attention_varlen_forward: no cross-sequence attention, and causal
    keeps key k for query q when k - cu_k[b] <= q - cu_q[b]; the window rules
    are those of the windowed forward on the positions within the sequence."""
    Tq, Tk = int(cq[-1]), int(ck[-1])
    vis = np.zeros((Tq, Tk), bool)
    for b in range(len(cq) - 1):
        for qi in range(cq[b], cq[b + 1]):
            for kj in range(ck[b], ck[b + 1]):
                pq, pk = qi - cq[b], kj - ck[b]
                ok = vis_causal_p1(pq, pk, window) if causal else vis_bidir_packed(pq, pk, window)
                vis[qi, kj] = ok
    return vis


def dense_varlen(q, k, v, cq, ck, *, scale, causal, window, softcap=0.0):
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    vis = varlen_visibility(cq, ck, causal, window)
    O = np.zeros((Tq, Hq, D))
    LSE = np.zeros((Hq, Tq))
    for h in range(Hq):
        s = scale * (q[:, h, :] @ k[:, h // g, :].T)
        if softcap > 0:
            s = softcap * np.tanh(s / softcap)
        s = np.where(vis, s, -np.inf)
        empty = ~vis.any(1)
        lse = np.where(empty, -np.inf, logsumexp(np.where(empty[:, None], 0.0, s), axis=1))
        O[:, h, :] = np.where(vis, np.exp(s - np.where(empty, 0.0, lse)[:, None]), 0.0) @ v[:, h // g, :]
        LSE[h] = lse
    return O, LSE


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


def pin_varlen_matches_dense(orc):
    rng = _rng(20)
    for lq, lk, causal, window, Hq, Hkv, softcap in [
            ([3, 7, 1, 5], [3, 7, 1, 5], True, 0, 4, 2, 0.0),
            ([4, 6, 2], [9, 2, 5], False, 0, 2, 1, 0.0),
            ([5, 0, 6], [5, 4, 0], True, 3, 2, 2, 1.5),
            ([8, 3], [8, 3], False, 4, 3, 1, 0.0)]:
        D = 8
        cq, ck = _cu(lq), _cu(lk)
        q = _rand(rng, (int(cq[-1]), Hq, D), 2.0)
        k, v = _rand(rng, (int(ck[-1]), Hkv, D), 2.0), _rand(rng, (int(ck[-1]), Hkv, D))
        kw = dict(scale=0.4, causal=causal, window=window, softcap=softcap)
        O, L, N = orc.varlen(q, k, v, cq, ck, **kw)
        Od, Ld = dense_varlen(q, k, v, cq, ck, **kw)
        _close(O, Od, TIGHT, f"varlen O {lq} {lk}")
        _close(L, Ld, TIGHT, f"varlen LSE {lq} {lk}")
        assert np.array_equal(N, np.broadcast_to(varlen_visibility(cq, ck, causal, window).sum(1), N.shape))


def pin_varlen_zero_query_closed_form(orc):
    """Q = 0: each row is the mean of its sequence's visible V rows and
    LSE = ln(count); the causal count of row q is min(q - cu_q + 1, len_k)."""
    rng = _rng(21)
    lq, lk = [4, 9, 3], [6, 5, 3]
    cq, ck = _cu(lq), _cu(lk)
    Hq, Hkv, D = 2, 1, 8
    q = np.zeros((int(cq[-1]), Hq, D), np.float32)
    k, v = _rand(rng, (int(ck[-1]), Hkv, D)), _rand(rng, (int(ck[-1]), Hkv, D))
    O, L, _ = orc.varlen(q, k, v, cq, ck, scale=0.8, causal=True)
    for b in range(3):
        for qi in range(cq[b], cq[b + 1]):
            cnt = min(qi - cq[b] + 1, lk[b])
            mean = v[ck[b]:ck[b] + cnt, 0, :].astype(np.float64).mean(0)
            for h in range(Hq):
                assert np.max(np.abs(O[qi, h] - mean)) <= TIGHT
                assert abs(L[h, qi] - math.log(cnt)) <= TIGHT


def pin_varlen_sequences_are_independent(orc):
    rng = _rng(22)
    lq, lk = [5, 6, 4], [7, 6, 2]
    cq, ck = _cu(lq), _cu(lk)
    q = _rand(rng, (int(cq[-1]), 2, 8))
    k, v = _rand(rng, (int(ck[-1]), 2, 8)), _rand(rng, (int(ck[-1]), 2, 8))
    O, L, _ = orc.varlen(q, k, v, cq, ck, scale=0.5, causal=False)
    k2, v2 = k.copy(), v.copy()
    k2[7:13] = 1e3
    v2[7:13] = -1e3
    O2, L2, _ = orc.varlen(q, k2, v2, cq, ck, scale=0.5, causal=False)
    keep = np.r_[0:5, 11:15]
    _close(O2[keep], O[keep], 0.0, "other sequences' keys perturbed")
    _close(L2[:, keep], L[:, keep], 0.0, "other sequences' keys perturbed LSE")


# ---------------------------------------------------------------------------
# additive score mask (broadcast) and attention dropout
# ---------------------------------------------------------------------------

def _numpy_philox_block(ctr, key):
    """First output block of NumPy's Philox (4x64-10) bit generator for the
    given 256-bit counter: NumPy advances the counter once before its first
    block, so it is started one below."""
    c = [int(x) for x in ctr]
    for w in range(4):                       # 256-bit decrement
        if c[w] > 0:
            c[w] -= 1
            break
        c[w] = (1 << 64) - 1
    bg = np.random.Philox(key=np.array(key, np.uint64), counter=np.array(c, np.uint64))
    return [int(x) for x in bg.random_raw(4)]


def _numpy_keep(seed, thr, b, h, i, j):
    """Dropout decision of weight (b, h, i, j) from NumPy's Philox: block
    (j // 16, i, h, b) under key (seed mod 2^32, 0); 16-bit field j % 16 (bits
    16 (f % 4) .. +15 of word f // 4) >= thr."""
    f = j % 16
    word = _numpy_philox_block([j // 16, i, h, b], [seed % 2 ** 32, 0])[f // 4]
    return ((word >> (16 * (f % 4))) & 0xFFFF) >= thr


def pin_philox_matches_numpy(orc):
    """The oracle's Philox4x64-10 against NumPy's implementation of it."""
    rng = _rng(23)
    cases = [([0, 0, 0, 0], [0, 0]), ([1, 0, 0, 0], [5, 7]), ([2**64 - 1] * 4, [2**64 - 1] * 2)]
    for _ in range(20):
        cases.append((rng.integers(0, 2**63, 4, dtype=np.uint64).tolist(),
                      rng.integers(0, 2**63, 2, dtype=np.uint64).tolist()))
    for ctr, key in cases:
        assert orc.philox4x64(ctr, key) == _numpy_philox_block(ctr, key), (ctr, key)


def dense_bias_dropout(q, k, v, *, scale, causal, window, q_offset, softcap=0.0, key_mask=None,
                       bias=None, dropout_p=0.0, seed=0):
    """Full score matrix, bias broadcast by NumPy, dropout pattern from NumPy's
    Philox: block (j // 16, i, hq, b) under key (seed mod 2^32, 0), 16-bit
    field j % 16."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    bb = None if bias is None else np.broadcast_to(np.asarray(bias, np.float64), (B, Hq, Lq, Lk))
    thr = int(round(dropout_p * 2 ** 16))
    O = np.zeros((B, Lq, Hq, D))
    L = np.zeros((B, Hq, Lq))
    for b in range(B):
        vis = dense_visibility(Lq, Lk, causal, window, q_offset,
                               None if key_mask is None else np.asarray(key_mask)[b])
        for h in range(Hq):
            s = scale * (q[b, :, h, :] @ k[b, :, h // g, :].T)
            if softcap > 0:
                s = softcap * np.tanh(s / softcap)
            if bb is not None:
                s = s + bb[b, h]
            s = np.where(vis, s, -np.inf)
            empty = ~np.isfinite(s).any(1)
            lse = np.where(empty, -np.inf, logsumexp(np.where(empty[:, None], 0.0, s), axis=1))
            p = np.where(vis & ~empty[:, None], np.exp(s - np.where(empty, 0.0, lse)[:, None]), 0.0)
            if dropout_p > 0:
                keep = np.zeros((Lq, Lk), bool)
                for i in range(Lq):
                    for j in range(Lk):
                        keep[i, j] = _numpy_keep(seed, thr, b, h, i, j)
                p = np.where(keep, p / (1.0 - dropout_p), 0.0)
            O[b, :, h, :] = p @ v[b, :, h // g, :]
            L[b, h, :] = lse
    return O, L


def pin_bias_matches_dense(orc):
    rng = _rng(24)
    B, Lq, Lk, Hq, Hkv, D = 2, 7, 9, 4, 2, 8
    q, k, v = _rand(rng, (B, Lq, Hq, D), 2.0), _rand(rng, (B, Lk, Hkv, D), 2.0), _rand(rng, (B, Lk, Hkv, D))
    mask = (rng.random((B, Lk)) > 0.2).astype(np.float32)
    for shape, causal, window, softcap in [((B, Hq, Lq, Lk), True, 0, 0.0), ((B, 1, 1, Lk), False, 6, 0.0),
                                           ((1, Hq, Lq, Lk), True, 4, 2.0), ((1, 1, Lq, Lk), False, 0, 0.0),
                                           ((B, 1, Lq, 1), True, 0, 0.0)]:
        bias = _rand(rng, shape, 1.5)
        kw = dict(scale=0.45, causal=causal, window=window, q_offset=Lk - Lq, softcap=softcap,
                  key_mask=mask, bias=bias)
        O, L, _ = orc.full(q, k, v, **kw)
        Od, Ld = dense_bias_dropout(q, k, v, **kw)
        _close(O, Od, TIGHT, f"bias O {shape}")
        _close(L, Ld, TIGHT, f"bias LSE {shape}")


def pin_bias_row_shift_and_neg_inf(orc):
    """A bias constant along each row moves only the LSE (softmax shift
    invariance); a bias of -inf on a key is the key mask."""
    rng = _rng(25)
    B, L, Hq, Hkv, D = 2, 8, 2, 1, 8
    q, k, v = _rand(rng, (B, L, Hq, D)), _rand(rng, (B, L, Hkv, D)), _rand(rng, (B, L, Hkv, D))
    O0, L0, _ = orc.full(q, k, v, scale=0.5, causal=True, q_offset=0)
    c = _rand(rng, (B, Hq, L, 1), 3.0)
    O1, L1, _ = orc.full(q, k, v, scale=0.5, causal=True, q_offset=0, bias=c)
    _close(O1, O0, 1e-12, "row-constant bias O")
    _close(L1, L0 + c[..., 0].astype(np.float64), 1e-12, "row-constant bias LSE")
    mask = (rng.random((B, L)) > 0.4).astype(np.float32)
    mask[:, 0] = 1.0
    neg = np.where(mask > 0.5, 0.0, -np.inf).astype(np.float32)[:, None, None, :]
    O2, L2, _ = orc.full(q, k, v, scale=0.5, causal=False, q_offset=0, bias=neg)
    O3, L3, _ = orc.full(q, k, v, scale=0.5, causal=False, q_offset=0, key_mask=mask)
    _close(O2, O3, 1e-12, "-inf bias vs key mask O")
    _close(L2, L3, 1e-12, "-inf bias vs key mask LSE")


def pin_dropout_keep_matches_numpy(orc):
    """Every dropout decision of a grid spanning several 16-key blocks, rows,
    heads and batches against NumPy's Philox with the field layout written
    out; the seed's bits above the low 32 change nothing (the pages: only the
    low 32 bits of the seed are used), its low bits do; the kept fraction is
    1 - p within five standard deviations."""
    for seed, p in [(0, 0.5), (2**32 + 11, 0.1), (2**63 + 5, 0.9)]:
        thr = int(round(p * 2 ** 16))
        for b in range(2):
            for h in (0, 3):
                for i in (0, 1, 17):
                    for j in range(0, 70, 3):
                        assert orc.dropout_keep(seed, p, b, h, i, j) == _numpy_keep(seed, thr, b, h, i, j), \
                            (seed, p, b, h, i, j)
    pairs = [(b, h, i, j) for b in range(2) for h in range(2) for i in range(3) for j in range(64)]
    for seed in (7, 2**40 + 7):
        a = [orc.dropout_keep(seed, 0.5, *x) for x in pairs]
        assert a == [orc.dropout_keep(seed + 2**32, 0.5, *x) for x in pairs]
        assert a != [orc.dropout_keep(seed + 1, 0.5, *x) for x in pairs]
    n = 0
    kept = 0
    for i in range(40):
        for j in range(256):
            kept += orc.dropout_keep(99, 0.3, 1, 2, i, j)
            n += 1
    sd = (0.3 * 0.7 / n) ** 0.5
    assert abs(kept / n - 0.7) < 5 * sd, kept / n


def pin_dropout_matches_dense(orc):
    """Dropout against the dense form with NumPy's Philox drawing the pattern
    over three 16-key blocks; the LSE ignores dropout and p = 0 is no
    dropout."""
    rng = _rng(26)
    B, Lq, Lk, Hq, Hkv, D = 2, 6, 40, 2, 1, 8
    q, k, v = _rand(rng, (B, Lq, Hq, D), 2.0), _rand(rng, (B, Lk, Hkv, D), 2.0), _rand(rng, (B, Lk, Hkv, D))
    for p, seed, causal in [(0.1, 1234, True), (0.5, 2**40 + 7, False), (0.9, 3, True)]:
        kw = dict(scale=0.5, causal=causal, window=0, q_offset=Lk - Lq, dropout_p=p, seed=seed)
        O, L, _ = orc.full(q, k, v, **kw)
        Od, Ld = dense_bias_dropout(q, k, v, **kw)
        _close(O, Od, TIGHT, f"dropout O p={p}")
        _close(L, Ld, TIGHT, f"dropout LSE p={p}")
    O0, L0, _ = orc.full(q, k, v, scale=0.5, causal=True, q_offset=Lk - Lq)
    O1, L1, _ = orc.full(q, k, v, scale=0.5, causal=True, q_offset=Lk - Lq, dropout_p=0.0, seed=99)
    _close(O1, O0, 0.0, "p = 0")
    _close(L1, L0, 0.0, "p = 0 LSE")


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def _grid(rng, shape, step=2.0 ** -6, spread=64):
    """Values on a coarse binary grid, so that +-h perturbations with a
    power-of-two h stay exact in float32."""
    return (rng.integers(-spread, spread + 1, shape) * step).astype(np.float32)


def pin_bwd_matches_finite_differences(orc):
    """dL/dX for L = sum(O * G) against central differences of the oracle's
    own forward (exact inputs on a binary grid, h = 2^-12)."""
    rng = _rng(27)
    B, Lq, Lk, Hq, Hkv, D = 1, 5, 7, 2, 1, 4
    for kw in [dict(causal=True, window=0, softcap=0.0), dict(causal=False, window=4, softcap=1.5),
               dict(causal=True, window=3, softcap=0.0, dropout_p=0.3, seed=9)]:
        q, k, v = _grid(rng, (B, Lq, Hq, D)), _grid(rng, (B, Lk, Hkv, D)), _grid(rng, (B, Lk, Hkv, D))
        G = _rand(rng, (B, Lq, Hq, D))
        mask = np.ones((B, Lk), np.float32)
        mask[0, 2] = 0.0
        bias = _grid(rng, (1, Hq, Lq, Lk), 2.0 ** -4, 16)
        args = dict(scale=0.7, q_offset=Lk - Lq, key_mask=mask, bias=bias, **kw)
        dq, dk, dv = orc.bwd(q, k, v, G, **args)
        h = 2.0 ** -12

        def loss(q_, k_, v_):
            O, _, _ = orc.full(q_, k_, v_, **args)
            return float(np.sum(O * G))
        for name, X, dX in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            for idx in [tuple(rng.integers(0, n) for n in X.shape) for _ in range(6)]:
                Xp, Xm = X.copy(), X.copy()
                Xp[idx] += h
                Xm[idx] -= h
                if name == "q":
                    fd = (loss(Xp, k, v) - loss(Xm, k, v)) / (2 * h)
                elif name == "k":
                    fd = (loss(q, Xp, v) - loss(q, Xm, v)) / (2 * h)
                else:
                    fd = (loss(q, k, Xp) - loss(q, k, Xm)) / (2 * h)
                assert abs(fd - dX[idx]) <= 1e-6 * (1 + abs(fd)), (name, idx, kw, fd, dX[idx])


def pin_bwd_matches_torch_autograd(orc):
    """Against torch float64 autograd through a dense formulation of the same
    forward (scale, soft-cap, additive mask, masks as -inf, softmax, dropout
    factors from NumPy's Philox, GQA by repeating K and V)."""
    rng = _rng(28)
    B, Lq, Lk, Hq, Hkv, D = 2, 6, 8, 4, 2, 8
    for kw in [dict(causal=True, window=0, softcap=0.0, bias=False, dropout_p=0.0),
               dict(causal=False, window=6, softcap=2.0, bias=True, dropout_p=0.0),
               dict(causal=True, window=4, softcap=0.0, bias=True, dropout_p=0.4)]:
        q, k, v = _rand(rng, (B, Lq, Hq, D)), _rand(rng, (B, Lk, Hkv, D)), _rand(rng, (B, Lk, Hkv, D))
        G = _rand(rng, (B, Lq, Hq, D))
        mask = (rng.random((B, Lk)) > 0.2).astype(np.float32)
        bias = _rand(rng, (B, 1, Lq, Lk)) if kw["bias"] else None
        seed = 77
        args = dict(scale=0.5, causal=kw["causal"], window=kw["window"], q_offset=Lk - Lq,
                    softcap=kw["softcap"], key_mask=mask, bias=bias, dropout_p=kw["dropout_p"], seed=seed)
        dq, dk, dv = orc.bwd(q, k, v, G, **args)
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        g = Hq // Hkv
        kr = tk.repeat_interleave(g, dim=2)
        vr = tv.repeat_interleave(g, dim=2)
        S = 0.5 * torch.einsum("bihd,bjhd->bhij", tq, kr)
        if kw["softcap"] > 0:
            S = kw["softcap"] * torch.tanh(S / kw["softcap"])
        if bias is not None:
            S = S + torch.tensor(bias, dtype=torch.float64)
        vis = np.stack([dense_visibility(Lq, Lk, kw["causal"], kw["window"], Lk - Lq, mask[b_]) for b_ in range(B)])
        S = S.masked_fill(~torch.tensor(vis)[:, None], -float("inf"))
        P = torch.softmax(S, dim=-1)
        if kw["dropout_p"] > 0:
            thr = int(round(kw["dropout_p"] * 2 ** 16))
            Z = np.zeros((B, Hq, Lq, Lk))
            for b_ in range(B):
                for h_ in range(Hq):
                    for i in range(Lq):
                        for j in range(Lk):
                            keep = _numpy_keep(seed, thr, b_, h_, i, j)
                            Z[b_, h_, i, j] = 1.0 / (1.0 - kw["dropout_p"]) if keep else 0.0
            P = P * torch.tensor(Z)
        O = torch.einsum("bhij,bjhd->bihd", P, vr)
        (O * torch.tensor(G, dtype=torch.float64)).sum().backward()
        _close(dq, tq.grad.numpy(), 1e-12, f"dq {kw}")
        _close(dk, tk.grad.numpy(), 1e-12, f"dk {kw}")
        _close(dv, tv.grad.numpy(), 1e-12, f"dv {kw}")


ALL_PINS = [
    pin_range_causal_matches_ferrotensor_rule,
    pin_range_causal_matches_forge_rule,
    pin_range_bidirectional_matches_packed_rule,
    pin_golden_visibility_tables,
    pin_visible_counts_match_predicates,
    pin_matches_torch_sdpa_float64,
    pin_matches_dense_bruteforce,
    pin_zero_query_closed_form,
    pin_rows_sum_to_one,
    pin_single_visible_key,
    pin_gqa_equals_mha_on_repeated_kv,
    pin_window_limits,
    pin_decode_rows_are_prefill_rows,
    pin_mask_tail_is_shorter_key_axis,
    pin_softcap_limits,
    pin_invisible_keys_have_no_influence,
    pin_empty_rows,
    pin_decode_len_matches_dense,
    pin_decode_len_zero_query_closed_form,
    pin_decode_len_ignores_rows_past_length,
    pin_decode_masked_matches_dense,
    pin_decode_masked_prefix_equals_decode_at_valid_length,
    pin_decode_masked_zero_query_closed_form,
    pin_packed_matches_dense,
    pin_packed_zero_query_closed_form,
    pin_packed_sequences_are_independent,
    pin_varlen_matches_dense,
    pin_varlen_zero_query_closed_form,
    pin_varlen_sequences_are_independent,
    pin_philox_matches_numpy,
    pin_bias_matches_dense,
    pin_bias_row_shift_and_neg_inf,
    pin_dropout_keep_matches_numpy,
    pin_dropout_matches_dense,
    pin_bwd_matches_finite_differences,
    pin_bwd_matches_torch_autograd,
]
