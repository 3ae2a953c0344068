"""ctypes wrapper and build step for the fp64 oracle in ``mfa_oracle.c``.

Test infrastructure only (see the header of ``mfa_oracle.c``).  Inputs are
float32 arrays holding the already-rounded input tensors exactly (bf16 and
fp16 widen to float32 without loss); results come back as float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import numpy as np

ORACLE_DIR = os.path.dirname(os.path.abspath(__file__))
ORACLE_SRC = os.path.join(ORACLE_DIR, "mfa_oracle.c")
ORACLE_LIB = os.path.join(ORACLE_DIR, "libmfa_oracle.so")


def build_oracle(out_path: str = ORACLE_LIB, mutant: int = 0) -> str:
    """Compile the oracle with gcc (-O2, no fast-math).  ``mutant`` > 0 plants
    the numbered deliberate mistake (used only by the mutation test)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-fPIC", "-shared", "-pthread",
           f"-DORACLE_MUTANT={int(mutant)}", ORACLE_SRC, "-o", out_path + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out_path + ".tmp", out_path)
    return out_path


def _f32(x):
    """float32, C-contiguous numpy view of a torch tensor or array (exact for
    fp32/bf16/fp16 inputs)."""
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float32).contiguous().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


_fp = ctypes.POINTER(ctypes.c_float)
_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int64)


def _ptr(a, t):
    return None if a is None else a.ctypes.data_as(t)


class Oracle:
    """One loaded build of the oracle library."""

    def __init__(self, path: str = ORACLE_LIB):
        if not os.path.exists(path):
            build_oracle(path)
        self.path = path
        lib = ctypes.CDLL(path)
        lib.mfa_oracle_rows.restype = ctypes.c_int
        lib.mfa_oracle_rows.argtypes = [_fp, _fp, _fp, _fp] + [ctypes.c_int64] * 6 + [
            ctypes.c_double, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
            _ip, ctypes.c_int64, _dp, _dp, _ip, ctypes.c_int]
        lib.mfa_oracle_rows_ext.restype = ctypes.c_int
        lib.mfa_oracle_rows_ext.argtypes = [_fp, _fp, _fp, _fp] + [ctypes.c_int64] * 6 + [
            ctypes.c_double, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
            _fp, _ip, ctypes.c_double, ctypes.c_uint64,
            _ip, ctypes.c_int64, _dp, _dp, _ip, ctypes.c_int]
        _u64p = ctypes.POINTER(ctypes.c_uint64)
        lib.mfa_oracle_philox4x64.restype = None
        lib.mfa_oracle_philox4x64.argtypes = [_u64p, _u64p, _u64p]
        lib.mfa_oracle_dropout_keep.restype = ctypes.c_int
        lib.mfa_oracle_dropout_keep.argtypes = [ctypes.c_uint64, ctypes.c_double] + [ctypes.c_int64] * 4
        lib.mfa_oracle_bwd.restype = ctypes.c_int
        lib.mfa_oracle_bwd.argtypes = [_fp] * 5 + [ctypes.c_int64] * 6 + [
            ctypes.c_double, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
            _fp, _ip, ctypes.c_double, ctypes.c_uint64, _dp, _dp, _dp, ctypes.c_int]
        lib.mfa_oracle_visible_counts.restype = ctypes.c_int64
        lib.mfa_oracle_visible_counts.argtypes = [_fp] + [ctypes.c_int64] * 3 + [
            ctypes.c_int, ctypes.c_int64, ctypes.c_int64, _ip]
        lib.mfa_oracle_key_range.restype = None
        lib.mfa_oracle_key_range.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                             ctypes.c_int64, _ip, _ip]
        lib.mfa_oracle_mutant.restype = ctypes.c_int
        self.lib = lib
        self.mutant = lib.mfa_oracle_mutant()

    def key_range(self, aq: int, Lk: int, causal: bool, window: int):
        lo, hi = ctypes.c_int64(), ctypes.c_int64()
        self.lib.mfa_oracle_key_range(aq, Lk, int(bool(causal)), window,
                                      ctypes.byref(lo), ctypes.byref(hi))
        return lo.value, hi.value

    def philox4x64(self, ctr, key):
        """Philox4x64-10 of a 4-word counter and 2-word key (four uint64)."""
        c = (ctypes.c_uint64 * 4)(*[int(x) for x in ctr])
        kk = (ctypes.c_uint64 * 2)(*[int(x) for x in key])
        out = (ctypes.c_uint64 * 4)()
        self.lib.mfa_oracle_philox4x64(c, kk, out)
        return [int(x) for x in out]

    def dropout_keep(self, seed, p, b, hq, i, j) -> bool:
        return bool(self.lib.mfa_oracle_dropout_keep(int(seed), float(p), int(b), int(hq), int(i), int(j)))

    def rows(self, q, k, v, rows, *, scale, causal=False, window=0, q_offset=None,
             softcap=0.0, key_mask=None, bias=None, dropout_p=0.0, seed=0, nthreads=1):
        """Evaluate the rows given as an (n, 3) array of (b, hq, i).

        q is [B, Lq, Hq, D]; k, v are [B, Lk, Hkv, D]; key_mask is [B, Lk] or
        None; bias is an additive score mask whose shape (bB, bH, bLq, bLk)
        has each dimension 1 (broadcast) or B, Hq, Lq, Lk, or None;
        dropout_p and seed drive attention dropout.  Returns (out [n, D]
        float64, lse [n] float64, nvis [n] int64).
        """
        q, k, v, m = _f32(q), _f32(k), _f32(v), _f32(key_mask)
        bias = _f32(bias)
        strides = None
        if bias is not None:
            assert bias.ndim == 4
            full = (q.shape[0], q.shape[2], q.shape[1], k.shape[1])
            st = [int(x) for x in np.array(bias.strides) // bias.itemsize]
            for e in range(4):
                assert bias.shape[e] in (1, full[e]), (bias.shape, full)
                if bias.shape[e] == 1:
                    st[e] = 0
            strides = np.array(st, np.int64)
        B, Lq, Hq, D = q.shape
        Lk, Hkv = k.shape[1], k.shape[2]
        assert k.shape == (B, Lk, Hkv, D) and v.shape == k.shape
        if m is not None:
            assert m.shape == (B, Lk)
        if q_offset is None:
            q_offset = Lk - Lq
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
        n = rows.shape[0]
        out = np.zeros((n, D), np.float64)
        lse = np.zeros(n, np.float64)
        nvis = np.zeros(n, np.int64)
        rc = self.lib.mfa_oracle_rows_ext(
            _ptr(q, _fp), _ptr(k, _fp), _ptr(v, _fp), _ptr(m, _fp),
            B, Lq, Lk, Hq, Hkv, D, float(scale), int(bool(causal)), int(window), int(q_offset),
            float(softcap), _ptr(bias, _fp), _ptr(strides, _ip), float(dropout_p), int(seed),
            _ptr(rows, _ip), n, _ptr(out, _dp), _ptr(lse, _dp), _ptr(nvis, _ip),
            int(nthreads))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return out, lse, nvis

    @staticmethod
    def _bias_strides(bias, q, k):
        if bias is None:
            return None, None
        full = (q.shape[0], q.shape[2], q.shape[1], k.shape[1])
        st = [int(x) for x in np.array(bias.strides) // bias.itemsize]
        for e in range(4):
            assert bias.shape[e] in (1, full[e]), (bias.shape, full)
            if bias.shape[e] == 1:
                st[e] = 0
        return bias, np.array(st, np.int64)

    def bwd(self, q, k, v, dout, *, scale, causal=False, window=0, q_offset=None, softcap=0.0,
            key_mask=None, bias=None, dropout_p=0.0, seed=0, nthreads=1):
        """Gradients (dq [B,Lq,Hq,D], dk, dv [B,Lk,Hkv,D], float64) of the
        forward with the same arguments for the upstream gradient dout."""
        q, k, v, g, m = _f32(q), _f32(k), _f32(v), _f32(dout), _f32(key_mask)
        bias, strides = self._bias_strides(_f32(bias), q, k)
        B, Lq, Hq, D = q.shape
        Lk, Hkv = k.shape[1], k.shape[2]
        if q_offset is None:
            q_offset = Lk - Lq
        dq = np.zeros(q.shape, np.float64)
        dk = np.zeros(k.shape, np.float64)
        dv = np.zeros(k.shape, np.float64)
        rc = self.lib.mfa_oracle_bwd(
            _ptr(q, _fp), _ptr(k, _fp), _ptr(v, _fp), _ptr(g, _fp), _ptr(m, _fp),
            B, Lq, Lk, Hq, Hkv, D, float(scale), int(bool(causal)), int(window), int(q_offset),
            float(softcap), _ptr(bias, _fp), _ptr(strides, _ip), float(dropout_p), int(seed),
            _ptr(dq, _dp), _ptr(dk, _dp), _ptr(dv, _dp), int(nthreads))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return dq, dk, dv

    def full(self, q, k, v, **kw):
        """Every row: returns O [B, Lq, Hq, D] and LSE [B, Hq, Lq] (float64)."""
        q = _f32(q)
        B, Lq, Hq, D = q.shape
        b, h, i = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(Lq), indexing="ij")
        rows = np.stack([b.ravel(), h.ravel(), i.ravel()], 1)
        out, lse, nvis = self.rows(q, k, v, rows, **kw)
        O = out.reshape(B, Hq, Lq, D).transpose(0, 2, 1, 3).copy()
        return O, lse.reshape(B, Hq, Lq), nvis.reshape(B, Hq, Lq)

    def decode_len(self, q, k, v, lens, *, scale, softcap=0.0, nthreads=1):
        """Decode over the first lens[b] keys of a fixed-capacity cache.

        brotensor flash_attention.h, flash_attention_decode_len: the R query
        rows of a batch are consecutive positions whose keys are the last R of
        the valid ones, so row r attends causally to the first len - R + 1 + r
        keys, and a length of 0 writes zeros.  That is the plain forward over
        the valid prefix with the rows at positions len - R .. len - 1, which
        is how it is evaluated here (rows before position 0 see no key).
        q [B, R, Hq, D]; k, v [B, Lmax, Hkv, D]; lens [B] integers, clamped to
        [0, Lmax].  Returns O [B, R, Hq, D], LSE [B, Hq, R] and the visible
        counts [B, Hq, R].
        """
        q, k, v = _f32(q), _f32(k), _f32(v)
        B, R, Hq, D = q.shape
        Lmax = k.shape[1]
        O = np.zeros((B, R, Hq, D), np.float64)
        L = np.full((B, Hq, R), -np.inf, np.float64)
        N = np.zeros((B, Hq, R), np.int64)
        lens = np.asarray(lens).reshape(-1)
        for b in range(B):
            n = min(max(int(lens[b]), 0), Lmax)
            if n == 0:
                continue
            Ob, Lb, Nb = self.full(q[b:b + 1], k[b:b + 1, :n], v[b:b + 1, :n], scale=scale,
                                   causal=True, window=0, q_offset=n - R, softcap=softcap)
            O[b], L[b], N[b] = Ob[0], Lb[0], Nb[0]
        return O, L, N

    def decode_masked(self, q, k, v, mask, *, scale, window=0, softcap=0.0, nthreads=1):
        """Single-query decode over a fixed-capacity cache whose valid keys are
        marked by a key mask (brotensor flash_attention.h,
        flash_attention_decode_masked).  Batch b's query sits at position p,
        the last key whose mask value is above 0.5; key j is kept when its
        mask value is above 0.5 and, with window > 0, j > p - window (keys
        [max(0, p - window + 1), p]); window <= 0 keeps every valid key.  A
        batch without a valid key gets O = 0 and LSE = -inf.  That is the
        plain causal forward at one query row with q_offset = p, the window
        and the mask, which is how it is evaluated here.
        q [B, 1, Hq, D]; k, v [B, Lmax, Hkv, D]; mask [B, Lmax].  Returns
        O [B, 1, Hq, D], LSE [B, Hq, 1] and the visible counts [B, Hq, 1].
        """
        q, k, v, m = _f32(q), _f32(k), _f32(v), _f32(mask)
        B, R, Hq, D = q.shape
        assert R == 1, "one query row per batch"
        Lmax = k.shape[1]
        assert m.shape == (B, Lmax)
        O = np.zeros((B, 1, Hq, D), np.float64)
        L = np.full((B, Hq, 1), -np.inf, np.float64)
        N = np.zeros((B, Hq, 1), np.int64)
        for b in range(B):
            valid = np.nonzero(m[b] > 0.5)[0]
            if valid.size == 0:
                continue
            p = int(valid[-1])
            Ob, Lb, Nb = self.full(q[b:b + 1], k[b:b + 1], v[b:b + 1], scale=scale, causal=True,
                                   window=window, q_offset=p, softcap=softcap, key_mask=m[b:b + 1],
                                   nthreads=nthreads)
            O[b], L[b], N[b] = Ob[0], Lb[0], Nb[0]
        return O, L, N

    def packed_qkv(self, qkv, seq_bounds, num_heads, *, scale, window=0, softcap=0.0, nthreads=1):
        """Bidirectional attention over sequences packed back to back in one
        fused QKV tensor (brotensor flash_attention.h,
        flash_attention_packed_qkv_forward): each row attends only inside its
        own sequence, with the bidirectional window (|r - j| <= window/2) when
        window > 0.  The sequences are independent problems, so each is the
        plain forward on its own rows.  qkv [L, 3*H*D] (per row: query heads,
        key heads, value heads); seq_bounds [L, 2].  Returns O [L, H, D],
        LSE [H, L] and the visible counts [H, L].
        """
        x = _f32(qkv)
        try:
            import torch
            if isinstance(seq_bounds, torch.Tensor):
                seq_bounds = seq_bounds.detach().cpu().numpy()
        except ImportError:  # pragma: no cover
            pass
        sb = np.asarray(seq_bounds, dtype=np.int64).reshape(-1, 2)
        L = x.shape[0]
        H = int(num_heads)
        D = x.shape[1] // (3 * H)
        q = x[:, :H * D].reshape(1, L, H, D)
        k = x[:, H * D:2 * H * D].reshape(1, L, H, D)
        v = x[:, 2 * H * D:].reshape(1, L, H, D)
        O = np.zeros((L, H, D), np.float64)
        LSE = np.full((H, L), -np.inf, np.float64)
        N = np.zeros((H, L), np.int64)
        r = 0
        while r < L:
            s0, s1 = int(sb[r, 0]), int(sb[r, 1])
            if not (s0 == r and s1 > r and s1 <= L and np.all(sb[s0:s1] == (s0, s1))):
                raise ValueError(f"row {r}: bounds ({s0}, {s1}) do not describe back-to-back sequences")
            Os, Ls, Ns = self.full(q[:, s0:s1], k[:, s0:s1], v[:, s0:s1], scale=scale, causal=False,
                                   window=window, q_offset=0, softcap=softcap, nthreads=nthreads)
            O[s0:s1], LSE[:, s0:s1], N[:, s0:s1] = Os[0], Ls[0], Ns[0]
            r = s1
        return O, LSE, N

    def varlen(self, q, k, v, cu_q, cu_k, *, scale, causal=False, window=0, softcap=0.0, nthreads=1):
        """Attention over sequences packed back to back with separate query
        and key packings (brotensor flash_attention.h,
        flash_attention_varlen_forward): sequence b owns query rows
        [cu_q[b], cu_q[b+1]) and key rows [cu_k[b], cu_k[b+1]) and nothing
        else; causal keeps key k for query q when k - cu_k[b] <= q - cu_q[b]
        (positions counted from each sequence's start).  Each sequence is the
        plain forward on its own rows with q_offset 0; rows of no sequence, and
        sequences without keys, give O = 0 and LSE = -inf.
        q [Tq, Hq, D]; k, v [Tk, Hkv, D]; cu_q, cu_k [batch + 1] prefix sums.
        Returns O [Tq, Hq, D], LSE [Hq, Tq] and the visible counts [Hq, Tq].
        """
        q, k, v = _f32(q), _f32(k), _f32(v)
        cq = np.asarray(cu_q.cpu() if hasattr(cu_q, "cpu") else cu_q, dtype=np.int64).reshape(-1)
        ck = np.asarray(cu_k.cpu() if hasattr(cu_k, "cpu") else cu_k, dtype=np.int64).reshape(-1)
        Tq, Hq, D = q.shape
        O = np.zeros((Tq, Hq, D), np.float64)
        LSE = np.full((Hq, Tq), -np.inf, np.float64)
        N = np.zeros((Hq, Tq), np.int64)
        for b in range(len(cq) - 1):
            q0, q1, k0, k1 = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
            if q1 <= q0 or k1 <= k0:
                continue
            Ob, Lb, Nb = self.full(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], scale=scale,
                                   causal=causal, window=window, q_offset=0, softcap=softcap,
                                   nthreads=nthreads)
            O[q0:q1], LSE[:, q0:q1], N[:, q0:q1] = Ob[0], Lb[0], Nb[0]
        return O, LSE, N

    def visible_counts(self, B, Lq, Lk, *, causal=False, window=0, q_offset=None, key_mask=None):
        """Visible-key count of every row, [B, Lq] int64, and the total."""
        m = _f32(key_mask)
        if q_offset is None:
            q_offset = Lk - Lq
        counts = np.zeros((B, Lq), np.int64)
        total = self.lib.mfa_oracle_visible_counts(_ptr(m, _fp), B, Lq, Lk, int(bool(causal)),
                                                   int(window), int(q_offset), _ptr(counts, _ip))
        return counts, int(total)


_default = None


def default_oracle() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
