"""GPU parity on seeded random combinations of the forward's options.

Each case draws its shape and flags from one seeded generator: dtype, head
size, batch, kv heads and group size, query and key lengths (decode rows
included), an arbitrary q_offset in [0, Lk - Lq], causal or bidirectional,
no window / a negative window / a window from 1 to 2 Lk, a soft-cap, no mask /
a padding mask / a random key mask, and the input scale (standard deviation 1
or 2).
Every row of every case is compared with the fp64 oracle, through the automatic
path and through each forced kernel path that serves the call (the split
decode with a drawn split count).
"""
import numpy as np
import pytest
import torch

import transformer_mfa_fwd_amd as mfa
from oracle import default_oracle
from tests import parity_util as pu
from transformer_mfa_fwd_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda"
N_CASES = 48


def draw_case(i: int):
    rng = np.random.default_rng(1000 + i)
    dtype = str(rng.choice(["bf16", "f16", "f32"], p=[0.45, 0.4, 0.15]))
    D = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 4))
    Hkv = int(rng.integers(1, 4))
    Hq = Hkv * int(rng.integers(1, 6))
    Lk = int(rng.integers(1, 401))
    Lq = 1 if rng.random() < 0.3 else int(rng.integers(1, Lk + 1))
    r = rng.random()
    q_offset = Lk - Lq if r < 0.4 else (0 if r < 0.6 else int(rng.integers(0, Lk - Lq + 1)))
    causal = bool(rng.random() < 0.6)
    r = rng.random()
    window = 0 if r < 0.4 else (-1 if r < 0.5 else int(rng.integers(1, 2 * Lk + 1)))
    softcap = 0.0 if rng.random() < 0.6 else float(rng.uniform(2.0, 50.0))
    r = rng.random()
    if r < 0.5:
        mask = dict(mask=None)
    elif r < 0.75:
        mask = dict(mask="pad_tail", pad_max=max(1, Lk // 2))
    else:
        mask = dict(mask="random_frac", mask_frac=float(rng.uniform(0.05, 0.6)))
    # std 2 with bf16 is the class of inputs that needs the fp16 P.V operands
    # (8-bit bf16 weights alone err by up to ~0.03 on short, peaked rows)
    std = float(rng.choice([1.0, 2.0]))
    w = wl.Workload(f"fuzz{i}", dtype, B, Lq, Lk, Hq, Hkv, D, causal, window=window, softcap=softcap,
                    std=std, **mask)
    splits = int(rng.choice([0, 1, 3, 7]))
    return w, q_offset, splits


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_options_every_row(i):
    w, q_offset, splits = draw_case(i)
    print(f"\n[fuzz] case {i}: {w} q_offset={q_offset} splits={splits}", flush=True)
    q, k, v, m = wl.make_inputs(w, DEV, seed=i)
    kw = dict(causal=w.causal, window=w.window, q_offset=q_offset, softcap=w.softcap, scale=w.scale)
    O, L, _ = default_oracle().full(q, k, v, key_mask=m, nthreads=pu.ORACLE_THREADS, **kw)
    O = O.transpose(0, 2, 1, 3)     # [B, Hq, Lq, D], lined up with LSE [B, Hq, Lq]
    paths = [("auto", mfa.PATH_AUTO, 0), ("generic", mfa.PATH_GENERIC, 0)]
    if w.dtype != "f32":
        paths.append(("mfma", mfa.PATH_MFMA, 0))
        if w.Lq == 1 and w.Hq // w.Hkv <= 16:
            paths.append(("split_decode", mfa.PATH_SPLIT_DECODE, splits))
    for name, path, s in paths:
        out, lse = mfa.fwd(q, k, v, key_mask=m, path=path, splits=s, **kw)
        torch.cuda.synchronize()
        og = out.double().cpu().numpy().transpose(0, 2, 1, 3)
        pu.compare(w.dtype, og, lse.double().cpu().numpy(), O, L, f"fuzz {i} {name}")


# --- the other entry points ---------------------------------------------------

def _dtype_D_std(rng, backward=False):
    dtype = str(rng.choice(["bf16", "f16", "f32"], p=[0.45, 0.4, 0.15]))
    D = int(rng.choice([64, 128]))
    # The backward's products take bf16 operands (P, dS: 8 significant bits),
    # whose rounding on wider data exceeds the per-row 1e-2 gradient bound
    # (std 1.5 with dropout 0.5 measured 0.023 against 0.022): its bf16 draws
    # keep std 1.  The forward keeps its weights in fp16 and draws std 2 too.
    stds = [1.0] if backward and dtype == "bf16" else [1.0, 1.5, 2.0]
    std = float(rng.choice(stds))
    return dtype, D, std


@pytest.mark.parametrize("i", range(24))
def test_random_decode_len_every_row(i):
    """mfa_decode_len: draft rows, GQA, capacity, per-batch lengths (0, below
    R, full and random), soft-cap and split count drawn at random."""
    rng = np.random.default_rng(2000 + i)
    dtype = str(rng.choice(["bf16", "f16"]))
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.integers(1, 4))
    g = int(rng.choice([1, 2, 4, 8]))
    R = int(rng.integers(1, 16 // g + 1))
    B = int(rng.integers(1, 5))
    Lmax = int(rng.integers(1, 601))
    lens = [int(rng.choice([0, max(0, R - 1), Lmax, int(rng.integers(0, Lmax + 1))])) for _ in range(B)]
    softcap = 0.0 if rng.random() < 0.6 else float(rng.uniform(2.0, 40.0))
    splits = int(rng.choice([0, 1, 3, 7]))
    std = float(rng.choice([1.0, 2.0]))
    print(f"\n[fuzz] decode_len {i}: {dtype} D={D} B={B} R={R} Hq={Hkv * g} Hkv={Hkv} Lmax={Lmax} "
          f"lens={lens} softcap={softcap:.2f} splits={splits} std={std}", flush=True)
    gen = torch.Generator(device="cpu").manual_seed(i)
    dt = wl.DTYPES[dtype]
    q = (torch.randn((B, R, Hkv * g, D), generator=gen) * std).to(dt)
    k = (torch.randn((B, Lmax, Hkv, D), generator=gen) * std).to(dt)
    v = (torch.randn((B, Lmax, Hkv, D), generator=gen) * std).to(dt)
    scale = 1.0 / np.sqrt(D)
    O, L, _ = default_oracle().decode_len(q, k, v, np.array(lens), scale=scale, softcap=softcap,
                                          nthreads=pu.ORACLE_THREADS)
    out, lse = mfa.decode_len(q.to(DEV), k.to(DEV), v.to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV),
                              softcap=softcap, scale=scale, splits=splits)
    torch.cuda.synchronize()
    og = out.double().cpu().numpy().transpose(0, 2, 1, 3)
    pu.compare(dtype, og, lse.double().cpu().numpy(), O.transpose(0, 2, 1, 3), L, f"decode_len {i}")


@pytest.mark.parametrize("i", range(24))
def test_random_varlen_every_row(i):
    """mfa_varlen_fwd: 1-5 sequences with query and key lengths drawn from
    0..150 (empty sequences included), GQA, causal or not, window, soft-cap."""
    rng = np.random.default_rng(3000 + i)
    dtype, D, std = _dtype_D_std(rng)
    nb = int(rng.integers(1, 6))
    lq = [int(rng.choice([0, 1, int(rng.integers(0, 151))])) for _ in range(nb)]
    lk = [int(rng.choice([0, 1, int(rng.integers(0, 151))])) for _ in range(nb)]
    if sum(lq) == 0:
        lq[0] = 1
    Hkv = int(rng.integers(1, 4))
    Hq = Hkv * int(rng.integers(1, 5))
    causal = bool(rng.random() < 0.6)
    window = 0 if rng.random() < 0.5 else int(rng.integers(1, 200))
    softcap = 0.0 if rng.random() < 0.6 else float(rng.uniform(2.0, 40.0))
    print(f"\n[fuzz] varlen {i}: {dtype} D={D} lq={lq} lk={lk} Hq={Hq} Hkv={Hkv} causal={causal} "
          f"window={window} softcap={softcap:.2f} std={std}", flush=True)
    gen = torch.Generator(device="cpu").manual_seed(i)
    dt = wl.DTYPES[dtype]
    Tq, Tk = sum(lq), sum(lk)
    q = (torch.randn((Tq, Hq, D), generator=gen) * std).to(dt)
    k = (torch.randn((Tk, Hkv, D), generator=gen) * std).to(dt)
    v = (torch.randn((Tk, Hkv, D), generator=gen) * std).to(dt)
    cq = torch.tensor(np.concatenate([[0], np.cumsum(lq)]), dtype=torch.int32)
    ck = torch.tensor(np.concatenate([[0], np.cumsum(lk)]), dtype=torch.int32)
    O, L, _ = default_oracle().varlen(q, k, v, cq, ck, scale=1.0 / np.sqrt(D), causal=causal, window=window,
                                      softcap=softcap, nthreads=pu.ORACLE_THREADS)
    # an empty key packing still passes valid (non-null) device pointers
    kd = torch.zeros((max(Tk, 1), Hkv, D), dtype=dt, device=DEV)[:Tk]
    vd = torch.zeros((max(Tk, 1), Hkv, D), dtype=dt, device=DEV)[:Tk]
    kd.copy_(k.to(DEV))
    vd.copy_(v.to(DEV))
    out, lse = mfa.varlen_fwd(q.to(DEV), kd, vd, cq.to(DEV), ck.to(DEV), causal=causal, window=window,
                              softcap=softcap)
    torch.cuda.synchronize()
    pu.compare(dtype, out.double().cpu().numpy().transpose(1, 0, 2), lse.double().cpu().numpy(),
               O.transpose(1, 0, 2), L, f"varlen {i}")


@pytest.mark.parametrize("i", range(16))
def test_random_packed_qkv_every_row(i):
    """mfa_packed_qkv_fwd: 1-6 sequences of 1..200 rows in one fused QKV
    tensor, bidirectional window or none, soft-cap."""
    rng = np.random.default_rng(4000 + i)
    dtype, D, std = _dtype_D_std(rng)
    lengths = [int(rng.integers(1, 201)) for _ in range(int(rng.integers(1, 7)))]
    H = int(rng.integers(1, 5))
    window = 0 if rng.random() < 0.4 else int(rng.integers(1, 300))
    softcap = 0.0 if rng.random() < 0.6 else float(rng.uniform(2.0, 40.0))
    print(f"\n[fuzz] packed {i}: {dtype} D={D} H={H} lengths={lengths} window={window} "
          f"softcap={softcap:.2f}", flush=True)
    qkv, sb = wl.make_packed_qkv(lengths, H, D, dtype, "cpu", seed=i, std=std)
    O, L, _ = default_oracle().packed_qkv(qkv, sb, H, scale=1.0 / np.sqrt(D), window=window, softcap=softcap,
                                          nthreads=pu.ORACLE_THREADS)
    out, lse = mfa.packed_qkv_fwd(qkv.to(DEV), sb.to(DEV), H, window=window, softcap=softcap)
    torch.cuda.synchronize()
    og = out.double().cpu().numpy().reshape(O.shape)
    pu.compare(dtype, og.transpose(1, 0, 2), lse.double().cpu().numpy(), O.transpose(1, 0, 2), L, f"packed {i}")


@pytest.mark.parametrize("i", range(16))
def test_random_backward_every_element(i):
    """mfa_bwd after libmfa's own forward: every forward option drawn at
    random, plus an additive mask of a random broadcast shape and dropout."""
    rng = np.random.default_rng(5000 + i)
    dtype, D, std = _dtype_D_std(rng, backward=True)
    B = int(rng.integers(1, 3))
    Hkv = int(rng.integers(1, 3))
    Hq = Hkv * int(rng.integers(1, 4))
    Lk = int(rng.integers(1, 161))
    Lq = 1 if rng.random() < 0.2 else int(rng.integers(1, Lk + 1))
    q_offset = int(rng.integers(0, Lk - Lq + 1))
    causal = bool(rng.random() < 0.6)
    window = 0 if rng.random() < 0.5 else int(rng.integers(1, 2 * Lk + 1))
    softcap = 0.0 if rng.random() < 0.7 else float(rng.uniform(2.0, 30.0))
    mask = dict(mask=None) if rng.random() < 0.6 else dict(mask="random_frac", mask_frac=0.25)
    bias_dims = None if rng.random() < 0.6 else [bool(rng.random() < 0.5) for _ in range(4)]
    p = 0.0 if rng.random() < 0.6 else float(rng.choice([0.1, 0.5]))
    w = wl.Workload(f"bwdfuzz{i}", dtype, B, Lq, Lk, Hq, Hkv, D, causal, window=window, softcap=softcap,
                    std=std, **mask)
    print(f"\n[fuzz] backward {i}: {w} q_offset={q_offset} bias={bias_dims} p={p}", flush=True)
    q, k, v, m = wl.make_inputs(w, DEV, seed=i)
    gen = torch.Generator(device="cpu").manual_seed(100 + i)
    dout = torch.randn(q.shape, generator=gen).to(q.dtype).to(DEV)
    bias = None
    if bias_dims is not None:
        full = (B, Hq, Lq, Lk)
        bias = (torch.randn(tuple(full[e] if bias_dims[e] else 1 for e in range(4)), generator=gen) * 1.5)
    kw = dict(causal=causal, window=window, q_offset=q_offset, softcap=softcap, key_mask=m, scale=w.scale,
              dropout_p=p, seed=7 + i)
    bd = None if bias is None else bias.contiguous().to(DEV)
    out, lse = mfa.fwd(q, k, v, bias=bd, **kw)
    dq, dk, dv = mfa.bwd(q, k, v, out, dout, lse, bias=bd, **kw)
    torch.cuda.synchronize()
    rq, rk, rv = default_oracle().bwd(q, k, v, dout, bias=bias, nthreads=pu.ORACLE_THREADS, **kw)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        pu.compare_grad(name, got, ref, dtype, w.name, dropout_p=p)


@pytest.mark.parametrize("i", range(12))
def test_random_medium_shapes_sampled_rows(i):
    """Longer axes (keys up to 6000, many query tiles), every forward option
    drawn as above; sampled rows at tile and window edges plus random rows."""
    rng = np.random.default_rng(6000 + i)
    dtype = str(rng.choice(["bf16", "f16"]))
    D = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 3))
    Hkv = int(rng.integers(1, 3))
    Hq = Hkv * int(rng.choice([1, 2, 4]))
    Lk = int(rng.integers(1000, 6001))
    Lq = 1 if rng.random() < 0.2 else int(rng.integers(1, Lk + 1))
    q_offset = Lk - Lq if rng.random() < 0.5 else int(rng.integers(0, Lk - Lq + 1))
    causal = bool(rng.random() < 0.6)
    window = 0 if rng.random() < 0.4 else int(rng.integers(1, Lk))
    softcap = 0.0 if rng.random() < 0.6 else float(rng.uniform(5.0, 50.0))
    r = rng.random()
    mask = dict(mask=None) if r < 0.5 else (dict(mask="pad_tail", pad_max=Lk // 3) if r < 0.75 else
                                            dict(mask="random_frac", mask_frac=0.1))
    std = float(rng.choice([1.0, 2.0]))
    w = wl.Workload(f"medium{i}", dtype, B, Lq, Lk, Hq, Hkv, D, causal, window=window, softcap=softcap,
                    std=std, **mask)
    print(f"\n[fuzz] medium {i}: {w} q_offset={q_offset}", flush=True)
    q, k, v, m = wl.make_inputs(w, DEV, seed=i)
    kw = dict(causal=causal, window=window, q_offset=q_offset, softcap=softcap, scale=w.scale)
    out, lse = mfa.fwd(q, k, v, key_mask=m, **kw)
    torch.cuda.synchronize()
    rows = pu.sample_rows(w, n_random=8, seed=i)
    O, L, _ = default_oracle().rows(q, k, v, rows, key_mask=m, nthreads=pu.ORACLE_THREADS, **kw)
    og, lg = pu.gather_rows(out, lse, rows)
    pu.compare(dtype, og, lg, O, L, f"medium {i}")


@pytest.mark.parametrize("i", range(16))
def test_random_bias_dropout_forward_every_row(i):
    """mfa_fwd_bias_dropout: an additive mask of a random broadcast shape
    and/or dropout, with the other forward options drawn at random."""
    rng = np.random.default_rng(7000 + i)
    dtype, D, std = _dtype_D_std(rng)
    B = int(rng.integers(1, 3))
    Hkv = int(rng.integers(1, 3))
    Hq = Hkv * int(rng.integers(1, 4))
    Lk = int(rng.integers(1, 301))
    Lq = 1 if rng.random() < 0.2 else int(rng.integers(1, Lk + 1))
    q_offset = int(rng.integers(0, Lk - Lq + 1))
    causal = bool(rng.random() < 0.6)
    window = 0 if rng.random() < 0.5 else int(rng.integers(1, 2 * Lk + 1))
    softcap = 0.0 if rng.random() < 0.7 else float(rng.uniform(2.0, 30.0))
    mask = dict(mask=None) if rng.random() < 0.6 else dict(mask="random_frac", mask_frac=0.25)
    bias_dims = None if rng.random() < 0.3 else [bool(rng.random() < 0.5) for _ in range(4)]
    p = float(rng.choice([0.0, 0.1, 0.5])) if bias_dims is not None else float(rng.choice([0.1, 0.5]))
    w = wl.Workload(f"biasfuzz{i}", dtype, B, Lq, Lk, Hq, Hkv, D, causal, window=window, softcap=softcap,
                    std=std, **mask)
    print(f"\n[fuzz] bias/dropout {i}: {w} q_offset={q_offset} bias={bias_dims} p={p}", flush=True)
    q, k, v, m = wl.make_inputs(w, DEV, seed=i)
    gen = torch.Generator(device="cpu").manual_seed(200 + i)
    bias = None
    if bias_dims is not None:
        full = (B, Hq, Lq, Lk)
        bias = torch.randn(tuple(full[e] if bias_dims[e] else 1 for e in range(4)), generator=gen) * 1.5
    kw = dict(causal=causal, window=window, q_offset=q_offset, softcap=softcap, key_mask=m, scale=w.scale,
              dropout_p=p, seed=11 + i)
    out, lse = mfa.fwd(q, k, v, bias=None if bias is None else bias.contiguous().to(DEV), **kw)
    torch.cuda.synchronize()
    O, L, _ = default_oracle().full(q, k, v, bias=bias, nthreads=pu.ORACLE_THREADS, **kw)
    og = out.double().cpu().numpy().transpose(0, 2, 1, 3)
    pu.compare(dtype, og, lse.double().cpu().numpy(), O.transpose(0, 2, 1, 3), L, f"bias/dropout {i}",
               o_scale=1.0 / (1.0 - p))


@pytest.mark.parametrize("i", range(8))
def test_random_backward_longer_axes(i):
    """mfa_bwd on 200-1500 query and 300-1500 key rows (many pipeline steps
    per key block), options drawn as above, every gradient element."""
    rng = np.random.default_rng(9000 + i)
    dtype = str(rng.choice(["bf16", "f16"]))
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.integers(1, 3))
    Hq = Hkv * int(rng.choice([1, 2, 4]))
    Lk = int(rng.integers(300, 1501))
    Lq = int(rng.integers(200, Lk + 1))
    q_offset = int(rng.integers(0, Lk - Lq + 1))
    causal = bool(rng.random() < 0.7)
    window = 0 if rng.random() < 0.5 else int(rng.integers(1, Lk))
    softcap = 0.0 if rng.random() < 0.7 else float(rng.uniform(5.0, 40.0))
    mask = dict(mask=None) if rng.random() < 0.7 else dict(mask="random_frac", mask_frac=0.2)
    p = float(rng.choice([0.1, 0.3])) if rng.random() < 0.3 else 0.0
    w = wl.Workload(f"bwdlong{i}", dtype, 1, Lq, Lk, Hq, Hkv, D, causal, window=window, softcap=softcap, **mask)
    print(f"\n[fuzz] backward longer {i}: {w} q_offset={q_offset} p={p}", flush=True)
    q, k, v, m = wl.make_inputs(w, DEV, seed=i)
    gen = torch.Generator(device="cpu").manual_seed(300 + i)
    dout = torch.randn(q.shape, generator=gen).to(q.dtype).to(DEV)
    kw = dict(causal=causal, window=window, q_offset=q_offset, softcap=softcap, key_mask=m, scale=w.scale,
              dropout_p=p, seed=5 + i)
    out, lse = mfa.fwd(q, k, v, **kw)
    dq, dk, dv = mfa.bwd(q, k, v, out, dout, lse, **kw)
    torch.cuda.synchronize()
    rq, rk, rv = default_oracle().bwd(q, k, v, dout, nthreads=pu.ORACLE_THREADS, **kw)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        pu.compare_grad(name, got, ref, dtype, w.name, dropout_p=p)
