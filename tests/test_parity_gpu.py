"""GPU parity: libmfa (through its C ABI) against the fp64 oracle.

Small shapes are compared on every row; they span several tiles with ragged
tails.  The full-size workloads are compared on sampled rows, and every row of
them is checked for the exact visible-key count through Q = 0.
"""
import math
import sys

import numpy as np
import pytest
import torch

import transformer_mfa_fwd_amd as mfa
from oracle import default_oracle
from tests import parity_util as pu
from transformer_mfa_fwd_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda"
PATHS = {"generic": mfa.PATH_GENERIC, "mfma": mfa.PATH_MFMA, "split_decode": mfa.PATH_SPLIT_DECODE}


def say(msg):
    print(f"\n[parity] {msg}", flush=True)
    sys.stdout.flush()


def path_available(path, w):
    """Probe whether a forced path serves these arguments (host-side check)."""
    if path == "generic":
        return True
    if path == "split_decode" and w.Lq != 1:
        return False
    # a tiny call through the forced path tells whether it is built
    q = torch.zeros((1, 1, w.Hq, w.D), dtype=w.torch_dtype, device=DEV)
    k = torch.zeros((1, 4, w.Hkv, w.D), dtype=w.torch_dtype, device=DEV)
    try:
        mfa.fwd(q, k, k, path=PATHS[path], causal=True)
        torch.cuda.synchronize()
        return True
    except mfa.MFAError as e:
        if e.status == 2:
            return False
        raise


def run_case(w, path="auto", seed=0, rows=None, q_zero=False):
    q, k, v, m = wl.make_inputs(w, DEV, seed)
    if q_zero:
        q = torch.zeros_like(q)
    say(f"{w.name} path={path} seed={seed}")
    out, lse = mfa.fwd(q, k, v, causal=w.causal, window=w.window, q_offset=w.q_offset,
                       softcap=w.softcap, key_mask=m, scale=w.scale,
                       path=PATHS.get(path, mfa.PATH_AUTO))
    torch.cuda.synchronize()
    return q, k, v, m, out, lse


def check_all_rows(w, path="auto", seed=0):
    q, k, v, m, out, lse = run_case(w, path, seed)
    O, L, _ = default_oracle().full(q, k, v, scale=w.scale, causal=w.causal, window=w.window,
                                    q_offset=w.q_offset, softcap=w.softcap, key_mask=m,
                                    nthreads=pu.ORACLE_THREADS)
    # row form: O as [B, Hq, Lq, D] so that it lines up with LSE [B, Hq, Lq]
    og = out.double().cpu().numpy().transpose(0, 2, 1, 3)
    return pu.compare(w.dtype, og, lse.double().cpu().numpy(), O.transpose(0, 2, 1, 3), L,
                      f"{w.name}/{path}")


# --- small shapes: several tiles, ragged tails, every flag -------------------

SMALL = []
for dtype in ("f32", "f16", "bf16"):
    for D in (64, 128):
        SMALL += [
            wl.Workload(f"causal_gqa_{dtype}_D{D}", dtype, 2, 200, 200, 4, 2, D, True),
            wl.Workload(f"bidir_{dtype}_D{D}", dtype, 1, 150, 150, 2, 2, D, False),
            wl.Workload(f"causal_win37_mask_{dtype}_D{D}", dtype, 2, 190, 190, 4, 1, D, True, window=37,
                        mask="random_frac", mask_frac=0.3),
            wl.Workload(f"bidir_win100_pad_{dtype}_D{D}", dtype, 2, 260, 260, 3, 3, D, False, window=100,
                        mask="pad_tail", pad_max=120),
            wl.Workload(f"decode_block_softcap_{dtype}_D{D}", dtype, 2, 70, 333, 8, 2, D, True, window=0,
                        softcap=5.0, std=2.0),
            wl.Workload(f"decode1_{dtype}_D{D}", dtype, 3, 1, 517, 8, 2, D, True, window=0),
            wl.Workload(f"decode1_win_mask_cap_{dtype}_D{D}", dtype, 2, 1, 700, 16, 1, D, True, window=300,
                        softcap=20.0, mask="random_frac", mask_frac=0.5),
        ]


@pytest.mark.parametrize("path", ["generic", "mfma", "split_decode", "auto"])
@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small_all_rows(w, path):
    if path != "auto" and not path_available(path, w):
        pytest.skip(f"path {path} does not serve {w.name}")
    if path == "mfma" and w.dtype == "f32":
        pytest.skip("MFMA path is fp16/bf16 only")
    check_all_rows(w, path)


MASKED = [w for w in SMALL if w.mask is not None]


@pytest.mark.parametrize("path", ["generic", "mfma", "split_decode", "auto"])
@pytest.mark.parametrize("w", MASKED, ids=lambda w: w.name)
def test_masked_rows_may_hold_nan(w, path):
    """K and V rows of masked keys hold NaN (never-written memory, say): every
    path keeps them out of the products, so the output is finite and matches
    the oracle, which never touches them."""
    if path != "auto" and not path_available(path, w):
        pytest.skip(f"path {path} does not serve {w.name}")
    if path == "mfma" and w.dtype == "f32":
        pytest.skip("MFMA path is fp16/bf16 only")
    q, k, v, m = wl.make_inputs(w, DEV, 0)
    k, v = k.clone(), v.clone()
    dropped = m <= 0.5
    k[dropped] = float("nan")
    v[dropped] = float("nan")
    say(f"{w.name} path={path} (NaN in {int(dropped.sum())} masked rows)")
    out, lse = mfa.fwd(q, k, v, causal=w.causal, window=w.window, q_offset=w.q_offset, softcap=w.softcap,
                       key_mask=m, scale=w.scale, path=PATHS.get(path, mfa.PATH_AUTO))
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    O, L, _ = default_oracle().full(q, k, v, scale=w.scale, causal=w.causal, window=w.window,
                                    q_offset=w.q_offset, softcap=w.softcap, key_mask=m,
                                    nthreads=pu.ORACLE_THREADS)
    pu.compare(w.dtype, out.double().cpu().numpy().transpose(0, 2, 1, 3), lse.double().cpu().numpy(),
               O.transpose(0, 2, 1, 3), L, f"{w.name}/{path}/nan")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_masked_rows_may_hold_nan_with_additive_mask(dtype):
    """The same through the additive-mask kernels."""
    w = wl.Workload(f"nan_rows_bias_{dtype}", dtype, 2, 190, 190, 4, 2, 128, True, window=37,
                    mask="random_frac", mask_frac=0.3)
    q, k, v, m = wl.make_inputs(w, DEV, 1)
    k, v = k.clone(), v.clone()
    k[m <= 0.5] = float("nan")
    v[m <= 0.5] = float("nan")
    bias = torch.randn((1, 1, w.Lq, w.Lk), generator=torch.Generator().manual_seed(5))
    out, lse = mfa.fwd(q, k, v, causal=True, window=w.window, key_mask=m, scale=w.scale, bias=bias.to(DEV))
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    O, L, _ = default_oracle().full(q, k, v, scale=w.scale, causal=True, window=w.window, q_offset=0,
                                    key_mask=m, bias=bias, nthreads=pu.ORACLE_THREADS)
    pu.compare(dtype, out.double().cpu().numpy().transpose(0, 2, 1, 3), lse.double().cpu().numpy(),
               O.transpose(0, 2, 1, 3), L, f"{w.name}/nan")


# --- edge cases ---------------------------------------------------------------

EDGE = [
    wl.Workload("single_key_bf16", "bf16", 1, 1, 1, 2, 1, 64, True),
    wl.Workload("window1_f16", "f16", 1, 130, 130, 2, 2, 128, True, window=1),
    wl.Workload("all_masked_tail_bf16", "bf16", 2, 100, 100, 2, 1, 64, False, mask="pad_tail", pad_max=100),
    wl.Workload("short_lk_many_heads_bf16", "bf16", 1, 3, 5, 32, 8, 128, False),
    wl.Workload("lq_lt_lk_causal_f32", "f32", 2, 65, 129, 2, 1, 64, True),
    wl.Workload("big_bidir_window_bf16", "bf16", 1, 96, 96, 1, 1, 128, False, window=1000),
    wl.Workload("mqa_g16_f16", "f16", 1, 80, 80, 16, 1, 64, True),
    wl.Workload("mqa_g32_decode_bf16", "bf16", 2, 1, 300, 32, 1, 128, True),
    wl.Workload("gqa16_ragged_f16_D64", "f16", 3, 333, 333, 16, 1, 64, True, window=100),
    wl.Workload("lq_1_of_many_keys_bidir_bf16", "bf16", 2, 1, 1000, 4, 4, 128, False, window=300),
    wl.Workload("long_window_cap_mask_bf16", "bf16", 1, 700, 900, 4, 2, 128, True, window=513, softcap=10.0,
                mask="random_frac", mask_frac=0.4, std=2.0),
]


@pytest.mark.parametrize("w", EDGE, ids=lambda w: w.name)
def test_edge_cases(w):
    check_all_rows(w)


def test_fully_masked_batch_gives_zero_and_neg_inf():
    w = wl.Workload("masked_batch", "bf16", 2, 70, 70, 2, 1, 64, False)
    q, k, v, _ = wl.make_inputs(w, DEV)
    m = torch.ones(2, 70, device=DEV)
    m[0] = 0.0
    for path in ("auto", "generic"):
        out, lse = mfa.fwd(q, k, v, key_mask=m, path=PATHS.get(path, 0))
        torch.cuda.synchronize()
        assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
        assert torch.all(torch.isfinite(lse[1]))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_softcap_rows_without_visible_keys(dtype, D):
    """Soft-capped prefill (its scores kept as the cap's reciprocal, hidden
    ones as +inf) with a batch whose keys are all masked and rows whose only
    keys are masked (a causal window over a key mask with a masked head):
    those rows get O = 0 and LSE = -inf, every other row the oracle's values."""
    w = wl.Workload(f"cap_empty_rows_{dtype}_D{D}", dtype, 2, 200, 200, 4, 2, D, True, window=20, softcap=7.0)
    q, k, v, _ = wl.make_inputs(w, DEV)
    m = torch.ones(2, 200)
    m[0] = 0.0              # batch 0: no key
    m[1, :90] = 0.0         # batch 1: rows 0 .. 89 see only masked keys (window 20)
    md = m.to(DEV)
    out, lse = mfa.fwd(q, k, v, causal=True, window=w.window, softcap=w.softcap, key_mask=md, scale=w.scale,
                       path=mfa.PATH_MFMA)
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.all(out[1, :90] == 0) and torch.all(torch.isneginf(lse[1, :, :90]))
    O, L, _ = default_oracle().full(q, k, v, scale=w.scale, causal=True, window=w.window, q_offset=0,
                                    softcap=w.softcap, key_mask=m, nthreads=pu.ORACLE_THREADS)
    pu.compare(dtype, out.double().cpu().numpy().transpose(0, 2, 1, 3), lse.double().cpu().numpy(),
               O.transpose(0, 2, 1, 3), L, w.name)


def test_deterministic_and_no_out_of_bounds_writes():
    w = wl.Workload("canary", "bf16", 2, 190, 190, 4, 2, 128, True, window=50, mask="random_frac",
                    mask_frac=0.2)
    q, k, v, m = wl.make_inputs(w, DEV)
    n = q.numel()
    guard = 4096
    for path in ("auto", "generic"):
        outs = []
        for rep in range(2):
            obuf = torch.full((n + 2 * guard,), 7.0, dtype=q.dtype, device=DEV)
            lbuf = torch.full((w.B * w.Hq * w.Lq + 2 * guard,), 7.0, dtype=torch.float32, device=DEV)
            out = obuf[guard:guard + n].view(q.shape)
            lse = lbuf[guard:guard + w.B * w.Hq * w.Lq].view(w.B, w.Hq, w.Lq)
            mfa.fwd(q, k, v, causal=True, window=50, key_mask=m, out=out, lse=lse,
                    path=PATHS.get(path, 0))
            torch.cuda.synchronize()
            assert torch.all(obuf[:guard] == 7.0) and torch.all(obuf[-guard:] == 7.0)
            assert torch.all(lbuf[:guard] == 7.0) and torch.all(lbuf[-guard:] == 7.0)
            outs.append((out.clone(), lse.clone()))
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_gqa_equals_mha_on_repeated_kv():
    w = wl.Workload("gqa", "bf16", 2, 150, 150, 8, 2, 128, True, window=70)
    q, k, v, _ = wl.make_inputs(w, DEV)
    o1, l1 = mfa.fwd(q, k, v, causal=True, window=70)
    o2, l2 = mfa.fwd(q, k.repeat_interleave(4, dim=2).contiguous(),
                     v.repeat_interleave(4, dim=2).contiguous(), causal=True, window=70)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_workspace_entry_point_matches_pool_entry_point():
    w = wl.Workload("ws", "bf16", 2, 1, 900, 8, 2, 128, True, mask="random_frac", mask_frac=0.1)
    q, k, v, m = wl.make_inputs(w, DEV)
    o1, l1 = mfa.fwd(q, k, v, causal=True, key_mask=m)
    nbytes = mfa.workspace_size(w.B, w.Lq, w.Lk, w.Hq, w.Hkv, w.D, q.dtype)
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=DEV)
    o2, l2 = mfa.fwd(q, k, v, causal=True, key_mask=m, workspace=ws[:nbytes] if nbytes else ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_pool_calls_leave_the_default_pool_alone():
    """Workspace from the library's own pool: the device's default pool keeps
    its release threshold, and repeated pool calls give the same result."""
    import ctypes
    from transformer_mfa_fwd_amd import _binding
    hip = _binding.load_library()     # symbols resolve in libmfa's own HIP runtime
    release_threshold = 0x4   # hipMemPoolAttrReleaseThreshold
    dev = torch.cuda.current_device()

    def default_threshold():
        pool, thr = ctypes.c_void_p(), ctypes.c_uint64()
        assert hip.hipDeviceGetDefaultMemPool(ctypes.byref(pool), dev) == 0
        assert hip.hipMemPoolGetAttribute(pool, release_threshold, ctypes.byref(thr)) == 0
        return thr.value

    before = default_threshold()
    w = wl.Workload("pool", "bf16", 2, 1, 700, 8, 2, 128, True, mask="random_frac", mask_frac=0.1)
    q, k, v, m = wl.make_inputs(w, DEV)
    o1, l1 = mfa.fwd(q, k, v, causal=True, key_mask=m)      # key mask words + split decode partials
    o2, l2 = mfa.fwd(q, k, v, causal=True, key_mask=m)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert default_threshold() == before


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B,L,Hq,Hkv,wg64", [(2, 512, 8, 2, 128), (2, 1024, 16, 4, 512)],
                         ids=["4_rows_per_wave", "16_rows_per_wave"])
def test_fp32_kernel_grid_forms_sampled_rows(D, B, L, Hq, Hkv, wg64):
    """fp32 inputs take the generic kernel, whose rows per wave follow the
    number of 64-row workgroups (below 64: 1, below 512: 4, else 16; the small
    shapes elsewhere take 1): the 4- and 16-row forms on sampled rows."""
    w = wl.Workload(f"fp32_B{B}_L{L}_H{Hq}_D{D}", "f32", B, L, L, Hq, Hkv, D, True, window=700,
                    mask="random_frac", mask_frac=0.2)
    assert (w.Lq + 63) // 64 * w.Hq * w.B == wg64
    q, k, v, m, out, lse = run_case(w)
    rows = pu.sample_rows(w, n_random=8)
    kw = dict(scale=w.scale, causal=w.causal, window=w.window, q_offset=w.q_offset, softcap=w.softcap)
    O, L_, _ = default_oracle().rows(q, k, v, rows, key_mask=m, nthreads=pu.ORACLE_THREADS, **kw)
    og, lg = pu.gather_rows(out, lse, rows)
    pu.compare(w.dtype, og, lg, O, L_, w.name)


def test_prefill_repeatable_with_three_workgroups_per_cu():
    """The D = 64 soft-capped causal prefill runs three workgroups per CU, where
    waves of one workgroup drift furthest apart: repeated calls must agree bit
    for bit and with the oracle (the first loop iteration's copy into the
    stage that the prologue's scores read waits for every wave)."""
    w = wl.Workload("repeat_d64_cap", "bf16", 2, 3392, 4803, 8, 2, 64, True, softcap=6.290779331842202)
    q, k, v, m = wl.make_inputs(w, DEV, seed=1174)
    kw = dict(causal=True, window=0, q_offset=314, softcap=w.softcap, scale=w.scale)
    out0, lse0 = mfa.fwd(q, k, v, **kw)
    for _ in range(24):
        out, lse = mfa.fwd(q, k, v, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out, out0) and torch.equal(lse, lse0)
    rows = pu.sample_rows(w, n_random=8, seed=1174)
    O, L, _ = default_oracle().rows(q, k, v, rows, key_mask=None, nthreads=pu.ORACLE_THREADS, **kw)
    og, lg = pu.gather_rows(out0, lse0, rows)
    pu.compare(w.dtype, og, lg, O, L, w.name)


def test_empty_torch_tensors():
    """Calls whose tensors hold no element, made with torch's empty tensors
    (null data pointers): they succeed, and the backward with no query rows
    still writes zero key gradients; varlen sequences without any key give
    O = 0 and LSE = -inf."""
    bf = torch.bfloat16
    z = lambda *s, dt=bf: torch.zeros(s, dtype=dt, device=DEV)
    out, lse = mfa.fwd(z(0, 16, 4, 64), z(0, 16, 2, 64), z(0, 16, 2, 64), causal=True)
    assert out.shape == (0, 16, 4, 64) and lse.shape == (0, 4, 16)
    out, lse = mfa.fwd(z(2, 0, 4, 64), z(2, 16, 2, 64), z(2, 16, 2, 64), causal=True)
    assert out.shape == (2, 0, 4, 64) and lse.shape == (2, 4, 0)
    q = torch.randn((5, 4, 64), device=DEV).to(bf)
    cq = torch.tensor([0, 2, 5], dtype=torch.int32, device=DEV)
    ck = torch.tensor([0, 0, 0], dtype=torch.int32, device=DEV)
    out, lse = mfa.varlen_fwd(q, z(0, 2, 64), z(0, 2, 64), cq, ck, causal=True)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    out, lse = mfa.packed_qkv_fwd(z(0, 3 * 2 * 64), torch.zeros((0, 2), dtype=torch.int32, device=DEV), 2)
    assert out.numel() == 0
    out, lse = mfa.decode_len(z(0, 1, 8, 128), z(0, 64, 2, 128), z(0, 64, 2, 128),
                              torch.zeros((0,), dtype=torch.int32, device=DEV))
    assert out.numel() == 0
    k = torch.randn((1, 20, 2, 64), device=DEV).to(bf)
    dq, dk, dv = mfa.bwd(z(1, 0, 4, 64), k, k, z(1, 0, 4, 64), z(1, 0, 4, 64),
                         torch.zeros((1, 4, 0), device=DEV), causal=True)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and torch.all(dk == 0) and torch.all(dv == 0)


# --- full-size workloads --------------------------------------------------------

FULL = [wl.SINGLE_HEAD_CAUSAL_FP32, wl.GQA_CAUSAL_PREFILL_BF16, wl.BIDIR_WINDOW_ENCODER_FP16,
        wl.LONG_CACHE_DECODE_BF16, wl.CAUSAL_WINDOW_SOFTCAP_BF16]


def _full_rows(w, m):
    if w.Lq * w.B * w.Hq <= 4096:
        b, h, i = np.meshgrid(np.arange(w.B), np.arange(w.Hq), np.arange(w.Lq), indexing="ij")
        return np.stack([b.ravel(), h.ravel(), i.ravel()], 1)
    rows = pu.sample_rows(w)
    if w.mask == "pad_tail":
        rows = np.concatenate([rows, pu.pad_boundary_rows(m.cpu(), w)])
    return rows


@pytest.mark.parametrize("w", FULL, ids=lambda w: w.name)
def test_full_workload_sampled_rows(w):
    q, k, v, m, out, lse = run_case(w)
    orc = default_oracle()
    kw = dict(scale=w.scale, causal=w.causal, window=w.window, q_offset=w.q_offset, softcap=w.softcap)
    if w.Lq == 1:
        # decode: whole batches through the oracle, a seeded subset of batches
        rng = np.random.default_rng(7)
        bs = sorted({0, w.B - 1} | set(rng.choice(w.B, size=min(w.B, 6), replace=False).tolist()))
        for b in bs:
            rows = np.array([(0, h, 0) for h in range(w.Hq)], np.int64)
            mb = None if m is None else m[b:b + 1]
            O, L, _ = orc.rows(q[b:b + 1], k[b:b + 1], v[b:b + 1], rows, key_mask=mb,
                               nthreads=pu.ORACLE_THREADS, **kw)
            og, lg = pu.gather_rows(out[b:b + 1], lse[b:b + 1], rows)
            pu.compare(w.dtype, og, lg, O, L, f"{w.name} batch {b}")
        return
    rows = _full_rows(w, m)
    say(f"oracle on {len(rows)} rows")
    O, L, _ = orc.rows(q, k, v, rows, key_mask=m, nthreads=pu.ORACLE_THREADS, **kw)
    og, lg = pu.gather_rows(out, lse, rows)
    pu.compare(w.dtype, og, lg, O, L, w.name)


PREFILL_FULL = [wl.GQA_CAUSAL_PREFILL_BF16, wl.BIDIR_WINDOW_ENCODER_FP16, wl.CAUSAL_WINDOW_SOFTCAP_BF16]


@pytest.mark.parametrize("w", PREFILL_FULL, ids=lambda w: w.name)
def test_full_workload_every_row(w):
    """Every query row of every head of the full-size prefill workloads
    against the oracle (one batch at a time), so the short rows at the start
    of causal and windowed axes, where a rounded weight weighs most, are all
    checked."""
    q, k, v, m, out, lse = run_case(w)
    orc = default_oracle()
    kw = dict(scale=w.scale, causal=w.causal, window=w.window, q_offset=w.q_offset, softcap=w.softcap)
    worst = (0.0, 0.0)
    for b in range(w.B):
        h, i = np.meshgrid(np.arange(w.Hq), np.arange(w.Lq), indexing="ij")
        rows = np.stack([np.zeros(h.size, np.int64), h.ravel(), i.ravel()], 1)
        say(f"{w.name} batch {b}: oracle on {len(rows)} rows")
        mb = None if m is None else m[b:b + 1]
        O, L, _ = orc.rows(q[b:b + 1], k[b:b + 1], v[b:b + 1], rows, key_mask=mb, nthreads=pu.ORACLE_THREADS, **kw)
        og, lg = pu.gather_rows(out[b:b + 1], lse[b:b + 1], rows)
        e = pu.compare(w.dtype, og, lg, O, L, f"{w.name} batch {b}")
        worst = (max(worst[0], e[0]), max(worst[1], e[1]))
    say(f"{w.name}: max |O - O_ref| {worst[0]:.3e}, max |LSE - LSE_ref| {worst[1]:.3e}")


@pytest.mark.parametrize("B,splits", [(1, 96), (4, 24)])
def test_long_cache_decode_small_batch_many_splits(B, splits):
    """The default split rule gives small batches of a long cache many splits:
    every head of every batch against the oracle."""
    w = wl.LONG_CACHE_DECODE_BF16.replace(name=f"long_cache_decode_B{B}", B=B)
    assert mfa.plan(w.B, w.Lq, w.Lk, w.Hq, w.Hkv, w.D, w.torch_dtype) == ("split_decode", splits)
    q, k, v, m, out, lse = run_case(w)
    rows = np.array([(b, h, 0) for b in range(B) for h in range(w.Hq)], np.int64)
    O, L, _ = default_oracle().rows(q, k, v, rows, scale=w.scale, causal=True, window=0,
                                    q_offset=w.q_offset, softcap=0.0, key_mask=None,
                                    nthreads=pu.ORACLE_THREADS)
    og, lg = pu.gather_rows(out, lse, rows)
    pu.compare(w.dtype, og, lg, O, L, w.name)


@pytest.mark.parametrize("w", FULL, ids=lambda w: w.name)
def test_full_workload_exact_visible_counts(w):
    """Q = 0: every visible score is 0, so exp(LSE) is the visible-key count."""
    q, k, v, m, out, lse = run_case(w, q_zero=True)
    counts, _ = default_oracle().visible_counts(w.B, w.Lq, w.Lk, causal=w.causal, window=w.window,
                                                q_offset=w.q_offset,
                                                key_mask=None if m is None else m.cpu())
    got = torch.exp(lse.double()).round().to(torch.int64).cpu().numpy()   # [B, Hq, Lq]
    want = np.broadcast_to(counts[:, None, :], got.shape)
    empty = want == 0
    assert np.array_equal(got[~empty], want[~empty])
    assert torch.all(torch.isneginf(lse.cpu()[torch.from_numpy(np.ascontiguousarray(empty))]))


# --- scale <= 0 ----------------------------------------------------------------

@pytest.mark.parametrize("scale", [0.0, -0.125, -0.7])
@pytest.mark.parametrize("path", ["generic", "mfma", "split_decode"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_nonpositive_scale_every_path(scale, path, dtype):
    """A zero or negative scale is used as given: with a causal window and a
    key mask (boundary tiles, masked keys) every path matches the oracle.
    Zero gives uniform weights over the visible keys."""
    if path == "split_decode":
        w = wl.Workload(f"scale{scale}_dec_{dtype}", dtype, 2, 1, 700, 8, 2, 128, True, window=300,
                        mask="random_frac", mask_frac=0.3)
    else:
        w = wl.Workload(f"scale{scale}_{path}_{dtype}", dtype, 2, 150, 200, 4, 2, 64, True, window=70,
                        mask="random_frac", mask_frac=0.3)
    q, k, v, m = wl.make_inputs(w, DEV)
    say(f"{w.name} path={path} scale={scale}")
    out, lse = mfa.fwd(q, k, v, causal=True, window=w.window, key_mask=m, scale=scale, path=PATHS[path])
    torch.cuda.synchronize()
    O, L, _ = default_oracle().full(q, k, v, scale=scale, causal=True, window=w.window, q_offset=w.q_offset,
                                    key_mask=m, nthreads=pu.ORACLE_THREADS)
    pu.compare(w.dtype, out.double().cpu().numpy().transpose(0, 2, 1, 3), lse.double().cpu().numpy(),
               O.transpose(0, 2, 1, 3), L, f"{w.name}/{path}")


@pytest.mark.parametrize("scale", [0.0, -0.2])
def test_nonpositive_scale_with_cap_and_bias(scale):
    """The soft-capped and additive-mask MFMA kernels turn scores into logits
    before masking; a zero or negative scale goes through them as given."""
    w = wl.Workload("scale_cap_bias", "bf16", 1, 128, 128, 2, 1, 128, True, window=50, softcap=4.0)
    q, k, v, _ = wl.make_inputs(w, DEV)
    out, lse = mfa.fwd(q, k, v, causal=True, window=50, softcap=4.0, scale=scale)
    torch.cuda.synchronize()
    O, L, _ = default_oracle().full(q, k, v, scale=scale, causal=True, window=50, q_offset=0, softcap=4.0)
    pu.compare("bf16", out.double().cpu().numpy().transpose(0, 2, 1, 3), lse.double().cpu().numpy(),
               O.transpose(0, 2, 1, 3), L, "cap")
    bias = torch.randn((1, 1, 128, 132), generator=torch.Generator().manual_seed(3))[..., :128].contiguous()
    out, lse = mfa.fwd(q, k, v, causal=True, window=50, scale=scale, bias=bias.to(DEV))
    torch.cuda.synchronize()
    O, L, _ = default_oracle().full(q, k, v, scale=scale, causal=True, window=50, q_offset=0, bias=bias)
    pu.compare("bf16", out.double().cpu().numpy().transpose(0, 2, 1, 3), lse.double().cpu().numpy(),
               O.transpose(0, 2, 1, 3), L, "bias")


# --- bf16 V beyond the fp16 range ------------------------------------------------

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("where", ["first_tile", "middle_tile", "last_tile", "two_tiles"])
def test_bf16_large_v_runs_on_bf16_operands(D, where):
    """bf16 P.V runs on fp16 operands, which cannot hold |v| >= 65504: the
    tile holding such values is noticed when its V rows are converted and the
    row block is computed again on bf16 operands.  Rows that see them are
    checked relative to the largest |V| they see (bf16 weights err by up to
    2^-8 of it), the others against the usual bound."""
    w = wl.Workload(f"bigv_{where}_D{D}", "bf16", 2, 300, 300, 4, 2, D, True)
    q, k, v, _ = wl.make_inputs(w, DEV)
    spans = {"first_tile": [(2, 5)], "middle_tile": [(130, 133)], "last_tile": [(290, 300)],
             "two_tiles": [(70, 72), (200, 201)]}[where]
    v = v.clone()
    for s0, s1 in spans:
        v[:, s0:s1, 0, :] = (v[:, s0:s1, 0, :].float() * 1e6).to(v.dtype)
        v[:, s0, 1, 3] = 1e30
    say(f"{w.name}")
    out, lse = mfa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    O, L, _ = default_oracle().full(q, k, v, scale=w.scale, causal=True, q_offset=0, nthreads=pu.ORACLE_THREADS)
    og = out.double().cpu().numpy()                               # [B, Lq, Hq, D]
    assert np.all(np.isfinite(og))
    vmax = v.double().abs().amax(dim=3).cpu().numpy()             # [B, Lk, Hkv]
    seen = np.maximum.accumulate(vmax, axis=1)                    # causal: row i sees keys 0..i
    g = w.Hq // w.Hkv
    scale = np.maximum(1.0, seen[:, :, np.arange(w.Hq) // g])     # [B, Lq, Hq]
    bound = pu.TOL_O["bf16"] * scale[..., None] + pu.half_ulp(O, "bf16")
    err = np.abs(og - O)
    worst = np.unravel_index(int(np.argmax(err - bound)), err.shape)
    assert np.all(err <= bound), (worst, err[worst], bound[worst])
    assert np.max(np.abs(lse.double().cpu().numpy() - L)) <= pu.TOL_LSE


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("spans", [[(16200, 16203)], [(16500, 16504)], [(40, 41), (16900, 16901)]],
                         ids=["in_first_16k", "past_16k", "both"])
def test_bf16_large_v_long_cache(D, spans):
    """The same with more than 16384 keys per (batch, kv head), where the
    conversion flags of the keys past the first 16384 are looked at only
    after the loop: a block seeing such a tile is computed again on bf16
    operands wherever the tile lies.  Only kv head 0 holds the large values;
    the other head is checked against the usual bound."""
    w = wl.Workload(f"bigv_long_D{D}", "bf16", 1, 100, 17000, 4, 2, D, False)
    q, k, v, _ = wl.make_inputs(w, DEV)
    v = v.clone()
    for s0, s1 in spans:
        v[:, s0:s1, 0, :] = (v[:, s0:s1, 0, :].float() * 1e6).to(v.dtype)
    say(f"{w.name} {spans}")
    out, lse = mfa.fwd(q, k, v, causal=False)
    torch.cuda.synchronize()
    O, L, _ = default_oracle().full(q, k, v, scale=w.scale, causal=False, q_offset=w.q_offset,
                                    nthreads=pu.ORACLE_THREADS)
    og = out.double().cpu().numpy()                               # [B, Lq, Hq, D]
    assert np.all(np.isfinite(og))
    vmax = v.double().abs().amax(dim=(1, 3)).cpu().numpy()        # [B, Hkv]: every row sees every key
    g = w.Hq // w.Hkv
    scale = np.maximum(1.0, vmax[:, np.arange(w.Hq) // g])[:, None, :]   # [B, 1, Hq]
    bound = pu.TOL_O["bf16"] * scale[..., None] + pu.half_ulp(O, "bf16")
    err = np.abs(og - O)
    worst = np.unravel_index(int(np.argmax(err - bound)), err.shape)
    assert np.all(err <= bound), (worst, err[worst], bound[worst])
    assert np.max(np.abs(lse.double().cpu().numpy() - L)) <= pu.TOL_LSE


def test_bf16_prefill_caller_workspace_matches_pool():
    """A bf16 prefill converts V to fp16 in its workspace: the caller-owned
    form (mfa_fwd_ws, sized by mfa_fwd_workspace_size) gives the pool form's
    bits, with and without a key mask."""
    w = wl.Workload("ws_bf16_prefill", "bf16", 2, 300, 333, 8, 2, 128, True, window=200, std=2.0,
                    mask="random_frac", mask_frac=0.2)
    q, k, v, m = wl.make_inputs(w, DEV)
    nbytes = mfa.workspace_size(w.B, w.Lq, w.Lk, w.Hq, w.Hkv, w.D, q.dtype)
    assert nbytes >= w.B * w.Lk * w.Hkv * w.D * 2
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    for mask in (None, m):
        o1, l1 = mfa.fwd(q, k, v, causal=True, window=200, key_mask=mask)
        o2, l2 = mfa.fwd(q, k, v, causal=True, window=200, key_mask=mask, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
