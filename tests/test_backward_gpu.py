"""GPU parity of the backward (mfa_bwd) against the fp64 oracle's gradients on
every element: causal/bidirectional windows with q_offset, key mask, GQA,
soft-cap, additive mask, dropout, every dtype and head size.  The forward
output and LSE fed to the backward come from libmfa's own forward, as a
caller would use them, so the 16-bit cases also carry the rounding of O."""
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
def say(msg):
    print(f"\n[backward] {msg}", flush=True)
    sys.stdout.flush()


def run_case(w, bias_shape=None, p=0.0, seed=0, nan_masked=False):
    q, k, v, m = wl.make_inputs(w, DEV)
    if nan_masked:
        # masked keys' rows hold NaN: no kernel may let them reach a gradient
        k, v = k.clone(), v.clone()
        k[m <= 0.5] = float("nan")
        v[m <= 0.5] = float("nan")
    g = torch.Generator(device="cpu")
    g.manual_seed(5)
    dout = (torch.randn(q.shape, generator=g)).to(q.dtype).to(DEV)
    full = (w.B, w.Hq, w.Lq, w.Lk)
    bias = None
    if bias_shape is not None:
        shape = tuple(full[e] if bias_shape[e] else 1 for e in range(4))
        bias = (torch.randn(shape, generator=g) * 1.5).contiguous()
    kw = dict(causal=w.causal, window=w.window, q_offset=w.q_offset, softcap=w.softcap, key_mask=m, scale=w.scale)
    say(f"{w.name} bias={bias_shape} p={p}")
    out, lse = mfa.fwd(q, k, v, bias=None if bias is None else bias.to(DEV), dropout_p=p, seed=seed, **kw)
    dq, dk, dv = mfa.bwd(q, k, v, out, dout, lse, bias=None if bias is None else bias.to(DEV), dropout_p=p,
                         seed=seed, **kw)
    torch.cuda.synchronize()
    rq, rk, rv = default_oracle().bwd(q, k, v, dout, bias=bias, dropout_p=p, seed=seed,
                                      nthreads=pu.ORACLE_THREADS, **kw)
    if nan_masked:
        assert torch.isfinite(out).all() and all(torch.isfinite(t).all() for t in (dq, dk, dv))
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        pu.compare_grad(name, got, ref, w.dtype, f"{w.name} bias={bias_shape} p={p}", dropout_p=p)


CASES = []
for dtype in ("f32", "f16", "bf16"):
    for D in (64, 128):
        CASES += [
            wl.Workload(f"bwd_causal_gqa_{dtype}_D{D}", dtype, 2, 100, 100, 4, 2, D, True),
            wl.Workload(f"bwd_win_mask_off_{dtype}_D{D}", dtype, 1, 70, 150, 2, 1, D, True, window=40,
                        mask="random_frac", mask_frac=0.3),
            wl.Workload(f"bwd_bidir_cap_{dtype}_D{D}", dtype, 2, 90, 90, 2, 2, D, False, window=50, softcap=6.0,
                        std=1.5),
        ]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_backward_matches_oracle(w):
    run_case(w)


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 64), ("f16", 128), ("bf16", 128)])
def test_backward_with_bias_and_dropout(dtype, D):
    """fp32 on the fp32 kernels, fp16/bf16 on the matrix cores' mask-and-dropout
    instantiations: several 32-row and 32-key tiles, ragged tails, a window."""
    w = wl.Workload(f"bwd_bias_drop_{dtype}_D{D}", dtype, 2, 80, 96, 4, 2, D, True, window=60)
    run_case(w, bias_shape=(0, 1, 1, 1), p=0.0)
    run_case(w, bias_shape=None, p=0.25, seed=2**35 + 1)
    run_case(w, bias_shape=(1, 0, 1, 0), p=0.5, seed=3)
    if dtype != "f32":
        wc = wl.Workload(f"bwd_bias_drop_cap_mask_{dtype}_D{D}", dtype, 2, 100, 130, 4, 1, D, False, window=70,
                         softcap=6.0, mask="random_frac", mask_frac=0.2)
        run_case(wc, bias_shape=(1, 1, 1, 1), p=0.1, seed=77)
        run_case(wc, bias_shape=(1, 0, 0, 1), p=0.9, seed=5)
        if not (dtype == "bf16" and D == 64):   # that one: test_bf16_cap_mask_delta_from_rounded_o
            run_case(wc, bias_shape=(1, 1, 1, 1), p=0.0)   # cap and mask alone: the unpipelined dQ kernel


@pytest.mark.xfail(strict=True, reason="known: Delta = <dO, O> from the bf16-rounded O the forward hands over "
                                       "moves dQ by 1.8e-2 here, past the 1e-2 bound against the exact gradient")
def test_bf16_cap_mask_delta_from_rounded_o():
    """bf16, D = 64, soft-cap 6, full additive mask, key mask, no dropout:
    dQ differs from the exact gradient by 1.84e-2 at one element (bound
    1.01e-2), the same on every kernel path and with dS carried as two bf16
    operands: the difference comes from Delta, which the backward computes
    from the rounded O it is given (fp16 O, 8x finer, passes)."""
    wc = wl.Workload("bwd_bias_drop_cap_mask_bf16_D64", "bf16", 2, 100, 130, 4, 1, 64, False, window=70,
                     softcap=6.0, mask="random_frac", mask_frac=0.2)
    run_case(wc, bias_shape=(1, 1, 1, 1), p=0.0)


MASKED = [w for w in CASES if w.mask is not None]


@pytest.mark.parametrize("w", MASKED, ids=lambda w: w.name)
def test_backward_masked_rows_may_hold_nan(w):
    """NaN in the K and V rows of masked keys: finite gradients equal to the
    oracle's (which never reads those rows), on every path."""
    run_case(w, nan_masked=True)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_backward_masked_rows_may_hold_nan_with_bias_and_dropout(dtype):
    wc = wl.Workload(f"bwd_nan_rows_extra_{dtype}", dtype, 2, 100, 130, 4, 1, 128, False, window=70,
                     softcap=6.0, mask="random_frac", mask_frac=0.2)
    run_case(wc, bias_shape=(1, 1, 1, 1), p=0.1, seed=77, nan_masked=True)


def test_backward_deterministic_and_zero_for_unseen_keys():
    """Same inputs give the same bits; keys no query sees get zero dK, dV."""
    w = wl.Workload("bwd_det", "bf16", 1, 64, 200, 2, 1, 128, True, window=16)
    q, k, v, _ = wl.make_inputs(w, DEV)
    dout = torch.randn_like(q)
    out, lse = mfa.fwd(q, k, v, causal=True, window=16)
    r1 = mfa.bwd(q, k, v, out, dout, lse, causal=True, window=16)
    r2 = mfa.bwd(q, k, v, out, dout, lse, causal=True, window=16)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    # rows sit at keys 136..199 and each sees 16 keys: keys < 121 are unseen
    assert torch.all(r1[1][:, :121] == 0) and torch.all(r1[2][:, :121] == 0)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 64)])
def test_matrix_core_backward_agrees_with_fp32_kernels(dtype, D):
    """The 16-bit call runs on the matrix cores; the same inputs widened to
    float32 run on the fp32 kernels.  With an all-zero additive mask the call
    takes the mask-and-dropout instantiations and must agree as well."""
    w = wl.Workload(f"bwd_paths_{dtype}", dtype, 2, 300, 300, 8, 2, D, True, window=200)
    q, k, v, _ = wl.make_inputs(w, DEV)
    dout = torch.randn_like(q)
    out, lse = mfa.fwd(q, k, v, causal=True, window=200)
    a = mfa.bwd(q, k, v, out, dout, lse, causal=True, window=200)
    zero = torch.zeros((1, 1, 1, w.Lk), device=DEV)
    z = mfa.bwd(q, k, v, out, dout, lse, causal=True, window=200, bias=zero)
    f = [x.float() for x in (q, k, v, out, dout)]
    g = mfa.bwd(*f, lse, causal=True, window=200)
    torch.cuda.synchronize()
    mant = 7 if dtype == "bf16" else 10   # stored fraction bits of the 16-bit outputs
    for name, x, y, zz in zip(("dq", "dk", "dv"), a, g, z):
        scale = max(1.0, float(y.abs().max()))
        err = float((x.float() - y).abs().max())
        assert err <= 1e-2 * scale, (name, err, scale)
        # the two instantiations may be different kernels that add the same
        # products in another order: each element within one unit in the last
        # place of the 16-bit output, on top of 1e-3 of the tensor's scale
        xf, zf = x.float(), zz.float()
        _, e = torch.frexp(torch.maximum(xf.abs(), zf.abs()))
        ulp = torch.ldexp(torch.ones_like(xf), e - 1 - mant)
        assert bool(((zf - xf).abs() <= 1e-3 * scale + ulp).all()), name
