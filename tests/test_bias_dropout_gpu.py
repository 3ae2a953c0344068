"""GPU parity of the additive score mask and attention dropout
(mfa_fwd_bias_dropout, generic and MFMA kernels) against the fp64 oracle on every row:
broadcast bias shapes, dropout probabilities and seeds, together with the
causal/window/key-mask/soft-cap features, every dtype and head size."""
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
    print(f"\n[bias_dropout] {msg}", flush=True)
    sys.stdout.flush()


def bias_tensor(shape, seed, std=1.5, neg_inf_frac=0.0):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g) * std
    if neg_inf_frac > 0:
        x[torch.rand(shape, generator=g) < neg_inf_frac] = -float("inf")
    return x.contiguous()


def run_and_check(w, bias_shape, p, seed, neg_inf_frac=0.0):
    q, k, v, m = wl.make_inputs(w, DEV)
    full = (w.B, w.Hq, w.Lq, w.Lk)
    shape = tuple(full[e] if bias_shape[e] else 1 for e in range(4)) if bias_shape else None
    bias = None if shape is None else bias_tensor(shape, seed=17, neg_inf_frac=neg_inf_frac)
    say(f"{w.name} bias={shape} p={p} seed={seed}")
    out, lse = mfa.fwd(q, k, v, causal=w.causal, window=w.window, q_offset=w.q_offset, softcap=w.softcap,
                       key_mask=m, scale=w.scale, bias=None if bias is None else bias.to(DEV),
                       dropout_p=p, seed=seed)
    torch.cuda.synchronize()
    O, L, _ = default_oracle().full(q, k, v, scale=w.scale, causal=w.causal, window=w.window,
                                    q_offset=w.q_offset, softcap=w.softcap, key_mask=m, bias=bias,
                                    dropout_p=p, seed=seed, nthreads=pu.ORACLE_THREADS)
    og = out.double().cpu().numpy().transpose(0, 2, 1, 3)
    return pu.compare(w.dtype, og, lse.double().cpu().numpy(), O.transpose(0, 2, 1, 3), L,
                      f"{w.name} bias={shape} p={p}", o_scale=1.0 / (1.0 - p))


BASE = []
for dtype in ("f32", "f16", "bf16"):
    for D in (64, 128):
        BASE.append(wl.Workload(f"bd_causal_gqa_{dtype}_D{D}", dtype, 2, 90, 130, 4, 2, D, True, window=60,
                                mask="random_frac", mask_frac=0.2))
        BASE.append(wl.Workload(f"bd_bidir_cap_{dtype}_D{D}", dtype, 2, 70, 70, 2, 2, D, False, softcap=8.0,
                                std=2.0))

SHAPES = [(1, 1, 1, 1), (1, 0, 0, 1), (0, 1, 1, 1), (0, 0, 1, 1), (1, 0, 1, 0)]


@pytest.mark.parametrize("p,seed", [(0.0, 0), (0.1, 7), (0.5, 2**40 + 3)])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "".join(map(str, s)))
@pytest.mark.parametrize("w", BASE, ids=lambda w: w.name)
def test_bias_dropout_all_rows(w, shape, p, seed):
    run_and_check(w, shape, p, seed)


def test_dropout_without_bias_and_neg_inf_bias():
    w = wl.Workload("bd_neginf", "bf16", 2, 64, 64, 2, 1, 128, True)
    run_and_check(w, None, 0.3, 11)
    run_and_check(w, (1, 1, 1, 1), 0.0, 0, neg_inf_frac=0.3)


def test_all_neg_inf_row_is_empty_and_seeds_differ():
    w = wl.Workload("bd_rows", "f16", 1, 40, 40, 2, 2, 64, False)
    q, k, v, _ = wl.make_inputs(w, DEV)
    bias = torch.zeros((1, 1, w.Lq, w.Lk), device=DEV)
    bias[0, 0, 5] = -float("inf")
    out, lse = mfa.fwd(q, k, v, bias=bias)
    torch.cuda.synchronize()
    assert torch.all(out[0, 5] == 0) and torch.all(torch.isneginf(lse[0, :, 5]))
    o1, _ = mfa.fwd(q, k, v, dropout_p=0.5, seed=1)
    o2, _ = mfa.fwd(q, k, v, dropout_p=0.5, seed=1)
    o3, _ = mfa.fwd(q, k, v, dropout_p=0.5, seed=2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and not torch.equal(o1, o3)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_dropout_seed_uses_its_low_32_bits(dtype):
    """Only the seed's low 32 bits drive the pattern (the pages' rule for the
    seed): seeds that differ above them give the same bits, on the MFMA and
    the fp32 kernels and in the backward."""
    w = wl.Workload(f"bd_seed32_{dtype}", dtype, 1, 70, 90, 2, 1, 64, True)
    q, k, v, _ = wl.make_inputs(w, DEV)
    outs = [mfa.fwd(q, k, v, causal=True, dropout_p=0.3, seed=s)[0] for s in (5, 5 + 2**32, 5 + 2**63, 6)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2]) and not torch.equal(outs[0], outs[3])
    g = torch.randn(q.shape, generator=torch.Generator().manual_seed(2)).to(q.dtype).to(DEV)
    out, lse = mfa.fwd(q, k, v, causal=True, dropout_p=0.3, seed=5)
    grads = [mfa.bwd(q, k, v, out, g, lse, causal=True, dropout_p=0.3, seed=s) for s in (5, 5 + 2**32)]
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(*grads))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("with_bias", [False, True])
def test_backward_dropout_pattern_shared_or_not(dtype, with_bias, D):
    """With dropout on the matrix cores the dK/dV kernel may store the pattern
    for the dQ kernel (the pool's workspace, or a caller's with room for it) or
    each kernel evaluates it (a caller workspace of exactly the Delta size):
    the gradients are bitwise the same.  Ragged sizes (Lk not a multiple of 16
    or of the D keys of a dK/dV workgroup, several query heads per kv head)."""
    w = wl.Workload(f"bd_share_{dtype}_d{D}", dtype, 2, 150, 203, 4, 2, D, True, window=120)
    q, k, v, _ = wl.make_inputs(w, DEV)
    bias = bias_tensor((1, 1, w.Lq, w.Lk), seed=3).to(DEV) if with_bias else None
    say(f"{w.name} bias={with_bias} shared vs evaluated dropout pattern")
    out, lse = mfa.fwd(q, k, v, causal=True, window=120, bias=bias, dropout_p=0.25, seed=11)
    g = torch.randn(q.shape, generator=torch.Generator().manual_seed(4)).to(q.dtype).to(DEV)
    need = mfa.bwd_workspace_size(w.B, w.Lq, w.Hq)
    keep = 2 * w.B * w.Hq * ((w.Lk + 15) // 16) * w.Lq
    kw = dict(causal=True, window=120, bias=bias, dropout_p=0.25, seed=11)
    pooled = mfa.bwd(q, k, v, out, g, lse, **kw)
    small = mfa.bwd(q, k, v, out, g, lse, workspace=torch.empty(need, dtype=torch.uint8, device=DEV), **kw)
    roomy = mfa.bwd(q, k, v, out, g, lse, workspace=torch.empty(need + keep, dtype=torch.uint8, device=DEV), **kw)
    torch.cuda.synchronize()
    for name, x, y, z in zip(("dq", "dk", "dv"), pooled, small, roomy):
        assert torch.equal(x, y) and torch.equal(x, z), name
        assert bool(torch.isfinite(x.float()).all()), name


# Additive masks the MFMA prefill kernel reads itself (no dropout, fp16/bf16,
# key dimension full, Lk a multiple of four): several tiles, ragged tails.
MFMA_BIAS = []
for dtype in ("f16", "bf16"):
    for D in (64, 128):
        MFMA_BIAS.append(wl.Workload(f"bm_causal_gqa_{dtype}_D{D}", dtype, 2, 150, 196, 4, 2, D, True, window=90,
                                     mask="random_frac", mask_frac=0.2))
        # unit-variance inputs: with |V| up to ~8 (std 2) the 16-bit rounding of the
        # weights that multiply V alone approaches the 1e-2 bound
        MFMA_BIAS.append(wl.Workload(f"bm_bidir_cap_{dtype}_D{D}", dtype, 2, 130, 132, 2, 2, D, False, softcap=8.0))


@pytest.mark.parametrize("shape", [(1, 1, 1, 1), (1, 0, 0, 1), (0, 1, 1, 1), (0, 0, 1, 1)],
                         ids=lambda s: "".join(map(str, s)))
@pytest.mark.parametrize("w", MFMA_BIAS, ids=lambda w: w.name)
def test_bias_on_mfma_kernel_all_rows(w, shape):
    run_and_check(w, shape, 0.0, 0)
    if shape == (1, 1, 1, 1):
        run_and_check(w, shape, 0.0, 0, neg_inf_frac=0.3)


def test_bias_mfma_matches_generic_rounding_free_case():
    """An all-zero mask on the MFMA kernel gives mfa_fwd's bits without a mask
    (same kernel arithmetic on the scores, bias added as +0)."""
    w = wl.Workload("bm_zero", "bf16", 2, 256, 256, 4, 2, 128, True)
    q, k, v, _ = wl.make_inputs(w, DEV)
    o1, l1 = mfa.fwd(q, k, v, causal=True)
    o2, l2 = mfa.fwd(q, k, v, causal=True, bias=torch.zeros((1, 1, 256, 256), device=DEV))
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() <= 1e-2
    assert (l1 - l2).abs().max().item() <= 1e-4


# Dropout on the MFMA prefill kernel, alone and with an additive mask it reads
# itself: several tiles and ragged tails, every combination of cap and key
# mask, keep probabilities from high to low.
@pytest.mark.parametrize("p,seed", [(0.1, 5), (0.5, 2**63 + 9), (0.9, 1)])
@pytest.mark.parametrize("shape", [None, (1, 1, 1, 1), (0, 1, 1, 1)], ids=lambda s: "nobias" if s is None else "".join(map(str, s)))
@pytest.mark.parametrize("w", MFMA_BIAS, ids=lambda w: w.name)
def test_dropout_on_mfma_kernel_all_rows(w, shape, p, seed):
    run_and_check(w, shape, p, seed)


def test_dropout_mfma_keep_rate_and_row_sums():
    """One head of 1024 rows and keys: V = 1 makes every output element the
    kept weights' sum times 1 / (1 - p); its mean over rows is near 1 and the
    LSE is the undropped call's."""
    w = wl.Workload("bm_rate", "bf16", 1, 1024, 1024, 1, 1, 128, False)
    q, k, _, _ = wl.make_inputs(w, DEV)
    v = torch.ones_like(k)
    o0, l0 = mfa.fwd(q, k, v)
    o1, l1 = mfa.fwd(q, k, v, dropout_p=0.25, seed=3)
    torch.cuda.synchronize()
    assert (l0 - l1).abs().max().item() <= 1e-5
    assert (o0.float() - 1).abs().max().item() <= 1e-2
    mean = o1.float()[0, :, 0, 0].mean().item()
    assert abs(mean - 1.0) < 0.02, mean
