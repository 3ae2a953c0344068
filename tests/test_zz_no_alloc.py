"""GPU checks of mfa_decode_len_noalloc, the decode over a device-held length
whose split partials live in the library's static device scratch: two calls
in a row (the second smaller, so the scratch holds the first call's partials
when it starts) give results bit-identical to mfa_decode_len with a
caller-owned workspace and the same split count, and sizes past the scratch
are rejected before anything is written."""
import sys

import pytest
import torch

import transformer_mfa_fwd_amd as mfa
from oracle import default_oracle
from tests import parity_util as pu
from transformer_mfa_fwd_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda"
SCRATCH_BYTES = 16 * 1024 * 1024

# the full device-length decode (8.5 MB of partials at the chosen split count),
# then a smaller call of another dtype and head size with a forced split count
BIG = wl.DEVICE_LENGTH_DECODE_BF16
SMALL = wl.Workload("noalloc_f16_B5_R2_cap700_H8_KV2_D64", "f16", 5, 2, 700, 8, 2, 64, True, softcap=4.0)


def say(msg):
    print(f"\n[noalloc] {msg}", flush=True)
    sys.stdout.flush()


def _case(w, seed):
    q, k, v, _ = wl.make_inputs(w, DEV)
    lens = wl.make_cache_lengths(w.B, w.Lk, w.Lq, seed=seed)
    return q, k, v, lens


def _reference(w, q, k, v, lens, splits):
    """mfa_decode_len with a caller-owned workspace."""
    n = mfa.decode_len_workspace_size(w.B, w.Lq, w.Lk, w.Hq, w.Hkv, w.D, q.dtype, splits=splits)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    return mfa.decode_len(q, k, v, lens.to(DEV), softcap=w.softcap, splits=splits, workspace=ws)


def test_noalloc_two_calls_match_decode_len():
    cases = [(BIG, 21, 0), (SMALL, 22, 3)]
    data, outs = [], []
    for w, seed, splits in cases:
        need = mfa.decode_len_workspace_size(w.B, w.Lq, w.Lk, w.Hq, w.Hkv, w.D,
                                             wl.DTYPES[w.dtype], splits=splits)
        say(f"{w.name}: splits={splits}, {need} bytes of scratch")
        assert 0 < need <= SCRATCH_BYTES
        q, k, v, lens = _case(w, seed)
        data.append((q, k, v, lens))
        outs.append((torch.full_like(q, float("nan")),
                     torch.full((w.B, w.Hq, w.Lq), float("nan"), dtype=torch.float32, device=DEV)))
    torch.cuda.synchronize()
    # the two calls back to back on one stream, nothing in between
    for (w, _, splits), (q, k, v, lens), (out, lse) in zip(cases, data, outs):
        mfa.decode_len_noalloc(q, k, v, lens.to(DEV), out, lse, softcap=w.softcap, splits=splits)
    torch.cuda.synchronize()
    for (w, _, splits), (q, k, v, lens), (out, lse) in zip(cases, data, outs):
        ref_out, ref_lse = _reference(w, q, k, v, lens, splits)
        torch.cuda.synchronize()
        say(f"{w.name}: compare with mfa_decode_len")
        assert torch.equal(out, ref_out), f"{w.name}: out differs from mfa_decode_len"
        assert torch.equal(lse, ref_lse), f"{w.name}: lse differs from mfa_decode_len"
    # the smaller case against the oracle as well, every row
    w = SMALL
    q, k, v, lens = data[1]
    out, lse = outs[1]
    O, L, _ = default_oracle().decode_len(q, k, v, lens, scale=w.scale, softcap=w.softcap,
                                          nthreads=pu.ORACLE_THREADS)
    pu.compare(w.dtype, out.double().cpu().numpy().transpose(0, 2, 1, 3), lse.double().cpu().numpy(),
               O.transpose(0, 2, 1, 3), L, f"{w.name} vs oracle")


def test_noalloc_repeated_calls_deterministic():
    """The same call three times over, with a different call in between,
    gives the same bits each time."""
    w = SMALL
    q, k, v, lens = _case(w, 23)
    d_len = lens.to(DEV)
    runs = []
    for i in range(3):
        out = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.Lq), dtype=torch.float32, device=DEV)
        mfa.decode_len_noalloc(q, k, v, d_len, out, lse, softcap=w.softcap, splits=5)
        if i == 1:
            other = torch.empty_like(q)
            mfa.decode_len_noalloc(q, k, v, d_len, other, None, softcap=0.0, splits=2)
        runs.append((out, lse))
    torch.cuda.synchronize()
    for out, lse in runs[1:]:
        assert torch.equal(out, runs[0][0]) and torch.equal(lse, runs[0][1])


def test_noalloc_rejects_sizes_past_the_scratch():
    w = wl.Workload("noalloc_oversize_bf16_B64_R4_cap4096_H32_KV8_D128", "bf16", 64, 4, 4096, 32, 8, 128, True)
    splits = 8
    need = mfa.decode_len_workspace_size(w.B, w.Lq, w.Lk, w.Hq, w.Hkv, w.D, torch.bfloat16, splits=splits)
    assert need > SCRATCH_BYTES
    q, k, v, lens = _case(w, 24)
    out = torch.full_like(q, 7.0)
    lse = torch.full((w.B, w.Hq, w.Lq), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(mfa.MFAError) as e:
        mfa.decode_len_noalloc(q, k, v, lens.to(DEV), out, lse, splits=splits)
    say(f"rejected: {e.value}")
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all()), "a rejected call wrote its outputs"
