"""GPU parity of the decode over a device-held length (mfa_decode_len) against
the fp64 oracle: every row of small shapes, sampled batches of the long-cache
shape, exact visible-key counts through Q = 0, graph capture with the length
rewritten between replays, and guard bands around the outputs."""
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
    print(f"\n[decode_len] {msg}", flush=True)
    sys.stdout.flush()


def check(w, lens, out, lse, q, k, v, batches=None, what=""):
    """Compare the given batches (all by default) with the oracle."""
    orc = default_oracle()
    bs = range(w.B) if batches is None else batches
    for b in bs:
        O, L, _ = orc.decode_len(q[b:b + 1], k[b:b + 1], v[b:b + 1], lens[b:b + 1], scale=w.scale,
                                 softcap=w.softcap, nthreads=pu.ORACLE_THREADS)
        og = out[b:b + 1].double().cpu().numpy().transpose(0, 2, 1, 3)   # [1, Hq, R, D]
        pu.compare(w.dtype, og, lse[b:b + 1].double().cpu().numpy(), O.transpose(0, 2, 1, 3), L,
                   f"{what} batch {b} len {int(lens[b])}")


SMALL = []
for dtype in ("f16", "bf16"):
    for D in (64, 128):
        for R, Hq, Hkv in ((1, 8, 2), (2, 8, 2), (4, 8, 2), (3, 4, 4), (1, 16, 1)):
            SMALL.append(wl.Workload(f"declen_{dtype}_D{D}_R{R}_H{Hq}_KV{Hkv}", dtype, 8, R, 333, Hq, Hkv,
                                     D, True))
SMALL.append(wl.Workload("declen_softcap_bf16_D128_R4", "bf16", 8, 4, 400, 8, 2, 128, True, softcap=5.0,
                         std=2.0))
# all 16 MFMA columns in use: R * Hq/Hkv = 16
SMALL.append(wl.Workload("declen_R2_g8_bf16_D128", "bf16", 6, 2, 300, 16, 2, 128, True))
SMALL.append(wl.Workload("declen_R16_g1_f16_D64", "f16", 6, 16, 300, 4, 4, 64, True))


@pytest.mark.parametrize("splits", [0, 1, 7])
@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_decode_len_small_all_rows(w, splits):
    q, k, v, _ = wl.make_inputs(w, DEV)
    lens = wl.make_cache_lengths(w.B, w.Lk, w.Lq, seed=3)
    say(f"{w.name} splits={splits} lens={lens.tolist()}")
    out, lse = mfa.decode_len(q, k, v, lens.to(DEV), softcap=w.softcap, splits=splits)
    torch.cuda.synchronize()
    check(w, lens, out, lse, q, k, v, what=f"{w.name}/s{splits}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_decode_len_never_reads_past_the_length(dtype, D):
    """Cache rows at and past each batch's length hold NaN (an unwritten
    cache, say): they are never read, so the results are finite and match the
    oracle on the valid prefix, also where the length ends inside a key tile
    and with several splits."""
    w = wl.Workload(f"declen_nan_tail_{dtype}_D{D}", dtype, 6, 4, 300, 8, 2, D, True)
    q, k, v, _ = wl.make_inputs(w, DEV)
    lens = torch.tensor([0, 3, 33, 64, 161, 300], dtype=torch.int32)
    k, v = k.clone(), v.clone()
    for b in range(w.B):
        k[b, int(lens[b]):] = float("nan")
        v[b, int(lens[b]):] = float("nan")
    for splits in (1, 3):
        say(f"{w.name} splits={splits} lens={lens.tolist()}")
        out, lse = mfa.decode_len(q, k, v, lens.to(DEV), splits=splits)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        check(w, lens, out, lse, q, k, v, what=f"{w.name}/s{splits}")


def test_decode_len_matches_forward_on_valid_prefix():
    """Where every row sees a key, decode_len equals mfa_fwd over the first
    len keys with the rows at positions len - R .. len - 1 (other kernels,
    so within tolerance rather than bit for bit)."""
    w = wl.Workload("declen_vs_fwd", "bf16", 4, 4, 600, 8, 2, 128, True)
    q, k, v, _ = wl.make_inputs(w, DEV)
    lens = torch.tensor([4, 65, 333, 600], dtype=torch.int32)
    out, lse = mfa.decode_len(q, k, v, lens.to(DEV))
    for b in range(w.B):
        n = int(lens[b])
        o2, l2 = mfa.fwd(q[b:b + 1].contiguous(), k[b:b + 1, :n].contiguous(), v[b:b + 1, :n].contiguous(),
                         causal=True, q_offset=n - w.Lq)
        torch.cuda.synchronize()
        assert (out[b:b + 1].float() - o2.float()).abs().max().item() <= 2e-2
        assert (lse[b:b + 1] - l2).abs().max().item() <= 1e-3


def test_decode_len_graph_replay_with_new_lengths():
    """Captured once with a caller workspace; the lengths are rewritten
    between replays and every replay matches the eager call bit for bit and
    the oracle within tolerance."""
    w = wl.Workload("declen_graph", "bf16", 6, 2, 1000, 8, 2, 128, True)
    q, k, v, _ = wl.make_inputs(w, DEV)
    nbytes = mfa.decode_len_workspace_size(w.B, w.Lq, w.Lk, w.Hq, w.Hkv, w.D, q.dtype)
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    d_len = torch.zeros(w.B, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Lq), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):        # warm-up call outside the capture
        mfa.decode_len(q, k, v, d_len, out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mfa.decode_len(q, k, v, d_len, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    for rep, seed in enumerate((5, 6, 7, 8)):
        lens = wl.make_cache_lengths(w.B, w.Lk, w.Lq, seed=seed, edges=(rep == 0))
        say(f"replay {rep} lens={lens.tolist()}")
        d_len.copy_(lens.to(DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        eo, el = mfa.decode_len(q, k, v, lens.to(DEV), workspace=ws)   # eager, same kernels
        torch.cuda.synchronize()
        assert torch.equal(got_o, eo) and torch.equal(got_l, el), f"replay {rep} differs from eager"
        check(w, lens, got_o, got_l, q, k, v, what=f"graph replay {rep}")


def test_decode_len_no_out_of_bounds_writes_and_deterministic():
    w = wl.Workload("declen_canary", "f16", 5, 3, 250, 8, 2, 64, True)
    q, k, v, _ = wl.make_inputs(w, DEV)
    lens = wl.make_cache_lengths(w.B, w.Lk, w.Lq, seed=9).to(DEV)
    n, nl, guard = q.numel(), w.B * w.Hq * w.Lq, 4096
    res = []
    for rep in range(2):
        obuf = torch.full((n + 2 * guard,), 7.0, dtype=q.dtype, device=DEV)
        lbuf = torch.full((nl + 2 * guard,), 7.0, dtype=torch.float32, device=DEV)
        out = obuf[guard:guard + n].view(q.shape)
        lse = lbuf[guard:guard + nl].view(w.B, w.Hq, w.Lq)
        mfa.decode_len(q, k, v, lens, out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.all(obuf[:guard] == 7.0) and torch.all(obuf[-guard:] == 7.0)
        assert torch.all(lbuf[:guard] == 7.0) and torch.all(lbuf[-guard:] == 7.0)
        res.append((out.clone(), lse.clone()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


@pytest.mark.parametrize("R", [1, 4])
def test_decode_len_long_cache_sampled_batches(R):
    w = wl.DEVICE_LENGTH_DECODE_BF16.replace(Lq=R)
    q, k, v, _ = wl.make_inputs(w, DEV)
    lens = wl.make_cache_lengths(w.B, w.Lk, R, seed=11)
    say(f"{w.name} R={R}")
    out, lse = mfa.decode_len(q, k, v, lens.to(DEV))
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    bs = sorted(set(range(6)) | {w.B - 1} | set(rng.choice(w.B, size=4, replace=False).tolist()))
    check(w, lens, out, lse, q, k, v, batches=bs, what=f"long cache R={R}")


def test_decode_len_long_cache_exact_counts():
    """Q = 0: exp(LSE) of row r of batch b is len_b - R + 1 + r exactly."""
    w = wl.DEVICE_LENGTH_DECODE_BF16
    _, k, v, _ = wl.make_inputs(w, DEV)
    q = torch.zeros((w.B, w.Lq, w.Hq, w.D), dtype=k.dtype, device=DEV)
    lens = wl.make_cache_lengths(w.B, w.Lk, w.Lq, seed=13)
    out, lse = mfa.decode_len(q, k, v, lens.to(DEV))
    torch.cuda.synchronize()
    want = (lens.to(torch.int64)[:, None] - w.Lq + 1 + torch.arange(w.Lq)[None, :]).clamp(min=0)  # [B, R]
    want = want[:, None, :].expand(w.B, w.Hq, w.Lq).numpy()
    got = torch.exp(lse.double()).round().to(torch.int64).cpu().numpy()
    empty = want == 0
    assert np.array_equal(got[~empty], want[~empty])
    assert torch.all(torch.isneginf(lse.cpu()[torch.from_numpy(np.ascontiguousarray(empty))]))
    assert torch.all(out.cpu().transpose(1, 2)[torch.from_numpy(np.ascontiguousarray(empty))] == 0)
