"""GPU parity of the single-query decode over a fixed-capacity cache with a
device key mask (mfa_decode_masked) against the fp64 oracle: every batch of
small shapes (prefix masks, holes, single valid keys, no valid key, windows,
GQA, soft-cap, split counts), bit-identity with the device-length decode on
prefix masks, the long-cache shape on sampled batches and exact counts
through Q = 0, graph capture with the mask rewritten between replays, and
guard bands around the outputs."""
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
    print(f"\n[decode_masked] {msg}", flush=True)
    sys.stdout.flush()


def check(w, mask, out, lse, q, k, v, window, batches=None, what=""):
    """Compare the given batches (all by default) with the oracle."""
    orc = default_oracle()
    bs = range(w.B) if batches is None else batches
    for b in bs:
        O, L, _ = orc.decode_masked(q[b:b + 1], k[b:b + 1], v[b:b + 1], mask[b:b + 1], scale=w.scale,
                                    window=window, softcap=w.softcap, nthreads=pu.ORACLE_THREADS)
        og = out[b:b + 1].double().cpu().numpy().transpose(0, 2, 1, 3)   # [1, Hq, 1, D]
        pu.compare(w.dtype, og, lse[b:b + 1].double().cpu().numpy(), O.transpose(0, 2, 1, 3), L,
                   f"{what} batch {b} valid {int((mask[b] > 0.5).sum())}")


SMALL = []
for dtype in ("f16", "bf16"):
    for D in (64, 128):
        SMALL.append(wl.Workload(f"decmask_{dtype}_D{D}_H8_KV2", dtype, 9, 1, 333, 8, 2, D, True))
SMALL.append(wl.Workload("decmask_g16_bf16_D128_cap", "bf16", 7, 1, 500, 16, 1, 128, True, softcap=5.0,
                         std=2.0))
SMALL.append(wl.Workload("decmask_mha_f16_D64", "f16", 6, 1, 64, 4, 4, 64, True))


@pytest.mark.parametrize("splits", [0, 1, 7])
@pytest.mark.parametrize("window", [0, 1, 37, 1000])
@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_decode_masked_small_every_batch(w, window, splits):
    q, k, v, _ = wl.make_inputs(w, DEV)
    mask = wl.make_cache_masks(w.B, w.Lk, seed=3 + window)
    say(f"{w.name} window={window} splits={splits}")
    out, lse = mfa.decode_masked(q, k, v, mask.to(DEV), window=window, softcap=w.softcap, splits=splits)
    torch.cuda.synchronize()
    check(w, mask, out, lse, q, k, v, window, what=f"{w.name}/w{window}/s{splits}")


@pytest.mark.parametrize("window", [0, 37])
@pytest.mark.parametrize("w", SMALL[:4], ids=lambda w: w.name)
def test_decode_masked_never_reads_unused_rows(w, window):
    """Masked cache rows, and with a window the valid rows before it, hold
    NaN: they are never read, so the results are finite and match the
    oracle (which never touches them), with one and several splits."""
    q, k, v, _ = wl.make_inputs(w, DEV)
    mask = wl.make_cache_masks(w.B, w.Lk, seed=11 + window)
    k, v = k.clone(), v.clone()
    for b in range(w.B):
        valid = torch.nonzero(mask[b] > 0.5).flatten()
        unused = mask[b] <= 0.5
        if window > 0 and valid.numel() > 0:
            unused[:max(0, int(valid[-1]) - window + 1)] = True
        k[b, unused.to(DEV)] = float("nan")
        v[b, unused.to(DEV)] = float("nan")
    for splits in (1, 4):
        say(f"{w.name} window={window} splits={splits} (NaN in unused rows)")
        out, lse = mfa.decode_masked(q, k, v, mask.to(DEV), window=window, softcap=w.softcap, splits=splits)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        check(w, mask, out, lse, q, k, v, window, what=f"{w.name}/w{window}/s{splits}/nan")


@pytest.mark.parametrize("splits", [0, 5])
def test_decode_masked_prefix_bit_identical_to_decode_len(splits):
    """mask = [1] * n + [0] * (Lmax - n) runs the same tiles and arithmetic as
    the device-length decode at d_len = n (R = 1, same split count)."""
    w = wl.Workload("decmask_prefix", "bf16", 6, 1, 700, 8, 2, 128, True)
    q, k, v, _ = wl.make_inputs(w, DEV)
    lens = torch.tensor([1, 2, 63, 64, 350, 700], dtype=torch.int32)
    mask = (torch.arange(w.Lk)[None, :] < lens[:, None]).float()
    o1, l1 = mfa.decode_masked(q, k, v, mask.to(DEV), splits=splits)
    o2, l2 = mfa.decode_len(q, k, v, lens.to(DEV), splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    check(w, mask, o1, l1, q, k, v, 0, what="prefix")


def test_decode_masked_matches_forward_on_valid_prefix_with_window():
    """With a prefix mask and a window, the result equals mfa_fwd over the
    first n keys at q_offset = n - 1 with that window (other kernels and
    splits, so within tolerance)."""
    w = wl.Workload("decmask_vs_fwd", "f16", 4, 1, 900, 8, 4, 64, True)
    q, k, v, _ = wl.make_inputs(w, DEV)
    lens = [5, 100, 513, 900]
    mask = torch.zeros((w.B, w.Lk))
    for b, n in enumerate(lens):
        mask[b, :n] = 1.0
    out, lse = mfa.decode_masked(q, k, v, mask.to(DEV), window=77)
    for b, n in enumerate(lens):
        o2, l2 = mfa.fwd(q[b:b + 1].contiguous(), k[b:b + 1, :n].contiguous(), v[b:b + 1, :n].contiguous(),
                         causal=True, window=77, q_offset=n - 1)
        torch.cuda.synchronize()
        assert (out[b:b + 1].float() - o2.float()).abs().max().item() <= 2e-2
        assert (lse[b:b + 1] - l2).abs().max().item() <= 1e-3


def test_decode_masked_graph_replay_with_new_masks():
    """Captured once with a caller workspace; the mask is rewritten between
    replays (new valid sets, so the query position moves) and every replay
    matches the eager call bit for bit and the oracle within tolerance."""
    w = wl.Workload("decmask_graph", "bf16", 6, 1, 1000, 8, 2, 128, True)
    window = 150
    q, k, v, _ = wl.make_inputs(w, DEV)
    nbytes = mfa.decode_masked_workspace_size(w.B, w.Lk, w.Hq, w.Hkv, w.D, q.dtype)
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    d_mask = torch.zeros((w.B, w.Lk), dtype=torch.float32, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, 1), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):        # warm-up call outside the capture
        mfa.decode_masked(q, k, v, d_mask, window=window, out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mfa.decode_masked(q, k, v, d_mask, window=window, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    for rep, seed in enumerate((5, 6, 7, 8)):
        mask = wl.make_cache_masks(w.B, w.Lk, seed=seed, edges=(rep == 0))
        say(f"replay {rep}")
        d_mask.copy_(mask.to(DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        eo, el = mfa.decode_masked(q, k, v, mask.to(DEV), window=window, workspace=ws)   # eager
        torch.cuda.synchronize()
        assert torch.equal(got_o, eo) and torch.equal(got_l, el), f"replay {rep} differs from eager"
        check(w, mask, got_o, got_l, q, k, v, window, what=f"graph replay {rep}")


def test_decode_masked_no_out_of_bounds_writes_and_deterministic():
    w = wl.Workload("decmask_canary", "f16", 5, 1, 250, 8, 2, 64, True)
    q, k, v, _ = wl.make_inputs(w, DEV)
    mask = wl.make_cache_masks(w.B, w.Lk, seed=9).to(DEV)
    n, nl, guard = q.numel(), w.B * w.Hq, 4096
    res = []
    for rep in range(2):
        obuf = torch.full((n + 2 * guard,), 7.0, dtype=q.dtype, device=DEV)
        lbuf = torch.full((nl + 2 * guard,), 7.0, dtype=torch.float32, device=DEV)
        out = obuf[guard:guard + n].view(q.shape)
        lse = lbuf[guard:guard + nl].view(w.B, w.Hq, 1)
        mfa.decode_masked(q, k, v, mask, window=40, out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.all(obuf[:guard] == 7.0) and torch.all(obuf[-guard:] == 7.0)
        assert torch.all(lbuf[:guard] == 7.0) and torch.all(lbuf[-guard:] == 7.0)
        res.append((out.clone(), lse.clone()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


LONG = wl.LONG_CACHE_DECODE_BF16


@pytest.mark.parametrize("window", [0, 4096])
def test_decode_masked_long_cache_sampled_batches(window):
    w = LONG
    q, k, v, _ = wl.make_inputs(w, DEV)
    mask = wl.make_cache_masks(w.B, w.Lk, seed=11)
    say(f"{w.name} window={window}")
    out, lse = mfa.decode_masked(q, k, v, mask.to(DEV), window=window)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    bs = sorted(set(range(6)) | {w.B - 1} | set(rng.choice(w.B, size=4, replace=False).tolist()))
    check(w, mask, out, lse, q, k, v, window, batches=bs, what=f"long cache w={window}")


@pytest.mark.parametrize("window", [0, 1000])
def test_decode_masked_long_cache_exact_counts(window):
    """Q = 0: exp(LSE) of batch b is its count of kept keys, exactly, on
    every batch of the long-cache shape."""
    w = LONG
    _, k, v, _ = wl.make_inputs(w, DEV)
    q = torch.zeros((w.B, 1, w.Hq, w.D), dtype=k.dtype, device=DEV)
    mask = wl.make_cache_masks(w.B, w.Lk, seed=13)
    out, lse = mfa.decode_masked(q, k, v, mask.to(DEV), window=window)
    torch.cuda.synchronize()
    want = np.zeros(w.B, np.int64)
    for b in range(w.B):
        valid = np.nonzero(mask[b].numpy() > 0.5)[0]
        if valid.size:
            p = valid[-1]
            want[b] = int(np.sum(valid > p - window)) if window > 0 else valid.size
    got = torch.exp(lse[:, :, 0].double()).round().to(torch.int64).cpu().numpy()   # [B, Hq]
    empty = want == 0
    assert np.array_equal(got[~empty], np.broadcast_to(want[~empty, None], got[~empty].shape))
    assert torch.all(torch.isneginf(lse[torch.from_numpy(empty)].cpu()))
    assert torch.all(out[torch.from_numpy(empty)].cpu() == 0)


@pytest.mark.parametrize("splits", [0, 1, 3])
def test_decode_masked_sparse_keys_far_apart(splits):
    """Valid keys thousands of positions apart (runs of empty tiles longer
    than the kernel keeps mask words of at a time), a lone key in a window's
    last tile, and valid keys only past the first 4096: every batch against
    the oracle, with and without a window."""
    w = wl.Workload("decmask_sparse_bf16_D128_cap20000", "bf16", 6, 1, 20000, 8, 2, 128, True)
    q, k, v, _ = wl.make_inputs(w, DEV)
    mask = torch.zeros((w.B, w.Lk), dtype=torch.float32)
    mask[0, [0, 4100, 12345, 19999]] = 1.0
    mask[1, [8191, 8192]] = 1.0
    mask[2, 4096:4160] = 1.0
    mask[3, [5, 17000]] = 1.0
    mask[4, ::4097] = 1.0
    mask[5, 19000:] = 1.0
    for window in (0, 3000):
        say(f"{w.name} splits={splits} window={window}")
        out, lse = mfa.decode_masked(q, k, v, mask.to(DEV), window=window, splits=splits)
        torch.cuda.synchronize()
        check(w, mask, out, lse, q, k, v, window, what=f"{w.name}/s{splits}/w{window}")
