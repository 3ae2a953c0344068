"""GPU parity of the varlen forward (mfa_varlen_fwd: separate query and key
packings with prefix sums) against the fp64 oracle: every row of ragged
packings (query longer or shorter than keys, empty sequences, sequences
straddling workgroup tiles), causal and bidirectional, windows, GQA, every
dtype and head size; equal-length packings against the batched forward and
the fused-QKV form bit for bit; a graph replayed with new prefix sums; guard
bands around the outputs."""
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
    print(f"\n[varlen] {msg}", flush=True)
    sys.stdout.flush()


def ragged(seed, n, equal=False):
    rng = np.random.default_rng(seed)
    kinds = [0, 1, 2, 63, 64, 65, 127, 128, 129, 200, 333]
    lq = [int(rng.choice(kinds)) if rng.random() < 0.6 else int(rng.integers(1, 400)) for _ in range(n)]
    if equal:
        return lq, list(lq)
    lk = [max(0, x + int(rng.integers(-70, 70))) if rng.random() < 0.7 else int(rng.choice(kinds))
          for x in lq]
    return lq, lk


def cu(lengths):
    return torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)


def make(lq, lk, Hq, Hkv, D, dtype, seed=0, std=1.0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    dt = wl.DTYPES[dtype]
    Tq, Tk = sum(lq), sum(lk)
    q = (torch.randn((Tq, Hq, D), generator=g, device=DEV) * std).to(dt)
    k = (torch.randn((max(Tk, 1), Hkv, D), generator=g, device=DEV) * std).to(dt)[:Tk].contiguous()
    v = torch.randn((max(Tk, 1), Hkv, D), generator=g, device=DEV).to(dt)[:Tk].contiguous()
    return q, k, v


def check(q, k, v, cq, ck, out, lse, dtype, *, causal, window, softcap, what):
    D = q.shape[-1]
    O, L, _ = default_oracle().varlen(q, k, v, cq, ck, scale=1.0 / np.sqrt(D), causal=causal, window=window,
                                      softcap=softcap, nthreads=pu.ORACLE_THREADS)
    og = out.double().cpu().numpy()
    pu.compare(dtype, og.transpose(1, 0, 2), lse.double().cpu().numpy(), O.transpose(1, 0, 2), L, what)


CASES = []
for dtype in ("f32", "f16", "bf16"):
    for D in (64, 128):
        for Hq, Hkv, causal, window, softcap in ((4, 2, True, 0, 0.0), (2, 2, False, 0, 0.0),
                                                 (4, 1, True, 50, 0.0), (3, 3, False, 90, 4.0)):
            CASES.append((dtype, D, Hq, Hkv, causal, window, softcap))


@pytest.mark.parametrize("idx", range(len(CASES)),
                         ids=[f"{c[0]}_D{c[1]}_H{c[2]}x{c[3]}_{'c' if c[4] else 'b'}_w{c[5]}_cap{c[6]}"
                              for c in CASES])
def test_varlen_small_all_rows(idx):
    dtype, D, Hq, Hkv, causal, window, softcap = CASES[idx]
    lq, lk = ragged(200 + idx, 7)
    q, k, v = make(lq, lk, Hq, Hkv, D, dtype, seed=idx, std=2.0 if softcap else 1.0)
    cq, ck = cu(lq), cu(lk)
    say(f"{CASES[idx]} lq={lq} lk={lk}")
    out, lse = mfa.varlen_fwd(q, k, v, cq.to(DEV), ck.to(DEV), causal=causal, window=window, softcap=softcap)
    torch.cuda.synchronize()
    check(q, k, v, cq, ck, out, lse, dtype, causal=causal, window=window, softcap=softcap, what=str(CASES[idx]))


def test_varlen_equal_lengths_equals_batched_forward():
    """Four sequences of 2048 (the causal GQA prefill shape) give the batched
    forward's bits: same tiles, same arithmetic."""
    w = wl.GQA_CAUSAL_PREFILL_BF16
    q, k, v, _ = wl.make_inputs(w, DEV)
    o1, l1 = mfa.fwd(q, k, v, causal=True)
    c = cu([w.Lq] * w.B).to(DEV)
    o2, l2 = mfa.varlen_fwd(q.view(-1, w.Hq, w.D), k.view(-1, w.Hkv, w.D), v.view(-1, w.Hkv, w.D), c, c,
                            causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(-1, w.Hq, w.D), o2)
    assert torch.equal(l1.permute(1, 0, 2).reshape(w.Hq, -1), l2)


def test_varlen_equals_fused_qkv_form():
    """Same sequences for queries and keys, bidirectional with a window: the
    separate-tensor form gives the fused-QKV form's bits."""
    H, D = 3, 64
    lq, _ = ragged(7, 9, equal=True)
    qkv, sb = wl.make_packed_qkv(lq, H, D, "f16", DEV, seed=3)
    x = qkv.view(-1, 3, H, D)
    o1, l1 = mfa.packed_qkv_fwd(qkv, sb, H, window=70)
    c = cu(lq).to(DEV)
    o2, l2 = mfa.varlen_fwd(x[:, 0].contiguous(), x[:, 1].contiguous(), x[:, 2].contiguous(), c, c,
                            window=70)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(-1, H, D), o2) and torch.equal(l1, l2)


def test_varlen_graph_replay_with_new_lengths():
    Hq, Hkv, D = 4, 2, 128
    lq_a, lk_a = ragged(11, 6)
    Tq, Tk = sum(lq_a), sum(lk_a)
    rng = np.random.default_rng(12)

    def split(total, n):
        cuts = sorted(rng.choice(np.arange(0, total + 1), size=n - 1).tolist())
        return [b - a for a, b in zip([0] + cuts, cuts + [total])]

    lq_b, lk_b = split(Tq, 6), split(Tk, 6)
    q, k, v = make(lq_a, lk_a, Hq, Hkv, D, "bf16", seed=13)
    cq, ck = cu(lq_a).to(DEV), cu(lk_a).to(DEV)
    ws = torch.empty(mfa.varlen_workspace_size(Tq, Tk, Hkv, D, q.dtype), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty((Hq, Tq), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mfa.varlen_fwd(q, k, v, cq, ck, causal=True, out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mfa.varlen_fwd(q, k, v, cq, ck, causal=True, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    for rep, (a, b) in enumerate(((lq_b, lk_b), (lq_a, lk_a), (lq_b, lk_b))):
        cq.copy_(cu(a).to(DEV))
        ck.copy_(cu(b).to(DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eo, el = mfa.varlen_fwd(q, k, v, cu(a).to(DEV), cu(b).to(DEV), causal=True, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, eo) and torch.equal(lse, el), f"replay {rep} differs from eager"
        check(q, k, v, cu(a), cu(b), out, lse, "bf16", causal=True, window=0, softcap=0.0,
              what=f"graph replay {rep}")


def test_varlen_no_out_of_bounds_writes_and_deterministic():
    Hq, Hkv, D = 4, 4, 64
    lq, lk = ragged(21, 5)
    q, k, v = make(lq, lk, Hq, Hkv, D, "f16", seed=22)
    cq, ck = cu(lq).to(DEV), cu(lk).to(DEV)
    n, nl, guard = q.numel(), Hq * q.shape[0], 4096
    res = []
    for rep in range(2):
        obuf = torch.full((n + 2 * guard,), 7.0, dtype=q.dtype, device=DEV)
        lbuf = torch.full((nl + 2 * guard,), 7.0, dtype=torch.float32, device=DEV)
        out = obuf[guard:guard + n].view(q.shape)
        lse = lbuf[guard:guard + nl].view(Hq, -1)
        mfa.varlen_fwd(q, k, v, cq, ck, causal=True, window=40, out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.all(obuf[:guard] == 7.0) and torch.all(obuf[-guard:] == 7.0)
        assert torch.all(lbuf[:guard] == 7.0) and torch.all(lbuf[-guard:] == 7.0)
        res.append((out.clone(), lse.clone()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


def test_varlen_many_tiny_sequences():
    """Hundreds of 0-5 row sequences: every 128-row block straddles dozens of
    them, and some have queries but no keys or keys but no queries."""
    rng = np.random.default_rng(31)
    lq = rng.integers(0, 6, 300).tolist()
    lk = rng.integers(0, 6, 300).tolist()
    for causal, window in ((True, 0), (False, 3)):
        q, k, v = make(lq, lk, 4, 2, 64, "bf16", seed=32)
        cq, ck = cu(lq), cu(lk)
        out, lse = mfa.varlen_fwd(q, k, v, cq.to(DEV), ck.to(DEV), causal=causal, window=window)
        torch.cuda.synchronize()
        check(q, k, v, cq, ck, out, lse, "bf16", causal=causal, window=window, softcap=0.0,
              what=f"tiny sequences causal={causal}")
