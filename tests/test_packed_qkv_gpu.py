"""GPU parity of the packed-QKV bidirectional forward (mfa_packed_qkv_fwd)
against the fp64 oracle: every row of packings with ragged sequence lengths
(single rows, tile-edge lengths, sequences crossing workgroup tiles), with and
without a window, soft-cap, every dtype and head size; the long encoder
packing on sampled sequences and exact counts through Q = 0; a graph replayed
with a different packing of the same L; guard bands around the outputs."""
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
    print(f"\n[packed] {msg}", flush=True)
    sys.stdout.flush()


def ragged_lengths(seed, total_min, kinds=(1, 2, 63, 64, 65, 127, 128, 129, 200, 300)):
    rng = np.random.default_rng(seed)
    out = []
    while sum(out) < total_min:
        out.append(int(rng.choice(kinds)) if rng.random() < 0.6 else int(rng.integers(1, 400)))
    return out


def check(qkv, sb, H, out, lse, dtype, *, scale, window, softcap, what):
    """Every row against the oracle."""
    O, L, _ = default_oracle().packed_qkv(qkv, sb, H, scale=scale, window=window, softcap=softcap,
                                          nthreads=pu.ORACLE_THREADS)
    og = out.double().cpu().numpy().reshape(O.shape)
    pu.compare(dtype, og.transpose(1, 0, 2), lse.double().cpu().numpy(), O.transpose(1, 0, 2), L, what)


CASES = []
for dtype in ("f32", "f16", "bf16"):
    for D in (64, 128):
        for H, window, softcap in ((1, 0, 0.0), (3, 128, 0.0), (2, 37, 5.0)):
            CASES.append((dtype, D, H, window, softcap))


@pytest.mark.parametrize("idx", range(len(CASES)),
                         ids=[f"{c[0]}_D{c[1]}_H{c[2]}_w{c[3]}_cap{c[4]}" for c in CASES])
def test_packed_small_all_rows(idx):
    case = CASES[idx]
    dtype, D, H, window, softcap = case
    lengths = ragged_lengths(100 + idx, 700)
    qkv, sb = wl.make_packed_qkv(lengths, H, D, dtype, DEV, seed=1, std=2.0 if softcap else 1.0)
    say(f"{case} L={qkv.shape[0]} sequences={len(lengths)}")
    scale = 1.0 / np.sqrt(D)
    out, lse = mfa.packed_qkv_fwd(qkv, sb, H, window=window, softcap=softcap)
    torch.cuda.synchronize()
    check(qkv, sb, H, out, lse, dtype, scale=scale, window=window, softcap=softcap, what=str(case))


def test_packed_single_sequence_equals_forward():
    """One sequence covering all rows is the plain bidirectional forward."""
    H, D, L = 4, 64, 300
    qkv, sb = wl.make_packed_qkv([L], H, D, "bf16", DEV, seed=2)
    out, lse = mfa.packed_qkv_fwd(qkv, sb, H, window=128)
    x = qkv.view(1, L, 3, H, D)
    o2, l2 = mfa.fwd(x[:, :, 0].contiguous(), x[:, :, 1].contiguous(), x[:, :, 2].contiguous(),
                     causal=False, window=128)
    torch.cuda.synchronize()
    assert torch.equal(out.view(1, L, H, D), o2) and torch.equal(lse.view(1, H, L), l2)


def test_packed_graph_replay_with_new_packing():
    H, D = 2, 128
    lengths_a = ragged_lengths(5, 900)
    L = sum(lengths_a)
    rng = np.random.default_rng(6)
    cuts = sorted(rng.choice(np.arange(1, L), size=7, replace=False).tolist())
    lengths_b = [b - a for a, b in zip([0] + cuts, cuts + [L])]
    qkv, sb_a = wl.make_packed_qkv(lengths_a, H, D, "f16", DEV, seed=7)
    sb_b = wl.seq_bounds_from_lengths(lengths_b).to(DEV)
    sb = sb_a.clone()
    out = torch.empty((L, H * D), dtype=qkv.dtype, device=DEV)
    lse = torch.empty((H, L), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mfa.packed_qkv_fwd(qkv, sb, H, window=100, out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mfa.packed_qkv_fwd(qkv, sb, H, window=100, out=out, lse=lse)
    torch.cuda.synchronize()
    for rep, bounds in enumerate((sb_b, sb_a, sb_b)):
        sb.copy_(bounds)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eo, el = mfa.packed_qkv_fwd(qkv, bounds, H, window=100)
        torch.cuda.synchronize()
        assert torch.equal(out, eo) and torch.equal(lse, el), f"replay {rep} differs from eager"
        check(qkv, bounds, H, out, lse, "f16", scale=1.0 / np.sqrt(D), window=100, softcap=0.0,
              what=f"graph replay {rep}")


def test_packed_no_out_of_bounds_writes_and_deterministic():
    H, D = 3, 64
    lengths = ragged_lengths(8, 500)
    qkv, sb = wl.make_packed_qkv(lengths, H, D, "bf16", DEV, seed=9)
    L = qkv.shape[0]
    n, nl, guard = L * H * D, H * L, 4096
    res = []
    for rep in range(2):
        obuf = torch.full((n + 2 * guard,), 7.0, dtype=qkv.dtype, device=DEV)
        lbuf = torch.full((nl + 2 * guard,), 7.0, dtype=torch.float32, device=DEV)
        out = obuf[guard:guard + n].view(L, H * D)
        lse = lbuf[guard:guard + nl].view(H, L)
        mfa.packed_qkv_fwd(qkv, sb, H, window=64, out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.all(obuf[:guard] == 7.0) and torch.all(obuf[-guard:] == 7.0)
        assert torch.all(lbuf[:guard] == 7.0) and torch.all(lbuf[-guard:] == 7.0)
        res.append((out.clone(), lse.clone()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


def _encoder():
    w = wl.BIDIR_WINDOW_ENCODER_FP16
    lengths = wl.encoder_packing_lengths(w)
    return w, lengths


def test_packed_encoder_sampled_sequences():
    """The padded encoder workload packed without its padding: first, last and
    seeded sequences, every row of each, against the oracle."""
    w, lengths = _encoder()
    qkv, sb = wl.make_packed_qkv(lengths, w.Hq, w.D, w.dtype, DEV, seed=0)
    say(f"encoder packing L={qkv.shape[0]} lengths={lengths}")
    out, lse = mfa.packed_qkv_fwd(qkv, sb, w.Hq, window=w.window)
    torch.cuda.synchronize()
    starts = np.cumsum([0] + lengths)
    # parts of sequences: first and last 300 rows of sequences 0, 3 and the last
    spans = []
    for i in sorted({0, 3, len(lengths) - 1}):
        s0, s1 = int(starts[i]), int(starts[i + 1])
        spans += [(s0, min(s1, s0 + 300))]
        if s1 - s0 > 600:
            spans += [(s1 - 300, s1)]
    check_spans_windowed(qkv, sb, w, out, lse, spans)


def check_spans_windowed(qkv, sb, w, out, lse, spans):
    """Rows of [s0, s1) whose whole window lies inside the span or its
    sequence edge compared with the oracle run on the span."""
    orc = default_oracle()
    sbc = sb.cpu().numpy()
    half = w.window // 2
    for s0, s1 in spans:
        seq_lo, seq_hi = int(sbc[s0, 0]), int(sbc[s1 - 1, 1])
        lo, hi = max(seq_lo, s0 - half), min(seq_hi, s1 + half)
        sub = torch.from_numpy(np.stack([np.maximum(sbc[lo:hi, 0], lo) - lo,
                                         np.minimum(sbc[lo:hi, 1], hi) - lo], 1).astype(np.int32))
        O, L, _ = orc.packed_qkv(qkv[lo:hi], sub, w.Hq, scale=w.scale, window=w.window,
                                 nthreads=pu.ORACLE_THREADS)
        a, b = s0 - lo, s1 - lo
        og = out[s0:s1].double().cpu().numpy().reshape(s1 - s0, w.Hq, w.D)
        pu.compare(w.dtype, og.transpose(1, 0, 2), lse[:, s0:s1].double().cpu().numpy(),
                   O[a:b].transpose(1, 0, 2), L[:, a:b], f"encoder rows [{s0}, {s1})")


def test_packed_encoder_exact_counts():
    """Q = 0 on the whole encoder packing: exp(LSE) is the exact number of keys
    of the row's sequence inside its window, for every row."""
    w, lengths = _encoder()
    qkv, sb = wl.make_packed_qkv(lengths, w.Hq, w.D, w.dtype, DEV, seed=0)
    qkv.view(qkv.shape[0], 3, -1)[:, 0].zero_()
    out, lse = mfa.packed_qkv_fwd(qkv, sb, w.Hq, window=w.window)
    torch.cuda.synchronize()
    sbc = sb.cpu().numpy().astype(np.int64)
    r = np.arange(qkv.shape[0])
    half = w.window // 2
    want = np.minimum(sbc[:, 1] - 1, r + half) - np.maximum(sbc[:, 0], r - half) + 1
    got = torch.exp(lse.double()).round().to(torch.int64).cpu().numpy()
    assert np.array_equal(got, np.broadcast_to(want, got.shape))


def test_packed_single_row_sequences():
    """Every sequence one row long: each row attends only to itself (O = V)."""
    H, D, L = 2, 128, 300
    qkv, sb = wl.make_packed_qkv([1] * L, H, D, "bf16", DEV, seed=12)
    out, lse = mfa.packed_qkv_fwd(qkv, sb, H)
    torch.cuda.synchronize()
    x = qkv.view(L, 3, H * D)
    assert torch.equal(out, x[:, 2])
    check(qkv, sb, H, out, lse, "bf16", scale=1.0 / np.sqrt(D), window=0, softcap=0.0, what="single rows")


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 64), ("f32", 64)])
def test_packed_hostile_bounds_stay_in_bounds(dtype, D):
    """Bounds that break the rules (negative, past L, reversed, INT_MIN/MAX)
    give unspecified values but every access stays inside the tensors: the
    sequence ends are clamped to [0, L] before any key range is formed.
    Guard bands around the outputs stay untouched; the outputs are finite."""
    H = 2
    lengths = ragged_lengths(4, 300)
    qkv, sb = wl.make_packed_qkv(lengths, H, D, dtype, DEV, seed=4)
    L = qkv.shape[0]
    rng = np.random.default_rng(21)
    hostile = np.array([-2**31, -2**31 + 1, -100000, -65, -1, 0, 1, 63, 64, 65, L - 1, L, L + 1, L + 64,
                        2**31 - 2, 2**31 - 1], dtype=np.int64)
    b = sb.cpu().numpy().astype(np.int64)
    pick = rng.random(b.shape) < 0.5
    b[pick] = rng.choice(hostile, size=int(pick.sum()))
    bounds = torch.from_numpy(b.astype(np.int32)).to(DEV)
    n, nl, guard = L * H * D, H * L, 4096
    obuf = torch.full((n + 2 * guard,), 7.0, dtype=qkv.dtype, device=DEV)
    lbuf = torch.full((nl + 2 * guard,), 7.0, dtype=torch.float32, device=DEV)
    out = obuf[guard:guard + n].view(L, H * D)
    lse = lbuf[guard:guard + nl].view(H, L)
    print(f"\n[packed] hostile bounds {dtype} D{D} L={L}", flush=True)
    for window in (0, 64):
        mfa.packed_qkv_fwd(qkv, bounds, H, window=window, out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.all(obuf[:guard] == 7.0) and torch.all(obuf[-guard:] == 7.0)
        assert torch.all(lbuf[:guard] == 7.0) and torch.all(lbuf[-guard:] == 7.0)
        assert torch.all(torch.isfinite(out.float()))
