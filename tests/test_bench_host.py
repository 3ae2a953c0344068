"""Host-side checks of bench.py's work accounting (no GPU)."""
import numpy as np
import pytest

import bench
from oracle import default_oracle
from transformer_mfa_fwd_amd import workloads as wl

SMALL = [
    wl.Workload("c", "bf16", 2, 300, 300, 4, 2, 128, True),
    wl.Workload("cw", "bf16", 2, 300, 300, 4, 2, 128, True, window=77, mask="random_frac", mask_frac=0.2),
    wl.Workload("bw", "f16", 3, 260, 260, 2, 2, 64, False, window=50, mask="pad_tail", pad_max=100),
    wl.Workload("b", "f16", 1, 40, 90, 2, 1, 64, False),
    wl.Workload("dec", "bf16", 4, 1, 700, 8, 2, 128, True, window=100),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_visible_pairs_matches_oracle_count(w):
    m = wl.make_key_mask(w)
    _, total = default_oracle().visible_counts(w.B, w.Lq, w.Lk, causal=w.causal, window=w.window,
                                               q_offset=w.q_offset, key_mask=m)
    assert bench.visible_pairs(w, m) == total * w.Hq


def test_full_workload_pair_counts():
    # closed forms for the unmasked workloads
    w = wl.GQA_CAUSAL_PREFILL_BF16
    assert bench.visible_pairs(w, None) == w.B * w.Hq * w.Lq * (w.Lq + 1) // 2
    w = wl.LONG_CACHE_DECODE_BF16
    assert bench.visible_pairs(w, None) == w.B * w.Hq * w.Lk
    w = wl.SINGLE_HEAD_CAUSAL_FP32
    assert bench.visible_pairs(w, None) == 128 * 129 // 2


def test_refuses_more_than_one_gpu():
    import subprocess, sys, os
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(bench.__file__), "bench.py"),
                        "--gpus", "4"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr
