"""Seeded synthetic inputs for the attention forward workloads.

This module draws random tensors and key masks and nothing else: it holds none
of the attention arithmetic, so both the HIP path and the fp64 oracle can take
their inputs from it.

Recipe (the same for every workload): one torch generator on the target
device, seeded with ``seed``, draws Q, then K, then V as float32 standard
normals times ``std``, each then rounded to nearest-even into the workload's
dtype.  The key mask, when there is one, comes from a separate CPU generator
seeded with ``seed`` so that it is identical on every device.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" | "f16" | "bf16"
    B: int
    Lq: int
    Lk: int
    Hq: int
    Hkv: int
    D: int
    causal: bool
    window: int = 0       # <= 0: no window
    softcap: float = 0.0  # <= 0: off
    mask: Optional[str] = None   # None | "pad_tail" | "random_frac"
    pad_max: int = 0      # pad_tail: per-batch padding drawn from [0, pad_max)
    mask_frac: float = 0.0  # random_frac: floor(frac * Lk) keys zeroed per batch
    std: float = 1.0

    @property
    def q_offset(self) -> int:
        return self.Lk - self.Lq

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def describe(self) -> dict:
        d = dataclasses.asdict(self)
        d["q_offset"] = self.q_offset
        d["scale"] = self.scale
        return d


# The five workloads of the method's feature set, named by what they are.
SINGLE_HEAD_CAUSAL_FP32 = Workload("single_head_causal_fp32_L128_D64", "f32", 1, 128, 128, 1, 1, 64, True)
GQA_CAUSAL_PREFILL_BF16 = Workload("gqa_causal_prefill_bf16_B4_L2048_H32_KV8_D128", "bf16",
                                   4, 2048, 2048, 32, 8, 128, True)
BIDIR_WINDOW_ENCODER_FP16 = Workload("bidir_window128_encoder_fp16_B8_L8192_H12_D64_padmask", "f16",
                                     8, 8192, 8192, 12, 12, 64, False, window=128,
                                     mask="pad_tail", pad_max=2048)
LONG_CACHE_DECODE_BF16 = Workload("long_cache_decode_bf16_B64_Lk32768_H32_KV8_D128", "bf16",
                                  64, 1, 32768, 32, 8, 128, True)
CAUSAL_WINDOW_SOFTCAP_BF16 = Workload("causal_window4096_softcap50_bf16_B2_L16384_H16_KV4_D128_mask5pct",
                                      "bf16", 2, 16384, 16384, 16, 4, 128, True, window=4096,
                                      softcap=50.0, mask="random_frac", mask_frac=0.05, std=2.0)

ALL = [SINGLE_HEAD_CAUSAL_FP32, GQA_CAUSAL_PREFILL_BF16, BIDIR_WINDOW_ENCODER_FP16,
       LONG_CACHE_DECODE_BF16, CAUSAL_WINDOW_SOFTCAP_BF16]
BY_NAME = {w.name: w for w in ALL}

# Decode over a device-held length: Lq is the number R of query rows per batch
# (a block of draft tokens) and Lk the cache capacity.
DEVICE_LENGTH_DECODE_BF16 = Workload("device_length_decode_bf16_B64_R4_cap32768_H32_KV8_D128", "bf16",
                                     64, 4, 32768, 32, 8, 128, True)


def make_key_mask(w: Workload, seed: int = 0) -> Optional[torch.Tensor]:
    """[B, Lk] float32 key mask on the CPU (1 = keep, 0 = drop), or None."""
    if w.mask is None:
        return None
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    m = torch.ones(w.B, w.Lk, dtype=torch.float32)
    if w.mask == "pad_tail":
        pads = torch.randint(0, max(w.pad_max, 1), (w.B,), generator=g)
        for b in range(w.B):
            p = int(pads[b])
            if p > 0:
                m[b, w.Lk - p:] = 0.0
    elif w.mask == "random_frac":
        n = int(math.floor(w.mask_frac * w.Lk))
        for b in range(w.B):
            perm = torch.randperm(w.Lk, generator=g)
            m[b, perm[:n]] = 0.0
    else:
        raise ValueError(f"unknown mask kind {w.mask!r}")
    return m


def make_cache_lengths(B: int, Lmax: int, R: int, seed: int = 0, edges: bool = True,
                       low: int = 0) -> torch.Tensor:
    """[B] int32 valid lengths on the CPU: with ``edges`` the first entries are
    0, 1, R - 1, R, Lmax - 1 and Lmax (as many as fit, duplicates allowed),
    the rest uniform in [low, Lmax] from a CPU generator seeded with ``seed``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    n = torch.randint(low, Lmax + 1, (B,), generator=g, dtype=torch.int64)
    if edges:
        fixed = [0, 1, max(R - 1, 0), R, Lmax - 1, Lmax]
        for i, x in enumerate(fixed[:B]):
            n[i] = min(max(x, 0), Lmax)
    return n.to(torch.int32)


def make_cache_masks(B: int, Lmax: int, seed: int = 0, edges: bool = True) -> torch.Tensor:
    """[B, Lmax] float32 validity masks of a fixed-capacity cache on the CPU
    (1 valid, 0 not): per batch a valid prefix of length uniform in [1, Lmax]
    in which each key is then dropped with a probability uniform in [0, 0.5),
    from a CPU generator seeded with ``seed``.  With ``edges`` the first
    batches get, as many as fit: no valid key, only key 0, only the last key,
    a full cache, a plain prefix of half the capacity, and valid keys spread
    over the whole capacity with the last one valid."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    m = torch.zeros((B, Lmax), dtype=torch.float32)
    n = torch.randint(1, Lmax + 1, (B,), generator=g)
    drop = torch.rand((B,), generator=g) * 0.5
    u = torch.rand((B, Lmax), generator=g)
    for b in range(B):
        m[b, :int(n[b])] = (u[b, :int(n[b])] >= drop[b]).float()
    if edges:
        fixed = []
        z = torch.zeros(Lmax)
        fixed.append(z.clone())                            # no valid key
        t = z.clone(); t[0] = 1.0; fixed.append(t)         # only key 0
        t = z.clone(); t[-1] = 1.0; fixed.append(t)        # only the last key
        fixed.append(torch.ones(Lmax))                     # full
        t = z.clone(); t[:max(1, Lmax // 2)] = 1.0; fixed.append(t)   # half prefix
        t = (u[0] < 0.3).float(); t[-1] = 1.0; fixed.append(t)        # spread, last valid
        for i, x in enumerate(fixed[:B]):
            m[i] = x
    return m


def seq_bounds_from_lengths(lengths) -> torch.Tensor:
    """[L, 2] int32 on the CPU for sequences of the given lengths packed back to
    back: row r of a sequence spanning rows [s, e) holds (s, e)."""
    rows = []
    s = 0
    for n in [int(x) for x in lengths]:
        rows += [(s, s + n)] * n
        s += n
    return torch.tensor(rows, dtype=torch.int32).reshape(-1, 2)


def make_packed_qkv(lengths, H: int, D: int, dtype: str, device="cpu", seed: int = 0, std: float = 1.0):
    """Fused QKV [L, 3*H*D] for sequences of the given lengths (L their sum):
    one generator seeded with ``seed`` on ``device`` draws float32 standard
    normals times ``std``, rounded to nearest-even into ``dtype``; plus the
    [L, 2] int32 sequence bounds on ``device``."""
    L = int(sum(int(x) for x in lengths))
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn((L, 3 * H * D), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(DTYPES[dtype]), seq_bounds_from_lengths(lengths).to(device)


def encoder_packing_lengths(w: Workload, seed: int = 0):
    """Valid lengths of the padded encoder workload w (pad_tail key mask): the
    sequences the packed form carries without their padding."""
    m = make_key_mask(w, seed)
    return [int(x) for x in m.sum(1).to(torch.int64).tolist()]


def make_inputs(w: Workload, device="cpu", seed: int = 0):
    """Q [B,Lq,Hq,D], K and V [B,Lk,Hkv,D] in the workload's dtype on
    ``device``, and the key mask [B,Lk] float32 (or None) on ``device``."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    dt = w.torch_dtype
    out = []
    for shape in ((w.B, w.Lq, w.Hq, w.D), (w.B, w.Lk, w.Hkv, w.D), (w.B, w.Lk, w.Hkv, w.D)):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if w.std != 1.0:
            x.mul_(w.std)
        out.append(x.to(dt))
        del x
    m = make_key_mask(w, seed)
    if m is not None:
        m = m.to(device)
    return out[0], out[1], out[2], m
