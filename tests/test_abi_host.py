"""C ABI checks that need no GPU: the library loads, exports every function
include/mfa.h declares, and rejects bad arguments on the host before any
device work."""
import ctypes
import os
import re
import subprocess

import pytest

import transformer_mfa_fwd_amd as mfa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mfa.h")

# Distinct, 256-byte aligned fake addresses: never dereferenced, because every
# call below fails validation (or is empty) before any HIP call.
FAKE = [ctypes.c_void_p(0x10000 * (i + 1)) for i in range(8)]


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(mfa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_expected_api():
    names = declared_functions()
    assert set(names) == set(mfa.EXPORTED), names


def test_library_exports_every_declared_symbol():
    lib = mfa.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", mfa.LIB_PATH], capture_output=True, text=True)
    if nm.returncode == 0:
        exported = {line.split()[-1] for line in nm.stdout.splitlines() if line.strip()}
        for name in declared_functions():
            assert name in exported, name


def call(**over):
    lib = mfa.load_library()
    a = dict(q=FAKE[0], k=FAKE[1], v=FAKE[2], out=FAKE[3], lse=FAKE[4], B=2, Lq=16, Lk=16, Hq=4,
             Hkv=2, D=64, scale=0.125, causal=1, window=0, q_offset=0, softcap=0.0, key_mask=None,
             dtype=2)
    a.update(over)
    return lib.mfa_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Lq"], a["Lk"],
                       a["Hq"], a["Hkv"], a["D"], a["scale"], a["causal"], a["window"],
                       a["q_offset"], a["softcap"], a["key_mask"], a["dtype"], None)


INVALID = [
    dict(q=None), dict(k=None), dict(v=None), dict(out=None),
    dict(B=-1), dict(Lq=-1), dict(Lk=0), dict(Hq=0), dict(Hkv=0), dict(D=0),
    dict(Hq=6, Hkv=4), dict(q_offset=-1), dict(Lq=16, Lk=16, q_offset=1), dict(Lq=17, Lk=16),
    dict(scale=float("nan")), dict(scale=float("inf")), dict(softcap=float("inf")),
    dict(softcap=float("nan")), dict(q=ctypes.c_void_p(0x10008)), dict(out=ctypes.c_void_p(0x10004)),
    dict(lse=ctypes.c_void_p(0x10002)), dict(key_mask=ctypes.c_void_p(0x10001)),
]


@pytest.mark.parametrize("over", INVALID, ids=lambda d: ",".join(f"{k}" for k in d))
def test_invalid_arguments_rejected(over):
    st = call(**over)
    assert st == 1, (over, st)
    msg = mfa.load_library().mfa_last_error().decode()
    assert msg


@pytest.mark.parametrize("over", [dict(D=96), dict(D=32), dict(D=256), dict(dtype=7), dict(dtype=-1)])
def test_unsupported_rejected(over):
    assert call(**over) == 2


@pytest.mark.parametrize("over", [dict(B=0), dict(Lq=0)])
def test_empty_call_succeeds_without_work(over):
    assert call(**over) == 0


def test_status_strings():
    lib = mfa.load_library()
    for s, text in [(0, "success"), (1, "invalid value"), (2, "not supported"), (3, "HIP error"),
                    (4, "out of memory")]:
        assert lib.mfa_status_string(s).decode() == text
    assert lib.mfa_status_string(99).decode() == "unknown status"


def test_forced_path_rejection():
    lib = mfa.load_library()
    # split decode needs Lq == 1; fp32 cannot take the MFMA path
    st = lib.mfa_fwd_ex(FAKE[0], FAKE[1], FAKE[2], FAKE[3], None, 1, 4, 16, 2, 1, 64, 0.125, 1, 0, 12,
                        0.0, None, 2, mfa.PATH_SPLIT_DECODE, 0, None, 0, None)
    assert st == 2
    st = lib.mfa_fwd_ex(FAKE[0], FAKE[1], FAKE[2], FAKE[3], None, 1, 4, 16, 2, 1, 64, 0.125, 1, 0, 12,
                        0.0, None, 0, mfa.PATH_MFMA, 0, None, 0, None)
    assert st == 2
    st = lib.mfa_fwd_ex(FAKE[0], FAKE[1], FAKE[2], FAKE[3], None, 1, 4, 16, 2, 1, 64, 0.125, 1, 0, 12,
                        0.0, None, 2, 9, 0, None, 0, None)
    assert st == 2


def test_workspace_size_and_plan():
    import torch
    # a bf16 prefill holds the fp16 copy of V
    bf = mfa.workspace_size(4, 2048, 2048, 32, 8, 128, torch.bfloat16)
    f16 = mfa.workspace_size(4, 2048, 2048, 32, 8, 128, torch.float16)   # key-mask words only
    assert f16 >= 4 * 32 * 8 and bf - f16 >= 4 * 2048 * 8 * 128 * 2
    path, splits = mfa.plan(64, 1, 32768, 32, 8, 128, torch.bfloat16)
    assert path in ("split_decode", "generic", "mfma")
    p32, _ = mfa.plan(1, 128, 128, 1, 1, 64, torch.float32)
    assert p32 == "generic"


def test_bf16_prefill_without_workspace_rejected_by_ws_form():
    lib = mfa.load_library()
    st = lib.mfa_fwd_ws(FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], 2, 16, 16, 4, 2, 64, 0.125, 1, 0, 0, 0.0,
                        None, 2, None, 0, None)
    assert st == 1 and "workspace" in lib.mfa_last_error().decode()
    # fp16 needs none
    st = lib.mfa_fwd_ws(FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], 0, 16, 16, 4, 2, 64, 0.125, 1, 0, 0, 0.0,
                        None, 1, None, 0, None)
    assert st == 0


def call_len(**over):
    lib = mfa.load_library()
    a = dict(q=FAKE[0], k=FAKE[1], v=FAKE[2], out=FAKE[3], lse=FAKE[4], d_len=FAKE[5], B=2, R=2,
             Lmax=64, Hq=8, Hkv=2, D=128, scale=0.1, softcap=0.0, dtype=2, splits=0,
             ws=None, ws_bytes=0)
    a.update(over)
    return lib.mfa_decode_len(a["q"], a["k"], a["v"], a["out"], a["lse"], a["d_len"], a["B"],
                              a["R"], a["Lmax"], a["Hq"], a["Hkv"], a["D"], a["scale"],
                              a["softcap"], a["dtype"], a["splits"], a["ws"], a["ws_bytes"], None)


LEN_INVALID = [
    dict(q=None), dict(k=None), dict(v=None), dict(out=None), dict(d_len=None),
    dict(B=-1), dict(R=0), dict(Lmax=0), dict(Hq=0), dict(Hkv=0), dict(D=0), dict(Hq=6, Hkv=4),
    dict(scale=float("nan")), dict(softcap=float("inf")),
    dict(q=ctypes.c_void_p(0x10008)), dict(lse=ctypes.c_void_p(0x10002)),
    dict(d_len=ctypes.c_void_p(0x10001)),
    dict(ws=None, ws_bytes=1024), dict(ws=ctypes.c_void_p(0x10010), ws_bytes=1 << 30),
    dict(ws=ctypes.c_void_p(0x10000), ws_bytes=256),
]


@pytest.mark.parametrize("over", LEN_INVALID, ids=lambda d: ",".join(f"{k}" for k in d))
def test_decode_len_invalid_arguments_rejected(over):
    assert call_len(**over) == 1, over
    assert mfa.load_library().mfa_last_error().decode()


@pytest.mark.parametrize("over", [dict(D=96), dict(dtype=0), dict(dtype=5), dict(R=5, Hq=8, Hkv=2),
                                  dict(R=2, Hq=32, Hkv=2)])
def test_decode_len_unsupported_rejected(over):
    assert call_len(**over) == 2, over


def test_decode_len_empty_batch_and_workspace_size():
    import torch
    assert call_len(B=0) == 0
    n = mfa.decode_len_workspace_size(64, 4, 32768, 32, 8, 128, torch.bfloat16)
    s = ctypes.c_int(0)
    mfa.load_library().mfa_fwd_plan(64, 1, 32768, 32, 8, 128, 2, ctypes.byref(s))
    # (m, l) and D partial sums for every (batch, row, head, split)
    assert n >= 64 * 4 * 32 * s.value * (128 + 2) * 4
    assert mfa.decode_len_workspace_size(64, 5, 32768, 32, 8, 128, torch.bfloat16) == 0
    assert mfa.decode_len_workspace_size(2, 1, 64, 8, 2, 128, torch.bfloat16, splits=3) >= \
        2 * 8 * 3 * (128 + 2) * 4


def call_len_noalloc(**over):
    lib = mfa.load_library()
    a = dict(q=FAKE[0], k=FAKE[1], v=FAKE[2], out=FAKE[3], lse=FAKE[4], d_len=FAKE[5], B=2, R=2,
             Lmax=64, Hq=8, Hkv=2, D=128, scale=0.1, softcap=0.0, dtype=2, splits=0)
    a.update(over)
    return lib.mfa_decode_len_noalloc(a["q"], a["k"], a["v"], a["out"], a["lse"], a["d_len"], a["B"],
                                      a["R"], a["Lmax"], a["Hq"], a["Hkv"], a["D"], a["scale"],
                                      a["softcap"], a["dtype"], a["splits"], None)


NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024


@pytest.mark.parametrize("over", [o for o in LEN_INVALID if "ws" not in o],
                         ids=lambda d: ",".join(f"{k}" for k in d))
def test_decode_len_noalloc_invalid_arguments_rejected(over):
    assert call_len_noalloc(**over) == 1, over
    assert mfa.load_library().mfa_last_error().decode()


@pytest.mark.parametrize("over", [dict(D=96), dict(dtype=0), dict(R=5, Hq=8, Hkv=2)])
def test_decode_len_noalloc_unsupported_rejected(over):
    assert call_len_noalloc(**over) == 2, over


def test_decode_len_noalloc_scratch_limit():
    """Sizes whose partials exceed the static scratch are rejected before any
    device work; the header states the same limit."""
    import torch
    assert call_len_noalloc(B=0) == 0
    assert re.search(r"#define\s+MFA_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)16 \* 1024 \* 1024\)",
                     open(HEADER).read())
    big = dict(B=64, R=4, Lmax=4096, Hq=32, Hkv=8, D=128, splits=8)
    need = mfa.decode_len_workspace_size(64, 4, 4096, 32, 8, 128, torch.bfloat16, splits=8)
    assert need > NOALLOC_SCRATCH_BYTES
    assert call_len_noalloc(**big) == 1
    msg = mfa.load_library().mfa_last_error().decode()
    assert str(need) in msg and str(NOALLOC_SCRATCH_BYTES) in msg, msg
    # the full device-length decode fits at its chosen split count
    assert mfa.decode_len_workspace_size(64, 4, 32768, 32, 8, 128, torch.bfloat16) <= NOALLOC_SCRATCH_BYTES


def call_masked(**over):
    lib = mfa.load_library()
    a = dict(q=FAKE[0], k=FAKE[1], v=FAKE[2], out=FAKE[3], lse=FAKE[4], d_mask=FAKE[5], B=2, Lmax=64,
             Hq=8, Hkv=2, D=128, scale=0.1, window=0, softcap=0.0, dtype=2, splits=0, ws=None, ws_bytes=0)
    a.update(over)
    return lib.mfa_decode_masked(a["q"], a["k"], a["v"], a["out"], a["lse"], a["d_mask"], a["B"],
                                 a["Lmax"], a["Hq"], a["Hkv"], a["D"], a["scale"], a["window"],
                                 a["softcap"], a["dtype"], a["splits"], a["ws"], a["ws_bytes"], None)


MASKED_INVALID = [
    dict(q=None), dict(k=None), dict(v=None), dict(out=None), dict(d_mask=None),
    dict(B=-1), dict(Lmax=0), dict(Hq=0), dict(Hkv=0), dict(D=0), dict(Hq=6, Hkv=4),
    dict(scale=float("nan")), dict(softcap=float("inf")),
    dict(q=ctypes.c_void_p(0x10008)), dict(lse=ctypes.c_void_p(0x10002)),
    dict(d_mask=ctypes.c_void_p(0x10001)),
    dict(ws=None, ws_bytes=1024), dict(ws=ctypes.c_void_p(0x10010), ws_bytes=1 << 30),
    dict(ws=ctypes.c_void_p(0x10000), ws_bytes=256),
]


@pytest.mark.parametrize("over", MASKED_INVALID, ids=lambda d: ",".join(f"{k}" for k in d))
def test_decode_masked_invalid_arguments_rejected(over):
    assert call_masked(**over) == 1, over
    assert mfa.load_library().mfa_last_error().decode()


@pytest.mark.parametrize("over", [dict(D=96), dict(dtype=0), dict(dtype=5), dict(Hq=32, Hkv=1)])
def test_decode_masked_unsupported_rejected(over):
    assert call_masked(**over) == 2, over


def test_decode_masked_empty_batch_and_workspace_size():
    import torch
    assert call_masked(B=0) == 0
    n = mfa.decode_masked_workspace_size(64, 32768, 32, 8, 128, torch.bfloat16)
    s = ctypes.c_int(0)
    mfa.load_library().mfa_fwd_plan(64, 1, 32768, 32, 8, 128, 2, ctypes.byref(s))
    # packed mask bits, then (m, l) and D partial sums for every (batch, head, split)
    assert n >= 64 * (32768 // 64) * 8 + 64 * 32 * s.value * (128 + 2) * 4
    assert mfa.decode_masked_workspace_size(64, 32768, 32, 1, 128, torch.bfloat16) == 0
    assert mfa.decode_masked_workspace_size(2, 100, 8, 2, 64, torch.float16, splits=3) >= \
        2 * 2 * 8 + 2 * 8 * 3 * (64 + 2) * 4


def call_packed(**over):
    lib = mfa.load_library()
    a = dict(qkv=FAKE[0], sb=FAKE[1], out=FAKE[2], lse=FAKE[3], L=100, H=4, D=64, scale=0.125,
             window=0, softcap=0.0, dtype=2)
    a.update(over)
    return lib.mfa_packed_qkv_fwd(a["qkv"], a["sb"], a["out"], a["lse"], a["L"], a["H"], a["D"],
                                  a["scale"], a["window"], a["softcap"], a["dtype"], None)


@pytest.mark.parametrize("over", [dict(qkv=None), dict(sb=None), dict(out=None), dict(L=-1), dict(H=0),
                                  dict(D=0), dict(scale=float("nan")), dict(softcap=float("inf")),
                                  dict(qkv=ctypes.c_void_p(0x10008)), dict(out=ctypes.c_void_p(0x10004)),
                                  dict(lse=ctypes.c_void_p(0x10002)), dict(sb=ctypes.c_void_p(0x10001))],
                         ids=lambda d: ",".join(d))
def test_packed_invalid_arguments_rejected(over):
    assert call_packed(**over) == 1, over
    assert mfa.load_library().mfa_last_error().decode()


@pytest.mark.parametrize("over", [dict(D=96), dict(D=256), dict(dtype=3)])
def test_packed_unsupported_rejected(over):
    assert call_packed(**over) == 2, over


def test_packed_empty_call_succeeds():
    assert call_packed(L=0) == 0


def call_varlen(**over):
    lib = mfa.load_library()
    a = dict(q=FAKE[0], k=FAKE[1], v=FAKE[2], out=FAKE[3], lse=FAKE[4], cq=FAKE[5], ck=FAKE[6], batch=3,
             Tq=100, Tk=120, Hq=4, Hkv=2, D=128, scale=0.1, causal=1, window=0, softcap=0.0, dtype=2,
             ws=FAKE[7], ws_bytes=1 << 20)
    a.update(over)
    return lib.mfa_varlen_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["cq"], a["ck"], a["batch"],
                              a["Tq"], a["Tk"], a["Hq"], a["Hkv"], a["D"], a["scale"], a["causal"],
                              a["window"], a["softcap"], a["dtype"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("over", [dict(q=None), dict(k=None), dict(v=None), dict(out=None), dict(cq=None),
                                  dict(ck=None), dict(batch=-1), dict(batch=0), dict(Tq=-1), dict(Tk=-1),
                                  dict(Hq=0), dict(Hkv=0), dict(D=0), dict(Hq=6, Hkv=4),
                                  dict(scale=float("nan")), dict(softcap=float("inf")),
                                  dict(q=ctypes.c_void_p(0x10008)), dict(lse=ctypes.c_void_p(0x10002)),
                                  dict(cq=ctypes.c_void_p(0x10001)), dict(ws=None, ws_bytes=64),
                                  dict(ws=ctypes.c_void_p(0x10010)), dict(ws_bytes=16)],
                         ids=lambda d: ",".join(d))
def test_varlen_invalid_arguments_rejected(over):
    assert call_varlen(**over) == 1, over
    assert mfa.load_library().mfa_last_error().decode()


@pytest.mark.parametrize("over", [dict(D=96), dict(dtype=4)])
def test_varlen_unsupported_rejected(over):
    assert call_varlen(**over) == 2, over


def test_varlen_empty_and_workspace_size():
    assert call_varlen(Tq=0) == 0
    assert call_varlen(Tq=0, batch=0) == 0
    import torch
    assert mfa.varlen_workspace_size(0, 100, 2, 64, torch.bfloat16) == 0
    assert mfa.varlen_workspace_size(1000, 100, 2, 64, torch.float16) >= 1000 * 3 * 4
    # bf16 adds the fp16 copy of V: total_k * Hkv * D * 2 bytes
    assert mfa.varlen_workspace_size(1000, 900, 2, 64, torch.bfloat16) >= 1000 * 3 * 4 + 900 * 2 * 64 * 2


def call_bd(**over):
    lib = mfa.load_library()
    a = dict(q=FAKE[0], k=FAKE[1], v=FAKE[2], out=FAKE[3], lse=FAKE[4], B=2, Lq=16, Lk=20, Hq=4, Hkv=2,
             D=64, scale=0.125, causal=1, window=0, q_offset=4, softcap=0.0, key_mask=None, bias=FAKE[5],
             bB=1, bH=4, bQ=16, bK=20, p=0.1, seed=5, dtype=2)
    a.update(over)
    return lib.mfa_fwd_bias_dropout(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Lq"], a["Lk"],
                                    a["Hq"], a["Hkv"], a["D"], a["scale"], a["causal"], a["window"],
                                    a["q_offset"], a["softcap"], a["key_mask"], a["bias"], a["bB"], a["bH"],
                                    a["bQ"], a["bK"], a["p"], a["seed"], a["dtype"], None)


@pytest.mark.parametrize("over", [dict(q=None), dict(bB=3), dict(bH=2), dict(bQ=8), dict(bK=0), dict(p=1.0),
                                  dict(p=-0.1), dict(p=float("nan")), dict(bias=ctypes.c_void_p(0x10002)),
                                  dict(Hq=6, Hkv=4), dict(q_offset=5)],
                         ids=lambda d: ",".join(d))
def test_bias_dropout_invalid_arguments_rejected(over):
    assert call_bd(**over) == 1, over
    assert mfa.load_library().mfa_last_error().decode()


def test_bias_dropout_unsupported_and_empty():
    assert call_bd(D=96) == 2
    assert call_bd(B=0) == 0
    assert call_bd(Lq=0, bQ=1) == 0


def call_bwd(**over):
    lib = mfa.load_library()
    a = dict(q=FAKE[0], k=FAKE[1], v=FAKE[2], out=FAKE[3], dout=FAKE[4], lse=FAKE[5], dq=FAKE[6], dk=FAKE[7],
             dv=ctypes.c_void_p(0x90000), B=2, Lq=16, Lk=20, Hq=4, Hkv=2, D=64, scale=0.1, causal=1, window=0,
             q_offset=4, softcap=0.0, key_mask=None, bias=None, bB=1, bH=1, bQ=1, bK=1, p=0.0, seed=0, dtype=2,
             ws=None, ws_bytes=0)
    a.update(over)
    return lib.mfa_bwd(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"], a["B"],
                       a["Lq"], a["Lk"], a["Hq"], a["Hkv"], a["D"], a["scale"], a["causal"], a["window"],
                       a["q_offset"], a["softcap"], a["key_mask"], a["bias"], a["bB"], a["bH"], a["bQ"], a["bK"],
                       a["p"], a["seed"], a["dtype"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("over", [dict(q=None), dict(out=None), dict(dout=None), dict(lse=None), dict(dq=None),
                                  dict(dk=None), dict(dv=None), dict(dout=ctypes.c_void_p(0x10008)),
                                  dict(dv=ctypes.c_void_p(0x10004)), dict(Hq=6, Hkv=4), dict(q_offset=5),
                                  dict(bias=FAKE[5], bQ=3), dict(p=1.0), dict(ws=None, ws_bytes=8),
                                  dict(ws=ctypes.c_void_p(0x10010), ws_bytes=1 << 20)],
                         ids=lambda d: ",".join(d))
def test_bwd_invalid_arguments_rejected(over):
    assert call_bwd(**over) == 1, over
    assert mfa.load_library().mfa_last_error().decode()


def test_bwd_unsupported_empty_and_workspace():
    assert call_bwd(D=96) == 2
    assert call_bwd(B=0) == 0
    assert mfa.bwd_workspace_size(2, 16, 4) >= 2 * 16 * 4 * 4
    assert mfa.bwd_workspace_size(0, 16, 4) == 0


def test_empty_calls_accept_null_pointers():
    """A tensor that holds no element may come as a null pointer (torch's empty
    tensors do); a tensor that holds elements may not."""
    assert call(B=0, q=None, k=None, v=None, out=None, lse=None) == 0
    assert call(Lq=0, q=None, out=None, lse=None) == 0
    assert call(Lq=0, q=None, out=None, k=None) == 1          # k and v still hold B * Lk rows
    assert call_len(B=0, q=None, k=None, v=None, out=None, lse=None, d_len=None) == 0
    assert call_packed(L=0, qkv=None, sb=None, out=None, lse=None) == 0
    assert call_varlen(Tq=0, q=None, out=None, lse=None) == 0
    assert call_varlen(Tq=0, Tk=0, q=None, out=None, k=None, v=None) == 0
    assert call_varlen(Tq=0, cq=None) == 1                     # the prefix sums always hold an entry
    assert call_bwd(B=0, q=None, k=None, v=None, out=None, dout=None, lse=None, dq=None, dk=None,
                    dv=None) == 0
    assert call_bwd(Lq=0, q_offset=0, q=None, out=None, dout=None, lse=None, dq=None, dk=None) == 1
