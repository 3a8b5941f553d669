"""The C-ABI library on the CPU: it loads, exports what include/*.h declares,
and its host-only validation returns the documented status codes.  No call
here touches a GPU."""

import ctypes
import glob
import os
import re
import subprocess

import pytest

import exact_attention_121_amd as ea
from exact_attention_121_amd.build import LIB_PATH

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(LIB_PATH),
                                reason="libattn_fwd.so not built (run __graft_entry__.build())")


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = re.sub(r"^\s*#.*$", "", text, flags=re.M)  # preprocessor lines (macros, guards)
        for m in re.finditer(r"\b([A-Za-z_]\w*)\s*\(([^;{}]*)\)\s*;", text):
            names.add(m.group(1))
    return names


def test_header_declares_the_boundary():
    assert _declared_functions() == set(ea.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True)
    exported = {line.split()[-1] for line in out.stdout.splitlines() if " T " in line}
    assert _declared_functions() <= exported


def test_status_strings_and_version():
    for st in (ea.ATTN_OK, ea.ATTN_ERR_INVALID_ARG, ea.ATTN_ERR_UNSUPPORTED, ea.ATTN_ERR_DEVICE, 99):
        assert isinstance(ea.attn_status_string(st), str) and ea.attn_status_string(st)
    assert "gfx950" in ea.attn_version()


P = 0x10000000  # fake, never dereferenced, well-separated addresses
GOOD = dict(q=P, k=2 * P, v=3 * P, o=4 * P, lse=5 * P, B=2, Hq=8, Hkv=2, N=100, d=128, scale=0.125)


def check(**over):
    a = dict(GOOD, **over)
    return ea.attn_check_args(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                              a["N"], a["d"], a["scale"])


def test_valid_arguments():
    assert check() == ea.ATTN_OK
    assert check(lse=None) == ea.ATTN_OK
    assert check(scale=0.0) == ea.ATTN_OK and check(scale=-0.5) == ea.ATTN_OK
    for d in (32, 64, 96, 128, 160, 192, 224, 256):
        assert check(d=d) == ea.ATTN_OK
    assert check(Hq=8, Hkv=8) == ea.ATTN_OK and check(Hq=8, Hkv=1) == ea.ATTN_OK
    assert check(q=P + 16, o=4 * P + 48, lse=5 * P + 4) == ea.ATTN_OK   # 16- and 4-byte alignment suffice
    # The largest head the kernel addresses: N * d = 2^30 elements (2 GiB).
    far = 1 << 44
    assert check(B=1, Hq=1, Hkv=1, N=(1 << 30) // 128, q=far, k=2 * far, v=3 * far, o=4 * far,
                 lse=5 * far) == ea.ATTN_OK
    # The largest grid: 2^24 - 1 workgroups of 256 threads.
    assert check(B=(1 << 24) - 1, Hq=1, Hkv=1, N=128, d=64, q=far, k=2 * far, v=3 * far, o=4 * far,
                 lse=5 * far) == ea.ATTN_OK


def test_empty_problems_are_ok_without_pointers():
    assert check(B=0, q=None, k=None, v=None, o=None, lse=None) == ea.ATTN_OK
    assert check(N=0, q=None, k=None, v=None, o=None, lse=None) == ea.ATTN_OK


@pytest.mark.parametrize("over", [
    dict(q=None), dict(k=None), dict(v=None), dict(o=None),
    dict(B=-1), dict(N=-3), dict(Hq=0), dict(Hkv=0), dict(Hq=-8), dict(d=0), dict(d=-64),
    dict(Hq=8, Hkv=3), dict(Hq=2, Hkv=4),
    dict(scale=float("inf")), dict(scale=float("-inf")), dict(scale=float("nan")),
    dict(N=(1 << 30) // 128 + 1), dict(N=1 << 40),             # N * d > 2^30
    dict(B=1 << 20, Hq=1 << 12, Hkv=1, N=128),                  # grid >= 2^31
    dict(B=1 << 12, Hq=1 << 12, Hkv=1, N=128),                  # 2^24 workgroups: 2^32 work-items
    dict(o=P + 64),                                             # o overlaps q
    dict(o=2 * P + 4096),                                       # o overlaps k
    dict(lse=4 * P + 2),                                        # lse overlaps o
    dict(lse=3 * P),                                            # lse overlaps v
    dict(q=P + 2), dict(k=2 * P + 8), dict(v=3 * P + 4), dict(o=4 * P + 1), dict(lse=5 * P + 2),  # alignment
])
def test_invalid_arguments(over):
    assert check(**over) == ea.ATTN_ERR_INVALID_ARG, over


@pytest.mark.parametrize("d", [1, 8, 16, 48, 80, 100, 129, 240, 288, 320, 512])
def test_unsupported_head_dims(d):
    # The pages fall back to unfused attention for head_dims their kernel does
    # not take; this library takes every multiple of 32 up to 256 and reports
    # anything else, whatever the pointers.
    assert check(d=d) == ea.ATTN_ERR_UNSUPPORTED
    assert check(d=d, q=None) == ea.ATTN_ERR_UNSUPPORTED


def test_attn_fwd_rejects_before_touching_the_device():
    lib = ea.load_library()
    # Invalid arguments return before any HIP call, so this is safe without a GPU.
    st = lib.attn_fwd(None, None, None, None, None, 1, 1, 1, 16, 64, 0.125, 0, None)
    assert st == ea.ATTN_ERR_INVALID_ARG
    st = lib.attn_fwd(P, 2 * P, 3 * P, 4 * P, None, 1, 1, 1, 16, 80, 0.125, 0, None)
    assert st == ea.ATTN_ERR_UNSUPPORTED
    st = lib.attn_fwd(None, None, None, None, None, 0, 4, 2, 16, 64, 0.125, 1, None)
    assert st == ea.ATTN_OK


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="AMD GPU"):
        ea.attn_fwd(q, q, q)
    with pytest.raises(TypeError):
        ea.attn_fwd(q.float(), q, q)


# --- decode (KV-cache) entry points -----------------------------------------

DGOOD = dict(q=P, k=2 * P, v=3 * P, o=4 * P, lse=5 * P, B=2, Hq=8, Hkv=2, Nq=4, Nk=1000, d=128, scale=0.125,
             workspace=6 * P, workspace_bytes=None)


def dcheck(**over):
    a = dict(DGOOD, **over)
    if a["workspace_bytes"] is None:
        try:
            a["workspace_bytes"] = ea.attn_decode_workspace_size(a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"],
                                                                 a["d"])
        except ea.AttnError:
            a["workspace_bytes"] = 1 << 40  # invalid shape: the shape check must reject it by itself
    return ea.attn_check_decode_args(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                     a["Nq"], a["Nk"], a["d"], a["scale"], a["workspace"], a["workspace_bytes"])


def _plan(B, Hq, Hkv, Nq, Nk, d):
    """The split plan: 128 packed rows per workgroup, splits aimed at one
    round of resident workgroups (512; 256 with head_dim 256), no empty key
    chunk; the workspace holds a partial O row and LSE per row slot."""
    rows = (Hq // Hkv) * Nq
    row_blocks = -(-rows // 128)
    bn = 32 if d > 128 else 64
    kv_tiles = -(-Nk // bn)
    groups = B * Hkv * row_blocks
    s = max(1, min(kv_tiles, -(-(256 if d == 256 else 512) // groups)))
    chunk = -(-kv_tiles // s)
    splits = -(-kv_tiles // chunk)
    return groups, splits, groups * splits * 128 * (d + 1) * 4


@pytest.mark.parametrize("shape", [
    (1, 1, 1, 1, 1, 64), (1, 32, 8, 1, 8192, 256), (1, 32, 1, 1, 131072, 128), (4, 32, 8, 16, 4096, 128),
    (2, 8, 2, 4, 1000, 64), (1, 64, 1, 16, 300, 128), (64, 32, 32, 1, 2048, 128),
    (1, 8, 2, 1, 5000, 32), (2, 16, 4, 3, 777, 96), (1, 32, 8, 1, 8192, 160), (1, 12, 4, 2, 999, 192),
    (3, 8, 1, 1, 4096, 224),
])
def test_decode_workspace_size(shape):
    groups, splits, nbytes = _plan(*shape)
    assert ea.attn_decode_workspace_size(*shape) == nbytes
    assert 1 <= splits and groups * splits < 2 * 512 + groups


def test_decode_workspace_size_empty_and_invalid():
    assert ea.attn_decode_workspace_size(0, 8, 2, 4, 100, 128) == 0
    assert ea.attn_decode_workspace_size(2, 8, 2, 0, 100, 128) == 0
    with pytest.raises(ea.AttnError):
        ea.attn_decode_workspace_size(2, 8, 2, 5, 4, 128)        # Nq > Nk
    with pytest.raises(ea.AttnError):
        ea.attn_decode_workspace_size(2, 8, 3, 1, 4, 128)        # Hq % Hkv != 0
    with pytest.raises(ea.AttnError):
        ea.attn_decode_workspace_size(2, 8, 2, 1, 4, 80)         # head_dim
    lib = ea.load_library()
    assert lib.attn_decode_workspace_size(1, 1, 1, 1, 1, 64, None) == ea.ATTN_ERR_INVALID_ARG


def test_decode_valid_arguments():
    assert dcheck() == ea.ATTN_OK
    assert dcheck(lse=None) == ea.ATTN_OK
    assert dcheck(Nq=1000) == ea.ATTN_OK                          # Nq == Nk
    assert dcheck(Hkv=1) == ea.ATTN_OK and dcheck(Hkv=8) == ea.ATTN_OK
    assert dcheck(scale=0.0) == ea.ATTN_OK and dcheck(scale=-1.0) == ea.ATTN_OK
    for d in (32, 64, 96, 128, 160, 192, 224, 256):
        assert dcheck(d=d) == ea.ATTN_OK
    assert dcheck(workspace_bytes=1 << 40) == ea.ATTN_OK          # larger than needed is fine
    far = 1 << 44
    assert dcheck(B=1, Hq=1, Hkv=1, Nq=1, Nk=(1 << 30) // 128, q=far, k=2 * far, v=3 * far, o=4 * far,
                  lse=5 * far, workspace=6 * far) == ea.ATTN_OK


def test_decode_empty_problems_are_ok_without_pointers():
    none = dict(q=None, k=None, v=None, o=None, lse=None, workspace=None, workspace_bytes=0)
    assert dcheck(B=0, **none) == ea.ATTN_OK
    assert dcheck(Nq=0, **none) == ea.ATTN_OK


@pytest.mark.parametrize("over", [
    dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(workspace=None),
    dict(B=-1), dict(Nq=-1), dict(Nk=-1), dict(Hq=0), dict(Hkv=0), dict(Hq=8, Hkv=3),
    dict(Nq=1001), dict(Nq=5, Nk=4),                               # more queries than positions
    dict(scale=float("nan")), dict(scale=float("inf")),
    dict(Nk=(1 << 30) // 128 + 1, Nq=1),                           # Nk * d > 2^30
    dict(workspace_bytes=0), dict(workspace_bytes=-5),
    dict(B=1 << 12, Hq=1 << 9, Hkv=1 << 9, Nq=2, Nk=4),              # merge: 2^24 workgroups
    dict(o=P + 64),                                                # o overlaps q
    dict(workspace=2 * P + 4096),                                  # workspace overlaps k
    dict(workspace=4 * P - 64),                                    # workspace overlaps o
    dict(lse=6 * P + 8),                                           # lse overlaps workspace
    dict(lse=4 * P),                                               # lse overlaps o
    dict(q=P + 2), dict(k=2 * P + 8), dict(o=4 * P + 4), dict(lse=5 * P + 2), dict(workspace=6 * P + 4),
])
def test_decode_invalid_arguments(over):
    assert dcheck(**over) == ea.ATTN_ERR_INVALID_ARG, over


def test_decode_short_workspace_is_rejected():
    need = ea.attn_decode_workspace_size(2, 8, 2, 4, 1000, 128)
    assert dcheck(workspace_bytes=need) == ea.ATTN_OK
    assert dcheck(workspace_bytes=need - 1) == ea.ATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("d", [16, 48, 80, 200, 288])
def test_decode_unsupported_head_dims(d):
    assert dcheck(d=d, workspace_bytes=1 << 30) == ea.ATTN_ERR_UNSUPPORTED


def test_attn_decode_rejects_before_touching_the_device():
    lib = ea.load_library()
    st = lib.attn_decode(None, None, None, None, None, 1, 1, 1, 1, 16, 64, 0.125, 1, None, 0, None)
    assert st == ea.ATTN_ERR_INVALID_ARG
    st = lib.attn_decode(P, 2 * P, 3 * P, 4 * P, None, 1, 1, 1, 1, 16, 80, 0.125, 1, 6 * P, 1 << 20, None)
    assert st == ea.ATTN_ERR_UNSUPPORTED
    st = lib.attn_decode(P, 2 * P, 3 * P, 4 * P, None, 1, 1, 1, 1, 16, 64, 0.125, 1, 6 * P, 16, None)
    assert st == ea.ATTN_ERR_INVALID_ARG                           # workspace too small
    st = lib.attn_decode(None, None, None, None, None, 1, 4, 2, 0, 16, 64, 0.125, 1, None, 0, None)
    assert st == ea.ATTN_OK


def test_decode_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 1, 64, dtype=torch.float16)
    k = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="AMD GPU"):
        ea.attn_decode(q, k, k)


# --- backward entry points ---------------------------------------------------

BGOOD = dict(q=P, k=2 * P, v=3 * P, o=4 * P, lse=5 * P, dout=6 * P, dq=7 * P, dk=8 * P, dv=9 * P,
             B=2, Hq=8, Hkv=2, N=1000, d=128, scale=0.125, workspace=10 * P, workspace_bytes=None)


def bcheck(**over):
    a = dict(BGOOD, **over)
    if a["workspace_bytes"] is None:
        try:
            a["workspace_bytes"] = ea.attn_bwd_workspace_size(a["B"], a["Hq"], a["N"], a["d"])
        except ea.AttnError:
            a["workspace_bytes"] = 1 << 40
    return ea.attn_check_bwd_args(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"], a["dk"], a["dv"],
                                  a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["scale"], a["workspace"],
                                  a["workspace_bytes"])


@pytest.mark.parametrize("shape", [(1, 1, 1, 64), (2, 8, 1000, 128), (1, 32, 8192, 256), (3, 5, 129, 64)])
def test_bwd_workspace_size(shape):
    B, Hq, N, d = shape
    npad = -(-N // 128) * 128
    assert ea.attn_bwd_workspace_size(*shape) == 2 * B * Hq * npad * 4


def test_bwd_workspace_size_empty_and_invalid():
    assert ea.attn_bwd_workspace_size(0, 8, 100, 128) == 0
    assert ea.attn_bwd_workspace_size(2, 8, 0, 128) == 0
    with pytest.raises(ea.AttnError):
        ea.attn_bwd_workspace_size(2, 8, 100, 80)
    with pytest.raises(ea.AttnError):
        ea.attn_bwd_workspace_size(-1, 8, 100, 128)
    assert ea.load_library().attn_bwd_workspace_size(1, 1, 1, 64, None) == ea.ATTN_ERR_INVALID_ARG


def test_bwd_valid_arguments():
    assert bcheck() == ea.ATTN_OK
    assert bcheck(scale=0.0) == ea.ATTN_OK and bcheck(scale=-0.3) == ea.ATTN_OK
    for d in (32, 64, 96, 128, 160, 192, 224, 256):
        assert bcheck(d=d) == ea.ATTN_OK
    assert bcheck(Hkv=8) == ea.ATTN_OK and bcheck(Hkv=1) == ea.ATTN_OK
    assert bcheck(workspace_bytes=1 << 40) == ea.ATTN_OK


def test_bwd_empty_problems_are_ok_without_pointers():
    none = dict(q=None, k=None, v=None, o=None, lse=None, dout=None, dq=None, dk=None, dv=None, workspace=None,
                workspace_bytes=0)
    assert bcheck(B=0, **none) == ea.ATTN_OK
    assert bcheck(N=0, **none) == ea.ATTN_OK


@pytest.mark.parametrize("over", [
    dict(q=None), dict(k=None), dict(v=None), dict(o=None), dict(lse=None), dict(dout=None),
    dict(dq=None), dict(dk=None), dict(dv=None), dict(workspace=None),
    dict(B=-1), dict(N=-1), dict(Hq=0), dict(Hkv=0), dict(Hq=8, Hkv=3), dict(scale=float("nan")),
    dict(N=(1 << 30) // 128 + 1),
    dict(workspace_bytes=0),
    dict(dq=P + 16),                        # dq overlaps q
    dict(dk=5 * P),                         # dk overlaps lse
    dict(dv=7 * P + 64),                    # dv overlaps dq
    dict(workspace=9 * P + 4096),           # workspace overlaps dv
    dict(dq=6 * P + 4096),                  # dq overlaps dout
    dict(q=P + 2), dict(dout=6 * P + 8), dict(dk=8 * P + 4), dict(lse=5 * P + 2), dict(workspace=10 * P + 4),
])
def test_bwd_invalid_arguments(over):
    assert bcheck(**over) == ea.ATTN_ERR_INVALID_ARG, over


@pytest.mark.parametrize("d", [16, 48, 80, 200, 288])
def test_bwd_unsupported_head_dims(d):
    assert bcheck(d=d, workspace_bytes=1 << 30) == ea.ATTN_ERR_UNSUPPORTED


def test_bwd_short_workspace_is_rejected():
    need = ea.attn_bwd_workspace_size(2, 8, 1000, 128)
    assert bcheck(workspace_bytes=need) == ea.ATTN_OK
    assert bcheck(workspace_bytes=need - 1) == ea.ATTN_ERR_INVALID_ARG


def test_attn_bwd_rejects_before_touching_the_device():
    lib = ea.load_library()
    nulls = [None] * 9
    assert lib.attn_bwd(*nulls, 1, 1, 1, 16, 64, 0.125, 1, None, 0, None) == ea.ATTN_ERR_INVALID_ARG
    ptrs = [P * (i + 1) for i in range(9)]
    assert lib.attn_bwd(*ptrs, 1, 1, 1, 16, 80, 0.125, 1, 10 * P, 1 << 20, None) == ea.ATTN_ERR_UNSUPPORTED
    assert lib.attn_bwd(*ptrs, 1, 1, 1, 16, 64, 0.125, 1, 10 * P, 8, None) == ea.ATTN_ERR_INVALID_ARG
    assert lib.attn_bwd(*nulls, 0, 4, 2, 16, 64, 0.125, 1, None, 0, None) == ea.ATTN_OK


def test_bwd_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    lse = torch.zeros(1, 1, 8)
    with pytest.raises(ValueError, match="AMD GPU"):
        ea.attn_bwd(x, x, x, x, lse, x)


def test_bwd_accepts_large_head_counts_at_d256():
    """B=1, Hq=64, N=2^21, d=256: 2^27 padded workspace rows and 2^20 dQ
    workgroups are within the kernels' limits (a limit of an earlier
    separate per-row pass, rows / 8 < 2^24, no longer applies); 2^31 rows are
    not."""
    T = 1 << 40  # pointers far enough apart for 2^36-byte tensors
    ptrs = dict(q=T, k=2 * T, v=3 * T, o=4 * T, lse=5 * T, dout=6 * T, dq=7 * T, dk=8 * T, dv=9 * T,
                workspace=10 * T)
    assert bcheck(B=1, Hq=64, Hkv=64, N=1 << 21, d=256, **ptrs) == ea.ATTN_OK
    assert bcheck(B=1, Hq=1024, Hkv=1024, N=1 << 21, d=256, **ptrs) == ea.ATTN_ERR_INVALID_ARG


def test_bwd_noalloc_validates_on_the_host():
    """attn_bwd_noalloc checks its arguments and its scratch limit before it
    touches a device: B * Hq * round_up(N, 128) <= 2^21 rows."""
    lib = ea.load_library()
    T = 1 << 36
    ptrs = [T * i for i in range(1, 10)]  # q, k, v, o, lse, dout, dq, dk, dv
    assert lib.attn_bwd_noalloc(*ptrs, 1, 64, 8, 32768 + 1, 32, 0.125, 0, None) == ea.ATTN_ERR_SCRATCH
    assert lib.attn_bwd_noalloc(*ptrs, 2, 64, 8, 32768, 32, 0.125, 0, None) == ea.ATTN_ERR_SCRATCH
    nulls = [None] * 9
    assert lib.attn_bwd_noalloc(*nulls, 1, 4, 2, 16, 64, 0.125, 1, None) == ea.ATTN_ERR_INVALID_ARG
    assert lib.attn_bwd_noalloc(*ptrs, 1, 4, 2, 16, 80, 0.125, 1, None) == ea.ATTN_ERR_UNSUPPORTED
    assert lib.attn_bwd_noalloc(*ptrs, 1, 4, 3, 16, 64, 0.125, 1, None) == ea.ATTN_ERR_INVALID_ARG
    assert lib.attn_bwd_noalloc(*nulls, 0, 4, 2, 16, 64, 0.125, 1, None) == ea.ATTN_OK
    assert ea.attn_status_string(ea.ATTN_ERR_SCRATCH).startswith("problem too large")
