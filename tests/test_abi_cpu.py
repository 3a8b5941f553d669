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
    for d in (64, 128, 256):
        assert check(d=d) == ea.ATTN_OK
    assert check(Hq=8, Hkv=8) == ea.ATTN_OK and check(Hq=8, Hkv=1) == ea.ATTN_OK
    # The largest head the kernel addresses: N * d = 2^30 elements (2 GiB).
    far = 1 << 44
    assert check(B=1, Hq=1, Hkv=1, N=(1 << 30) // 128, q=far, k=2 * far, v=3 * far, o=4 * far,
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
    dict(o=P + 64),                                             # o overlaps q
    dict(o=2 * P + 4096),                                       # o overlaps k
    dict(lse=4 * P + 2),                                        # lse overlaps o
    dict(lse=3 * P),                                            # lse overlaps v
])
def test_invalid_arguments(over):
    assert check(**over) == ea.ATTN_ERR_INVALID_ARG, over


@pytest.mark.parametrize("d", [1, 32, 80, 96, 100, 129, 192, 512])
def test_unsupported_head_dims(d):
    # The pages fall back to unfused attention for other head_dims; the library
    # reports it instead, whatever the pointers.
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
