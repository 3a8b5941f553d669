"""Package-level checks on the CPU: the product path never reaches the
oracle, the offline tile sweep's variant table is well formed, and the
differentiable entry points refuse what the kernels do not compute."""

import ast
import os

import pytest

import exact_attention_121_amd as ea

PKG = os.path.dirname(os.path.abspath(ea.__file__))


def test_package_never_imports_the_oracle():
    for name in sorted(os.listdir(PKG)):
        if not name.endswith(".py"):
            continue
        tree = ast.parse(open(os.path.join(PKG, name)).read())
        for node in ast.walk(tree):
            mods = []
            if isinstance(node, ast.Import):
                mods = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                mods = [node.module or ""]
            for m in mods:
                assert not m.split(".")[0] == "oracle", f"{name} imports {m}"


def test_tile_sweep_table():
    from exact_attention_121_amd import tile_sweep as ts
    for d, variants in ts.VARIANTS.items():
        names = [ts.variant_name(d, v) for v in variants]
        assert len(set(names)) == len(names)
        row_chunks = 8 if d <= 64 else (16 if d <= 128 else 32)  # 16-byte chunks per (padded) LDS row
        for v in variants:
            flags = ts.variant_flags(d, v)   # raises for a query-block count without a hook
            assert f"-DATTN_ONLY_D={d}" in flags
            assert v["BN"] % 32 == 0 and v["BN"] * row_chunks % 256 == 0, "a tile must split evenly over 256 threads"
            assert v["FORM"] in ("", "pp") and (v["FORM"] != "pp" or d == 128)
    assert {c[0] for c in ts.CASES} <= set(ts.VARIANTS)
    for d, causal, N in ts.CASES:
        B, H, n = ts.case_shape(d, causal, N)
        assert n == N and B * H * (-(-N // 256)) >= 256, "every case fills the chip"


def test_tile_sweep_run_needs_the_oracle_check(capsys):
    from exact_attention_121_amd import tile_sweep as ts
    import sys
    argv = sys.argv
    try:
        sys.argv = ["tile_sweep", "run"]
        assert ts.main() == 2
    finally:
        sys.argv = argv
    assert "oracle check" in capsys.readouterr().err


def test_sdpa_refuses_what_the_kernels_do_not_compute():
    """scaled_dot_product_attention refuses masks and dropout before any GPU
    call, and flash_attention, like attn_fwd, refuses host tensors."""
    import torch

    import exact_attention_121_amd as ea

    q = torch.zeros(1, 2, 8, 64, dtype=torch.float16)
    k = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(NotImplementedError):
        ea.scaled_dot_product_attention(q, q, q, attn_mask=torch.ones(8, 8, dtype=torch.bool))
    with pytest.raises(NotImplementedError):
        ea.scaled_dot_product_attention(q, q, q, dropout_p=0.1)
    with pytest.raises(ValueError):
        ea.scaled_dot_product_attention(q, k, k, enable_gqa=False)
    with pytest.raises(ValueError):
        ea.flash_attention(q, q, q)
