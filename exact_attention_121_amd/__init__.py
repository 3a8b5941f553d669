"""Fused exact-attention forward for AMD Instinct MI355X (gfx950).

Placeholder: the Python binding of the C-ABI library is added with the
library itself.
"""
