"""Lookahead decoding step on one AMD MI355X (gfx950).

The computation lives in the HIP library libla.so (C-ABI: include/la.h);
`binding` marshals arguments to it and `runtime` wraps it with torch-owned
device memory and streams.
"""
from . import binding  # noqa: F401

__all__ = ["binding", "runtime"]
