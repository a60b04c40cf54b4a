"""Torch-side plumbing around libqgemv: device buffers for packed weights and workspaces.

torch only provides device memory and the stream here; every byte of the packed layout is
written by the library's own pack kernel.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _binding as B


def to_device(a, device="cuda") -> torch.Tensor:
    """Host numpy array -> contiguous device tensor (synchronous copy)."""
    a = np.ascontiguousarray(a)
    if not a.flags.writeable:
        a = a.copy()
    return torch.from_numpy(a).to(device)


def pack(fmt: int, w_gguf, N: int, K: int, device="cuda", stream=None,
         codebook=None) -> torch.Tensor:
    """GGUF-native blocks (numpy uint8 [N, row_bytes] or a device tensor) -> packed device buffer.

    codebook: the 16 signed entries of the IQ4 formats (host values), None for the others."""
    src = w_gguf if isinstance(w_gguf, torch.Tensor) else to_device(w_gguf, device)
    nbytes = B.qgemv_packed_bytes(fmt, N, K)
    if nbytes < 0:
        raise ValueError(f"invalid format/shape for packing: fmt={fmt} N={N} K={K}")
    out = torch.empty(nbytes, dtype=torch.uint8, device=src.device)
    if codebook is None:
        B.qgemv_pack(fmt, src, N, K, out, stream=stream)
    else:
        B.qgemv_pack_codebook(fmt, src, N, K, codebook, out, stream=stream)
    return out


def workspace(op: int, fmt: int, N: int, K: int, nb: int, n_exp: int = 0, topk: int = 0,
              device="cuda") -> torch.Tensor | None:
    """Zero-filled workspace of the size the operation needs (None if it needs none)."""
    n = B.qgemv_workspace_bytes(op, fmt, N, K, nb, n_exp, topk)
    if n < 0:
        raise ValueError("invalid sizes for the workspace query")
    if n == 0:
        return None
    return torch.zeros(n, dtype=torch.uint8, device=device)
