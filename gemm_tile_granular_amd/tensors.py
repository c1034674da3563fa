"""Device-memory plumbing for callers of the binding (tests, bench).

Moves the generator's numpy buffers into HBM as torch tensors of the dtypes
the C ABI expects; no arithmetic of the method happens here.
"""
from __future__ import annotations

import numpy as np


def upload(a_bits: np.ndarray, b_bits: np.ndarray, peers: np.ndarray, device="cuda:0"):
    """bfloat16 bit patterns and fp32 peers -> (A, B, peers-or-None, C) on `device`."""
    import torch
    A = torch.from_numpy(np.ascontiguousarray(a_bits).view(np.int16)).to(device).view(torch.bfloat16)
    B = torch.from_numpy(np.ascontiguousarray(b_bits).view(np.int16)).to(device).view(torch.bfloat16)
    P = torch.from_numpy(np.ascontiguousarray(peers)).to(device) if peers.shape[0] else None
    C = torch.empty((a_bits.shape[0], b_bits.shape[1]), dtype=torch.float32, device=device)
    return A, B, P, C
