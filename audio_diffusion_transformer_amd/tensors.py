"""Device-memory plumbing: numpy arrays from the input generator to torch
device tensors (bf16 kept as raw 16-bit patterns), workspaces, read-back."""
from __future__ import annotations

import numpy as np
import torch


def to_dev(a, device="cuda"):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to(device)
    if a.dtype == np.int32:
        return torch.from_numpy(a).to(device)
    raise TypeError(f"unsupported dtype {a.dtype}")


def bf16_empty(shape, device="cuda"):
    return torch.empty(shape, dtype=torch.int16, device=device)


def to_host_bf16(t):
    """device int16 (raw bf16 bits) -> numpy uint16."""
    return t.cpu().numpy().view(np.uint16)


def bf16_bits_to_f64(u):
    return ((np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
            .astype(np.float64))


def workspace(nbytes, device="cuda"):
    # torch's caching allocator returns blocks aligned to at least 512 bytes
    t = torch.empty(int(nbytes), dtype=torch.uint8, device=device)
    assert t.data_ptr() % 256 == 0
    return t


def weights_to_dev(w, device="cuda"):
    return {k: to_dev(v, device) for k, v in w.items()}
