"""Device-memory plumbing for the GPU parity tests (torch is used only to
allocate HBM, copy bytes and pick the stream)."""
import numpy as np
import torch

import async_tensor_tile_amd as att


def require_native():
    # fails loudly (no fallback) when the HIP library is missing
    att.lib()


def to_dev(a: np.ndarray, pad: int = 0) -> torch.Tensor:
    b = np.ascontiguousarray(a).view(np.uint8).reshape(-1)
    t = torch.empty(b.size + pad, dtype=torch.uint8, device="cuda")
    t[: b.size].copy_(torch.from_numpy(b))
    if pad:
        t[b.size:].fill_(0xEE)
    return t


def empty_dev(nbytes: int, fill: int = None) -> torch.Tensor:
    t = torch.empty(max(1, nbytes), dtype=torch.uint8, device="cuda")
    if fill is not None:
        t.fill_(fill)
    return t


def to_host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def encode(t: torch.Tensor, dtype, dims, strides, box, estride=None, swizzle="none", fill="zero"):
    return att.tmap_encode(dtype, len(dims), t.data_ptr(), dims, strides, box, estride, swizzle, fill)
