"""Physically contiguous device memory for K/V pools, from the library's
gp_contiguous_malloc / gp_contiguous_free.  Allocation plumbing only: the compaction's
row moves address pool pages at random, and their speed depends on the physical pages
behind the pools, which contiguity did not reliably change in measurements; the kernels
themselves work on any device memory.

The memory is handed to torch through the CUDA array interface, so torch's own caching
allocator never sees it: the returned tensor keeps the owning object alive, and the
object frees the memory when the last view of it dies (not during interpreter shutdown,
when process exit reclaims device memory anyway)."""
from __future__ import annotations

import sys

import torch

from . import binding as B


class _Contiguous:
    """Owner of one contiguous device allocation, exposed as a byte array."""

    def __init__(self, nbytes: int, device: int):
        self.lib = B.load()
        self.nbytes, self.device = int(nbytes), int(device)
        self.ptr = self.lib.gp_contiguous_malloc(self.nbytes, self.device, None) or 0
        self.__cuda_array_interface__ = {"shape": (self.nbytes,), "typestr": "|u1",
                                         "data": (self.ptr, False), "version": 3}

    def __del__(self):
        if self.ptr and not sys.is_finalizing():
            self.lib.gp_contiguous_free(self.ptr, self.nbytes, self.device, None)
        self.ptr = 0


def empty(shape, dtype, device="cuda", contiguous: bool = True):
    """Returns (tensor, kind): the tensor in physically contiguous memory ("contiguous")
    when asked and the device can supply it, in ordinary memory ("ordinary") otherwise."""
    dev = torch.device(device)
    if contiguous and dev.type == "cuda":
        idx = dev.index if dev.index is not None else torch.cuda.current_device()
        numel = 1
        for s in shape:
            numel *= int(s)
        nbytes = max(1, numel * torch.empty((), dtype=dtype).element_size())
        owner = _Contiguous(nbytes, idx)
        if owner.ptr:
            raw = torch.as_tensor(owner, device=f"cuda:{idx}")
            assert raw.data_ptr() == owner.ptr and raw.numel() == nbytes
            return raw.view(dtype).view(tuple(int(s) for s in shape)), "contiguous"
    return torch.empty(shape, dtype=dtype, device=device), "ordinary"
