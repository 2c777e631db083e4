"""Device-memory plumbing for the MoE layer library: weights and workspaces as
torch tensors on the GPU.  Nothing here computes part of the layer; it copies
host arrays (numpy, in the layouts of include/moe_decode.h) to HBM.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch


def _dev(a: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device, non_blocking=False)


@dataclasses.dataclass
class DeviceExperts:
    """An expert set resident in HBM.  NVFP4: w13 u8 [n,2,I,H/2], w13_scale u8
    [n,2,I,H/16], w2 u8 [n,H,I/2], w2_scale u8 [n,H,I/16], glob f32 [n,3].
    BF16: w13 bf16 [n,2,I,H], w2 bf16 [n,H,I].  MXFP8: w13 u8 [n,2,I,H],
    w13_scale u8 [n,2,I,H/32], w2 u8 [n,H,I], w2_scale u8 [n,H,I/32]."""
    fmt: str
    n: int
    w13: torch.Tensor
    w2: torch.Tensor
    w13_scale: torch.Tensor | None = None
    w2_scale: torch.Tensor | None = None
    glob: torch.Tensor | None = None

    @classmethod
    def from_host(cls, ex, device="cuda") -> "DeviceExperts":
        """ex: host expert set with the same field names (numpy arrays)."""
        if ex.fmt == "nvfp4":
            return cls("nvfp4", ex.n, _dev(ex.w13, device), _dev(ex.w2, device),
                       _dev(ex.w13_scale, device), _dev(ex.w2_scale, device),
                       _dev(ex.glob, device))
        if ex.fmt == "mxfp8":
            return cls("mxfp8", ex.n, _dev(ex.w13, device), _dev(ex.w2, device),
                       _dev(ex.w13_scale, device), _dev(ex.w2_scale, device))
        return cls("bf16", ex.n, _dev(ex.w13, device), _dev(ex.w2, device))

    def nbytes_per_expert(self) -> int:
        tot = self.w13.numel() * self.w13.element_size() + self.w2.numel() * self.w2.element_size()
        if self.fmt in ("nvfp4", "mxfp8"):
            tot += self.w13_scale.numel() + self.w2_scale.numel()
        if self.fmt == "nvfp4":
            tot += self.glob.numel() * 4
        return tot // self.n


@dataclasses.dataclass
class DeviceLayer:
    fmt: str
    router: torch.Tensor          # bf16 [E, H]
    routed: DeviceExperts
    shared: DeviceExperts | None      # None when the layer has no shared expert

    @classmethod
    def from_host(cls, layer, device="cuda") -> "DeviceLayer":
        """layer: host layer with router (u16 [E, H]), routed and shared expert sets."""
        return cls(layer.routed.fmt, _dev(layer.router, device),
                   DeviceExperts.from_host(layer.routed, device),
                   None if layer.shared is None else DeviceExperts.from_host(layer.shared, device))


def to_device_bf16(a: np.ndarray, device="cuda") -> torch.Tensor:
    """bf16 bit patterns (np.uint16) to a device bf16 tensor."""
    return _dev(a, device)


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace (the library needs zeroed counters on first use).
    torch's caching allocator returns 512-byte-aligned blocks."""
    ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
    assert ws.data_ptr() % 256 == 0
    return ws
