"""Device-memory plumbing for the binding: torch allocates, libnanoflow computes.

Converts host bf16 bit arrays (uint16) into torch bfloat16 device tensors and wraps their
pointers in the ABI structures. No arithmetic of the layer happens here.
"""

from __future__ import annotations

import numpy as np
import torch

from . import abi


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor on ``device``."""
    a = np.ascontiguousarray(bits).view(np.int16)
    return torch.from_numpy(a).to(device).view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """torch.bfloat16 tensor -> host uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class DeviceWeights:
    """A layer's weights resident on the device, plus the nf_layer_weights view of them."""

    NAMES = ("g_attn", "w_qkv", "w_o", "g_ffn", "w_gate_up", "w_down", "w_router")  # w_router: MoE only

    def __init__(self, host: dict | None, device, tensors: dict | None = None):
        self.t = tensors if tensors is not None else {
            k: bf16_tensor(host[k], device) for k in self.NAMES if k in host}
        self.desc = abi.nf_layer_weights(*[self.t[k].data_ptr() if k in self.t else None for k in self.NAMES])

    @classmethod
    def from_int16(cls, t16: dict) -> "DeviceWeights":
        """From device int16 tensors holding bf16 bit patterns (no copy)."""
        return cls(None, None, {k: t16[k].view(torch.bfloat16) for k in cls.NAMES if k in t16})

    def host_bits(self) -> dict:
        return {k: bf16_bits(v) for k, v in self.t.items()}


class DevicePool:
    """Paged KV pool of one layer on the device (K in 32-dim column chunks, each token-major,
    and V dim-major within a block)."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor):
        assert k.dtype == torch.bfloat16 and v.dtype == torch.bfloat16
        self.k = k
        self.v = v
        self.desc = abi.nf_kv_pool(k.data_ptr(), v.data_ptr(), k.shape[0])

    @classmethod
    def from_host(cls, k_bits: np.ndarray, v_bits: np.ndarray, device) -> "DevicePool":
        return cls(bf16_tensor(k_bits, device), bf16_tensor(v_bits, device))

    @classmethod
    def from_int16(cls, k16: torch.Tensor, v16: torch.Tensor) -> "DevicePool":
        return cls(k16.view(torch.bfloat16), v16.view(torch.bfloat16))

    def host_bits(self):
        return bf16_bits(self.k), bf16_bits(self.v)


_HIP = None


def copy_device(dst_ptr: int, src_ptr: int, nbytes: int) -> None:
    """Synchronous device-to-device copy between raw device pointers (hipMemcpy)."""
    global _HIP
    import ctypes

    if _HIP is None:
        _HIP = ctypes.CDLL("libamdhip64.so")
        _HIP.hipMemcpy.restype = ctypes.c_int
        _HIP.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    rc = _HIP.hipMemcpy(dst_ptr, src_ptr, nbytes, 3)  # hipMemcpyDeviceToDevice
    if rc != 0:
        raise RuntimeError(f"hipMemcpy failed with {rc}")


def current_stream_ptr(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream
