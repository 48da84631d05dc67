"""Host-side helpers for the GPU parity tests (moving bytes, no arithmetic)."""

import numpy as np
import torch


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bfloat16 bit patterns -> device bfloat16 tensor (same bytes)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to("cuda")


def to_dev_u8(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes)).to("cuda")


def to_dev_f32(v: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to("cuda")


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host numpy array of its raw bits."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.cpu().numpy()
