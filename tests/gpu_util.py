"""Device plumbing for the GPU tests: numpy byte arrays <-> torch cuda tensors."""
import sys

import numpy as np
import torch


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda()
    return t.view(torch.bfloat16)


def host_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def poison_bf16(shape) -> torch.Tensor:
    """bf16 output buffer filled with NaN patterns (0xFFFF), so unwritten outputs show."""
    return torch.full(shape, -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def note(msg: str):
    """Names the case about to run on the GPU (flushed, so it survives a crash)."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)
