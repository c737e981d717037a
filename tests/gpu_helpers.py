"""Host <-> device helpers for the GPU parity tests (no method arithmetic)."""
import sys

import numpy as np
import torch


def announce(*parts):
    """Name the case on stdout before a GPU step, flushed, so a dying run says which."""
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host_bf16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def f32_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def unpack_weights(packed, N: int, K: int, keep_padding: bool = False) -> np.ndarray:
    """Tile-packed INT8 weights (include/quasar.h layout) -> row-major [N, K].

    Byte ((t*C + c)*64 + g*16 + r)*16 + b holds row 16t + r, column 64c + 16g + b.
    """
    if hasattr(packed, "codes"):
        packed = packed.codes
    if isinstance(packed, torch.Tensor):
        packed = packed.cpu().numpy()
    T, C = (N + 15) // 16, (K + 63) // 64
    a = np.asarray(packed, dtype=np.int8)[: T * C * 1024].reshape(T, C, 4, 16, 16)
    w = a.transpose(0, 3, 1, 2, 4).reshape(T * 16, C * 64)
    return w if keep_padding else w[:N, :K]
