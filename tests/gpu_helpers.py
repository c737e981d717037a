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


def unpack_weights_w4(packed, N: int, K: int, keep_padding: bool = False) -> np.ndarray:
    """4-bit packed weights (include/quasar.h layout) -> row-major int8 [N, K].

    Byte ((t*CP + c)*64 + g*16 + r)*16 + b holds row 16t + r: column
    128c + 16g + b in its low nibble, 128c + 64 + 16g + b in its high nibble,
    as 4-bit two's complement.
    """
    if hasattr(packed, "codes"):
        packed = packed.codes
    if isinstance(packed, torch.Tensor):
        packed = packed.cpu().numpy()
    T, CP = (N + 15) // 16, K // 128
    a = np.asarray(packed, dtype=np.uint8)[: T * CP * 1024].reshape(T, CP, 4, 16, 16)
    lo = (a & 0x0F).astype(np.int16)
    hi = (a >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    w = np.empty((T, 16, CP, 2, 4, 16), np.int16)        # [t, r, c, half, g, b]
    w[:, :, :, 0] = lo.transpose(0, 3, 1, 2, 4)
    w[:, :, :, 1] = hi.transpose(0, 3, 1, 2, 4)
    w = w.reshape(T * 16, K).astype(np.int8)
    return w if keep_padding else w[:N, :K]
