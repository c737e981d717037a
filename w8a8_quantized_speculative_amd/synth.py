"""Seeded synthetic inputs for the W8A8 verify path.

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It holds no step of the quantized-verification method itself: it only draws
random tensors with the shapes and value distributions of the Qwen3-8B-shaped
verify workload, rounds them to bfloat16 with torch's own conversion, and
calibrates the per-channel smoothing vector that the method takes as an input.

Every draw comes from numpy's PCG64 seeded by ``SeedSequence([workload, layer,
role, block])``, so any block of any tensor can be regenerated on its own.

Smoothing-vector direction.  The Quasar pages write the smoothing identity as
``Y = (W diag(s)^-1)(diag(s) X)`` [Quasar, zh page, technical summary §2,
enhanced SmoothQuant], i.e. activations are *multiplied* by ``s``.  For the
smoothing to move outlier magnitude from activations into weights (the stated
purpose on every page, §2), ``s_j`` must be small on outlier channels, so the
default calibration is ``s_j = (max_n |W_nj| / max_m |X_mj|) ** alpha`` with
``alpha = 0.5``.  ``literal=True`` instead returns the reciprocal ratio
``(max|X_j| / max|W_j|) ** alpha`` (SmoothQuant's divisor written as a
multiplier); the kernels accept either, they only ever see the numbers.
"""
from __future__ import annotations

import numpy as np
import torch

# Roles: one independent stream per kind of tensor.
ROLE_X = 0
ROLE_W = 1
ROLE_OUTLIER_CH = 2
ROLE_OUTLIER_SCALE = 3
ROLE_DRAFT = 4
ROLE_UNIFORM = 5
ROLE_LOGITS = 6
ROLE_MISC = 7

# Qwen3-8B-shaped decoder layer: (name, K, N) of the four verify linears.
QWEN3_8B_HIDDEN = 4096
QWEN3_8B_INTERMEDIATE = 12288
QWEN3_8B_LAYERS = 36
QWEN3_8B_VOCAB = 151936
QWEN3_8B_LINEARS = (
    ("qkv", 4096, 6144),       # 32 q heads + 2 x 8 kv heads, head dim 128
    ("o", 4096, 4096),
    ("gate_up", 4096, 24576),  # gate and up fused
    ("down", 12288, 4096),
)
QWEN3_8B_LM_HEAD = ("lm_head", 4096, QWEN3_8B_VOCAB)

W_BLOCK_ROWS = 1024  # weights are drawn in row blocks of this many rows


def rng(*key: int) -> np.random.Generator:
    """Independent PCG64 stream for a tuple of small non-negative integers."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bfloat16 bit patterns (uint16) via torch's RNE conversion."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact widening)."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def activations(M: int, K: int, key: tuple, n_outliers: int | None = None,
                scale_lo: float = 30.0, scale_hi: float = 100.0,
                fixed_scale: float | None = None) -> np.ndarray:
    """Verify-window activations X [M, K] as bf16 bits.

    Entries are N(0, 1).  ``n_outliers`` seeded channels (default: 0.1 % of K,
    at least one) are multiplied by a per-channel factor drawn from
    U[scale_lo, scale_hi], or by ``fixed_scale`` when given.
    """
    x = rng(*key, ROLE_X).standard_normal((M, K), dtype=np.float32)
    if n_outliers is None:
        n_outliers = max(1, int(round(0.001 * K)))
    n_outliers = min(n_outliers, K)
    if n_outliers > 0:
        ch = rng(*key, ROLE_OUTLIER_CH).choice(K, size=n_outliers, replace=False)
        if fixed_scale is not None:
            sc = np.full(n_outliers, fixed_scale, dtype=np.float32)
        else:
            sc = rng(*key, ROLE_OUTLIER_SCALE).uniform(scale_lo, scale_hi, n_outliers).astype(np.float32)
        x[:, ch] *= sc[None, :]
    return to_bf16_bits(x)


def weight_block(N: int, K: int, key: tuple, block: int, std: float = 0.02) -> np.ndarray:
    """Rows [block*W_BLOCK_ROWS, ...) of W [N, K] ~ N(0, std^2) as bf16 bits."""
    r0 = block * W_BLOCK_ROWS
    rows = min(W_BLOCK_ROWS, N - r0)
    w = rng(*key, ROLE_W, block).standard_normal((rows, K), dtype=np.float32) * np.float32(std)
    return to_bf16_bits(w)


def weights(N: int, K: int, key: tuple, std: float = 0.02) -> np.ndarray:
    """Full W [N, K] as bf16 bits, assembled from its row blocks."""
    nb = (N + W_BLOCK_ROWS - 1) // W_BLOCK_ROWS
    return np.concatenate([weight_block(N, K, key, b, std) for b in range(nb)], axis=0) if N else \
        np.zeros((0, K), np.uint16)


def weight_rows(N: int, K: int, key: tuple, rows: np.ndarray, std: float = 0.02) -> np.ndarray:
    """Only the listed rows of W (regenerating just the blocks that hold them)."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, K), np.uint16)
    for b in np.unique(rows // W_BLOCK_ROWS):
        blk = weight_block(N, K, key, int(b), std)
        sel = np.nonzero(rows // W_BLOCK_ROWS == b)[0]
        out[sel] = blk[rows[sel] - b * W_BLOCK_ROWS]
    return out


def col_absmax_bf16(bits: np.ndarray) -> np.ndarray:
    """max over rows of |value| for each column of a bf16-bit matrix (float64)."""
    if bits.shape[0] == 0:
        return np.zeros(bits.shape[1], np.float64)
    return np.abs(bf16_bits_to_f32(bits)).max(axis=0).astype(np.float64)


def smoothing_vector(x_colmax: np.ndarray, w_colmax: np.ndarray, alpha: float = 0.5,
                     literal: bool = False) -> np.ndarray:
    """Per-input-channel smoothing factors s [K] (float32, all > 0).

    Default: s_j = (wmax_j / xmax_j) ** alpha.  ``literal``: (xmax_j / wmax_j) ** alpha.
    A channel with a zero maximum on either side gets s_j = 1.
    """
    xm = np.asarray(x_colmax, np.float64)
    wm = np.asarray(w_colmax, np.float64)
    ok = (xm > 0) & (wm > 0)
    ratio = np.ones_like(xm)
    if literal:
        ratio[ok] = xm[ok] / wm[ok]
    else:
        ratio[ok] = wm[ok] / xm[ok]
    return (ratio ** alpha).astype(np.float32)


def linear_case(M: int, K: int, N: int, key: tuple, n_outliers: int | None = None,
                fixed_scale: float | None = None, literal: bool = False, std: float = 0.02):
    """(X bits [M,K], W bits [N,K], s [K]) for one synthetic W8A8 linear."""
    x = activations(M, K, key, n_outliers=n_outliers, fixed_scale=fixed_scale)
    w = weights(N, K, key, std=std)
    s = smoothing_vector(col_absmax_bf16(x), col_absmax_bf16(w), literal=literal)
    return x, w, s


def draft_tokens(target: np.ndarray, V: int, p_match: float, key: tuple) -> np.ndarray:
    """Drafts [B, k] that equal ``target[b, i]`` with probability ``p_match``.

    ``target`` holds the token each draft position is planted against; on a miss
    the draft is uniform over the other V-1 tokens.
    """
    target = np.asarray(target, np.int64)
    g = rng(*key, ROLE_DRAFT)
    hit = g.random(target.shape) < p_match
    other = g.integers(0, V - 1, size=target.shape)
    other = other + (other >= target)  # skip the target itself
    return np.where(hit, target, other).astype(np.int32)


def uniforms(B: int, k: int, key: tuple) -> np.ndarray:
    """Seeded float32 uniforms in [0, 1), shape [B, k+1]."""
    u = rng(*key, ROLE_UNIFORM).random((B, k + 1), dtype=np.float32)
    return np.minimum(u, np.float32(np.nextafter(np.float32(1), np.float32(0))))


def logits(B: int, k: int, V: int, key: tuple, sigma: float = 3.0) -> np.ndarray:
    """Synthetic verifier logits [B, k+1, V] ~ N(0, sigma^2) as bf16 bits."""
    z = rng(*key, ROLE_LOGITS).standard_normal((B, k + 1, V), dtype=np.float32) * np.float32(sigma)
    return to_bf16_bits(z)
