"""CPU oracle for the decoder steps around the W8A8 linears -- TEST
INFRASTRUCTURE ONLY.

Only the test suite may import this module (like ``quasar_oracle``, it is
never imported by the product and shares no code with it).

A verify step runs the whole target model over the drafted positions in one
pass [Quasar, pt page §2 execution pipeline; zh page §2]; the pages quantize
its linears and leave the rest of the model as it is.  To measure the
linears' share of such a step, the repository also runs the rest of a
Qwen3-8B-shaped decoder layer.  The pages do not describe that model, so its
steps follow the plain definitions of the standard operations (the readings
are listed in the design notes):

* RMSNorm: ``h / sqrt(mean(h^2) + eps) * gamma``, with the residual stream
  ``h`` updated by ``h + delta`` first;
* per-head RMSNorm of the queries and keys, then the rotary embedding: the
  pair ``(j, j + D/2)`` of a head at position p is rotated by the angle
  ``p * base^(-2j/D)``;
* causal grouped-query attention: query head h reads key/value head
  ``h // (Hq / Hkv)``; position i of the verify window sees the cached
  positions ``0 .. pos0 + i``; ``softmax(q.k / sqrt(D)) v``;
* the MLP activation ``silu(gate) * up`` over the two halves of the gate_up
  output.

Everything here is float64 on float64 inputs (BF16 inputs are widened
exactly); the tests round the result to BF16 with ``quasar_oracle`` and allow
the one-ulp differences that the kernels' binary32 arithmetic produces at
rounding boundaries.
"""
from __future__ import annotations

import numpy as np

__all__ = ["embed", "rmsnorm", "head_rmsnorm", "rope", "qk_norm_rope", "attention",
           "silu_mul"]


def embed(tokens: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Rows of the embedding table (float64 [V, H]) for the token ids; an id
    outside [0, V) gives a zero row."""
    V, H = table.shape
    out = np.zeros((len(tokens), H), np.float64)
    for m, t in enumerate(np.asarray(tokens).tolist()):
        if 0 <= t < V:
            out[m] = table[t]
    return out


def rmsnorm(h: np.ndarray, gamma: np.ndarray, eps: float, delta: np.ndarray | None = None):
    """Residual add (when ``delta`` is given), then RMSNorm of every row.
    Returns (updated residual, normalised rows), both float64."""
    h = np.asarray(h, np.float64)
    if delta is not None:
        h = h + np.asarray(delta, np.float64)
    ms = np.mean(h * h, axis=1, keepdims=True)
    return h, h / np.sqrt(ms + eps) * np.asarray(gamma, np.float64)[None, :]


def head_rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis (one attention head's D values)."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, np.float64)


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotary embedding of x [..., n, D] at positions pos [n]: the pair
    (j, j + D/2) turns by pos * base^(-2j/D) radians."""
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    half = D // 2
    j = np.arange(half, dtype=np.float64)
    ang = np.asarray(pos, np.float64)[:, None] * base ** (-2.0 * j / D)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def qk_norm_rope(qkv: np.ndarray, q_gamma, k_gamma, B: int, T: int, Hq: int, Hkv: int, D: int,
                 pos0: int, base: float, eps: float):
    """Split the QKV output [B*T, (Hq + 2 Hkv) D] into heads, normalise q and
    k per head, rotate them at positions pos0 + i.  Returns q [B*T, Hq, D],
    k [B*T, Hkv, D], v [B*T, Hkv, D] (float64)."""
    qkv = np.asarray(qkv, np.float64).reshape(B * T, Hq + 2 * Hkv, D)
    q = head_rmsnorm(qkv[:, :Hq], q_gamma, eps)
    k = head_rmsnorm(qkv[:, Hq:Hq + Hkv], k_gamma, eps)
    v = qkv[:, Hq + Hkv:]
    pos = np.tile(pos0 + np.arange(T), B)
    q = np.stack([rope(q[:, h], pos, base) for h in range(Hq)], axis=1)
    k = np.stack([rope(k[:, g], pos, base) for g in range(Hkv)], axis=1)
    return q, k, v


def attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, B: int, T: int,
              Hq: int, pos0: int) -> np.ndarray:
    """Causal grouped-query attention of the verify positions.
    q [B*T, Hq, D]; caches [B, Hkv, L, D] with positions 0 .. pos0+T-1 filled.
    Returns [B*T, Hq, D] float64."""
    Hkv, D = k_cache.shape[1], k_cache.shape[3]
    G = Hq // Hkv
    q = np.asarray(q, np.float64).reshape(B, T, Hq, D)
    out = np.zeros((B, T, Hq, D), np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            K = np.asarray(k_cache[b, g], np.float64)
            V = np.asarray(v_cache[b, g], np.float64)
            for i in range(T):
                n = pos0 + i + 1  # visible positions
                sc = K[:n] @ q[b, i, h] / np.sqrt(D)
                sc = sc - sc.max()
                p = np.exp(sc)
                out[b, i, h] = (p / p.sum()) @ V[:n]
    return out.reshape(B * T, Hq, D)


def silu_mul(gate_up: np.ndarray) -> np.ndarray:
    """silu(gate) * up over [M, 2I] -> [M, I], float64."""
    gu = np.asarray(gate_up, np.float64)
    I = gu.shape[1] // 2
    g, u = gu[:, :I], gu[:, I:]
    return g / (1.0 + np.exp(-g)) * u
