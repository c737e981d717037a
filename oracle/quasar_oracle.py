"""CPU oracle for the Quasar W8A8 verify path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product (the HIP library and its
Python binding) never calls it, and it shares no code with the product: it
neither imports the package nor reads its headers or kernels.

What it computes
----------------
Quasar verifies speculative drafts with a W8A8 copy of the target model
[Quasar, all four pages, technical summary §2 "Methodology"].  Each linear:

1. offline: the weights are smoothed and quantized to INT8 and kept resident
   [pt §2 execution pipeline item 1; ko §2 pipeline "offline"];
2. online: the BF16 input activations are smoothed and quantized dynamically
   [pt §2 item 2; nl §2 pipeline "Online"];
3. an INT8 x INT8 matrix product is taken on integer matrix units
   [pt §2 item 3; zh §2 item 3];
4. the result is dequantized back to BF16 before the nonlinear layers and the
   softmax [pt §2 item 4; ko §2 "dequantization"].

Smoothing follows the identity ``Y = (W diag(s)^-1)(diag(s) X)`` [zh §2 item 2];
quantization is symmetric and uniform [pt §2].  The verify decision is greedy
at T = 0 [ko §4 results, "Qwen3 (Greedy, T=0)"] or rejection sampling on the
dequantized logits, which keeps the target distribution exactly [pt §2 item 4;
zh §2 pipeline "lossless rejection sampling"].

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):

* per-output-channel weight scales, per-token dynamic activation scales;
* INT8 range [-127, 127], rounding half to even, scale = absmax / 127 and
  codes = round(v * RN32(127 / absmax)) in binary32 -- the precision in which
  the kernels take the same integer decisions;
* ``diag(s)^-1`` is applied as a multiply by ``RN32(1 / s_k)``;
* the smoothed activation ``xs = RN32(x * s)`` stays binary32 (never BF16);
* an all-zero row gets codes 0 and scale 0;
* dequant ``Y = BF16(RN32(RN32(RN32(acc) * sx_m) * sw_n))``, no bias;
* greedy: argmax over the BF16 logits, lowest index on ties; the accept length
  is the longest draft prefix equal to the argmax, the next token is the argmax
  at the first mismatch (or the bonus position);
* rejection with a one-hot draft: accept iff u < p(d) (strict), residual =
  p with p(d) removed and renormalised, sampled by inverse CDF in index order
  with the last uniform of the row.

Conventions: BF16 tensors are numpy ``uint16`` bit patterns; float32 steps use
numpy float32 arithmetic (each operation rounded to nearest even, no fused
multiply-add); reference values that decide nothing are taken in float64.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_to_f32", "f32_to_bf16", "rn32_reciprocal", "quantize_rows",
    "smooth_weights", "quantize_weights", "smooth_activations",
    "quantize_activations", "int_matmul", "dequantize", "dequantize_f64",
    "w8a8_linear", "w8a8_linear_rows", "argmax_lowest", "greedy_accept",
    "softmax_f64", "rejection_accept", "QMAX_W4", "quantize_weights_w4", "w4a8_linear_rows",
]

QMAX = 127  # symmetric INT8: codes in [-127, 127]
QMAX_W4 = 7  # symmetric INT4 weights (the 4-bit variant): codes in [-7, 7]


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32: the 16 bits become the high half."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest, ties to even.

    Written out on the bit pattern: add 0x7FFF plus the lowest kept bit, then
    drop the low 16 bits.  Inputs are finite (the path never produces NaN).
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return (r & np.uint64(0xFFFF)).astype(np.uint16)


def rn32_reciprocal(s: np.ndarray) -> np.ndarray:
    """RN32(1 / s): the exact quotient rounded once to binary32.

    Dividing in binary64 and rounding to binary32 gives the correctly rounded
    binary32 quotient (53 >= 2*24 + 2, so the double rounding is innocuous).
    """
    return (1.0 / np.asarray(s, dtype=np.float64)).astype(np.float32)


# --------------------------------------------------------------------------
# symmetric per-row quantizer   [pt §2: symmetric uniform quantization]
# --------------------------------------------------------------------------
def quantize_rows(v: np.ndarray, qmax: int = QMAX):
    """Per-row symmetric quantization of a float32 matrix to [-qmax, qmax].

    For each row: A = max |v| (exact); if A == 0 the codes are 0 and the scale
    is 0; otherwise scale = RN32(A / qmax), inv = RN32(qmax / A) and
    code = clamp(round_half_even(RN32(v * inv)), -qmax, qmax).  qmax = 127 is
    INT8; the 4-bit weight variant uses qmax = 7.
    Returns (codes int8 [R, C], scale float32 [R]).
    """
    v = np.asarray(v, dtype=np.float32)
    R = v.shape[0]
    codes = np.zeros(v.shape, dtype=np.int8)
    scale = np.zeros(R, dtype=np.float32)
    for r in range(R):
        row = v[r]
        a = np.float32(np.max(np.abs(row))) if row.size else np.float32(0)
        if a == 0:
            continue
        scale[r] = np.float32(np.float64(a) / qmax)
        inv = np.float32(qmax / np.float64(a))
        prod = row * inv                      # binary32 product, one rounding
        q = np.rint(prod)                     # ties to even
        codes[r] = np.clip(q, -qmax, qmax).astype(np.int8)
    return codes, scale


# --------------------------------------------------------------------------
# step a0: offline weight smoothing + quantization   [pt §2 item 1; zh §2]
# --------------------------------------------------------------------------
def smooth_weights(w_bits: np.ndarray, s: np.ndarray) -> np.ndarray:
    """W diag(s)^-1 in binary32: w'_nk = RN32(f32(W_nk) * RN32(1/s_k))."""
    r = rn32_reciprocal(s)
    return bf16_to_f32(w_bits) * r[None, :]


def quantize_weights(w_bits: np.ndarray, s: np.ndarray):
    """Smoothed weights -> (INT8 codes [N, K], per-output-channel scale [N])."""
    return quantize_rows(smooth_weights(w_bits, s))


def quantize_weights_w4(w_bits: np.ndarray, s: np.ndarray):
    """4-bit verifier weights [pt §5 and zh §5: lower-bit verification as future
    work].  The pages give no group size, zero point or range, so this reads
    them as the INT8 rule at qmax = 7: the same smoothed weights, one symmetric
    scale per output channel, codes in [-7, 7].
    Returns (codes int8 [N, K] in [-7, 7], scale float32 [N])."""
    return quantize_rows(smooth_weights(w_bits, s), qmax=QMAX_W4)


# --------------------------------------------------------------------------
# steps a1-a3: online activation smoothing + dynamic per-token quantization
#   [pt §2 item 2; nl §2 "Online"; zh §2 item 2]
# --------------------------------------------------------------------------
def smooth_activations(x_bits: np.ndarray, s: np.ndarray) -> np.ndarray:
    """diag(s) X in binary32: xs_mk = RN32(f32(X_mk) * s_k)."""
    return bf16_to_f32(x_bits) * np.asarray(s, dtype=np.float32)[None, :]


def quantize_activations(x_bits: np.ndarray, s: np.ndarray):
    """BF16 activations -> (codes int8 [M, K], per-token scale [M], xs float32 [M, K])."""
    xs = smooth_activations(x_bits, s)
    q, sx = quantize_rows(xs)
    return q, sx, xs


# --------------------------------------------------------------------------
# step a4: INT8 x INT8 -> exact integer accumulation   [pt §2 item 3]
# --------------------------------------------------------------------------
def int_matmul(qx: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k qx[m, k] * qw[n, k], exact, returned as int64.

    The product is taken as a float64 matrix product of the integer codes: every
    partial sum is an integer of magnitude <= K * 127^2 < 2^53, so it is
    represented exactly whatever order the library sums in.
    """
    a = np.asarray(qx, dtype=np.float64)
    b = np.asarray(qw, dtype=np.float64)
    return np.rint(a @ b.T).astype(np.int64)


# --------------------------------------------------------------------------
# step a5: dequantize to BF16   [pt §2 item 4; ko §2 "dequantization"]
# --------------------------------------------------------------------------
def dequantize(acc: np.ndarray, sx: np.ndarray, sw: np.ndarray) -> np.ndarray:
    """Y = BF16(RN32(RN32(RN32(acc) * sx_m) * sw_n)) as bf16 bits [M, N]."""
    a = np.asarray(acc, dtype=np.int64).astype(np.float32)   # RN32 of the integer
    t = a * np.asarray(sx, np.float32)[:, None]
    t = t * np.asarray(sw, np.float32)[None, :]
    return f32_to_bf16(t)


def dequantize_f64(acc: np.ndarray, sx: np.ndarray, sw: np.ndarray) -> np.ndarray:
    """acc * sx * sw in float64 (no intermediate rounding): the value Y approximates."""
    return (np.asarray(acc, np.float64) * np.asarray(sx, np.float64)[:, None]
            * np.asarray(sw, np.float64)[None, :])


def w8a8_linear(x_bits: np.ndarray, s: np.ndarray, qw: np.ndarray, sw: np.ndarray):
    """One W8A8 SmoothQuant linear over the verify window.

    Returns dict(y=bf16 bits [M,N], acc=int64 [M,N], qx, sx, xs).
    """
    qx, sx, xs = quantize_activations(x_bits, s)
    acc = int_matmul(qx, qw)
    return {"y": dequantize(acc, sx, sw), "acc": acc, "qx": qx, "sx": sx, "xs": xs}


def w8a8_linear_rows(x_bits: np.ndarray, s: np.ndarray, w_rows_bits: np.ndarray):
    """Same linear restricted to a subset of output channels (rows of W).

    Weight quantization is per output row, so any subset of rows is quantized
    and multiplied exactly as it would be inside the full matrix.
    """
    qw, sw = quantize_weights(w_rows_bits, s)
    out = w8a8_linear(x_bits, s, qw, sw)
    out["qw"], out["sw"] = qw, sw
    return out


def w4a8_linear_rows(x_bits: np.ndarray, s: np.ndarray, w_rows_bits: np.ndarray):
    """The linear with 4-bit weights: INT4 weight codes (quantize_weights_w4),
    the same dynamic INT8 activations, exact integer accumulation and dequant."""
    qw, sw = quantize_weights_w4(w_rows_bits, s)
    out = w8a8_linear(x_bits, s, qw, sw)
    out["qw"], out["sw"] = qw, sw
    return out


# --------------------------------------------------------------------------
# steps a7-a8: verification decision
# --------------------------------------------------------------------------
def argmax_lowest(logit_bits: np.ndarray) -> np.ndarray:
    """Per-row argmax over BF16 logits [..., V]; ties go to the lowest index.

    Values are compared as reals (so -0 equals +0).
    """
    v = bf16_to_f32(logit_bits).astype(np.float64)
    return np.argmax(v, axis=-1).astype(np.int64)   # numpy returns the first maximum


def greedy_accept(logit_bits: np.ndarray, draft: np.ndarray):
    """Greedy (T = 0) verification   [ko §4, "Qwen3 (Greedy, T=0)"].

    logit_bits [B, k+1, V], draft [B, k].  For each sequence: g_i = argmax of
    position i; L = number of leading drafts equal to g (draft i is checked
    against the target's prediction at position i); next = g_L.
    Returns (L int64 [B], next int64 [B], g int64 [B, k+1]).
    """
    g = argmax_lowest(logit_bits)
    B, kp1 = g.shape
    k = kp1 - 1
    draft = np.asarray(draft, np.int64).reshape(B, k)
    L = np.zeros(B, np.int64)
    nxt = np.zeros(B, np.int64)
    for b in range(B):
        n = 0
        while n < k and draft[b, n] == g[b, n]:
            n += 1
        L[b] = n
        nxt[b] = g[b, n]
    return L, nxt, g


def softmax_f64(logit_bits_row: np.ndarray, temperature: float) -> np.ndarray:
    """softmax(logits / T) in float64, max-subtracted."""
    z = bf16_to_f32(logit_bits_row).astype(np.float64) / float(temperature)
    z = z - np.max(z)
    e = np.exp(z)
    return e / np.sum(e)


def rejection_accept(logit_bits: np.ndarray, draft: np.ndarray, temperature: float,
                     u: np.ndarray):
    """Rejection-sampling verification of one-hot drafts (T > 0).

    Standard speculative sampling with the draft distribution a point mass on
    d: draft i is accepted iff u[b, i] < p_i(d) where p_i = softmax(logits_i/T);
    a draft id outside [0, V) has p = 0.  At the first rejection the next token
    is drawn from p_i with d removed and renormalised; when all k drafts pass,
    from p_k.  The draw is the smallest j with cumsum(r)_j > u[b, k] * sum(r).
    This keeps the emitted tokens distributed exactly as the verifier's own p
    [pt §2 item 4; zh §2 "lossless rejection sampling"].
    Returns (L [B], next [B], p_draft float64 [B, k], sample_row [B],
    target float64 [B], cdf_rows list of float64 cumsum arrays).
    """
    B, kp1, V = logit_bits.shape
    k = kp1 - 1
    draft = np.asarray(draft, np.int64).reshape(B, k)
    u = np.asarray(u, np.float64).reshape(B, kp1)
    L = np.zeros(B, np.int64)
    nxt = np.zeros(B, np.int64)
    p_draft = np.zeros((B, k), np.float64)
    rows = np.zeros(B, np.int64)
    targets = np.zeros(B, np.float64)
    cdfs = []
    for b in range(B):
        probs = [softmax_f64(logit_bits[b, i], temperature) for i in range(kp1)]
        for i in range(k):
            d = draft[b, i]
            p_draft[b, i] = probs[i][d] if 0 <= d < V else 0.0
        n = 0
        while n < k and u[b, n] < p_draft[b, n]:
            n += 1
        r = probs[n].copy()
        if n < k and 0 <= draft[b, n] < V:
            r[draft[b, n]] = 0.0
        c = np.cumsum(r)
        target = u[b, k] * c[-1]
        j = int(np.searchsorted(c, target, side="right"))  # smallest j with c[j] > target
        L[b], nxt[b], rows[b], targets[b] = n, min(j, V - 1), n, target
        cdfs.append(c)
    return L, nxt, p_draft, rows, targets, cdfs
