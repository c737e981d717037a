"""Pins of the decoder-step oracle and the N-gram drafter (CPU only).

The decoder oracle (oracle/decoder_oracle.py) follows the plain definitions of
RMSNorm, the rotary embedding, causal grouped-query attention and SiLU.  Each
test pins it to something other than its own formula: a closed form, an
invariant, an independent formulation (complex rotation, a library sigmoid),
or a brute-force special case, chosen so that a dropped term, a wrong sign or
a transposed index fails one of them.  The drafter's cases are worked by hand.
"""
import numpy as np
import pytest
from scipy.special import expit

from oracle import decoder_oracle as dec
from w8a8_quantized_speculative_amd.drafter import ngram_draft


def rng(*key):
    return np.random.default_rng(list(key))


# ------------------------------------------------------------------ RMSNorm
def test_rmsnorm_unit_rms_and_scale_invariance():
    h = rng(1).normal(size=(5, 64)) * rng(2).uniform(0.1, 10, size=(5, 1))
    _, y = dec.rmsnorm(h, np.ones(64), eps=0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-12)
    _, y3 = dec.rmsnorm(3.5 * h, np.ones(64), eps=0.0)
    assert np.allclose(y, y3, rtol=1e-12)
    # the direction of each row is kept
    cos = np.sum(y * h, axis=1) / np.linalg.norm(y, axis=1) / np.linalg.norm(h, axis=1)
    assert np.allclose(cos, 1.0, rtol=1e-12)


def test_rmsnorm_weights_and_residual_add():
    h = rng(3).normal(size=(3, 16))
    d = rng(4).normal(size=(3, 16))
    gamma = rng(5).uniform(0.5, 2, size=16)
    h2, y = dec.rmsnorm(h, gamma, eps=0.0, delta=d)
    assert np.array_equal(h2, h + d)
    _, y1 = dec.rmsnorm(h + d, np.ones(16), eps=0.0)
    assert np.allclose(y, y1 * gamma[None, :], rtol=1e-13)
    # eps acts as an extra mean square: a constant row c gives c / sqrt(c^2 + eps)
    _, yc = dec.rmsnorm(np.full((1, 8), 0.5), np.ones(8), eps=0.75)
    assert np.allclose(yc, 0.5 / np.sqrt(0.25 + 0.75), rtol=1e-15)


# ------------------------------------------------------------------ RoPE
def test_rope_equals_complex_rotation():
    """Pair (j, j + D/2) as the complex number x_j + i x_{j+D/2}, multiplied by
    exp(i p base^(-2j/D))."""
    D, base = 16, 1e6
    x = rng(6).normal(size=(4, D))
    pos = np.array([0, 1, 17, 2047])
    z = x[:, :D // 2] + 1j * x[:, D // 2:]
    theta = np.array([[p * base ** (-2.0 * j / D) for j in range(D // 2)] for p in pos])
    zr = z * np.exp(1j * theta)
    ref = np.concatenate([zr.real, zr.imag], axis=1)
    assert np.allclose(dec.rope(x, pos, base), ref, rtol=1e-12, atol=1e-12)


def test_rope_position_zero_norms_and_relative_positions():
    D, base = 128, 1e6
    x = rng(7).normal(size=(3, D))
    assert np.array_equal(dec.rope(x, np.zeros(3, int), base), x)
    r = dec.rope(x, np.array([5, 900, 2047]), base)
    assert np.allclose(np.linalg.norm(r, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    q, k = rng(8).normal(size=(1, D)), rng(9).normal(size=(1, D))
    d1 = dec.rope(q, np.array([40]), base) @ dec.rope(k, np.array([33]), base).T
    d2 = dec.rope(q, np.array([1040]), base) @ dec.rope(k, np.array([1033]), base).T
    assert np.allclose(d1, d2, rtol=1e-9)
    # the first pair turns by exactly p radians (base^0 = 1)
    e = np.zeros((1, D))
    e[0, 0] = 1.0
    t = dec.rope(e, np.array([3]), base)
    assert np.isclose(t[0, 0], np.cos(3.0)) and np.isclose(t[0, D // 2], np.sin(3.0))


def test_qk_norm_rope_splits_heads_in_order():
    B, T, Hq, Hkv, D = 2, 3, 4, 2, 8
    qkv = rng(10).normal(size=(B * T, (Hq + 2 * Hkv) * D))
    q, k, v = dec.qk_norm_rope(qkv, np.ones(D), np.ones(D), B, T, Hq, Hkv, D, pos0=0,
                               base=1e6, eps=0.0)
    # v is passed through; at position 0 (row 0 of each sequence) q and k are
    # the per-head normalised slices
    assert np.array_equal(v, qkv.reshape(B * T, -1, D)[:, Hq + Hkv:])
    heads = qkv.reshape(B * T, Hq + 2 * Hkv, D)
    for m in (0, T):
        for h in range(Hq):
            x = heads[m, h]
            assert np.allclose(q[m, h], x / np.sqrt(np.mean(x * x)), rtol=1e-12)
        for g in range(Hkv):
            x = heads[m, Hq + g]
            assert np.allclose(k[m, g], x / np.sqrt(np.mean(x * x)), rtol=1e-12)
    # row i of a sequence sits at position pos0 + i: norms unchanged by rotation
    assert np.allclose(np.linalg.norm(q[1], axis=-1), np.sqrt(D), rtol=1e-12)


# ------------------------------------------------------------------ attention
def caches(B, Hkv, L, D, seed):
    g = rng(seed)
    return g.normal(size=(B, Hkv, L, D)), g.normal(size=(B, Hkv, L, D))


def test_attention_single_visible_key_returns_its_value():
    B, T, Hq, Hkv, D = 1, 1, 4, 2, 8
    kc, vc = caches(B, Hkv, 4, D, 11)
    q = rng(12).normal(size=(B * T, Hq, D))
    out = dec.attention(q, kc, vc, B, T, Hq, pos0=0)
    for h in range(Hq):
        assert np.allclose(out[0, h], vc[0, h // 2, 0], rtol=1e-15)


def test_attention_equal_keys_average_the_values_and_causality():
    B, T, Hq, Hkv, D, pos0 = 1, 3, 2, 1, 8, 5
    kc, vc = caches(B, Hkv, 16, D, 13)
    kc[:] = kc[:, :, :1]  # every key the same: uniform weights
    q = rng(14).normal(size=(B * T, Hq, D))
    out = dec.attention(q, kc, vc, B, T, Hq, pos0)
    for i in range(T):
        assert np.allclose(out[i, 0], vc[0, 0, :pos0 + i + 1].mean(axis=0), rtol=1e-12)
    # positions past pos0 + i are invisible to query i
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, :, pos0 + 1:] = 99.0
    vc2[:, :, pos0 + 1:] = -99.0
    out2 = dec.attention(q, kc2, vc2, B, T, Hq, pos0)
    assert np.array_equal(out2[0], out[0])


def test_attention_matches_a_library_softmax_and_groups_heads():
    from scipy.special import softmax
    B, T, Hq, Hkv, D, pos0 = 2, 2, 4, 2, 16, 9
    kc, vc = caches(B, Hkv, 12, D, 15)
    q = rng(16).normal(size=(B * T, Hq, D))
    q[:, 1] = q[:, 0]  # heads 0 and 1 share KV head 0
    out = dec.attention(q, kc, vc, B, T, Hq, pos0)
    assert np.allclose(out[:, 0], out[:, 1], rtol=1e-15)
    b, i, h = 1, 1, 3
    n = pos0 + i + 1
    p = softmax(kc[b, h // 2, :n] @ q[b * T + i, h] / 4.0)
    assert np.allclose(out[b * T + i, h], p @ vc[b, h // 2, :n], rtol=1e-12)


# ------------------------------------------------------------------ SiLU
def test_silu_mul_against_library_sigmoid():
    gu = rng(17).normal(size=(3, 40)) * 6
    ref = gu[:, :20] * expit(gu[:, :20]) * gu[:, 20:]
    assert np.allclose(dec.silu_mul(gu), ref, rtol=1e-13, atol=1e-300)
    z = np.zeros((1, 4))
    z[0, 2:] = 5.0
    assert np.array_equal(dec.silu_mul(z), np.zeros((1, 2)))  # silu(0) = 0


def test_embed_rows_and_out_of_range():
    table = rng(18).normal(size=(10, 4))
    out = dec.embed(np.array([3, -1, 9, 10]), table)
    assert np.array_equal(out[0], table[3]) and np.array_equal(out[2], table[9])
    assert not out[1].any() and not out[3].any()


# ------------------------------------------------------------------ drafter
@pytest.mark.parametrize("history,k,n_max,expected", [
    ([1, 2, 3, 4, 5, 1, 2, 3], 3, 3, [4, 5, 1]),         # 3-gram match
    ([7, 8, 9], 3, 3, [9, 9, 9]),                         # no match: repeat the last token
    ([5, 9, 1, 2, 3, 7, 2, 3, 8, 1, 2, 3], 3, 3, [7, 2, 3]),  # the longest n-gram wins
    ([1, 2, 9, 1, 2, 8, 1, 2], 3, 2, [8, 1, 2]),          # the most recent occurrence wins
    ([4, 6, 4], 4, 3, [6, 4, 4, 4]),                      # short continuation, padded
    ([3], 2, 3, [3, 3]),                                  # a one-token history
    ([2, 2, 2, 2], 2, 3, [2, 2]),                         # overlapping occurrences
])
def test_ngram_draft_hand_worked(history, k, n_max, expected):
    assert ngram_draft(np.array(history), k, n_max).tolist() == expected


def test_ngram_draft_brute_force():
    """Against a direct scan on random short histories over a 4-token alphabet."""
    g = rng(19)
    for _ in range(300):
        h = g.integers(0, 4, size=g.integers(1, 14)).tolist()
        k, n_max = int(g.integers(1, 5)), int(g.integers(1, 4))
        expected = None
        for n in range(min(n_max, len(h) - 1), 0, -1):
            suf = h[-n:]
            for p in range(len(h) - n - 1, -1, -1):
                if h[p:p + n] == suf and h[p + n:p + n + k]:
                    cont = h[p + n:p + n + k]
                    expected = cont + [cont[-1]] * (k - len(cont))
                    break
            if expected:
                break
        if expected is None:
            expected = [h[-1]] * k
        assert ngram_draft(np.array(h), k, n_max).tolist() == expected, (h, k, n_max)
