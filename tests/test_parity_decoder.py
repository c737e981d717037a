"""GPU parity of the decoder steps around the W8A8 linears, every element
against the float64 oracle (oracle/decoder_oracle.py).

The kernels compute in binary32 and round their outputs to BF16; the oracle
is float64.  The bar for a BF16 output is elementwise

    |gpu - oracle| <= one BF16 spacing at the oracle value + A,

A the binary32 error bound of the kernel's arithmetic (stated per test: a
dot product of n terms is off by at most ~n 2^-24 times the sum of the
terms' magnitudes), and nearly every element identical to the oracle
rounded to BF16 (99%; 95% for the rotary embedding).  Without A, outputs
formed by cancellation (a rotated pair, an attention average of mixed-sign
values) would fail a pure ulp bar on binary32 error far below the BF16
spacing of their inputs.  Exact copies (the embedding rows, v into the
cache, the residual add) must be bit-identical.  Shapes are Qwen3-8B's
(hidden 4096, 32 query / 8 KV heads of 128, intermediate 12288) at verify
windows of 6, 48 and 96 tokens, with cached contexts from 0 to 2047
positions (chunk edges at 63/64 included).
"""
import numpy as np
import pytest
import torch

from oracle import decoder_oracle as dec
from oracle import quasar_oracle as orc
from w8a8_quantized_speculative_amd import binding, synth
from tests.gpu_helpers import announce, dev, dev_bf16, host, host_bf16

pytestmark = pytest.mark.gpu

H, HQ, HKV, D, I = 4096, 32, 8, 128, 12288
EPS, BASE = 1e-6, 1e6


def bf16_normal(shape, key, scale=1.0):
    return synth.to_bf16_bits(synth.rng(*key).normal(size=shape).astype(np.float32) * np.float32(scale))


U = 2.0 ** -24


def bf16_spacing(ref):
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


def assert_bf16_close(got_bits, ref_f64, exact_frac, allow=0.0):
    """|got - ref| <= BF16 spacing at ref + allow, elementwise, and at least
    exact_frac of the elements equal to the oracle rounded to BF16."""
    ref = np.asarray(ref_f64, np.float64)
    got = orc.bf16_to_f32(got_bits).astype(np.float64)
    excess = np.abs(got - ref) - (bf16_spacing(ref) + allow)
    assert excess.max() <= 0, f"worst excess {excess.max():.3e} at {np.unravel_index(excess.argmax(), excess.shape)}"
    frac = np.mean(got_bits == orc.f32_to_bf16(ref.astype(np.float32)))
    assert frac >= exact_frac, f"only {frac:.4f} identical"


def rope_allow(x_heads, D):
    """Allowance of a rotated pair: the pair's norm times the angle error
    (binary64 angle rounded to binary32 and its sine/cosine: < 1e-6 rad) plus
    the relative error of the binary32 head norm ((D + 8) 2^-24)."""
    half = D // 2
    a, b = x_heads[..., :half], x_heads[..., half:]
    r = np.sqrt(a * a + b * b)
    return np.concatenate([r, r], axis=-1) * (1e-6 + (D + 8) * U)


def attention_allow(q, kc, vc, B, T, Hq, pos0):
    """(n + 8) 2^-24 sum_t p_t |v_t|, n = pos0 + T visible positions at most."""
    return (pos0 + T + 8) * U * dec.attention(q, kc, np.abs(vc), B, T, Hq, pos0)


def f32(bits):
    return orc.bf16_to_f32(bits).astype(np.float64)


def test_embed_rows_exact():
    V, M = 1000, 8
    announce("embed", V, H)
    table = bf16_normal((V, H), (60, 0))
    tok = np.array([0, 999, 5, -1, 1000, 17, 17, 3], np.int32)
    h = binding.quasar_embed(dev(tok), dev_bf16(table))
    torch.cuda.synchronize()
    ref = dec.embed(tok, orc.bf16_to_f32(table).astype(np.float64))
    assert np.array_equal(host(h), ref.astype(np.float32))


@pytest.mark.parametrize("M", [6, 48, 96])
@pytest.mark.parametrize("with_delta", [False, True])
def test_rmsnorm(M, with_delta):
    announce("rmsnorm", M, with_delta)
    g = synth.rng(61, M)
    h0 = (g.normal(size=(M, H)) * g.uniform(0.05, 20, size=(M, 1))).astype(np.float32)
    h0[:, :4] *= 30  # outlier channels
    gamma = g.uniform(0.5, 1.5, size=H).astype(np.float32)
    delta = bf16_normal((M, H), (61, M, 1), 3.0) if with_delta else None
    hd = dev(h0)
    out = binding.quasar_rmsnorm(hd, dev(gamma), EPS, delta=dev_bf16(delta) if with_delta else None)
    torch.cuda.synchronize()
    h_exp = h0 + orc.bf16_to_f32(delta) if with_delta else h0  # binary32 add, as the kernel
    assert np.array_equal(host(hd), h_exp)
    _, ref = dec.rmsnorm(h_exp, gamma, EPS)
    assert_bf16_close(host_bf16(out), ref, 0.99, allow=(H + 8) * U * np.abs(ref))


@pytest.mark.parametrize("B,pos0", [(1, 0), (1, 1), (1, 100), (1, 2047), (16, 64), (8, 500)])
def test_qk_rope_cache(B, pos0):
    T = 6
    announce("qk_rope_cache", B, pos0)
    Lmax = pos0 + T + 3
    qkv = bf16_normal((B * T, (HQ + 2 * HKV) * D), (62, B, pos0), 2.0)
    g = synth.rng(62, B, pos0, 1)
    qg = g.uniform(0.5, 1.5, size=D).astype(np.float32)
    kg = g.uniform(0.5, 1.5, size=D).astype(np.float32)
    sentinel = np.full((B, HKV, Lmax, D), 0x3F80, np.uint16)  # 1.0 everywhere
    kc, vc = dev_bf16(sentinel), dev_bf16(sentinel)
    q = binding.quasar_qk_rope_cache(dev_bf16(qkv), dev(qg), dev(kg), kc, vc, B, HQ, pos0,
                                     rope_base=BASE, eps=EPS)
    torch.cuda.synchronize()
    qr, kr, vr = dec.qk_norm_rope(f32(qkv), qg, kg, B, T, HQ, HKV, D, pos0, BASE, EPS)
    heads = f32(qkv).reshape(B * T, HQ + 2 * HKV, D)
    q_allow = rope_allow(dec.head_rmsnorm(heads[:, :HQ], qg, EPS), D)
    k_allow = rope_allow(dec.head_rmsnorm(heads[:, HQ:HQ + HKV], kg, EPS), D)
    assert_bf16_close(host_bf16(q).reshape(B * T, HQ, D), qr, 0.95, q_allow)
    kh, vh = host_bf16(kc), host_bf16(vc)
    new = slice(pos0, pos0 + T)
    k_new = kh[:, :, new].transpose(0, 2, 1, 3).reshape(B * T, HKV, D)
    v_new = vh[:, :, new].transpose(0, 2, 1, 3).reshape(B * T, HKV, D)
    assert_bf16_close(k_new, kr, 0.95, k_allow)
    qkv_heads = qkv.reshape(B * T, HQ + 2 * HKV, D)
    assert np.array_equal(v_new, qkv_heads[:, HQ + HKV:])
    # every other cache position is untouched
    for c in (kh, vh):
        rest = np.delete(c, np.arange(pos0, pos0 + T), axis=2)
        assert np.all(rest == 0x3F80)


# T = 6: 24 query rows per KV head (the matrix-core kernel); T = 9 and 16: 36 and
# 64 rows (the vector-ALU kernel for groups wider than 32).  Batches whose chunk
# workgroups exceed ~1024 walk several chunks per workgroup: 8 x 1100 (2 per
# workgroup) and 16 x 2047 (5 per workgroup, the 96-token window at a 2048 context).
@pytest.mark.parametrize("B,pos0,T", [(1, 0, 6), (1, 63, 6), (1, 64, 6), (1, 1000, 6), (1, 2047, 6),
                                      (8, 200, 6), (16, 130, 6), (8, 1100, 6), (16, 2047, 6),
                                      (1, 100, 9), (2, 64, 16), (1, 0, 16)])
def test_attention(B, pos0, T):
    announce("attention", B, pos0, T)
    Lmax = pos0 + T + 5
    kc = bf16_normal((B, HKV, Lmax, D), (63, B, pos0, 0))
    vc = bf16_normal((B, HKV, Lmax, D), (63, B, pos0, 1))
    q = bf16_normal((B * T, HQ * D), (63, B, pos0, 2), 1.5)
    out = binding.quasar_attention(dev_bf16(q), dev_bf16(kc), dev_bf16(vc), HQ, pos0)
    torch.cuda.synchronize()
    qf = f32(q).reshape(B * T, HQ, D)
    ref = dec.attention(qf, f32(kc), f32(vc), B, T, HQ, pos0)
    allow = attention_allow(qf, f32(kc), f32(vc), B, T, HQ, pos0)
    assert_bf16_close(host_bf16(out).reshape(B * T, HQ, D), ref, 0.99, allow)


# other head groupings: one query head per KV head, eight per KV head, a one-token
# decode (T = 1), and group widths R = (Hq / Hkv) T of 1, 4, 32 (the widest the
# matrix-core kernel takes) and 40 (the vector-ALU kernel)
@pytest.mark.parametrize("Hq,Hkv,B,pos0,T", [(8, 8, 2, 100, 1), (8, 8, 1, 300, 4), (16, 2, 1, 95, 4),
                                             (32, 8, 3, 33, 1), (4, 4, 2, 40, 32), (16, 4, 1, 70, 8),
                                             (8, 1, 1, 200, 5)])
def test_attention_head_groupings(Hq, Hkv, B, pos0, T):
    announce("attention_groupings", Hq, Hkv, B, pos0, T)
    Lmax = pos0 + T + 2
    kc = bf16_normal((B, Hkv, Lmax, D), (66, Hq, Hkv, T, 0))
    vc = bf16_normal((B, Hkv, Lmax, D), (66, Hq, Hkv, T, 1))
    q = bf16_normal((B * T, Hq * D), (66, Hq, Hkv, T, 2), 1.5)
    out = binding.quasar_attention(dev_bf16(q), dev_bf16(kc), dev_bf16(vc), Hq, pos0)
    torch.cuda.synchronize()
    qf = f32(q).reshape(B * T, Hq, D)
    ref = dec.attention(qf, f32(kc), f32(vc), B, T, Hq, pos0)
    allow = attention_allow(qf, f32(kc), f32(vc), B, T, Hq, pos0)
    assert_bf16_close(host_bf16(out).reshape(B * T, Hq, D), ref, 0.99, allow)


def test_attention_repeated_calls_of_different_shapes():
    """Calls of different batch sizes and contexts in turn, each into a zeroed
    output and reusing the library's per-call state: a repeated call must give
    the same bits as the first, and each first call matches the oracle."""
    announce("attention_repeats")
    cases = [(1, 2047), (16, 130), (3, 700), (1, 2047), (16, 130)]
    seen = {}
    for B, pos0 in cases:
        T = 6
        Lmax = pos0 + T
        kc = bf16_normal((B, HKV, Lmax, D), (67, B, pos0, 0))
        vc = bf16_normal((B, HKV, Lmax, D), (67, B, pos0, 1))
        q = bf16_normal((B * T, HQ * D), (67, B, pos0, 2), 1.5)
        out = torch.zeros((B * T, HQ * D), dtype=torch.bfloat16, device="cuda")
        binding.quasar_attention(dev_bf16(q), dev_bf16(kc), dev_bf16(vc), HQ, pos0, out=out)
        torch.cuda.synchronize()
        got = host_bf16(out)
        if (B, pos0) in seen:
            assert np.array_equal(got, seen[(B, pos0)])
            continue
        seen[(B, pos0)] = got
        qf = f32(q).reshape(B * T, HQ, D)
        ref = dec.attention(qf, f32(kc), f32(vc), B, T, HQ, pos0)
        allow = attention_allow(qf, f32(kc), f32(vc), B, T, HQ, pos0)
        assert_bf16_close(got.reshape(B * T, HQ, D), ref, 0.99, allow)


def test_attention_ignores_positions_past_the_window():
    """Cache positions >= pos0 + T (not yet written in a real step) never
    reach the output: filling them with large values changes nothing."""
    B, T, pos0 = 2, 6, 70
    announce("attention_causal", B, pos0)
    Lmax = pos0 + T + 64
    kc = bf16_normal((B, HKV, Lmax, D), (64, 0))
    vc = bf16_normal((B, HKV, Lmax, D), (64, 1))
    q = bf16_normal((B * T, HQ * D), (64, 2))
    a = binding.quasar_attention(dev_bf16(q), dev_bf16(kc), dev_bf16(vc), HQ, pos0)
    kc[:, :, pos0 + T:] = 0x4700  # 32768.0
    vc[:, :, pos0 + T:] = 0xC700
    b = binding.quasar_attention(dev_bf16(q), dev_bf16(kc), dev_bf16(vc), HQ, pos0)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("M", [6, 96])
def test_silu_mul(M):
    announce("silu_mul", M)
    gu = bf16_normal((M, 2 * I), (65, M), 4.0)
    out = binding.quasar_silu_mul(dev_bf16(gu))
    torch.cuda.synchronize()
    ref = dec.silu_mul(f32(gu))
    assert_bf16_close(host_bf16(out), ref, 0.99, allow=8 * U * np.abs(ref))
