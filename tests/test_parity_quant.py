"""GPU parity of the two quantizers against the oracle: bit-exact INT8 codes,
bit-exact binary32 scales and bit-exact smoothed activations."""
import numpy as np
import pytest
import torch

from oracle import quasar_oracle as orc
from w8a8_quantized_speculative_amd import binding, synth
from tests.gpu_helpers import announce, dev, dev_bf16, f32_bits, host, unpack_weights

pytestmark = pytest.mark.gpu

ACT_SHAPES = [(6, 1024), (1, 16), (7, 1040), (17, 4096), (96, 4096), (6, 12288), (3, 20000),
              (128, 2048)]


@pytest.mark.parametrize("M,K", ACT_SHAPES)
def test_quantize_activations_bit_exact(M, K):
    announce("quantize_activations", M, K)
    x = synth.activations(M, K, (10, M, K), n_outliers=max(1, K // 1000))
    if M > 2:
        x[1] = 0                      # all-zero token row
    w_cm = np.full(K, 0.05)
    s = synth.smoothing_vector(synth.col_absmax_bf16(x), w_cm)
    qx, sx, xs = binding.quasar_quantize_activations(dev_bf16(x), dev(s), want_xs=True)
    torch.cuda.synchronize()
    q_ref, sx_ref, xs_ref = orc.quantize_activations(x, s)
    assert np.array_equal(host(qx), q_ref)
    assert np.array_equal(f32_bits(host(sx)), f32_bits(sx_ref))
    assert np.array_equal(f32_bits(host(xs)), f32_bits(xs_ref))
    # the fp32 smoothed path is within 1e-6 relative of the exact product
    exact = orc.bf16_to_f32(x).astype(np.float64) * s.astype(np.float64)[None, :]
    got = host(xs).astype(np.float64)
    assert np.all(np.abs(got - exact) <= 1e-6 * np.abs(exact))


W_SHAPES = [(1024, 1024), (37, 80), (100, 4096), (64, 12288), (5, 65536), (2, 16), (17, 1040)]


@pytest.mark.parametrize("N,K", W_SHAPES)
def test_quantize_weights_bit_exact(N, K):
    announce("quantize_weights", N, K)
    w = synth.weights(N, K, (11, N, K))
    if N > 3:
        w[2] = 0                      # all-zero output channel
    g = np.random.default_rng(N + K)
    s = np.exp(g.uniform(np.log(0.05), np.log(20), K)).astype(np.float32)
    wq, sw = binding.quasar_quantize_weights(dev_bf16(w), dev(s))
    torch.cuda.synchronize()
    q_ref, sw_ref = orc.quantize_weights(w, s)
    full = unpack_weights(wq, N, K, keep_padding=True)
    assert np.array_equal(full[:N, :K], q_ref)
    assert not np.any(full[N:]) and not np.any(full[:, K:])   # zero padding
    assert np.array_equal(f32_bits(host(sw)), f32_bits(sw_ref))


def test_quantize_empty_is_a_noop():
    announce("quantize_empty")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    s = torch.ones(64, dtype=torch.float32, device="cuda")
    qx, sx, _ = binding.quasar_quantize_activations(x, s)
    wq, sw = binding.quasar_quantize_weights(x, s)
    torch.cuda.synchronize()
    assert qx.shape == (0, 64) and wq.N == 0 and sw.shape == (0,)
