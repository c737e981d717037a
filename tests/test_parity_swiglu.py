"""GPU parity of the gate_up linear with the gated MLP's activation applied in
its epilogue (quasar_quantize_weights_gated + quasar_w8a8_linear_swiglu).

Three checks per shape:
  * the gated pack quantizes every row exactly as the plain pack: its weight
    scales are the plain ones permuted into the gated order, bit for bit;
  * the fused result equals the unfused pair (quasar_w8a8_linear on the
    [gate | up] rows, then quasar_silu_mul) bit for bit;
  * against the oracles: the linear's BF16 product bit-exact (the float64
    oracle of the W8A8 linear), and silu(gate) * up of that product to the
    SiLU bar of the decoder tests (one BF16 spacing + 8 2^-24 |y|).
Windows of 1, 6 and 8 tokens run in the one-launch kernel (its epilogue applies
the activation); 12 and 48 tokens run the wide kernel, then the gated SiLU kernel.
"""
import numpy as np
import pytest
import torch

from oracle import decoder_oracle as dec
from oracle import quasar_oracle as orc
from w8a8_quantized_speculative_amd import binding, synth
from tests.gpu_helpers import announce, dev, dev_bf16, host, host_bf16
from tests.test_parity_decoder import U, assert_bf16_close

pytestmark = pytest.mark.gpu


def gated_order(I):
    """Source row of each packed row in the gated order."""
    r = np.arange(2 * I)
    t, i = r // 16, r % 16
    return np.where(i < 8, 8 * t + i, I + 8 * t + (i - 8))


@pytest.mark.parametrize("M,I,K", [(6, 12288, 4096), (1, 1024, 512), (8, 520, 1024),
                                   (12, 1024, 512), (48, 2048, 1024)])
def test_swiglu_linear(M, I, K):
    announce("swiglu", M, I, K)
    N = 2 * I
    key = (80, M, I, K)
    w = synth.weights(N, K, key)
    x = synth.activations(M, K, key + (1,))
    s = synth.smoothing_vector(synth.col_absmax_bf16(synth.activations(64, K, key + (2,))),
                               synth.col_absmax_bf16(w))
    wd, sd, xd = dev_bf16(w), dev(s), dev_bf16(x)
    wq, sw = binding.quasar_quantize_weights(wd, sd)
    wqg, swg = binding.quasar_quantize_weights_gated(wd, sd)
    y = binding.quasar_w8a8_linear(xd, sd, wq, sw)
    act_pair = binding.quasar_silu_mul(y)
    act = binding.quasar_w8a8_linear_swiglu(xd, sd, wqg, swg)
    torch.cuda.synchronize()
    assert np.array_equal(host(swg).view(np.uint32), host(sw).view(np.uint32)[gated_order(I)])
    got = host_bf16(act)
    assert np.array_equal(got, host_bf16(act_pair))
    # oracles: the product over a sample of output pairs (every column at small N)
    cols = np.arange(I) if I <= 2048 else np.sort(
        np.random.default_rng(list(key)).choice(I, size=512, replace=False))
    rows = np.concatenate([cols, I + cols])
    ref = orc.w8a8_linear_rows(x, s, w[rows])
    assert np.array_equal(host_bf16(y)[:, rows], ref["y"])
    yf = orc.bf16_to_f32(ref["y"]).astype(np.float64)
    a_ref = dec.silu_mul(yf)
    assert_bf16_close(got[:, cols], a_ref, 0.99, 8 * U * np.abs(a_ref))


def test_swiglu_rejects_bad_widths():
    x = torch.zeros((6, 512), dtype=torch.bfloat16, device="cuda")
    s = torch.ones(512, dtype=torch.float32, device="cuda")
    w = torch.zeros((40, 512), dtype=torch.bfloat16, device="cuda")  # 40 % 16 != 0
    with pytest.raises(binding.QuasarError):
        binding.quasar_quantize_weights_gated(w, s)
