"""GPU parity of the 4-bit weight variant against the oracle.

The oracle's reading (quantize_weights_w4): the INT8 weight rule at qmax = 7,
i.e. smoothed weights, one symmetric scale per output channel, codes in
[-7, 7]; dynamic per-token INT8 activations; exact integer accumulation;
the same dequant.  The bar is the INT8 path's: codes, scales and INT32
accumulators bit-identical, BF16 outputs bit-identical to the oracle's
rounding of the same binary32 operations.
"""
import numpy as np
import pytest
import torch

from oracle import quasar_oracle as orc
from w8a8_quantized_speculative_amd import binding, synth
from tests.gpu_helpers import (announce, dev, dev_bf16, f32_bits, host, host_bf16,
                               unpack_weights_w4)

pytestmark = pytest.mark.gpu


def run_gpu(x, s, w):
    wq, sw = binding.quasar_quantize_weights_w4(dev_bf16(w), dev(s))
    acc = torch.empty((x.shape[0], w.shape[0]), dtype=torch.int32, device="cuda")
    y = binding.quasar_w4a8_linear(dev_bf16(x), dev(s), wq, sw, acc_out=acc)
    torch.cuda.synchronize()
    return host_bf16(y), host(acc), wq, sw


@pytest.mark.parametrize("N,K", [(37, 128), (1000, 1024), (16, 12288), (300, 4096)])
def test_w4_weight_codes_and_scales(N, K):
    announce("w4_weights", N, K)
    _, w, s = synth.linear_case(1, K, N, (50, N, K))
    wq, sw = binding.quasar_quantize_weights_w4(dev_bf16(w), dev(s))
    torch.cuda.synchronize()
    q_ref, sw_ref = orc.quantize_weights_w4(w, s)
    full = unpack_weights_w4(wq, N, K, keep_padding=True)
    assert np.array_equal(full[:N], q_ref)
    assert not np.any(full[N:])                          # rows past N of the last tile
    assert np.array_equal(f32_bits(host(sw)), f32_bits(sw_ref))
    assert np.abs(full).max() <= 7


# every token-row variant (2/4/6/8), every K variant (1/2/3 phases), ragged N,
# 1/16 to 35 tiles per workgroup
SHAPES = [
    (1, 16, 128), (6, 1000, 1024), (6, 4096, 256), (2, 7, 384), (8, 300, 4096), (3, 40, 6144),
    (7, 100, 8064), (8, 64, 10112), (4, 520, 12288), (6, 9000, 1024), (5, 33, 12288),
    (6, 16400, 512), (1, 143000, 128),
    # K past 8192 with three 4-bit buffers: 2 and 3 tiles per workgroup, ragged N
    (6, 9000, 12288), (3, 5000, 9216), (8, 4100, 12288),
    # wide windows (and K > 12288): the wide kernel with 4-bit weight blocks --
    # every token-block count it takes (1..6), an odd number of chunk pairs
    # (a last item with fewer than 4 pairs), single tiles, tile pairs (K > 8192;
    # more tiles than workgroups past 64 tokens, odd tile count) and groups of
    # 4 split across workgroups, empty ranges
    (9, 100, 1024), (20, 64, 4096), (33, 1000, 2176), (48, 520, 4096), (64, 260, 1152),
    (80, 300, 4096), (96, 77, 3072), (96, 520, 12288), (40, 8000, 512), (24, 6144, 4096),
    (96, 6152, 4096), (72, 4104, 2048), (6, 64, 16384), (50, 48, 20480), (20, 16400, 384),
    (96, 16384, 1024), (9, 16390, 4224), (17, 500, 65536),
    # token blocks split over two workgroups (3 + 3 blocks with a ragged last
    # one, 2 + 2), ragged N, K past 8192 with 256 tiles
    (90, 4090, 4096), (64, 3072, 8192), (96, 4096, 12288),
    # groups of 3 tiles split over two workgroups
    (96, 6100, 2048), (90, 6130, 4224),
    # groups of 6 tiles (3 to 5 token blocks): one per workgroup and split
    (48, 20000, 512), (80, 17000, 1152), (40, 30000, 256), (16, 17000, 512), (30, 20000, 1152),
    (96, 24576, 1024),
    # a tile group's K over many workgroups: empty ranges and 63 contributors,
    # more than 64 contributors, 96 tokens
    (16, 16, 16384), (20, 48, 20480), (96, 64, 4096),
]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_w4_linear_every_element(M, N, K):
    announce("w4_linear", M, N, K)
    x, w, s = synth.linear_case(M, K, N, (51, M, N, K))
    y, acc, _, _ = run_gpu(x, s, w)
    ref = orc.w4a8_linear_rows(x, s, w)
    assert np.array_equal(acc, ref["acc"].astype(np.int32))
    assert np.array_equal(y, ref["y"])


def test_w4_zero_rows_and_extreme_codes():
    """An all-zero activation row, an all-zero weight row, and weight rows whose
    codes hit both ends of [-7, 7] on every position."""
    M, N, K = 6, 48, 512
    announce("w4_extremes", M, N, K)
    x, w, s = synth.linear_case(M, K, N, (52, 0))
    x[2] = 0
    w[5] = 0
    v = orc.bf16_to_f32(w)
    v[9] = np.where(np.arange(K) % 2 == 0, 1.0, -1.0).astype(np.float32) * s   # w' ~ +-1: codes +-7
    w = synth.to_bf16_bits(v)
    y, acc, wq, _ = run_gpu(x, s, w)
    ref = orc.w4a8_linear_rows(x, s, w)
    assert np.array_equal(acc, ref["acc"].astype(np.int32)) and np.array_equal(y, ref["y"])
    assert not np.any(acc[2]) and not np.any(acc[:, 5])
    assert np.abs(unpack_weights_w4(wq, N, K)[9]).min() >= 6


@pytest.mark.parametrize("M", [6, 48, 96])
@pytest.mark.parametrize("name,K,N", synth.QWEN3_8B_LINEARS + (synth.QWEN3_8B_LM_HEAD,))
def test_w4_qwen3_shapes_sampled(name, K, N, M):
    """The Qwen3-8B-shaped layer linears and the LM head at M = 6, 48 and 96:
    every output of sampled channels (the oracle quantizes just those rows)."""
    announce("w4_qwen3", name, M, N, K)
    key = (53, ["qkv", "o", "gate_up", "down", "lm_head"].index(name))
    x = synth.activations(M, K, key)
    g = torch.Generator(device="cuda")
    g.manual_seed(53 + N)
    w = (torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    s = synth.smoothing_vector(synth.col_absmax_bf16(x),
                               w.float().abs().amax(dim=0).cpu().numpy().astype(np.float64))
    wq, sw = binding.quasar_quantize_weights_w4(w, dev(s))
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y = binding.quasar_w4a8_linear(dev_bf16(x), dev(s), wq, sw, acc_out=acc)
    torch.cuda.synchronize()
    rng = np.random.default_rng(N)
    cols = np.unique(np.concatenate([np.arange(32), np.arange(N - 32, N),
                                     rng.choice(N, 256, replace=False)]))
    w_rows = host_bf16(w[torch.from_numpy(cols).cuda()])
    ref = orc.w4a8_linear_rows(x, s, w_rows)
    assert np.array_equal(host(acc)[:, cols], ref["acc"].astype(np.int32))
    assert np.array_equal(host_bf16(y)[:, cols], ref["y"])
    assert np.array_equal(unpack_weights_w4(wq, N, K)[cols], ref["qw"])


def test_w4_repeated_calls_are_bit_identical():
    M, N, K = 6, 6144, 4096
    announce("w4_repeat", M, N, K)
    x, w, s = synth.linear_case(M, K, N, (54, 0))
    wq, sw = binding.quasar_quantize_weights_w4(dev_bf16(w), dev(s))
    xd, sd = dev_bf16(x), dev(s)
    first = binding.quasar_w4a8_linear(xd, sd, wq, sw).clone()
    for _ in range(30):
        assert torch.equal(binding.quasar_w4a8_linear(xd, sd, wq, sw).view(torch.int16),
                           first.view(torch.int16))
    assert np.array_equal(host_bf16(first), orc.w4a8_linear_rows(x, s, w)["y"])
