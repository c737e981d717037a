"""GPU parity on seeded random shapes, every element against the oracle.

40 (M, N, K) drawn once from a fixed seed: M from 1 to the 128-token limit
(every path: the one-launch kernel and the wide kernel's one- and four-tile
groups), K any multiple of 16 up to 16384, N from
1 to 70000; N*K <= 1.2e8 and M*N*K <= 2e9 keep the oracle within seconds.
The 4-bit path gets 15 shapes of its own (M <= 8, K a multiple of 128 up to
12288).
"""
import numpy as np
import pytest
import torch

from oracle import quasar_oracle as orc
from w8a8_quantized_speculative_amd import binding, synth
from tests.gpu_helpers import announce, dev, dev_bf16, host, host_bf16

pytestmark = pytest.mark.gpu


def _shapes(n=40, seed=2026):
    g = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(g.choice([1, 2, 3, 5, 6, 7, 8, 9, 12, 15, 16, 17, 24, 31, 33, 47, 48, 63, 64, 65,
                          96, 97, 127, 128]))
        K = min(16384, int(g.integers(1, 65)) * 16 * int(g.choice([1, 1, 2, 4])))
        N = int(g.choice([g.integers(1, 300), g.integers(300, 5000), g.integers(5000, 70000)]))
        if N * K > 1.2e8 or M * N * K > 2e9:
            continue
        out.append((M, N, K))
    return out


SHAPES = _shapes()


def _shapes_w4(n=15, seed=2027):
    g = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(g.integers(1, 9))
        K = 128 * int(g.integers(1, 97))
        N = int(g.choice([g.integers(1, 300), g.integers(300, 5000), g.integers(5000, 40000)]))
        if N * K > 1.2e8:
            continue
        out.append((M, N, K))
    return out


SHAPES_W4 = _shapes_w4()


def _shapes_w4_wide(n=10, seed=2028):
    """Random windows of 9 to 96 tokens for the wide kernel's 4-bit path."""
    g = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(g.integers(9, 97))
        K = 128 * int(g.integers(1, 97))
        N = int(g.choice([g.integers(1, 300), g.integers(300, 5000), g.integers(5000, 40000)]))
        if N * K > 1.2e8:
            continue
        out.append((M, N, K))
    return out


SHAPES_W4_WIDE = _shapes_w4_wide()


@pytest.mark.parametrize("i", range(len(SHAPES)), ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
def test_random_shape_every_element(i):
    M, N, K = SHAPES[i]
    announce("random_shape", i, M, N, K)
    x, w, s = synth.linear_case(M, K, N, (60, i))
    xd, sd, wd = dev_bf16(x), dev(s), dev_bf16(w)
    wq, sw = binding.quasar_quantize_weights(wd, sd)
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y = binding.quasar_w8a8_linear(xd, sd, wq, sw, acc_out=acc)
    torch.cuda.synchronize()
    ref = orc.w8a8_linear_rows(x, s, w)
    assert np.array_equal(host(acc), ref["acc"].astype(np.int32))
    assert np.array_equal(host_bf16(y), ref["y"])


@pytest.mark.parametrize("i", range(len(SHAPES_W4)), ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES_W4])
def test_random_shape_w4_every_element(i):
    M, N, K = SHAPES_W4[i]
    announce("random_shape_w4", i, M, N, K)
    x, w, s = synth.linear_case(M, K, N, (61, i))
    wq4, sw4 = binding.quasar_quantize_weights_w4(dev_bf16(w), dev(s))
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y = binding.quasar_w4a8_linear(dev_bf16(x), dev(s), wq4, sw4, acc_out=acc)
    torch.cuda.synchronize()
    ref = orc.w4a8_linear_rows(x, s, w)
    assert np.array_equal(host(acc), ref["acc"].astype(np.int32))
    assert np.array_equal(host_bf16(y), ref["y"])


@pytest.mark.parametrize("i", range(len(SHAPES_W4_WIDE)),
                         ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES_W4_WIDE])
def test_random_shape_w4_wide_every_element(i):
    M, N, K = SHAPES_W4_WIDE[i]
    announce("random_shape_w4_wide", i, M, N, K)
    x, w, s = synth.linear_case(M, K, N, (62, i))
    wq4, sw4 = binding.quasar_quantize_weights_w4(dev_bf16(w), dev(s))
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y = binding.quasar_w4a8_linear(dev_bf16(x), dev(s), wq4, sw4, acc_out=acc)
    torch.cuda.synchronize()
    ref = orc.w4a8_linear_rows(x, s, w)
    assert np.array_equal(host(acc), ref["acc"].astype(np.int32))
    assert np.array_equal(host_bf16(y), ref["y"])
