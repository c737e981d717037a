"""GPU parity on seeded random shapes, every element against the oracle.

40 (M, N, K) drawn once from a fixed seed: M from 1 to the 128-token limit
(every path: the one-launch kernel and the wide kernel's one- and four-tile
groups), K any multiple of 16 up to 16384, N from
1 to 70000; N*K <= 1.2e8 and M*N*K <= 2e9 keep the oracle within seconds.
The 4-bit path gets 15 shapes of its own (M <= 8, K a multiple of 128 up to
12288).  A third set of 16 aims at the wide kernel's token-block split and its
groups of 6 tiles (49 to 128 tokens), each also through the 4-bit path where
M <= 96 and K is a multiple of 128.
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


def _shapes_plans(n=16, seed=2029):
    """Random windows aimed at the wide kernel's later plans: the token-block
    split (an even block count from 64 tokens, up to 384 tiles in a multiple
    of 8 pairs or triples) and the groups of 6 tiles (beyond 1024 tiles).
    The plan each shape takes is whatever the library picks; the pairs and
    triples are made likely by drawing N near multiples of 256 and 384
    channels."""
    g = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(g.choice([49, 64, 70, 80, 90, 96, 100, 112, 128]))
        kind = int(g.integers(0, 3))
        if kind == 0:
            N = 256 * int(g.integers(1, 17)) - int(g.integers(0, 16))
        elif kind == 1:
            N = 6144 - 384 * int(g.integers(0, 3)) - int(g.integers(0, 16))
        else:
            N = int(g.integers(16400, 40000))
        K = 16 * int(g.integers(1, 513)) if kind < 2 else 16 * int(g.integers(1, 65))
        if N * K > 1.2e8 or M * N * K > 2e9:
            continue
        out.append((M, N, K))
    return out


SHAPES_PLANS = _shapes_plans()


def test_plan_shapes_reach_the_later_plans():
    """The seeded plan shapes keep covering the split and 6-tile kernels."""
    L = binding.lib()
    names = [L.quasar_w8a8_kernel_name(M, N, K).decode() for M, N, K in SHAPES_PLANS]
    assert sum("split_kernel" in n for n in names) >= 3, names
    assert sum(n.endswith(", 6>") for n in names) >= 3, names


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


@pytest.mark.parametrize("i", range(len(SHAPES_PLANS)),
                         ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES_PLANS])
def test_random_plan_shape_every_element(i):
    M, N, K = SHAPES_PLANS[i]
    announce("random_plan_shape", i, M, N, K)
    x, w, s = synth.linear_case(M, K, N, (63, i))
    xd, sd, wd = dev_bf16(x), dev(s), dev_bf16(w)
    wq, sw = binding.quasar_quantize_weights(wd, sd)
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y = binding.quasar_w8a8_linear(xd, sd, wq, sw, acc_out=acc)
    ref = orc.w8a8_linear_rows(x, s, w)
    torch.cuda.synchronize()
    assert np.array_equal(host(acc), ref["acc"].astype(np.int32))
    assert np.array_equal(host_bf16(y), ref["y"])
    if M <= 96 and K % 128 == 0:
        wq4, sw4 = binding.quasar_quantize_weights_w4(wd, sd)
        acc4 = torch.empty((M, N), dtype=torch.int32, device="cuda")
        y4 = binding.quasar_w4a8_linear(xd, sd, wq4, sw4, acc_out=acc4)
        torch.cuda.synchronize()
        ref4 = orc.w4a8_linear_rows(x, s, w)
        assert np.array_equal(host(acc4), ref4["acc"].astype(np.int32))
        assert np.array_equal(host_bf16(y4), ref4["y"])
