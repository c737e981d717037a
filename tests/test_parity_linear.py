"""GPU parity of the W8A8 verify linear against the oracle.

Small and ragged shapes are checked on every element; the Qwen3-8B-shaped
linears and the LM head at full size (the shapes the benchmark times, in the
same launch configuration) are checked on sampled output channels, which the
oracle quantizes and multiplies row by row exactly as inside the full matrix.
The bar: INT32 accumulators and INT8-derived BF16 outputs bit-identical to the
oracle, and every output within 1 bf16 ulp of acc * sx * sw taken in float64.
"""
import functools

import numpy as np
import pytest
import torch

from oracle import quasar_oracle as orc
from w8a8_quantized_speculative_amd import binding, synth
from tests.gpu_helpers import announce, dev, dev_bf16, host, host_bf16, unpack_weights

pytestmark = pytest.mark.gpu


def run_gpu(x, s, w):
    wq, sw = binding.quasar_quantize_weights(dev_bf16(w), dev(s))
    xd = dev_bf16(x)
    acc = torch.empty((x.shape[0], w.shape[0]), dtype=torch.int32, device="cuda")
    y = binding.quasar_w8a8_linear(xd, dev(s), wq, sw, acc_out=acc)
    torch.cuda.synchronize()
    return host_bf16(y), host(acc), wq, sw


def check_against_oracle(x, s, w, y, acc, cols=None):
    if cols is None:
        cols = np.arange(w.shape[0])
        ref = orc.w8a8_linear_rows(x, s, w)
    else:
        ref = orc.w8a8_linear_rows(x, s, w[cols] if w.shape[0] > len(cols) else w)
    assert np.array_equal(acc[:, cols], ref["acc"].astype(np.int32))
    assert np.array_equal(y[:, cols], ref["y"])
    exact = orc.dequantize_f64(ref["acc"], ref["sx"], ref["sw"])
    got = orc.bf16_to_f32(y[:, cols]).astype(np.float64)
    nz = exact != 0
    ulp = np.zeros_like(exact)
    ulp[nz] = 2.0 ** (np.floor(np.log2(np.abs(exact[nz]))) - 7)
    assert np.all(np.abs(got - exact) <= ulp)
    return ref


def test_single_linear_1024_m6_every_element():
    """One W8A8 linear, M = 6 (1 sequence x 1+5 drafts), K = N = 1024, four
    outlier channels x50, W ~ N(0, 0.02)."""
    announce("linear", 6, 1024, 1024)
    x, w, s = synth.linear_case(6, 1024, 1024, (0, 0), n_outliers=4, fixed_scale=50.0)
    y, acc, _, _ = run_gpu(x, s, w)
    check_against_oracle(x, s, w, y, acc)


RAGGED = [
    (1, 16, 16), (6, 1000, 1040), (16, 257, 4096), (17, 300, 1024), (48, 513, 2048),
    (96, 129, 4096), (128, 64, 512), (5, 33, 12288), (2, 7, 3072), (6, 4096, 192),
    # one-launch kernel: every token-row variant (2, 4, 6, 8) and every K variant
    # (<= 4096, <= 8192, <= 12288), with ragged N and partial last streamer ranges
    (4, 48, 4096), (8, 300, 4096), (3, 40, 6144), (7, 100, 8000), (8, 64, 10000),
    (4, 520, 12288),
    # K just past each variant's range start (a last phase nearly all zero
    # padding) and just past one 2048-wide phase; QKV at 8 token rows
    (6, 300, 4112), (7, 500, 8208), (2, 1000, 2064), (8, 6144, 4096),
    # many tiles per compute unit: uneven contiguous tile ranges per workgroup
    (6, 9000, 1024), (2, 8336, 80), (8, 12000, 256),
    # 1.5 tiles per workgroup (QKV-like), one more tile for the first
    # workgroups and a last tile half past N, one tile per workgroup
    (6, 6144, 512), (6, 6152, 512), (5, 24, 64), (3, 4104, 1024),
    # 4 to 16 tiles per workgroup, ragged N, every K variant
    (6, 16400, 512), (3, 20008, 1040), (8, 40000, 128), (1, 65536, 64), (4, 16400, 8000),
    (6, 16400, 12288),
    # wide windows: every 16-token block count (1..8), ragged N and K, groups
    # shared by several workgroups (partial sums), and ranges that are empty
    (9, 100, 1024), (20, 64, 4096), (33, 1000, 2112), (64, 520, 4096), (80, 260, 1040),
    (112, 77, 3072), (128, 300, 4096), (16, 64, 4096), (40, 8000, 512), (24, 6144, 4096),
    # one-tile groups over a 96 x 12288 code matrix; groups of 4 just past it
    (96, 520, 12288), (128, 300, 12288),
    # K beyond the one-launch small-window kernel, up to the largest supported K
    (6, 64, 16384), (1, 40, 65536), (50, 48, 20480),
    # a tile group's K over many workgroups, all their flags waited for at once:
    # fewer items than workgroups (empty ranges, 63 contributors), more than 64
    # contributors (two rounds of lanes), 96 and 33 tokens
    (16, 16, 16384), (20, 48, 20480), (96, 64, 4096), (33, 100, 8192),
    # 4 to 5 tiles per workgroup: groups of 4 tiles split across workgroups
    (20, 16400, 320), (100, 16384, 1040), (128, 16500, 2112), (9, 16390, 4160),
    (70, 20000, 576),
    # pairs of tiles per group in the wide kernel: K past 8192 (ragged N and K),
    # and more tiles than workgroups at more than 64 tokens (an odd tile count:
    # the last group holds one tile)
    (20, 1000, 8208), (90, 200, 10000), (96, 6152, 4096), (72, 4104, 2048),
    # at least 16 tiles per workgroup (groups of 4 tiles): every token-block
    # count, ragged N and K (odd chunk counts), groups split across workgroups
    (9, 65600, 320), (20, 66000, 208), (48, 70000, 208), (33, 66000, 96), (64, 65540, 576),
    (70, 65600, 1040), (96, 65600, 64), (100, 65536, 192), (128, 66000, 320),
    # token blocks split over two workgroups of one XCD (one pair of tiles per
    # range): 2 + 2, 3 + 3 (a ragged last block) and 4 + 4 blocks, ragged N,
    # 32 to 128 pairs, K up to 8192; 256 tiles at K > 8192; more codes than
    # 96 x 12288
    (64, 2048, 4096), (90, 4090, 4096), (128, 2040, 4096), (64, 3072, 8192), (96, 1530, 2112),
    (96, 4096, 12288), (128, 2048, 12288), (128, 2048, 16384),
    # the split with groups of 3 tiles (up to 384 tiles): ragged M, N and K
    (90, 6130, 4224), (128, 6100, 1024), (64, 6144, 2048),
    # groups of 6 tiles (beyond 4 tiles per CU, 3 to 6 token blocks): one
    # group per workgroup, and groups split across workgroups (partial sums
    # of 6 tiles), ragged N and K
    (70, 17000, 1040), (48, 20000, 512), (96, 30000, 256), (64, 16400, 2112), (81, 24576, 4160),
    (32, 17000, 1040), (20, 24576, 512),
]


@pytest.mark.parametrize("M,N,K", RAGGED)
@pytest.mark.parametrize("literal", [False, True])
def test_linear_ragged_every_element(M, N, K, literal):
    announce("linear", M, N, K, "literal" if literal else "smoothing")
    x, w, s = synth.linear_case(M, K, N, (1, M, N, K), literal=literal)
    y, acc, _, _ = run_gpu(x, s, w)
    check_against_oracle(x, s, w, y, acc)


def test_zero_rows_and_channels():
    announce("linear_zero_rows", 6, 200, 256)
    x, w, s = synth.linear_case(6, 256, 200, (2, 0))
    x[3] = 0
    w[17] = 0
    y, acc, _, _ = run_gpu(x, s, w)
    check_against_oracle(x, s, w, y, acc)
    assert not np.any(acc[3]) and not np.any(orc.bf16_to_f32(y[3]))
    assert not np.any(acc[:, 17])


def test_empty_linear_is_a_noop():
    announce("linear_empty")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    s = torch.ones(64, dtype=torch.float32, device="cuda")
    wq, sw = binding.quasar_quantize_weights(torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda"), s)
    y = binding.quasar_w8a8_linear(x, s, wq, sw)
    torch.cuda.synchronize()
    assert y.shape == (0, 8)


@functools.lru_cache(maxsize=4)
def qwen3_weights(N, K, key):
    w = synth.weights(N, K, key)
    return w, synth.col_absmax_bf16(w)


def sampled_cols(N, n_random, seed):
    g = np.random.default_rng(seed)
    cols = np.concatenate([np.arange(min(32, N)), np.arange(max(0, N - 32), N),
                           g.choice(N, size=min(n_random, N), replace=False)])
    return np.unique(cols)


@pytest.mark.parametrize("M", [6, 48, 96])
@pytest.mark.parametrize("name,K,N", synth.QWEN3_8B_LINEARS)
def test_qwen3_layer_linear_full_size_sampled(name, K, N, M):
    """Qwen3-8B layer linears at the verify window (M = 6, 48, 96), 0.1 %
    outlier channels x U[30, 100]; sampled channels checked exactly."""
    announce("qwen3_linear", name, M, N, K)
    key = (1, 0, ["qkv", "o", "gate_up", "down"].index(name))
    x = synth.activations(M, K, key)
    w, w_colmax = qwen3_weights(N, K, key)
    s = synth.smoothing_vector(synth.col_absmax_bf16(x), w_colmax)
    y, acc, wq, sw = run_gpu(x, s, w)
    cols = sampled_cols(N, 256, N + M)
    ref = check_against_oracle(x, s, w, y, acc, cols)
    assert np.array_equal(unpack_weights(wq, N, K)[cols], ref["qw"])


# One GPU's share of each Qwen3-8B linear under 8-way tensor parallelism:
# column-parallel QKV, gate_up and LM head (N / 8), row-parallel O and down
# (K / 8).  (name, K, N)
TP8_SHARDS = [("qkv/8", 4096, 768), ("o/8", 512, 4096), ("gate_up/8", 4096, 3072),
              ("down/8", 1536, 4096), ("lm_head/8", 4096, 18992)]


@pytest.mark.parametrize("M", [1, 6, 8, 48, 96])
@pytest.mark.parametrize("name,K,N", TP8_SHARDS)
def test_tp8_shard_shapes_every_element(name, K, N, M):
    """The 8-way tensor-parallel shard shapes, every output element (the
    shard's weights are a slice of the full layer's: any slice must match)."""
    announce("tp8_shard", name, M, N, K)
    key = (8, ["qkv/8", "o/8", "gate_up/8", "down/8", "lm_head/8"].index(name))
    x = synth.activations(M, K, key)
    w = synth.weights(N, K, key)
    s = synth.smoothing_vector(synth.col_absmax_bf16(x), synth.col_absmax_bf16(w))
    y, acc, _, _ = run_gpu(x, s, w)
    check_against_oracle(x, s, w, y, acc)


@pytest.mark.parametrize("M", [6, 48, 96, 128])
def test_lm_head_full_size_sampled(M):
    """W8A8 LM head 4096 -> 151936 at the verify window M = 6, 48, 96, 128."""
    K, N = 4096, synth.QWEN3_8B_VOCAB
    announce("lm_head", M, N, K)
    key = (3, 0, 0)
    x = synth.activations(M, K, key)
    w = synth.weights(N, K, key)
    s = synth.smoothing_vector(synth.col_absmax_bf16(x), synth.col_absmax_bf16(w))
    y, acc, _, _ = run_gpu(x, s, w)
    cols = sampled_cols(N, 512, 7)
    check_against_oracle(x, s, w, y, acc, cols)


@pytest.mark.parametrize("M,N,K", [(5, 33, 12288), (96, 300, 4096), (48, 6144, 4096),
                                   (40, 17000, 1040), (96, 66000, 128), (6, 16400, 256)])
def test_repeated_calls_are_bit_identical(M, N, K):
    """Partial sums shared between workgroups and LDS reductions are integer
    sums, and every launch of the wide kernel waits for its own token rows:
    no run-to-run drift, including back-to-back launches on one workspace."""
    announce("linear_determinism", M, N, K)
    x, w, s = synth.linear_case(M, K, N, (4, M))
    wq, sw = binding.quasar_quantize_weights(dev_bf16(w), dev(s))
    xd, sd = dev_bf16(x), dev(s)
    ws = binding.new_workspace(binding.workspace_bytes_linear(M, N, K))
    first = binding.quasar_w8a8_linear(xd, sd, wq, sw, workspace=ws).clone()
    for _ in range(50):
        again = binding.quasar_w8a8_linear(xd, sd, wq, sw, workspace=ws)
        assert torch.equal(again.view(torch.int16), first.view(torch.int16))
    y = host_bf16(first)
    ref = orc.w8a8_linear_rows(x, s, w)
    assert np.array_equal(y, ref["y"])


def test_alternating_inputs_on_one_workspace():
    """Back-to-back launches on one workspace with two different inputs of the
    same shape: every launch must read the token rows and partial sums of its
    own input, never those a previous launch left at the same addresses."""
    M, N, K = 96, 700, 4096
    ws = binding.new_workspace(binding.workspace_bytes_linear(M, N, K))
    sets = []
    for i in range(2):
        x, w, s = synth.linear_case(M, K, N, (6, i))
        wq, sw = binding.quasar_quantize_weights(dev_bf16(w), dev(s))
        sets.append((x, s, w, dev_bf16(x), dev(s), wq, sw))
    announce("linear_alternating", M, N, K)
    outs = []
    for r in range(20):
        x, s, w, xd, sd, wq, sw = sets[r % 2]
        outs.append(binding.quasar_w8a8_linear(xd, sd, wq, sw, workspace=ws))
    torch.cuda.synchronize()
    refs = [orc.w8a8_linear_rows(x, s, w)["y"] for x, s, w, *_ in sets]
    for r, y in enumerate(outs):
        assert np.array_equal(host_bf16(y), refs[r % 2]), f"launch {r}"


def test_interleaved_wide_shapes_on_one_stream():
    """Wide launches of different token-block counts and shapes, back to back
    with no synchronisation between them, each against the oracle; a second
    round with new activations checks that no launch reads the rows of the
    one before it."""
    cases = [(48, 500, 4096), (96, 130, 2048), (17, 2000, 1024), (128, 64, 4096), (9, 40, 12288),
             (40, 17000, 1024), (64, 66000, 64), (5, 20000, 512), (6, 66000, 64)]
    for rnd in range(2):
        outs = []
        for i, (M, N, K) in enumerate(cases):
            announce("linear_interleaved", rnd, M, N, K)
            x, w, s = synth.linear_case(M, K, N, (5, rnd, i))
            wq, sw = binding.quasar_quantize_weights(dev_bf16(w), dev(s))
            acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
            y = binding.quasar_w8a8_linear(dev_bf16(x), dev(s), wq, sw, acc_out=acc)
            outs.append((x, s, w, y, acc))
        torch.cuda.synchronize()
        for x, s, w, y, acc in outs:
            check_against_oracle(x, s, w, host_bf16(y), host(acc))

