"""GPU parity of quasar_lm_head_verify: the W8A8 LM head and the accept step
in one call.

The expected results are the oracle's: its LM head logits (bit-exact BF16)
and its greedy or rejection decisions on those logits.  Greedy decisions and
argmax are exact; rejection decisions are compared under the precision band of
the accept tests (the sums of exp are binary32 here and float64 there).  Shapes
cover the fused path (M <= 8: the LM head's own epilogue reduces each
workgroup's channel range) with 1 to 16 channels tiles per workgroup and a
ragged last tile, and every fallback (M > 8, K > 12288, channel ranges wider
than one finalize chunk).  At the full Qwen3-8B LM head (V = 151936) the fused
call must agree with the two separate calls.
"""
import numpy as np
import pytest
import torch

from oracle import quasar_oracle as orc
from w8a8_quantized_speculative_amd import binding, synth
from tests.gpu_helpers import announce, dev, dev_bf16, host, host_bf16
from tests.test_parity_accept import check_rejection

pytestmark = pytest.mark.gpu


def lm_head_case(B, k, V, K, key):
    x, w, s = synth.linear_case(B * (k + 1), K, V, key)
    ref = orc.w8a8_linear_rows(x, s, w)
    return x, w, s, ref["y"].reshape(B, k + 1, V)


def gpu_lm_head_verify(x, w, s, B, draft, T=0.0, u=None):
    wq, sw = binding.quasar_quantize_weights(dev_bf16(w), dev(s))
    k = x.shape[0] // B - 1
    d = dev(np.asarray(draft, np.int32).reshape(B, k)) if k > 0 else None
    ud = dev(np.asarray(u, np.float32)) if u is not None else None
    lg, L, nxt, g, pd = binding.quasar_lm_head_verify(
        dev_bf16(x), dev(s), wq, sw, B, d, T, ud, want_argmax=(T == 0), want_p_draft=(T > 0))
    torch.cuda.synchronize()
    return (host_bf16(lg), host(L), host(nxt), host(g) if g is not None else None,
            host(pd) if pd is not None else None)


# (B, k, V, K): fused path (B (k+1) <= 8, K <= 12288) -- tiles per workgroup from
# 1/4 (V = 1000) to 16 (V = 65536), ragged V, every K variant -- then the
# fallbacks: 18 rows (wide kernel), K = 16384, and 600000 channels (a
# workgroup's range wider than one 2048-logit finalize chunk)
GREEDY = [
    (1, 5, 20000, 1024), (1, 7, 5003, 512), (2, 3, 30011, 1040), (4, 1, 1000, 256),
    (1, 0, 777, 64), (1, 5, 65536, 64), (1, 3, 9000, 8000), (1, 5, 4100, 12288),
    (3, 5, 20000, 512), (1, 5, 3000, 16384), (1, 1, 600000, 64),
]


@pytest.mark.parametrize("B,k,V,K", GREEDY)
def test_greedy_lm_head_verify(B, k, V, K):
    announce("lm_head_verify_greedy", B, k, V, K)
    x, w, s, lg_ref = lm_head_case(B, k, V, K, (40, B, k, V % 1000))
    g_ref = orc.argmax_lowest(lg_ref)
    draft = synth.draft_tokens(g_ref[:, :k], V, 0.5, (40, B, k)) if k else np.zeros((B, 0), np.int32)
    lg, L, nxt, g, _ = gpu_lm_head_verify(x, w, s, B, draft)
    assert np.array_equal(lg, lg_ref)
    L_ref, n_ref, _ = orc.greedy_accept(lg_ref, draft)
    assert np.array_equal(g, g_ref) and np.array_equal(L, L_ref) and np.array_equal(nxt, n_ref)


def test_greedy_ties_between_workgroups_go_to_the_lowest_index():
    """A row whose maximum appears in several workgroups' channel ranges (all
    channels identical): the argmax is channel 0."""
    B, k, V, K = 1, 2, 8192, 256
    announce("lm_head_verify_ties", B, k, V, K)
    x, _, s = synth.linear_case(B * (k + 1), K, 1, (41, 0))
    w = np.repeat(synth.weights(1, K, (41, 1)), V, axis=0)
    ref = orc.w8a8_linear_rows(x, s, w)
    lg_ref = ref["y"].reshape(B, k + 1, V)
    draft = np.zeros((B, k), np.int32)
    lg, L, nxt, g, _ = gpu_lm_head_verify(x, w, s, B, draft)
    assert np.array_equal(lg, lg_ref)
    assert np.all(g == 0) and L[0] == k and nxt[0] == 0


@pytest.mark.parametrize("B,k,V,K,T", [
    (1, 5, 20000, 1024, 1.0), (2, 3, 5003, 512, 0.5), (1, 5, 65536, 64, 0.05),
    (1, 7, 3000, 4096, 2.0), (3, 5, 7000, 256, 1.0), (1, 1, 600000, 64, 1.0),
])
def test_rejection_lm_head_verify(B, k, V, K, T):
    announce("lm_head_verify_rejection", B, k, V, K, T)
    x, w, s, lg_ref = lm_head_case(B, k, V, K, (42, B, k, V % 1000))
    g_ref = orc.argmax_lowest(lg_ref)
    draft = synth.draft_tokens(g_ref[:, :k], V, 0.5, (42, B, k))
    u = synth.uniforms(B, k, (42, B, k, int(T * 100)))
    lg, L, nxt, _, pd = gpu_lm_head_verify(x, w, s, B, draft, T, u)
    assert np.array_equal(lg, lg_ref)
    band = check_rejection(lg_ref, draft, T, u, L, nxt, pd)
    assert band <= 1


@pytest.fixture(scope="module")
def full_lm_head():
    """The Qwen3-8B LM head 4096 -> 151936 at M = 6 (B = 1, k = 5), every logit
    by the oracle (quantized and multiplied in blocks of rows, which is exact:
    weight scales are per row), and the packed weights on the GPU."""
    B, k, V, K = 1, 5, synth.QWEN3_8B_VOCAB, 4096
    key = (43, 0)
    x = synth.activations(B * (k + 1), K, key)
    w = synth.weights(V, K, key)
    s = synth.smoothing_vector(synth.col_absmax_bf16(x), synth.col_absmax_bf16(w))
    y_ref = np.empty((B * (k + 1), V), np.uint16)
    for r0 in range(0, V, 16384):
        y_ref[:, r0:r0 + 16384] = orc.w8a8_linear_rows(x, s, w[r0:r0 + 16384])["y"]
    wq, sw = binding.quasar_quantize_weights(dev_bf16(w), dev(s))
    del w
    return B, k, V, K, x, s, wq, sw, y_ref.reshape(B, k + 1, V)


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_full_lm_head_against_the_oracle(full_lm_head, T):
    """The benchmark's exact call -- quasar_lm_head_verify on the 4096 -> 151936
    head at M = 6, fused epilogue partials and finalize -- against the oracle:
    all 911616 logits bit-exact, the argmax exact, and the greedy decision exact
    (T = 0), or the rejection decision exact outside the binary32 band (T = 1).
    Drafts are planted against the oracle's argmax (p = 0.3, one set all
    correct), and the separate calls (linear, then accept) agree with it."""
    B, k, V, K, x, s, wq, sw, lg_ref = full_lm_head
    announce("lm_head_verify_full_oracle", B, k, V, K, T)
    g_ref = orc.argmax_lowest(lg_ref)
    xd, sd = dev_bf16(x), dev(s)
    for trial in range(4):
        draft = (g_ref[:, :k].astype(np.int32) if trial == 0 else
                 synth.draft_tokens(g_ref[:, :k], V, 0.3, (43, trial)).astype(np.int32))
        u = synth.uniforms(B, k, (43, trial))
        lg, L, nxt, g1, pd = binding.quasar_lm_head_verify(
            xd, sd, wq, sw, B, dev(draft), T, dev(u) if T > 0 else None,
            want_argmax=(T == 0), want_p_draft=(T > 0))
        torch.cuda.synchronize()
        lg_h = host_bf16(lg).reshape(B, k + 1, V)
        assert np.array_equal(lg_h, lg_ref)
        if T == 0:
            L_ref, n_ref, _ = orc.greedy_accept(lg_ref, draft)
            assert np.array_equal(host(g1), g_ref)
            assert np.array_equal(host(L), L_ref) and np.array_equal(host(nxt), n_ref)
            if trial == 0:
                assert int(L_ref[0]) == k
        else:
            assert check_rejection(lg_ref, draft, T, u, host(L), host(nxt), host(pd)) <= 1
        # the separate calls (linear, then accept) take the same decisions
        y = binding.quasar_w8a8_linear(xd, sd, wq, sw)
        L2, n2, _, pd2 = binding.quasar_verify_accept(y.view(B, k + 1, V), dev(draft), T,
                                                      dev(u) if T > 0 else None,
                                                      want_p_draft=(T > 0))
        torch.cuda.synchronize()
        assert np.array_equal(host_bf16(y).reshape(B, k + 1, V), lg_ref)
        if T == 0:
            assert torch.equal(L, L2) and torch.equal(nxt, n2)
        else:
            assert check_rejection(lg_ref, draft, T, u, host(L2), host(n2), host(pd2)) <= 1
