"""GPU parity of chained W8A8 linears in one launch (quasar_w8a8_chain,
quasar_chain_verify) against the oracle.

A chain follows a decoder layer's data flow: QKV, then O reading the query
columns of QKV's output (a column slice, through ldx), gate_up with SiLU * up
in its epilogue reading O's output, down reading that activation, the next
layer's QKV reading down's output, and so on.  Each link's output is checked
against the oracle applied to the link's actual input (the previous link's
GPU output, itself checked): the plain links bit-exact (BF16 outputs and
INT32 accumulators), the gated link bit-exact against the separate
quasar_w8a8_linear_swiglu call on the same input and, through the oracle's
product, to the SiLU bar of the decoder tests.
"""
import numpy as np
import pytest
import torch

from oracle import decoder_oracle as dec
from oracle import quasar_oracle as orc
from w8a8_quantized_speculative_amd import binding, synth
from tests.gpu_helpers import announce, dev, dev_bf16, host, host_bf16
from tests.test_parity_accept import check_rejection
from tests.test_parity_decoder import U, assert_bf16_close

pytestmark = pytest.mark.gpu


class Lin:
    """One synthetic linear: BF16 weights, s calibrated on synthetic inputs of its
    width, packed INT8 weights (and the gated pack for gate_up)."""

    def __init__(self, N, K, key, gated=False):
        self.N, self.K, self.gated = N, K, gated
        self.w = synth.weights(N, K, key)
        x_cal = synth.activations(64, K, key + (7,))
        self.s = synth.smoothing_vector(synth.col_absmax_bf16(x_cal), synth.col_absmax_bf16(self.w))
        wd, self.sd = dev_bf16(self.w), dev(self.s)
        if gated:
            self.wq, self.sw = binding.quasar_quantize_weights_gated(wd, self.sd)
        else:
            self.wq, self.sw = binding.quasar_quantize_weights(wd, self.sd)
        del wd


def layer(H, Q, KV, I, key):
    return {"qkv": Lin(Q + 2 * KV, H, key + (0,)), "o": Lin(H, Q, key + (1,)),
            "gate_up": Lin(2 * I, H, key + (2,), gated=True), "down": Lin(H, I, key + (3,))}


def build_chain(M, layers, x0, head=None, acc=False):
    """Chain over `layers` (dicts of Lin); returns (chain, records) where each
    record is (name, lin, x_tensor, y_tensor, acc_tensor)."""
    ch = binding.Chain(M)
    recs = []
    x = x0
    for li, L in enumerate(layers):
        dep_prev = len(recs) - 1
        q = L["qkv"]
        y_qkv = torch.empty((M, q.N), dtype=torch.bfloat16, device="cuda")
        a = torch.empty((M, q.N), dtype=torch.int32, device="cuda") if acc else None
        ch.add(x, q.sd, q.wq, q.sw, y_qkv, dep=dep_prev, acc_out=a)
        recs.append(("qkv%d" % li, q, x, y_qkv, a))
        o = L["o"]
        xo = y_qkv[:, :o.K]  # the query columns stand in for attention's output
        y_o = torch.empty((M, o.N), dtype=torch.bfloat16, device="cuda")
        ch.add(xo, o.sd, o.wq, o.sw, y_o, dep=len(recs) - 1)
        recs.append(("o%d" % li, o, xo, y_o, None))
        g = L["gate_up"]
        act = torch.empty((M, g.N // 2), dtype=torch.bfloat16, device="cuda")
        ch.add(y_o, g.sd, g.wq, g.sw, act, dep=len(recs) - 1, swiglu=True)
        recs.append(("gate_up%d" % li, g, y_o, act, None))
        d = L["down"]
        y_d = torch.empty((M, d.N), dtype=torch.bfloat16, device="cuda")
        ad = torch.empty((M, d.N), dtype=torch.int32, device="cuda") if acc else None
        ch.add(act, d.sd, d.wq, d.sw, y_d, dep=len(recs) - 1, acc_out=ad)
        recs.append(("down%d" % li, d, act, y_d, ad))
        x = y_d
    if head is not None:
        logits = torch.empty((M, head.N), dtype=torch.bfloat16, device="cuda")
        ch.add(x, head.sd, head.wq, head.sw, logits, dep=len(recs) - 1)
        recs.append(("head", head, x, logits, None))
    return ch.finalize(), recs


def check_records(recs, cols=None):
    """Every link against the oracle on its GPU input (sampled output columns
    when `cols` gives a count)."""
    for name, lin, x, y, a in recs:
        xb = host_bf16(x)
        if lin.gated:
            I = lin.N // 2
            sep = binding.quasar_w8a8_linear_swiglu(x.contiguous(), lin.sd, lin.wq, lin.sw)
            torch.cuda.synchronize()
            got = host_bf16(y)
            assert np.array_equal(got, host_bf16(sep)), name
            pick = np.arange(I) if cols is None else np.sort(
                np.random.default_rng(len(name)).choice(I, size=min(cols, I), replace=False))
            ref = orc.w8a8_linear_rows(xb, lin.s, lin.w[np.concatenate([pick, I + pick])])
            yf = orc.bf16_to_f32(ref["y"]).astype(np.float64)
            a_ref = dec.silu_mul(yf)
            assert_bf16_close(got[:, pick], a_ref, 0.99, 8 * U * np.abs(a_ref))
            continue
        pick = np.arange(lin.N) if cols is None else np.sort(
            np.random.default_rng(len(name)).choice(lin.N, size=min(cols, lin.N), replace=False))
        ref = orc.w8a8_linear_rows(xb, lin.s, lin.w[pick])
        assert np.array_equal(host_bf16(y)[:, pick], ref["y"]), name
        if a is not None:
            assert np.array_equal(host(a)[:, pick], ref["acc"].astype(np.int32)), name


@pytest.mark.parametrize("M", [6, 1, 3, 8])
def test_chain_two_layers_every_element(M):
    """Two small layers (hidden 1024, 16 query heads of 64 = 1024, KV 256,
    intermediate 1536) and a 2000-wide head, every output element."""
    announce("chain two layers", M)
    layers = [layer(1024, 1024, 256, 1536, (100, M, i)) for i in range(2)]
    head = Lin(2000, 1024, (100, M, 9))
    x0 = dev_bf16(synth.activations(M, 1024, (100, M, 8)))
    ch, recs = build_chain(M, layers, x0, head=head, acc=True)
    ch.run()
    torch.cuda.synchronize()
    check_records(recs)
    assert binding.device_check() == (binding.QUASAR_OK, 0)


def test_chain_ragged_shapes_and_independent_links():
    """Links with ragged K (not a multiple of the 2048-wide phase or the 4096-wide
    quantization step), fewer tiles than workgroups (empty ranges), K up to
    12288, column slices that do not start at 0, and links with inputs of
    their own between dependent ones.  (N, K, dep, first column of the slice)"""
    M = 5
    announce("chain ragged", M)
    ch = binding.Chain(M)
    recs = []
    specs = [(64, 80, -1, 0), (4112, 3008, -1, 0), (48, 4112, 1, 0), (1040, 32, 2, 16),
             (16, 12288, -1, 0), (6160, 1040, -1, 0), (2048, 6144, 5, 16), (32, 2048, 6, 0),
             (12288, 16, 7, 16), (64, 12288, 8, 0)]
    outs = []
    for i, (N, K, dep, col0) in enumerate(specs):
        lin = Lin(N, K, (101, i))
        if dep < 0:
            x = dev_bf16(synth.activations(M, K, (101, i, 1)))
        else:
            assert dep == i - 1
            x = outs[dep][:, col0:col0 + K]
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        a = torch.empty((M, N), dtype=torch.int32, device="cuda")
        ch.add(x, lin.sd, lin.wq, lin.sw, y, dep=dep, acc_out=a)
        outs.append(y)
        recs.append(("l%d" % i, lin, x, y, a))
    ch.finalize()
    for rep in range(3):  # launch parities alternate; each run must stand on its own
        for _, _, _, y, _ in recs:
            y.zero_()
        ch.run()
        torch.cuda.synchronize()
        check_records(recs)
    assert binding.device_check() == (binding.QUASAR_OK, 0)


def test_chain_qwen3_8b_layer_sampled():
    """The Qwen3-8B layer shapes the benchmark chains, at 6 tokens: QKV
    4096 -> 6144, O 4096 -> 4096 (query columns), gate_up 4096 -> 24576 with
    SiLU * up, down 12288 -> 4096, then the next layer's QKV; sampled output
    columns against the oracle."""
    M = 6
    announce("chain qwen3-8b layer", M)
    layers = [layer(4096, 4096, 1024, 12288, (102, 0))]
    nxt = Lin(6144, 4096, (102, 1, 0))
    x0 = dev_bf16(synth.activations(M, 4096, (102, 9)))
    ch, recs = build_chain(M, layers, x0)
    y = torch.empty((M, 6144), dtype=torch.bfloat16, device="cuda")
    ch.add(recs[-1][3], nxt.sd, nxt.wq, nxt.sw, y, dep=3)
    recs.append(("qkv1", nxt, recs[-1][3], y, None))
    ch.finalize()
    ch.run()
    torch.cuda.synchronize()
    check_records(recs, cols=512)
    assert binding.device_check() == (binding.QUASAR_OK, 0)


def test_chain_forced_expiry_is_reported():
    M = 6
    binding.device_check()
    layers = [layer(1024, 1024, 256, 1536, (103, 0))]
    x0 = dev_bf16(synth.activations(M, 1024, (103, 8)))
    ch, recs = build_chain(M, layers, x0)
    announce("chain forced expiry")
    binding.force_wait_expiry(True)
    try:
        ch.run()
    finally:
        binding.force_wait_expiry(False)
    st, bits = binding.device_check()
    assert st == binding.QUASAR_ERR_INCOMPLETE and bits & binding.QUASAR_WAIT_CHAIN, bits
    ch.run()  # the same workspace, hook off
    torch.cuda.synchronize()
    check_records(recs)
    assert binding.device_check() == (binding.QUASAR_OK, 0)


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_chain_verify_small_vocab(T):
    """One small layer and a 4000-token head, then the accept step: the logits
    bit-exact, argmax and greedy accept exact; at T = 1 the rejection decision
    exact outside the binary32 band."""
    M, B, k = 6, 1, 5
    announce("chain verify", T)
    layers = [layer(1024, 1024, 256, 1536, (104, 0))]
    head = Lin(4000, 1024, (104, 9))
    x0 = dev_bf16(synth.activations(M, 1024, (104, 8)))
    ch, recs = build_chain(M, layers, x0, head=head)
    ch.run()
    torch.cuda.synchronize()
    check_records(recs)
    logits = host_bf16(recs[-1][3]).reshape(B, k + 1, 4000)
    g_ref = orc.argmax_lowest(logits)
    for trial in range(4):
        draft = synth.draft_tokens(g_ref[:, :k], 4000, 0.6, (104, trial))
        u = synth.uniforms(B, k, (104, trial))
        L, nxt, g, pd = ch.run_verify(B, k, dev(draft.astype(np.int32)), T,
                                      dev(u) if T > 0 else None, want_argmax=T == 0,
                                      want_p_draft=T > 0)
        torch.cuda.synchronize()
        assert np.array_equal(host_bf16(recs[-1][3]).reshape(B, k + 1, 4000), logits)
        if T == 0:
            L_ref, n_ref, _ = orc.greedy_accept(logits, draft)
            assert np.array_equal(host(g), g_ref)
            assert np.array_equal(host(L), L_ref) and np.array_equal(host(nxt), n_ref)
        else:
            assert check_rejection(logits, draft, T, u, host(L), host(nxt), host(pd)) <= 1
    assert binding.device_check() == (binding.QUASAR_OK, 0)
