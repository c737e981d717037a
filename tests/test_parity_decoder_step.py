"""GPU parity of a whole decoder verify step (w8a8_quantized_speculative_amd/decoder.py).

A small Qwen3-shaped model (2 layers, 4 query / 2 KV heads of 128, hidden
512, intermediate 1024, vocabulary 1000) runs one verify step with every
intermediate recorded.  Each step is then checked against the oracles on the
GPU's own inputs to that step, so the chain is checked link by link:
W8A8 linears bit-exact, residual adds bit-exact, RMSNorm / RoPE / attention
/ SiLU to the bar of the kernel tests (one BF16 spacing plus the binary32
error bound, nearly all elements identical), and the accept decision exact
on the GPU's logits.
Two windows: one sequence (6 tokens: the one-launch linear) and two
sequences (12 tokens: the wide linear), with a 70-position cached context that
crosses an attention step edge; and one layer at Qwen3-8B's dimensions (hidden
4096, 32 / 8 heads, intermediate 12288) over a 2048-position context.  Each runs
twice: gate_up then SiLU as two calls, and gate_up in the gated order with SiLU
applied in the linear's epilogue (6 tokens) or by the gated SiLU kernel (12
tokens), where the activation is checked against the oracle linear of the GPU's
input.  The drafts come from the N-gram drafter on a synthetic history.
"""
import numpy as np
import pytest
import torch

from oracle import decoder_oracle as dec
from oracle import quasar_oracle as orc
from w8a8_quantized_speculative_amd import binding, synth
from w8a8_quantized_speculative_amd.decoder import (DecoderConfig, DecoderStep, Linear,
                                                     ngram_history, random_norms)
from w8a8_quantized_speculative_amd.drafter import ngram_draft
from tests.gpu_helpers import announce, dev, dev_bf16, host, host_bf16
from tests.test_parity_decoder import U, assert_bf16_close, attention_allow, rope_allow

pytestmark = pytest.mark.gpu

CFG = DecoderConfig(hidden=512, heads_q=4, heads_kv=2, head_dim=128, intermediate=1024, layers=2,
                    vocab=1000)
# one layer at Qwen3-8B's dimensions (vocabulary cut to 1000 to keep the oracle's
# LM head small), a 2048-position context
QWEN3_LAYER = DecoderConfig(hidden=4096, heads_q=32, heads_kv=8, head_dim=128, intermediate=12288,
                            layers=1, vocab=1000)


def make_linear(N, K, key, gated=False):
    w = synth.weights(N, K, key)
    prof = synth.activations(64, K, key + (9,))
    s = synth.smoothing_vector(synth.col_absmax_bf16(prof), synth.col_absmax_bf16(w))
    pack = binding.quasar_quantize_weights_gated if gated else binding.quasar_quantize_weights
    wq, sw = pack(dev_bf16(w), dev(s))
    return Linear(wq, sw, dev(s), N, K, gated=gated), (w, s)


def bits(t):
    return host_bf16(t)


@pytest.mark.parametrize("cfg_name,B,pos0,gated", [("small", 1, 70, False), ("small", 2, 70, False),
                                                    ("qwen3_layer", 1, 2048, False),
                                                    ("small", 1, 70, True), ("small", 2, 70, True),
                                                    ("qwen3_layer", 1, 2048, True)])
def test_decoder_step_link_by_link(cfg_name, B, pos0, gated):
    c = CFG if cfg_name == "small" else QWEN3_LAYER
    k = 5
    T = k + 1
    announce("decoder_step", cfg_name, B, k, pos0)
    H, D, I = c.hidden, c.head_dim, c.intermediate
    qkv_n = (c.heads_q + 2 * c.heads_kv) * D
    layers, host_w = [], []
    for li in range(c.layers):
        L, Lh = {}, {}
        for name, N, K in (("qkv", qkv_n, H), ("o", H, c.heads_q * D), ("gate_up", 2 * I, H),
                           ("down", H, I)):
            L[name], Lh[name] = make_linear(N, K, (70, B, li, len(L)),
                                            gated=gated and name == "gate_up")
        layers.append(L)
        host_w.append(Lh)
    lm, lm_host = make_linear(c.vocab, H, (70, B, 99))
    table = synth.to_bf16_bits(synth.rng(70, B, 98).normal(size=(c.vocab, H)).astype(np.float32))
    norms = random_norms(c, "cuda", seed=B)
    step = DecoderStep(c, layers, lm, dev_bf16(table), norms, B, k, pos0)
    step.fill_context(seed=B)
    hist = [ngram_history(200, c.vocab, seed=B + s) for s in range(B)]
    drafts = np.stack([ngram_draft(h, k) for h in hist])
    tokens = np.concatenate([np.concatenate([h[-1:], d]) for h, d in zip(hist, drafts)])
    step.tokens.copy_(dev(tokens.astype(np.int32)))
    step.draft.copy_(dev(drafts.astype(np.int32)))
    rec = {}
    step.run(record=rec)
    torch.cuda.synchronize()

    def lin_check(x_t, y_t, wh):
        ref = orc.w8a8_linear_rows(bits(x_t), wh[1], wh[0])
        assert np.array_equal(bits(y_t), ref["y"])

    g = {n: [host(t) for t in norms[n]] for n in ("input", "post", "q", "k")}
    g_final = host(norms["final"])
    h = host(rec["h_embed"][0])
    assert np.array_equal(h, dec.embed(tokens, orc.bf16_to_f32(table).astype(np.float64)).astype(np.float32))
    for li in range(c.layers):
        Lh = host_w[li]
        ref = dec.rmsnorm(h, g["input"][li], c.eps)[1]
        assert_bf16_close(bits(rec["x_attn_in"][li]), ref, 0.99, (H + 8) * U * np.abs(ref))
        lin_check(rec["x_attn_in"][li], rec["qkv"][li], Lh["qkv"])
        qkv = orc.bf16_to_f32(bits(rec["qkv"][li])).astype(np.float64)
        qr, kr, vr = dec.qk_norm_rope(qkv, g["q"][li], g["k"][li], B, T, c.heads_q, c.heads_kv, D,
                                      pos0, c.rope_base, c.eps)
        heads = qkv.reshape(B * T, -1, D)
        q_allow = rope_allow(dec.head_rmsnorm(heads[:, :c.heads_q], g["q"][li], c.eps), D)
        k_allow = rope_allow(dec.head_rmsnorm(heads[:, c.heads_q:c.heads_q + c.heads_kv],
                                              g["k"][li], c.eps), D)
        assert_bf16_close(bits(rec["q"][li]).reshape(B * T, c.heads_q, D), qr, 0.95, q_allow)
        kc, vc = bits(step.k_cache[li]), bits(step.v_cache[li])
        new = slice(pos0, pos0 + T)
        assert_bf16_close(kc[:, :, new].transpose(0, 2, 1, 3).reshape(B * T, c.heads_kv, D), kr,
                          0.95, k_allow)
        assert np.array_equal(vc[:, :, new].transpose(0, 2, 1, 3).reshape(B * T, c.heads_kv, D),
                              bits(rec["qkv"][li]).reshape(B * T, -1, D)[:, c.heads_q + c.heads_kv:])
        q_gpu = orc.bf16_to_f32(bits(rec["q"][li])).astype(np.float64).reshape(B * T, c.heads_q, D)
        kf, vf = orc.bf16_to_f32(kc).astype(np.float64), orc.bf16_to_f32(vc).astype(np.float64)
        att = dec.attention(q_gpu, kf, vf, B, T, c.heads_q, pos0)
        assert_bf16_close(bits(rec["att"][li]).reshape(B * T, c.heads_q, D), att, 0.99,
                          attention_allow(q_gpu, kf, vf, B, T, c.heads_q, pos0))
        lin_check(rec["att"][li], rec["o"][li], Lh["o"])
        h_o = host(rec["h_before_o"][li])
        assert np.array_equal(h_o, h)
        h = h_o + orc.bf16_to_f32(bits(rec["o"][li]))  # binary32 residual add
        assert np.array_equal(host(rec["h_before_down"][li]), h)
        ref = dec.rmsnorm(h, g["post"][li], c.eps)[1]
        assert_bf16_close(bits(rec["x_mlp_in"][li]), ref, 0.99, (H + 8) * U * np.abs(ref))
        if gated:  # no product is written: the oracle linear of the GPU's input
            gu_bits = orc.w8a8_linear_rows(bits(rec["x_mlp_in"][li]), Lh["gate_up"][1],
                                           Lh["gate_up"][0])["y"]
        else:
            lin_check(rec["x_mlp_in"][li], rec["gu"][li], Lh["gate_up"])
            gu_bits = bits(rec["gu"][li])
        gu = orc.bf16_to_f32(gu_bits).astype(np.float64)
        ref = dec.silu_mul(gu)
        assert_bf16_close(bits(rec["act"][li]), ref, 0.99, 8 * U * np.abs(ref))
        lin_check(rec["act"][li], rec["dn"][li], Lh["down"])
        h = h + orc.bf16_to_f32(bits(rec["dn"][li]))
    assert np.array_equal(host(step.h), h)
    ref = dec.rmsnorm(h, g_final, c.eps)[1]
    assert_bf16_close(bits(rec["x_head_in"][0]), ref, 0.99, (H + 8) * U * np.abs(ref))
    logits = bits(step.logits)
    ref = orc.w8a8_linear_rows(bits(rec["x_head_in"][0]), lm_host[1], lm_host[0])
    assert np.array_equal(logits.reshape(B * T, -1), ref["y"])
    L_ref, n_ref, _ = orc.greedy_accept(logits, drafts)
    assert np.array_equal(host(step.accept_len), L_ref)
    assert np.array_equal(host(step.next_token), n_ref)
