"""A Qwen3-8B-shaped decoder verify step built on the library's calls.

One verify step runs the target model once over the T = 1 + k positions of
every sequence [Quasar, pt page §2 execution pipeline; zh page §2]: the
embedding of the last accepted token and the k drafts, then per layer

    x = RMSNorm(h)                  -> QKV (W8A8) -> q/k norm, RoPE, KV append
      -> attention over the cache   -> O (W8A8)   -> h += o
    x = RMSNorm(h)                  -> gate_up (W8A8) -> silu(gate) * up (in the
                                       linear's epilogue for gated weights)
      -> down (W8A8)                -> h += down

then the final RMSNorm and the W8A8 LM head with the accept step
(``quasar_lm_head_verify``).  Every step is a libquasar call; this module
only allocates the buffers and issues the calls in order (host
orchestration; no arithmetic here).  Weights are random (no trained
checkpoint exists here), so acceptance is not meaningful -- the step exists
to time the linears inside a complete pass with all dependencies in place.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import binding


@dataclass(frozen=True)
class DecoderConfig:
    hidden: int
    heads_q: int
    heads_kv: int
    head_dim: int
    intermediate: int
    layers: int
    vocab: int
    eps: float = 1e-6
    rope_base: float = 1e6


QWEN3_8B = DecoderConfig(hidden=4096, heads_q=32, heads_kv=8, head_dim=128, intermediate=12288,
                         layers=36, vocab=151936)


@dataclass
class Linear:
    """One W8A8 linear: packed INT8 weights, per-channel scales, smoothing s.
    ``gated``: a gate_up linear packed by quasar_quantize_weights_gated, run as
    quasar_w8a8_linear_swiglu (the activation in the linear's epilogue)."""
    wq: binding.PackedWeights
    sw: torch.Tensor
    s: torch.Tensor
    N: int
    K: int
    gated: bool = False


class DecoderStep:
    """Buffers and call sequence of one verify step for B sequences at cached
    context length pos0 (the same for every sequence), T = 1 + k positions.

    ``layers`` holds per layer the dict {"qkv", "o", "gate_up", "down"} of
    Linear; ``lm_head`` the LM head's Linear; ``embed`` the bf16 table
    [V, hidden]; norm weights are f32.
    """

    def __init__(self, cfg: DecoderConfig, layers, lm_head: Linear, embed: torch.Tensor,
                 norms: dict, B: int, k: int, pos0: int, Lmax: int | None = None):
        self.cfg, self.layers, self.lm_head, self.embed = cfg, layers, lm_head, embed
        self.norms = norms
        self.B, self.k, self.T, self.pos0 = B, k, k + 1, pos0
        self.M = B * self.T
        self.Lmax = Lmax if Lmax is not None else pos0 + self.T
        dev = embed.device
        c = cfg
        M, H, D = self.M, c.hidden, c.head_dim
        qkv_n = (c.heads_q + 2 * c.heads_kv) * D
        bf = torch.bfloat16
        self.tokens = torch.zeros(M, dtype=torch.int32, device=dev)
        self.draft = torch.zeros((B, k), dtype=torch.int32, device=dev)
        self.uniforms = torch.zeros((B, self.T), dtype=torch.float32, device=dev)
        self.h = torch.empty((M, H), dtype=torch.float32, device=dev)
        self.x = torch.empty((M, H), dtype=bf, device=dev)
        self.qkv = torch.empty((M, qkv_n), dtype=bf, device=dev)
        self.q = torch.empty((M, c.heads_q * D), dtype=bf, device=dev)
        self.att = torch.empty((M, c.heads_q * D), dtype=bf, device=dev)
        self.o = torch.empty((M, H), dtype=bf, device=dev)
        self.gu = torch.empty((M, 2 * c.intermediate), dtype=bf, device=dev)
        self.act = torch.empty((M, c.intermediate), dtype=bf, device=dev)
        self.dn = torch.empty((M, H), dtype=bf, device=dev)
        self.logits = torch.empty((B, self.T, c.vocab), dtype=bf, device=dev)
        self.accept_len = torch.empty(B, dtype=torch.int32, device=dev)
        self.next_token = torch.empty(B, dtype=torch.int32, device=dev)
        self.k_cache = [torch.zeros((B, c.heads_kv, self.Lmax, D), dtype=bf, device=dev)
                        for _ in range(c.layers)]
        self.v_cache = [torch.zeros((B, c.heads_kv, self.Lmax, D), dtype=bf, device=dev)
                        for _ in range(c.layers)]
        lin_ws = max((binding.workspace_bytes_linear_swiglu if l.gated else
                      binding.workspace_bytes_linear)(M, l.N, l.K)
                     for L in layers for l in L.values())
        self.ws_lin = binding.new_workspace(lin_ws, dev)
        self.ws_att = binding.new_workspace(
            binding.workspace_bytes_attention(B, self.T, c.heads_q, c.heads_kv, pos0), dev)
        self.ws_head = binding.new_workspace(
            binding.workspace_bytes_lm_head_verify(B, k, c.vocab, H), dev)

    def fill_context(self, seed: int = 0):
        """Synthetic cached context: positions 0 .. pos0-1 of every layer's
        caches hold seeded N(0, 1) values (BF16)."""
        g = torch.Generator(device=self.embed.device)
        g.manual_seed(seed)
        for kc, vc in zip(self.k_cache, self.v_cache):
            for c in (kc, vc):
                c[:, :, :self.pos0].normal_(generator=g)

    def _linear(self, x, lin: Linear, out):
        binding.quasar_w8a8_linear(x, lin.s, lin.wq, lin.sw, out=out, workspace=self.ws_lin)

    def run(self, temperature: float = 0.0, record: dict | None = None):
        """Issue the whole step on the current stream.  With ``record`` (a
        dict), every intermediate is copied there (host arrays) per layer."""
        c = self.cfg

        def rec(name, t):
            if record is not None:
                record.setdefault(name, []).append(t.detach().clone())

        binding.quasar_embed(self.tokens, self.embed, out=self.h)
        rec("h_embed", self.h)
        binding.quasar_rmsnorm(self.h, self.norms["input"][0], c.eps, out=self.x)
        for li, L in enumerate(self.layers):
            rec("x_attn_in", self.x)
            self._linear(self.x, L["qkv"], self.qkv)
            rec("qkv", self.qkv)
            binding.quasar_qk_rope_cache(self.qkv, self.norms["q"][li], self.norms["k"][li],
                                         self.k_cache[li], self.v_cache[li], self.B, c.heads_q,
                                         self.pos0, rope_base=c.rope_base, eps=c.eps, q_out=self.q)
            rec("q", self.q)
            binding.quasar_attention(self.q, self.k_cache[li], self.v_cache[li], c.heads_q,
                                     self.pos0, out=self.att, workspace=self.ws_att)
            rec("att", self.att)
            self._linear(self.att, L["o"], self.o)
            rec("o", self.o)
            rec("h_before_o", self.h)
            binding.quasar_rmsnorm(self.h, self.norms["post"][li], c.eps, delta=self.o, out=self.x)
            rec("x_mlp_in", self.x)
            gu = L["gate_up"]
            if gu.gated:
                binding.quasar_w8a8_linear_swiglu(self.x, gu.s, gu.wq, gu.sw, out=self.act,
                                                  workspace=self.ws_lin)
            else:
                self._linear(self.x, gu, self.gu)
                rec("gu", self.gu)
                binding.quasar_silu_mul(self.gu, out=self.act)
            rec("act", self.act)
            self._linear(self.act, L["down"], self.dn)
            rec("dn", self.dn)
            rec("h_before_down", self.h)
            nxt = self.norms["input"][li + 1] if li + 1 < len(self.layers) else self.norms["final"]
            binding.quasar_rmsnorm(self.h, nxt, c.eps, delta=self.dn, out=self.x)
        rec("x_head_in", self.x)
        lh = self.lm_head
        binding.quasar_lm_head_verify(
            self.x, lh.s, lh.wq, lh.sw, self.B, self.draft if self.k else None, temperature,
            self.uniforms if temperature > 0 else None, want_argmax=False, want_p_draft=False,
            logits=self.logits, accept_len=self.accept_len, next_token=self.next_token,
            workspace=self.ws_head)


def random_norms(cfg: DecoderConfig, device, seed: int = 0) -> dict:
    """Norm weights near 1 (seeded), f32."""
    g = np.random.default_rng([seed, 7])

    def v(n):
        return torch.from_numpy(g.uniform(0.8, 1.2, size=n).astype(np.float32)).to(device)

    return {"input": [v(cfg.hidden) for _ in range(cfg.layers)],
            "post": [v(cfg.hidden) for _ in range(cfg.layers)],
            "q": [v(cfg.head_dim) for _ in range(cfg.layers)],
            "k": [v(cfg.head_dim) for _ in range(cfg.layers)],
            "final": v(cfg.hidden)}


def ngram_history(length: int, vocab: int, seed: int = 0) -> np.ndarray:
    """A synthetic token history with repeated phrases, so that the N-gram
    drafter finds matches: a pool of 64 seeded 12-token phrases, drawn with
    replacement and concatenated."""
    g = np.random.default_rng([seed, 8])
    phrases = g.integers(0, vocab, size=(64, 12))
    out = np.concatenate([phrases[i] for i in g.integers(0, 64, size=length // 12 + 1)])
    return out[:length].astype(np.int32)
