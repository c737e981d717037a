"""GPU parity of the verify/accept step against the oracle.

Greedy: argmax indices, accept lengths and next tokens bit-identical.
Rejection: the kernel works in binary32 with the device expf while the oracle
uses float64, so decisions are compared exactly except inside a band where the
two precisions may legitimately disagree: a uniform within 1e-5 (relative) of
p(draft), or an inverse-CDF target within 1e-5 of the total mass of a CDF
edge.  Outside the band everything must match; inside it the GPU's choice must
still be valid for the oracle's distribution.
"""
import numpy as np
import pytest
import torch

from oracle import quasar_oracle as orc
from w8a8_quantized_speculative_amd import binding, synth
from tests.gpu_helpers import announce, dev, dev_bf16, host

pytestmark = pytest.mark.gpu

V_QWEN = synth.QWEN3_8B_VOCAB


def gpu_accept(lg, draft, T=0.0, u=None):
    B, kp1, V = lg.shape
    d = dev(np.asarray(draft, np.int32).reshape(B, kp1 - 1)) if kp1 > 1 else None
    ud = dev(np.asarray(u, np.float32)) if u is not None else None
    L, nxt, g, pd = binding.quasar_verify_accept(dev_bf16(lg), d, T, ud, want_argmax=(T == 0),
                                                 want_p_draft=(T > 0))
    torch.cuda.synchronize()
    return host(L), host(nxt), (host(g) if g is not None else None), (host(pd) if pd is not None else None)


# ---------------------------------------------------------------- greedy
@pytest.mark.parametrize("B", [1, 16])
def test_greedy_full_vocab_planted_drafts(B):
    """LM-head-sized logits (V = 151936), k = 5, drafts equal to the argmax
    with probability 0.3 each."""
    k = 5
    for seed in range(4):
        announce("greedy", B, k, V_QWEN, seed)
        lg = synth.logits(B, k, V_QWEN, (20, B, seed), sigma=3.0)
        g_ref = orc.argmax_lowest(lg)
        draft = synth.draft_tokens(g_ref[:, :k], V_QWEN, 0.3, (20, B, seed))
        L, nxt, g, _ = gpu_accept(lg, draft)
        L_ref, n_ref, _ = orc.greedy_accept(lg, draft)
        assert np.array_equal(g, g_ref)
        assert np.array_equal(L, L_ref) and np.array_equal(nxt, n_ref)


def test_greedy_all_match_patterns():
    k, V = 5, 5000
    B = 2 ** k
    lg = synth.logits(B, k, V, (21, 0), sigma=2.0)
    g_ref = orc.argmax_lowest(lg)
    draft = np.zeros((B, k), np.int32)
    for b in range(B):
        for i in range(k):
            draft[b, i] = g_ref[b, i] if (b >> i) & 1 else (g_ref[b, i] + 1) % V
    announce("greedy_patterns", B, k, V)
    L, nxt, g, _ = gpu_accept(lg, draft)
    L_ref, n_ref, _ = orc.greedy_accept(lg, draft)
    assert np.array_equal(g, g_ref) and np.array_equal(L, L_ref) and np.array_equal(nxt, n_ref)


def test_greedy_ties_across_chunks_and_signed_zero():
    V, k = 3 * 2048 + 5, 2
    v = np.full((1, k + 1, V), -1.0, np.float32)
    v[0, 0, [2047, 2048, 6000]] = 7.0        # equal maxima in three different chunks
    v[0, 1, [6100, 4097]] = 3.5
    v[0, 2, :] = -2.0
    v[0, 2, 3000] = 0.0
    v[0, 2, 100] = -0.0                       # -0 == +0: the lower index wins
    lg = synth.to_bf16_bits(v)
    announce("greedy_ties", V)
    L, nxt, g, _ = gpu_accept(lg, np.array([[2047, 4097]]))
    assert g[0].tolist() == [2047, 4097, 100] == orc.argmax_lowest(lg)[0].tolist()
    assert L[0] == 2 and nxt[0] == 100


@pytest.mark.parametrize("V", [1, 7, 2048, 2049, 100000])
def test_greedy_small_and_ragged_vocab(V):
    B, k = 3, 4
    lg = synth.logits(B, k, V, (22, V))
    g_ref = orc.argmax_lowest(lg)
    draft = synth.draft_tokens(g_ref[:, :k], max(V, 2), 0.7, (22, V)) % V
    announce("greedy_vocab", B, k, V)
    L, nxt, g, _ = gpu_accept(lg, draft)
    L_ref, n_ref, _ = orc.greedy_accept(lg, draft)
    assert np.array_equal(g, g_ref) and np.array_equal(L, L_ref) and np.array_equal(nxt, n_ref)


def test_greedy_k0_and_out_of_range_drafts():
    announce("greedy_k0")
    lg = synth.logits(4, 0, 1000, (23, 0))
    L, nxt, g, _ = gpu_accept(lg, np.zeros((4, 0), np.int32))
    assert not np.any(L) and np.array_equal(nxt, orc.argmax_lowest(lg)[:, 0])
    announce("greedy_out_of_range")
    lg = synth.logits(3, 3, 1000, (23, 1))
    g_ref = orc.argmax_lowest(lg)
    draft = g_ref[:, :3].astype(np.int32).copy()
    draft[0, 0] = -1
    draft[1, 1] = 1000
    draft[2, 2] = 2**31 - 1
    L, nxt, _, _ = gpu_accept(lg, draft)
    L_ref, n_ref, _ = orc.greedy_accept(lg, draft)
    assert L.tolist() == [0, 1, 2] == L_ref.tolist() and np.array_equal(nxt, n_ref)


# ---------------------------------------------------------------- rejection
def check_rejection(lg, draft, T, u, L, nxt, pd):
    """Compare with the oracle under the precision band; returns the band count."""
    L_ref, n_ref, p_ref, rows, targets, cdfs = orc.rejection_accept(lg, draft, T, u)
    B, k = np.asarray(draft).reshape(lg.shape[0], -1).shape
    band = 0
    if k:
        assert np.allclose(pd.astype(np.float64), p_ref, rtol=1e-4, atol=1e-12)
    for b in range(B):
        near = [abs(float(u[b, i]) - p_ref[b, i]) <= 1e-5 * p_ref[b, i] + 1e-12 for i in range(k)]
        if L[b] != L_ref[b]:
            first = min(L[b], L_ref[b])
            assert near[first], (b, L[b], L_ref[b], u[b], p_ref[b])
            band += 1
            continue
        c = cdfs[b]
        tol = 1e-5 * c[-1]
        t = targets[b]
        j = int(nxt[b])
        lo = c[j - 1] if j > 0 else 0.0
        assert lo - tol <= t <= c[j] + tol, (b, j, n_ref[b])   # a valid draw for the oracle's p
        if j != n_ref[b]:
            jo = n_ref[b]
            lo_o = c[jo - 1] if jo > 0 else 0.0
            assert t - lo_o <= tol or c[jo] - t <= tol, (b, j, jo)
            band += 1
    return band


@pytest.mark.parametrize("B", [1, 16])
def test_rejection_t1_full_vocab(B):
    """T = 1 over LM-head-sized logits with seeded float32 uniforms."""
    k = 5
    for seed in range(3):
        announce("rejection", B, k, V_QWEN, seed)
        lg = synth.logits(B, k, V_QWEN, (30, B, seed), sigma=3.0)
        g_ref = orc.argmax_lowest(lg)
        draft = synth.draft_tokens(g_ref[:, :k], V_QWEN, 0.3, (30, B, seed))
        u = synth.uniforms(B, k, (30, B, seed))
        L, nxt, _, pd = gpu_accept(lg, draft, 1.0, u)
        band = check_rejection(lg, draft, 1.0, u, L, nxt, pd)
        assert band <= max(1, B // 8)


def test_rejection_peaked_logits_accept_and_bonus():
    """A dominant token per position: drafts that hit it are accepted and the
    bonus token comes from the last position."""
    B, k, V = 8, 5, 40000
    z = synth.logits(B, k, V, (31, 0), sigma=1.0)
    v = orc.bf16_to_f32(z).copy()
    top = np.random.default_rng(31).integers(0, V, (B, k + 1))
    for b in range(B):
        v[b, np.arange(k + 1), top[b]] = 25.0
    lg = synth.to_bf16_bits(v)
    draft = top[:, :k].astype(np.int32).copy()
    draft[1, 3] = (draft[1, 3] + 1) % V      # one early rejection
    u = synth.uniforms(B, k, (31, 0))
    announce("rejection_peaked", B, k, V)
    L, nxt, _, pd = gpu_accept(lg, draft, 1.0, u)
    check_rejection(lg, draft, 1.0, u, L, nxt, pd)
    assert L[0] == k and L[1] == 3


@pytest.mark.parametrize("T", [0.5, 2.0])
def test_rejection_small_vocab_temperatures(T):
    B, k, V = 64, 3, 8
    lg = synth.logits(B, k, V, (32, int(T * 10)), sigma=1.0)
    g_ref = orc.argmax_lowest(lg)
    draft = synth.draft_tokens(g_ref[:, :k], V, 0.5, (32, 0))
    u = synth.uniforms(B, k, (32, int(T * 10)))
    announce("rejection_small", B, k, V, T)
    L, nxt, _, pd = gpu_accept(lg, draft, T, u)
    band = check_rejection(lg, draft, T, u, L, nxt, pd)
    assert band <= 2


def chi_square_pvalue(counts, p):
    """Pearson chi-square p-value; bins expecting fewer than 5 draws are pooled."""
    from scipy.stats import chi2
    n = counts.sum()
    expected = n * np.asarray(p, np.float64)
    small = expected < 5
    obs = np.append(counts[~small], counts[small].sum())
    exp_ = np.append(expected[~small], expected[small].sum())
    if exp_[-1] < 5:  # the pooled bin joins the least likely remaining one
        j = int(np.argmin(exp_[:-1]))
        obs[j] += obs[-1]
        exp_[j] += exp_[-1]
        obs, exp_ = obs[:-1], exp_[:-1]
    return float(chi2.sf(((obs - exp_) ** 2 / exp_).sum(), len(obs) - 1))


@pytest.mark.parametrize("T", [0.5, 1.0])
def test_rejection_is_lossless_chi_square(T):
    """Losslessness of the GPU's speculative sampling with a one-hot draft.

    Accepting draft d with probability p(d), and otherwise drawing from p with
    d removed and renormalised, emits a first token distributed exactly as p.
    After an accept, the bonus token is drawn from the next position's p.
    12000 seeded sequences share one logits row.  For a likely, an unlikely
    and a middling draft token, both distributions must pass a chi-square
    test at p > 1e-6.  The seeds are fixed, so the outcome is deterministic.
    """
    V, n = 12, 12000
    base = synth.logits(1, 1, V, (35, int(T * 10)), sigma=1.0)      # [1, 2, V]
    probs = []
    for pos in range(2):
        v = orc.bf16_to_f32(base[0, pos]).astype(np.float64) / T
        e = np.exp(v - v.max())
        probs.append(e / e.sum())
    lg = np.repeat(base, n, axis=0)
    for d in (int(np.argmax(probs[0])), int(np.argmin(probs[0])), 5):
        announce("rejection_lossless", T, d, n, V)
        draft = np.full((n, 1), d, np.int32)
        u = synth.uniforms(n, 1, (35, int(T * 10), d))
        L, nxt, _, pd = gpu_accept(lg, draft, T, u)
        assert np.allclose(pd[:, 0], probs[0][d], rtol=1e-4)
        first = np.where(L >= 1, d, nxt)
        assert chi_square_pvalue(np.bincount(first, minlength=V), probs[0]) > 1e-6
        # the acceptance rate is p(d) (binomial, 5 standard deviations)
        acc = int((L >= 1).sum())
        sd = np.sqrt(n * probs[0][d] * (1 - probs[0][d]))
        assert abs(acc - n * probs[0][d]) <= 5 * sd + 1
        if acc >= 2000:
            bonus = np.bincount(nxt[L >= 1], minlength=V)
            assert chi_square_pvalue(bonus, probs[1]) > 1e-6


def test_rejection_out_of_range_draft_rejected_with_full_residual():
    B, k, V = 2, 2, 3000
    lg = synth.logits(B, k, V, (33, 0))
    draft = np.array([[V, 5], [-7, 5]], np.int32)
    u = synth.uniforms(B, k, (33, 0))
    announce("rejection_out_of_range")
    L, nxt, _, pd = gpu_accept(lg, draft, 1.0, u)
    assert L.tolist() == [0, 0] and pd[0, 0] == 0 and pd[1, 0] == 0
    check_rejection(lg, draft, 1.0, u, L, nxt, pd)


def test_accept_repeated_calls_identical():
    B, k = 16, 5
    lg = dev_bf16(synth.logits(B, k, V_QWEN, (34, 0)))
    draft = dev(np.zeros((B, k), np.int32))
    u = dev(synth.uniforms(B, k, (34, 0)))
    ws = binding.new_workspace(binding.workspace_bytes_accept(B, k, V_QWEN))
    announce("accept_determinism")
    first = [t.clone() for t in binding.quasar_verify_accept(lg, draft, 1.0, u, workspace=ws)[:2]]
    for _ in range(20):
        again = binding.quasar_verify_accept(lg, draft, 1.0, u, workspace=ws)[:2]
        assert all(torch.equal(a, f) for a, f in zip(again, first))
