"""Statistical pins for the oracle's verification decisions.

* Greedy acceptance: with drafts that match the target's argmax independently
  with probability p, the mean accepted length tau = accepted + 1 has the closed
  form (1 - p^(k+1)) / (1 - p).
* Rejection sampling with a one-hot draft keeps the verifier's distribution:
  the first emitted token is distributed as p_0 whatever the draft is
  [Quasar, pt page §2 item 4 and zh page §2 pipeline: lossless rejection sampling].
"""
import json
import os

import numpy as np
from scipy import stats

from oracle import quasar_oracle as orc
from w8a8_quantized_speculative_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_greedy_mean_acceptance_matches_closed_form():
    k, V, p, B = 5, 97, 0.3, 4000
    lg = synth.logits(B, k, V, (3, 0), sigma=3.0)
    g = orc.argmax_lowest(lg)
    draft = synth.draft_tokens(g[:, :k], V, p, (3, 0))
    L, nxt, g2 = orc.greedy_accept(lg, draft)
    tau = L + 1
    mean_closed = (1 - p ** (k + 1)) / (1 - p)
    # exact second moment of tau under the same model, for the 4-sigma band
    probs = np.array([(p ** t) * (1 - p) for t in range(k)] + [p ** k])
    values = np.arange(1, k + 2)
    assert abs(probs.sum() - 1) < 1e-12 and abs((probs * values).sum() - mean_closed) < 1e-12
    sd = np.sqrt((probs * values ** 2).sum() - mean_closed ** 2)
    assert abs(tau.mean() - mean_closed) < 4 * sd / np.sqrt(B)
    assert np.array_equal(nxt, g2[np.arange(B), L])


def test_synthetic_acceptance_model_is_near_the_pages_numbers():
    """The p = 0.3, k = 5 drafts give E[tau] = 1.4275, close to the pages' 1.40
    (Quasar on Qwen3 at T = 0); int8 halves the weight bytes (2 -> 1 per param)."""
    nums = json.load(open(os.path.join(GOLDEN, "pages_numbers.json")))
    k = nums["draft_length_example"]["value"]
    e_tau = (1 - 0.3 ** (k + 1)) / (1 - 0.3)
    assert abs(e_tau - nums["mean_acceptance_length_quasar_qwen3_t0"]["value"]) < 0.05
    assert nums["bytes_per_weight_int8"]["value"] / nums["bytes_per_weight_bf16"]["value"] == \
        nums["weight_footprint_reduction"]["value"]


def _first_token_counts(lg_bits, draft_tok, T, trials, seed):
    V = lg_bits.shape[-1]
    g = np.random.default_rng(seed)
    counts = np.zeros(V, np.int64)
    for _ in range(trials):
        u = g.random((1, 2))
        L, nxt, *_ = orc.rejection_accept(lg_bits, np.array([[draft_tok]]), T, u)
        counts[draft_tok if L[0] == 1 else nxt[0]] += 1
    return counts


def test_rejection_sampling_is_lossless_chi_square():
    V = 8
    lg = synth.to_bf16_bits(np.array([[[1.0, -0.5, 2.0, 0.0, 0.3, -1.0, 1.5, 0.7]] * 2], np.float32))
    T = 1.0
    p0 = orc.softmax_f64(lg[0, 0], T)
    for d in (2, 5):     # a likely and an unlikely draft
        counts = _first_token_counts(lg, d, T, 20000, seed=100 + d)
        chi2, pval = stats.chisquare(counts, p0 * counts.sum())
        assert pval > 1e-3, (d, counts, p0)


def test_rejection_one_hot_logits_always_accept_that_token():
    V = 16
    lg = np.full((1, 3, V), -80.0, np.float32)
    lg[0, :, 4] = 80.0
    bits = synth.to_bf16_bits(lg)
    g = np.random.default_rng(1)
    for _ in range(200):
        u = g.random((1, 3))
        L, nxt, p_d, *_ = orc.rejection_accept(bits, np.array([[4, 4]]), 1.0, u)
        assert L[0] == 2 and nxt[0] == 4
        L, nxt, *_ = orc.rejection_accept(bits, np.array([[3, 4]]), 1.0, u)
        assert L[0] == 0 and nxt[0] == 4


def test_rejection_at_low_temperature_equals_greedy():
    B, k, V = 30, 4, 50
    lg = synth.logits(B, k, V, (4, 0), sigma=3.0)
    vals = orc.bf16_to_f32(lg)
    # untied maxima: the gap to the runner-up is large compared with T
    top2 = np.sort(vals, axis=-1)[..., -2:]
    keep = np.all(top2[..., 1] - top2[..., 0] > 0.05, axis=1)
    lg = lg[keep]
    g = orc.argmax_lowest(lg)
    draft = synth.draft_tokens(g[:, :k], V, 0.6, (4, 0))
    Lg, ng, _ = orc.greedy_accept(lg, draft)
    u = synth.uniforms(lg.shape[0], k, (4, 0)).astype(np.float64) * 0.999
    Lr, nr, *_ = orc.rejection_accept(lg, draft, 1e-3, u)
    assert np.array_equal(Lg, Lr) and np.array_equal(ng, nr)


def test_rejection_out_of_range_draft_has_zero_probability():
    lg = synth.logits(1, 2, 10, (5, 0))
    L, nxt, p_d, *_ = orc.rejection_accept(lg, np.array([[10, -3]]), 1.0, np.zeros((1, 3)))
    assert L[0] == 0 and p_d[0, 0] == 0 and p_d[0, 1] == 0
