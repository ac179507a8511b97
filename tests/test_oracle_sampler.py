"""Pins of the oracle's sampler and block loop with stub models (CPU only).

The stub "models" return hand-made logits whose entropy is known in closed
form, so lock masks and the stop step are fixed by arithmetic, not by the
oracle itself."""
import json
import os

import numpy as np
import pytest
from scipy import stats

from discrete_diffusion_decoding_amd.configs import SamplerParams
from oracle import sampler as osmp

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))
V, T = 64, 16


def peaked(tokens_hot, margin):
    """logits [B, T, V]: zero except `margin` at tokens_hot[b, i]."""
    B, Tn = tokens_hot.shape
    l = np.zeros((B, Tn, V), np.float32)
    l[np.arange(B)[:, None], np.arange(Tn)[None, :], tokens_hot] = margin
    return l


def h_closed_form(a, n=V):
    """Entropy of softmax([a, 0, ..., 0]) over n entries."""
    p1 = np.exp(a) / (np.exp(a) + n - 1)
    q = 1 / (np.exp(a) + n - 1)
    return -p1 * np.log(p1) - (n - 1) * q * np.log(q)


def test_closed_form_entropy_matches_oracle():
    for a in (0.0, 1.0, 5.0, 12.0):
        l = np.zeros(V)
        l[3] = a
        assert np.isclose(osmp.entropy(l), h_closed_form(a), rtol=1e-12)


def run(stub, B=1, sp=SamplerParams(), seeds=(11, 12, 13, 14)):
    tok0 = np.stack([osmp.init_canvas(seeds[b], T, V) for b in range(B)])
    return osmp.generate_block(None, None, 0, tok0, list(seeds[:B]), sp,
                               logits_fn=stub, record=True)


def test_collapsed_model_stops_after_one_step():
    stub = lambda tok, s_prev, s: peaked(np.full((1, T), 7), 60.0)
    tokens, steps, hist = run(stub)
    assert steps.tolist() == [1] and len(hist) == 1
    assert np.all(tokens == 7)


def test_never_confident_model_runs_the_full_budget():
    stub = lambda tok, s_prev, s: np.zeros((1, T, V), np.float32)
    tokens, steps, hist = run(stub)
    assert steps.tolist() == [GOLD["max_steps"]["value"]] == [len(hist)]
    assert not any(h["lock"].any() for h in hist)
    assert np.allclose(hist[0]["entropy"], np.log(V))


def test_stop_step_follows_closed_form_entropy():
    margins = np.linspace(0.0, 14.0, 48)
    stub = lambda tok, s_prev, s: peaked(np.full((1, T), 5), margins[s])
    expect = next(s for s in range(48) if h_closed_form(np.float32(margins[s])) < 0.1) + 1
    _, steps, hist = run(stub)
    assert steps[0] == expect
    # the lock rule is per-position H < 0.5: the first step with H < 0.5 locks everything
    first_lock = next(s for s in range(48) if h_closed_form(np.float32(margins[s])) < 0.5)
    for s, h in enumerate(hist):
        assert h["lock"].all() == (s >= first_lock) and (h["lock"].any() == (s >= first_lock))


def test_locked_tokens_stay_editable():
    hot = lambda s: np.full((1, T), 3 if s == 0 else 9)
    stub = lambda tok, s_prev, s: peaked(hot(s), 40.0) if s < 2 else np.zeros((1, T, V), np.float32)
    sp = SamplerParams(stop_thresh=-1.0)          # never stop early
    _, _, hist = run(stub, sp=sp)
    assert np.all(hist[0]["lock"]) and np.all(hist[0]["tokens"] == 3)
    assert np.all(hist[1]["lock"]) and np.all(hist[1]["tokens"] == 9)   # changed after lock


def test_unlocked_positions_are_rerandomised_uniformly():
    sp = SamplerParams(stop_thresh=-1.0)
    stub = lambda tok, s_prev, s: np.zeros((1, T, V), np.float32)
    _, _, hist = run(stub, sp=sp)
    for s, h in enumerate(hist[:-1]):
        assert np.array_equal(h["tokens"][0], osmp.rerandomized_tokens(11, s, T, V))
    # the last round outputs its samples, not noise
    assert np.array_equal(hist[-1]["tokens"][0], hist[-1]["xhat"][0])
    draws = np.concatenate([osmp.rerandomized_tokens(5, s, 4096, V) for s in range(16)])
    assert stats.chisquare(np.bincount(draws, minlength=V)).pvalue > 1e-4


def test_lock_rule_thresholds_and_cumulative_variant():
    H = np.array([0.5 - 1e-6, 0.5, 0.5 + 1e-6, 0.0])
    assert osmp.lock_mask(H, 0, 0.5).tolist() == [True, False, False, True]
    thr = GOLD["lock_cumulative_entropy"]["value"]
    H = np.array([0.05, 0.02, 0.04, 0.3, 0.01])
    assert osmp.lock_mask(H, 1, thr).tolist() == [False, True, True, False, True]
    H = np.array([0.03, 0.03, 0.03, 0.03, 0.2])   # ties broken by position
    assert osmp.lock_mask(H, 1, thr).tolist() == [True, True, True, False, False]
    assert not osmp.lock_mask(np.array([0.2, 0.3]), 1, thr).any()


def test_stop_rule_variant_needs_stable_argmax():
    thr = GOLD["stop_mean_entropy"]["value"]
    H = np.full(T, 0.001)
    a = np.arange(T)
    assert not osmp.stop_decision(H, a, a, False, 0, 48, 1, thr)[0]
    assert osmp.stop_decision(H, a, a, True, 3, 48, 1, thr)[0]
    assert not osmp.stop_decision(H, a, a[::-1], True, 3, 48, 1, thr)[0]
    assert osmp.stop_decision(np.full(T, 1.0), a, a[::-1], True, 47, 48, 1, thr)[0]


def test_rows_stop_independently():
    def stub(tok, s_prev, s):
        l = np.zeros((2, T, V), np.float32)
        l[0] = peaked(np.full((1, T), 2), 60.0)[0]
        return l
    tokens, steps, hist = run(stub, B=2)
    assert steps.tolist() == [1, 48]
    assert np.all(tokens[0] == 2)
    assert np.all(hist[-1]["tokens"][0] == 2)          # frozen after stopping


def test_sample_step_uses_temperature_schedule():
    l = np.random.default_rng(0).standard_normal((1, T, V)).astype(np.float32)
    sp = SamplerParams()
    for s in (0, 20, 47):
        _, _, _, _, info = osmp.sample_step(l, np.zeros((1, T)), np.zeros((1, T)), False,
                                            np.zeros(1, bool), np.zeros(1), s, [3], sp)
        assert info["inv_tau"] == osmp.temperature(s, 0.8, 0.4, 48)[1]
        xhat, _, _ = osmp.gumbel_argmax(l[0], info["inv_tau"], 3, s)
        assert np.array_equal(info["xhat"][0], xhat)


def test_init_canvas_reproducible_uniform():
    a = osmp.init_canvas(77, 256, 262144)
    assert np.array_equal(a, osmp.init_canvas(77, 256, 262144))
    assert a.min() >= 0 and a.max() < 262144 and len(set(a.tolist())) > 250
    assert not np.array_equal(a, osmp.init_canvas(78, 256, 262144))


def test_ar_sample_is_a_softmax_sample_at_its_temperature():
    """The autoregressive next token is a Gumbel-max draw, so over seeds (and
    over decode positions) it is distributed as softmax(l / tau); a tiny tau
    gives the argmax; the entropy and argmax outputs are those of the logits."""
    l = np.array([1.0, 0.0, -0.5, 2.0, 0.3, -1.0, 0.8, 0.1, 0.4, -0.2], np.float32)
    tau = 0.7
    z = np.exp((l.astype(np.float64) - l.max()) / tau)
    p = z / z.sum()
    n = 4000
    by_seed = np.bincount([osmp.ar_sample(l, tau, 1000 + s, 5)[0] for s in range(n)], minlength=l.size)
    by_pos = np.bincount([osmp.ar_sample(l, tau, 77, 100 + q)[0] for q in range(n)], minlength=l.size)
    assert stats.chisquare(by_seed, n * p).pvalue > 1e-4
    assert stats.chisquare(by_pos, n * p).pvalue > 1e-4
    # draws at different positions are independent: they agree about sum p^2 of the time
    a = np.array([osmp.ar_sample(l, tau, 5 + s, 9)[0] for s in range(n)])
    b = np.array([osmp.ar_sample(l, tau, 5 + s, 10)[0] for s in range(n)])
    agree = float(np.mean(a == b))
    assert abs(agree - float(np.sum(p * p))) < 4 * np.sqrt(agree * (1 - agree) / n)
    for s in range(20):
        tok, amax, H, gap = osmp.ar_sample(l, 1e-4, s, 3)
        assert tok == 3 and amax == 3 and gap > 0
    assert np.isclose(osmp.ar_sample(l, 1.0, 0, 0)[2], osmp.entropy(l), rtol=0, atol=1e-12)
    assert osmp.ar_inv_tau(0.8) == np.float32(1.25)
