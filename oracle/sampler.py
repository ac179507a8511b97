"""The denoising sampler: entropy, Gumbel-max sampling, locking, stopping.

Test infrastructure only (see oracle/__init__.py).

What the pages fix (laozijiushiniubi.cn article, sections 1 and 4):
* multinomial (uniform-noise) diffusion: noise is any vocabulary token, and a
  token that was locked can still change in a later round;
* per-position entropy measures the model's uncertainty; positions whose
  prediction is confident are kept, the rest are re-randomised ("maximum
  uncertainty") and refined again in the next round;
* the temperature falls linearly from 0.8 to 0.4 over the rounds;
* generation stops adaptively on low mean entropy, with a cap of 48 rounds.
The pages' own thresholds (lock by sorted cumulative entropy <= 0.1; stop on
mean entropy < 0.005 with an unchanged argmax sequence) are rule 1 below; rule
0 is the per-position form (lock H_i < 0.5, stop mean H < 0.1).

Readings taken where the pages are silent: entropy at temperature 1 in nats;
the locked token is this round's sample; the lock is recomputed every round;
re-randomised tokens are uniform over the vocabulary; the round that stops
outputs its samples without re-randomising; the temperature is linear over the
step budget.  Random numbers are Philox4x32-10 words keyed by the row seed:
  Gumbel of (position i, vocab v) at step s: counter (v, i >> 2, s, 0), word i & 3
  re-randomised token of position i:         counter (i, 0, s, 1), word 0
  initial canvas token of position i:        counter (i, 0, 2^32 - 1, 1), word 0
  autoregressive token at position p, vocab v: counter (v >> 2, p, 0, 2), word v & 3
(the last is for the one-token AR step that the pages compare against, article
section 5; the next token is a Gumbel-max sample of softmax(l / tau)).
"""
from __future__ import annotations

import numpy as np

from .rng import philox4x32, seed_key, uniform_open01, uniform_index, gumbel_f32

INIT_STEP = 0xFFFFFFFF


def temperature(step: int, tau_start, tau_end, max_steps: int):
    """tau_s = tau0 + (tau1 - tau0) * s / (S - 1) in float64 (tau0, tau1 are the
    fp32 parameters widened); returns (tau, fp32(1 / tau))."""
    t0 = float(np.float32(tau_start))
    t1 = float(np.float32(tau_end))
    if max_steps > 1:
        tau = t0 + ((t1 - t0) * float(step)) / float(max_steps - 1)
    else:
        tau = t0
    return tau, np.float32(1.0 / tau)


def entropy(logits):
    """H = -sum p ln p of softmax(logits) along the last axis, float64, nats."""
    l = np.asarray(logits, dtype=np.float64)
    m = np.max(l, axis=-1, keepdims=True)
    z = l - m
    e = np.exp(z)
    Z = np.sum(e, axis=-1, keepdims=True)
    return (np.log(Z) - np.sum(e * z, axis=-1, keepdims=True) / Z)[..., 0]


def gumbel_argmax(logits_f32, inv_tau, seed, step: int):
    """x_hat_i = argmax_v fp32(l_iv * inv_tau) + G_iv (ties -> lowest v) for one
    canvas row [T, V].  Also returns the best score and the gap to the runner-up."""
    l = np.asarray(logits_f32, dtype=np.float32)
    T, V = l.shape
    k0, k1 = seed_key(seed)
    v = np.arange(V, dtype=np.uint64)
    xhat = np.empty(T, dtype=np.int64)
    best = np.empty(T, dtype=np.float32)
    gap = np.empty(T, dtype=np.float32)
    inv = np.float32(inv_tau)
    for g in range((T + 3) // 4):
        words = philox4x32(v, g, step & 0xFFFFFFFF, 0, k0, k1)
        for j in range(4):
            i = 4 * g + j
            if i >= T:
                break
            score = (l[i] * inv).astype(np.float32) + gumbel_f32(uniform_open01(words[j]))
            a = int(np.argmax(score))
            xhat[i] = a
            best[i] = score[a]
            s2 = score.copy()
            s2[a] = -np.inf
            gap[i] = score[a] - np.max(s2)
    return xhat, best, gap


def rerandomized_tokens(seed, step: int, T: int, V: int):
    k0, k1 = seed_key(seed)
    i = np.arange(T, dtype=np.uint64)
    w = philox4x32(i, 0, step & 0xFFFFFFFF, 1, k0, k1)[0]
    return uniform_index(w, V)


def init_canvas(seed, T: int, V: int):
    """Initial canvas: T tokens uniform over the vocabulary."""
    return rerandomized_tokens(seed, INIT_STEP, T, V)


def lock_mask(H, rule: int, thresh: float):
    H = np.asarray(H, dtype=np.float64)
    if rule == 0:
        return H < thresh
    # rule 1: sort positions by (entropy, index) ascending, lock the longest
    # prefix of that order whose cumulative entropy stays <= thresh.
    order = np.lexsort((np.arange(H.size), H))
    cum = np.cumsum(H[order])
    n = int(np.searchsorted(cum, thresh, side="right"))
    out = np.zeros(H.size, dtype=bool)
    out[order[:n]] = True
    return out


def stop_decision(H, amax, prev_amax, prev_valid: bool, step: int, max_steps: int,
                  rule: int, thresh: float):
    meanH = float(np.mean(np.asarray(H, dtype=np.float64)))
    if rule == 0:
        crit = meanH < thresh
    else:
        crit = meanH < thresh and prev_valid and np.array_equal(amax, prev_amax)
    return bool(crit or step + 1 >= max_steps), meanH


def sample_step(logits, tokens, prev_amax, prev_valid, stopped, steps, step: int,
                seeds, sp):
    """One sampler round for B canvas rows.

    logits [B, T, V] (fp32 values define the Gumbel scores; entropy in fp64);
    tokens, prev_amax [B, T]; stopped, steps [B].  Rows already stopped are left
    unchanged.  Returns the new state and per-row diagnostics."""
    l32 = np.asarray(logits, dtype=np.float32)
    B, T, V = l32.shape
    tokens = np.array(tokens, dtype=np.int64, copy=True)
    amax_out = np.array(prev_amax, dtype=np.int64, copy=True)
    stopped = np.array(stopped, dtype=bool, copy=True)
    steps = np.array(steps, dtype=np.int64, copy=True)
    _, inv_tau = temperature(step, sp.tau_start, sp.tau_end, sp.max_steps)
    out = {"entropy": np.zeros((B, T)), "xhat": np.zeros((B, T), np.int64),
           "lock": np.zeros((B, T), bool), "gap": np.zeros((B, T), np.float32),
           "mean_entropy": np.zeros(B), "inv_tau": inv_tau}
    for b in range(B):
        if stopped[b]:
            continue
        H = entropy(l32[b])
        xhat, _, gap = gumbel_argmax(l32[b], inv_tau, seeds[b], step)
        amax = np.argmax(l32[b], axis=-1)
        lock = lock_mask(H, sp.lock_rule, sp.lock_thresh)
        stop, meanH = stop_decision(H, amax, prev_amax[b], prev_valid, step, sp.max_steps,
                                    sp.stop_rule, sp.stop_thresh)
        if stop:
            tokens[b] = xhat
        else:
            noise = rerandomized_tokens(seeds[b], step, T, V)
            tokens[b] = np.where(lock, xhat, noise)
        amax_out[b] = amax
        stopped[b] = stop
        steps[b] = step + 1
        out["entropy"][b], out["xhat"][b], out["lock"][b] = H, xhat, lock
        out["gap"][b], out["mean_entropy"][b] = gap, meanH
    return tokens, amax_out, stopped, steps, out


def generate_block(model, kv, P, tokens0, seeds, sp, logits_fn=None, record=False):
    """Refine B canvases until every row stops (or the step budget ends).

    `model` is an oracle.model.Model; kv[b] the per-layer prefix (K, V) seen by
    canvas b.  `logits_fn(tokens [B,T], s_prev [B,T,d]) -> logits` may replace
    the model (stub models in tests).  Returns tokens, steps, history."""
    tokens = np.array(tokens0, dtype=np.int64, copy=True)
    B, T = tokens.shape
    d = model.m.d_model if model is not None else 0
    s_prev = np.zeros((B, T, d)) if d else None
    amax = np.zeros((B, T), np.int64)
    stopped = np.zeros(B, bool)
    steps = np.zeros(B, np.int64)
    hist = []
    for s in range(sp.max_steps):
        if stopped.all():
            break
        if logits_fn is not None:
            logits = logits_fn(tokens, s_prev, s)
        else:
            logits = np.stack([model.head(model.canvas_hidden(
                model.canvas_input(tokens[b], s_prev[b]), kv[b], P)[0]) for b in range(B)])
        live = ~stopped
        tokens, amax, stopped, steps, info = sample_step(
            logits, tokens, amax, s > 0, stopped, steps, s, seeds, sp)
        if model is not None and model.m.self_cond:
            for b in np.nonzero(live)[0]:
                s_prev[b] = model.soft_embedding(logits[b])
        if record:
            hist.append({"tokens": tokens.copy(), **info})
    return tokens, steps, hist


def ar_inv_tau(tau) -> np.float32:
    """fp32(1 / tau) of the fp32 temperature, the quotient taken in float64."""
    return np.float32(1.0 / float(np.float32(tau)))


def ar_sample(logits_f32, tau, seed, pos: int):
    """Next token of an autoregressive step at decode position pos: argmax_v
    fp32(l_v * inv_tau) + G_v, ties to the lowest v, with G_v the Gumbel noise
    of Philox block (v >> 2, pos, 0, 2), word v & 3.  Returns (token, argmax of
    the logits, entropy in nats, gap between the best two scores)."""
    l = np.asarray(logits_f32, dtype=np.float32)
    V = l.shape[0]
    k0, k1 = seed_key(seed)
    blocks = philox4x32(np.arange((V + 3) // 4, dtype=np.uint64), pos & 0xFFFFFFFF, 0, 2, k0, k1)
    words = np.stack(blocks, axis=1).reshape(-1)[:V]
    score = (l * ar_inv_tau(tau)).astype(np.float32) + gumbel_f32(uniform_open01(words))
    tok = int(np.argmax(score))
    rest = score.copy()
    rest[tok] = -np.inf
    return tok, int(np.argmax(l)), float(entropy(l)), float(score[tok] - np.max(rest))
