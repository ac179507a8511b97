"""Plain CPU forward pass of the discrete-diffusion MoE transformer.

Test infrastructure only (see oracle/__init__.py).  Float64 throughout; bf16
weights (uint16 bit patterns) are widened exactly.  Dense algebra uses numpy
matmul; everything else is written out as defined.

What the pages fix (DiffusionGemma technical report, laozijiushiniubi.cn
article section 2; gxsgwd.com news item): the model is a mixture-of-experts
transformer with 128 experts of which 8 are used per token; the prompt is
encoded with causal attention and the 256-token canvas with bidirectional
attention (every canvas token sees every other); self-conditioning feeds the
previous round's prediction back as an extra input.  Everything else below is
the plainest standard reading, chosen where the pages are silent:
pre-norm residual blocks, RMSNorm (eps 1e-6, multiplicative weight), per-head
QK RMSNorm, rotate-half RoPE (theta 1e4) at absolute positions, attention
scale 1/sqrt(head_dim), grouped-query heads, tanh-approximated GELU gated
FFNs, router softmax restricted to the top-k logits (ties to the lower
expert index), an always-on shared FFN, a tied embedding / LM head without
scaling, and a gated self-conditioning projection
h += sigmoid(g) * (s_prev W_sc) of the previous soft-prediction embedding.
"""
from __future__ import annotations

import numpy as np

F = np.float64


def widen(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(F)


def rms_norm(x, w, eps):
    x = np.asarray(x, dtype=F)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def rope(x, pos, theta):
    """Rotate-half rotary embedding over the full head dim.
    x: [n, heads, hd]; pos: [n] absolute positions."""
    hd = x.shape[-1]
    half = hd // 2
    j = np.arange(half, dtype=F)
    freq = np.exp(-(2.0 * j / hd) * np.log(theta))
    ang = np.asarray(pos, dtype=F)[:, None] * freq[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def gelu_tanh(x):
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))


def softmax(x, axis=-1):
    z = x - np.max(x, axis=axis, keepdims=True)
    e = np.exp(z)
    return e / np.sum(e, axis=axis, keepdims=True)


def attention(q, k, v, allowed):
    """q [n, H, hd]; k, v [m, Hkv, hd]; allowed [n, m] bool -> [n, H, hd].
    Query head h reads key/value head h // (H / Hkv)."""
    n, H, hd = q.shape
    Hkv = k.shape[1]
    grp = H // Hkv
    out = np.empty((n, H, hd), dtype=F)
    for h in range(H):
        g = h // grp
        s = (q[:, h, :] @ k[:, g, :].T) / np.sqrt(hd)
        s = np.where(allowed, s, -np.inf)
        out[:, h, :] = softmax(s, axis=-1) @ v[:, g, :]
    return out


def gated_ffn(x, wg, wu, wd):
    """(gelu_tanh(x Wg^T) * (x Wu^T)) Wd^T with [out, in] weight matrices."""
    return (gelu_tanh(x @ wg.T) * (x @ wu.T)) @ wd.T


def route(xn2, w_router, k):
    """Router logits, top-k expert ids (descending logit, ties -> lower id),
    and gates = softmax of the selected logits."""
    r = xn2 @ w_router.T
    order = np.argsort(-r, axis=-1, kind="stable")
    idx = order[:, :k]
    sel = np.take_along_axis(r, idx, axis=-1)
    return r, idx, softmax(sel, axis=-1)


class Model:
    """Forward pass over a weight provider with .glob() and .layer(l), each a
    dict of bf16 bit arrays named as in the synthetic generator."""

    def __init__(self, shape, weights):
        self.m = shape
        self.w = weights
        self._glob = None

    # -- weights --------------------------------------------------------------
    def glob(self):
        if self._glob is None:
            self._glob = {k: widen(v) for k, v in self.w.glob().items()}
        return self._glob

    def layer_dense(self, l):
        lw = self.w.layer(l)
        out = {k: widen(v) for k, v in lw.items()
               if k not in ("w_gate", "w_up", "w_down")}
        out["_bits"] = lw          # expert matrices are widened one expert at a time
        return out

    # -- blocks ---------------------------------------------------------------
    def qkv(self, h, lw, pos):
        m = self.m
        n = h.shape[0]
        xn = rms_norm(h, lw["attn_norm"], m.rms_eps)
        qkv = xn @ lw["w_qkv"].T
        qd, kd = m.n_heads * m.head_dim, m.n_kv_heads * m.head_dim
        q = qkv[:, :qd].reshape(n, m.n_heads, m.head_dim)
        k = qkv[:, qd:qd + kd].reshape(n, m.n_kv_heads, m.head_dim)
        v = qkv[:, qd + kd:].reshape(n, m.n_kv_heads, m.head_dim)
        q = rope(rms_norm(q, lw["q_norm"], m.rms_eps), pos, m.rope_theta)
        k = rope(rms_norm(k, lw["k_norm"], m.rms_eps), pos, m.rope_theta)
        return q, k, v

    def moe(self, xn2, lw):
        """Shared FFN + sum_j gate_j * expert_{e_j}(x); sparse dispatch."""
        m = self.m
        bits = lw["_bits"]
        logits, idx, gates = route(xn2, lw["w_router"], m.top_k)
        y = np.zeros_like(xn2)
        for e in range(m.n_experts):
            tok, slot = np.nonzero(idx == e)
            if tok.size == 0:
                continue
            ye = gated_ffn(xn2[tok], widen(bits["w_gate"][e]), widen(bits["w_up"][e]),
                           widen(bits["w_down"][e]))
            y[tok] += gates[tok, slot][:, None] * ye
        if m.d_shared:
            y += gated_ffn(xn2, lw["w_gate_sh"], lw["w_up_sh"], lw["w_down_sh"])
        return y, {"router_logits": logits, "experts": idx, "gates": gates}

    def post_attention(self, h, o, lw):
        m = self.m
        h = h + o.reshape(h.shape[0], m.n_heads * m.head_dim) @ lw["w_o"].T
        xn2 = rms_norm(h, lw["ffn_norm"], m.rms_eps)
        y, info = self.moe(xn2, lw)
        return h + y, info

    # -- prefix (causal) ------------------------------------------------------
    def prefill_hidden(self, h, records=None):
        """Causal forward of one prefix given its input hidden states [P, d].
        Returns per-layer (K, V) after QK-norm and RoPE, and the final hidden;
        if `records` is a list, each layer's routing record is appended to it."""
        h = np.asarray(h, dtype=F)
        P = h.shape[0]
        pos = np.arange(P)
        causal = np.tril(np.ones((P, P), dtype=bool))
        kv = []
        for l in range(self.m.n_layers):
            lw = self.layer_dense(l)
            q, k, v = self.qkv(h, lw, pos)
            o = attention(q, k, v, causal)
            h, info = self.post_attention(h, o, lw)
            if records is not None:
                records.append(info)
            kv.append((k, v))
        return kv, h

    def embed(self, tokens):
        return self.glob()["embed"][np.asarray(tokens)]

    def prefill_tokens(self, tokens, records=None):
        return self.prefill_hidden(self.embed(tokens), records)

    # -- canvas (bidirectional over prefix + canvas) ---------------------------
    def canvas_hidden(self, h, kv, P):
        """Forward of one canvas [T, d] whose queries see every prefix key and
        every canvas key.  Returns the final hidden and per-layer records."""
        h = np.asarray(h, dtype=F)
        T = h.shape[0]
        pos = P + np.arange(T)
        allowed = np.ones((T, P + T), dtype=bool)
        recs = []
        for l in range(self.m.n_layers):
            lw = self.layer_dense(l)
            h_in = h
            q, k, v = self.qkv(h, lw, pos)
            kp, vp = kv[l]
            kk = np.concatenate([kp, k], axis=0)
            vv = np.concatenate([vp, v], axis=0)
            o = attention(q, kk, vv, allowed)
            h, info = self.post_attention(h, o, lw)
            info["h_in"] = h_in
            recs.append(info)
        return h, recs

    def canvas_input(self, tokens, s_prev):
        """Embedding of the canvas tokens plus the self-conditioning term."""
        g = self.glob()
        h = g["embed"][np.asarray(tokens)]
        if self.m.self_cond and s_prev is not None:
            gate = 1.0 / (1.0 + np.exp(-g["self_cond_gate"]))
            h = h + gate * (np.asarray(s_prev, dtype=F) @ g["self_cond_w"].T)
        return h

    # -- autoregressive decoding (one token against the cache) ----------------
    def decode_token(self, token, kv, P):
        """One token at position P decoded against the cached K/V of positions
        0..P-1 (the model also generates autoregressively: arXiv abstract page;
        the per-step comparison of article section 5 is against this step).
        The token's query sees every cached key and its own.  Returns the final
        hidden [1, d] and per layer the token's own (K, V) [1, Hkv, hd]."""
        h = self.embed([token])
        pos = np.array([P])
        new = []
        for l in range(self.m.n_layers):
            lw = self.layer_dense(l)
            q, k, v = self.qkv(h, lw, pos)
            kp, vp = kv[l]
            kk = np.concatenate([kp[:P], k], axis=0)
            vv = np.concatenate([vp[:P], v], axis=0)
            o = attention(q, kk, vv, np.ones((1, P + 1), dtype=bool))
            h, _ = self.post_attention(h, o, lw)
            new.append((k, v))
        return h, new

    def head(self, h):
        """Final RMSNorm and tied LM head: logits [T, V]."""
        g = self.glob()
        hn = rms_norm(h, g["final_norm"], self.m.rms_eps)
        return hn @ g["embed"].T

    def soft_embedding(self, logits):
        """sum_v softmax(l)_v E_v: the prediction fed back by self-conditioning."""
        return softmax(np.asarray(logits, dtype=F), axis=-1) @ self.glob()["embed"]
