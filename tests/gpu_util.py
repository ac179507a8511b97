"""Shared helpers of the GPU parity tests (import only from gpu-marked tests)."""
import sys

import numpy as np
import torch


def announce(msg: str):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(x, dtype=None):
    t = torch.as_tensor(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def kv_layer(kv, m, Bp, P_max, l, bp, P):
    """(K, V) of prefix bp at layer l as float64 [P][Hkv][hd]; the cache holds
    per layer K [Bp][Hkv][P_max][hd] then V^T [Bp][Hkv][P_max / 32][hd][32]
    (tile-major)."""
    from discrete_diffusion_decoding_amd import synth
    n = Bp * m.n_kv_heads * P_max * m.head_dim
    x = kv.view(torch.int16)[2 * n * l: 2 * n * (l + 1)]
    K = x[:n].view(Bp, m.n_kv_heads, P_max, m.head_dim)[bp, :, :P, :]
    Vt = x[n:].view(Bp, m.n_kv_heads, P_max // 32, m.head_dim, 32)[bp]
    Vt = Vt.permute(1, 3, 0, 2).reshape(P_max, m.n_kv_heads, m.head_dim)[:P]
    K = synth.bf16_bits_to_f32(K.permute(1, 0, 2).contiguous().cpu().numpy().view(np.uint16))
    V = synth.bf16_bits_to_f32(Vt.contiguous().cpu().numpy().view(np.uint16))
    return K.astype(np.float64), V.astype(np.float64)


def near_tie_rows(router_logits, k, margin):
    """Rows whose k-th and (k+1)-th largest router logits lie within `margin`:
    there a rounding-level difference may swap an expert (ties aside, the
    choice is otherwise fixed)."""
    s = -np.sort(-np.asarray(router_logits, dtype=np.float64), axis=-1)
    return np.nonzero(s[:, k - 1] - s[:, k] < margin)[0]


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def topk_margin(router_logits, k):
    """Gap between the k-th and (k+1)-th largest router logit of each row."""
    s = -np.sort(-np.asarray(router_logits, dtype=np.float64), axis=-1)
    if s.shape[-1] <= k:
        return np.full(s.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]


def check_experts(gpu_idx, gpu_gate, orc_idx, orc_gate, orc_logits, k, margin_tol=1e-3, gate_tol=2e-3,
                  gate_rtol=0.0):
    """Expert sets must be equal except where the oracle's k-th / (k+1)-th
    router-logit margin is below margin_tol; gates within gate_tol + gate_rtol
    times the oracle's gate; returns the excused row count."""
    margin = topk_margin(orc_logits, k)
    excused = 0
    for r in range(orc_idx.shape[0]):
        gs, os_ = set(gpu_idx[r].tolist()), set(orc_idx[r].tolist())
        if gs != os_:
            assert margin[r] < margin_tol, (r, sorted(gs), sorted(os_), margin[r])
            excused += 1
            continue
        og = dict(zip(orc_idx[r].tolist(), orc_gate[r].tolist()))
        for e, gv in zip(gpu_idx[r].tolist(), gpu_gate[r].tolist()):
            assert abs(gv - og[e]) <= gate_tol + gate_rtol * og[e], (r, e, gv, og[e])
        assert abs(float(np.sum(gpu_gate[r])) - 1.0) < 1e-5
    return excused


class ScaledFinalNorm:
    """A weight provider whose final RMSNorm weight is `alpha` instead of 1:
    the logits scale by alpha, so the entropy falls and positions lock and
    canvases stop within a few steps (the random model's logits have std ~0.3
    at alpha 1, far from any lock).  Both the GPU model and the oracle read
    the same provider."""

    def __init__(self, base, alpha: float):
        from discrete_diffusion_decoding_amd import synth
        self.base, self.m = base, base.m
        self._fn = synth.f32_to_bf16_bits(np.full(base.m.d_model, alpha, np.float32))

    def glob(self):
        g = dict(self.base.glob())
        g["final_norm"] = self._fn
        return g

    def layer(self, l):
        return self.base.layer(l)


def lock_margin(H, rule: int, thresh: float):
    """Distance of each position's lock decision from its threshold: |H_i - t|
    for rule 0; for rule 1 (positions sorted by (H, index), locked while the
    running sum stays <= t) the distance of the running sum at the position's
    rank."""
    H = np.asarray(H, dtype=np.float64)
    if rule == 0:
        return np.abs(H - thresh)
    order = np.lexsort((np.arange(H.size), H))
    cum = np.empty(H.size)
    cum[order] = np.cumsum(H[order])
    return np.abs(cum - thresh)



def moe_given_experts(shape, xn2, lw, idx):
    """The oracle's MoE output with the expert ids fixed to idx [n][k]: gates
    are the softmax of the oracle's router logits at those ids (for rows where
    the GPU's choice differs from the oracle's inside the near-tie margin)."""
    from oracle import model as om
    bits = lw["_bits"]
    logits = xn2 @ lw["w_router"].T
    gates = om.softmax(np.take_along_axis(logits, idx, axis=1), axis=-1)
    y = np.zeros_like(xn2)
    for r in range(xn2.shape[0]):
        for j in range(idx.shape[1]):
            e = int(idx[r, j])
            y[r] += gates[r, j] * om.gated_ffn(xn2[r:r + 1], om.widen(bits["w_gate"][e]),
                                               om.widen(bits["w_up"][e]), om.widen(bits["w_down"][e]))[0]
    if shape.d_shared:
        y += om.gated_ffn(xn2, lw["w_gate_sh"], lw["w_up_sh"], lw["w_down_sh"])
    return y


def layer_teacher_forced(M, lw, h_in, kp, vp, P, g_idx, g_gate, margin_tol=1e-3, gate_tol=2e-3):
    """Layer output of one canvas [T, d] recomputed by the oracle from the GPU's
    layer input h_in and the GPU's prefix cache (kp, vp) of that layer.
    Expert sets must match the GPU's (g_idx, g_gate) except where the oracle's
    k-th / (k+1)-th router-logit margin is below margin_tol; there the oracle
    adopts the GPU's experts.  Returns (output, excused row count)."""
    from oracle import model as om
    m = M.m
    T = h_in.shape[0]
    q, k, v = M.qkv(h_in, lw, P + np.arange(T))
    o = om.attention(q, np.concatenate([kp, k]), np.concatenate([vp, v]), np.ones((T, P + T), dtype=bool))
    h_out, info = M.post_attention(h_in, o, lw)
    excused = []
    margin = topk_margin(info["router_logits"], m.top_k)
    for r in range(T):
        gs, os_ = set(g_idx[r].tolist()), set(info["experts"][r].tolist())
        if gs != os_:
            assert margin[r] < margin_tol, (r, sorted(gs ^ os_), float(margin[r]))
            excused.append(r)
            continue
        og = dict(zip(info["experts"][r].tolist(), info["gates"][r].tolist()))
        for e, gv in zip(g_idx[r].tolist(), g_gate[r].tolist()):
            assert abs(gv - og[e]) <= gate_tol, (r, e, gv, og[e])
    if excused:
        ex = np.array(excused)
        h_att = h_in[ex] + o[ex].reshape(len(ex), -1) @ lw["w_o"].T
        xn2 = om.rms_norm(h_att, lw["ffn_norm"], m.rms_eps)
        h_out[ex] = h_att + moe_given_experts(m, xn2, lw, np.asarray(g_idx[ex], dtype=np.int64))
    return h_out, len(excused)
