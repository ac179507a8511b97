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
