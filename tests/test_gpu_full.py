"""Parity at the full model sizes, in the launch configuration bench.py times
(hipGraph replay on a non-default stream): the 30-layer full_step, the 48-step
full_block and the long_block case (4 canvases over one 32768-token prefix).

The oracle cannot run a 25B-parameter step in seconds, so every check samples
what the oracle can recompute one piece at a time:
* layer outputs of sampled canvas rows, teacher-forced: the oracle takes the
  GPU's layer input (all rows, for the canvas keys and values) and the GPU's
  prefix KV cache of that layer, and recomputes the layer for the sampled rows
  (hidden state, expert choice, gates);
* the prefix KV of layer 0 at sampled positions, from the prefix embeddings;
* logits of sampled rows from the GPU's final hidden state;
* the sampler on the GPU's own fp32 logits at every position (Gumbel-max
  sample bit-exact; entropy; lock mask; re-randomised tokens; stop);
* the self-conditioning state of sampled rows and the next step's input.
Tolerances are those of test_gpu_step.py."""
import numpy as np
import pytest
import torch

from discrete_diffusion_decoding_amd import dg, synth
from discrete_diffusion_decoding_amd.configs import WORKLOADS, SamplerParams
from discrete_diffusion_decoding_amd.device import DeviceModel
from oracle import model as om
from oracle import sampler as osmp
from tests.gpu_util import announce, check_experts, dev, host, kv_layer, rel_l2

pytestmark = pytest.mark.gpu
SEED = 2024
FULL = WORKLOADS["full_step"].model
CHECK_LAYERS = (0, 1, FULL.n_layers // 2, FULL.n_layers - 1)
# Router logits (std ~1 in this model) inherit the relative error of the
# layer's hidden state, held to 1e-2, so each logit may move by up to
# LOGIT_ERR.  Two experts whose logits the oracle separates by less than twice
# that may swap (ROUTER_MARGIN), and a softmax gate g over the selected logits
# may move by up to 2 LOGIT_ERR g (first order: dg_i = g_i (dl_i - sum_j g_j
# dl_j)).  Deep layers and the 32768-key attention reach that level; the
# single-layer tests keep the tighter 1e-3 margin and 2e-3 gate bound.
LOGIT_ERR = 1e-2
ROUTER_MARGIN = 2 * LOGIT_ERR
GATE_RTOL = 2 * LOGIT_ERR


@pytest.fixture(scope="module")
def full():
    announce("full model: generate and upload 25.2B parameters")
    dm = DeviceModel(FULL, SEED)
    M = om.Model(FULL, synth.SynthWeights(FULL, SEED, cache_layers=True))
    yield dm, M
    dm.close()
    torch.cuda.empty_cache()


def _check_prefix_layer0(M, kv, Bp, P_max, prefix, positions):
    lw = M.layer_dense(0)
    for bp in range(Bp):
        K, V = kv_layer(kv, FULL, Bp, P_max, 0, bp, prefix.shape[1])
        _, k, v = M.qkv(M.embed(prefix[bp][positions]), lw, positions)
        assert rel_l2(K[positions], k) <= 1e-2
        assert rel_l2(V[positions], v) <= 1e-2


def _moe_given_experts(M, xn2, lw, idx):
    """The oracle's MoE output with the expert ids fixed to idx [n][k]: gates
    are the softmax of the oracle's router logits at those ids (used where the
    GPU's choice differs from the oracle's inside the near-tie margin)."""
    bits = lw["_bits"]
    logits = xn2 @ lw["w_router"].T
    sel = np.take_along_axis(logits, idx, axis=1)
    gates = om.softmax(sel, axis=-1)
    y = np.zeros_like(xn2)
    for r in range(xn2.shape[0]):
        for j in range(idx.shape[1]):
            e = int(idx[r, j])
            y[r] += gates[r, j] * om.gated_ffn(xn2[r:r + 1], om.widen(bits["w_gate"][e]),
                                               om.widen(bits["w_up"][e]), om.widen(bits["w_down"][e]))[0]
    if FULL.d_shared:
        y += om.gated_ffn(xn2, lw["w_gate_sh"], lw["w_up_sh"], lw["w_down_sh"])
    return y


def _check_layers(M, got, kv, Bp, P_max, P, T, rows_by_canvas):
    """Teacher-forced layer outputs for the sampled rows of each canvas.

    The layer's own contribution h_out - h_in is held to rel-L2 <= 2e-2, the
    bar of the single-layer test (the full model's layer inputs start as
    embeddings of norm ~1, so the contribution dominates h_out).  Expert sets
    must agree except inside the near-tie margin, where the oracle adopts the
    GPU's choice for its recomputation."""
    hd = got["hidden_dump"]
    ed, gd = got["expert_dump"], got["gate_dump"]
    pos = P + np.arange(T)
    for l in CHECK_LAYERS:
        lw = M.layer_dense(l)
        for b, rows in rows_by_canvas.items():
            r0 = b * T
            h_in = hd[l][r0:r0 + T].astype(np.float64)
            q, k, v = M.qkv(h_in, lw, pos)
            Kp, Vp = kv_layer(kv, FULL, Bp, P_max, l, 0 if Bp == 1 else b, P)
            kk = np.concatenate([Kp, k], axis=0)
            vv = np.concatenate([Vp, v], axis=0)
            o = om.attention(q[rows], kk, vv, np.ones((len(rows), P + T), dtype=bool))
            h_out, info = M.post_attention(h_in[rows], o, lw)
            gidx = ed[l][r0 + rows]
            excused = check_experts(gidx, gd[l][r0 + rows], info["experts"], info["gates"],
                                    info["router_logits"], FULL.top_k, margin_tol=ROUTER_MARGIN,
                                    gate_rtol=GATE_RTOL)
            if excused:
                h_att = h_in[rows] + o.reshape(len(rows), -1) @ lw["w_o"].T
                xn2 = om.rms_norm(h_att, lw["ffn_norm"], FULL.rms_eps)
                h_out = h_att + _moe_given_experts(M, xn2, lw, gidx.astype(np.int64))
            got_out = hd[l + 1][r0 + rows].astype(np.float64)
            per_row = np.linalg.norm(got_out - h_out, axis=1) / np.linalg.norm(h_out - h_in[rows], axis=1)
            err = rel_l2(got_out - h_in[rows], h_out - h_in[rows])
            assert err <= 2e-2, (l, b, err, np.round(per_row, 4).tolist(), excused)


def _check_sampler(got, b, T, seed, step, sp, stopped_expect=None):
    """The sampler decisions of canvas b against the oracle on the GPU's logits."""
    l32 = got["logits_dump"][b]
    H = osmp.entropy(l32)
    assert np.allclose(got["entropy"][b], H, rtol=1e-3)
    tau, inv_tau = osmp.temperature(step, sp.tau_start, sp.tau_end, sp.max_steps)
    xhat, _, _ = osmp.gumbel_argmax(l32, inv_tau, seed, step)
    assert np.array_equal(got["xhat"][b], xhat)
    assert np.array_equal(got["argmax"][b], np.argmax(l32, axis=-1))
    lock = osmp.lock_mask(H, sp.lock_rule, sp.lock_thresh)
    far = np.abs(H - sp.lock_thresh) > 1e-4
    assert np.array_equal(got["locked"][b].astype(bool)[far], lock[far])
    stop = step + 1 >= sp.max_steps or H.mean() < sp.stop_thresh
    if stopped_expect is not None:
        assert stop == stopped_expect
    assert bool(got["stopped"][b]) == stop and got["steps"][b] == step + 1
    if stop:
        assert np.array_equal(got["tokens"][b], got["xhat"][b])
    else:
        noise = osmp.rerandomized_tokens(seed, step, T, FULL.vocab)
        expect = np.where(got["locked"][b].astype(bool), got["xhat"][b], noise)
        assert np.array_equal(got["tokens"][b], expect)


def _check_logits_rows(M, got, rows_by_canvas, T):
    for b, rows in rows_by_canvas.items():
        logits = M.head(got["hidden_dump"][FULL.n_layers][b * T + rows].astype(np.float64))
        assert rel_l2(got["logits_dump"][b][rows], logits) <= 1e-2, b


def test_full_step_sampled_rows(full):
    """full_step: steps 0 and 1 (step 1 consumes step 0's self-conditioning)."""
    dm, M = full
    wl = WORKLOADS["full_step"]
    B, T, P = wl.batch, wl.canvas_len, wl.prefix_len
    prefix = synth.tokens(SEED, "prefix", (1, P), FULL.vocab)
    seeds = synth.row_seeds(SEED, B)
    kv = dm.kv_cache(1, P)
    ws = dm.workspace(B * T, P + T)
    stream = torch.cuda.Stream()
    announce("full_step: prefill 2048 tokens")
    pre = dev(prefix)
    torch.cuda.synchronize()   # the upload ran on the default stream
    dg.dg_prefill_prefix(dm.handle, pre, 1, P, P, kv, ws, stream=stream)
    sp = SamplerParams()
    sampler, keep = dg.make_sampler(sp, seeds)
    st = dm.canvas_state(B, T, dumps=True)
    torch.cuda.synchronize()   # zero-filled on the default stream
    dg.dg_init_canvas(dm.handle, dg.make_canvas(st), B, T, seeds, stream=stream)
    stream.synchronize()
    tok0 = host(st["tokens"])
    rng = np.random.default_rng(7)
    rows = {0: np.sort(rng.choice(T, 6, replace=False))}
    announce("full_step: prefix KV of layer 0")
    _check_prefix_layer0(M, kv, 1, P, prefix, np.sort(rng.choice(P, 16, replace=False)))
    prev = None
    for step in (0, 1):
        announce(f"full_step: step {step} (graph replay on a side stream)")
        dg.dg_denoise_step(dm.handle, kv, 1, P, P, B, T, dg.make_canvas(st), step, sampler, ws, stream=stream)
        stream.synchronize()
        got = {k: host(v) for k, v in st.items()}
        announce(f"full_step: oracle checks of step {step}")
        if step == 0:
            h0 = M.canvas_input(tok0[0][rows[0]], None)
        else:
            s_prev = synth.bf16_bits_to_f32(prev["self_cond"][0][rows[0]].view(np.uint16))
            h0 = M.canvas_input(prev["tokens"][0][rows[0]], s_prev)
        assert rel_l2(got["hidden_dump"][0][rows[0]], h0) <= 1e-2
        _check_layers(M, got, kv, 1, P, P, T, rows)
        _check_logits_rows(M, got, rows, T)
        _check_sampler(got, 0, T, int(seeds[0]), step, sp, stopped_expect=False)
        s_next = M.soft_embedding(got["logits_dump"][0][rows[0]])
        assert rel_l2(synth.bf16_bits_to_f32(got["self_cond"][0][rows[0]].view(np.uint16)), s_next) <= 1e-2
        prev = got
    del kv, ws, st
    torch.cuda.empty_cache()


def test_full_block_runs_the_step_budget(full):
    """full_block: dg_generate_block on the full model.  With random weights
    the entropy stays near ln V, nothing locks and the block takes all 48
    steps; the last step's sampler decisions match the oracle bit for bit."""
    dm, M = full
    wl = WORKLOADS["full_block"]
    B, T, P = wl.batch, wl.canvas_len, wl.prefix_len
    prefix = synth.tokens(SEED, "prefix", (1, P), FULL.vocab)
    seeds = synth.row_seeds(SEED + 1, B)
    kv = dm.kv_cache(1, P)
    ws = dm.workspace(B * T, P + T)
    stream = torch.cuda.Stream()
    pre = dev(prefix)
    torch.cuda.synchronize()   # the upload ran on the default stream
    dg.dg_prefill_prefix(dm.handle, pre, 1, P, P, kv, ws, stream=stream)
    sp = SamplerParams()
    sampler, keep = dg.make_sampler(sp, seeds)
    st = dm.canvas_state(B, T)
    st["logits_dump"] = torch.zeros(B, T, FULL.vocab, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()   # zero-filled on the default stream
    dg.dg_init_canvas(dm.handle, dg.make_canvas(st), B, T, seeds, stream=stream)
    announce("full_block: generate_block (48 steps)")
    dg.dg_generate_block(dm.handle, kv, 1, P, P, B, T, dg.make_canvas(st), sampler, ws, poll_every=8,
                         stream=stream)
    stream.synchronize()
    got = {k: host(v) for k, v in st.items()}
    assert got["steps"].tolist() == [sp.max_steps] and got["stopped"].tolist() == [1]
    assert not got["locked"].any()
    announce("full_block: oracle replay of the last step's sampler")
    _check_sampler(got, 0, T, int(seeds[0]), sp.max_steps - 1, sp, stopped_expect=True)
    del kv, ws, st
    torch.cuda.empty_cache()


def test_long_block_four_canvases_sampled_rows(full):
    """long_block: 4 canvases over one shared 32768-token prefix, one step."""
    dm, M = full
    wl = WORKLOADS["long_block"]
    B, T, P = wl.batch, wl.canvas_len, wl.prefix_len
    assert wl.prefix_batch == 1
    prefix = synth.tokens(SEED, "long_prefix", (1, P), FULL.vocab)
    seeds = synth.row_seeds(SEED + 2, B)
    kv = dm.kv_cache(1, P)
    ws = dm.workspace(B * T, P + T)
    stream = torch.cuda.Stream()
    announce("long_block: prefill 32768 tokens")
    pre = dev(prefix)
    torch.cuda.synchronize()   # the upload ran on the default stream
    dg.dg_prefill_prefix(dm.handle, pre, 1, P, P, kv, ws, stream=stream)
    sp = SamplerParams()
    sampler, keep = dg.make_sampler(sp, seeds)
    st = dm.canvas_state(B, T, dumps=True)
    torch.cuda.synchronize()   # zero-filled on the default stream
    dg.dg_init_canvas(dm.handle, dg.make_canvas(st), B, T, seeds, stream=stream)
    stream.synchronize()
    tok0 = host(st["tokens"])
    rng = np.random.default_rng(11)
    rows = {b: np.sort(rng.choice(T, 3, replace=False)) for b in range(B)}
    announce("long_block: prefix KV of layer 0")
    _check_prefix_layer0(M, kv, 1, P, prefix, np.sort(rng.choice(P, 16, replace=False)))
    announce("long_block: step 0 for 4 canvases")
    dg.dg_denoise_step(dm.handle, kv, 1, P, P, B, T, dg.make_canvas(st), 0, sampler, ws, stream=stream)
    stream.synchronize()
    got = {k: host(v) for k, v in st.items()}
    announce("long_block: oracle checks")
    for b in range(B):
        h0 = M.canvas_input(tok0[b][rows[b]], None)
        assert rel_l2(got["hidden_dump"][0][b * T + rows[b]], h0) <= 1e-2
    _check_layers(M, got, kv, 1, P, P, T, rows)
    _check_logits_rows(M, got, rows, T)
    for b in range(B):
        _check_sampler(got, b, T, int(seeds[b]), 0, sp, stopped_expect=False)
    del kv, ws, st
    torch.cuda.empty_cache()


def test_full_ar_steps(full):
    """Autoregressive steps of the full model after a 2048-token prompt, at
    positions 2048..2050 (the last two unaligned): the K/V each step writes
    in layer 0 match the oracle's projection of the token's embedding; on the
    GPU's own fp32 logits over the full vocabulary the sampled token and the
    argmax are the oracle sampler's, bit for bit, and the entropy agrees."""
    dm, M = full
    P0, n, tau = 2048, 3, 0.8
    P_max = P0 + 32
    prefix = synth.tokens(SEED, "prefix", (1, P0), FULL.vocab)
    seeds = synth.row_seeds(SEED + 7, 1)
    kv = dm.kv_cache(1, P_max)
    ws = dm.workspace(256, P_max)
    stream = torch.cuda.Stream()
    announce("full ar: prefill 2048")
    dg.dg_prefill_prefix(dm.handle, dev(prefix), 1, P0, P_max, kv, ws, stream=stream)
    tok = dev(np.array([int(prefix[0, -1])], np.int32))
    toks_in = [int(prefix[0, -1])]
    logits = torch.zeros(n, FULL.vocab, device="cuda")
    nxt = torch.zeros(n, dtype=torch.int32, device="cuda")
    amax = torch.zeros(n, dtype=torch.int32, device="cuda")
    ent = torch.zeros(n, device="cuda")
    for i in range(n):
        announce(f"full ar: dg_ar_step at P={P0 + i}")
        dg.dg_ar_step(dm.handle, kv, 1, P0 + i, P_max, tok, tau, seeds, nxt[i:i + 1], ws, argmax=amax[i:i + 1],
                      entropy=ent[i:i + 1], logits_dump=logits[i:i + 1], stream=stream)
        tok = nxt[i:i + 1]
    torch.cuda.synchronize()
    lg, nx, am, H = host(logits), host(nxt), host(amax), host(ent)
    K, V = kv_layer(kv, FULL, 1, P_max, 0, 0, P_max)
    toks_in += [int(x) for x in nx[:-1]]
    announce("full ar: oracle checks")
    lw = M.layer_dense(0)
    pos = np.arange(P0, P0 + n)
    _, k, v = M.qkv(M.embed(np.array(toks_in)), lw, pos)
    assert rel_l2(K[P0:P0 + n], k) <= 1e-2
    assert rel_l2(V[P0:P0 + n], v) <= 1e-2
    assert not K[P0 + n:].any() and not V[P0 + n:].any()
    for i in range(n):
        assert np.isfinite(lg[i]).all()
        t_g, a_g, H_g, _ = osmp.ar_sample(lg[i], tau, seeds[0], P0 + i)
        assert nx[i] == t_g and am[i] == a_g, i
        assert np.isclose(H[i], H_g, rtol=1e-4), i
