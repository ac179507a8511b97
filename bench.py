"""Benchmark of one denoising step on one MI355X.

Workload (default "full_step"): the 30-layer random-init MoE model (d_model
2816, 16/8 heads of 256, 128 experts top-8 of width 704 plus a shared FFN of
2112, vocabulary 262144, tied embedding, self-conditioning; ~25.2B params in
bf16), one shared 2048-token prefix already encoded in the KV cache, one
256-token canvas.  A step is one full pass of the hot path: embedding +
self-conditioning, 30 layers, LM head, entropy, Gumbel-max sampling, lock /
re-randomise / stop, soft-prediction embedding.

Prints ONE JSON line: output tokens/s (= B * 256 / (steps per block * time per
step), steps per block measured with dg_generate_block), ms per step, the
roofline of the dominant kernel (grouped expert gate/up GEMM, timed with HIP
events inside libdg during a profiled pass right after the timed region) and
the CPU oracle timed on a bounded sample on this machine's host cores."""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "output tok/s at batch 1 (256-tok canvas), ms per denoising step, % roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(m, B, T, P, touched, Bp=1):
    """HBM bytes a step must move at minimum: every touched weight once, the
    embedding table once, each prompt's KV once, canvas activations ignored."""
    d, hd = m.d_model, m.head_dim
    dense = (m.qkv_dim * d + d * m.n_heads * hd + m.n_experts * d + 3 * d * m.d_shared) * 2
    expert = 3 * m.d_expert * d * 2
    kv = Bp * 2 * P * m.n_kv_heads * hd * 2
    per_layer = [dense + t * expert + kv for t in touched]
    glob = m.vocab * d * 2 + (d * d * 2 if m.self_cond else 0)
    return sum(per_layer) + glob


def algorithmic_flops(m, B, T, P):
    R = B * T
    d, hd = m.d_model, m.head_dim
    per_layer = 2 * R * (m.qkv_dim * d + d * m.n_heads * hd + m.n_experts * d)
    per_layer += 2 * R * m.top_k * 3 * d * m.d_expert + 2 * R * 3 * d * m.d_shared
    per_layer += 4 * R * (P + T) * m.n_heads * hd
    head = 2 * R * m.vocab * d * (2 if m.self_cond else 1) + (2 * R * d * d if m.self_cond else 0)
    return m.n_layers * per_layer + head


def gateup_bytes(m, R, touched_mean):
    """Algorithmic bytes of one grouped gate/up launch: touched experts' W_gate
    and W_up, the gathered activation rows, the GELU-gated outputs."""
    return touched_mean * 2 * m.d_expert * m.d_model * 2 + R * m.top_k * (m.d_model + m.d_expert) * 2


def kernel_hash():
    h = hashlib.sha256()
    p = os.path.join(ROOT, "discrete_diffusion_decoding_amd", "csrc", "k_gemm.hip")
    h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def profile_record(kh, workload):
    """The committed rocprofv3 record of the gate/up kernel (HBM bytes per
    launch from the counter runs, mean duration from the kernel trace), if it
    was taken on the current kernel source and on this workload."""
    p = os.path.join(ROOT, "profiles", "expert_gateup_full_step_counters.json")
    if not os.path.exists(p):
        return {}
    try:
        d = json.load(open(p))
    except Exception:
        return {}
    if d.get("kernel_source_sha256_16") != kh or d.get("workload") != workload:
        return {}
    return d


def cpu_baseline(m_full, seed):
    """Time the oracle on a bounded sample of the same step: one full-width
    layer over a 2048-token prefix KV (synthetic K/V) for 256 canvas rows, and
    the LM head + sampler + soft embedding over 1/16 of the vocabulary; scaled
    to a whole 30-layer step and to the block's output tokens/s."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from discrete_diffusion_decoding_amd import synth
    from discrete_diffusion_decoding_amd.configs import FULL_LAYER
    from oracle import model as om
    from oracle import sampler as osmp

    T, P = 256, 2048
    lm = om.Model(FULL_LAYER, synth.SynthWeights(FULL_LAYER, seed, cache_layers=True))
    hc = synth.hidden(seed, "cpu_canvas", (T, FULL_LAYER.d_model))
    Kp = synth.hidden(seed, "cpu_k", (P, FULL_LAYER.n_kv_heads, FULL_LAYER.head_dim))
    Vp = synth.hidden(seed, "cpu_v", (P, FULL_LAYER.n_kv_heads, FULL_LAYER.head_dim))
    lm.layer_dense(0)  # generate the weights outside the timed region
    t0 = time.perf_counter()
    lm.canvas_hidden(hc, [(Kp.astype(np.float64), Vp.astype(np.float64))], P)
    t_layer = time.perf_counter() - t0
    frac = 16
    Vs = m_full.vocab // frac
    E = synth.normal_bf16(seed, "embed", (m_full.vocab, m_full.d_model))[:Vs]
    g = {"embed": E, "final_norm": np.full(m_full.d_model, synth.BF16_ONE, np.uint16)}

    class _W:
        def glob(self):
            return g

    hm = om.Model(m_full, _W())
    hm.glob()
    t0 = time.perf_counter()
    logits = hm.head(hc)
    osmp.entropy(logits)
    osmp.gumbel_argmax(logits.astype(np.float32), np.float32(1.25), 1, 1)
    hm.soft_embedding(logits)
    t_head = time.perf_counter() - t0
    step_s = m_full.n_layers * t_layer + frac * t_head
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    try:
        host_cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        host_cores = os.cpu_count() or 1
    return {
        "value": round(T / (48 * step_s), 4), "unit": "tok/s", "cores": int(threads), "host_cores": int(host_cores),
        "kind": "oracle",
        "sample": (f"float64 numpy oracle: one full-width layer step (256 canvas rows, 2048-key prefix) "
                   f"{t_layer:.2f}s x {m_full.n_layers} layers + LM head/entropy/Gumbel/soft-embedding on 1/{frac} "
                   f"of the vocabulary {t_head:.2f}s x {frac} = {step_s:.1f}s per step, 48 steps per block"),
        "ms_per_step": round(step_s * 1e3, 1),
    }


def multi_block(dg, synth, dm, prefix, B, T, P, nb, sp, seed, stream):
    """Generation as the pages time it: the prompt is prefilled once, then nb
    blocks are denoised one after another; each finished block is encoded onto
    the cache (dg_prefill_append) so the next block sees it as prefix."""
    import torch
    P_max = P + nb * T
    kv = dm.kv_cache(B, P_max)
    ws = dm.workspace(B * T, P_max + T)
    st = dm.canvas_state(B, T)
    canvas = dg.make_canvas(st)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 + 2 * nb)]
    ev[0].record()
    dg.dg_prefill_prefix(dm.handle, prefix, B, P, P_max, kv, ws, stream=stream)
    ev[1].record()
    steps, Pc = [], P
    for k in range(nb):
        seeds = synth.row_seeds(seed + 1 + k, B)
        sampler, keep = dg.make_sampler(sp, seeds)
        dg.dg_init_canvas(dm.handle, canvas, B, T, seeds, stream=stream)
        dg.dg_generate_block(dm.handle, kv, B, Pc, P_max, B, T, canvas, sampler, ws, poll_every=8, stream=stream)
        ev[2 + 2 * k].record()
        dg.dg_prefill_append(dm.handle, st["tokens"], B, Pc, T, P_max, kv, ws, stream=stream)
        ev[3 + 2 * k].record()
        Pc += T
        torch.cuda.synchronize()
        steps.append(st["steps"].cpu().numpy().tolist())
    torch.cuda.synchronize()
    e2e = ev[0].elapsed_time(ev[-1])
    blocks_ms = ev[1].elapsed_time(ev[-1])
    append = [ev[2 + 2 * k].elapsed_time(ev[3 + 2 * k]) for k in range(nb)]
    del kv, ws
    return {"blocks": nb, "tokens": nb * B * T, "prompt": P, "prompt_prefill_ms": round(ev[0].elapsed_time(ev[1]), 2),
            "e2e_ms": round(e2e, 2), "tok_s_e2e": round(nb * B * T / (e2e / 1e3), 2),
            "tok_s_blocks": round(nb * B * T / (blocks_ms / 1e3), 2),
            "append_ms": [round(x, 2) for x in append], "steps_taken": steps}


# kernel classes summed into the groups the article's section 5 compares
AR_GROUPS = {"moe": ("router", "expert_gateup", "expert_down", "shared"), "attention": ("attn",),
             "sampling": ("lmhead", "sampler", "softemb")}


def ar_leg(dg, synth, dm, prefix, P, n, seed, stream, step_kernel_ms, step_ms):
    """Autoregressive decoding of n tokens after the prompt (dg_ar_step, one
    token per call, kernels launched directly), timed with events; then one
    profiled AR step, and the per-step ratios diffusion step / AR step."""
    import torch
    P_max = P + ((n + 3 + 31) // 32) * 32
    kv = dm.kv_cache(1, P_max)
    ws = dm.workspace(256, P_max)
    dg.dg_prefill_prefix(dm.handle, prefix[:1], 1, P, P_max, kv, ws, stream=stream)
    seeds = synth.row_seeds(seed + 100, 1)
    # decoded in place (the next token overwrites the input), so one captured
    # graph serves every position
    tok = prefix[:1, -1].contiguous()
    pos = P
    for _ in range(2):   # warm-up, and the graph capture
        dg.dg_ar_step(dm.handle, kv, 1, pos, P_max, tok, 0.8, seeds, tok, ws, stream=stream)
        pos += 1
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(n):
        dg.dg_ar_step(dm.handle, kv, 1, pos, P_max, tok, 0.8, seeds, tok, ws, stream=stream)
        pos += 1
    e1.record()
    torch.cuda.synchronize()
    ms_tok = e0.elapsed_time(e1) / n
    dg.dg_profile_enable(dm.handle, True)
    dg.dg_ar_step(dm.handle, kv, 1, pos, P_max, tok, 0.8, seeds, tok, ws, stream=stream)
    torch.cuda.synchronize()
    prof = dg.dg_profile_read(dm.handle)
    dg.dg_profile_enable(dm.handle, False)
    ar_k = {k: round(v[0], 4) for k, v in prof.items()}
    del kv, ws
    out = {"tokens": n, "prompt": P, "ms_per_token": round(ms_tok, 4), "tok_s": round(1e3 / ms_tok, 2),
           "launch": "graph replay (position read on the device)", "kernel_ms": ar_k, "kernel_sum_ms": round(sum(ar_k.values()), 4)}
    if step_kernel_ms:
        sk = {k: v["ms_per_step"] for k, v in step_kernel_ms.items()}
        ratios = {"step_over_ar_wall": round(step_ms / ms_tok, 3),
                  "step_over_ar_kernels": round(sum(sk.values()) / max(1e-9, sum(ar_k.values())), 3)}
        for g, ks in AR_GROUPS.items():
            a = sum(ar_k.get(k, 0.0) for k in ks)
            d = sum(sk.get(k, 0.0) for k in ks)
            ratios[g] = round(d / a, 3) if a > 0 else None
        out["ratios"] = ratios
    return out


def routing_leg(dg, synth, seed, stream):
    """One full-width layer (2048-token prefix, 256 canvas rows) at three
    routing spreads: iid canvas rows (every expert touched), rows sharing a
    common direction so that about 84 distinct experts are touched (the
    article's section 5 count), and a stronger common direction.  Reports the
    touched experts and the grouped expert products' time and byte rate."""
    import numpy as np
    import torch
    from discrete_diffusion_decoding_amd.configs import WORKLOADS
    from discrete_diffusion_decoding_amd.device import DeviceModel
    wl = WORKLOADS["layer_step_routed"]
    m = wl.model
    P, T, d = wl.prefix_len, wl.canvas_len, m.d_model
    dm = DeviceModel(m, seed)
    kv = dm.kv_cache(1, P)
    ws = dm.workspace(T, P + T)
    hp = torch.as_tensor(synth.hidden(seed, "prefix_hidden", (P, d))).cuda()
    dg.dg_prefill_hidden(dm.handle, hp, 1, P, P, kv, ws, stream=stream)
    out = []
    reps = 5
    for label, a in (("iid", 0.0), ("article_84", wl.hidden_common), ("concentrated", 2.5)):
        hc = torch.as_tensor(synth.hidden_common(seed, "canvas_hidden", (T, d), a)).cuda()
        h = hc.clone()
        ed = torch.zeros(1, T, m.top_k, dtype=torch.int32, device="cuda")
        dg.dg_forward_hidden(dm.handle, kv, 1, P, P, 1, T, h, ws, expert_dump=ed, stream=stream)
        torch.cuda.synchronize()
        touched = int(len(np.unique(ed.cpu().numpy())))
        dg.dg_profile_enable(dm.handle, True)
        for _ in range(reps):
            h.copy_(hc)
            dg.dg_forward_hidden(dm.handle, kv, 1, P, P, 1, T, h, ws, stream=stream)
        torch.cuda.synchronize()
        prof = dg.dg_profile_read(dm.handle)
        dg.dg_profile_enable(dm.handle, False)
        gu, dn = prof["expert_gateup"][0] / reps, prof["expert_down"][0] / reps
        w_bytes = touched * 3 * m.d_expert * d * 2
        out.append({"rows": label, "common": a, "touched_experts": touched,
                    "expert_gateup_ms": round(gu, 4), "expert_down_ms": round(dn, 4),
                    "expert_weight_bytes": int(w_bytes),
                    "expert_GB_s": round(w_bytes / ((gu + dn) * 1e-3) / 1e9, 1),
                    "layer_ms": round(sum(v[0] for v in prof.values()) / reps, 4)})
    del kv, ws
    dm.close()
    return out


def copy_bandwidth_gbs(torch):
    """Achievable HBM rate: a device-to-device copy of 2 GiB (reads and writes
    counted), best of 5 after 2 warm-up copies."""
    x = torch.empty(1 << 30, dtype=torch.int16, device="cuda")
    y = torch.empty_like(x)
    for _ in range(2):
        y.copy_(x)
    best = None
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        y.copy_(x)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del x, y
    torch.cuda.synchronize()
    return 2 * 2 * (1 << 30) / (best * 1e-3) / 1e9


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="full_step")
    ap.add_argument("--seed", type=int, default=2024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-block", action="store_true")
    ap.add_argument("--no-profile", action="store_true")
    ap.add_argument("--ar-steps", type=int, default=32,
                    help="autoregressive tokens decoded after the prompt for the per-step comparison "
                         "(0 skips it)")
    ap.add_argument("--no-routing", action="store_true",
                    help="skip the one-layer leg at three routing spreads (iid / ~84 / fewer experts)")
    ap.add_argument("--blocks", type=int, default=2,
                    help="blocks generated one after another over a growing cache, each appended to it when "
                         "finished (end-to-end leg, prompt prefill included; 0 skips it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one elementwise copy of 256 MiB fp32 first (reads and writes 256 MiB each): "
                         "the reference dispatch that scales rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from discrete_diffusion_decoding_amd import dg, synth
    from discrete_diffusion_decoding_amd.configs import WORKLOADS, SamplerParams
    from discrete_diffusion_decoding_amd.device import DeviceModel

    wl = WORKLOADS[args.workload]
    m = wl.model
    if wl.hidden_input:
        raise SystemExit("bench.py times token workloads (full_step, full_block, long_block, tiny_step)")
    B, T, P, Bp = wl.batch, wl.canvas_len, wl.prefix_len, wl.prefix_batch
    torch.cuda.set_device(0)
    dg.lib()
    if args.copy_calibration:
        xs = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        ys = torch.empty_like(xs)
        torch.mul(xs, 1.0, out=ys)
        torch.cuda.synchronize()
        del xs, ys
    t0 = time.perf_counter()
    log(f"generating and uploading the {m.param_counts()['total'] / 1e9:.2f}B-parameter model")
    dm = DeviceModel(m, args.seed)
    setup_s = time.perf_counter() - t0
    log(f"model resident after {setup_s:.1f}s")
    prefix = torch.as_tensor(synth.tokens(args.seed, "prefix", (Bp, P), m.vocab)).cuda()
    torch.cuda.synchronize()
    # a non-default stream: libdg replays each step as a captured hipGraph there
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    seeds = synth.row_seeds(args.seed, B)
    kv = dm.kv_cache(Bp, P)
    ws = dm.workspace(B * T, P + T)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    dg.dg_prefill_prefix(dm.handle, prefix, Bp, P, P, kv, ws, stream=stream)
    e1.record()
    torch.cuda.synchronize()
    prefill_ms = e0.elapsed_time(e1)
    log(f"prefill {P} tokens x {Bp}: {prefill_ms:.1f} ms")

    sp = SamplerParams()
    sampler, keep = dg.make_sampler(sp, seeds)
    st = dm.canvas_state(B, T)
    canvas = dg.make_canvas(st)
    dg.dg_init_canvas(dm.handle, canvas, B, T, seeds, stream=stream)

    # one dumped step: touched experts per layer
    ed = torch.zeros(m.n_layers, B * T, m.top_k, dtype=torch.int32, device="cuda")
    st_d = dict(st)
    st_d["expert_dump"] = ed
    dg.dg_denoise_step(dm.handle, kv, Bp, P, P, B, T, dg.make_canvas(st_d), 0, sampler, ws, stream=stream)
    torch.cuda.synchronize()
    edh = ed.cpu().numpy()
    touched = [len(np.unique(edh[l])) for l in range(m.n_layers)]
    # 64-row work items of the grouped expert products per layer (an expert
    # with c rows is cut into ceil(c / 64) chunks)
    items = [int(sum((c + 63) // 64 for c in np.bincount(edh[l].ravel(), minlength=m.n_experts)))
             for l in range(m.n_layers)]

    step_idx = 1
    for _ in range(args.warmup):
        dg.dg_denoise_step(dm.handle, kv, Bp, P, P, B, T, canvas, step_idx, sampler, ws, stream=stream)
        step_idx = step_idx % (sp.max_steps - 2) + 1
    torch.cuda.synchronize()
    st["stopped"].zero_()
    torch.cuda.synchronize()
    e0.record()
    h0 = time.perf_counter()
    for _ in range(args.steps):
        dg.dg_denoise_step(dm.handle, kv, Bp, P, P, B, T, canvas, step_idx, sampler, ws, stream=stream)
        step_idx = step_idx % (sp.max_steps - 2) + 1
    e1.record()
    torch.cuda.synchronize()
    host_s = time.perf_counter() - h0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step (host clock {host_s * 1e3 / args.steps:.3f})")

    kernel_ms = {}
    if not args.no_profile:
        dg.dg_profile_enable(dm.handle, True)
        kp = max(1, min(args.steps, 5))
        for _ in range(kp):
            dg.dg_denoise_step(dm.handle, kv, Bp, P, P, B, T, canvas, step_idx, sampler, ws, stream=stream)
            step_idx = step_idx % (sp.max_steps - 2) + 1
        torch.cuda.synchronize()
        prof = dg.dg_profile_read(dm.handle)
        dg.dg_profile_enable(dm.handle, False)
        kernel_ms = {k: {"ms_per_step": round(v[0] / kp, 4), "launches_per_step": v[1] // kp}
                     for k, v in prof.items()}

    steps_taken, block_ms = None, None
    if not args.no_block:
        dg.dg_init_canvas(dm.handle, canvas, B, T, seeds, stream=stream)
        e0.record()
        dg.dg_generate_block(dm.handle, kv, Bp, P, P, B, T, canvas, sampler, ws, poll_every=8, stream=stream)
        e1.record()
        torch.cuda.synchronize()
        block_ms = e0.elapsed_time(e1)
        steps_taken = st["steps"].cpu().numpy().tolist()
        log(f"block: steps taken {steps_taken}, {block_ms:.1f} ms")
    ar = None
    if args.ar_steps > 0 and Bp == B == 1:
        ar = ar_leg(dg, synth, dm, prefix, P, args.ar_steps, args.seed, stream, kernel_ms, ms_per_step)
        log(f"AR decode: {ar['ms_per_token']:.3f} ms/token; ratios {ar.get('ratios')}")
    multi = None
    if args.blocks > 0 and Bp == B:
        multi = multi_block(dg, synth, dm, prefix, B, T, P, args.blocks, sp, args.seed, stream)
        log(f"{args.blocks} blocks end to end: {multi['e2e_ms']:.1f} ms, {multi['tok_s_e2e']:.1f} tok/s")
    spb = max(steps_taken) if steps_taken else sp.max_steps
    tok_s = B * T / (spb * ms_per_step / 1e3)

    copy_gbs = copy_bandwidth_gbs(torch)
    log(f"device-to-device copy: {copy_gbs:.0f} GB/s")
    alg_b = algorithmic_bytes(m, B, T, P, touched, Bp)
    alg_f = algorithmic_flops(m, B, T, P)
    floor_ms = max(alg_b / (HBM_PEAK_GBS * 1e9), alg_f / (BF16_PEAK_TFLOPS * 1e12)) * 1e3
    roof = None
    if kernel_ms:
        gu = kernel_ms["expert_gateup"]
        per_launch_ms = gu["ms_per_step"] / max(1, gu["launches_per_step"])
        bytes_l = gateup_bytes(m, B * T, float(np.mean(touched)))
        ach = bytes_l / (per_launch_ms * 1e-3) / 1e9
        kh = kernel_hash()
        rec = profile_record(kh, wl.name)
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": rec.get("hbm_bytes_per_launch"),
                "kernel": "grouped expert gate/up GEMM (dg::gemm_kernel<4, true>)",
                "bytes_per_launch": int(bytes_l), "avg_launch_ms": round(per_launch_ms, 4),
                "rocprof_avg_launch_ms": rec.get("rocprof_avg_launch_ms"),
                "rocprof_avg_launch_ms_graph_replays": rec.get("rocprof_avg_launch_ms_graph_replays"),
                "kernel_source_sha256_16": kh}

    out = {
        "metric": METRIC, "value": round(tok_s, 2), "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "layers": m.n_layers, "d_model": m.d_model,
                   "heads": f"{m.n_heads}q/{m.n_kv_heads}kv x {m.head_dim}",
                   "experts": f"{m.n_experts} top-{m.top_k} x {m.d_expert} + shared {m.d_shared}",
                   "vocab": m.vocab, "batch": B, "prefix": P, "canvas": T,
                   "params_B": round(m.param_counts()["total"] / 1e9, 2)},
        "roofline": roof,
        "steps_per_block": spb, "steps_taken": steps_taken, "block_ms": block_ms,
        "tokens_per_forward": round(T / spb, 3),
        "step_roofline": {"bound": "hbm" if alg_b / (HBM_PEAK_GBS * 1e9) >= alg_f / (BF16_PEAK_TFLOPS * 1e12)
                          else "mfma", "alg_bytes": int(alg_b), "alg_flops": int(alg_f),
                          "floor_ms": round(floor_ms, 4), "frac": round(floor_ms / ms_per_step, 4),
                          # the same floor against the measured copy rate instead of the 8 TB/s peak
                          "hbm_copy_GBps": round(copy_gbs, 1),
                          "floor_ms_copy": round(max(alg_b / (copy_gbs * 1e9), alg_f / (BF16_PEAK_TFLOPS * 1e12)) * 1e3, 4),
                          "frac_copy": round(max(alg_b / (copy_gbs * 1e9), alg_f / (BF16_PEAK_TFLOPS * 1e12)) * 1e3
                                             / ms_per_step, 4)},
        "touched_experts_per_layer": float(np.mean(touched)),
        "touched_experts_by_layer": touched, "expert_items_by_layer": items,
        "kernel_ms": kernel_ms, "prefill_ms": round(prefill_ms, 2), "setup_s": round(setup_s, 1),
        "multi_block": multi, "ar_decode": ar,
    }
    dm.close()
    if not args.no_routing and m.n_experts == 128:
        out["routing"] = routing_leg(dg, synth, args.seed, stream)
        log("routing: " + ", ".join(f"{r['rows']} {r['touched_experts']} experts "
                                    f"{r['expert_gateup_ms'] + r['expert_down_ms']:.3f} ms" for r in out["routing"]))
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(m, args.seed)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
