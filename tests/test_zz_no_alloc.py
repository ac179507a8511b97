"""dg_sample_logits_noalloc (the sampler over the library's own static scratch
area, for callers that cannot allocate) against dg_sample_logits over a
caller-given workspace: the same kernels, so the same results bit for bit.
Two calls in a row share the scratch area, the second on a smaller request
(fewer rows and vocabulary slices than the first left behind), with one
canvas stopped on entry."""
import numpy as np
import pytest
import torch

from discrete_diffusion_decoding_amd import dg, synth
from discrete_diffusion_decoding_amd.configs import SamplerParams
from tests.gpu_util import announce, dev, host

pytestmark = pytest.mark.gpu

FIELDS = ("tokens", "locked", "entropy", "xhat", "argmax", "stopped", "steps")


def _state(B, T, V, seed):
    g = np.random.default_rng(seed)
    st = {
        "tokens": dev(g.integers(0, V, (B, T)).astype(np.int32)),
        "locked": torch.zeros(B, T, dtype=torch.uint8, device="cuda"),
        "entropy": torch.zeros(B, T, dtype=torch.float32, device="cuda"),
        "xhat": torch.zeros(B, T, dtype=torch.int32, device="cuda"),
        "argmax": dev(g.integers(0, V, (B, T)).astype(np.int32)),
        "stopped": torch.zeros(B, dtype=torch.int32, device="cuda"),
        "steps": torch.zeros(B, dtype=torch.int32, device="cuda"),
    }
    return st


def test_noalloc_sampler_equals_workspace_sampler():
    sp = SamplerParams()
    # (B, T, V, step, logit scale, peak, canvases stopped on entry)
    calls = [(4, 256, 262144, 3, 1.0, 0.0, ()), (2, 64, 2048, 9, 2.0, 12.0, (1,))]
    for i, (B, T, V, step, scale, peak, stopped) in enumerate(calls):
        announce(f"noalloc sampler call {i}: B={B} T={T} V={V} step={step}")
        logits = dev(synth.logits(11 + i, f"noalloc{i}", (B, T, V), scale=scale, peaked=peak))
        seeds = synth.row_seeds(40 + i, B)
        sampler, keep = dg.make_sampler(sp, seeds)
        a, b = _state(B, T, V, i), _state(B, T, V, i)
        for s in (a, b):
            for r in stopped:
                s["stopped"][r] = 1
                s["steps"][r] = 7
        ws = torch.empty(dg.dg_sample_workspace_bytes(B, T, V), dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        dg.dg_sample_logits(logits, B, T, V, dg.make_canvas(a), step, sampler, ws)
        dg.dg_sample_logits_noalloc(logits, B, T, V, dg.make_canvas(b), step, sampler)
        torch.cuda.synchronize()
        for k in FIELDS:
            assert np.array_equal(host(a[k]), host(b[k])), (i, k)
        for r in stopped:
            assert host(b["steps"])[r] == 7 and host(b["stopped"])[r] == 1
        live = [r for r in range(B) if r not in stopped]
        assert (host(b["steps"])[live] == step + 1).all()
