"""The C-ABI library without a GPU: it loads, exports every declared entry
point, validates arguments before enqueueing anything, and its host-compiled
sampler arithmetic (the same source the kernels use) is bit-identical to the
oracle's independent implementation."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from discrete_diffusion_decoding_amd import dg, synth
from discrete_diffusion_decoding_amd.configs import TINY, FULL, FULL_LAYER, ModelShape, SamplerParams
from oracle import rng
from oracle.sampler import temperature

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "dg.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 20
    L = dg.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    assert dg.status_string(0) == "ok"
    assert dg.status_string(dg.DG_ERR_WORKSPACE) == "workspace too small"


@pytest.mark.parametrize("shape", [TINY, FULL_LAYER, FULL])
def test_layer_layout_matches_tensor_specs(shape):
    lay = dg.layer_layout(shape)
    spans = []
    for name, shp, _ in synth.layer_tensor_specs(shape):
        off = lay[name]
        assert off % 128 == 0
        spans.append((off, off + int(np.prod(shp)), name))
    spans.sort()
    for (a0, a1, _), (b0, _, _) in zip(spans, spans[1:]):
        assert a1 <= b0
    assert spans[-1][1] <= lay["total"]


def _fake_weights(shape):
    ptrs = (C.c_void_p * shape.n_layers)(*([0x1000] * shape.n_layers))
    w = dg.Weights(0x1000, 0x1000, 0x1000, 0x1000, C.cast(ptrs, C.POINTER(C.c_void_p)))
    return w, ptrs


def test_model_create_validates_shapes():
    w, keep = _fake_weights(TINY)
    h = dg.dg_model_create(TINY, w)
    assert dg.dg_kv_bytes(h, 1, 64) == 2 * 2 * 2 * 64 * 64 * 2
    assert dg.dg_workspace_bytes(h, 32, 96) > 0
    dg.dg_model_destroy(h)
    bad = [ModelShape(2, 256, 4, 2, 48, 8, 2, 512, 0, 2048, 0),     # head_dim 48
           ModelShape(2, 256, 6, 1, 64, 8, 2, 512, 0, 2048, 0),     # 6 q heads per kv head
           ModelShape(2, 256, 4, 2, 64, 8, 9, 512, 0, 2048, 0),     # top_k > experts
           ModelShape(2, 200, 4, 2, 64, 8, 2, 512, 0, 2048, 0),     # d_model not multiple of 64
           ModelShape(2, 256, 4, 2, 64, 8, 2, 512, 0, 2000, 0)]     # vocab not multiple of 128
    for s in bad:
        with pytest.raises(dg.DgError) as e:
            dg.dg_model_create(s, w)
        assert e.value.status == dg.DG_ERR_SHAPE
    w0 = dg.Weights(None, None, None, None, C.cast(keep, C.POINTER(C.c_void_p)))
    with pytest.raises(dg.DgError) as e:
        dg.dg_model_create(TINY, w0)
    assert e.value.status == dg.DG_ERR_ARG


def test_step_rejects_bad_arguments_before_any_device_work():
    w, keep = _fake_weights(TINY)
    h = dg.dg_model_create(TINY, w)
    sp, seeds = dg.make_sampler(SamplerParams(), [1])
    cv = dg.Canvas(*([0x2000] * 12))
    L = dg.lib()
    ws_need = dg.dg_workspace_bytes(h, 32, 96)
    # T not a multiple of 32
    st = L.dg_denoise_step(h, C.c_void_p(0x3000), 1, 64, 64, 1, 40, C.byref(cv), 0, C.byref(sp),
                           C.c_void_p(0x4000), ws_need, None)
    assert st == dg.DG_ERR_SHAPE
    # workspace too small
    st = L.dg_denoise_step(h, C.c_void_p(0x3000), 1, 64, 64, 1, 32, C.byref(cv), 0, C.byref(sp),
                           C.c_void_p(0x4000), ws_need - 1, None)
    assert st == dg.DG_ERR_WORKSPACE
    # Bp must be 1 or B; negative step; P_max < P
    assert L.dg_denoise_step(h, C.c_void_p(0x3000), 2, 64, 64, 1, 32, C.byref(cv), 0, C.byref(sp),
                             C.c_void_p(0x4000), ws_need, None) == dg.DG_ERR_ARG
    assert L.dg_denoise_step(h, C.c_void_p(0x3000), 1, 64, 64, 1, 32, C.byref(cv), -1, C.byref(sp),
                             C.c_void_p(0x4000), ws_need, None) == dg.DG_ERR_ARG
    assert L.dg_denoise_step(h, C.c_void_p(0x3000), 1, 64, 32, 1, 32, C.byref(cv), 0, C.byref(sp),
                             C.c_void_p(0x4000), ws_need, None) == dg.DG_ERR_ARG
    # missing canvas buffer
    cv2 = dg.Canvas(*([0x2000] * 12))
    cv2.entropy = None
    assert L.dg_denoise_step(h, C.c_void_p(0x3000), 1, 64, 64, 1, 32, C.byref(cv2), 0, C.byref(sp),
                             C.c_void_p(0x4000), ws_need, None) == dg.DG_ERR_ARG
    # the sampler alone: T must be a multiple of 4, B <= 16
    assert L.dg_sample_logits(C.c_void_p(0x5000), 1, 30, 2048, C.byref(cv), 0, C.byref(sp),
                              C.c_void_p(0x4000), 1 << 20, None) == dg.DG_ERR_SHAPE
    assert L.dg_sample_logits(C.c_void_p(0x5000), 17, 32, 2048, C.byref(cv), 0, C.byref(sp),
                              C.c_void_p(0x4000), 1 << 20, None) == dg.DG_ERR_SHAPE
    dg.dg_model_destroy(h)


def test_prefill_append_rejects_bad_arguments_before_any_device_work():
    w, keep = _fake_weights(TINY)
    h = dg.dg_model_create(TINY, w)
    L = dg.lib()
    kv, ws, tok = C.c_void_p(0x3000), C.c_void_p(0x4000), C.c_void_p(0x5000)
    big = 1 << 30
    # capacity not a multiple of 32 (any start and length are accepted)
    assert L.dg_prefill_append(h, tok, 1, 48, 40, 100, kv, ws, big, None) == dg.DG_ERR_SHAPE
    # P0 + n beyond the cache capacity; no tokens; n < 1
    assert L.dg_prefill_append(h, tok, 1, 96, 64, 128, kv, ws, big, None) == dg.DG_ERR_ARG
    assert L.dg_prefill_append(h, None, 1, 64, 32, 128, kv, ws, big, None) == dg.DG_ERR_ARG
    assert L.dg_prefill_append(h, tok, 1, 64, 0, 128, kv, ws, big, None) == dg.DG_ERR_ARG
    # workspace too small
    assert L.dg_prefill_append(h, tok, 1, 64, 32, 128, kv, ws, 1024, None) == dg.DG_ERR_WORKSPACE
    dg.dg_model_destroy(h)


def test_ar_step_rejects_bad_arguments_before_any_device_work():
    w, keep = _fake_weights(TINY)
    h = dg.dg_model_create(TINY, w)
    L = dg.lib()
    kv, ws, tok, nxt = C.c_void_p(0x3000), C.c_void_p(0x4000), C.c_void_p(0x5000), C.c_void_p(0x6000)
    seeds = (C.c_uint64 * 16)(*range(16))
    sp = C.cast(seeds, C.POINTER(C.c_uint64))
    big = 1 << 30

    def call(B=1, P=70, P_max=96, tau=0.8, token=tok, seeds=sp, ws_bytes=big, next_=nxt):
        return L.dg_ar_step(h, kv, B, P, P_max, token, tau, seeds, next_, None, None, None, ws, ws_bytes, None)

    assert call(P=96) == dg.DG_ERR_ARG       # no room for position P
    assert call(B=0) == dg.DG_ERR_ARG
    assert call(B=17) == dg.DG_ERR_ARG
    assert call(tau=0.0) == dg.DG_ERR_ARG
    assert call(tau=float("nan")) == dg.DG_ERR_ARG
    assert call(token=None) == dg.DG_ERR_ARG
    assert call(next_=None) == dg.DG_ERR_ARG
    assert call(seeds=None) == dg.DG_ERR_ARG
    assert call(P_max=100) == dg.DG_ERR_SHAPE
    assert call(ws_bytes=1024) == dg.DG_ERR_WORKSPACE
    dg.dg_model_destroy(h)


def test_gemm_rejects_bad_shapes_before_any_device_work():
    L = dg.lib()
    p = C.c_void_p(0x4000)
    # K not a multiple of 64; row pitches not multiples of 8 (16-byte rows)
    assert L.dg_gemm_bf16(p, 96, p, 96, 256, 64, 96, p, 64, None) == dg.DG_ERR_SHAPE
    assert L.dg_gemm_bf16(p, 132, p, 128, 256, 64, 128, p, 64, None) == dg.DG_ERR_SHAPE
    assert L.dg_gemm_bf16(p, 128, p, 130, 8, 64, 128, p, 64, None) == dg.DG_ERR_SHAPE
    assert L.dg_gemm_bf16(p, 64, p, 128, 8, 64, 128, p, 64, None) == dg.DG_ERR_ARG   # lda < K
    # K-major weights: W [K][N]
    assert L.dg_gemm_bf16_kn(p, 96, p, 64, 256, 64, 96, p, 64, None) == dg.DG_ERR_SHAPE   # K % 64
    assert L.dg_gemm_bf16_kn(p, 128, p, 68, 256, 68, 128, p, 68, None) == dg.DG_ERR_SHAPE  # N % 8
    assert L.dg_gemm_bf16_kn(p, 132, p, 64, 256, 64, 128, p, 64, None) == dg.DG_ERR_SHAPE  # lda % 8
    assert L.dg_gemm_bf16_kn(p, 128, p, 56, 8, 64, 128, p, 64, None) == dg.DG_ERR_ARG      # ldw < N
    assert L.dg_gemm_bf16_kn(p, 128, p, 64, 8, 64, 128, p, 32, None) == dg.DG_ERR_ARG      # ldc < N


def test_sample_noalloc_rejects_bad_arguments_before_any_device_work():
    """The no-allocation sampler checks its arguments before it looks up its
    scratch area (no GPU here: any device call would fail with DG_ERR_HIP)."""
    L = dg.lib()
    assert L.dg_sample_noalloc_max_bytes() == 1 << 20
    # the largest accepted request fits the scratch area
    assert L.dg_sample_workspace_bytes(16, 1024, 262144) <= L.dg_sample_noalloc_max_bytes()
    p = C.c_void_p(0x4000)
    sp, keep = dg.make_sampler(SamplerParams(), [1])
    cv = dg.Canvas(*([0x8000] * 5 + [None] + [0x8000] * 2 + [None] * 4))   # no self_cond, no dumps
    f = L.dg_sample_logits_noalloc
    assert f(None, 1, 32, 2048, C.byref(cv), 0, C.byref(sp), None) == dg.DG_ERR_ARG
    assert f(p, 0, 32, 2048, C.byref(cv), 0, C.byref(sp), None) == dg.DG_ERR_ARG
    assert f(p, 1, 30, 2048, C.byref(cv), 0, C.byref(sp), None) == dg.DG_ERR_SHAPE
    assert f(p, 17, 32, 2048, C.byref(cv), 0, C.byref(sp), None) == dg.DG_ERR_SHAPE
    assert f(p, 1, 32, 2048, C.byref(cv), -1, C.byref(sp), None) == dg.DG_ERR_ARG
    assert f(p, 1, 32, 2048, None, 0, C.byref(sp), None) == dg.DG_ERR_ARG


def test_host_philox_equals_oracle_definition():
    g = np.random.default_rng(0)
    for _ in range(200):
        c = [int(x) for x in g.integers(0, 2**32, 4, dtype=np.uint64)]
        k = [int(x) for x in g.integers(0, 2**32, 2, dtype=np.uint64)]
        assert dg.host_philox(c, k) == rng.philox_generic(c, k)


def test_host_ln_bit_equal_on_every_sampler_input():
    u = ((np.arange(1 << 23, dtype=np.uint32) * np.uint32(2) + np.uint32(1)).astype(np.float32)
         * np.float32(2.0 ** -24))
    a_lib = dg.host_ln_batch(u)
    a_orc = rng.ln_f32(u)
    assert np.array_equal(a_lib.view(np.uint32), a_orc.view(np.uint32))
    b = -a_orc
    assert np.array_equal(dg.host_ln_batch(b).view(np.uint32), rng.ln_f32(b).view(np.uint32))


def test_host_gumbel_bit_equal():
    w = np.random.default_rng(1).integers(0, 2**32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    w[:4] = [0, 0xFFFFFFFF, 0x1FF, 0x80000000]
    assert np.array_equal(dg.host_gumbel_batch(w).view(np.uint32),
                          rng.gumbel_f32(rng.uniform_open01(w)).view(np.uint32))


def test_host_inv_tau_equals_oracle_schedule():
    for S in (1, 2, 48):
        for s in range(S):
            assert dg.host_inv_tau(0.8, 0.4, S, s) == temperature(s, 0.8, 0.4, S)[1]
