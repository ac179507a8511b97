"""ctypes binding of libdg (include/dg.h): the same entry points, argument
marshalling only.  Every step of the denoising path runs in libdg's HIP
kernels; torch is used for device memory and streams.

Loading fails loudly if libdg.so has not been built (python -m
discrete_diffusion_decoding_amd.build)."""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

# DG_LIBRARY may name another build of the same sources (the host-sanitizer
# build that the CPU tests load); by default the in-tree libdg.so
_LIB_PATH = os.environ.get("DG_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdg.so")

DG_OK, DG_ERR_ARG, DG_ERR_SHAPE, DG_ERR_WORKSPACE, DG_ERR_HIP, DG_ERR_UNSUPPORTED = 0, -1, -2, -3, -4, -5


class DgError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status} ({status_string(status)})")
        self.status = status


class ModelDesc(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_layers", "d_model", "n_heads", "n_kv_heads", "head_dim",
                                         "n_experts", "top_k", "d_expert", "d_shared", "vocab",
                                         "self_cond")] + [("rope_theta", C.c_float), ("rms_eps", C.c_float)]


LAYOUT_FIELDS = ("attn_norm", "w_qkv", "q_norm", "k_norm", "w_o", "ffn_norm", "w_router",
                 "w_gate", "w_up", "w_down", "w_gate_sh", "w_up_sh", "w_down_sh", "total")


class LayerLayout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in LAYOUT_FIELDS]


class Weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("final_norm", C.c_void_p),
                ("self_cond_w", C.c_void_p), ("self_cond_gate", C.c_void_p),
                ("layers", C.POINTER(C.c_void_p))]


class Sampler(C.Structure):
    _fields_ = [("tau_start", C.c_float), ("tau_end", C.c_float), ("max_steps", C.c_int32),
                ("lock_rule", C.c_int32), ("lock_thresh", C.c_float), ("stop_rule", C.c_int32),
                ("stop_thresh", C.c_float), ("row_seeds", C.POINTER(C.c_uint64))]


class Canvas(C.Structure):
    _fields_ = [("tokens", C.c_void_p), ("locked", C.c_void_p), ("entropy", C.c_void_p),
                ("xhat", C.c_void_p), ("argmax", C.c_void_p), ("self_cond", C.c_void_p),
                ("stopped", C.c_void_p), ("steps", C.c_void_p), ("logits_dump", C.c_void_p),
                ("hidden_dump", C.c_void_p), ("expert_dump", C.c_void_p), ("gate_dump", C.c_void_p),
                ("router_dump", C.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"libdg.so is not built ({_LIB_PATH}); run "
                               "python -m discrete_diffusion_decoding_amd.build")
        L = C.CDLL(_LIB_PATH)
        vp, i32, sz, st = C.c_void_p, C.c_int32, C.c_size_t, C.c_int
        sig = {
            "dg_status_string": (C.c_char_p, [st]),
            "dg_layer_layout_get": (st, [C.POINTER(ModelDesc), C.POINTER(LayerLayout)]),
            "dg_model_create": (st, [C.POINTER(ModelDesc), C.POINTER(Weights), C.POINTER(vp)]),
            "dg_model_destroy": (None, [vp]),
            "dg_kv_bytes": (sz, [vp, i32, i32]),
            "dg_workspace_bytes": (sz, [vp, i32, i32]),
            "dg_prefill_prefix": (st, [vp, vp, i32, i32, i32, vp, vp, sz, vp]),
            "dg_prefill_append": (st, [vp, vp, i32, i32, i32, i32, vp, vp, sz, vp]),
            "dg_prefill_hidden": (st, [vp, vp, i32, i32, i32, vp, vp, sz, vp]),
            "dg_prefill_dump": (st, [vp, vp, i32, i32, i32, i32, vp, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
            "dg_ar_step": (st, [vp, vp, i32, i32, i32, vp, C.c_float, C.POINTER(C.c_uint64), vp, vp, vp, vp,
                                vp, sz, vp]),
            "dg_forward_hidden": (st, [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
            "dg_denoise_step": (st, [vp, vp, i32, i32, i32, i32, i32, C.POINTER(Canvas), i32,
                                     C.POINTER(Sampler), vp, sz, vp]),
            "dg_generate_block": (st, [vp, vp, i32, i32, i32, i32, i32, C.POINTER(Canvas),
                                       C.POINTER(Sampler), i32, vp, sz, vp]),
            "dg_sample_workspace_bytes": (sz, [i32, i32, i32]),
            "dg_sample_logits": (st, [vp, i32, i32, i32, C.POINTER(Canvas), i32, C.POINTER(Sampler),
                                      vp, sz, vp]),
            "dg_sample_noalloc_max_bytes": (sz, []),
            "dg_sample_logits_noalloc": (st, [vp, i32, i32, i32, C.POINTER(Canvas), i32, C.POINTER(Sampler), vp]),
            "dg_init_canvas": (st, [vp, C.POINTER(Canvas), i32, i32, C.POINTER(C.c_uint64), vp]),
            "dg_gemm_bf16": (st, [vp, C.c_int64, vp, C.c_int64, i32, i32, i32, vp, C.c_int64, vp]),
            "dg_gemm_bf16_kn": (st, [vp, C.c_int64, vp, C.c_int64, i32, i32, i32, vp, C.c_int64, vp]),
            "dg_profile_enable": (st, [vp, i32]),
            "dg_set_graphs": (st, [vp, i32]),
            "dg_profile_read": (st, [vp, i32, C.POINTER(C.c_double), C.POINTER(C.c_int32)]),
            "dg_host_philox": (None, [C.POINTER(C.c_uint32), C.POINTER(C.c_uint32), C.POINTER(C.c_uint32)]),
            "dg_host_ln": (C.c_float, [C.c_float]),
            "dg_host_gumbel_of_word": (C.c_float, [C.c_uint32]),
            "dg_host_inv_tau": (C.c_float, [C.c_float, C.c_float, i32, i32]),
            "dg_host_ln_batch": (None, [vp, vp, C.c_int64]),
            "dg_host_gumbel_batch": (None, [vp, vp, C.c_int64]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().dg_status_string(s).decode()


def _ck(status: int, what: str):
    if status != DG_OK:
        raise DgError(status, what)


def model_desc(shape) -> ModelDesc:
    return ModelDesc(shape.n_layers, shape.d_model, shape.n_heads, shape.n_kv_heads, shape.head_dim,
                     shape.n_experts, shape.top_k, shape.d_expert, shape.d_shared, shape.vocab,
                     shape.self_cond, shape.rope_theta, shape.rms_eps)


def layer_layout(shape) -> dict:
    out = LayerLayout()
    _ck(lib().dg_layer_layout_get(C.byref(model_desc(shape)), C.byref(out)), "dg_layer_layout_get")
    return {n: int(getattr(out, n)) for n in LAYOUT_FIELDS}


# ---- thin wrappers (same names as the C ABI) --------------------------------

def _ptr(t):
    """Device address of a torch tensor (or None)."""
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    return C.c_void_p(stream.cuda_stream if stream is not None else 0)


def dg_model_create(shape, weights: Weights):
    h = C.c_void_p()
    _ck(lib().dg_model_create(C.byref(model_desc(shape)), C.byref(weights), C.byref(h)), "dg_model_create")
    return h


def dg_model_destroy(h):
    lib().dg_model_destroy(h)


def dg_kv_bytes(h, Bp, P_max):
    return int(lib().dg_kv_bytes(h, Bp, P_max))


def dg_workspace_bytes(h, rows, keys):
    return int(lib().dg_workspace_bytes(h, rows, keys))


def dg_prefill_prefix(h, prefix, Bp, P, P_max, kv, ws, stream=None):
    _ck(lib().dg_prefill_prefix(h, _ptr(prefix), Bp, P, P_max, _ptr(kv), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream)), "dg_prefill_prefix")


def dg_prefill_append(h, tokens, Bp, P0, n, P_max, kv, ws, stream=None):
    _ck(lib().dg_prefill_append(h, _ptr(tokens), Bp, P0, n, P_max, _ptr(kv), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream)), "dg_prefill_append")


def dg_prefill_dump(h, tokens, Bp, P0, n, P_max, kv, dump_pos, dump_n, ws, hidden_dump=None, expert_dump=None,
                    gate_dump=None, router_dump=None, stream=None):
    _ck(lib().dg_prefill_dump(h, _ptr(tokens), Bp, P0, n, P_max, _ptr(kv), dump_pos, dump_n, _ptr(hidden_dump),
                              _ptr(expert_dump), _ptr(gate_dump), _ptr(router_dump), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream)), "dg_prefill_dump")


def dg_ar_step(h, kv, B, P, P_max, token, tau, seeds, nxt, ws, argmax=None, entropy=None, logits_dump=None,
               stream=None):
    arr = (C.c_uint64 * len(seeds))(*[int(s) for s in seeds])
    _ck(lib().dg_ar_step(h, _ptr(kv), B, P, P_max, _ptr(token), tau, C.cast(arr, C.POINTER(C.c_uint64)), _ptr(nxt),
                         _ptr(argmax), _ptr(entropy), _ptr(logits_dump), _ptr(ws), ws.numel() * ws.element_size(),
                         _stream(stream)), "dg_ar_step")


def dg_prefill_hidden(h, prefix_hidden, Bp, P, P_max, kv, ws, stream=None):
    _ck(lib().dg_prefill_hidden(h, _ptr(prefix_hidden), Bp, P, P_max, _ptr(kv), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream)), "dg_prefill_hidden")


def dg_forward_hidden(h, kv, Bp, P, P_max, B, T, hidden, ws, hidden_dump=None, expert_dump=None,
                      gate_dump=None, stream=None):
    _ck(lib().dg_forward_hidden(h, _ptr(kv), Bp, P, P_max, B, T, _ptr(hidden), _ptr(hidden_dump),
                                _ptr(expert_dump), _ptr(gate_dump), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream)), "dg_forward_hidden")


def make_sampler(sp, seeds) -> tuple:
    arr = (C.c_uint64 * len(seeds))(*[int(s) for s in seeds])
    s = Sampler(sp.tau_start, sp.tau_end, sp.max_steps, sp.lock_rule, sp.lock_thresh, sp.stop_rule,
                sp.stop_thresh, C.cast(arr, C.POINTER(C.c_uint64)))
    return s, arr


def make_canvas(st: dict) -> Canvas:
    """Canvas struct from a dict of torch tensors (missing keys -> NULL)."""
    names = [f[0] for f in Canvas._fields_]
    return Canvas(*[_ptr(st.get(n)) for n in names])


def dg_denoise_step(h, kv, Bp, P, P_max, B, T, canvas: Canvas, step, sampler: Sampler, ws, stream=None):
    _ck(lib().dg_denoise_step(h, _ptr(kv), Bp, P, P_max, B, T, C.byref(canvas), step, C.byref(sampler), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream)), "dg_denoise_step")


def dg_generate_block(h, kv, Bp, P, P_max, B, T, canvas: Canvas, sampler: Sampler, ws, poll_every=8, stream=None):
    _ck(lib().dg_generate_block(h, _ptr(kv), Bp, P, P_max, B, T, C.byref(canvas), C.byref(sampler), poll_every,
                                _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "dg_generate_block")


def dg_sample_workspace_bytes(B, T, V):
    return int(lib().dg_sample_workspace_bytes(B, T, V))


def dg_sample_logits(logits, B, T, V, canvas: Canvas, step, sampler: Sampler, ws, stream=None):
    _ck(lib().dg_sample_logits(_ptr(logits), B, T, V, C.byref(canvas), step, C.byref(sampler), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(stream)), "dg_sample_logits")


def dg_sample_noalloc_max_bytes():
    return int(lib().dg_sample_noalloc_max_bytes())


def dg_sample_logits_noalloc(logits, B, T, V, canvas: Canvas, step, sampler: Sampler, stream=None):
    _ck(lib().dg_sample_logits_noalloc(_ptr(logits), B, T, V, C.byref(canvas), step, C.byref(sampler),
                                       _stream(stream)), "dg_sample_logits_noalloc")


def dg_init_canvas(h, canvas: Canvas, B, T, seeds, stream=None):
    arr = (C.c_uint64 * len(seeds))(*[int(s) for s in seeds])
    _ck(lib().dg_init_canvas(h, C.byref(canvas), B, T, arr, _stream(stream)), "dg_init_canvas")


def dg_gemm_bf16_kn(A, W, Cout, M, N, K, lda=None, ldw=None, ldc=None, stream=None):
    _ck(lib().dg_gemm_bf16_kn(_ptr(A), lda or K, _ptr(W), ldw or N, M, N, K, _ptr(Cout), ldc or N,
                              _stream(stream)), "dg_gemm_bf16_kn")


def dg_gemm_bf16(A, W, Cout, M, N, K, lda=None, ldw=None, ldc=None, stream=None):
    _ck(lib().dg_gemm_bf16(_ptr(A), lda or K, _ptr(W), ldw or K, M, N, K, _ptr(Cout), ldc or N, _stream(stream)),
        "dg_gemm_bf16")


PROF_CLASSES = ("dense", "attn", "router", "expert_gateup", "expert_down", "shared", "lmhead", "sampler",
                "softemb", "other")


def dg_set_graphs(h, on: bool):
    _ck(lib().dg_set_graphs(h, 1 if on else 0), "dg_set_graphs")


def dg_profile_enable(h, on: bool):
    _ck(lib().dg_profile_enable(h, 1 if on else 0), "dg_profile_enable")


def dg_profile_read(h) -> dict:
    out = {}
    for i, name in enumerate(PROF_CLASSES):
        t, n = C.c_double(), C.c_int32()
        _ck(lib().dg_profile_read(h, i, C.byref(t), C.byref(n)), "dg_profile_read")
        out[name] = (float(t.value), int(n.value))
    return out


# host reference of the sampler arithmetic (no GPU)
def host_philox(ctr, key):
    c = (C.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in ctr])
    k = (C.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    o = (C.c_uint32 * 4)()
    lib().dg_host_philox(c, k, o)
    return list(o)


def host_ln_batch(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(x)
    lib().dg_host_ln_batch(x.ctypes.data_as(C.c_void_p), out.ctypes.data_as(C.c_void_p), x.size)
    return out


def host_gumbel_batch(words: np.ndarray) -> np.ndarray:
    w = np.ascontiguousarray(words, dtype=np.uint32)
    out = np.empty(w.shape, dtype=np.float32)
    lib().dg_host_gumbel_batch(w.ctypes.data_as(C.c_void_p), out.ctypes.data_as(C.c_void_p), w.size)
    return out


def host_inv_tau(t0, t1, S, s):
    return np.float32(lib().dg_host_inv_tau(t0, t1, S, s))
