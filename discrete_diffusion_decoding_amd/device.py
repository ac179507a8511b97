"""Device memory plumbing around libdg: packed weight blocks, KV cache,
workspace and canvas state as torch tensors on the GPU.  No arithmetic of the
method happens here (weights arrive as bf16 bit patterns and are copied)."""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import dg, synth


def _dev_u16(n: int, device) -> torch.Tensor:
    return torch.empty(int(n), dtype=torch.int16, device=device)


def _upload(dst: torch.Tensor, host_u16: np.ndarray):
    dst.copy_(torch.from_numpy(host_u16.reshape(-1).view(np.int16)), non_blocking=False)


class DeviceModel:
    """Random-init model resident in HBM, built from the synthetic generator."""

    def __init__(self, shape, seed: int, device="cuda", weights=None):
        self.shape, self.seed, self.device = shape, seed, device
        self.layout = dg.layer_layout(shape)
        total = self.layout["total"]
        self.layers = []
        staging = np.zeros(total, dtype=np.uint16)
        src = weights if weights is not None else synth.SynthWeights(shape, seed)
        for l in range(shape.n_layers):
            lw = src.layer(l) if weights is not None else None
            for name, shp, kind in synth.layer_tensor_specs(shape):
                off = self.layout[name]
                n = int(np.prod(shp))
                view = staging[off:off + n]
                if lw is not None:
                    view[...] = lw[name].reshape(-1)
                else:
                    synth.make_tensor(seed, f"layers.{l}.{name}", shp, kind, out=view)
            t = _dev_u16(total, device)
            _upload(t, staging)
            self.layers.append(t)
        del staging
        g = src.glob()
        self.glob = {}
        for name, arr in g.items():
            t = _dev_u16(arr.size, device)
            _upload(t, arr)
            self.glob[name] = t
        torch.cuda.synchronize()
        self._layer_ptrs = (C.c_void_p * shape.n_layers)(*[t.data_ptr() for t in self.layers])
        w = dg.Weights()
        for name in ("embed", "final_norm", "self_cond_w", "self_cond_gate"):
            setattr(w, name, self.glob[name].data_ptr() if name in self.glob else None)
        w.layers = C.cast(self._layer_ptrs, C.POINTER(C.c_void_p))
        self._w = w
        self.handle = dg.dg_model_create(shape, w)

    def close(self):
        if self.handle is not None:
            dg.dg_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- buffers ----------------------------------------------------------
    def kv_cache(self, Bp: int, P_max: int) -> torch.Tensor:
        n = dg.dg_kv_bytes(self.handle, Bp, P_max)
        return torch.zeros(max(n, 256), dtype=torch.uint8, device=self.device)

    def workspace(self, rows: int, keys: int) -> torch.Tensor:
        n = dg.dg_workspace_bytes(self.handle, rows, keys)
        return torch.empty(n, dtype=torch.uint8, device=self.device)

    def canvas_state(self, B: int, T: int, tokens=None, dumps: bool = False) -> dict:
        m, dev = self.shape, self.device
        st = {
            "tokens": torch.zeros(B, T, dtype=torch.int32, device=dev),
            "locked": torch.zeros(B, T, dtype=torch.uint8, device=dev),
            "entropy": torch.zeros(B, T, dtype=torch.float32, device=dev),
            "xhat": torch.zeros(B, T, dtype=torch.int32, device=dev),
            "argmax": torch.zeros(B, T, dtype=torch.int32, device=dev),
            "stopped": torch.zeros(B, dtype=torch.int32, device=dev),
            "steps": torch.zeros(B, dtype=torch.int32, device=dev),
        }
        if m.self_cond:
            st["self_cond"] = torch.zeros(B, T, m.d_model, dtype=torch.int16, device=dev)
        if tokens is not None:
            st["tokens"].copy_(torch.as_tensor(np.asarray(tokens, dtype=np.int32)))
        if dumps:
            R = B * T
            st["logits_dump"] = torch.zeros(B, T, m.vocab, dtype=torch.float32, device=dev)
            st["hidden_dump"] = torch.zeros(m.n_layers + 1, R, m.d_model, dtype=torch.float32, device=dev)
            st["expert_dump"] = torch.zeros(m.n_layers, R, m.top_k, dtype=torch.int32, device=dev)
            st["gate_dump"] = torch.zeros(m.n_layers, R, m.top_k, dtype=torch.float32, device=dev)
            st["router_dump"] = torch.zeros(m.n_layers, R, m.n_experts, dtype=torch.float32, device=dev)
        return st
