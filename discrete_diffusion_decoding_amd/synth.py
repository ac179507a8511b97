"""Seeded synthetic inputs: random-init weights, token ids, hidden states, logits.

Both the HIP path and the CPU oracle take their inputs from here, so this
module holds none of the method's arithmetic: it only draws numbers.

Weights are bf16 ~ N(0, 0.02) (norm weights 1), stored as uint16 bit patterns.
A value is drawn by looking a uniform 16-bit integer up in a 65536-entry table
of the N(0, 0.02) quantiles at (j + 0.5) / 65536 (each rounded to bf16), i.e.
an equiprobable discretisation of the normal with tails cut at ~4.3 sigma.
The integers come from numpy's Philox4x64 bit generator keyed by
(hash(seed, tensor name), chunk index) for fixed 2**22-element chunks, so any
tensor (or any chunk of it) can be regenerated alone and in parallel, and the
values do not depend on the thread count.
"""
from __future__ import annotations

import hashlib
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
from scipy.special import ndtri

CHUNK = 1 << 22
WEIGHT_STD = 0.02
BF16_ONE = np.uint16(0x3F80)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest even), return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_table(std: float) -> np.ndarray:
    q = std * ndtri((np.arange(65536, dtype=np.float64) + 0.5) / 65536.0)
    return f32_to_bf16_bits(q.astype(np.float32))


_TABLE = _normal_table(WEIGHT_STD)


def tensor_seed(seed: int, name: str) -> int:
    h = hashlib.blake2b(f"{int(seed)}/{name}".encode(), digest_size=8).digest()
    return int.from_bytes(h, "little")


def _fill_chunk(key0: int, c: int, out: np.ndarray, table: np.ndarray) -> None:
    n = out.size
    raw = np.random.Philox(key=[key0, c]).random_raw((n + 3) // 4)
    np.take(table, raw.view(np.uint16)[:n], out=out)


def normal_bf16(seed: int, name: str, shape, out: np.ndarray | None = None,
                std: float = WEIGHT_STD) -> np.ndarray:
    """bf16 bits ~ N(0, std), reproducible per (seed, name), chunk-parallel."""
    n = int(np.prod(shape))
    if out is None:
        out = np.empty(n, dtype=np.uint16)
    flat = out.reshape(-1)
    assert flat.size == n and flat.dtype == np.uint16
    table = _TABLE if std == WEIGHT_STD else _normal_table(std)
    key0 = tensor_seed(seed, name)
    nch = (n + CHUNK - 1) // CHUNK
    if nch <= 1:
        _fill_chunk(key0, 0, flat, table)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(lambda c: _fill_chunk(key0, c, flat[c * CHUNK:(c + 1) * CHUNK], table),
                        range(nch)))
    return out.reshape(shape)


# ----------------------------------------------------------------------------
# named tensors of the model
# ----------------------------------------------------------------------------

def layer_tensor_specs(m) -> list:
    """(short name, shape, kind) of one layer, kind in {'norm', 'normal'}.

    Matrices are [out_features, in_features] (rows are output features)."""
    d, hd, E = m.d_model, m.head_dim, m.n_experts
    specs = [
        ("attn_norm", (d,), "norm"),
        ("w_qkv", (m.qkv_dim, d), "normal"),
        ("q_norm", (hd,), "norm"),
        ("k_norm", (hd,), "norm"),
        ("w_o", (d, m.n_heads * hd), "normal"),
        ("ffn_norm", (d,), "norm"),
        ("w_router", (E, d), "normal"),
        ("w_gate", (E, m.d_expert, d), "normal"),
        ("w_up", (E, m.d_expert, d), "normal"),
        ("w_down", (E, d, m.d_expert), "normal"),
    ]
    if m.d_shared:
        specs += [
            ("w_gate_sh", (m.d_shared, d), "normal"),
            ("w_up_sh", (m.d_shared, d), "normal"),
            ("w_down_sh", (d, m.d_shared), "normal"),
        ]
    return specs


def global_tensor_specs(m) -> list:
    specs = []
    if m.vocab:
        specs += [("embed", (m.vocab, m.d_model), "normal"),
                  ("final_norm", (m.d_model,), "norm")]
    if m.self_cond:
        specs += [("self_cond_w", (m.d_model, m.d_model), "normal"),
                  ("self_cond_gate", (m.d_model,), "normal")]
    return specs


def make_tensor(seed: int, full_name: str, shape, kind: str, out=None) -> np.ndarray:
    if kind == "norm":
        if out is None:
            out = np.empty(shape, dtype=np.uint16)
        out[...] = BF16_ONE
        return out
    return normal_bf16(seed, full_name, shape, out=out)


def layer_weights(m, seed: int, layer: int) -> dict:
    return {s: make_tensor(seed, f"layers.{layer}.{s}", shp, kind)
            for s, shp, kind in layer_tensor_specs(m)}


def global_weights(m, seed: int) -> dict:
    return {s: make_tensor(seed, s, shp, kind) for s, shp, kind in global_tensor_specs(m)}


class SynthWeights:
    """Lazy, regenerate-on-demand view of a random-init model's bf16 weights.

    `layer(l)` and `glob()` return dicts of uint16 arrays; nothing is cached
    beyond the last layer, so a 50 GB model never has to sit in host memory."""

    def __init__(self, m, seed: int, cache_layers: bool = False):
        self.m, self.seed = m, seed
        self._g = None
        self._cache = {} if cache_layers else None

    def glob(self) -> dict:
        if self._g is None:
            self._g = global_weights(self.m, self.seed)
        return self._g

    def layer(self, l: int) -> dict:
        if self._cache is not None:
            if l not in self._cache:
                self._cache[l] = layer_weights(self.m, self.seed, l)
            return self._cache[l]
        return layer_weights(self.m, self.seed, l)


# ----------------------------------------------------------------------------
# activations / tokens / seeds
# ----------------------------------------------------------------------------

def tokens(seed: int, name: str, shape, vocab: int) -> np.ndarray:
    g = np.random.Generator(np.random.Philox(key=[tensor_seed(seed, name), 1]))
    return g.integers(0, vocab, size=shape, dtype=np.int64).astype(np.int32)


def hidden(seed: int, name: str, shape, std: float = 1.0) -> np.ndarray:
    g = np.random.Generator(np.random.Philox(key=[tensor_seed(seed, name), 2]))
    return (std * g.standard_normal(size=shape)).astype(np.float32)


def hidden_common(seed: int, name: str, shape, common: float) -> np.ndarray:
    """Rows of N(0, 1) noise plus `common` times one fixed N(0, 1) direction
    shared by every row: the larger `common`, the more alike the rows look to
    a router, and the fewer distinct experts they pick."""
    z = hidden(seed, name, shape).astype(np.float64)
    c = hidden(seed, name + "/common", (shape[-1],)).astype(np.float64)
    return (z + common * c).astype(np.float32)


def row_seeds(seed: int, n: int) -> np.ndarray:
    g = np.random.Generator(np.random.Philox(key=[tensor_seed(seed, "row_seeds"), 3]))
    return g.integers(0, 2**63 - 1, size=n, dtype=np.int64).astype(np.uint64)


def logits(seed: int, name: str, shape, scale: float = 1.0, peaked: float = 0.0) -> np.ndarray:
    """Synthetic fp32 logits: N(0, scale) plus, if `peaked` > 0, a random winner
    per row raised by `peaked` (lets entropy span near-zero to near-ln V)."""
    g = np.random.Generator(np.random.Philox(key=[tensor_seed(seed, name), 4]))
    out = (scale * g.standard_normal(size=shape)).astype(np.float32)
    if peaked:
        rows = out.reshape(-1, shape[-1])
        win = g.integers(0, shape[-1], size=rows.shape[0])
        boost = (peaked * g.uniform(0.0, 1.0, size=rows.shape[0])).astype(np.float32)
        rows[np.arange(rows.shape[0]), win] += boost
    return out
