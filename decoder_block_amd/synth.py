"""Seeded synthetic workloads for the decoder layer.

This module holds no arithmetic of the layer itself: only the random draws
that make up weights, activations, context lengths and cache contents, and the
fp32 -> bf16 storage rounding (round-to-nearest-even, done by torch's
conversion routine) applied to those draws.  The oracle-based tests and the GPU
harness both take their inputs from here, so both sides see bit-identical
values.

Recipe (each array has its own seed, ``1000 * workload_id + k``):

  k = 0   x                     ~ N(0, 1)
  k = 1-7 q,k,v,o,gate,up,down  ~ N(0, w_std^2), nn.Linear layout [out, in], no biases
  k = 8-9 input/post-attention RMSNorm gamma: 1 (or 1 + N(0, gamma_std^2))
  k = 10  per-sequence context lengths, integers uniform in [ctx_lo, ctx_hi]
  k = 11  physical-block permutation of the paged cache
  k = 12  decode-step activations x_t ~ N(0, 1), one fresh draw per step
  k = 13  pre-filled cache contents K, V ~ N(0, 1)
  k = 14  sample of rows checked at full size

Large arrays are drawn in fixed 4 Mi-element chunks, each from its own child
of ``numpy.random.SeedSequence(seed)``, so the values do not depend on how
many threads fill them.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np
import torch

_CHUNK = 1 << 22


@dataclass(frozen=True)
class Workload:
    """One workload: the layer's config fields plus the shape of the job."""
    wid: int
    name: str
    dtype: str                 # "f32" or "bf16": storage of weights/activations/cache
    hidden_size: int
    intermediate_size: int
    num_attention_heads: int
    num_key_value_heads: int
    rms_norm_eps: float
    rope_theta: float
    batch: int
    seq_len: int               # prefill tokens per sequence (0 for a decode-only job)
    w_std: float = 0.02
    gamma_std: float = 0.0     # 0: gamma = 1
    decode_steps: int = 0
    ctx_lo: int = 0            # decode-only jobs: pre-filled context lengths
    ctx_hi: int = 0
    block_size: int = 16
    max_position: int = 0      # RoPE table length; 0: derived from the job
    rope_style: str = "interleaved"  # or "half_split": which head elements RoPE pairs

    @property
    def head_dim(self) -> int:
        return self.hidden_size // self.num_attention_heads

    def positions_needed(self) -> int:
        if self.max_position:
            return self.max_position
        longest = max(self.seq_len, self.ctx_hi)
        return longest + self.decode_steps + 1

    def seed(self, k: int) -> int:
        return 1000 * self.wid + k

    def config_dict(self) -> dict:
        return dict(hidden_size=self.hidden_size,
                    intermediate_size=self.intermediate_size,
                    num_attention_heads=self.num_attention_heads,
                    num_key_value_heads=self.num_key_value_heads,
                    rms_norm_eps=self.rms_norm_eps,
                    rope_theta=self.rope_theta,
                    rope_style=self.rope_style)


WORKLOADS = {
    1: Workload(1, "tiny-gqa-fp32", "f32", 256, 688, 4, 2, 1e-5, 10000.0,
                batch=1, seq_len=64, gamma_std=0.1, decode_steps=8),
    2: Workload(2, "llama-7b-layer-prefill", "bf16", 4096, 11008, 32, 32, 1e-6, 10000.0,
                batch=1, seq_len=2048),
    3: Workload(3, "llama3-8b-layer-prefill", "bf16", 4096, 14336, 32, 8, 1e-5, 500000.0,
                batch=1, seq_len=8192),
    4: Workload(4, "llama3-8b-layer-decode", "bf16", 4096, 14336, 32, 8, 1e-5, 500000.0,
                batch=64, seq_len=0, decode_steps=128, ctx_lo=512, ctx_hi=8192),
    5: Workload(5, "llama3-70b-layer-prefill", "bf16", 8192, 28672, 64, 8, 1e-5, 500000.0,
                batch=4, seq_len=4096, w_std=0.01),
}


def scaled(w: Workload, **kw) -> Workload:
    """A copy of ``w`` with some fields replaced (smaller parity cases)."""
    return replace(w, **kw)


# The GQA ratio sweep: the LLaMA-3-8B jobs with one K/V head for all 32 query
# heads (MQA), and the LLaMA-3-405B layer shape (d 16384, 128 query heads over
# 8 K/V heads, I 53248).  Same recipes and seeds as the jobs they derive from.
_L405 = dict(hidden_size=16384, intermediate_size=53248, num_attention_heads=128, num_key_value_heads=8,
             w_std=0.01)
VARIANTS = {
    "llama3-8b-mqa-layer-prefill": replace(WORKLOADS[3], name="llama3-8b-mqa-layer-prefill",
                                           num_key_value_heads=1),
    "llama3-8b-mqa-layer-decode": replace(WORKLOADS[4], name="llama3-8b-mqa-layer-decode",
                                          num_key_value_heads=1),
    "llama3-405b-layer-prefill": replace(WORKLOADS[5], name="llama3-405b-layer-prefill", batch=1,
                                         seq_len=8192, **_L405),
    "llama3-405b-layer-decode": replace(WORKLOADS[4], name="llama3-405b-layer-decode", **_L405),
}
PREFILL_JOBS = {w.name: w for w in (WORKLOADS[2], WORKLOADS[3], WORKLOADS[5],
                                    VARIANTS["llama3-8b-mqa-layer-prefill"],
                                    VARIANTS["llama3-405b-layer-prefill"])}
DECODE_JOBS = {w.name: w for w in (WORKLOADS[4], VARIANTS["llama3-8b-mqa-layer-decode"],
                                   VARIANTS["llama3-405b-layer-decode"])}


# ----------------------------------------------------------------------------
# raw draws
# ----------------------------------------------------------------------------

def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_f32(seed, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """float32 array of N(mean, std^2) draws, chunk-seeded (thread-count independent)."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.float32)
    nch = max(1, (n + _CHUNK - 1) // _CHUNK)
    kids = np.random.SeedSequence(seed).spawn(nch)

    def fill(i):
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(kids[i]))
        g.standard_normal(out=out[lo:hi], dtype=np.float32)
        if std != 1.0:
            out[lo:hi] *= np.float32(std)
        if mean != 0.0:
            out[lo:hi] += np.float32(mean)

    if nch == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nch)))
    return out.reshape(shape)


def storage(a: np.ndarray, dtype: str) -> torch.Tensor:
    """CPU tensor in the workload's storage dtype (bf16: round-to-nearest-even)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t.clone()
    raise ValueError(dtype)


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a stored tensor (what the oracle consumes)."""
    return t.to(torch.float64).numpy()


# ----------------------------------------------------------------------------
# workload pieces
# ----------------------------------------------------------------------------

WEIGHT_NAMES = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")
NORM_NAMES = ("input_layernorm", "post_attention_layernorm")


def weight_shapes(w: Workload) -> dict:
    d, I = w.hidden_size, w.intermediate_size
    hq, hk = w.num_attention_heads * w.head_dim, w.num_key_value_heads * w.head_dim
    return {"q_proj": (hq, d), "k_proj": (hk, d), "v_proj": (hk, d), "o_proj": (d, hq),
            "gate_proj": (I, d), "up_proj": (I, d), "down_proj": (d, I),
            "input_layernorm": (d,), "post_attention_layernorm": (d,)}


def layer_weights(w: Workload, gamma_std: float | None = None, layer: int = 0) -> dict:
    """All nine parameter tensors in storage dtype (CPU).  Layer l > 0 of a
    stack draws from seeds of its own (layer 0 is the single-layer draw)."""
    shapes = weight_shapes(w)
    gs = w.gamma_std if gamma_std is None else gamma_std

    def sd(k):
        return w.seed(k) if layer == 0 else [w.seed(k), layer]

    out = {}
    for k, name in enumerate(WEIGHT_NAMES, start=1):
        out[name] = storage(normal_f32(sd(k), shapes[name], w.w_std), w.dtype)
    for k, name in enumerate(NORM_NAMES, start=8):
        if gs > 0:
            g = normal_f32(sd(k), shapes[name], gs, mean=1.0)
        else:
            g = np.ones(shapes[name], np.float32)
        out[name] = storage(g, w.dtype)
    return out


def final_norm_weight(w: Workload, gamma_std: float = 0.1) -> torch.Tensor:
    """Gamma [d] of a stack's final RMSNorm: N(1, gamma_std^2) in storage dtype."""
    return storage(normal_f32(w.seed(15), (w.hidden_size,), gamma_std, mean=1.0), w.dtype)


def layer_input(w: Workload) -> torch.Tensor:
    """Prefill activations x [B, S, d] in storage dtype."""
    return storage(normal_f32(w.seed(0), (w.batch, w.seq_len, w.hidden_size)), w.dtype)


def decode_input(w: Workload, step: int) -> torch.Tensor:
    """Decode-step activations x_t [B, d] (a fresh draw per step)."""
    seed = [w.seed(12), step]
    return storage(normal_f32(seed, (w.batch, w.hidden_size)), w.dtype)


def context_lengths(w: Workload) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(w.seed(10)))
    return g.integers(w.ctx_lo, w.ctx_hi, size=w.batch, endpoint=True).astype(np.int32)


def block_permutation(w: Workload, num_blocks: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(w.seed(11)))
    return g.permutation(num_blocks).astype(np.int32)


def cache_contents(w: Workload, seq: int, length: int):
    """Pre-filled (already rotated) K and V for one sequence: [length, G, D] each."""
    G, D = w.num_key_value_heads, w.head_dim
    k = storage(normal_f32([w.seed(13), seq, 0], (length, G, D)), w.dtype)
    v = storage(normal_f32([w.seed(13), seq, 1], (length, G, D)), w.dtype)
    return k, v


def sample_rows(w: Workload, seq_len: int, n_random: int = 448, edge: int = 64) -> np.ndarray:
    """Rows checked at full size: the first and last ``edge`` plus ``n_random`` seeded ones."""
    g = np.random.Generator(np.random.PCG64(w.seed(14)))
    edges = set(range(min(edge, seq_len))) | set(range(max(0, seq_len - edge), seq_len))
    rest = np.array(sorted(set(range(seq_len)) - edges), dtype=np.int64)
    pick = g.choice(rest, size=min(n_random, rest.size), replace=False) if rest.size else rest
    return np.array(sorted(edges | set(int(v) for v in pick)), dtype=np.int64)
