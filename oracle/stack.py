"""Plain float64 CPU oracle of an N-layer stack of decoder layers plus the
final RMSNorm.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
smoke check and the benchmark's CPU-baseline leg may import it, and it shares
no code with the HIP path.

The model-level use of the layer:

  x_0 = input;  x_{l+1} = layer_l(x_l) for l = 0 .. L-1;  y = RMSNorm_f(x_L)

  * layers run in order, each with its own weights and its own K/V cache, all
    caches indexed by the same token positions ("From Transformer to the LLaMA
    series", section 8, LlamaModel.forward; "Chapter 10: the modern LLaMA
    architecture", section 8, one K and one V per layer in the cache size);
  * after the last layer comes one more RMSNorm with its own gamma and the
    layer's eps (Pre-LN leaves the last block's output unnormalised: the same
    page, section 3.3 and self-test Q1; "From Transformer to LLaMA: an
    overview", 4.1, the block stack followed by a final RMSNorm).

Reading taken where the pages are silent: the hidden state handed from one
layer to the next (and to the final norm) is held in the model's storage dtype,
as in a model run in that dtype, so it is rounded to nearest-even at each
layer boundary (`round_storage`).  Everything else stays float64.
"""
from __future__ import annotations

import numpy as np

from .layer import layer_forward, rms_norm


def round_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the nearest value of the storage dtype (ties to even).

    "f32": IEEE single (numpy's correctly rounded conversion).
    "bf16": 8 significant bits and float32's exponent range: with
    x = m * 2^e, 0.5 <= |m| < 1, the result is rint(m * 2^8) * 2^(e-8), rint
    rounding halves to even.  Values here are normal numbers far from
    overflow; bf16 subnormals are not modelled.
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        m, e = np.frexp(x)
        return np.ldexp(np.rint(m * 256.0), e - 8)
    raise ValueError(dtype)


def stack_prefill(cfg: dict, layers: list, final_gamma: np.ndarray, x: np.ndarray, dtype: str):
    """Causal prefill of a batch x [B, S, d] through len(layers) layers from empty caches.

    layers[l] is the weight dict of layer l (as for layer_forward).
    Returns (y [B, S, d] after the final norm, K [L, B, S, G, D], V [L, B, S, G, D]).
    """
    ys, ks, vs = [], [], []
    for b in range(x.shape[0]):
        h = np.asarray(x[b], dtype=np.float64)
        kb, vb = [], []
        for w in layers:
            out, k, v = layer_forward(cfg, w, h, 0)
            h = round_storage(out, dtype)
            kb.append(k)
            vb.append(v)
        ys.append(rms_norm(h, final_gamma, cfg["rms_norm_eps"]))
        ks.append(np.stack(kb))
        vs.append(np.stack(vb))
    return np.stack(ys), np.stack(ks, axis=1), np.stack(vs, axis=1)


def stack_decode_step(cfg: dict, layers: list, final_gamma: np.ndarray, x: np.ndarray, caches: list,
                      dtype: str):
    """One decode step through the stack: x [B, d]; caches[l][b] = (K [len_b, G, D], V).

    Every layer's token of sequence b sits at position len_b (the same for all
    layers) and is appended to that layer's cache before its attention.
    Returns (y [B, d], updated caches).
    """
    ys = []
    new = [list(c) for c in caches]
    for b in range(x.shape[0]):
        h = np.asarray(x[b:b + 1], dtype=np.float64)
        for l, w in enumerate(layers):
            pk, pv = new[l][b]
            out, k, v = layer_forward(cfg, w, h, pk.shape[0], pk, pv)
            new[l][b] = (np.concatenate([pk, k]), np.concatenate([pv, v]))
            h = round_storage(out, dtype)
        ys.append(rms_norm(h, final_gamma, cfg["rms_norm_eps"])[0])
    return np.stack(ys), new
