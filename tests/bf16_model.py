"""A float64 model of where the bf16 layer rounds, used to derive the parity
tolerances of cases the workload definitions give no tolerance for (stacks of
layers, gamma != 1).

TEST INFRASTRUCTURE.  This is not the oracle and not the HIP path: it is the
plain layer definition (the oracle's primitives) with a round-to-nearest-even
bf16 rounding inserted at every point where the bf16 kernels store a value in
bf16 and nowhere else.  Everything between those points stays float64, so the
model isolates the error the storage roundings cause.  The rounding points of
the bf16 kernels, in layer order:

  * W'_qkv = bf16(W_qkv * gamma_1): gamma_1 folded into the q/k/v weights
    (exact when gamma_1 = 1);
  * q, k, v after the row scale and RoPE: q stored as bf16(q * log2(e)/sqrt(D))
    (scores then come out in exp2 units), k and v stored in the cache;
  * P = exp2(s - m), rounded to bf16 as the second product's operand; the
    row sum l adds the same rounded values.  The kernels take m as a
    running maximum of the keys seen so far (online softmax; the prefill
    kernel keeps it at 0, or stale, until a score exceeds it by 32 in exp2
    units), so P is rounded at a scale 2^(m_final - m) that is not a power
    of two: a
    realisation (below) rounds each row's P in 64-key tiles at a random
    scale 2^u, u ~ U(0, 1), and divides it out again;
  * the attention output o / l;
  * h * gamma_2 as the gate/up operand (h itself stays fp32);
  * s = SiLU(r2 g) * (r2 u);
  * the output, only when the caller asks for bf16 (out_bf16), and the hidden
    state between the layers of a stack.

With round=False every rounding is skipped and the model is the oracle's
layer (tests/test_oracle_pins.py checks that), which pins it to the oracle.
"""
from __future__ import annotations

import math

import numpy as np

import oracle

LOG2E = 1.4426950408889634

# Realisations.  The kernels compute between their bf16 roundings in fp32,
# whose accumulation order shifts each value by a relative 1e-7 .. 1e-6; that
# decides which values near a rounding boundary round up or down, so the
# kernels' error is one draw from a distribution the model can sample: with a
# generator set, every value is scaled by (1 + u * PERTURB_EPS), u ~ U(-1, 1),
# before each bf16 rounding (2^-18 is the size of fp32 rounding accumulated
# over the 4096-term dot products).  None: the plain model.
PERTURB_EPS = 2.0 ** -18
_perturb_rng = None


def set_realisation(seed):
    """Perturb the values before each rounding with a generator of this seed (None: off)."""
    global _perturb_rng
    _perturb_rng = None if seed is None else np.random.Generator(np.random.PCG64(seed))


def rb(a: np.ndarray, on: bool = True, accumulated: bool = True) -> np.ndarray:
    """Round to bf16, nearest-even (identity when on is False).  `accumulated`:
    the value comes out of fp32 accumulation on the GPU, so a realisation
    perturbs it first (the weight fold W * gamma is one fp32 product: not)."""
    if not on:
        return np.asarray(a, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    if _perturb_rng is not None and accumulated:
        a = a * (1.0 + PERTURB_EPS * _perturb_rng.uniform(-1.0, 1.0, size=a.shape))
    return oracle.round_storage(a, "bf16")


P_TILE = 64  # keys that share one rounding scale of P in a realisation


def _round_p(p: np.ndarray, on: bool) -> np.ndarray:
    """P rounded to bf16: at the final row maximum (plain model), or in a
    realisation at a random scale 2^u per row and 64-key tile."""
    if not on or _perturb_rng is None:
        return rb(p, on, accumulated=False)
    nt = -(-p.shape[1] // P_TILE)
    c = np.repeat(np.exp2(_perturb_rng.uniform(0.0, 1.0, size=(p.shape[0], nt))), P_TILE, axis=1)[:, :p.shape[1]]
    return rb(p * c, True, accumulated=False) / c


def _attention(qs, k, v, q_pos, k_pos, round_p: bool):
    """Causal GQA attention with q pre-scaled to exp2 units, P rounded to bf16."""
    Tq, H, D = qs.shape
    G = k.shape[1]
    R = H // G
    visible = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]
    out = np.empty((Tq, H, D))
    for h in range(H):
        g = h // R
        s = qs[:, h, :] @ k[:, g, :].T
        s = np.where(visible, s, -np.inf)
        p = _round_p(np.exp2(s - np.max(s, axis=1, keepdims=True)), round_p)
        out[:, h, :] = (p @ v[:, g, :]) / np.sum(p, axis=1, keepdims=True)
    return out


def layer_forward(cfg: dict, w: dict, x: np.ndarray, start_pos: int = 0, past_k=None, past_v=None,
                  rows=None, round: bool = True, out_bf16: bool = False):
    """One sequence through the layer with the bf16 kernels' roundings.

    Arguments and returns as oracle.layer_forward (x [T, d]; past K/V as
    stored, i.e. bf16 values; rows: subset of query rows), with K/V returned
    as the kernels store them.
    """
    H, G = cfg["num_attention_heads"], cfg["num_key_value_heads"]
    d = cfg["hidden_size"]
    D = d // H
    eps = cfg["rms_norm_eps"]
    style = cfg.get("rope_style", "interleaved")
    T = x.shape[0]
    pos = start_pos + np.arange(T)
    g1 = w["input_layernorm"][None, :]
    r1 = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)

    def proj(name):
        return r1 * (x @ rb(w[name] * g1, round, accumulated=False).T)

    k = oracle.apply_rope(proj("k_proj").reshape(T, G, D), pos, cfg["rope_theta"], style)
    k = rb(k, round)
    v = rb(proj("v_proj").reshape(T, G, D), round)
    if past_k is None:
        past_k, past_v = np.zeros((0, G, D)), np.zeros((0, G, D))
    k_all = np.concatenate([past_k, k])
    v_all = np.concatenate([past_v, v])
    sel = np.arange(T) if rows is None else np.asarray(rows)
    xs = x[sel]
    q = oracle.apply_rope(proj("q_proj")[sel].reshape(len(sel), H, D), pos[sel], cfg["rope_theta"], style)
    c = LOG2E / math.sqrt(D)
    qs = rb(q * c, round)
    a = _attention(qs, k_all, v_all, pos[sel], np.arange(k_all.shape[0]), round)
    a = rb(a.reshape(len(sel), H * D), round)
    h = xs + a @ w["o_proj"].T
    r2 = 1.0 / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    hb = rb(h * w["post_attention_layernorm"][None, :], round)
    gate = r2 * (hb @ w["gate_proj"].T)
    up = r2 * (hb @ w["up_proj"].T)
    s = rb(oracle.silu(gate) * up, round)
    out = h + s @ w["down_proj"].T
    return (rb(out, round) if out_bf16 else out), k, v


def prefill(cfg, w, x, rows=None, round=True, out_bf16=False):
    """x [B, S, d] from empty caches: (out [B, S or len(rows), d], K, V)."""
    res = [layer_forward(cfg, w, x[b], 0, rows=rows, round=round, out_bf16=out_bf16) for b in range(x.shape[0])]
    return tuple(np.stack([r[i] for r in res]) for i in range(3))


def decode_step(cfg, w, x, caches, round=True):
    """One decode step: x [B, d], caches[b] = (K, V) as stored; returns (out, new caches)."""
    outs, new = [], []
    for b in range(x.shape[0]):
        pk, pv = caches[b]
        o, k, v = layer_forward(cfg, w, x[b:b + 1], pk.shape[0], pk, pv, round=round)
        outs.append(o[0])
        new.append((np.concatenate([pk, k]), np.concatenate([pv, v])))
    return np.stack(outs), new


def stack_prefill(cfg, layers, final_gamma, x, round=True):
    """The stack with the hidden state held in bf16 between layers, final norm in fp32."""
    ys, ks, vs = [], [], []
    for b in range(x.shape[0]):
        h = x[b]
        kb, vb = [], []
        for w in layers:
            out, k, v = layer_forward(cfg, w, h, 0, round=round)
            h = rb(out, True)  # the stack's storage rounding (the oracle rounds its own hidden state too)
            kb.append(k)
            vb.append(v)
        ys.append(oracle.rms_norm(h, final_gamma, cfg["rms_norm_eps"]))
        ks.append(np.stack(kb))
        vs.append(np.stack(vb))
    return np.stack(ys), np.stack(ks, axis=1), np.stack(vs, axis=1)


def stack_decode_step(cfg, layers, final_gamma, x, caches, round=True, out_bf16=False):
    """One decode step through the stack; caches[l][b] = (K, V) as stored."""
    ys = []
    new = [list(c) for c in caches]
    for b in range(x.shape[0]):
        h = x[b:b + 1]
        for l, w in enumerate(layers):
            pk, pv = new[l][b]
            out, k, v = layer_forward(cfg, w, h, pk.shape[0], pk, pv, round=round)
            new[l][b] = (np.concatenate([pk, k]), np.concatenate([pv, v]))
            h = rb(out, True)
        y = oracle.rms_norm(h, final_gamma, cfg["rms_norm_eps"])[0]
        ys.append(rb(y, round) if out_bf16 else y)
    return np.stack(ys), new
