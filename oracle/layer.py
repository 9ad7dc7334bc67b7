"""Plain float64 CPU oracle of one LLaMA-style pre-norm decoder layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module; it exists so that the tests, the smoke check and the benchmark's CPU
baseline have an obviously correct definition to compare against.  It shares
no code with the HIP path and imports nothing from it.

Every step is the plain definition written out in float64, using numpy's
matmul as the only library primitive.  There is no tiling, no online softmax,
no paging and no fusion.  Sources (pages are cited by title and section):

  [P1] "From Transformer to the LLaMA series" (guide, ch. 12), section 8
       "implementing a LLaMA block from scratch" (RMSNorm, rotary tables,
       GQA attention with repeat_interleave, SwiGLU, LlamaBlock).
  [P2] "3.2 Core components, one by one" (LLM full-stack book): 3.2.1 RMSNorm,
       3.2.2 SwiGLU FFN and the 8d/3 sizing rule, 3.2.3 residual connections.
  [P3] "Chapter 10: the modern LLaMA architecture": section 2-3 RoPE with
       even/odd pairs, section 4 RMSNorm, section 5 SwiGLU, section 6 GQA,
       section 7 KV cache prefill/decode, section 8 cache sizes, section 9 the
       block pseudocode.
  [P4] "From Transformer to LLaMA: an overview of modern LLM architecture":
       section 1.1 scaled dot-product attention, 4.2 RoPE frequencies.
  [P5] "LLaMA3 Block: from parts to engine": section 3.1 the two residual
       sub-blocks, 3.2 the 8/3 rule, 4.1 LlamaMLP, 4.2 the decoder layer.

Readings taken where the pages are silent or disagree:
  * eps sits inside the square root: rsqrt(mean(x^2) + eps) (the code on
    P1/P2/P3/P4; P2's displayed formula with eps outside is taken as a typo).
  * RoPE pairs are interleaved (2i, 2i+1) with angle pos * theta^(-2i/D), D the
    head dimension (P3 section 3, P4 section 4.2).  P1's half-split variant
    (pairs (i, i + D/2), same angles) is an option: cfg["rope_style"] =
    "half_split".
  * softmax scale is 1/sqrt(D); query head h reads KV head floor(h / (H/G)).
  * key j is visible to a query iff pos_j <= pos_q (diagonal included); a
    decoded token sits at position = current cache length and is appended to
    the cache before attention.
  * intermediates are kept in float64 (the inputs are the stored bf16 or fp32
    values, converted exactly).
"""
from __future__ import annotations

import math

import numpy as np


# ----------------------------------------------------------------------------
# primitives
# ----------------------------------------------------------------------------

def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x * 1/sqrt(mean(x^2) + eps) * gamma.

    [P1] section 8 RMSNorm; [P2] 3.2.1 (rsqrt of mean of squares plus eps,
    computed at high precision); [P3] section 4; [P4] section 3.2.
    """
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x * (1.0 / np.sqrt(ms + eps)) * gamma


def linear(x: np.ndarray, weight: np.ndarray) -> np.ndarray:
    """Bias-free nn.Linear: y = x @ W^T with W stored [out_features, in_features].

    [P1] section 8 (nn.Linear(..., bias=False)); [P5] section 4.1.
    """
    return x @ weight.T


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """theta_i = theta^(-2i/D) for pair i in [0, D/2).  [P4] 4.2; [P1] section 8."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return theta ** (-2.0 * i / head_dim)


def apply_rope(x: np.ndarray, positions: np.ndarray, theta: float, style: str = "interleaved") -> np.ndarray:
    """Rotate the pairs of every head by pos * theta_i.

    x: [T, heads, D]; positions: [T] absolute positions.
    interleaved ([P3] section 3): pair i = (x[2i], x[2i+1]);
    half_split ([P1] section 8, apply_rope): pair i = (x[i], x[i + D/2]).
    For a pair (e, o): new_e = e cos - o sin, new_o = e sin + o cos.
    """
    D = x.shape[-1]
    if D % 2:
        raise ValueError("RoPE needs an even head dimension")
    ang = np.asarray(positions, dtype=np.float64)[:, None] * rope_inv_freq(D, theta)[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    if style == "interleaved":
        e, o = x[..., 0::2], x[..., 1::2]
    elif style == "half_split":
        e, o = x[..., : D // 2], x[..., D // 2:]
    else:
        raise ValueError(f"unknown RoPE style {style!r}")
    new_e = e * c - o * s
    new_o = e * s + o * c
    if style == "interleaved":
        y = np.empty_like(x)
        y[..., 0::2] = new_e
        y[..., 1::2] = new_o
        return y
    return np.concatenate([new_e, new_o], axis=-1)


def causal_gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                         q_pos: np.ndarray, k_pos: np.ndarray) -> np.ndarray:
    """softmax(q k^T / sqrt(D) + causal mask) v for grouped-query heads.

    q: [Tq, H, D]; k, v: [Tk, G, D]; query head h uses KV head h // (H // G)
    ([P1] section 8 repeat_interleave; [P3] section 6).  Key j is visible to
    query t iff k_pos[j] <= q_pos[t] ([P1] is_causal; [P3] section 7).
    Scale 1/sqrt(D) ([P4] section 1.1).  Returns [Tq, H, D].
    """
    Tq, H, D = q.shape
    G = k.shape[1]
    if H % G:
        raise ValueError("num_attention_heads must be a multiple of num_key_value_heads")
    R = H // G
    visible = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]
    out = np.empty((Tq, H, D), dtype=np.float64)
    scale = 1.0 / math.sqrt(D)
    for h in range(H):
        g = h // R
        s = (q[:, h, :] @ k[:, g, :].T) * scale
        s = np.where(visible, s, -np.inf)
        m = np.max(s, axis=1, keepdims=True)
        w = np.exp(s - m)
        out[:, h, :] = (w @ v[:, g, :]) / np.sum(w, axis=1, keepdims=True)
    return out


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU / Swish with beta = 1: z * sigmoid(z).  [P1] section 5.1; [P2] 3.2.2."""
    return z / (1.0 + np.exp(-z))


def swiglu_ffn(n: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
               w_down: np.ndarray) -> np.ndarray:
    """down( SiLU(gate(n)) * up(n) ): SiLU on the gate branch only.

    [P2] 3.2.2; [P3] section 5; [P5] 4.1 and the gate/up pitfall in section 6.
    """
    return linear(silu(linear(n, w_gate)) * linear(n, w_up), w_down)


# ----------------------------------------------------------------------------
# the layer
# ----------------------------------------------------------------------------

def _split_heads(t: np.ndarray, heads: int) -> np.ndarray:
    T, F = t.shape
    return t.reshape(T, heads, F // heads)


def project_kv(cfg: dict, w: dict, x: np.ndarray, positions: np.ndarray):
    """K (rotated) and V of tokens x [T, d] at the given positions: ([T,G,D], [T,G,D])."""
    G = cfg["num_key_value_heads"]
    n1 = rms_norm(x, w["input_layernorm"], cfg["rms_norm_eps"])
    k = apply_rope(_split_heads(linear(n1, w["k_proj"]), G), positions, cfg["rope_theta"],
                   cfg.get("rope_style", "interleaved"))
    v = _split_heads(linear(n1, w["v_proj"]), G)
    return k, v


def attention_block(cfg: dict, w: dict, x: np.ndarray, positions: np.ndarray,
                    k_all: np.ndarray, v_all: np.ndarray, k_pos: np.ndarray) -> np.ndarray:
    """h = x + o_proj(attn(RoPE(q), K, V)) for query rows x [T, d].

    K/V hold every visible key (cache plus the new tokens), already rotated.
    [P3] section 9; [P5] 3.1 and 4.2 steps 1-4.
    """
    H = cfg["num_attention_heads"]
    n1 = rms_norm(x, w["input_layernorm"], cfg["rms_norm_eps"])
    q = apply_rope(_split_heads(linear(n1, w["q_proj"]), H), positions, cfg["rope_theta"],
                   cfg.get("rope_style", "interleaved"))
    a = causal_gqa_attention(q, k_all, v_all, positions, k_pos)
    return x + linear(a.reshape(x.shape[0], -1), w["o_proj"])


def mlp_block(cfg: dict, w: dict, h: np.ndarray) -> np.ndarray:
    """out = h + SwiGLU(RMSNorm(h)) with the second, separate gamma.  [P5] 4.2 steps 5-8."""
    n2 = rms_norm(h, w["post_attention_layernorm"], cfg["rms_norm_eps"])
    return h + swiglu_ffn(n2, w["gate_proj"], w["up_proj"], w["down_proj"])


def layer_forward(cfg: dict, w: dict, x: np.ndarray, start_pos: int = 0,
                  past_k: np.ndarray | None = None, past_v: np.ndarray | None = None,
                  rows: np.ndarray | None = None):
    """One sequence through the layer.

    x: [T, d] new tokens at positions start_pos .. start_pos+T-1.
    past_k/past_v: [start_pos, G, D] cached keys/values (already rotated).
    rows: optional subset of the T new tokens whose outputs are wanted (the
      outputs of other rows are not computed; K/V of all rows always are).
    Returns (out [len(rows) or T, d], k_new [T,G,D], v_new [T,G,D]).
    """
    T = x.shape[0]
    G = cfg["num_key_value_heads"]
    D = cfg["hidden_size"] // cfg["num_attention_heads"]
    pos = start_pos + np.arange(T)
    k_new, v_new = project_kv(cfg, w, x, pos)
    if past_k is None:
        past_k = np.zeros((0, G, D))
        past_v = np.zeros((0, G, D))
    if past_k.shape[0] != start_pos:
        raise ValueError("cache length must equal the first new position")
    k_all = np.concatenate([past_k, k_new], axis=0)
    v_all = np.concatenate([past_v, v_new], axis=0)
    k_pos = np.arange(k_all.shape[0])
    sel = np.arange(T) if rows is None else np.asarray(rows)
    h = attention_block(cfg, w, x[sel], pos[sel], k_all, v_all, k_pos)
    return mlp_block(cfg, w, h), k_new, v_new


def prefill(cfg: dict, w: dict, x: np.ndarray, rows: np.ndarray | None = None):
    """Causal prefill of a batch x [B, S, d] from empty caches.

    Returns (out [B, S or len(rows), d], K [B,S,G,D], V [B,S,G,D]).
    """
    outs, ks, vs = [], [], []
    for b in range(x.shape[0]):
        o, k, v = layer_forward(cfg, w, x[b], 0, rows=rows)
        outs.append(o)
        ks.append(k)
        vs.append(v)
    return np.stack(outs), np.stack(ks), np.stack(vs)


def decode_step(cfg: dict, w: dict, x: np.ndarray, caches: list):
    """One decode step for B sequences: x [B, d]; caches[b] = (K [len_b,G,D], V).

    The new token of sequence b sits at position len_b, is appended to its
    cache, and attends to all len_b + 1 keys ([P3] sections 3 and 7).  The
    projections, the norms and the MLP act on each row alone, so they are
    applied to the B rows at once; attention runs per sequence over its own
    cache.  Returns (out [B, d], list of updated (K, V)).
    """
    B = x.shape[0]
    H = cfg["num_attention_heads"]
    pos = np.array([c[0].shape[0] for c in caches], dtype=np.int64)
    k_new, v_new = project_kv(cfg, w, x, pos)
    new = [(np.concatenate([pk, k_new[b:b + 1]]), np.concatenate([pv, v_new[b:b + 1]]))
           for b, (pk, pv) in enumerate(caches)]
    n1 = rms_norm(x, w["input_layernorm"], cfg["rms_norm_eps"])
    q = apply_rope(_split_heads(linear(n1, w["q_proj"]), H), pos, cfg["rope_theta"],
                   cfg.get("rope_style", "interleaved"))
    a = np.stack([causal_gqa_attention(q[b:b + 1], new[b][0], new[b][1], pos[b:b + 1],
                                       np.arange(pos[b] + 1))[0] for b in range(B)])
    h = x + linear(a.reshape(B, -1), w["o_proj"])
    return mlp_block(cfg, w, h), new


# ----------------------------------------------------------------------------
# sizing helpers stated on the pages
# ----------------------------------------------------------------------------

def swiglu_hidden(dim: int, multiple_of: int) -> int:
    """int(8d/3) rounded up to a multiple ([P2] 3.2.2 SwiGLUFFN sizing)."""
    mid = int(8 * dim / 3)
    return multiple_of * ((mid + multiple_of - 1) // multiple_of)


def kv_cache_elements(layers: int, batch: int, kv_heads: int, tokens: int, head_dim: int) -> int:
    """K and V elements of a contiguous cache: 2 * L * B * G * T * D ([P3] sections 6 and 8)."""
    return 2 * layers * batch * kv_heads * tokens * head_dim


def layer_parameter_count(hidden: int, heads: int, kv_heads: int, intermediate: int) -> int:
    """Parameters of one layer: q, k, v, o, gate, up, down weights plus two gammas."""
    D = hidden // heads
    attn = hidden * heads * D + 2 * hidden * kv_heads * D + heads * D * hidden
    return attn + 3 * hidden * intermediate + 2 * hidden
