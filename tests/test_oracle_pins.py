"""Pins of the float64 oracle to facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: numbers the
pages print (fixtures under tests/golden/), closed forms, invariants, special
cases, or a scalar brute force on tiny inputs.  A plausible slip anywhere in
the oracle (eps outside the root, half-split RoPE, wrong frequency exponent,
a missing 1/sqrt(D), the diagonal masked out, h % G instead of h // R, SiLU on
the up branch, a dropped residual, a transposed weight) fails one of them.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import layer as L
from tests.conftest import golden

rng = np.random.default_rng(12345)


# ----------------------------------------------------------------------------
# RMSNorm
# ----------------------------------------------------------------------------

def test_rmsnorm_page_worked_example():
    g = golden("rmsnorm_worked_example.json")
    x = np.array([g["x"]])
    y = oracle.rms_norm(x, np.ones(2), g["eps"])
    assert math.sqrt(np.mean(x * x)) == pytest.approx(g["rms"], abs=g["abs_tol"])
    np.testing.assert_allclose(y[0], g["y"], atol=g["abs_tol"])


@pytest.mark.parametrize("eps", [0.0, 1e-6, 1e-5, 1e-2])
def test_rmsnorm_unit_rms_closed_form(eps):
    # gamma = 1: mean(y^2) = ms / (ms + eps) exactly ("unit RMS" of the overview page, section 3.2)
    x = rng.standard_normal((7, 96)) * rng.uniform(0.01, 10, size=(7, 1))
    ms = np.mean(x * x, axis=1)
    y = oracle.rms_norm(x, np.ones(96), eps)
    np.testing.assert_allclose(np.mean(y * y, axis=1), ms / (ms + eps), rtol=1e-12)


def test_rmsnorm_eps_inside_the_root():
    # a row whose mean square equals eps: eps inside gives RMS(y) = 1/sqrt(2);
    # eps added outside the root would give sqrt(eps)/(sqrt(eps)+eps) ~ 0.9968.
    eps = 1e-5
    x = np.full((1, 64), math.sqrt(eps))
    y = oracle.rms_norm(x, np.ones(64), eps)
    assert math.sqrt(np.mean(y * y)) == pytest.approx(1 / math.sqrt(2), rel=1e-12)


def test_rmsnorm_does_not_centre_and_scales_by_gamma():
    # constant row: RMSNorm keeps it (LayerNorm would zero it)
    y = oracle.rms_norm(np.full((1, 8), -3.0), np.ones(8), 0.0)
    np.testing.assert_allclose(y, -1.0, rtol=1e-15)
    x = rng.standard_normal((3, 16))
    gam = rng.standard_normal(16)
    np.testing.assert_allclose(oracle.rms_norm(x, gam, 1e-6),
                               oracle.rms_norm(x, np.ones(16), 1e-6) * gam, rtol=1e-14)
    # scale invariance with eps = 0
    np.testing.assert_allclose(oracle.rms_norm(37.5 * x, gam, 0.0),
                               oracle.rms_norm(x, gam, 0.0), rtol=1e-13)


# ----------------------------------------------------------------------------
# Linear orientation
# ----------------------------------------------------------------------------

def test_linear_uses_out_in_layout():
    x = np.array([[1.0, 2.0, 3.0]])
    W = np.array([[1.0, 0.0, 0.0], [0.0, 0.0, 2.0]])     # [out=2, in=3]
    np.testing.assert_array_equal(oracle.linear(x, W), [[1.0, 6.0]])


# ----------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("p", [0, 1, 5, 1000])
def test_rope_interleaved_pairs_and_frequencies(p):
    theta = 10000.0
    pos = np.array([p])
    e = np.eye(4)[:, None, :]                         # four unit vectors, one head, D = 4
    y = oracle.apply_rope(e, np.repeat(pos, 4), theta)[:, 0, :]
    a0, a1 = p * 1.0, p * theta ** (-2.0 / 4)          # theta_0 = 1, theta_1 = theta^(-2/D)
    c0, s0, c1, s1 = math.cos(a0), math.sin(a0), math.cos(a1), math.sin(a1)
    # pair (0, 1) rotates by a0 and pair (2, 3) by a1; half-split pairing would mix 0 with 2
    np.testing.assert_allclose(y[0], [c0, s0, 0, 0], atol=1e-15)
    np.testing.assert_allclose(y[1], [-s0, c0, 0, 0], atol=1e-15)
    np.testing.assert_allclose(y[2], [0, 0, c1, s1], atol=1e-15)
    np.testing.assert_allclose(y[3], [0, 0, -s1, c1], atol=1e-15)


def test_rope_two_dim_closed_form_and_identity_at_zero():
    x = rng.standard_normal((3, 2, 2))
    pos = np.array([0, 3, 7])
    y = oracle.apply_rope(x, pos, 500000.0)
    np.testing.assert_array_equal(y[0], x[0])
    for t in (1, 2):
        c, s = math.cos(pos[t]), math.sin(pos[t])
        x1, x2 = x[t, :, 0], x[t, :, 1]
        np.testing.assert_allclose(y[t, :, 0], x1 * c - x2 * s, rtol=1e-14)
        np.testing.assert_allclose(y[t, :, 1], x1 * s + x2 * c, rtol=1e-14)


def test_rope_preserves_pair_norms():
    x = rng.standard_normal((50, 3, 128))
    pos = rng.integers(0, 8192, size=50)
    y = oracle.apply_rope(x, pos, 500000.0)
    nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(ny, nx, rtol=1e-12)


def test_rope_scores_depend_only_on_offset():
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    def score(m, n):
        return float(np.sum(oracle.apply_rope(q, np.array([m]), 1e4) *
                            oracle.apply_rope(k, np.array([n]), 1e4)))
    for m, n, s in [(5, 2, 100), (0, 0, 4000), (9, 30, 17)]:
        assert score(m, n) == pytest.approx(score(m + s, n + s), rel=1e-10, abs=1e-10)
    # q = k = e0 (frequency 1): q_m . k_n = cos(m - n)
    e0 = np.zeros((1, 1, 64)); e0[..., 0] = 1.0
    for m, n in [(3, 1), (10, 4), (2, 9)]:
        val = np.sum(oracle.apply_rope(e0, np.array([m]), 1e4) * oracle.apply_rope(e0, np.array([n]), 1e4))
        assert val == pytest.approx(math.cos(m - n), abs=1e-14)


@pytest.mark.parametrize("p", [0, 1, 5, 1000])
def test_rope_half_split_pairs_and_frequencies(p):
    # "From Transformer to the LLaMA series", section 8 (apply_rope): x1 = first
    # half, x2 = second half, result [x1 cos - x2 sin, x2 cos + x1 sin], angle
    # pos * theta^(-2i/D) for element i of a half
    theta = 10000.0
    e = np.eye(4)[:, None, :]
    y = oracle.apply_rope(e, np.full(4, p), theta, "half_split")[:, 0, :]
    a0, a1 = p * 1.0, p * theta ** (-2.0 / 4)
    c0, s0, c1, s1 = math.cos(a0), math.sin(a0), math.cos(a1), math.sin(a1)
    # pair (0, 2) rotates by a0 and pair (1, 3) by a1
    np.testing.assert_allclose(y[0], [c0, 0, s0, 0], atol=1e-15)
    np.testing.assert_allclose(y[1], [0, c1, 0, s1], atol=1e-15)
    np.testing.assert_allclose(y[2], [-s0, 0, c0, 0], atol=1e-15)
    np.testing.assert_allclose(y[3], [0, -s1, 0, c1], atol=1e-15)


def test_rope_half_split_is_interleaved_in_reordered_coordinates():
    # reordering a head's elements as (0, D/2, 1, D/2+1, ...) turns the
    # half-split pairs into interleaved ones with the same angles
    D = 16
    perm = np.ravel(np.stack([np.arange(D // 2), np.arange(D // 2) + D // 2], axis=1))
    x = rng.standard_normal((6, 3, D))
    pos = np.array([0, 1, 2, 50, 999, 8191])
    half = oracle.apply_rope(x, pos, 500000.0, "half_split")
    inter = oracle.apply_rope(x[..., perm], pos, 500000.0)
    np.testing.assert_allclose(half[..., perm], inter, rtol=1e-14, atol=1e-14)


def test_rope_half_split_preserves_norms_and_depends_on_offset_only():
    x = rng.standard_normal((20, 2, 64))
    pos = rng.integers(0, 8192, size=20)
    y = oracle.apply_rope(x, pos, 500000.0, "half_split")
    np.testing.assert_allclose(y[..., :32] ** 2 + y[..., 32:] ** 2, x[..., :32] ** 2 + x[..., 32:] ** 2, rtol=1e-12)
    q, k = rng.standard_normal((1, 1, 64)), rng.standard_normal((1, 1, 64))
    def score(m, n):
        return float(np.sum(oracle.apply_rope(q, np.array([m]), 1e4, "half_split") *
                            oracle.apply_rope(k, np.array([n]), 1e4, "half_split")))
    for m, n, sh in [(5, 2, 100), (9, 30, 17)]:
        assert score(m, n) == pytest.approx(score(m + sh, n + sh), rel=1e-10, abs=1e-10)


def test_rope_rejects_odd_head_dim():
    with pytest.raises(ValueError):
        oracle.apply_rope(np.zeros((1, 1, 3)), np.array([0]), 1e4)


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------

def test_attention_position_zero_returns_first_value():
    q = rng.standard_normal((4, 2, 8)); k = rng.standard_normal((4, 1, 8)); v = rng.standard_normal((4, 1, 8))
    o = oracle.causal_gqa_attention(q, k, v, np.arange(4), np.arange(4))
    np.testing.assert_array_equal(o[0, 0], v[0, 0])
    np.testing.assert_array_equal(o[0, 1], v[0, 0])


def test_attention_equal_keys_average_visible_values():
    # identical keys: uniform weights over the visible prefix, diagonal included
    T = 6
    q = rng.standard_normal((T, 1, 4)); k = np.tile(rng.standard_normal((1, 1, 4)), (T, 1, 1))
    v = rng.standard_normal((T, 1, 4))
    o = oracle.causal_gqa_attention(q, k, v, np.arange(T), np.arange(T))
    for t in range(T):
        np.testing.assert_allclose(o[t, 0], v[: t + 1, 0].mean(axis=0), rtol=1e-13, atol=1e-15)


def test_attention_scale_is_inverse_sqrt_head_dim():
    D = 16
    q = np.zeros((2, 1, D)); q[1, 0, 0] = 3.0
    k = np.zeros((2, 1, D)); k[0, 0, 0] = 1.0; k[1, 0, 0] = 2.0
    v = np.zeros((2, 1, D)); v[0, 0, 1] = 1.0; v[1, 0, 2] = 1.0
    o = oracle.causal_gqa_attention(q, k, v, np.arange(2), np.arange(2))
    # scores 3 and 6 scaled by 1/4: weight of key 1 = 1 / (1 + exp(-(6-3)/4))
    w1 = 1.0 / (1.0 + math.exp(-0.75))
    np.testing.assert_allclose(o[1, 0, 1:3], [1 - w1, w1], rtol=1e-14)


def test_attention_query_head_to_kv_head_map():
    # H = 4, G = 2: heads 0,1 read KV head 0 and heads 2,3 read KV head 1 (h // R, not h % G)
    q = rng.standard_normal((1, 4, 8)); k = rng.standard_normal((1, 2, 8)); v = rng.standard_normal((1, 2, 8))
    o = oracle.causal_gqa_attention(q, k, v, np.array([0]), np.array([0]))
    for h, g in [(0, 0), (1, 0), (2, 1), (3, 1)]:
        np.testing.assert_array_equal(o[0, h], v[0, g])


def test_gqa_equals_mha_with_repeated_kv():
    T, G, R, D = 9, 2, 3, 8
    q = rng.standard_normal((T, G * R, D)); k = rng.standard_normal((T, G, D)); v = rng.standard_normal((T, G, D))
    gqa = oracle.causal_gqa_attention(q, k, v, np.arange(T), np.arange(T))
    mha = oracle.causal_gqa_attention(q, np.repeat(k, R, axis=1), np.repeat(v, R, axis=1),
                                      np.arange(T), np.arange(T))
    np.testing.assert_allclose(gqa, mha, rtol=1e-15, atol=1e-15)


def _brute_attention(q, k, v, qp, kp):
    """Scalar-loop softmax attention (tiny inputs only)."""
    Tq, H, D = q.shape
    G = k.shape[1]
    out = [[[0.0] * D for _ in range(H)] for _ in range(Tq)]
    for t in range(Tq):
        for h in range(H):
            g = h * G // H
            scores = []
            for j in range(k.shape[0]):
                if kp[j] <= qp[t]:
                    s = 0.0
                    for d in range(D):
                        s += q[t, h, d] * k[j, g, d]
                    scores.append((j, s / math.sqrt(D)))
            mx = max(s for _, s in scores)
            den = sum(math.exp(s - mx) for _, s in scores)
            for d in range(D):
                out[t][h][d] = sum(math.exp(s - mx) * v[j, g, d] for j, s in scores) / den
    return np.array(out)


def test_attention_matches_brute_force_with_offset_positions():
    q = rng.standard_normal((3, 4, 4)); k = rng.standard_normal((7, 2, 4)); v = rng.standard_normal((7, 2, 4))
    qp, kp = np.array([4, 5, 6]), np.arange(7)
    np.testing.assert_allclose(oracle.causal_gqa_attention(q, k, v, qp, kp),
                               _brute_attention(q, k, v, qp, kp), rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------
# SwiGLU and residuals
# ----------------------------------------------------------------------------

def test_silu_shape():
    assert float(oracle.silu(np.array(0.0))) == 0.0
    assert float(oracle.silu(np.array(30.0))) == pytest.approx(30.0, rel=1e-12)
    assert abs(float(oracle.silu(np.array(-40.0)))) < 1e-15
    # z*sigmoid(z) has its minimum where 1 + z(1 - sigmoid(z)) = 0 (z ~ -1.2785)
    from scipy.optimize import brentq, minimize_scalar
    z0 = brentq(lambda z: 1 + z * (1 - 1 / (1 + math.exp(-z))), -3, 0)
    r = minimize_scalar(lambda z: float(oracle.silu(np.array(z))), bounds=(-5, 0), method="bounded",
                        options={"xatol": 1e-10})
    assert r.x == pytest.approx(z0, abs=1e-5)
    assert r.fun == pytest.approx(z0 / (1 + math.exp(-z0)), abs=1e-12)
    assert r.fun == pytest.approx(-0.2785, abs=1e-4)


def test_gating_page_example_through_the_ffn():
    # up and activated gate from the page; pre-activations found by root finding
    g = golden("gating_example.json")
    from scipy.optimize import brentq
    pre = [brentq(lambda z, t=t: z / (1 + math.exp(-z)) - t, -0.5, 10) if t > 0 else 0.0
           for t in g["gate"]]
    n = np.array([[1.0, 0.0, 0.0]])
    w_gate = np.zeros((3, 3)); w_gate[:, 0] = pre
    w_up = np.zeros((3, 3)); w_up[:, 0] = g["up"]
    y = oracle.swiglu_ffn(n, w_gate, w_up, np.eye(3))
    np.testing.assert_allclose(y[0], g["after"], atol=1e-12)
    # swapping gate and up (SiLU on the up branch) gives something else
    y_swapped = oracle.swiglu_ffn(n, w_up, w_gate, np.eye(3))
    assert np.max(np.abs(y_swapped - y)) > 0.1


def test_zero_gate_weights_zero_ffn():
    n = rng.standard_normal((4, 6))
    y = oracle.swiglu_ffn(n, np.zeros((10, 6)), rng.standard_normal((10, 6)), rng.standard_normal((6, 10)))
    np.testing.assert_array_equal(y, 0.0)


def _tiny_cfg(H=4, G=2, d=32, I=24, eps=1e-5, theta=10000.0):
    return dict(hidden_size=d, intermediate_size=I, num_attention_heads=H,
                num_key_value_heads=G, rms_norm_eps=eps, rope_theta=theta)


def _tiny_weights(cfg, std=0.3, seed=0):
    r = np.random.default_rng(seed)
    d, I = cfg["hidden_size"], cfg["intermediate_size"]
    H, G = cfg["num_attention_heads"], cfg["num_key_value_heads"]
    D = d // H
    return {"q_proj": r.standard_normal((H * D, d)) * std, "k_proj": r.standard_normal((G * D, d)) * std,
            "v_proj": r.standard_normal((G * D, d)) * std, "o_proj": r.standard_normal((d, H * D)) * std,
            "gate_proj": r.standard_normal((I, d)) * std, "up_proj": r.standard_normal((I, d)) * std,
            "down_proj": r.standard_normal((d, I)) * std,
            "input_layernorm": 1 + 0.1 * r.standard_normal(d),
            "post_attention_layernorm": 1 + 0.1 * r.standard_normal(d)}


def test_residual_identities():
    cfg = _tiny_cfg()
    w = _tiny_weights(cfg)
    x = rng.standard_normal((5, 32))
    w0 = dict(w, o_proj=np.zeros_like(w["o_proj"]))
    k, v = oracle.project_kv(cfg, w0, x, np.arange(5))
    np.testing.assert_array_equal(oracle.attention_block(cfg, w0, x, np.arange(5), k, v, np.arange(5)), x)
    h = rng.standard_normal((5, 32))
    wd0 = dict(w, down_proj=np.zeros_like(w["down_proj"]))
    np.testing.assert_array_equal(oracle.mlp_block(cfg, wd0, h), h)
    both = dict(w0, down_proj=np.zeros_like(w["down_proj"]))
    out, _, _ = oracle.layer_forward(cfg, both, x)
    np.testing.assert_array_equal(out, x)


def test_values_are_not_rotated():
    cfg = _tiny_cfg()
    w = _tiny_weights(cfg)
    x = rng.standard_normal((3, 32))
    k0, v0 = oracle.project_kv(cfg, w, x, np.arange(3))
    k1, v1 = oracle.project_kv(cfg, w, x, np.arange(3) + 100)
    np.testing.assert_array_equal(v0, v1)
    assert np.max(np.abs(k0 - k1)) > 1e-3


# ----------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------

def _brute_layer(cfg, w, x):
    """Scalar-loop decoder layer for one short sequence from empty cache."""
    half = cfg.get("rope_style", "interleaved") == "half_split"
    d, I = cfg["hidden_size"], cfg["intermediate_size"]
    H, G = cfg["num_attention_heads"], cfg["num_key_value_heads"]
    D, eps, th = d // H, cfg["rms_norm_eps"], cfg["rope_theta"]
    T = x.shape[0]

    def norm(row, gam):
        ms = sum(v * v for v in row) / len(row)
        r = 1.0 / math.sqrt(ms + eps)
        return [row[i] * r * gam[i] for i in range(len(row))]

    def mat(row, W):
        return [sum(W[o][i] * row[i] for i in range(len(row))) for o in range(len(W))]

    def rot(vec, p):
        out = list(vec)
        for hd in range(len(vec) // D):
            for i in range(D // 2):
                a = p * th ** (-2.0 * i / D)
                # pair i: interleaved (2i, 2i+1), or the two halves (i, i + D/2)
                ie, io = (hd * D + i, hd * D + i + D // 2) if half else (hd * D + 2 * i, hd * D + 2 * i + 1)
                e, o = vec[ie], vec[io]
                out[ie] = e * math.cos(a) - o * math.sin(a)
                out[io] = e * math.sin(a) + o * math.cos(a)
        return out

    xs = [list(r) for r in x]
    n1 = [norm(r, w["input_layernorm"]) for r in xs]
    qs = [rot(mat(n1[t], w["q_proj"]), t) for t in range(T)]
    ks = [rot(mat(n1[t], w["k_proj"]), t) for t in range(T)]
    vs = [mat(n1[t], w["v_proj"]) for t in range(T)]
    outs = []
    for t in range(T):
        att = []
        for h in range(H):
            g = h // (H // G)
            sc = [sum(qs[t][h * D + i] * ks[j][g * D + i] for i in range(D)) / math.sqrt(D) for j in range(t + 1)]
            mx = max(sc)
            ws = [math.exp(s - mx) for s in sc]
            att += [sum(ws[j] * vs[j][g * D + i] for j in range(t + 1)) / sum(ws) for i in range(D)]
        h_row = [xs[t][i] + v for i, v in enumerate(mat(att, w["o_proj"]))]
        n2 = norm(h_row, w["post_attention_layernorm"])
        gt, up = mat(n2, w["gate_proj"]), mat(n2, w["up_proj"])
        s = [gt[i] / (1 + math.exp(-gt[i])) * up[i] for i in range(I)]
        outs.append([h_row[i] + v for i, v in enumerate(mat(s, w["down_proj"]))])
    return np.array(outs)


@pytest.mark.parametrize("H,G,style", [(4, 2, "interleaved"), (2, 2, "interleaved"), (4, 1, "interleaved"),
                                       (4, 2, "half_split")])
def test_layer_matches_scalar_brute_force(H, G, style):
    cfg = dict(_tiny_cfg(H=H, G=G, d=16, I=12), rope_style=style)
    w = _tiny_weights(cfg, seed=H * 10 + G)
    x = rng.standard_normal((5, 16))
    out, _, _ = oracle.layer_forward(cfg, w, x)
    np.testing.assert_allclose(out, _brute_layer(cfg, w, x), rtol=1e-11, atol=1e-12)


def test_gqa_layer_equals_mha_layer_with_repeated_kv_rows():
    cfg = _tiny_cfg(H=6, G=2, d=48, I=20)
    w = _tiny_weights(cfg)
    D, R = 8, 3
    def rep(W):  # repeat each KV head's D rows R times, in repeat_interleave order
        return np.concatenate([np.tile(W[g * D:(g + 1) * D], (R, 1)) for g in range(2)], axis=0)
    mha_cfg = dict(cfg, num_key_value_heads=6)
    mha_w = dict(w, k_proj=rep(w["k_proj"]), v_proj=rep(w["v_proj"]))
    x = rng.standard_normal((7, 48))
    a, _, _ = oracle.layer_forward(cfg, w, x)
    b, _, _ = oracle.layer_forward(mha_cfg, mha_w, x)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)


def test_causal_outputs_ignore_later_tokens():
    cfg = _tiny_cfg()
    w = _tiny_weights(cfg)
    x = rng.standard_normal((10, 32))
    y = x.copy(); y[6:] += rng.standard_normal((4, 32)) * 5
    a, _, _ = oracle.layer_forward(cfg, w, x)
    b, _, _ = oracle.layer_forward(cfg, w, y)
    np.testing.assert_array_equal(a[:6], b[:6])
    assert np.max(np.abs(a[6:] - b[6:])) > 1e-3


def test_decode_equals_full_recompute():
    cfg = _tiny_cfg(H=4, G=2)
    w = _tiny_weights(cfg)
    S, steps = 9, 5
    x = rng.standard_normal((1, S + steps, 32))
    full, kf, vf = oracle.prefill(cfg, w, x)
    _, k, v = oracle.prefill(cfg, w, x[:, :S])
    caches = [(k[0], v[0])]
    for t in range(steps):
        o, caches = oracle.decode_step(cfg, w, x[:, S + t], caches)
        np.testing.assert_allclose(o[0], full[0, S + t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(caches[0][0], kf[0], rtol=1e-12, atol=1e-12)


def test_batched_decode_of_ragged_sequences_equals_full_recompute():
    # three sequences at different lengths decode together for three steps;
    # each step of each sequence equals its own full causal recompute
    cfg = _tiny_cfg(H=4, G=2)
    w = _tiny_weights(cfg, seed=3)
    lens, steps = [1, 6, 11], 3
    xs = [rng.standard_normal((n + steps, 32)) for n in lens]
    caches = []
    for b, n in enumerate(lens):
        _, k, v = oracle.layer_forward(cfg, w, xs[b][:n])
        caches.append((k, v))
    for t in range(steps):
        xt = np.stack([xs[b][lens[b] + t] for b in range(3)])
        o, caches = oracle.decode_step(cfg, w, xt, caches)
        for b, n in enumerate(lens):
            full, _, _ = oracle.layer_forward(cfg, w, xs[b][:n + t + 1])
            np.testing.assert_allclose(o[b], full[-1], rtol=1e-12, atol=1e-12)
    assert [c[0].shape[0] for c in caches] == [n + steps for n in lens]


def test_subset_rows_equal_full_rows():
    cfg = _tiny_cfg()
    w = _tiny_weights(cfg)
    x = rng.standard_normal((2, 12, 32))
    full, _, _ = oracle.prefill(cfg, w, x)
    rows = np.array([0, 3, 11])
    sub, _, _ = oracle.prefill(cfg, w, x, rows=rows)
    np.testing.assert_array_equal(sub, full[:, rows])


def test_batch_sequences_are_independent():
    cfg = _tiny_cfg()
    w = _tiny_weights(cfg)
    x = rng.standard_normal((3, 6, 32))
    full, _, _ = oracle.prefill(cfg, w, x)
    one, _, _ = oracle.prefill(cfg, w, x[1:2])
    np.testing.assert_array_equal(full[1], one[0])


# ----------------------------------------------------------------------------
# sizes printed on the pages
# ----------------------------------------------------------------------------

def test_parameter_counts_of_page_model():
    g = golden("parameter_counts.json")
    def total(kv):
        per = oracle.layer_parameter_count(g["hidden"], g["heads"], kv, g["ffn_hidden"])
        return g["layers"] * per + 2 * g["vocab"] * g["hidden"] + g["hidden"]
    assert total(g["gqa_kv_heads"]) == g["gqa_total"]
    assert total(g["mha_kv_heads"]) == g["mha_total"]
    assert total(g["mha_kv_heads"]) - total(g["gqa_kv_heads"]) == g["saved"]


def test_kv_cache_bytes_of_page_example():
    g = golden("kv_cache_bytes.json")
    gqa = oracle.kv_cache_elements(g["layers"], g["batch"], g["kv_heads"], g["tokens"], g["head_dim"])
    mha = oracle.kv_cache_elements(g["layers"], g["batch"], g["heads"], g["tokens"], g["head_dim"])
    assert gqa * g["bytes_per_element"] == g["gqa_bytes"]
    assert mha // gqa == g["mha_over_gqa"]


def test_swiglu_sizing_rule():
    # int(8d/3) rounded up to a multiple: reproduces the tiny and the 7B-shaped layers
    assert oracle.swiglu_hidden(256, 16) == 688
    assert oracle.swiglu_hidden(4096, 256) == 11008
    for d, m in [(256, 16), (4096, 256), (512, 64)]:
        I = oracle.swiglu_hidden(d, m)
        assert abs(3 * d * I - 8 * d * d) <= 3 * d * m     # 3 d I = 8 d^2 up to the rounding
    # the LLaMA-3 table widths are not from this rule: 3 d I / 8 d^2 = 1.3125 for both
    g = golden("llama3_shapes.json")["models"]
    for name in ("8B", "70B"):
        d, I = g[name]["hidden"], g[name]["intermediate"]
        assert 3 * d * I / (8 * d * d) == pytest.approx(1.3125)
        assert g[name]["q_heads"] // g[name]["kv_heads"] == g[name]["ratio"]


# ----------------------------------------------------------------------------
# N-layer stack + final RMSNorm
# ----------------------------------------------------------------------------

def test_round_storage_bf16_known_values_and_ties():
    from oracle.stack import round_storage
    cases = [(1.0 + 2.0 ** -8, 1.0),                    # half-way, 1.0 is even
             (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),    # half-way, the upper neighbour is even
             (1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0 + 2.0 ** -7),  # just above half-way
             (-(1.0 + 2.0 ** -8), -1.0),
             (0.1, 0.10009765625),                     # 0x3DCD
             (3.0, 3.0), (-2.0 ** -20, -2.0 ** -20), (0.0, 0.0)]
    for v, want in cases:
        assert round_storage(np.array([v]), "bf16")[0] == want, v


def test_round_storage_bf16_matches_torch_rounding_of_float32():
    import torch
    from oracle.stack import round_storage
    v = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_storage(v.astype(np.float64), "bf16"), want)


def test_round_storage_f32_matches_struct_packing():
    import struct
    from oracle.stack import round_storage
    v = rng.standard_normal(2000) * 3.0
    want = np.array([struct.unpack("<f", struct.pack("<f", float(a)))[0] for a in v])
    np.testing.assert_array_equal(round_storage(v, "f32"), want)


def _stack_case(n_layers=3, H=4, G=2, d=16, I=12, gamma_std=0.2):
    cfg = _tiny_cfg(H=H, G=G, d=d, I=I)
    layers = [_tiny_weights(cfg, seed=100 + l) for l in range(n_layers)]
    gf = 1.0 + gamma_std * rng.standard_normal(d)
    return cfg, layers, gf


def test_stack_with_zero_residual_branches_is_the_final_norm_of_its_input():
    # o_proj = 0 and down_proj = 0 make every layer the identity on x
    cfg, layers, gf = _stack_case()
    for w in layers:
        w["o_proj"] = np.zeros_like(w["o_proj"])
        w["down_proj"] = np.zeros_like(w["down_proj"])
    from oracle.stack import round_storage
    x = round_storage(rng.standard_normal((2, 7, 16)), "bf16")
    y, _, _ = oracle.stack_prefill(cfg, layers, gf, x, "bf16")
    for b in range(2):
        for t in range(7):
            row = x[b, t]
            r = 1.0 / math.sqrt(sum(v * v for v in row) / len(row) + cfg["rms_norm_eps"])
            np.testing.assert_allclose(y[b, t], [row[i] * r * gf[i] for i in range(16)], rtol=1e-13, atol=1e-14)


def test_stack_matches_scalar_brute_force_composition():
    from oracle.stack import round_storage
    cfg, layers, gf = _stack_case(n_layers=2, H=4, G=1)
    x = round_storage(rng.standard_normal((5, 16)), "bf16")
    h = x
    for w in layers:
        h = round_storage(_brute_layer(cfg, w, h), "bf16")
    eps = cfg["rms_norm_eps"]
    want = [[v / math.sqrt(sum(u * u for u in row) / len(row) + eps) * gf[i] for i, v in enumerate(row)]
            for row in h.tolist()]
    y, k, v = oracle.stack_prefill(cfg, layers, gf, x[None], "bf16")
    np.testing.assert_allclose(y[0], want, rtol=1e-10, atol=1e-12)
    assert k.shape == (2, 1, 5, 1, 4) and v.shape == (2, 1, 5, 1, 4)


def test_stack_boundary_rounding_is_applied():
    # without the rounding between layers the result moves by about 2^-9
    from oracle.stack import round_storage
    cfg, layers, gf = _stack_case(n_layers=2)
    x = round_storage(rng.standard_normal((1, 6, 16)), "bf16")
    y_bf, _, _ = oracle.stack_prefill(cfg, layers, gf, x, "bf16")
    y_f32, _, _ = oracle.stack_prefill(cfg, layers, gf, x, "f32")
    rel = np.abs(y_bf - y_f32).max() / np.abs(y_f32).max()
    assert 1e-5 < rel < 2e-2


def test_stack_decode_reproduces_full_recompute():
    # a token decoded against the per-layer caches of a prefill gets the output
    # the full prefill gives at its position ("Chapter 10", section 7)
    from oracle.stack import round_storage
    cfg, layers, gf = _stack_case(n_layers=3, H=4, G=2)
    x = round_storage(rng.standard_normal((2, 9, 16)), "bf16")
    full, _, _ = oracle.stack_prefill(cfg, layers, gf, x, "bf16")
    part, k, v = oracle.stack_prefill(cfg, layers, gf, x[:, :7], "bf16")
    np.testing.assert_allclose(part, full[:, :7], rtol=1e-12, atol=1e-13)
    caches = [[(k[l, b], v[l, b]) for b in range(2)] for l in range(3)]
    for t in (7, 8):
        y, caches = oracle.stack_decode_step(cfg, layers, gf, x[:, t], caches, "bf16")
        np.testing.assert_allclose(y, full[:, t], rtol=1e-10, atol=1e-12)
    assert caches[2][1][0].shape == (9, 2, 4)
