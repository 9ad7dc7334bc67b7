"""CPU checks of the bf16 rounding model behind the derived tolerances: with
its roundings switched off it is the oracle's layer, decode and stack; with
them on, exactly the stored tensors are bf16 values and the error is of the
size one bf16 rounding per stored tensor gives."""
import numpy as np

import oracle
from tests import bf16_model as M

rng = np.random.default_rng(7)


def _cfg(H=4, G=2, d=64, I=40):
    return {"hidden_size": d, "intermediate_size": I, "num_attention_heads": H, "num_key_value_heads": G,
            "rms_norm_eps": 1e-5, "rope_theta": 10000.0}


def _weights(cfg, gamma=True):
    d, I = cfg["hidden_size"], cfg["intermediate_size"]
    D = d // cfg["num_attention_heads"]
    G = cfg["num_key_value_heads"]
    sh = {"q_proj": (d, d), "k_proj": (G * D, d), "v_proj": (G * D, d), "o_proj": (d, d),
          "gate_proj": (I, d), "up_proj": (I, d), "down_proj": (d, I)}
    w = {k: oracle.round_storage(rng.standard_normal(s) * 0.2, "bf16") for k, s in sh.items()}
    for n in ("input_layernorm", "post_attention_layernorm"):
        w[n] = oracle.round_storage(1 + 0.1 * rng.standard_normal(d), "bf16") if gamma else np.ones(d)
    return w


def test_without_rounding_the_model_is_the_oracle_layer():
    cfg = _cfg()
    w = _weights(cfg)
    x = oracle.round_storage(rng.standard_normal((2, 9, 64)), "bf16")
    a, ka, va = oracle.prefill(cfg, w, x)
    b, kb, vb = M.prefill(cfg, w, x, round=False)
    np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(kb, ka, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(vb, va, rtol=1e-12, atol=1e-12)
    rows = np.array([0, 4, 8])
    a2, _, _ = oracle.prefill(cfg, w, x, rows=rows)
    b2, _, _ = M.prefill(cfg, w, x, rows=rows, round=False)
    np.testing.assert_allclose(b2, a2, rtol=1e-12, atol=1e-12)
    caches = [(ka[i], va[i]) for i in range(2)]
    xt = rng.standard_normal((2, 64))
    a3, _ = oracle.decode_step(cfg, w, xt, caches)
    b3, _ = M.decode_step(cfg, w, xt, caches, round=False)
    np.testing.assert_allclose(b3, a3, rtol=1e-12, atol=1e-12)


def test_without_rounding_the_model_stack_is_the_oracle_stack():
    cfg = _cfg()
    layers = [_weights(cfg) for _ in range(2)]
    gf = 1 + 0.1 * rng.standard_normal(64)
    x = oracle.round_storage(rng.standard_normal((1, 7, 64)), "bf16")
    a, ka, va = oracle.stack_prefill(cfg, layers, gf, x, "bf16")
    b, kb, vb = M.stack_prefill(cfg, layers, gf, x, round=False)
    np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-12)
    caches_a = [[(ka[l, 0], va[l, 0])] for l in range(2)]
    xt = rng.standard_normal((1, 64))
    ya, _ = oracle.stack_decode_step(cfg, layers, gf, xt, caches_a, "bf16")
    yb, _ = M.stack_decode_step(cfg, layers, gf, xt, caches_a, round=False)
    np.testing.assert_allclose(yb, ya, rtol=1e-12, atol=1e-12)


def test_rounded_model_stores_bf16_values_and_errs_at_bf16_scale():
    cfg = _cfg()
    w = _weights(cfg)
    x = oracle.round_storage(rng.standard_normal((1, 16, 64)), "bf16")
    ref, kr, _ = oracle.prefill(cfg, w, x)
    got, k, v = M.prefill(cfg, w, x)
    # the cached K/V are what the kernels store: bf16 values
    np.testing.assert_array_equal(oracle.round_storage(k, "bf16"), k)
    np.testing.assert_array_equal(oracle.round_storage(v, "bf16"), v)
    # cached K differs from the oracle's by about one bf16 rounding of itself
    rel = np.abs(k - kr) / np.abs(kr).max()
    assert 0 < rel.max() < 2 ** -7
    e = np.abs(got - ref).mean() / np.sqrt(np.mean(ref ** 2))
    assert 1e-4 < e < 2e-2
    # the bf16 output option rounds the output once more
    got_b, _, _ = M.prefill(cfg, w, x, out_bf16=True)
    np.testing.assert_array_equal(got_b, oracle.round_storage(got, "bf16"))
