"""CPU checks that the far-from-zero score inputs of tests/score_cases.py have
the attention scores their docstring states (float64, the oracle's own
projection and RoPE), so that the GPU test built on them exercises what it
claims to."""
from __future__ import annotations

import numpy as np
import pytest

import oracle.layer as L
from decoder_block_amd import synth
from tests import score_cases as SC


def _scores(name):
    """Causal scores in exp2 units [H, T, T] (upper triangle -inf)."""
    w, ws, x = SC.score_case(name)
    cfg = w.config_dict()
    wo = {k: synth.as_f64(v) for k, v in ws.items()}
    x = synth.as_f64(x)[0]
    T, H, G = x.shape[0], cfg["num_attention_heads"], cfg["num_key_value_heads"]
    D = cfg["hidden_size"] // H
    n1 = L.rms_norm(x, wo["input_layernorm"], cfg["rms_norm_eps"])
    pos = np.arange(T)
    q = L.apply_rope(L._split_heads(L.linear(n1, wo["q_proj"]), H), pos, cfg["rope_theta"])
    k = L.apply_rope(L._split_heads(L.linear(n1, wo["k_proj"]), G), pos, cfg["rope_theta"])
    kh = np.repeat(k, H // G, axis=1)
    s = np.einsum("thd,jhd->htj", q, kh) * np.log2(np.e) / np.sqrt(D)
    return np.where(np.tril(np.ones((T, T), bool))[None], s, -np.inf)


def test_case_names():
    assert SC.CASES == ("qk_x2", "qk_x4", "all_high", "all_low", "lane_split")
    with pytest.raises(ValueError):
        SC.score_case("nope")


def test_qk_scaled_cases_cross_the_rise_bound():
    s2 = _scores("qk_x2")
    first = s2[:, :, :64].max(axis=-1)  # max over the first 64-key tile
    whole = s2.max(axis=-1)
    # most rows start below 32 (the running max stays 0), some pass it on a later tile
    assert np.mean(first <= 32) > 0.5
    assert np.any((first <= 32) & (whole > 32))
    s4 = _scores("qk_x4")
    assert np.mean(s4[:, :, :64].max(axis=-1) > 32) > 0.5  # rows exceed 32 on their first tile


def test_all_high_and_all_low_are_uniform_far_from_zero():
    hi = _scores("all_high")
    lo = _scores("all_low")
    vis = np.isfinite(hi)
    assert np.all((hi[vis] > 90) & (hi[vis] < 110))
    assert np.all((lo[vis] < -90) & (lo[vis] > -110))


def test_lane_split_puts_the_high_scores_on_one_lane_half():
    s = _scores("lane_split")
    T = s.shape[1]
    sel = np.arange(T) % 8 >= 4
    vis = np.isfinite(s)
    both = vis & sel[None, :, None] & sel[None, None, :]
    other = vis & ~both
    assert np.all((s[both] > 128) & (s[both] < 170))  # 2^score overflows fp32 without the shift by the row max
    assert np.all(np.abs(s[other]) < 1e-9)
