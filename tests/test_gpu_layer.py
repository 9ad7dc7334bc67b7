"""GPU parity of the C-ABI decoder layer against the float64 oracle.

Every case calls the HIP library through its C ABI on seeded synthetic inputs
and compares element by element with the oracle on the same inputs, at the
tolerances of tests/parity.py.  Small cases cover several tiles and ragged
tails in full; full-size cases compare a seeded sample of rows.
"""
import numpy as np
import pytest
import torch

import oracle
from decoder_block_amd import synth
from tests import parity as P

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _cfg(w):
    return w.config_dict()


def _prefill_case(w, rows=None, out_dtype="f32", gamma_std=None, block_seed=None):
    ws, wo = P.weights_for(w, gamma_std)
    x = synth.layer_input(w)
    layer = P.make_layer(w, ws)
    cache = P.make_cache(layer, w, w.seq_len, w.batch, block_order_seed=block_seed)
    out, sids = P.gpu_prefill(layer, cache, x, out_dtype)
    ref, k_ref, v_ref = oracle.prefill(_cfg(w), wo, synth.as_f64(x), rows=rows)
    got = P.to_np(out) if rows is None else P.to_np(out)[:, rows]
    return got, ref, (layer, cache, sids, k_ref, v_ref)


# ----------------------------------------------------------------------------
# tiny fp32 layer: prefill + 8 decode steps, everything in full
# ----------------------------------------------------------------------------

def test_tiny_fp32_prefill_decode_and_cache():
    w = W[1]
    ws, wo = P.weights_for(w)
    x = synth.layer_input(w)
    layer = P.make_layer(w, ws)
    cache = P.make_cache(layer, w, w.seq_len + w.decode_steps, 1, block_order_seed=5)
    out, sids = P.gpu_prefill(layer, cache, x)
    ref, k_ref, v_ref = oracle.prefill(_cfg(w), wo, synth.as_f64(x))
    e = P.assert_close(P.to_np(out), ref, "f32", "prefill")
    print("prefill", e)
    k, v = cache.read(sids[0], 0, w.seq_len)
    P.assert_close(P.to_np(k), k_ref[0], "f32", "cached K")
    P.assert_close(P.to_np(v), v_ref[0], "f32", "cached V")
    caches = [(k_ref[0], v_ref[0])]
    for step in range(w.decode_steps):
        xt = synth.decode_input(w, step)
        o = layer.decode(cache, sids, xt.cuda())
        torch.cuda.synchronize()
        r, caches = oracle.decode_step(_cfg(w), wo, synth.as_f64(xt), caches)
        e = P.assert_close(P.to_np(o), r, "f32", f"decode step {step}")
    assert cache.seq_len(sids[0]) == w.seq_len + w.decode_steps
    print("decode", e)


# ----------------------------------------------------------------------------
# bf16 layers at reduced sequence length (several tiles, ragged tails), in full
# ----------------------------------------------------------------------------

SMALL = {
    "llama7b-S300": synth.scaled(W[2], seq_len=300),
    "llama3-8b-S333": synth.scaled(W[3], seq_len=333),
    "llama3-8b-B3-S77": synth.scaled(W[3], batch=3, seq_len=77),
    "llama3-70b-B2-S160": synth.scaled(W[5], batch=2, seq_len=160),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_bf16_prefill_small(name):
    w = SMALL[name]
    got, ref, (layer, cache, sids, k_ref, v_ref) = _prefill_case(w, block_seed=11)
    e = P.assert_close(got, ref, "bf16", name)
    print(name, e)
    k, v = cache.read(sids[-1], 0, w.seq_len)
    # cached K/V are bf16-rounded projections of the same inputs
    P.assert_close(P.to_np(k), k_ref[-1], "bf16", "cached K")
    P.assert_close(P.to_np(v), v_ref[-1], "bf16", "cached V")
