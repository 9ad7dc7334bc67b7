"""Device-side checks for reads of memory a call has not written.

* LLAMA_LAYER_POISON=1 fills every call's workspace with 0xFF bytes (NaN in
  fp32 and bf16) before its kernels run: outputs must not change by a bit.
* A cache whose K/V pools start out as NaN (their block table zeroed) must
  give the same outputs as one that starts out as zeros: keys past a
  sequence's end are masked and their values zeroed before use.
"""
import os

import pytest
import torch

from decoder_block_amd import synth
from tests import parity as P

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _run(w, layer, pool_byte=None, decode_steps=2):
    cache = P.make_cache(layer, w, w.seq_len + decode_steps, w.batch, block_order_seed=3)
    if pool_byte is not None:
        cache.pool.fill_(pool_byte)
        cfg = layer.cfg
        D = cfg.hidden_size // cfg.num_attention_heads
        es = 2 if w.dtype == "bf16" else 4
        nb = w.batch * ((w.seq_len + decode_steps + 15) // 16)
        kv = nb * cfg.num_key_value_heads * 16 * D * es
        table = 2 * ((kv + 255) // 256 * 256)
        cache.pool[table:].zero_()  # block tables: never NaN (they are addresses)
        torch.cuda.synchronize()
    x = synth.layer_input(w)
    outs = [P.gpu_prefill(layer, cache, x)[0]]
    sids = list(range(w.batch))
    for step in range(decode_steps):
        outs.append(layer.decode(cache, sids, synth.decode_input(w, step).cuda()))
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("name", ["tiny-fp32", "llama3-8b-B2-S300"])
def test_workspace_poison_changes_nothing(name):
    w = W[1] if name == "tiny-fp32" else synth.scaled(W[3], batch=2, seq_len=300)
    ws, _ = P.weights_for(w)
    layer = P.make_layer(w, ws, max_position=w.seq_len + 4)
    clean = _run(w, layer)
    os.environ["LLAMA_LAYER_POISON"] = "1"
    try:
        poisoned = _run(w, layer)
    finally:
        del os.environ["LLAMA_LAYER_POISON"]
    for a, b in zip(clean, poisoned):
        assert torch.isfinite(b).all()
        assert torch.equal(a, b)


def test_workspace_poison_stack_changes_nothing():
    from decoder_block_amd.llama_layer import DecoderStack
    w = synth.scaled(W[3], batch=2, seq_len=200)
    layers = [P.make_layer(w, synth.layer_weights(w, layer=l), max_position=w.seq_len + 4) for l in range(2)]
    stack = DecoderStack(layers, synth.final_norm_weight(w))
    x = synth.layer_input(w).cuda()
    xt = synth.decode_input(w, 0).cuda()

    def run():
        cache = stack.cache(w.batch * ((w.seq_len + 1 + 15) // 16), w.batch)
        sids = [cache.add_seq() for _ in range(w.batch)]
        y = stack.prefill(cache, sids, x)
        d = stack.decode(cache, sids, xt)
        torch.cuda.synchronize()
        return y, d

    y0, d0 = run()
    os.environ["LLAMA_LAYER_POISON"] = "1"
    try:
        y1, d1 = run()
    finally:
        del os.environ["LLAMA_LAYER_POISON"]
    assert torch.equal(y0, y1) and torch.equal(d0, d1)


@pytest.mark.parametrize("name", ["tiny-fp32", "llama3-8b-B2-S300"])
def test_stale_cache_contents_do_not_leak(name):
    # 300 and 64 tokens end inside a 16-key block and inside a 64-key tile
    w = W[1] if name == "tiny-fp32" else synth.scaled(W[3], batch=2, seq_len=300)
    ws, _ = P.weights_for(w)
    layer = P.make_layer(w, ws, max_position=w.seq_len + 4)
    zeros = _run(w, layer, pool_byte=0)
    nans = _run(w, layer, pool_byte=0xFF)
    for a, b in zip(zeros, nans):
        assert torch.isfinite(b).all()
        assert torch.equal(a, b)
