"""GPU check of llama_layer_decode_noalloc (the decode entry point that takes
its workspace from the library's static scratch buffer) against
llama_layer_decode on identical caches: two calls in a row, the second with a
smaller batch, outputs and appended K/V bit-identical."""
import numpy as np
import pytest
import torch

from decoder_block_amd import llama_layer as L
from decoder_block_amd import synth
from tests import parity as P

pytestmark = pytest.mark.gpu


def _cache(layer, w, lens, order_seed):
    nb = int(sum((l + 4 + 15) // 16 for l in lens))
    order = np.random.Generator(np.random.PCG64(order_seed)).permutation(nb).tolist()
    cache = L.PagedKVCache(layer, nb, len(lens), block_order=order)
    sids = []
    for b, n in enumerate(lens):
        sid = cache.add_seq()
        k, v = synth.cache_contents(w, b, int(n))
        cache.write(sid, k.cuda(), v.cuda())
        sids.append(sid)
    return cache, sids


@pytest.mark.parametrize("wid", [1, 4])
def test_decode_noalloc_matches_decode(wid):
    w = synth.scaled(synth.WORKLOADS[wid], batch=9)
    ws, _ = P.weights_for(w)
    layer = P.make_layer(w, ws, max_position=3000)
    lens = [1, 15, 16, 17, 300, 1023, 1024, 1025, 2500]
    ref_cache, ref_ids = _cache(layer, w, lens, 3)
    na_cache, na_ids = _cache(layer, w, lens, 3)
    odt = "f32"
    for step, pick in enumerate([list(range(9)), [8, 2, 5]]):  # the second call is smaller
        x = synth.decode_input(w, step)[pick].contiguous().cuda()
        a = layer.decode(ref_cache, [ref_ids[i] for i in pick], x, out_dtype=odt)
        b = torch.full_like(a, float("nan"))
        L.llama_layer_decode_noalloc(layer.handle, na_cache.handle, len(pick), [na_ids[i] for i in pick], x, b,
                                     L.LLAMA_DTYPE_F32)
        torch.cuda.synchronize()
        assert torch.equal(a, b), f"call {step}: max diff {(a - b).abs().max().item()}"
        for i in pick:
            n = ref_cache.seq_len(ref_ids[i])
            assert na_cache.seq_len(na_ids[i]) == n
            k1, v1 = ref_cache.read(ref_ids[i], 0, n)
            k2, v2 = na_cache.read(na_ids[i], 0, n)
            assert torch.equal(k1, k2) and torch.equal(v1, v2)


def test_decode_noalloc_rejects_a_batch_beyond_the_scratch_buffer():
    # 2048 tokens of the LLaMA-3-8B shape need more workspace than the static
    # buffer holds: refused on the host, nothing launched
    w = synth.WORKLOADS[4]
    cfg = L.make_config(w.hidden_size, w.intermediate_size, w.num_attention_heads, w.num_key_value_heads,
                        w.rms_norm_eps, w.rope_theta, 9000, "bf16")
    ws, _ = P.weights_for(synth.scaled(w, batch=1))
    layer = P.make_layer(synth.scaled(w, batch=1), ws, max_position=9000)
    assert L.llama_layer_workspace_bytes(layer.handle, 2048, 2048) > L.SCRATCH_BYTES
    cache = L.PagedKVCache(layer, 4, 1)
    x = torch.zeros(2048, cfg.hidden_size, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(L.LlamaError) as e:
        L.llama_layer_decode_noalloc(layer.handle, cache.handle, 2048, [0] * 2048, x, x, L.LLAMA_DTYPE_BF16)
    assert L.STATUS[e.value.status] == "LLAMA_ERR_SCRATCH"
