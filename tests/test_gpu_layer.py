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

# The bf16 error is set by the bf16 storage of q/k/v, P, attn, h and s; it
# shrinks with sequence length (attention averages the value rounding), so the
# reduced cases use at least 300 tokens per sequence.
SMALL = {
    "llama7b-S300": synth.scaled(W[2], seq_len=300),
    "llama3-8b-S333": synth.scaled(W[3], seq_len=333),
    "llama3-8b-B2-S300": synth.scaled(W[3], batch=2, seq_len=300),
    "llama3-70b-B2-S300": synth.scaled(W[5], batch=2, seq_len=300),
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


# ----------------------------------------------------------------------------
# full-size prefill workloads, compared on a seeded sample of rows
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("wid,n_random,edge", [(2, 448, 64), (3, 448, 64), (5, 448, 64)])
def test_bf16_prefill_full_size_sampled_rows(wid, n_random, edge):
    w = W[wid]
    rows = synth.sample_rows(w, w.seq_len, n_random=n_random, edge=edge)
    got, ref, _ = _prefill_case(w, rows=rows)
    e = P.assert_close(got, ref, "bf16", w.name)
    print(w.name, len(rows), "rows/seq", e)


# ----------------------------------------------------------------------------
# batched decode over a paged cache pre-filled with N(0,1) keys/values
# ----------------------------------------------------------------------------

def _decode_setup(w, n_seqs=None, lens=None, block_seed=None, max_position=None, steps=None):
    ws, wo = P.weights_for(w)
    steps = w.decode_steps if steps is None else steps
    layer = P.make_layer(w, ws, max_position or (w.ctx_hi + steps + 1 if lens is None else None))
    lens = synth.context_lengths(w) if lens is None else np.asarray(lens)
    B = len(lens)
    nb = int(sum((l + steps + 15) // 16 for l in lens))
    from decoder_block_amd.llama_layer import PagedKVCache
    order = None
    if block_seed is not None:
        order = np.random.Generator(np.random.PCG64(block_seed)).permutation(nb).tolist()
    cache = PagedKVCache(layer, nb, B, block_order=order)
    sids, host = [], []
    for b in range(B):
        sid = cache.add_seq()
        k, v = synth.cache_contents(w, b, int(lens[b]))
        cache.write(sid, k.cuda(), v.cuda())
        sids.append(sid)
        host.append((k.float().numpy(), v.float().numpy()))
    torch.cuda.synchronize()
    return layer, cache, sids, host, wo


@pytest.mark.timeout(900)
def test_decode_llama3_8b_batch64_33_steps():
    # the decode workload (B 64, contexts U[512, 8192]) over 33 consecutive
    # steps, each compared with the oracle: every sequence crosses at least two
    # 16-token block boundaries, so blocks are allocated mid-decode
    w = W[4]
    layer, cache, sids, host, wo = _decode_setup(w, steps=33)
    lens0 = [cache.seq_len(s) for s in sids]
    worst = {"max_rel": 0.0, "mean_rel": 0.0}
    for step in range(33):
        xt = synth.decode_input(w, step)
        o = layer.decode(cache, sids, xt.cuda())
        torch.cuda.synchronize()
        ref, host = oracle.decode_step(_cfg(w), wo, synth.as_f64(xt), host)
        e = P.assert_close(P.to_np(o), ref, "bf16", f"decode step {step}")
        worst = {k: max(worst[k], e[k]) for k in worst}
    print("decode B=64, 33 steps, worst step", worst)
    for b in range(w.batch):
        assert cache.seq_len(sids[b]) == len(host[b][0]) == lens0[b] + 33
        assert (lens0[b] + 33 + 15) // 16 - (lens0[b] + 15) // 16 >= 2


def test_decode_ragged_lengths_and_group_ratios():
    # lengths straddling block and split boundaries, GQA ratios 16 (G=2) and MHA
    for w in (synth.scaled(W[4], num_key_value_heads=2, batch=5),
              synth.scaled(W[4], num_attention_heads=32, num_key_value_heads=32, batch=5)):
        lens = [1, 15, 16, 1023, 1025]
        layer, cache, sids, host, wo = _decode_setup(w, lens=lens, block_seed=3)
        xt = synth.decode_input(w, 0)
        o = layer.decode(cache, sids, xt.cuda())
        torch.cuda.synchronize()
        ref, _ = oracle.decode_step(_cfg(w), wo, synth.as_f64(xt), host)
        P.assert_close(P.to_np(o), ref, "bf16", f"decode G={w.num_key_value_heads}")


@pytest.mark.parametrize("wid", [1, 4])
def test_decode_context_past_64_key_chunks(wid):
    # 70000 keys: more key chunks than a wave has lanes, so the combine pass
    # takes its chunk statistics in two rounds; a 3-key sequence rides along
    w = synth.scaled(W[wid], batch=2)
    lens = [70000, 3]
    layer, cache, sids, host, wo = _decode_setup(w, lens=lens, block_seed=11, max_position=70008)
    xt = synth.decode_input(w, 0)
    o = layer.decode(cache, sids, xt.cuda())
    torch.cuda.synchronize()
    ref, _ = oracle.decode_step(_cfg(w), wo, synth.as_f64(xt), host)
    e = P.assert_close(P.to_np(o), ref, w.dtype, "decode past 64 chunks")
    print("decode 70000 keys", e)


# ----------------------------------------------------------------------------
# properties of the GPU path
# ----------------------------------------------------------------------------

MID = synth.scaled(W[3], batch=1, seq_len=300)


def test_causal_rows_bitwise_unchanged_by_later_tokens():
    w = MID
    ws, _ = P.weights_for(w)
    layer = P.make_layer(w, ws)
    x = synth.layer_input(w)
    y = x.clone()
    y[:, 150:] = (y[:, 150:].float() * -2.0 + 0.5).to(y.dtype)
    a, _ = P.gpu_prefill(layer, P.make_cache(layer, w, w.seq_len, 1), x)
    b, _ = P.gpu_prefill(layer, P.make_cache(layer, w, w.seq_len, 1), y)
    assert torch.equal(a[:, :150], b[:, :150])
    assert not torch.equal(a[:, 150:], b[:, 150:])


def test_paging_and_reruns_are_bitwise_identical():
    w = synth.scaled(W[3], batch=2, seq_len=200)
    ws, _ = P.weights_for(w)
    layer = P.make_layer(w, ws)
    x = synth.layer_input(w)
    outs, decs = [], []
    for seed in (None, 7, 7):
        cache = P.make_cache(layer, w, w.seq_len + 2, 2, block_order_seed=seed, spare_blocks=3)
        o, sids = P.gpu_prefill(layer, cache, x)
        d = layer.decode(cache, sids, synth.decode_input(w, 0).cuda())
        torch.cuda.synchronize()
        outs.append(o)
        decs.append(d)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])
    assert torch.equal(decs[0], decs[1]) and torch.equal(decs[1], decs[2])


def test_decode_matches_full_recompute_and_continuation_prefill():
    w = synth.scaled(W[3], batch=1, seq_len=301)
    ws, wo = P.weights_for(w)
    layer = P.make_layer(w, ws)
    x = synth.layer_input(w)
    full, _ = P.gpu_prefill(layer, P.make_cache(layer, w, 301, 1), x)
    # prefill 300 then decode the last token
    c1 = P.make_cache(layer, w, 301, 1)
    _, sids = P.gpu_prefill(layer, c1, x[:, :300])
    last = layer.decode(c1, sids, x[:, 300].cuda())
    # prefill 180 then continue with 121 more
    c2 = P.make_cache(layer, w, 301, 1)
    p1, sids2 = P.gpu_prefill(layer, c2, x[:, :180])
    p2, _ = P.gpu_prefill(layer, c2, x[:, 180:].contiguous(), sids=sids2)
    torch.cuda.synchronize()
    ref, _, _ = oracle.prefill(_cfg(w), wo, synth.as_f64(x))
    P.assert_close(P.to_np(last)[0], ref[0, 300], "bf16", "decode vs oracle")
    P.assert_close(P.to_np(full)[0, 300], ref[0, 300], "bf16", "prefill vs oracle")
    P.assert_close(P.to_np(torch.cat([p1, p2], 1)), ref, "bf16", "continuation vs oracle")
    # the first chunk of a continued prefill is the same computation as a plain prefill
    assert torch.equal(p1, full[:, :180])


def test_random_gammas_bf16_full_size_sampled_rows():
    # gamma ~ 1 + N(0, 0.1^2) at the LLaMA-3-8B workload size (B 1, S 8192),
    # compared on the seeded row sample at the workloads' bf16 limits
    w = W[3]
    rows = synth.sample_rows(w, w.seq_len, n_random=448, edge=64)
    got, ref, _ = _prefill_case(w, rows=rows, gamma_std=0.1)
    e = P.assert_close(got, ref, "bf16", "gamma ~ 1 + N(0, 0.1^2), S 8192")
    print("random gammas, S 8192", len(rows), "rows", e)


def test_random_gammas_bf16_300_tokens():
    # the same gammas at 300 tokens: folding gamma_1 into the q/k/v weights adds
    # one bf16 rounding of them, and at this length the error exceeds the
    # workloads' 3e-3 mean limit; held to what the rounding placement predicts
    w = synth.scaled(W[3], batch=1, seq_len=300)
    got, ref, _ = _prefill_case(w, gamma_std=0.1)
    e = P.assert_close(got, ref, P.model_tol("gamma_by_length/300/gamma"), "gamma ~ 1 + N(0, 0.1^2), S 300")
    print("random gammas, S 300", e)


@pytest.mark.parametrize("B,S", [(3, 77), (1, 16)])
def test_bf16_short_prompts(B, S):
    # prompts shorter than the workloads': with few keys per query, attention
    # averages out less of the q/k/v rounding; held to what the rounding
    # placement predicts for these inputs (B 3 S 77 sits just above 3e-3)
    w = synth.scaled(W[3], batch=B, seq_len=S)
    got, ref, _ = _prefill_case(w, block_seed=B + S)
    e = P.assert_close(got, ref, P.model_tol(f"short_prompts/B{B}_S{S}"), f"short prompt B {B} S {S}")
    print("short prompt", B, S, e)


@pytest.mark.parametrize("name", ["qk_x2", "qk_x4", "all_high", "all_low", "lane_split"])
def test_bf16_attention_scores_far_from_zero(name):
    # the prefill attention's running max starts at 0 and moves only for
    # scores outside [-64, 32] (exp2 units): these inputs take every branch
    # of that (a rise on a later tile, a rise on the first tile, all scores
    # about +100 or about -100), and the last puts the high scores on the
    # keys of one lane half only (a row maximum must see both halves);
    # tests/score_cases.py builds them
    from tests import score_cases as SC
    w, ws, x = SC.score_case(name)
    layer = P.make_layer(w, ws)
    cache = P.make_cache(layer, w, w.seq_len, w.batch)
    out, sids = P.gpu_prefill(layer, cache, x)
    wo = {k: synth.as_f64(v) for k, v in ws.items()}
    ref, k_ref, _ = oracle.prefill(_cfg(w), wo, synth.as_f64(x))
    e = P.assert_close(P.to_np(out), ref, P.model_tol(f"score_ranges/{name}"), f"scores far from 0: {name}")
    print("scores far from 0", name, e)


def test_cache_restore_gives_identical_decode():
    w = synth.scaled(W[3], batch=1, seq_len=100)
    ws, _ = P.weights_for(w)
    layer = P.make_layer(w, ws)
    x = synth.layer_input(w)
    c1 = P.make_cache(layer, w, 101, 1)
    _, s1 = P.gpu_prefill(layer, c1, x)
    k, v = c1.read(s1[0], 0, 100)
    c2 = P.make_cache(layer, w, 101, 1, block_order_seed=9)
    s2 = c2.add_seq()
    c2.write(s2, k, v)
    xt = synth.decode_input(w, 3).cuda()
    d1 = layer.decode(c1, s1, xt)
    d2 = layer.decode(c2, [s2], xt)
    torch.cuda.synchronize()
    assert torch.equal(d1, d2)
    k2, v2 = c2.read(s2, 0, 101)
    k1, v1 = c1.read(s1[0], 0, 101)
    assert torch.equal(k1, k2) and torch.equal(v1, v2)


def test_bf16_output_dtype():
    w = synth.scaled(W[3], batch=1, seq_len=64)
    ws, _ = P.weights_for(w)
    layer = P.make_layer(w, ws)
    x = synth.layer_input(w)
    a, _ = P.gpu_prefill(layer, P.make_cache(layer, w, 64, 1), x, out_dtype="f32")
    b, _ = P.gpu_prefill(layer, P.make_cache(layer, w, 64, 1), x, out_dtype="bf16")
    assert b.dtype == torch.bfloat16
    assert torch.equal(a.to(torch.bfloat16), b)


# ----------------------------------------------------------------------------
# half-split RoPE (pairs (i, i + D/2)), a create-time option of the layer
# ----------------------------------------------------------------------------

def test_half_split_rope_tiny_fp32_prefill_decode_and_cache():
    w = synth.scaled(W[1], rope_style="half_split")
    ws, wo = P.weights_for(w)
    x = synth.layer_input(w)
    layer = P.make_layer(w, ws)
    cache = P.make_cache(layer, w, w.seq_len + 3, 1, block_order_seed=2)
    out, sids = P.gpu_prefill(layer, cache, x)
    ref, k_ref, v_ref = oracle.prefill(_cfg(w), wo, synth.as_f64(x))
    P.assert_close(P.to_np(out), ref, "f32", "half-split prefill")
    k, v = cache.read(sids[0], 0, w.seq_len)
    P.assert_close(P.to_np(k), k_ref[0], "f32", "half-split cached K")
    P.assert_close(P.to_np(v), v_ref[0], "f32", "half-split cached V")
    caches = [(k_ref[0], v_ref[0])]
    for step in range(3):
        xt = synth.decode_input(w, step)
        o = layer.decode(cache, sids, xt.cuda())
        torch.cuda.synchronize()
        r, caches = oracle.decode_step(_cfg(w), wo, synth.as_f64(xt), caches)
        P.assert_close(P.to_np(o), r, "f32", f"half-split decode step {step}")


def test_half_split_rope_bf16_prefill_and_decode():
    w = synth.scaled(W[3], batch=2, seq_len=300, rope_style="half_split")
    ws, wo = P.weights_for(w)
    x = synth.layer_input(w)
    layer = P.make_layer(w, ws)
    cache = P.make_cache(layer, w, w.seq_len + 16, w.batch, block_order_seed=4)
    out, sids = P.gpu_prefill(layer, cache, x)
    ref, k_ref, v_ref = oracle.prefill(_cfg(w), wo, synth.as_f64(x))
    e = P.assert_close(P.to_np(out), ref, "bf16", "half-split bf16 prefill")
    print("half-split prefill", e)
    k, _ = cache.read(sids[1], 0, w.seq_len)
    P.assert_close(P.to_np(k), k_ref[1], "bf16", "half-split cached K")
    # one decode step over both sequences (the few-token GEMM path)
    xt = synth.decode_input(w, 0)
    o = layer.decode(cache, sids, xt.cuda())
    torch.cuda.synchronize()
    r, _ = oracle.decode_step(_cfg(w), wo, synth.as_f64(xt), [(k_ref[b], v_ref[b]) for b in range(w.batch)])
    P.assert_close(P.to_np(o), r, "bf16", "half-split decode")


# ----------------------------------------------------------------------------
# GQA ratio sweep: MQA (one K/V head shared by all 32 query heads) and the
# LLaMA-3-405B layer shape (d 16384, 128 query heads over 8 K/V heads, I 53248)
# ----------------------------------------------------------------------------

def test_mqa_bf16_prefill_and_cache():
    w = synth.scaled(synth.VARIANTS["llama3-8b-mqa-layer-prefill"], batch=2, seq_len=300)
    got, ref, (layer, cache, sids, k_ref, v_ref) = _prefill_case(w, block_seed=6)
    e = P.assert_close(got, ref, "bf16", "MQA prefill")
    print("MQA prefill", e)
    k, v = cache.read(sids[1], 0, w.seq_len)
    P.assert_close(P.to_np(k), k_ref[1], "bf16", "MQA cached K")
    P.assert_close(P.to_np(v), v_ref[1], "bf16", "MQA cached V")


def test_mqa_decode_ragged_lengths_two_steps():
    # 32 query heads on one K/V head: two 16-head workgroups per key chunk
    w = synth.scaled(synth.VARIANTS["llama3-8b-mqa-layer-decode"], batch=5)
    layer, cache, sids, host, wo = _decode_setup(w, lens=[1, 16, 333, 1024, 2049], block_seed=8)
    for step in range(2):
        xt = synth.decode_input(w, step)
        o = layer.decode(cache, sids, xt.cuda())
        torch.cuda.synchronize()
        ref, host = oracle.decode_step(_cfg(w), wo, synth.as_f64(xt), host)
        e = P.assert_close(P.to_np(o), ref, "bf16", f"MQA decode step {step}")
        print("MQA decode step", step, e)


def test_mqa_tiny_fp32_prefill_and_decode():
    # head_dim 64, 32 query heads on one K/V head
    w = synth.scaled(W[1], hidden_size=2048, num_attention_heads=32, num_key_value_heads=1, seq_len=200)
    ws, wo = P.weights_for(w)
    x = synth.layer_input(w)
    layer = P.make_layer(w, ws)
    cache = P.make_cache(layer, w, w.seq_len + 2, 1, block_order_seed=1)
    out, sids = P.gpu_prefill(layer, cache, x)
    ref, k_ref, v_ref = oracle.prefill(_cfg(w), wo, synth.as_f64(x))
    P.assert_close(P.to_np(out), ref, "f32", "MQA fp32 prefill")
    caches = [(k_ref[0], v_ref[0])]
    for step in range(2):
        xt = synth.decode_input(w, step)
        o = layer.decode(cache, sids, xt.cuda())
        torch.cuda.synchronize()
        r, caches = oracle.decode_step(_cfg(w), wo, synth.as_f64(xt), caches)
        P.assert_close(P.to_np(o), r, "f32", f"MQA fp32 decode step {step}")


LLAMA3_405B = synth.scaled(synth.VARIANTS["llama3-405b-layer-prefill"], batch=2, seq_len=300)


def test_llama3_405b_layer_prefill_sampled_rows_and_decode():
    # 3.2 G parameters: built here rather than through the shared weight cache
    # so that they are released when the test ends
    w = LLAMA3_405B
    ws = synth.layer_weights(w)
    wo = {k: synth.as_f64(v) for k, v in ws.items()}
    layer = P.make_layer(w, ws)
    del ws
    x = synth.layer_input(w)
    cache = P.make_cache(layer, w, w.seq_len + 1, w.batch, block_order_seed=12)
    out, sids = P.gpu_prefill(layer, cache, x)
    rows = synth.sample_rows(w, w.seq_len, n_random=24, edge=8)
    ref, k_ref, v_ref = oracle.prefill(_cfg(w), wo, synth.as_f64(x), rows=rows)
    e = P.assert_close(P.to_np(out)[:, rows], ref, "bf16", "405B prefill")
    print("405B prefill", len(rows), "rows/seq", e)
    k, v = cache.read(sids[1], 0, w.seq_len)
    P.assert_close(P.to_np(k), k_ref[1], "bf16", "405B cached K")
    P.assert_close(P.to_np(v), v_ref[1], "bf16", "405B cached V")
    # one decode step after the prefill (both sequences at 301 tokens)
    xt = synth.decode_input(w, 0)
    o = layer.decode(cache, sids, xt.cuda())
    torch.cuda.synchronize()
    r, _ = oracle.decode_step(_cfg(w), wo, synth.as_f64(xt), [(k_ref[b], v_ref[b]) for b in range(w.batch)])
    e = P.assert_close(P.to_np(o), r, "bf16", "405B decode")
    print("405B decode", e)


@pytest.mark.parametrize("name,n_random,edge", [("llama3-8b-mqa-layer-prefill", 448, 64),
                                                ("llama3-405b-layer-prefill", 32, 8)])
def test_gqa_sweep_full_size_prefill_sampled_rows(name, n_random, edge):
    # the sweep variants at the sizes bench.py times (B 1, S 8192), compared on
    # a seeded row sample; the 405B weights are built outside the shared cache
    w = synth.VARIANTS[name]
    ws = synth.layer_weights(w)
    wo = {k: synth.as_f64(v) for k, v in ws.items()}
    layer = P.make_layer(w, ws)
    del ws
    x = synth.layer_input(w)
    cache = P.make_cache(layer, w, w.seq_len, w.batch)
    out, _ = P.gpu_prefill(layer, cache, x, out_dtype="bf16")
    rows = synth.sample_rows(w, w.seq_len, n_random=n_random, edge=edge)
    ref, _, _ = oracle.prefill(_cfg(w), wo, synth.as_f64(x), rows=rows)
    e = P.assert_close(P.to_np(out)[:, rows], ref, "bf16", w.name)
    print(w.name, len(rows), "rows", e)


def test_mqa_decode_batch64_full_contexts():
    w = synth.VARIANTS["llama3-8b-mqa-layer-decode"]
    layer, cache, sids, host, wo = _decode_setup(w)
    xt = synth.decode_input(w, 0)
    o = layer.decode(cache, sids, xt.cuda())
    torch.cuda.synchronize()
    ref, _ = oracle.decode_step(_cfg(w), wo, synth.as_f64(xt), host)
    e = P.assert_close(P.to_np(o), ref, "bf16", "MQA decode B=64")
    print("MQA decode B=64", e)



# ----------------------------------------------------------------------------
# bf16 at head_dim 64 (d 2048, 32 query heads) and GQA ratios 2 and 4
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("G", [16, 8])
def test_bf16_head_dim_64_prefill_and_decode(G):
    w = synth.scaled(W[3], hidden_size=2048, intermediate_size=5632, num_key_value_heads=G, batch=2, seq_len=300)
    got, ref, (layer, cache, sids, k_ref, v_ref) = _prefill_case(w, block_seed=G)
    e = P.assert_close(got, ref, "bf16", f"D=64 R={32 // G} prefill")
    print("D=64 prefill", G, e)
    k, v = cache.read(sids[0], 0, w.seq_len)
    P.assert_close(P.to_np(k), k_ref[0], "bf16", "D=64 cached K")
    P.assert_close(P.to_np(v), v_ref[0], "bf16", "D=64 cached V")
    wd = synth.scaled(W[4], hidden_size=2048, intermediate_size=5632, num_key_value_heads=G, batch=4)
    layer_d, cache_d, sids_d, host, wo = _decode_setup(wd, lens=[1, 17, 1024, 2500], block_seed=G + 1)
    xt = synth.decode_input(wd, 0)
    o = layer_d.decode(cache_d, sids_d, xt.cuda())
    torch.cuda.synchronize()
    r, _ = oracle.decode_step(_cfg(wd), wo, synth.as_f64(xt), host)
    e = P.assert_close(P.to_np(o), r, "bf16", f"D=64 R={32 // G} decode")
    print("D=64 decode", G, e)


def test_single_token_prefill_and_wide_decode_batch():
    # a one-token continuation prefill (prefill attention with S = 1) and a
    # decode batch wider than the few-token GEMM path (160 tokens), both
    # against the oracle
    w = synth.scaled(W[3], batch=1, seq_len=120)
    ws, wo = P.weights_for(w)
    layer = P.make_layer(w, ws, max_position=w.seq_len + 2)
    x = synth.layer_input(w)
    cache = P.make_cache(layer, w, w.seq_len + 1, 1)
    _, sids = P.gpu_prefill(layer, cache, x[:, :119])
    one, _ = P.gpu_prefill(layer, cache, x[:, 119:].contiguous(), sids=sids)
    ref, _, _ = oracle.prefill(_cfg(w), wo, synth.as_f64(x), rows=[119])
    P.assert_close(P.to_np(one)[:, 0], ref[:, 0], "bf16", "one-token continuation prefill")
    assert cache.seq_len(sids[0]) == 120

    wd = synth.scaled(W[4], batch=160, ctx_lo=16, ctx_hi=700)
    layer_d, cache_d, sids_d, host, wo_d = _decode_setup(wd, block_seed=13)
    xt = synth.decode_input(wd, 0)
    o = layer_d.decode(cache_d, sids_d, xt.cuda())
    torch.cuda.synchronize()
    r, _ = oracle.decode_step(_cfg(wd), wo_d, synth.as_f64(xt), host)
    P.assert_close(P.to_np(o), r, "bf16", "decode B=160")


@pytest.mark.parametrize("n_new", [100, 128])
def test_few_token_gemm_path_with_two_token_blocks(n_new):
    # 65..128 tokens take the weight-streaming GEMMs with two 64-token blocks
    # (the second ragged at 100): a continuation prefill of that many tokens
    # after 250 cached ones (so every row attends to at least 250 keys, where
    # the bf16 limits hold) and a decode batch of 100 sequences, against the
    # oracle
    w = synth.scaled(W[3], batch=1, seq_len=250 + n_new)
    ws, wo = P.weights_for(w)
    layer = P.make_layer(w, ws)
    x = synth.layer_input(w)
    cache = P.make_cache(layer, w, w.seq_len, 1, block_order_seed=21)
    _, sids = P.gpu_prefill(layer, cache, x[:, :250].contiguous())
    got, _ = P.gpu_prefill(layer, cache, x[:, 250:].contiguous(), sids=sids)
    rows = list(range(250, 250 + n_new))
    ref, k_ref, v_ref = oracle.prefill(_cfg(w), wo, synth.as_f64(x), rows=rows)
    P.assert_close(P.to_np(got), ref, "bf16", f"continuation prefill of {n_new}")
    k, v = cache.read(sids[0], 0, w.seq_len)
    P.assert_close(P.to_np(k), k_ref[0], "bf16", "cached K")
    P.assert_close(P.to_np(v), v_ref[0], "bf16", "cached V")
    if n_new != 100:
        return
    wd = synth.scaled(W[4], batch=100, ctx_lo=16, ctx_hi=700)
    layer_d, cache_d, sids_d, host, wo_d = _decode_setup(wd, block_seed=22)
    for step in range(2):
        xt = synth.decode_input(wd, step)
        o = layer_d.decode(cache_d, sids_d, xt.cuda())
        torch.cuda.synchronize()
        r, host = oracle.decode_step(_cfg(wd), wo_d, synth.as_f64(xt), host)
        P.assert_close(P.to_np(o), r, "bf16", f"decode B=100 step {step}")


def test_hidden_size_not_a_multiple_of_256():
    # d = 17 x 128 = 2176: the o_proj and down weights keep padding rows
    # (2304 stored rows for 2176 features), so their K blocks are 2304 rows
    # apart while the GEMMs produce 2176 features (64-wide tiles)
    w = synth.scaled(W[3], hidden_size=2176, intermediate_size=5888, num_attention_heads=17,
                     num_key_value_heads=17, batch=1, seq_len=300)
    got, ref, (layer, cache, sids, k_ref, v_ref) = _prefill_case(w, block_seed=31)
    P.assert_close(got, ref, "bf16", "d=2176 prefill")
    k, v = cache.read(sids[0], 0, w.seq_len)
    P.assert_close(P.to_np(k), k_ref[0], "bf16", "d=2176 cached K")
    wd = synth.scaled(W[4], hidden_size=2176, intermediate_size=5888, num_attention_heads=17,
                      num_key_value_heads=17, batch=4)
    layer_d, cache_d, sids_d, host, wo = _decode_setup(wd, lens=[5, 300, 1025, 2000], block_seed=32)
    xt = synth.decode_input(wd, 0)
    o = layer_d.decode(cache_d, sids_d, xt.cuda())
    torch.cuda.synchronize()
    r, _ = oracle.decode_step(_cfg(wd), wo, synth.as_f64(xt), host)
    P.assert_close(P.to_np(o), r, "bf16", "d=2176 decode")
