"""Pins of the seeded input generator (shared by the oracle tests and the GPU harness)."""
import numpy as np
import torch

from decoder_block_amd import synth


def test_bf16_storage_is_round_to_nearest_even():
    one = 1.0
    cases = {
        one + 2 ** -8: one,                      # tie between 1 and 1+2^-7: even mantissa wins
        one + 3 * 2 ** -8: one + 2 ** -6,        # tie between 1+2^-7 and 1+2^-6: even wins
        one + 2 ** -8 + 2 ** -20: one + 2 ** -7,  # just above the tie rounds up
        one + 2 ** -8 - 2 ** -20: one,           # just below the tie rounds down
        -(one + 3 * 2 ** -8): -(one + 2 ** -6),
        0.02: 0.02001953125,
    }
    src = np.array(list(cases.keys()), dtype=np.float32)
    got = synth.storage(src, "bf16").to(torch.float64).numpy()
    np.testing.assert_array_equal(got, np.array(list(cases.values())))


def test_draws_do_not_depend_on_thread_count(monkeypatch):
    a = synth.normal_f32(7, (3, 3_000_000), std=0.5)
    monkeypatch.setattr(synth, "_threads", lambda: 1)
    b = synth.normal_f32(7, (3, 3_000_000), std=0.5)
    np.testing.assert_array_equal(a, b)
    assert abs(float(a.std()) - 0.5) < 1e-3


def test_workload_recipes():
    w = synth.WORKLOADS[4]
    lens = synth.context_lengths(w)
    assert lens.min() >= 512 and lens.max() <= 8192 and lens.shape == (64,)
    rows = synth.sample_rows(synth.WORKLOADS[3], 8192)
    assert rows.size == 576 and rows[0] == 0 and rows[-1] == 8191
    tiny = synth.WORKLOADS[1]
    ws = synth.layer_weights(tiny)
    assert ws["q_proj"].dtype == torch.float32 and ws["q_proj"].shape == (256, 256)
    assert ws["k_proj"].shape == (128, 256)
    assert abs(float(ws["input_layernorm"].mean()) - 1.0) < 0.05
    w2 = synth.scaled(synth.WORKLOADS[2], seq_len=8)
    assert synth.layer_input(w2).dtype == torch.bfloat16
