"""Inputs whose attention scores sit far from 0, for the prefill attention
kernel's lazy running max (it starts at 0, rises only when a score exceeds it
by more than 32 in exp2 units, and on the first tile also drops to a row max
below -64).  TEST INFRASTRUCTURE: deterministic changes to the seeded draws of
decoder_block_amd/synth.py, no layer arithmetic.  Used by the GPU parity test
and by tests/golden/bf16_error_budget.py.

Cases on the LLaMA-3-8B layer shape, B 1, S 300:
  qk_x2     q and k weights x2 (scores x4, std about 9 in exp2 units): most
            rows start below 32 and some exceed it on a later tile;
  qk_x4     q and k weights x4 (scores x16): rows exceed 32 on their first tile;
  all_high  every score about +100: q and k read only the row's first 64
            features (all set to 1) into the lowest-frequency RoPE pair of
            every head, which barely rotates over 300 positions;
  all_low   the same with k = -q: every score about -100.
  lane_split  the keys at positions 4-7 mod 8 (in the prefill attention
            kernel's score layout, the keys that lanes 32-63 of a wave hold)
            score 139-156 against the queries at positions 4-7 mod 8, and
            every other score is 0: the first 64 features are 1 at those
            positions and 0 elsewhere, and q and k read them with weights
            17/32 into the lowest-frequency RoPE pair of every head.  A row
            maximum that missed one lane half would leave P = 2^139 or more,
            past fp32.
The bf16 scalings by 2 and 4 and the values 7/16 and 17/32 are exact in bf16.
"""
from __future__ import annotations

import torch

from decoder_block_amd import synth

CASES = ("qk_x2", "qk_x4", "all_high", "all_low", "lane_split")


def workload() -> synth.Workload:
    return synth.scaled(synth.WORKLOADS[3], batch=1, seq_len=300)


def score_case(name: str):
    """(workload, weights in storage dtype, x [1, 300, d]) of case `name`."""
    w = workload()
    ws = dict(synth.layer_weights(w))
    x = synth.layer_input(w).clone()
    if name in ("qk_x2", "qk_x4"):
        f = 2.0 if name == "qk_x2" else 4.0
        ws["q_proj"] = ws["q_proj"] * f
        ws["k_proj"] = ws["k_proj"] * f
    elif name in ("all_high", "all_low"):
        D = w.hidden_size // w.num_attention_heads
        x[..., :64] = 1.0
        # score = (64 * 7/16 * r1)^2 * log2(e) / sqrt(D) = 784 * 0.1275 = 100 at r1 = 1
        q = torch.zeros_like(ws["q_proj"])
        k = torch.zeros_like(ws["k_proj"])
        for h in range(w.num_attention_heads):
            q[h * D + D - 2, :64] = 0.4375
        sign = 1.0 if name == "all_high" else -1.0
        for g in range(w.num_key_value_heads):
            k[g * D + D - 2, :64] = 0.4375 * sign
        ws["q_proj"], ws["k_proj"] = q, k
    elif name == "lane_split":
        D = w.hidden_size // w.num_attention_heads
        sel = torch.arange(x.shape[1]) % 8 >= 4
        x[:, sel, :64] = 1.0
        x[:, ~sel, :64] = 0.0
        # score = (64 * 17/32)^2 * log2(e) / sqrt(D) = 1156 * 0.1275 = 147 between selected positions
        q = torch.zeros_like(ws["q_proj"])
        k = torch.zeros_like(ws["k_proj"])
        for h in range(w.num_attention_heads):
            q[h * D + D - 2, :64] = 0.53125
        for g in range(w.num_key_value_heads):
            k[g * D + D - 2, :64] = 0.53125
        ws["q_proj"], ws["k_proj"] = q, k
    else:
        raise ValueError(name)
    return w, ws, x
