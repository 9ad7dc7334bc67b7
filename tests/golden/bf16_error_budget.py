"""Write tests/golden/bf16_error_budget.json: the error that the bf16 kernels'
storage roundings cause, predicted by tests/bf16_model.py against the float64
oracle on the exact inputs of the GPU parity cases that the workload
definitions give no tolerance for, plus the single layers they build on.

    python -m tests.golden.bf16_error_budget [--only NAME ...]

Calls only the oracle, the rounding model and the seeded input generators;
nothing here touches the GPU path.  Errors are those of tests/parity.py
(divided by the RMS of the oracle output).  The tolerances derived from these
predictions are in tests/parity.py.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from decoder_block_amd import synth  # noqa: E402
from tests import bf16_model as M  # noqa: E402

OUT = os.path.join(ROOT, "tests", "golden", "bf16_error_budget.json")
W = synth.WORKLOADS


def errors(got, ref) -> dict:
    d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    rms = float(np.sqrt(np.mean(np.asarray(ref, np.float64) ** 2)))
    return {"max_rel": float(d.max()) / rms, "mean_rel": float(d.mean()) / rms}


def _weights(w, gamma_std=None, layer=0):
    ws = synth.layer_weights(w, gamma_std, layer=layer)
    return {k: synth.as_f64(v) for k, v in ws.items()}


REALISATIONS = 16  # perturbed draws of the model per case (tests/bf16_model.py set_realisation)


def over_realisations(compute):
    """Errors of the plain model and of REALISATIONS perturbed draws: `compute()`
    returns {case: (model output, oracle output)}; the result per case holds the
    largest max and mean over the draws and the plain model's own errors."""
    out = {}
    for r in range(REALISATIONS + 1):
        M.set_realisation(None if r == 0 else 1000 + r)
        try:
            pairs = compute()
        finally:
            M.set_realisation(None)
        for case, (got, ref) in pairs.items():
            e = errors(got, ref)
            ent = out.setdefault(case, {"max_rel": 0.0, "mean_rel": 0.0, "draws": []})
            ent["max_rel"] = max(ent["max_rel"], e["max_rel"])
            ent["mean_rel"] = max(ent["mean_rel"], e["mean_rel"])
            ent["draws"].append([e["max_rel"], e["mean_rel"]])
            if r == 0:
                ent["plain"] = e
    return out


def stack3(_):
    """The bf16 stack case: LLaMA-3-8B shape, B 2, S 300, 3 layers, prefill + 2 decode steps."""
    w = synth.scaled(W[3], batch=2, seq_len=300)
    cfg = w.config_dict()
    NL = 3
    wo = [_weights(w, None, l) for l in range(NL)]
    gf = synth.as_f64(synth.final_norm_weight(w))
    x = synth.as_f64(synth.layer_input(w))
    ref, k_ref, v_ref = oracle.stack_prefill(cfg, wo, gf, x, "bf16")
    o1, _, _ = oracle.prefill(cfg, wo[0], x)
    steps = []
    c_ref = [[(k_ref[l, b], v_ref[l, b]) for b in range(w.batch)] for l in range(NL)]
    for step in range(2):
        xt = synth.as_f64(synth.decode_input(w, step))
        r, c_ref = oracle.stack_decode_step(cfg, wo, gf, xt, c_ref, "bf16")
        steps.append((xt, r))

    def compute():
        got, k_m, v_m = M.stack_prefill(cfg, wo, gf, x)
        m1, _, _ = M.prefill(cfg, wo[0], x)
        res = {"prefill": (got, ref), "last_layer_k": (k_m[NL - 1, 1], k_ref[NL - 1, 1]),
               "last_layer_v": (v_m[NL - 1, 1], v_ref[NL - 1, 1]), "single_layer_prefill": (m1, o1)}
        c_m = [[(k_m[l, b], v_m[l, b]) for b in range(w.batch)] for l in range(NL)]
        for step, (xt, r) in enumerate(steps):
            g, c_m = M.stack_decode_step(cfg, wo, gf, xt, c_m, out_bf16=True)
            res[f"decode_step{step}"] = (g, r)
        return res

    res = over_realisations(compute)
    res["case"] = "llama3-8b shape, B 2, S 300, 3 layers (prefill f32 out, 2 decode steps bf16 out)"
    return res


def gamma_rows(args):
    """gamma ~ 1 + N(0, 0.1^2), LLaMA-3-8B shape, B 1, by sequence length (row
    samples past S 300); the 300-token case (a GPU test) over realisations."""
    out = {}
    for S in args.gamma_lengths:
        w = synth.scaled(W[3], batch=1, seq_len=S)
        cfg = w.config_dict()
        x = synth.as_f64(synth.layer_input(w))
        rows = None if S <= 300 else synth.sample_rows(w, S, n_random=448, edge=64)
        ent = {"rows": "all" if rows is None else f"{len(rows)} sampled (first/last 64 + 448 seeded)"}
        for tag, gstd in (("gamma", 0.1), ("gamma_one", None)):
            wo = _weights(w, gstd)
            ref, _, _ = oracle.prefill(cfg, wo, x, rows=rows)
            if S == 300 and tag == "gamma":
                ent[tag] = over_realisations(lambda: {"e": (M.prefill(cfg, wo, x, rows=rows)[0], ref)})["e"]
            else:
                got, _, _ = M.prefill(cfg, wo, x, rows=rows)
                ent[tag] = errors(got, ref)
        out[str(S)] = ent
        print("gamma", S, ent, flush=True)
    return out


def short_prompts(_):
    """gamma = 1 prompts shorter than the workloads': LLaMA-3-8B shape, B 3, S 77 and B 1, S 16."""
    out = {}
    for B, S in ((3, 77), (1, 16)):
        w = synth.scaled(W[3], batch=B, seq_len=S)
        cfg = w.config_dict()
        wo = _weights(w)
        x = synth.as_f64(synth.layer_input(w))
        ref, _, _ = oracle.prefill(cfg, wo, x)
        out[f"B{B}_S{S}"] = over_realisations(lambda: {"e": (M.prefill(cfg, wo, x)[0], ref)})["e"]
        print("short", B, S, out[f"B{B}_S{S}"], flush=True)
    return out


def score_ranges(_):
    """Attention scores far from 0 (tests/score_cases.py): the 8B shape, B 1, S 300."""
    from tests import score_cases as SC
    out = {}
    for name in SC.CASES:
        w, ws, x = SC.score_case(name)
        cfg = w.config_dict()
        wo = {k: synth.as_f64(v) for k, v in ws.items()}
        xx = synth.as_f64(x)
        ref, _, _ = oracle.prefill(cfg, wo, xx)
        out[name] = over_realisations(lambda: {"e": (M.prefill(cfg, wo, xx)[0], ref)})["e"]
        print("scores", name, out[name]["max_rel"], out[name]["mean_rel"], flush=True)
    return out


PARTS = {"stack3": stack3, "gamma_by_length": gamma_rows, "short_prompts": short_prompts,
         "score_ranges": score_ranges}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--only", nargs="*", choices=sorted(PARTS))
    ap.add_argument("--gamma-lengths", nargs="*", type=int, default=[300, 500, 700, 1000, 2048, 4096, 8192])
    args = ap.parse_args()
    data = json.load(open(OUT)) if os.path.exists(OUT) else {}
    data["about"] = ("errors of tests/bf16_model.py (bf16 storage roundings of the bf16 kernels) against the "
                     "float64 oracle on the GPU parity cases' inputs; max/mean |diff| / RMS(oracle)")
    for name in args.only or sorted(PARTS):
        t0 = time.time()
        data[name] = PARTS[name](args)
        print(name, f"{time.time() - t0:.0f} s", json.dumps(data[name]), flush=True)
        with open(OUT, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main()
