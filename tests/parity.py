"""Shared helpers of the GPU parity tests and the smoke check: run the C-ABI
library on seeded workloads and compare with the float64 oracle."""
from __future__ import annotations

import functools
import json
import os

import numpy as np
import torch

import oracle
from decoder_block_amd import synth

# Tolerances, errors divided by the RMS of the oracle output ("unit-scale"):
#   fp32 layer: max |gpu - oracle| / RMS <= 1e-4
#   bf16 layer: max <= 3e-2 and mean <= 3e-3
TOL = {"f32": {"max_rel": 1e-4}, "bf16": {"max_rel": 3e-2, "mean_rel": 3e-3}}

# Cases the workload definitions give no tolerance for (a stack of layers,
# gamma != 1, prompts shorter than the workloads') are held to the error that
# the bf16 kernels' storage roundings cause on that case's own inputs, as
# predicted by tests/bf16_model.py (the oracle with a bf16 rounding at each
# point where the kernels store bf16, float64 everywhere else) and recorded in
# tests/golden/bf16_error_budget.json by tests/golden/bf16_error_budget.py,
# times a margin for what the model leaves out: the hardware exp2 and
# reciprocal, the fp32 RoPE table.  Which values round up or down at a bf16
# boundary depends on the kernels' fp32 accumulation order and, for the
# attention weights P, on the running maximum they are rounded at, so the
# budget holds the largest errors over the plain model and sixteen draws of
# it (each accumulated value shifted by a relative 2^-18 or less before its
# rounding, P rounded at a random scale per 64-key tile); the max error moves
# in discrete jumps when one rounding of a stored value flips, which is why a
# single draw does not bound it.  The margins are 10% on the mean and 30% on
# the max (the max is one extreme element, the mean averages millions).
BUDGET_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "bf16_error_budget.json")
MODEL_MARGIN = {"mean_rel": 1.10, "max_rel": 1.30}


@functools.lru_cache(maxsize=None)
def _budget() -> dict:
    with open(BUDGET_FILE) as f:
        return json.load(f)


def model_tol(path: str) -> str:
    """Tolerance key for the case at `path` ("part/case/.../errors") of the error
    budget: the model's max and mean errors times MODEL_MARGIN."""
    key = "model:" + path
    if key not in TOL:
        e = _budget()
        for part in path.split("/"):
            e = e[part]
        TOL[key] = {k: e[k] * m for k, m in MODEL_MARGIN.items()}
    return key


def errors(gpu, ref) -> dict:
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    d = np.abs(g - r)
    rms = float(np.sqrt(np.mean(r * r)))
    return {"max_abs": float(d.max()), "mean_abs": float(d.mean()), "rms": rms,
            "max_rel": float(d.max()) / rms, "mean_rel": float(d.mean()) / rms,
            "finite": bool(np.isfinite(g).all())}


def assert_close(gpu, ref, dtype: str, what: str = "") -> dict:
    e = errors(gpu, ref)
    log = os.environ.get("PARITY_LOG")
    if log:  # one JSON line per comparison: the measured errors beside the bound
        with open(log, "a") as f:
            test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
            f.write(json.dumps({"test": test, "what": what, "tol": dtype, "bound": TOL[dtype], **e}) + "\n")
    assert e["finite"], f"{what}: non-finite GPU output"
    for k, lim in TOL[dtype].items():
        assert e[k] <= lim, f"{what}: {k}={e[k]:.3e} > {lim:.1e} ({e})"
    return e


@functools.lru_cache(maxsize=2)
def weights_for(w: synth.Workload, gamma_std: float | None = None):
    """(storage tensors on CPU, float64 arrays for the oracle) of a workload's weights."""
    ws = synth.layer_weights(w, gamma_std)
    return ws, {k: synth.as_f64(v) for k, v in ws.items()}


def make_layer(w: synth.Workload, ws: dict, max_position: int | None = None):
    from decoder_block_amd.llama_layer import DecoderLayer
    return DecoderLayer(w.config_dict(), ws, w.dtype, max_position or w.positions_needed(), device="cuda")


def make_cache(layer, w: synth.Workload, tokens_per_seq: int, seqs: int, block_order_seed: int | None = None,
               spare_blocks: int = 0):
    from decoder_block_amd.llama_layer import PagedKVCache
    nb = seqs * ((tokens_per_seq + 15) // 16) + spare_blocks
    order = None
    if block_order_seed is not None:
        order = np.random.Generator(np.random.PCG64(block_order_seed)).permutation(nb).tolist()
    return PagedKVCache(layer, nb, seqs, block_order=order)


def gpu_prefill(layer, cache, x: torch.Tensor, out_dtype="f32", sids=None):
    B = x.shape[0]
    if sids is None:
        sids = [cache.add_seq() for _ in range(B)]
    out = layer.prefill(cache, sids, x.cuda(), out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, sids


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()
