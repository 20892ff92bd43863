"""Shared helpers of the GPU parity tests: upload synthetic inputs, run the HIP
layer through the C ABI, and compare with the fp64 oracle under the parity
protocol:

1. routing  : sel_gpu == sel_oracle bit-exactly for every token whose top-k
              margin (oracle, fp64, biased scores) is >= 1e-3; tokens below
              it are counted and reported (either routing is correct);
2. dispatch : counts, offsets, gather, scatter of the GPU equal, bit for bit,
              the oracle's histogram and stable permutation of sel_gpu;
3. output   : max|out_gpu - out_ref| <= tol * max|out_ref| with out_ref the
              oracle's output under the GPU's own routing (tol = 2e-2 for bf16
              layers, 1e-5 for fp32);
4. gates    : max|gate_gpu - gate_ref| <= 2e-5 (fp32 softmax of fp32 logits).
"""

from __future__ import annotations

import warnings

import numpy as np
import torch

from oracle import moe_oracle as O
from synth import gen

TOL = {"bf16": 2e-2, "f32": 1e-5}
GATE_TOL = 2e-5


def _host(arr: np.ndarray) -> torch.Tensor:
    """A CPU tensor over `arr` (read-only cached inputs included: the tensor is
    only read, for the copy to the device)."""
    with warnings.catch_warnings():
        warnings.filterwarnings("ignore", message="The given NumPy array is not writable")
        return torch.from_numpy(arr)


def to_torch(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16" and arr.dtype == np.uint16:
        return _host(np.ascontiguousarray(arr).view(np.int16)).to(device).view(torch.bfloat16)
    return _host(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def device_weights(inputs: dict) -> dict:
    cfg = inputs["cfg"]
    return {"rms_gain": to_torch(inputs["gain"], cfg.dtype),
            "w_router": to_torch(inputs["w_router"], cfg.dtype),
            "b_router": to_torch(inputs["bias"], "f32"),
            "w_gate": to_torch(inputs["w_gate"], cfg.dtype),
            "w_up": to_torch(inputs["w_up"], cfg.dtype),
            "w_down": to_torch(inputs["w_down"], cfg.dtype)}


def make_layer(inputs: dict, max_tokens: int | None = None):
    from moe_ffn_amd import MoELayer
    cfg = inputs["cfg"]
    w = device_weights(inputs)
    layer = MoELayer(cfg.d, cfg.F, cfg.E, cfg.k, cfg.dtype, w, max_tokens or cfg.T,
                     rms_eps=cfg.eps)
    torch.cuda.synchronize()
    return layer


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def check_parity(inputs: dict, layer, sample: int | None = None, seed: int = 0,
                 label: str = "", vals: dict | None = None, fp8_act: bool = False) -> dict:
    """Run the layer on ``inputs`` and assert the parity protocol.

    sample: number of tokens whose output rows are compared (all when None);
    routing and dispatch are always compared in full.
    vals: the exact values the oracle runs on (default: those of ``inputs``;
    fp8 layers pass their dequantised expert weights).
    fp8_act: the oracle quantises the expert activations (O12).  Tokens whose
    quantisation scale the oracle reports undecided (scale_tie: the device's
    finite-precision value may round the row's largest element either way,
    re-deciding every code of the row) are held to validity only (a row rms
    error under 10%), counted and reported, like routing near-ties; every
    other row meets the output bar."""
    cfg = inputs["cfg"]
    if vals is None:
        vals = gen.values_f32(inputs)
    hidden = to_torch(inputs["hidden"], cfg.dtype)
    out, r = layer.forward(hidden, routing=True)
    torch.cuda.synchronize()
    sel = r["sel"].cpu().numpy()
    gate = r["gate"].cpu().numpy().astype(np.float64)
    T, k, E = cfg.T, cfg.k, cfg.E
    assert sel.shape == (T, k)
    assert sel.min() >= 0 and sel.max() < E

    if sample is None or sample >= T:
        tokens = None
    else:
        rng = np.random.default_rng(seed)
        tokens = np.unique(np.concatenate([[0, T - 1], rng.choice(T, size=sample, replace=False)]))
    ref = O.oracle_forward(vals, forced_sel=sel, tokens=tokens, fp8_act=fp8_act)
    # 1. routing against the oracle's own choice
    margin = ref["margin"]
    firm = margin >= O.MARGIN_TOL
    mism = np.any(sel != ref["sel_oracle"], axis=1)
    assert not np.any(mism & firm), (
        f"{label}: {int(np.sum(mism & firm))} tokens with margin >= 1e-3 route differently; "
        f"first {np.nonzero(mism & firm)[0][:5]}")
    # 2. dispatch arrays on the GPU's routing
    np.testing.assert_array_equal(r["counts"].cpu().numpy(), ref["counts"])
    np.testing.assert_array_equal(r["offsets"].cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(r["gather"].cpu().numpy(), ref["gather"])
    np.testing.assert_array_equal(r["scatter"].cpu().numpy(), ref["scatter"])
    # 4. gates
    gerr = float(np.max(np.abs(gate - ref["gate"])))
    assert gerr <= GATE_TOL, f"{label}: gate error {gerr}"
    # 3. output
    got = out_to_f64(out)
    if tokens is not None:
        got = got[tokens]
    want = ref["out"]
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    tie = ref["scale_tie"] if fp8_act else np.zeros(got.shape[0], bool)
    scale = float(np.max(np.abs(want)))
    d = got - want
    err = float(np.max(np.abs(d[~tie]))) if np.any(~tie) else 0.0
    assert err <= TOL[cfg.dtype] * scale, (
        f"{label}: max|err| {err:.3e} > {TOL[cfg.dtype]} * max|ref| {scale:.3e}")
    row_rms = np.sqrt(np.mean(d ** 2, axis=1)) / np.maximum(np.sqrt(np.mean(want ** 2, axis=1)), 1e-300)
    assert np.all(row_rms[tie] <= 0.1), f"{label}: a row with an undecided fp8 scale is off by {row_rms[tie].max():.3f}"
    strict_rms = (float(np.sqrt(np.mean(d[~tie] ** 2)) / max(np.sqrt(np.mean(want[~tie] ** 2)), 1e-300))
                  if np.any(~tie) else 0.0)
    stats = {"label": label, "T": T, "k": k, "near_ties": int(np.sum(~firm)),
             "near_tie_flips": int(np.sum(mism & ~firm)), "max_err_rel": err / max(scale, 1e-300),
             "rms_err_rel": strict_rms, "gate_err": gerr, "rows_compared": int(got.shape[0])}
    if fp8_act:
        stats["scale_ties"] = int(np.sum(tie))
        stats["scale_tie_max_row_rms"] = float(row_rms[tie].max()) if np.any(tie) else 0.0
        stats["max_row_rms_decided"] = float(row_rms[~tie].max()) if np.any(~tie) else 0.0
    print(f"[parity] {stats}", flush=True)
    return stats
