"""Parity of fp8 (E4M3) expert weights with the fp64 oracle.

The layer is built with moe_layer_create_fp8 from codes and per-row scales
(synth.gen.fp8_expert_weights); the oracle runs on the exact dequantised
weights value(code) * scale (oracle.fp8_weights), so the comparison measures
the kernels' arithmetic, not the quantisation.  Covers the decode streams
(k-step-pair fp8 loads) and the tile GEMMs (bf16 code values, scales in the
epilogue) at full size (every output row) and at ragged reduced sizes, top-1 and top-2.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import WORKLOADS, make_inputs
from synth.gen import fp8_expert_weights, values_f32
from tests._parity import check_parity, device_weights, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_ffn_amd import load_library
    load_library()


_deq = {}


def fp8_vals(inputs: dict) -> dict:
    """values_f32(inputs) with the expert weights replaced by the oracle's
    dequantisation of their fp8 codes (cached per weight set)."""
    key = id(inputs["w_gate"])
    if key not in _deq:
        q = fp8_expert_weights(inputs)
        _deq[key] = {name: O.fp8_weights(q[name], q[sname]) for name, sname in
                     (("w_gate", "s_gate"), ("w_up", "s_up"), ("w_down", "s_down"))}
    vals = values_f32(inputs)
    vals.update(_deq[key])
    return vals


def fp8_layer(inputs: dict, max_tokens: int):
    from moe_ffn_amd import MoELayer
    cfg = inputs["cfg"]
    q = fp8_expert_weights(inputs)
    w = device_weights(inputs)
    for name in ("w_gate", "w_up", "w_down"):
        w[name] = torch.from_numpy(q[name]).cuda()
    scales = {s: torch.from_numpy(q["s_" + s]).cuda() for s in ("gate", "up", "down")}
    layer = MoELayer(cfg.d, cfg.F, cfg.E, cfg.k, cfg.dtype, w, max_tokens, rms_eps=cfg.eps,
                     fp8_scales=scales)
    torch.cuda.synchronize()
    return layer


_layers = {}


def family_fp8_layer(cid: int, k: int):
    key = (WORKLOADS[cid].family, k, WORKLOADS[cid].bias)
    if key not in _layers:
        _layers[key] = fp8_layer(make_inputs(replace(WORKLOADS[cid], k=k)), max_tokens=16384)
    return _layers[key]


@pytest.mark.parametrize("cid,T,k,sample", [
    (1, None, 1, None),   # decode T = 32: fp8 streams, full rows
    (1, 7, 1, None),      # decode, ragged
    (3, 32, 2, None),     # decode + combine (64 assignments)
    (2, None, 1, None),   # prefill T = 4096: tile GEMMs, every row
    (2, 300, 1, None),    # tile GEMMs, ragged tails
    (3, 200, 2, None),    # tile GEMMs + combine
    (3, None, 2, None),   # top-2 T = 4096, every row
])
def test_fp8_parity(cid, T, k, sample):
    base = replace(WORKLOADS[cid], k=k)
    inp = make_inputs(base, T=T) if T is not None else make_inputs(base)
    st = check_parity(inp, family_fp8_layer(cid, k), sample=sample, vals=fp8_vals(inp),
                      label=f"fp8 c{cid} T={inp['cfg'].T} k={k}")
    assert st["rms_err_rel"] < 5e-3
    assert st["rows_compared"] == inp["cfg"].T


def test_fp8_matches_bf16_layer_on_code_values():
    """With unit scales the fp8 layer computes with the code values
    themselves; a bf16 layer given those values (exact in bf16) runs the same
    products.  The tile GEMMs (T = 300) also run them in the same order and
    match bit for bit; the decode streams split the reduction axis over four
    waves for fp8 and eight for bf16, so only the fp32 summation order differs
    there."""
    from moe_ffn_amd import MoELayer
    inp = make_inputs(WORKLOADS[1])
    cfg = inp["cfg"]
    q = fp8_expert_weights(inp)
    w8 = device_weights(inp)
    w16 = device_weights(inp)
    for name in ("w_gate", "w_up", "w_down"):
        codes = torch.from_numpy(q[name]).cuda()
        w8[name] = codes
        w16[name] = codes.view(torch.float8_e4m3fn).to(torch.bfloat16)  # exact
    ones = {"gate": torch.ones(cfg.E, cfg.F, device="cuda"),
            "up": torch.ones(cfg.E, cfg.F, device="cuda"),
            "down": torch.ones(cfg.E, cfg.d, device="cuda")}
    l8 = MoELayer(cfg.d, cfg.F, cfg.E, cfg.k, "bf16", w8, 512, rms_eps=cfg.eps, fp8_scales=ones)
    l16 = MoELayer(cfg.d, cfg.F, cfg.E, cfg.k, "bf16", w16, 512, rms_eps=cfg.eps)
    for T in (32, 300):
        h = to_torch(make_inputs(WORKLOADS[1], T=T)["hidden"], "bf16")
        o8, r8 = l8.forward(h, routing=True)
        o16, r16 = l16.forward(h, routing=True)
        torch.cuda.synchronize()
        assert torch.equal(r8["sel"], r16["sel"])
        assert torch.isfinite(o8.float()).all()
        if T > 64:
            assert torch.equal(o8, o16), f"T={T}"
        else:
            a, b = o8.float(), o16.float()
            assert (a - b).abs().max().item() <= 1e-2 * b.abs().max().item(), f"T={T}"
    l8.close()
    l16.close()


def test_fp8_create_rejects_f32_and_small_dff():
    from moe_ffn_amd import MoELayer, MoELayerError
    inp = make_inputs(WORKLOADS[1])
    cfg = inp["cfg"]
    q = fp8_expert_weights(inp)
    w = device_weights(inp)
    for name in ("w_gate", "w_up", "w_down"):
        w[name] = torch.from_numpy(q[name]).cuda()
    scales = {s: torch.from_numpy(q["s_" + s]).cuda() for s in ("gate", "up", "down")}
    with pytest.raises(MoELayerError):
        # d_ff = 3072 is fine; a d_ff of 128 (bf16-legal) is not for fp8
        small = {k2: (v[:, :128].contiguous() if k2 in ("w_gate", "w_up") else
                      v[..., :128].contiguous() if k2 == "w_down" else v) for k2, v in w.items()}
        sm = {"gate": scales["gate"][:, :128].contiguous(),
              "up": scales["up"][:, :128].contiguous(), "down": scales["down"]}
        MoELayer(cfg.d, 128, cfg.E, cfg.k, "bf16", small, 64, fp8_scales=sm)


@pytest.mark.parametrize("T", [32, 96])
def test_fp8_moe_layers_in_a_stack(T):
    """A stack of bf16 dense layers and fp8 MoE layers (decode streams at T=32,
    tile GEMMs at T=96) equals the layer-by-layer loop bit for bit and the
    oracle's stack on the dequantised weights to the layer tolerance."""
    from moe_ffn_amd import MoEStack
    from tests._parity import TOL, make_layer, out_to_f64
    from tests.test_gpu_stack import _loop, _small_stack_inputs
    inps = _small_stack_inputs(T)
    layers, vals = [], []
    for inp in inps:
        if inp["cfg"].E > 1:
            layers.append(fp8_layer(inp, max_tokens=T))
            vals.append(fp8_vals(inp))
        else:
            layers.append(make_layer(inp, max_tokens=T))
            vals.append(values_f32(inp))
    stack = MoEStack(layers, max_tokens=T)
    h0 = to_torch(inps[0]["hidden"], "bf16")
    out = stack.forward(h0)
    ref_loop, sels = _loop(layers, h0)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_loop.view(torch.int16))
    ref = O.stack_forward(vals, vals[0]["hidden"], [inp["cfg"].k for inp in inps],
                          inps[0]["cfg"].eps, forced_sels=sels)["out"]
    err = np.abs(out_to_f64(out) - ref).max()
    assert err <= TOL["bf16"] * np.abs(ref).max(), (err, np.abs(ref).max())
    stack.close()
    for L in layers:
        L.close()
