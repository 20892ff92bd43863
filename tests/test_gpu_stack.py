"""The FFN stack (moe_stack_*) on the GPU.

A stack h_{l+1} = h_l + FFN_l(h_l) over dense (one-expert), top-1 and top-2
layers must equal, bit for bit, the same layers run one by one through the
layer ABI with the bf16 residual add done in torch; it must follow the fp64
oracle's stack (O10, on the GPU's own routing of every layer) to the layer
tolerance; and its captured HIP graph must reproduce eager runs on every
replay, also after the input buffer's contents change.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import WORKLOADS, make_inputs
from synth.gen import values_f32
from synth.configs import LayerConfig
from tests._parity import TOL, make_layer, to_torch, out_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_ffn_amd import load_library
    load_library()


def _small_stack_inputs(T):
    """Six layers at d=256, F=512: dense, dense, MoE top-1 (x2), MoE top-2, dense."""
    moe = LayerConfig(80, "stack_moe_bf16_d256_E4_F512", T=T, d=256, E=4, F=512, k=1,
                      dtype="bf16", bias="normal", family="stack_moe_d256")
    dense = LayerConfig(81, "stack_dense_bf16_d256_F512", T=T, d=256, E=1, F=512, k=1,
                        dtype="bf16", bias="zero", family="stack_dense_d256")
    plan = [(dense, 1), (dense, 1), (moe, 1), (moe, 1), (moe, 2), (dense, 1)]
    return [make_inputs(replace(cfg, k=k), T=T, layer=l) for l, (cfg, k) in enumerate(plan)]


def _loop(layers, h):
    sels = []
    for L in layers:
        y, r = L.forward(h, routing=True)
        sels.append(r["sel"].cpu().numpy())
        h = (h.float() + y.float()).to(torch.bfloat16)
    return h, sels


@pytest.mark.parametrize("T", [48, 300])
def test_small_stack_matches_layer_loop_and_oracle(T):
    from moe_ffn_amd import MoEStack
    inps = _small_stack_inputs(T)
    layers = [make_layer(inp, max_tokens=T) for inp in inps]
    stack = MoEStack(layers, max_tokens=T)
    h0 = to_torch(inps[0]["hidden"], "bf16")
    out = stack.forward(h0)
    ref_loop, sels = _loop(layers, h0)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_loop.view(torch.int16))
    vals = [values_f32(inp) for inp in inps]
    ref = O.stack_forward(vals, vals[0]["hidden"], [inp["cfg"].k for inp in inps],
                          inps[0]["cfg"].eps, forced_sels=sels)["out"]
    err = np.abs(out_to_f64(out) - ref).max()
    assert err <= TOL["bf16"] * np.abs(ref).max(), (err, np.abs(ref).max())
    stack.close()


def test_stack_graph_replays_match_eager():
    from moe_ffn_amd import MoEStack
    T = 300
    inps = _small_stack_inputs(T)
    layers = [make_layer(inp, max_tokens=T) for inp in inps]
    stack = MoEStack(layers, max_tokens=T)
    h_in = to_torch(inps[0]["hidden"], "bf16")
    h_alt = to_torch(make_inputs(inps[0]["cfg"], T=T, hidden_seed=5, layer=0)["hidden"], "bf16")
    want = [stack.forward(h_in).clone(), stack.forward(h_alt).clone()]
    side = torch.cuda.Stream()
    buf_in = h_in.clone()
    buf_out = torch.empty_like(h_in)
    torch.cuda.synchronize()
    stack.capture(buf_in, buf_out, side)
    for rep in range(4):
        src = h_in if rep % 2 == 0 else h_alt
        buf_in.copy_(src)
        torch.cuda.synchronize()
        buf_out.zero_()
        stack.replay(side)
        side.synchronize()
        assert torch.equal(buf_out.view(torch.int16), want[rep % 2].view(torch.int16)), rep
        # eager work between replays
        stack.forward(h_alt)
        torch.cuda.synchronize()
    stack.close()


def test_full_width_stack_matches_layer_loop():
    """d=2048, F=3072: dense, MoE top-1, MoE top-2 (16 experts), dense; T=32."""
    from moe_ffn_amd import MoEStack
    T = 32
    dense = LayerConfig(82, "stack_dense_bf16_d2048_F3072", T=T, d=2048, E=1, F=3072, k=1,
                        dtype="bf16", bias="zero", family="stack_dense_d2048")
    inps = [make_inputs(dense, T=T, layer=0), make_inputs(WORKLOADS[1], T=T),
            make_inputs(replace(WORKLOADS[1], k=2), T=T), make_inputs(dense, T=T, layer=1)]
    layers = [make_layer(inp, max_tokens=T) for inp in inps]
    stack = MoEStack(layers, max_tokens=T)
    h0 = to_torch(inps[1]["hidden"], "bf16")
    out = stack.forward(h0)
    ref_loop, _ = _loop(layers, h0)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_loop.view(torch.int16))
    stack.close()


# ------------------------------- depth averaging of the router logits (O11)
def test_eda_at_rate_zero_equals_the_plain_stack():
    from moe_ffn_amd import MoEStack
    for T in (48, 300):
        inps = _small_stack_inputs(T)
        layers = [make_layer(inp, max_tokens=T) for inp in inps]
        stack = MoEStack(layers, max_tokens=T)
        h0 = to_torch(inps[0]["hidden"], "bf16")
        plain = stack.forward(h0).clone()
        stack.set_eda(0.0)
        eda0 = stack.forward(h0).clone()
        stack.set_eda(None)
        again = stack.forward(h0)
        torch.cuda.synchronize()
        assert torch.equal(eda0.view(torch.int16), plain.view(torch.int16)), T
        assert torch.equal(again.view(torch.int16), plain.view(torch.int16)), T
        stack.close()


@pytest.mark.parametrize("T,alpha", [(48, 0.5), (128, 0.5), (200, 0.5)])
def test_eda_stack_matches_oracle(T, alpha):
    """T = 48 routes the top-1 layers with the per-token router and the top-2
    layer with the MFMA router; 128 and 200 take the MFMA router throughout.
    The inputs are chosen so that no token of any MoE layer has a top-k margin
    below 1e-3 in the oracle, so the routing must agree everywhere."""
    from moe_ffn_amd import MoEStack
    inps = _small_stack_inputs(T)
    vals = [values_f32(inp) for inp in inps]
    ks = [inp["cfg"].k for inp in inps]
    ref = O.stack_forward(vals, vals[0]["hidden"], ks, inps[0]["cfg"].eps, eda_alpha=alpha)
    plain = O.stack_forward(vals, vals[0]["hidden"], ks, inps[0]["cfg"].eps)
    moe = [l for l, inp in enumerate(inps) if inp["cfg"].E > 1]
    assert min(float(np.min(ref["margin"][l])) for l in moe) >= O.MARGIN_TOL
    assert any(np.any(ref["sel"][l] != plain["sel"][l]) for l in moe)  # the averaging matters
    layers = [make_layer(inp, max_tokens=T) for inp in inps]
    stack = MoEStack(layers, max_tokens=T)
    stack.set_eda(alpha)
    h0 = to_torch(inps[0]["hidden"], "bf16")
    out = stack.forward(h0).clone()
    # a captured graph of the same pass replays to the same bytes
    side = torch.cuda.Stream()
    buf_out = torch.empty_like(h0)
    torch.cuda.synchronize()
    stack.capture(h0, buf_out, side)
    for _ in range(2):
        buf_out.zero_()
        torch.cuda.synchronize()
        stack.replay(side)
        side.synchronize()
        assert torch.equal(buf_out.view(torch.int16), out.view(torch.int16))
    err = np.abs(out_to_f64(out) - ref["out"]).max()
    assert err <= TOL["bf16"] * np.abs(ref["out"]).max(), (err, np.abs(ref["out"]).max())
    stack.close()


def test_eda_rejects_bad_rates_and_fp32_stacks():
    from moe_ffn_amd import MoEStack
    from moe_ffn_amd.layer import MoELayerError
    inps = _small_stack_inputs(48)
    layers = [make_layer(inp, max_tokens=48) for inp in inps[:3]]
    stack = MoEStack(layers, max_tokens=48)
    for bad in (1.0, -0.1, float("nan")):
        with pytest.raises(MoELayerError):
            stack.set_eda(bad)
    stack.close()
    f32 = make_inputs(WORKLOADS[0], T=16)
    s32 = MoEStack([make_layer(f32, max_tokens=16)], max_tokens=16)
    with pytest.raises(MoELayerError):
        s32.set_eda(0.5)
    s32.close()
