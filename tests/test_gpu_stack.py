"""The FFN stack (moe_stack_*) on the GPU.

A stack h_{l+1} = h_l + FFN_l(h_l) over dense (one-expert), top-1 and top-2
layers must equal, bit for bit, the same layers run one by one through the
layer ABI with the bf16 residual add done in torch; it must follow the fp64
oracle's stack (O10, on the GPU's own routing of every layer) to the layer
tolerance, at d_model = 256 and at the full width d_model = 2048; and its
captured HIP graph must reproduce eager runs on every replay, also after the
input buffer's contents change.  With the router logits depth-averaged (O11)
every MoE layer's routing is compared with the oracle's, layer by layer.
fp32 stacks (a separate residual launch after each layer) equal their layer
loop with the fp32 add in torch.
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


def _small_stack_inputs(T, E=4):
    """Six layers at d=256, F=512: dense, dense, MoE top-1 (x2), MoE top-2, dense."""
    moe = LayerConfig(80, f"stack_moe_bf16_d256_E{E}_F512", T=T, d=256, E=E, F=512, k=1,
                      dtype="bf16", bias="normal", family=f"stack_moe_d256_E{E}")
    dense = LayerConfig(81, "stack_dense_bf16_d256_F512", T=T, d=256, E=1, F=512, k=1,
                        dtype="bf16", bias="zero", family="stack_dense_d256")
    plan = [(dense, 1), (dense, 1), (moe, 1), (moe, 1), (moe, 2), (dense, 1)]
    return [make_inputs(replace(cfg, k=k), T=T, layer=l) for l, (cfg, k) in enumerate(plan)]


def _loop(layers, h, inputs=None):
    """The stack as a loop of layer forwards with the bf16 residual add in
    torch; `inputs`, if a list, receives every layer's input (as float64)."""
    sels = []
    for L in layers:
        if inputs is not None:
            inputs.append(out_to_f64(h))
        y, r = L.forward(h, routing=True)
        sels.append(r["sel"].cpu().numpy())
        h = (h.float() + y.float()).to(torch.bfloat16)
    return h, sels


def _check_layer_routing(vals, h_in, sels, ks, eps, alpha=None, label=""):
    """Each layer's routing against the oracle's router (O1-O3, with O11's
    depth averaging when alpha is given) run on the input that layer really
    received on the GPU (the bf16 residual stream): bit-exact for every token
    whose top-k margin is at least 1e-3.  The fp64 stack of O10 carries an
    unrounded residual, so its own later-layer choices are not comparable
    token by token.  Returns (near-ties, flips) summed over the layers."""
    near = flips = 0
    zp = None
    none = np.zeros(0, np.int64)
    for l, v in enumerate(vals):
        moe = np.asarray(v["w_router"]).shape[0] > 1
        if alpha is not None and moe:
            r = O.oracle_forward(dict(v, hidden=h_in[l]), k=ks[l], eps=eps, tokens=none,
                                 z_prev=zp, eda_alpha=alpha)
            zp = r["z"]
        else:
            r = O.oracle_forward(dict(v, hidden=h_in[l]), k=ks[l], eps=eps, tokens=none)
        firm = r["margin"] >= O.MARGIN_TOL
        same = (sels[l] == r["sel_oracle"]).all(axis=1)
        assert np.all(same | ~firm), (label, l, np.nonzero(~same & firm)[0][:5])
        near += int(np.sum(~firm))
        flips += int(np.sum(~same & ~firm))
    return near, flips


@pytest.mark.parametrize("T", [48, 300])
def test_small_stack_matches_layer_loop_and_oracle(T):
    from moe_ffn_amd import MoEStack
    inps = _small_stack_inputs(T)
    layers = [make_layer(inp, max_tokens=T) for inp in inps]
    stack = MoEStack(layers, max_tokens=T)
    h0 = to_torch(inps[0]["hidden"], "bf16")
    out = stack.forward(h0)
    h_in = []
    ref_loop, sels = _loop(layers, h0, h_in)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_loop.view(torch.int16))
    vals = [values_f32(inp) for inp in inps]
    ks = [inp["cfg"].k for inp in inps]
    _check_layer_routing(vals, h_in, sels, ks, inps[0]["cfg"].eps, label=f"d256 T={T}")
    ref = O.stack_forward(vals, vals[0]["hidden"], ks, inps[0]["cfg"].eps, forced_sels=sels)["out"]
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


def _full_width_inputs(T):
    """d=2048, F=3072: dense, MoE top-1, MoE top-2 (16 experts), dense."""
    dense = LayerConfig(82, "stack_dense_bf16_d2048_F3072", T=T, d=2048, E=1, F=3072, k=1,
                        dtype="bf16", bias="zero", family="stack_dense_d2048")
    return [make_inputs(dense, T=T, layer=0), make_inputs(WORKLOADS[1], T=T),
            make_inputs(replace(WORKLOADS[1], k=2), T=T), make_inputs(dense, T=T, layer=1)]


@pytest.mark.parametrize("T", [32, 200])
def test_full_width_stack_matches_layer_loop_and_oracle(T):
    """Four layers at the backbone's width; T = 32 runs the decode path of
    every layer, T = 200 the tiled one."""
    from moe_ffn_amd import MoEStack
    inps = _full_width_inputs(T)
    layers = [make_layer(inp, max_tokens=T) for inp in inps]
    stack = MoEStack(layers, max_tokens=T)
    h0 = to_torch(inps[1]["hidden"], "bf16")
    out = stack.forward(h0)
    h_in = []
    ref_loop, sels = _loop(layers, h0, h_in)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_loop.view(torch.int16))
    vals = [values_f32(inp) for inp in inps]
    ks = [inp["cfg"].k for inp in inps]
    _check_layer_routing(vals, h_in, sels, ks, inps[0]["cfg"].eps, label=f"d2048 T={T}")
    ref = O.stack_forward(vals, vals[1]["hidden"], ks, inps[0]["cfg"].eps, forced_sels=sels)
    err = np.abs(out_to_f64(out) - ref["out"]).max()
    assert err <= TOL["bf16"] * np.abs(ref["out"]).max(), (err, np.abs(ref["out"]).max())
    stack.close()
    for L in layers:
        L.close()


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


def _eda_parity(inps, T, alpha, label):
    """One depth-averaged pass with every layer's routing: each MoE layer's
    choice equals the oracle's (O1-O3 with O11 on the layer inputs the GPU
    computed) for every token whose top-k margin is at least 1e-3, the
    dispatch arrays equal O5-O6 of the GPU's choice, and the output follows
    the oracle's stack (O10 with O11 on the GPU's routing) to the layer
    tolerance.  Returns (near-ties, flips) over the layers."""
    from moe_ffn_amd import MoEStack
    vals = [values_f32(inp) for inp in inps]
    ks = [inp["cfg"].k for inp in inps]
    layers = [make_layer(inp, max_tokens=T) for inp in inps]
    stack = MoEStack(layers, max_tokens=T)
    stack.set_eda(alpha)
    h0 = to_torch(inps[0]["hidden"], "bf16")
    out, routs = stack.forward_routing(h0)
    torch.cuda.synchronize()
    sels = [r["sel"].cpu().numpy() for r in routs]
    # every layer's input on the GPU: the output of the stack of the layers
    # before it, depth averaging on (the same launches as the full pass)
    h_in = [out_to_f64(h0)]
    for l in range(1, len(layers)):
        pre = MoEStack(layers[:l], max_tokens=T)
        if any(L.E > 1 for L in layers[:l]):
            pre.set_eda(alpha)
        h_in.append(out_to_f64(pre.forward(h0)))
        pre.close()
    torch.cuda.synchronize()
    near, flips = _check_layer_routing(vals, h_in, sels, ks, inps[0]["cfg"].eps, alpha, label)
    ref = O.stack_forward(vals, vals[0]["hidden"], ks, inps[0]["cfg"].eps, forced_sels=sels,
                          eda_alpha=alpha)
    for l, inp in enumerate(inps):
        c, o = O.histogram(sels[l], inp["cfg"].E)
        g, sc = O.permutation(sels[l])
        np.testing.assert_array_equal(routs[l]["counts"].cpu().numpy(), c)
        np.testing.assert_array_equal(routs[l]["offsets"].cpu().numpy(), o)
        np.testing.assert_array_equal(routs[l]["gather"].cpu().numpy(), g)
        np.testing.assert_array_equal(routs[l]["scatter"].cpu().numpy(), sc)
    err = np.abs(out_to_f64(out) - ref["out"]).max()
    assert err <= TOL["bf16"] * np.abs(ref["out"]).max(), (label, err, np.abs(ref["out"]).max())
    # the plain pass of the same stack matches the routing-less forward
    again = stack.forward(h0)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), out.view(torch.int16))
    print(f"[eda] {label}: near-ties {near}, flips {flips}", flush=True)
    stack.close()
    for L in layers:
        L.close()
    return near, flips


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
    near, _ = _eda_parity(inps, T, alpha, f"d256 E4 T={T}")
    assert near == 0
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


@pytest.mark.parametrize("E,T", [(32, 48), (32, 200), (64, 300)])
def test_eda_wide_routers_match_oracle(E, T):
    """More than 16 experts: the MFMA router's generic branch (and the
    per-token router at T = 48 for the top-1 layers)."""
    _eda_parity(_small_stack_inputs(T, E=E), T, 0.5, f"d256 E{E} T={T}")


@pytest.mark.parametrize("T", [32, 200])
def test_eda_full_width_matches_oracle(T):
    """d_model = 2048 with 16 experts: the decode routers at T = 32, the MFMA
    router at T = 200."""
    _eda_parity(_full_width_inputs(T), T, 0.5, f"d2048 E16 T={T}")


def test_eda_rejects_mixed_expert_counts():
    """Depth averaging passes expert e's logit to the next MoE layer, so a
    stack whose MoE layers differ in n_experts cannot turn it on (the oracle
    refuses the same stack)."""
    from moe_ffn_amd import MoEStack, MOE_ERR_INVALID_ARG
    from moe_ffn_amd.layer import MoELayerError
    T = 48
    a = _small_stack_inputs(T, E=4)
    b = _small_stack_inputs(T, E=8)
    inps = [a[0], a[2], b[3], a[5]]   # dense, MoE E=4, MoE E=8, dense
    layers = [make_layer(inp, max_tokens=T) for inp in inps]
    stack = MoEStack(layers, max_tokens=T)
    with pytest.raises(MoELayerError) as ei:
        stack.set_eda(0.5)
    assert ei.value.status == MOE_ERR_INVALID_ARG
    h0 = to_torch(inps[0]["hidden"], "bf16")
    stack.forward(h0)   # without averaging the stack runs
    torch.cuda.synchronize()
    vals = [values_f32(inp) for inp in inps]
    with pytest.raises(ValueError):
        O.stack_forward(vals, vals[0]["hidden"], [1, 1, 1, 1], 1e-6, eda_alpha=0.5)
    stack.close()
    for L in layers:
        L.close()


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


@pytest.mark.parametrize("T", [32, 200])
def test_stack_in_place(T):
    """hidden_out may be hidden_in: in a one-layer stack the layer's last
    kernel then reads each residual value and writes the sum in its place
    (k = 1: the down projection; k = 2: the combine), on the weight streams
    (T = 32) and on the tile path (T = 200); a longer stack ends in place."""
    from moe_ffn_amd import MoEStack
    inps = _small_stack_inputs(T)
    layers = [make_layer(inp, max_tokens=T) for inp in inps]
    h0 = to_torch(inps[0]["hidden"], "bf16")
    for label, sub in (("k=1 layer", [layers[2]]), ("k=2 layer", [layers[4]]), ("six layers", layers)):
        print(f"[case] in-place stack {label} T={T}", flush=True)
        stack = MoEStack(sub, max_tokens=T)
        want = stack.forward(h0)
        h = h0.clone()
        got = stack.forward(h, out=h)
        torch.cuda.synchronize()
        assert got.data_ptr() == h.data_ptr()
        assert torch.equal(h.view(torch.int16), want.view(torch.int16)), label
        stack.close()


@pytest.mark.parametrize("T", [16, 100])
def test_fp32_stack_matches_layer_loop(T):
    """fp32 layers keep a residual launch after each layer (bf16 layers add in
    their last kernel): the stack equals the loop with the fp32 add in torch."""
    from moe_ffn_amd import MoEStack
    base = WORKLOADS[0]
    plan = [replace(base, E=1, bias="zero"), base, replace(base, k=2)]
    inps = [make_inputs(cfg, T=T, layer=l) for l, cfg in enumerate(plan)]
    layers = [make_layer(inp, max_tokens=T) for inp in inps]
    stack = MoEStack(layers, max_tokens=T)
    h = to_torch(inps[0]["hidden"], "f32")
    print(f"[case] fp32 stack T={T}", flush=True)
    out = stack.forward(h)
    ref = h
    for L in layers:
        ref = ref + L.forward(ref)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    stack.close()


@pytest.mark.parametrize("T", [40, 300])
def test_w8a8_stack_matches_layer_loop_and_oracle(T):
    """A stack of layers with fp8 weights and fp8 activations (moe_layer_create_w8a8;
    T=40 streams the weights, T=300 runs the fp8 MFMA GEMMs): the stack equals
    the layer loop bit for bit, and every layer, on the input it received on
    the GPU and the GPU's routing, matches the oracle's fp8-activation step
    (O12) with undecided quantisation scales held to validity only."""
    from moe_ffn_amd import MoEStack
    from tests.test_gpu_fp8 import fp8_vals
    from tests.test_gpu_w8a8 import w8a8_layer
    inps = _small_stack_inputs(T)
    layers = [w8a8_layer(inp, T) for inp in inps]
    stack = MoEStack(layers, max_tokens=T)
    h = to_torch(inps[0]["hidden"], "bf16")
    out = stack.forward(h)
    ties = 0
    for l, (L, inp) in enumerate(zip(layers, inps)):
        h_in = out_to_f64(h)
        y, r = L.forward(h, routing=True)
        torch.cuda.synchronize()
        sel = r["sel"].cpu().numpy()
        vals = dict(fp8_vals(inp), hidden=h_in)
        ref = O.oracle_forward(vals, k=inp["cfg"].k, eps=inp["cfg"].eps, forced_sel=sel,
                               fp8_act=True)
        got = out_to_f64(y)
        tie = ref["scale_tie"]
        scale = np.abs(ref["out"]).max()
        err = np.abs(got - ref["out"])[~tie].max()
        assert err <= TOL["bf16"] * scale, (l, err, scale)
        row = np.sqrt(np.mean((got - ref["out"]) ** 2, axis=1) / np.mean(ref["out"] ** 2, axis=1))
        assert np.all(row[tie] <= 0.1), (l, row[tie].max())
        ties += int(tie.sum())
        h = (h.float() + y.float()).to(torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), h.view(torch.int16))
    print(f"[w8a8 stack] T={T}: {len(layers)} layers, undecided scales {ties}", flush=True)
    stack.close()
