"""moe_layer_forward_static, the forward that allocates nothing (its per-call
buffers live in the library's static scratch array), against
moe_layer_forward on the same layer and inputs: routing and output bytes
must be identical.  Two calls in a row, the second with fewer tokens, so the
second call's zero row lies where the first call left other data; a second
layer then uses the same array; a T whose buffers exceed the array is
rejected."""

from dataclasses import replace

import numpy as np
import pytest
import torch

from synth import WORKLOADS, make_inputs
from tests._parity import check_parity, make_layer, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_ffn_amd import load_library
    load_library()


def _same(layer, h):
    want, rw = layer.forward(h, routing=True)
    out = torch.full_like(h, float("nan"))
    rs, _ = layer.routing_buffers(h.shape[0], h.device)
    for v in rs.values():
        v.fill_(-7)
    got, rg = layer.forward(h, out=out, routing=True, static_scratch=True)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    for key in rw:
        assert torch.equal(rg[key], rw[key]), key
    return got


@pytest.mark.parametrize("k,T1,T2", [(1, 300, 32), (2, 200, 20), (1, 815, 64)])
def test_static_forward_equals_the_workspace_forward(k, T1, T2):
    base = replace(WORKLOADS[1], k=k)
    layer = make_layer(make_inputs(base, T=T1), max_tokens=1024)
    for T in (T1, T2):   # tile path, then (for T2) the decode path, smaller
        inp = make_inputs(base, T=T)
        h = to_torch(inp["hidden"], "bf16")
        _same(layer, h)
    # the oracle's bar as well, on the last call's inputs
    check_parity(inp, layer, label=f"static k={k} T={T2}")
    layer.close()


def test_two_layers_share_the_array():
    a = make_layer(make_inputs(WORKLOADS[1], T=64), max_tokens=512)
    inp2 = make_inputs(replace(WORKLOADS[0], T=40))    # fp32 layer, other shapes
    b = make_layer(inp2, max_tokens=64)
    ha = to_torch(make_inputs(WORKLOADS[1], T=500)["hidden"], "bf16")
    hb = to_torch(inp2["hidden"], "f32")
    for _ in range(2):
        _same(a, ha)
        _same(b, hb)
    a.close()
    b.close()


def test_too_many_tokens_for_the_array_is_rejected():
    from moe_ffn_amd import MoELayerError, MOE_ERR_INVALID_ARG
    layer = make_layer(make_inputs(WORKLOADS[1], T=32), max_tokens=2048)
    h = to_torch(make_inputs(WORKLOADS[1], T=816)["hidden"], "bf16")
    with pytest.raises(MoELayerError) as ei:
        layer.forward(h, static_scratch=True)
    assert ei.value.status == MOE_ERR_INVALID_ARG and "static scratch" in str(ei.value)
    layer.forward(h)   # the workspace forward takes it
    torch.cuda.synchronize()
    layer.close()
