"""The auxiliary-loss-free balancing step (moe_layer_update_bias) on the GPU.

Each updated bias is compared bit for bit with the oracle's O9 step applied to
the GPU's own counts of the same forward; the routing that follows is checked
under the parity protocol; and repeated steps on one batch flatten the expert
load, which is what the step is for.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import WORKLOADS, make_inputs
from tests._parity import check_parity, make_layer, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_ffn_amd import load_library
    load_library()


@pytest.mark.parametrize("cid,T", [(1, 32), (2, 2000), (3, 700)])
def test_update_matches_oracle_bit_for_bit(cid, T):
    inp = make_inputs(replace(WORKLOADS[cid], bias="normal"), T=T)
    layer = make_layer(inp, max_tokens=T)
    h = to_torch(inp["hidden"], "bf16")
    b = np.asarray(inp["bias"], np.float32)
    for rate, use_routing in [(0.01, True), (2.0 ** -7, False), (-0.003, True)]:
        if use_routing:
            _, r = layer.forward(h, routing=True)
            counts = r["counts"]
            layer.update_bias(rate, counts=counts)
        else:
            layer.forward(h)           # counts land in the layer's own buffer
            _, r = layer.forward(h, routing=True)   # same batch: same counts, for the oracle
            counts = r["counts"]
            layer.forward(h)           # refresh the layer's own buffer last
            layer.update_bias(rate)
        torch.cuda.synchronize()
        want = O.bias_update(b, counts.cpu().numpy(), rate)
        got = layer.get_bias().cpu().numpy()
        assert got.dtype == np.float32
        np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
        b = want
    # routing with the updated bias follows the oracle with that bias
    check_parity(dict(inp, bias=b), layer, sample=256 if T > 512 else None,
                 label=f"after bias steps c{cid} T={T}")


def test_repeated_steps_flatten_the_load():
    T = 4096
    inp = make_inputs(replace(WORKLOADS[2], bias="normal"), T=T)
    layer = make_layer(inp, max_tokens=T)
    h = to_torch(inp["hidden"], "bf16")
    _, r = layer.forward(h, routing=True)
    c0 = r["counts"].cpu().numpy()
    for _ in range(60):
        layer.forward(h)
        layer.update_bias(0.01)
    _, r = layer.forward(h, routing=True)
    c1 = r["counts"].cpu().numpy()
    assert c0.sum() == c1.sum() == T
    mean = T / 16
    # the step moves every bias toward balance, so the worst deviation shrinks
    assert np.abs(c1 - mean).max() < 0.5 * np.abs(c0 - mean).max()
