"""A forward captured into a HIP graph, and the layer at an expert-parallel
shard's shape.

Graph: the forward launches only kernels (no memset, copy or host sync), so it
can be captured.  Each replay must give, bit for bit, the eager forward's
output; replays are interleaved with eager forwards of the same layer on other
data (which reuse the same workspace) and with unrelated torch work, and every
replay is checked.

Shard shape: under expert parallelism over 8 GPUs each GPU holds 2 of the 16
experts and receives about T*k*2/16 rows; the same kernels run such a shard
as a 2-expert layer.  Checked against the oracle under the usual protocol.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

from synth import WORKLOADS, make_inputs
from synth.configs import LayerConfig
from tests._parity import check_parity, make_layer, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_ffn_amd import load_library
    load_library()  # fails loudly if the library is not built


@pytest.mark.parametrize("cid,T,k", [
    (1, 32, 1),     # decode path: router per token + streaming experts
    (2, 300, 1),    # tile path
    (3, 200, 2),    # tile path + combine
])
def test_graph_replay_matches_eager(cid, T, k):
    inp = make_inputs(replace(WORKLOADS[cid], k=k), T=T)
    other = make_inputs(replace(WORKLOADS[cid], k=k), T=T, hidden_seed=7)
    layer = make_layer(inp, max_tokens=T)
    h = to_torch(inp["hidden"], "bf16")
    h_other = to_torch(other["hidden"], "bf16")
    ref = layer.forward(h)
    torch.cuda.synchronize()
    ref = ref.clone()

    out = torch.empty_like(h)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm the capture stream once
        layer.forward(h, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(h, out=out)
    torch.cuda.synchronize()

    scratch = torch.empty_like(h)
    for rep in range(3):
        out.zero_()
        layer.forward(h_other, out=scratch)          # eager forward on other data
        junk = (h_other.float() * 3.0).sum()         # unrelated torch work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs from the eager forward"
        assert torch.isfinite(junk)
    layer.close()


def test_expert_parallel_shard_shape():
    # one GPU's share under 8-way expert parallelism of the T=4096 top-1 layer:
    # 2 experts, 4096 * 2 / 16 = 512 rows, full d_model and d_ff
    cfg = LayerConfig(91, "ep_shard_bf16_T512_d2048_E2_F3072_top1", T=512, d=2048, E=2, F=3072,
                      k=1, dtype="bf16", bias="normal", family="ep_shard_bf16")
    inp = make_inputs(cfg)
    layer = make_layer(inp)
    st = check_parity(inp, layer, label="EP shard E=2 T=512")
    _, r = layer.forward(to_torch(inp["hidden"], "bf16"), routing=True)
    c = r["counts"].cpu().numpy()
    assert c.sum() == 512 and (c > 0).all()
    assert st["rows_compared"] == 512
    layer.close()
