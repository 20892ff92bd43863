"""Synthetic inputs: rounding, reproducibility, and the workloads' structure."""

import json
import os

import numpy as np
import pytest
import torch

from synth import WORKLOADS, make_inputs, round_to_bf16_bits, bf16_bits_to_f32
from synth import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-20, 20, 100000)).astype(np.float32)
    # exact halfway cases, both tie directions
    base = rng.integers(0, 0x7F00, 4000).astype(np.uint32) << 16
    halves = np.concatenate([(base | 0x8000), (base | 0x18000)]).view(np.float32)
    x = np.concatenate([x, halves, np.array([0.0, -0.0, 1e-40, -3e38], np.float32)])
    ours = round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(ours),
                                  torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16)
                                  .float().numpy())


def test_inputs_reproducible_and_distributed_as_stated():
    a = make_inputs(0)
    b = make_inputs(0)
    for name in ("hidden", "gain", "w_router", "bias", "w_gate", "w_up", "w_down"):
        np.testing.assert_array_equal(a[name], b[name])
    cfg = a["cfg"]
    assert a["hidden"].dtype == np.float32 and a["hidden"].shape == (64, 256)
    # N(0, v) with v the variance
    assert abs(np.std(a["w_gate"]) - 1 / np.sqrt(cfg.d)) < 0.01 / np.sqrt(cfg.d)
    assert abs(np.std(a["w_down"]) - 1 / np.sqrt(cfg.F)) < 0.01 / np.sqrt(cfg.F)
    assert abs(np.std(a["gain"]) - np.sqrt(0.1)) < 0.05
    assert abs(np.mean(a["gain"]) - 1.0) < 0.06
    # a different T draws different hidden states, same weights
    c = make_inputs(0, T=17)
    assert c["hidden"].shape == (17, 256)
    np.testing.assert_array_equal(c["w_up"], a["w_up"])


def test_pages_structure_matches_workloads():
    with open(os.path.join(GOLDEN, "zonos2_structure.json")) as f:
        s = json.load(f)
    for cid in (1, 2, 3, 4):
        assert WORKLOADS[cid].E == s["experts_per_moe_layer"]
    assert {WORKLOADS[c].k for c in (1, 2, 4)} == {s["top_k_moe_layers"]}
    assert WORKLOADS[3].k == s["top_k_last_moe_layer"]
    # assumed widths are consistent with 8B total / 900M active parameters
    cfg = WORKLOADS[1]
    moe_layers = s["layers"] - len(s["dense_layers"])
    per_expert = 3 * cfg.d * cfg.F
    assert moe_layers * cfg.E * per_expert < s["total_params"]
    active = (moe_layers - 1) * 1 * per_expert + 1 * 2 * per_expert
    assert active < s["active_params"]


@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_large_workloads_bf16_storage(cid):
    cfg = WORKLOADS[cid]
    w = gen.family_weights(cfg)
    assert w["w_gate"].dtype == np.uint16 and w["w_gate"].shape == (16, 3072, 2048)
    assert w["w_down"].shape == (16, 2048, 3072)


def test_skewed_workload_bias_realises_zipf():
    """The stored bias of the skewed workload gives Zipf(1.2) shares under the
    oracle's top-1 selection, with at least one empty expert."""
    from oracle import moe_oracle as O
    from oracle.calibrate_zipf_bias import zipf_targets
    inp = gen.values_f32(make_inputs(4))
    x = O.rmsnorm(inp["hidden"], inp["gain"], 1e-6)
    _, s = O.router_scores(x, inp["w_router"], inp["bias"])
    sel, _ = O.select_topk(s, 1)
    share = np.bincount(sel[:, 0], minlength=16) / sel.shape[0]
    tgt = zipf_targets(16)
    live = tgt > 0
    assert np.all(np.abs(share[live] - tgt[live]) / tgt[live] < 0.02)
    assert np.sum(share == 0) >= 1
    assert 0.36 < share.max() < 0.41
