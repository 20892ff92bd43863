"""fp8 weights with fp8 activations (moe_layer_create_w8a8) against the
oracle's O12 reading.

The quantisation step itself (moe_fp8_quantize_rows, the device code that the
layer's tile quantiser shares) is compared bit for bit with
oracle.quantize_rows_e4m3 on bf16 rows that include zero rows, exact ties
between E4M3 neighbours and values in E4M3's subnormal range.  The layer is
compared with oracle_forward(fp8_act=True) on the exact dequantised weights,
every output row, at the decode, prefill, top-2 and skewed workloads and at
ragged sizes; routing and dispatch as for the bf16 layer.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import WORKLOADS, make_inputs
from synth.gen import fp8_expert_weights
from tests._parity import check_parity, device_weights, to_torch
from tests.test_gpu_fp8 import fp8_vals

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_ffn_amd import load_library
    load_library()


def _bf16_rows(rng, R, K):
    x = rng.standard_normal((R, K)) * np.exp2(rng.integers(-20, 20, (R, 1)))
    x[1] = 0.0                                       # a zero row
    x[2, :] = 0.0
    x[2, 5] = -3.0                                   # one non-zero entry
    # row 3: scale exactly 2^-4 (amax 448 * 2^-4), the rest on ties between
    # E4M3 neighbours (normal and subnormal ones) and their negatives
    vals = O.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[1:] + vals[:-1]) / 2
    t = np.resize(np.concatenate([mids, -mids]), K)
    t[0] = 448.0
    x[3] = t * 2.0 ** -4
    x[4] = rng.standard_normal(K) * 2.0 ** -12      # many codes in the subnormal range
    x[4, 7] = 1.0
    xb = O.bf16_round(x)
    assert np.array_equal(O.bf16_round(x[3]), x[3])  # the ties are bf16 values
    return xb


# K up to 4096: each row held in registers; beyond, two passes over the row
@pytest.mark.parametrize("R,K", [(64, 2048), (9, 8), (33, 3072), (5, 4096), (6, 5000)])
def test_quantize_rows_bit_exact(R, K):
    from moe_ffn_amd import fp8_quantize_rows
    rng = np.random.default_rng(R * 7 + K)
    x = _bf16_rows(rng, R, K) if K >= 256 else O.bf16_round(rng.standard_normal((R, K)))
    print(f"[quant] R={R} K={K}", flush=True)
    xt = torch.from_numpy(x.astype(np.float32)).cuda().to(torch.bfloat16)   # exact: bf16 values
    codes, scales = fp8_quantize_rows(xt)
    torch.cuda.synchronize()
    want_c, want_a = O.quantize_rows_e4m3(x)
    got_c = codes.cpu().numpy()
    np.testing.assert_array_equal(scales.cpu().numpy(), want_a)
    bad = np.argwhere(got_c != want_c)
    assert bad.size == 0, (f"{len(bad)} codes differ, first at {bad[:3].tolist()}: "
                           f"got {got_c[tuple(bad[0])]:#x} want {want_c[tuple(bad[0])]:#x}")


def w8a8_layer(inputs: dict, max_tokens: int):
    from moe_ffn_amd import MoELayer
    cfg = inputs["cfg"]
    q = fp8_expert_weights(inputs)
    w = device_weights(inputs)
    for name in ("w_gate", "w_up", "w_down"):
        w[name] = torch.from_numpy(q[name]).cuda()
    scales = {s: torch.from_numpy(q["s_" + s]).cuda() for s in ("gate", "up", "down")}
    layer = MoELayer(cfg.d, cfg.F, cfg.E, cfg.k, cfg.dtype, w, max_tokens, rms_eps=cfg.eps,
                     fp8_scales=scales, fp8_act=True)
    torch.cuda.synchronize()
    return layer


_layers = {}


def family_w8a8_layer(cid: int, k: int):
    key = (WORKLOADS[cid].family, k, WORKLOADS[cid].bias)
    if key not in _layers:
        _layers[key] = w8a8_layer(make_inputs(replace(WORKLOADS[cid], k=k)), max_tokens=16384)
    return _layers[key]


@pytest.mark.parametrize("cid,T,k", [
    (1, None, 1),   # decode T = 32 (the tile path: one subtile per expert)
    (1, 7, 1),      # ragged, most experts empty
    (3, 32, 2),     # top-2, 64 assignments
    (2, 300, 1),    # ragged tails
    (3, 200, 2),    # + combine
    (2, None, 1),   # prefill T = 4096, every row
    (3, None, 2),   # top-2 T = 4096, every row
    (4, None, 1),   # skewed T = 16384 (an empty expert, a 37% one), every row
])
def test_w8a8_parity(cid, T, k):
    base = replace(WORKLOADS[cid], k=k)
    inp = make_inputs(base, T=T) if T is not None else make_inputs(base)
    label = f"w8a8 c{cid} T={inp['cfg'].T} k={k}"
    print(f"[case] {label}", flush=True)
    st = check_parity(inp, family_w8a8_layer(cid, k), vals=fp8_vals(inp), fp8_act=True,
                      label=label)
    assert st["rows_compared"] == inp["cfg"].T
    # the layer against the oracle of the same reading: only fp32 rounding and
    # the rare E4M3 code that a bf16 rounding difference moves remain
    assert st["rms_err_rel"] < 5e-3


def test_w8a8_differs_from_weight_only_by_the_quantisation():
    # the same codes and scales with bf16 activations (R18) and with fp8
    # activations: outputs differ by about 2^-5 relative, the size of the two
    # E4M3 roundings, and the routing is the same
    from tests.test_gpu_fp8 import fp8_layer
    inp = make_inputs(WORKLOADS[2], T=512)
    l8 = w8a8_layer(inp, 512)
    l16 = fp8_layer(inp, 512)
    h = to_torch(inp["hidden"], "bf16")
    o8, r8 = l8.forward(h, routing=True)
    o16, r16 = l16.forward(h, routing=True)
    torch.cuda.synchronize()
    assert torch.equal(r8["sel"], r16["sel"])
    d = (o8.float() - o16.float()).pow(2).mean().sqrt() / o16.float().pow(2).mean().sqrt()
    assert 3e-3 < float(d) < 0.1


def test_w8a8_static_and_repeat_are_byte_identical():
    inp = make_inputs(WORKLOADS[2], T=160)
    layer = family_w8a8_layer(2, 1)
    h = to_torch(inp["hidden"], "bf16")
    a = layer.forward(h)
    b = layer.forward(h)
    c = layer.forward(h, static_scratch=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


@pytest.mark.parametrize("E,k,T", [(4, 1, 100), (40, 3, 1000), (16, 2, 333)])
def test_w8a8_small_shapes(E, k, T):
    # d_ff = 256: 2 * d_ff is not a multiple of 384, so the gate/up GEMM takes
    # its two-tile (RT = 2) fp8 form; many experts and top-3 as well
    from synth.configs import LayerConfig
    cfg = LayerConfig(94, f"w8a8_small_E{E}_k{k}_T{T}", T=T, d=256, E=E, F=256, k=k,
                      dtype="bf16", bias="normal", family=f"w8a8_small_d256_E{E}_F256")
    inp = make_inputs(cfg)
    print(f"[case] {cfg.name}", flush=True)
    st = check_parity(inp, w8a8_layer(inp, T), vals=fp8_vals(inp), fp8_act=True, label=cfg.name)
    assert st["rows_compared"] == T
    assert st["rms_err_rel"] < 5e-3


@pytest.mark.parametrize("T", [1, 40, 300])
def test_w8a8_edge_cases(T):
    """Zero hidden rows (scale 0, codes 0 all the way through), every token
    routed to one expert by a large bias, and single tokens, on the weight
    streams (T * k <= 64) and on the fp8 MFMA GEMMs."""
    base = make_inputs(WORKLOADS[2], T=T)
    h = base["hidden"].copy()
    h[::7] = 0                                  # rows 0, 7, 14, ... all bf16 +0
    zero_rows = dict(base, hidden=h)
    b = np.array(base["bias"], np.float32).copy()
    b[5] += 1e4
    one_expert = dict(base, bias=b)
    for label, inp in (("zero rows", zero_rows), ("one expert", one_expert)):
        print(f"[case] w8a8 {label} T={T}", flush=True)
        st = check_parity(inp, w8a8_layer(inp, T), vals=fp8_vals(inp), fp8_act=True,
                          label=f"w8a8 {label} T={T}")
        assert st["rows_compared"] == T
    out = w8a8_layer(zero_rows, T).forward(to_torch(h, "bf16"))
    torch.cuda.synchronize()
    assert torch.all(out[::7] == 0)             # a zero row's output is exactly zero
