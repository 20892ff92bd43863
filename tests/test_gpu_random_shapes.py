"""Parity on seeded random layer shapes, all three precisions.

36 cases drawn once from a fixed seed: expert counts 1 to 64 (padded and
unpadded), top-k 1 to 8, d_model 256 to 768, d_ff 128 to 512, batch sizes from
one token through the weight streams (T*k <= 64) to the tile GEMMs, zero and
normal router biases; bf16 layers, E4M3 weights (R18) and E4M3 weights with
E4M3 activations (R20); and 8 fp32 layers whose d_model and d_ff are any
multiple of 4 (4 to 800).  Each case runs the full parity protocol of
tests/_parity.py against the oracle: routing and dispatch arrays in full,
every output row.
"""

import random

import pytest
import torch

from synth import make_inputs
from synth.configs import LayerConfig
from tests._parity import check_parity, make_layer

pytestmark = pytest.mark.gpu


def _cases(n=36, seed=20261204):
    rng = random.Random(seed)
    out = []
    for i in range(n):
        mode = rng.choice(["bf16", "fp8", "w8a8"])
        E = rng.choice([1, 2, 3, 5, 8, 16, 24, 40, 64])
        k = 1 if E == 1 else rng.randint(1, min(8, E))
        d = rng.choice([256, 512, 768])
        F = rng.choice([256, 512]) if mode != "bf16" else rng.choice([128, 256, 384, 512])
        T = rng.choice([1, 2, 5, 17, 32, 40, 64, 65, 100, 300, 1000, 2500])
        bias = rng.choice(["normal", "zero"])
        out.append((mode, T, d, E, F, k, bias, i))
    return out


def _f32_cases(n=8, seed=9):
    rng = random.Random(seed)
    out = []
    for i in range(n):
        E = rng.choice([1, 2, 3, 4, 7, 16, 33, 64])
        k = 1 if E == 1 else rng.randint(1, min(8, E))
        d, F = 4 * rng.randint(1, 200), 4 * rng.randint(1, 200)
        T = rng.choice([1, 2, 7, 31, 64, 65, 200, 1000])
        out.append((T, d, E, F, k, rng.choice(["normal", "zero"]), i))
    return out


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("mode,T,d,E,F,k,bias,i", _cases())
def test_random_shape_parity(mode, T, d, E, F, k, bias, i):
    from tests.test_gpu_fp8 import fp8_layer, fp8_vals
    from tests.test_gpu_w8a8 import w8a8_layer
    cfg = LayerConfig(900 + i, f"random{i}_{mode}_T{T}_d{d}_E{E}_F{F}_k{k}", T=T, d=d, E=E, F=F,
                      k=k, dtype="bf16", bias=bias, family=f"random{i}")
    print(f"[case] {cfg.name} bias={bias}", flush=True)
    inp = make_inputs(cfg)
    if mode == "bf16":
        layer = make_layer(inp, max_tokens=T)
        st = check_parity(inp, layer, label=cfg.name)
    elif mode == "fp8":
        layer = fp8_layer(inp, T)
        st = check_parity(inp, layer, vals=fp8_vals(inp), label=cfg.name)
    else:
        layer = w8a8_layer(inp, T)
        st = check_parity(inp, layer, vals=fp8_vals(inp), fp8_act=True, label=cfg.name)
    assert st["rows_compared"] == T
    layer.close()


@pytest.mark.parametrize("T,d,E,F,k,bias,i", _f32_cases())
def test_random_fp32_shape_parity(T, d, E, F, k, bias, i):
    cfg = LayerConfig(980 + i, f"random_f32_{i}_T{T}_d{d}_E{E}_F{F}_k{k}", T=T, d=d, E=E, F=F,
                      k=k, dtype="f32", bias=bias, family=f"random_f32_{i}")
    print(f"[case] {cfg.name} bias={bias}", flush=True)
    inp = make_inputs(cfg)
    layer = make_layer(inp, max_tokens=T)
    st = check_parity(inp, layer, label=cfg.name)
    assert st["rows_compared"] == T
    layer.close()
