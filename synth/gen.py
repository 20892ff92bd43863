"""Seeded synthetic inputs: random draws and rounding to the storage type.

Every tensor comes from its own PCG64 stream, keyed by
``SeedSequence(0, spawn_key=(family, tensor, extra...))``, so that any tensor
can be regenerated alone.  Draws are float32 standard normals, scaled by the
standard deviation, then (for bf16 layers) rounded to bf16 with
round-to-nearest-even.  The arrays handed out are the storage form:
``uint16`` bf16 bit patterns or ``float32``; :func:`values_f32` widens them
exactly to float32 for consumers that want numbers.

Nothing here evaluates any part of the MoE layer.  The only derived input,
the router bias of the skewed workload, is read from a text file written by
the oracle's calibration script.
"""

from __future__ import annotations

import os
from dataclasses import replace

import numpy as np

from .configs import WORKLOADS, LayerConfig, ZIPF_EMPTY_BIAS  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
ZIPF_BIAS_FILE = os.path.join(_HERE, "zipf_bias_T16384_d2048_E16.txt")

_FAMILY_KEY = {"d256_E4_F512": 1, "d2048_E16_F3072": 2}
_TENSOR_KEY = {"gain": 0, "w_router": 1, "bias": 2, "w_gate": 3, "w_up": 4,
               "w_down": 5, "hidden": 6, "perm": 7}

_weight_cache: dict = {}


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(0, spawn_key=tuple(key))))


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16 rounding of synthetic inputs expects finite values")
    u = x.view(np.uint32)
    # finite values stay below 2**32 after adding the rounding increment
    t = (u >> 16) & np.uint32(1)
    t += np.uint32(0x7FFF)
    t += u
    t >>= 16
    return t.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _normal(key, shape, std: float) -> np.ndarray:
    g = _rng(*key).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        g *= np.float32(std)
    return g


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return round_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def family_weights(cfg: LayerConfig, layer: int | None = None) -> dict:
    """Gain, router and expert weights; shared by every config of one family.

    ``layer`` selects the weights of one layer of a stack (an independent
    stream per layer index); None is the single-layer family."""
    ck = (cfg.family, cfg.d, cfg.E, cfg.F, cfg.dtype, layer)
    if ck in _weight_cache:
        return _weight_cache[ck]
    fam = _FAMILY_KEY.get(cfg.family, 99)
    d, E, F = cfg.d, cfg.E, cfg.F
    extra = () if layer is None else (1000 + int(layer),)
    key = lambda name: (fam, _TENSOR_KEY[name], d, E, F) + extra  # noqa: E731
    gain = _normal(key("gain"), (d,), float(np.sqrt(0.1)))
    gain += np.float32(1.0)
    w = {
        "gain": _store(gain, cfg.dtype),
        "w_router": _store(_normal(key("w_router"), (E, d), 1.0 / np.sqrt(d)), cfg.dtype),
        "w_gate": _store(_normal(key("w_gate"), (E, F, d), 1.0 / np.sqrt(d)), cfg.dtype),
        "w_up": _store(_normal(key("w_up"), (E, F, d), 1.0 / np.sqrt(d)), cfg.dtype),
        "w_down": _store(_normal(key("w_down"), (E, d, F), 1.0 / np.sqrt(F)), cfg.dtype),
        "bias_normal": _normal(key("bias"), (E,), float(np.sqrt(0.1))),
    }
    for v in w.values():
        v.setflags(write=False)
    _weight_cache[ck] = w
    return w


def load_zipf_bias(E: int) -> np.ndarray:
    if not os.path.exists(ZIPF_BIAS_FILE):
        raise FileNotFoundError(
            f"{ZIPF_BIAS_FILE} is missing; it is written by oracle/calibrate_zipf_bias.py")
    vals = []
    with open(ZIPF_BIAS_FILE) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                vals.append(float.fromhex(line) if line.startswith(("0x", "-0x")) else float(line))
    b = np.array(vals, dtype=np.float32)
    if b.shape != (E,):
        raise ValueError(f"zipf bias file holds {b.shape[0]} values, expected {E}")
    return b


def make_inputs(cid_or_cfg, T: int | None = None, hidden_seed: int = 0,
                layer: int | None = None) -> dict:
    """Inputs of one layer workload in storage form.

    ``T`` overrides the token count (hidden states then come from a stream keyed
    by T as well); ``hidden_seed`` selects another hidden-state stream;
    ``layer`` selects one layer's weights (and bias) of a stack.
    Returned keys: cfg, hidden, gain, w_router, bias, w_gate, w_up, w_down.
    """
    cfg = WORKLOADS[int(cid_or_cfg)] if not isinstance(cid_or_cfg, LayerConfig) else cid_or_cfg
    if T is not None and T != cfg.T:
        cfg = replace(cfg, T=int(T))
    w = family_weights(cfg, layer)
    fam = _FAMILY_KEY.get(cfg.family, 99)
    hidden = _store(_normal((fam, _TENSOR_KEY["hidden"], cfg.cid, cfg.T, hidden_seed),
                            (cfg.T, cfg.d), 1.0), cfg.dtype)
    if cfg.bias == "zero":
        bias = np.zeros(cfg.E, np.float32)
    elif cfg.bias == "zipf":
        bias = load_zipf_bias(cfg.E)
    else:
        bias = np.array(w["bias_normal"], np.float32)
    out = {"cfg": cfg, "hidden": hidden, "bias": bias}
    for name in ("gain", "w_router", "w_gate", "w_up", "w_down"):
        out[name] = w[name]
    return out


def zipf_rank_permutation(E: int) -> np.ndarray:
    """Seeded assignment of Zipf ranks to expert ids (entry r = expert of rank r)."""
    return _rng(_FAMILY_KEY["d2048_E16_F3072"], _TENSOR_KEY["perm"], E).permutation(E)


def values_f32(inputs: dict) -> dict:
    """Exact float32 values of every array in ``inputs`` (bf16 bits widened)."""
    cfg = inputs["cfg"]
    out = {"cfg": cfg}
    for name, v in inputs.items():
        if name == "cfg":
            continue
        if name != "bias" and cfg.dtype == "bf16":
            out[name] = bf16_bits_to_f32(v)
        else:
            out[name] = np.asarray(v, np.float32)
    return out


def fp8_expert_weights(inputs: dict) -> dict:
    """E4M3 (OCP) codes and per-output-row float32 scales for the expert
    weights of a bf16 layer's inputs: scale = max|w_row| / 448 (448 being the
    largest E4M3 value), code = the E4M3 nearest to w / scale (torch's
    float8_e4m3fn cast, round to nearest even).  This prepares inputs only:
    the layer consumes the codes and scales as given.
    Returns w_gate, w_up, w_down (uint8) and s_gate [E,F], s_up [E,F],
    s_down [E,d] (float32)."""
    import torch
    cfg = inputs["cfg"]
    ck = ("fp8", cfg.family, cfg.d, cfg.E, cfg.F, id(inputs["w_gate"]))
    if ck in _weight_cache:
        return _weight_cache[ck]
    out = {}
    for name, sname in (("w_gate", "s_gate"), ("w_up", "s_up"), ("w_down", "s_down")):
        w = torch.from_numpy(bf16_bits_to_f32(inputs[name]))
        amax = w.abs().amax(dim=-1)
        scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).to(torch.float32)
        q = (w / scale[..., None]).to(torch.float8_e4m3fn)
        out[name] = q.view(torch.uint8).numpy().copy()
        out[sname] = scale.numpy().copy()
    _weight_cache[ck] = out
    return out
