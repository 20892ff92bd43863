"""Parity of the HIP layer (through the C ABI) with the fp64 oracle.

Covers the five workloads at full size (routing, dispatch and every output
row), reduced sizes that span several tiles with ragged tails on both expert
paths, and the edge cases: T = 0, T = 1, T = max_tokens, every token on one
expert, exact score ties (the lower expert index wins on every router), a
single-expert (dense) layer, expert counts from 5 to 64 and top-k up to 8 on
both paths and both dtypes, NaN rows, bias updates, determinism and bad
arguments.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

from synth import WORKLOADS, make_inputs
from synth.configs import LayerConfig
from tests._parity import check_parity, make_layer, to_torch, device_weights, out_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from moe_ffn_amd import load_library
    load_library()  # fails loudly if the library is not built


_layers = {}


def family_layer(cid: int, k: int | None = None, max_tokens: int | None = None, bias=None):
    """One library layer per (family, k, max_tokens, bias) reused across tests."""
    base = WORKLOADS[cid]
    k = k or base.k
    max_tokens = max_tokens or 16384
    key = (base.family, k, max_tokens, base.bias if bias is None else bias)
    if key not in _layers:
        inp = make_inputs(replace(base, k=k, bias=base.bias if bias is None else bias))
        _layers[key] = make_layer(inp, max_tokens=max_tokens)
    return _layers[key]


# ----------------------------------------------------------- full workloads
def test_tiny_fp32_T64_full():
    inp = make_inputs(0)
    check_parity(inp, make_layer(inp), label="c0 tiny fp32")


def test_decode_bf16_T32_full():
    inp = make_inputs(1)
    check_parity(inp, family_layer(1), label="c1 decode T=32")


def test_prefill_bf16_T4096_full():
    inp = make_inputs(2)
    st = check_parity(inp, family_layer(2), label="c2 prefill T=4096")
    assert st["rows_compared"] == 4096


def test_top2_bf16_T4096_full():
    inp = make_inputs(3)
    st = check_parity(inp, family_layer(3), label="c3 top-2 T=4096")
    assert st["rows_compared"] == 4096


def test_skewed_bf16_T16384_full():
    inp = make_inputs(4)
    layer = family_layer(4)
    st = check_parity(inp, layer, label="c4 skewed T=16384")
    assert st["rows_compared"] == 16384
    _, r = layer.forward(to_torch(inp["hidden"], "bf16"), routing=True)
    counts = r["counts"].cpu().numpy()
    assert counts.sum() == 16384 and (counts == 0).sum() >= 1
    assert 0.36 < counts.max() / 16384 < 0.41


# ------------------------------------------------- reduced sizes, ragged tails
@pytest.mark.parametrize("cid,T,k", [
    (2, 300, 1),    # tile path: several 128-token tiles per expert, ragged tails
    (2, 129, 1),
    (3, 200, 2),    # tile path + combine
    (3, 33, 2),     # 66 assignments: just above the decode path's limit
    (3, 32, 2),     # 64 assignments: decode path + combine
    (1, 45, 1),     # decode path
    (1, 7, 1),
    (1, 1, 1),
    (4, 1000, 1),   # skewed bias at a reduced size
])
def test_reduced_sizes_full_rows(cid, T, k):
    base = WORKLOADS[cid]
    inp = make_inputs(replace(base, k=k), T=T)
    check_parity(inp, family_layer(cid, k=k), label=f"c{cid} T={T} k={k}")


# Batch sizes at which the launches choose other spans per unit than at the
# workloads above (the down projection takes at most 4 subtiles per unit at
# 2048 assignments and 5 at 12288, 6 at 4096 and 16384).
@pytest.mark.parametrize("T", [2048, 12288])
def test_other_span_caps(T):
    inp = make_inputs(WORKLOADS[2], T=T)
    st = check_parity(inp, family_layer(2), label=f"c2 T={T}")
    assert st["rows_compared"] == T


def test_tiny_fp32_ragged_and_top2():
    for T, k in [(1, 1), (37, 1), (64, 2), (5, 3)]:
        inp = make_inputs(replace(WORKLOADS[0], k=k), T=T)
        check_parity(inp, make_layer(inp, max_tokens=64), label=f"c0 T={T} k={k}")


# ------------------------------------------------------------------ edges
def test_T0_launches_nothing_and_T_max():
    layer = family_layer(1, max_tokens=256)
    h = torch.empty((0, 2048), dtype=torch.bfloat16, device="cuda")
    out = layer.forward(h)
    assert out.shape == (0, 2048)
    inp = make_inputs(WORKLOADS[1], T=256)   # same weights and bias as the layer
    check_parity(inp, layer, label="T = max_tokens = 256")


def test_every_token_on_one_expert():
    for T in (64, 300):   # decode path with two 32-token passes; tile path with 3 tiles
        cfg = replace(WORKLOADS[2], T=T)
        inp = make_inputs(cfg)
        b = np.zeros(16, np.float32)
        b[5] = 1e4
        inp = dict(inp, bias=b)
        layer = make_layer(inp, max_tokens=T)
        st = check_parity(inp, layer, label=f"all on expert 5, T={T}")
        _, r = layer.forward(to_torch(inp["hidden"], "bf16"), routing=True)
        c = r["counts"].cpu().numpy()
        assert c[5] == T and c.sum() == T
        assert np.array_equal(r["gather"].cpu().numpy(), np.arange(T))
        assert st["near_ties"] == 0


@pytest.mark.parametrize("dtype,T,k", [
    ("bf16", 32, 1),    # per-token router (decode path)
    ("bf16", 16, 2),
    ("bf16", 300, 1),   # MFMA router (tile path)
    ("bf16", 300, 2),
    ("f32", 40, 1),     # fp32 router
    ("f32", 40, 2),
])
def test_exact_score_tie_goes_to_the_lower_expert(dtype, T, k):
    """Two experts with the same router row and the same bias score every
    token identically.  The tie is exact, so the near-tie exemption does not
    apply: the lower index must come first (and for top-2 the pair must be
    (lower, higher) with equal gates)."""
    base = WORKLOADS[1] if dtype == "bf16" else WORKLOADS[0]
    lo, hi = (3, 9) if dtype == "bf16" else (1, 3)
    inp = make_inputs(replace(base, k=k), T=T)
    wr = inp["w_router"].copy()
    wr[hi] = wr[lo]
    b = np.asarray(inp["bias"], np.float32).copy()
    b[lo] = b[hi] = 8.0   # both far above every other score
    inp = dict(inp, w_router=wr, bias=b)
    layer = make_layer(inp, max_tokens=T)
    st = check_parity(inp, layer, label=f"tie {dtype} T={T} k={k}")
    assert st["near_ties"] == T   # margin 0 on every token
    _, r = layer.forward(to_torch(inp["hidden"], dtype), routing=True)
    sel = r["sel"].cpu().numpy()
    assert np.all(sel[:, 0] == lo), np.unique(sel[:, 0])
    if k == 2:
        assert np.all(sel[:, 1] == hi)
        g = r["gate"].cpu().numpy()
        assert np.all(g == 0.5)   # softmax of two equal logits
    layer.close()


@pytest.mark.parametrize("dtype,d,F", [("bf16", 256, 128), ("f32", 64, 96)])
def test_single_expert_dense_layer(dtype, d, F):
    cfg = LayerConfig(90, "dense", T=77, d=d, E=1, F=F, k=1, dtype=dtype, bias="zero",
                      family="dense_" + dtype)
    inp = make_inputs(cfg)
    layer = make_layer(inp)
    st = check_parity(inp, layer, label=f"E=1 dense {dtype}")
    assert st["near_ties"] == 0  # a single expert has an infinite margin
    _, r = layer.forward(to_torch(inp["hidden"], dtype), routing=True)
    assert torch.all(r["gate"] == 1.0) and torch.all(r["sel"] == 0)


@pytest.mark.parametrize("dtype,E,k,T", [
    ("bf16", 5, 3, 20),     # 60 assignments: decode path, odd expert count
    ("bf16", 5, 3, 100),    # tile path
    ("bf16", 24, 2, 32),    # 64 assignments: decode path at its limit
    ("bf16", 24, 2, 200),
    ("bf16", 33, 4, 50),    # 33..64 experts: the widest router tiles
    ("bf16", 64, 8, 8),     # the limits: 64 experts, top-8 (64 assignments)
    ("bf16", 64, 8, 150),
    ("bf16", 64, 1, 64),
    ("f32", 64, 8, 40),
    ("f32", 7, 2, 33),
])
def test_expert_counts_and_top_k_up_to_the_limits(dtype, E, k, T):
    d, F = (256, 256) if dtype == "bf16" else (64, 96)
    cfg = LayerConfig(92, f"limits_{dtype}_E{E}_k{k}_T{T}", T=T, d=d, E=E, F=F, k=k,
                      dtype=dtype, bias="normal", family=f"limits_{dtype}_d{d}_E{E}_F{F}")
    inp = make_inputs(cfg)
    st = check_parity(inp, make_layer(inp, max_tokens=T), label=cfg.name)
    assert st["rows_compared"] == T


@pytest.mark.parametrize("E,k,T", [
    (16, 8, 9000),   # 72,000 assignments: 225 groups of 5 chunks, the last one ragged
    (64, 2, 40000),  # 80,000 assignments over 64 experts: 250 groups
    (8, 4, 16384),   # 65,536 assignments: exactly 256 groups of 4 chunks
])
def test_permutation_over_many_groups(E, k, T):
    """The two-launch permutation at sizes where its groups grow past four
    chunks each: dispatch arrays and output rows in full."""
    cfg = LayerConfig(93, f"groups_bf16_E{E}_k{k}_T{T}", T=T, d=256, E=E, F=256, k=k,
                      dtype="bf16", bias="normal", family=f"groups_bf16_d256_E{E}_F256")
    inp = make_inputs(cfg)
    st = check_parity(inp, make_layer(inp, max_tokens=T), label=cfg.name)
    assert st["rows_compared"] == T


@pytest.mark.parametrize("E,k,T", [
    (64, 2, 4096),   # 8192 assignments: exactly 128 chunks, the largest one-launch batch
    (40, 3, 2730),   # 8190: one launch, ragged last chunk, 40 experts (64 padded)
    (5, 1, 389),     # 7 chunks: the second workgroup places three
    (64, 1, 8193),   # one assignment past the one-launch limit: two launches
])
def test_permutation_one_launch_and_its_limit(E, k, T):
    """The one-launch permutation (every workgroup counts all chunks, places
    four) up to its limit and the two-launch form just past it: dispatch
    arrays and output rows in full."""
    cfg = LayerConfig(94, f"perm_bf16_E{E}_k{k}_T{T}", T=T, d=256, E=E, F=256, k=k,
                      dtype="bf16", bias="normal", family=f"groups_bf16_d256_E{E}_F256")
    inp = make_inputs(cfg)
    print(f"[case] {cfg.name}", flush=True)
    st = check_parity(inp, make_layer(inp, max_tokens=T), label=cfg.name)
    assert st["rows_compared"] == T


def test_deterministic_bytes():
    inp = make_inputs(3, T=1000)
    layer = family_layer(3)
    h = to_torch(inp["hidden"], "bf16")
    o1, r1 = layer.forward(h, routing=True)
    o2, r2 = layer.forward(h, routing=True)
    o3 = layer.forward(h)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
    for key in r1:
        assert torch.equal(r1[key], r2[key]), key


def test_nan_row_stays_in_bounds_and_leaves_other_rows_alone():
    for cid, T in [(1, 32), (2, 300)]:
        inp = make_inputs(WORKLOADS[cid], T=T)
        layer = family_layer(cid)
        h = to_torch(inp["hidden"], "bf16")
        hn = h.clone()
        hn[3, 17] = float("nan")
        o, r = layer.forward(h, routing=True)
        on, rn = layer.forward(hn, routing=True)
        torch.cuda.synchronize()
        sel = rn["sel"]
        assert int(sel.min()) >= 0 and int(sel.max()) < 16
        assert int(rn["counts"].sum()) == T
        g = rn["gather"].cpu().numpy()
        assert sorted(g.tolist()) == list(range(T))
        keep = torch.ones(T, dtype=torch.bool, device="cuda")
        keep[3] = False
        # rows do not interact: every other row is bit-identical when its route is
        assert torch.equal(rn["sel"][keep], r["sel"][keep])
        assert torch.equal(on[keep].view(torch.int16), o[keep].view(torch.int16))


def test_set_bias_steers_routing():
    inp = make_inputs(WORKLOADS[1])
    layer = make_layer(inp, max_tokens=32)
    b = torch.zeros(16, dtype=torch.float32, device="cuda")
    b[11] = 1e4
    layer.set_bias(b)
    inp2 = dict(inp, bias=b.cpu().numpy())
    check_parity(inp2, layer, label="after set_bias")
    _, r = layer.forward(to_torch(inp["hidden"], "bf16"), routing=True)
    assert int(r["counts"][11]) == 32


def test_bad_arguments_raise():
    from moe_ffn_amd import MoELayerError, MOE_ERR_INVALID_ARG
    layer = family_layer(1, max_tokens=256)
    h = torch.zeros((257, 2048), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(MoELayerError) as ei:
        layer.forward(h)
    assert ei.value.status == MOE_ERR_INVALID_ARG
    h = torch.zeros((64, 2048), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(MoELayerError) as ei:
        layer.forward(h, out=h)
    assert ei.value.status == MOE_ERR_INVALID_ARG
    buf = torch.zeros(64 * 2048 + 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(MoELayerError):
        layer.forward(h, out=buf[1:1 + 64 * 2048].view(64, 2048))   # misaligned out
    for bad in (torch.zeros((63, 2048), dtype=torch.bfloat16, device="cuda"),   # too few rows
                torch.zeros((64, 2048), dtype=torch.float32, device="cuda"),    # wrong dtype
                torch.zeros((2048, 64), dtype=torch.bfloat16, device="cuda").t()):  # strided
        with pytest.raises(ValueError):
            layer.forward(h, out=bad)



@pytest.mark.parametrize("w8a8,F", [(False, 1152), (True, 1280)])
def test_grouped_unit_order_with_a_partial_group(w8a8, F):
    """Experts with eight or more token spans take their weight blocks in
    groups of four, span-major.  bf16 d_ff 1152: six 384-row gate/up blocks
    (a group of four, then one of two); fp8 activations d_ff 1280: ten 256-row
    blocks (4, 4, 2).  A bias steers most of the 3000 tokens to expert 0 (some
    80 subtiles, 16 or more spans), the rest over three others: output rows
    and dispatch arrays in full."""
    cfg = LayerConfig(95, f"grouped_bf16_T3000_d2048_E4_F{F}", T=3000, d=2048, E=4, F=F, k=1,
                      dtype="bf16", bias="normal", family=f"grouped_bf16_d2048_E4_F{F}")
    inp = dict(make_inputs(cfg), bias=np.array([2.0, 0.0, 0.0, 0.0], np.float32))
    print(f"[case] {cfg.name} w8a8={w8a8}", flush=True)
    if w8a8:
        from tests.test_gpu_w8a8 import fp8_vals, w8a8_layer
        layer = w8a8_layer(inp, cfg.T)
        st = check_parity(inp, layer, vals=fp8_vals(inp), fp8_act=True, label=cfg.name)
    else:
        layer = make_layer(inp, max_tokens=cfg.T)
        st = check_parity(inp, layer, label=cfg.name)
    assert st["rows_compared"] == cfg.T
    _, r = layer.forward(to_torch(inp["hidden"], "bf16"), routing=True)
    c = r["counts"].cpu().numpy()
    assert c[0] >= 8 * 5 * 32, c  # expert 0 holds at least 8 spans of 5 subtiles
