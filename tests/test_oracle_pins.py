"""Pins of the fp64 oracle against things other than itself.

Each check is chosen so that a plausible slip in the oracle (a dropped eps or
gain, the bias leaking into a gate, a transposed weight, a wrong SiLU, a
wrong combine index, an unstable permutation) fails at least one of them:

* pure-Python brute force on tiny inputs (every expert for every token,
  dense one-hot gate matrix, bucket permutation);
* hand-worked closed-form examples;
* library routines for the steps that have one (torch rms_norm / silu /
  linear, scipy softmax / expit);
* the E=1, k=1 special case, which is a dense SwiGLU FFN;
* invariants (token permutation, expert relabelling, linearity in W_down,
  zero input, forced routing by a huge bias, determinism).
"""

import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import moe_oracle as O
from oracle.brute import brute_forward


def _rand_layer(rng, T, d, E, F, bias_std=0.3):
    return {
        "hidden": rng.standard_normal((T, d)),
        "gain": 1.0 + 0.3 * rng.standard_normal(d),
        "w_router": rng.standard_normal((E, d)) / math.sqrt(d),
        "bias": bias_std * rng.standard_normal(E),
        "w_gate": rng.standard_normal((E, F, d)) / math.sqrt(d),
        "w_up": rng.standard_normal((E, F, d)) / math.sqrt(d),
        "w_down": rng.standard_normal((E, d, F)) / math.sqrt(F),
    }


# ----------------------------------------------------------------- brute force
@pytest.mark.parametrize("T,d,E,F,k,seed", [
    (7, 5, 3, 4, 1, 0), (6, 4, 4, 3, 2, 1), (5, 6, 2, 7, 2, 2), (8, 3, 4, 2, 1, 3),
    (4, 5, 3, 6, 3, 4), (1, 4, 4, 5, 1, 5),
])
def test_oracle_matches_brute_force(T, d, E, F, k, seed):
    rng = np.random.default_rng(seed)
    L = _rand_layer(rng, T, d, E, F)
    eps = 1e-6
    ref = brute_forward(L["hidden"], L["gain"], L["w_router"], L["bias"], L["w_gate"],
                        L["w_up"], L["w_down"], k, eps)
    got = O.oracle_forward(L, k=k, eps=eps)
    np.testing.assert_array_equal(got["sel"], np.array(ref["sel"]))
    np.testing.assert_allclose(got["gate"], np.array(ref["gate"]), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(got["out"], np.array(ref["out"]), rtol=1e-11, atol=1e-13)
    np.testing.assert_array_equal(got["counts"], ref["counts"])
    np.testing.assert_array_equal(got["gather"], ref["gather"])
    np.testing.assert_array_equal(got["scatter"], ref["scatter"])


def test_oracle_matches_brute_force_forced_routing():
    rng = np.random.default_rng(11)
    T, d, E, F, k = 6, 4, 4, 3, 2
    L = _rand_layer(rng, T, d, E, F)
    forced = np.array([[3, 0], [1, 2], [2, 1], [0, 3], [3, 2], [1, 0]], np.int32)
    got = O.oracle_forward(L, k=k, eps=1e-6, forced_sel=forced)
    # no single bias vector reproduces an arbitrary per-token choice, so the
    # forced routing is evaluated here with scalar loops
    H, g = L["hidden"], L["gain"]
    x = np.array([[g[i] * H[t][i] / math.sqrt(sum(v * v for v in H[t]) / d + 1e-6)
                   for i in range(d)] for t in range(T)])
    z = np.array([[sum(L["w_router"][e][i] * x[t][i] for i in range(d)) for e in range(E)]
                  for t in range(T)])
    for t in range(T):
        zz = z[t, forced[t]]
        gt = np.exp(zz - zz.max())
        gt /= gt.sum()
        ref = np.zeros(d)
        for j in range(k):
            e = forced[t, j]
            a = [0.0] * F
            for f in range(F):
                gg = sum(L["w_gate"][e][f][i] * x[t][i] for i in range(d))
                uu = sum(L["w_up"][e][f][i] * x[t][i] for i in range(d))
                a[f] = gg / (1 + math.exp(-gg)) * uu
            for m in range(d):
                ref[m] += gt[j] * sum(L["w_down"][e][m][f] * a[f] for f in range(F))
        np.testing.assert_allclose(got["out"][t], ref, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------ closed forms
def test_hand_worked_top1_bias_flips_selection_not_gate():
    """d=2, E=2, F=1, eps=0, worked by hand.

    h = (1, -1): mean square 1, so x = g*h = (1, -2) for g = (1, 2).
    W_r = [[1, .5], [0, 1]] gives z = (0, -2)  (the transpose would give (1, -1.5)).
    b = (0, 3): s = (0, 1), expert 1 wins although z favours expert 0; margin 1.
    gate = softmax(z)[1] = 1 / (1 + e^2)   (with s it would be e / (1 + e)).
    Expert 1: G = 0.5*1 + 1*(-2) = -1.5, U = 2*1 + 0.25*(-2) = 1.5,
    a = SiLU(-1.5)*1.5, y = W_down[1] a = (a, -3a), out = gate*y.
    """
    L = {
        "hidden": np.array([[1.0, -1.0]]),
        "gain": np.array([1.0, 2.0]),
        "w_router": np.array([[1.0, 0.5], [0.0, 1.0]]),
        "bias": np.array([0.0, 3.0]),
        "w_gate": np.array([[[7.0, 7.0]], [[0.5, 1.0]]]),
        "w_up": np.array([[[7.0, 7.0]], [[2.0, 0.25]]]),
        "w_down": np.array([[[7.0], [7.0]], [[1.0], [-3.0]]]),
    }
    r = O.oracle_forward(L, k=1, eps=0.0)
    np.testing.assert_allclose(r["x"], [[1.0, -2.0]], rtol=0, atol=0)
    np.testing.assert_allclose(r["z"], [[0.0, -2.0]], rtol=0, atol=0)
    assert r["sel"].tolist() == [[1]]
    assert r["margin"][0] == pytest.approx(1.0, abs=0)
    gate = 1.0 / (1.0 + math.exp(2.0))
    assert r["gate"][0, 0] == pytest.approx(gate, rel=1e-15)
    a = (-1.5 / (1.0 + math.exp(1.5))) * 1.5
    np.testing.assert_allclose(r["out"], [[gate * a, gate * -3.0 * a]], rtol=1e-15)
    assert r["counts"].tolist() == [0, 1]
    assert r["offsets"].tolist() == [0, 0, 1]


def test_hand_worked_top2_pair_softmax():
    """E=3, k=2 with W_r = I, g = 1, h chosen with mean square 1:
    h = (sqrt(1.5), -sqrt(1.5), 0) so x = h and z = h.  b = (0, 0, 5) makes
    s = (1.2247, -1.2247, 5): the pair is (2, 0) in that order, and the gates
    are softmax over (z_2, z_0) = (0, 1.2247): (1/(1+e^r), e^r/(1+e^r))."""
    r15 = math.sqrt(1.5)
    L = {
        "hidden": np.array([[r15, -r15, 0.0]]),
        "gain": np.ones(3),
        "w_router": np.eye(3),
        "bias": np.array([0.0, 0.0, 5.0]),
        "w_gate": np.zeros((3, 2, 3)), "w_up": np.zeros((3, 2, 3)),
        "w_down": np.zeros((3, 3, 2)),
    }
    r = O.oracle_forward(L, k=2, eps=0.0)
    assert r["sel"].tolist() == [[2, 0]]
    np.testing.assert_allclose(r["gate"][0], [1 / (1 + math.exp(r15)),
                                              math.exp(r15) / (1 + math.exp(r15))], rtol=1e-14)
    # margin: min(s_(1)-s_(2), s_(2)-s_(3)) = min(5 - r15, 2 r15)
    assert r["margin"][0] == pytest.approx(min(5 - r15, 2 * r15), rel=1e-14)
    assert r["gather"].tolist() == [0, 0]
    assert r["scatter"].tolist() == [1, 0]      # assignment (t0, j0)=expert 2 -> slot 1


def test_exact_ties_go_to_lower_index():
    s = np.array([[1.0, 1.0, 0.0], [0.0, 2.0, 2.0], [3.0, 3.0, 3.0]])
    sel1, m1 = O.select_topk(s, 1)
    assert sel1[:, 0].tolist() == [0, 1, 0]
    np.testing.assert_array_equal(m1, [0.0, 0.0, 0.0])
    sel2, _ = O.select_topk(s, 2)
    assert sel2.tolist() == [[0, 1], [1, 2], [0, 1]]


def test_topk_agrees_with_lexsort_and_margin_definition():
    rng = np.random.default_rng(3)
    s = rng.standard_normal((200, 6))
    for k in (1, 2, 3):
        sel, margin = O.select_topk(s, k)
        for t in range(s.shape[0]):
            order = np.lexsort((np.arange(6), -s[t]))
            assert sel[t].tolist() == order[:k].tolist()
            srt = np.sort(s[t])[::-1]
            gaps = [srt[i] - srt[i + 1] for i in range(k)]
            assert margin[t] == pytest.approx(min(gaps), abs=0)


def test_single_expert_margin_is_infinite():
    _, m = O.select_topk(np.zeros((3, 1)), 1)
    assert np.all(np.isinf(m))


def test_gates_against_scipy_softmax_and_k_equals_E():
    rng = np.random.default_rng(4)
    z = 3 * rng.standard_normal((50, 5))
    sel, _ = O.select_topk(z + rng.standard_normal(5), 1)
    p = scipy.special.softmax(z, axis=1)
    np.testing.assert_allclose(O.gates(z, sel)[:, 0], p[np.arange(50), sel[:, 0]], rtol=1e-13)
    # k = E = 2: the renormalised pair is the full softmax
    z2 = z[:, :2]
    sel2, _ = O.select_topk(z2, 2)
    p2 = scipy.special.softmax(z2, axis=1)
    np.testing.assert_allclose(O.gates(z2, sel2), np.take_along_axis(p2, sel2, axis=1),
                               rtol=1e-13)
    # equal logits: every gate is 1/E for k = 1
    np.testing.assert_allclose(O.gates(np.zeros((2, 4)), np.array([[1], [3]])), 0.25, rtol=0)
    # large logits do not overflow
    g = O.gates(np.array([[1000.0, 999.0, -1000.0]]), np.array([[0, 1]]))
    np.testing.assert_allclose(g, [[1 / (1 + math.exp(-1)), 1 / (1 + math.exp(1))]], rtol=1e-14)


def test_silu_against_scipy_expit():
    v = np.linspace(-40, 40, 1001)
    np.testing.assert_allclose(O.silu(v), v * scipy.special.expit(v), rtol=1e-14, atol=1e-300)
    assert O.silu(np.array([-800.0]))[0] == 0.0


def test_rmsnorm_against_torch_and_closed_form():
    rng = np.random.default_rng(5)
    H = rng.standard_normal((9, 33)) * 3.0
    g = 1 + rng.standard_normal(33)
    for eps in (1e-6, 0.5):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(H), (33,), torch.from_numpy(g),
                                           eps=eps).numpy()
        np.testing.assert_allclose(O.rmsnorm(H, g, eps), ref, rtol=1e-14, atol=1e-15)
    # constant row c: x = g * c / sqrt(c^2 + eps)
    c, eps = -2.5, 0.75
    x = O.rmsnorm(np.full((1, 4), c), np.array([1.0, 2.0, 3.0, 4.0]), eps)
    np.testing.assert_allclose(x[0], np.array([1, 2, 3, 4]) * c / math.sqrt(c * c + eps),
                               rtol=1e-15)
    np.testing.assert_array_equal(O.rmsnorm(np.zeros((2, 3)), np.ones(3), 1e-6), 0.0)


# ------------------------------------------------------ dense special case
def test_single_expert_layer_is_dense_swiglu_ffn():
    """E=1, k=1: the gate is softmax over one logit = 1 and the layer is the
    dense SwiGLU FFN W_down(SiLU(W_gate x) * W_up x) on the RMSNorm output
    (the digest's dense layers 0-2 and 27 are this case)."""
    rng = np.random.default_rng(6)
    T, d, F = 12, 16, 24
    L = _rand_layer(rng, T, d, 1, F)
    r = O.oracle_forward(L, k=1, eps=1e-6)
    np.testing.assert_array_equal(r["gate"], 1.0)
    tt = {k: torch.from_numpy(np.asarray(v, np.float64)) for k, v in L.items()}
    x = torch.nn.functional.rms_norm(tt["hidden"], (d,), tt["gain"], eps=1e-6)
    f = torch.nn.functional
    ref = f.linear(f.silu(f.linear(x, tt["w_gate"][0])) * f.linear(x, tt["w_up"][0]),
                   tt["w_down"][0]).numpy()
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-14)
    assert r["gather"].tolist() == list(range(T))


# ------------------------------------------------------------ permutation
def test_permutation_against_bucket_sort_and_invariants():
    rng = np.random.default_rng(7)
    for T, E, k in [(50, 5, 2), (33, 4, 1), (1, 3, 1), (64, 16, 2)]:
        sel = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        counts, offsets = O.histogram(sel, E)
        gather, scatter = O.permutation(sel)
        buckets = [[] for _ in range(E)]
        for t in range(T):
            for j in range(k):
                buckets[sel[t, j]].append(t * k + j)
        assert counts.tolist() == [len(b) for b in buckets]
        assert int(counts.sum()) == T * k and offsets[-1] == T * k
        flat = [a for b in buckets for a in b]
        assert gather.tolist() == [a // k for a in flat]
        # bijection: scatter inverts the assignment order
        assert sorted(scatter.tolist()) == list(range(T * k))
        for p, a in enumerate(flat):
            assert scatter[a] == p
        # every token appears exactly k times; stable (increasing) within an expert
        assert np.bincount(gather, minlength=T).tolist() == [k] * T
        for e in range(E):
            seg = gather[offsets[e]:offsets[e + 1]]
            assert np.all(np.diff(seg) > 0)


# ------------------------------------------------------------- invariants
def test_invariants():
    rng = np.random.default_rng(8)
    T, d, E, F = 20, 12, 4, 10
    L = _rand_layer(rng, T, d, E, F)
    base = O.oracle_forward(L, k=2, eps=1e-6)
    # determinism
    again = O.oracle_forward(L, k=2, eps=1e-6)
    np.testing.assert_array_equal(base["out"], again["out"])
    # token permutation
    p = rng.permutation(T)
    Lp = dict(L, hidden=L["hidden"][p])
    rp = O.oracle_forward(Lp, k=2, eps=1e-6)
    np.testing.assert_array_equal(rp["sel"], base["sel"][p])
    np.testing.assert_allclose(rp["out"], base["out"][p], rtol=1e-13, atol=1e-15)
    # expert relabelling: new expert i is old expert q[i]
    q = rng.permutation(E)
    Lq = dict(L, w_router=L["w_router"][q], bias=L["bias"][q], w_gate=L["w_gate"][q],
              w_up=L["w_up"][q], w_down=L["w_down"][q])
    rq = O.oracle_forward(Lq, k=2, eps=1e-6)
    np.testing.assert_array_equal(q[rq["sel"]], base["sel"])
    np.testing.assert_allclose(rq["out"], base["out"], rtol=1e-13, atol=1e-15)
    # linear in W_down
    rs = O.oracle_forward(dict(L, w_down=L["w_down"] * -2.5), k=2, eps=1e-6)
    np.testing.assert_allclose(rs["out"], -2.5 * base["out"], rtol=1e-13, atol=1e-15)
    # zero input -> zero output, everyone on argmax(b)
    r0 = O.oracle_forward(dict(L, hidden=np.zeros((T, d))), k=1, eps=1e-6)
    np.testing.assert_array_equal(r0["out"], 0.0)
    assert set(r0["sel"][:, 0].tolist()) == {int(np.argmax(L["bias"]))}
    # a +1e4 bias routes every token to that expert
    b = np.zeros(E)
    b[2] = 1e4
    rb = O.oracle_forward(dict(L, bias=b), k=1, eps=1e-6)
    assert rb["counts"].tolist() == [0, 0, T, 0]
    assert rb["gather"].tolist() == list(range(T))
    # a sampled-token evaluation reproduces the full rows
    tok = np.array([3, 0, 19, 7])
    rt = O.oracle_forward(L, k=2, eps=1e-6, tokens=tok)
    np.testing.assert_allclose(rt["out"], base["out"][tok], rtol=1e-14, atol=1e-16)


# ------------------------------------------------------- O9 balancing step
def test_bias_update_hand_example():
    # E = 3, counts (5, 1, 2): mean 8/3, so expert 0 is over-loaded (bias
    # down) and experts 1, 2 under-loaded (bias up); worked by hand.
    b = np.array([0.25, -0.5, 1.0], np.float32)
    got = O.bias_update(b, [5, 1, 2], 0.125)
    np.testing.assert_array_equal(got, np.array([0.125, -0.375, 1.125], np.float32))
    assert got.dtype == np.float32


def test_bias_update_balanced_and_exact_mean():
    b = np.array([0.1, 0.2, 0.3, 0.4], np.float32)
    # perfectly uniform load: nothing moves
    np.testing.assert_array_equal(O.bias_update(b, [7, 7, 7, 7], 1e-3), b)
    # an expert exactly at the mean load (sum 12, E 4, mean 3) stays put
    got = O.bias_update(b, [3, 5, 1, 3], 1e-3)
    assert got[0] == b[0] and got[3] == b[3]
    assert got[1] < b[1] and got[2] > b[2]


def test_bias_update_single_float32_rounding():
    # the exact sum b + rate is rounded once to float32 (not rate rounded
    # then added in float64 and kept): 1 + 2**-30 rounds back to 1
    b = np.array([1.0, 1.0], np.float32)
    got = O.bias_update(b, [0, 2], 2.0 ** -30)
    np.testing.assert_array_equal(got, np.array([1.0, 1.0], np.float32))
    got = O.bias_update(b, [0, 2], 2.0 ** -20)
    np.testing.assert_array_equal(got, np.array([1.0 + 2.0 ** -20, 1.0 - 2.0 ** -20], np.float32))


def test_bias_update_relabelling_and_balance_direction():
    rng = np.random.default_rng(3)
    b = rng.standard_normal(16).astype(np.float32)
    c = rng.integers(0, 50, 16)
    perm = rng.permutation(16)
    np.testing.assert_array_equal(O.bias_update(b[perm], c[perm], 0.01), O.bias_update(b, c, 0.01)[perm])
    d = O.bias_update(b, c, 0.01).astype(np.float64) - b
    mean = c.mean()
    assert np.all(d[c > mean] < 0) and np.all(d[c < mean] > 0) and np.all(d[c == mean] == 0)


# ------------------------------------------------------------ O10 FFN stack
def test_stack_matches_brute_force_composition():
    # a 3-layer stack (dense, top-1 MoE, top-2 MoE) against the pure-Python
    # brute force applied layer by layer with the residual added by hand
    rng = np.random.default_rng(11)
    d, F, T = 4, 5, 6
    shapes = [(1, 1), (3, 1), (3, 2)]
    layers = []
    for E, k in shapes:
        L = _rand_layer(rng, T, d, E, F)
        L.pop("hidden")
        layers.append(L)
    H = rng.standard_normal((T, d))
    got = O.stack_forward(layers, H, [k for _, k in shapes], 1e-6)
    h = [list(map(float, r)) for r in H]
    for L, (E, k) in zip(layers, shapes):
        r = brute_forward(h, L["gain"], L["w_router"], L["bias"], L["w_gate"], L["w_up"],
                          L["w_down"], k, 1e-6)
        h = [[a + b for a, b in zip(hr, orow)] for hr, orow in zip(h, r["out"])]
    np.testing.assert_allclose(got["out"], np.array(h), rtol=1e-11, atol=1e-12)


def test_stack_of_zero_output_layers_is_identity():
    rng = np.random.default_rng(12)
    layers = []
    for E in (1, 4):
        L = _rand_layer(rng, 5, 6, E, 3)
        L.pop("hidden")
        L["w_down"] = np.zeros_like(L["w_down"])
        layers.append(L)
    H = rng.standard_normal((5, 6))
    np.testing.assert_array_equal(O.stack_forward(layers, H, [1, 1], 1e-6)["out"], H)


# ------------------------------------------- depth averaging of router logits
def _moe_stack_layers(rng, d, F, shapes):
    layers = []
    for E, k in shapes:
        L = _rand_layer(rng, 1, d, E, F)
        L.pop("hidden")
        layers.append(L)
    return layers


def test_depth_average_at_rate_zero_is_the_plain_stack():
    rng = np.random.default_rng(21)
    shapes = [(1, 1), (4, 1), (4, 1), (1, 1), (4, 2), (1, 1)]
    layers = _moe_stack_layers(rng, 6, 5, shapes)
    H = rng.standard_normal((9, 6))
    ks = [k for _, k in shapes]
    plain = O.stack_forward(layers, H, ks, 1e-6)
    eda0 = O.stack_forward(layers, H, ks, 1e-6, eda_alpha=0.0)
    np.testing.assert_array_equal(eda0["out"], plain["out"])
    for a, b in zip(eda0["sel"], plain["sel"]):
        np.testing.assert_array_equal(a, b)


def test_depth_average_recursion_closed_form():
    # three MoE layers: z~_3 = a^2 z_1 + a(1-a) z_2 + (1-a) z_3 (dyadic values,
    # exact in float64); a swapped weight or a missing term fails it
    z1, z2, z3 = np.array([[4.0, -2.0]]), np.array([[1.0, 8.0]]), np.array([[-6.0, 2.0]])
    a = 0.25
    t = O.depth_average(O.depth_average(O.depth_average(None, z1, a), z2, a), z3, a)
    np.testing.assert_array_equal(t, a * a * z1 + a * (1 - a) * z2 + (1 - a) * z3)
    np.testing.assert_array_equal(O.depth_average(None, z2, a), z2)


def test_depth_average_hand_worked_two_layers():
    # d = 2, E = 2, k = 1, zero expert weights (h is the same at both layers):
    # h = (1, 1), gain 1, inv = 1/sqrt(1 + eps); layer 1 logits (2 inv, 0),
    # layer 2 logits (0, inv).  At alpha = 0.5 layer 2 averages to (inv,
    # inv/2): expert 0 instead of 1, gate sigmoid(inv/2).  With a bias
    # (0, 0.6) on layer 2 the choice is expert 1 (score inv/2 + 0.6 > inv)
    # but the gate still comes from the averaged logits: sigmoid(-inv/2).
    eps = 1e-6
    inv = 1.0 / math.sqrt(1.0 + eps)
    zero = np.zeros((2, 1, 2))

    def layer(wr, b):
        return {"gain": np.ones(2), "w_router": np.array(wr, float), "bias": np.array(b, float),
                "w_gate": zero, "w_up": zero, "w_down": np.zeros((2, 2, 1))}
    H = np.array([[1.0, 1.0]])
    l1 = layer([[1, 1], [0, 0]], [0, 0])
    for b2, want_sel, want_gate in [([0, 0], 0, 1 / (1 + math.exp(-inv / 2))),
                                    ([0, 0.6], 1, 1 / (1 + math.exp(inv / 2)))]:
        l2 = layer([[0, 0], [0.5, 0.5]], b2)
        r1 = O.oracle_forward(dict(l1, hidden=H), k=1, eps=eps, z_prev=None, eda_alpha=0.5)
        np.testing.assert_allclose(r1["z"], [[2 * inv, 0.0]], rtol=1e-15)
        r2 = O.oracle_forward(dict(l2, hidden=H), k=1, eps=eps, z_prev=r1["z"], eda_alpha=0.5)
        np.testing.assert_allclose(r2["z"], [[inv, inv / 2]], rtol=1e-15)
        assert int(r2["sel"][0, 0]) == want_sel
        assert abs(r2["gate"][0, 0] - want_gate) < 1e-14
        plain = O.oracle_forward(dict(l2, hidden=H), k=1, eps=eps)
        assert int(plain["sel"][0, 0]) == 1
        st = O.stack_forward([l1, l2], H, [1, 1], eps, eda_alpha=0.5)
        assert int(st["sel"][1][0, 0]) == want_sel


def test_depth_average_needs_one_expert_count():
    # averaging expert e's logit from a 4-expert layer into a 6-expert layer
    # has no meaning: the oracle refuses it rather than pad or truncate
    rng = np.random.default_rng(22)
    layers = _moe_stack_layers(rng, 6, 5, [(1, 1), (4, 1), (6, 1), (1, 1)])
    H = rng.standard_normal((3, 6))
    with pytest.raises(ValueError):
        O.stack_forward(layers, H, [1, 1, 1, 1], 1e-6, eda_alpha=0.5)
    with pytest.raises(ValueError):
        O.depth_average(np.zeros((3, 4)), np.zeros((3, 6)), 0.5)
    # without the averaging the same stack is fine, and dense layers never count
    O.stack_forward(layers, H, [1, 1, 1, 1], 1e-6)
    same = _moe_stack_layers(rng, 6, 5, [(1, 1), (6, 1), (6, 2), (1, 1)])
    O.stack_forward(same, H, [1, 1, 2, 1], 1e-6, eda_alpha=0.5)


# ------------------------------------------------------------- fp8 weights
def test_e4m3_decoder_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_value(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2   # 0x7f and 0xff
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    # a few by hand: max normal, min normal, min subnormal, -1.5
    assert O.e4m3_value([0x7e])[0] == 448.0 and O.e4m3_value([0x08])[0] == 2.0 ** -6
    assert O.e4m3_value([0x01])[0] == 2.0 ** -9 and O.e4m3_value([0xbc])[0] == -1.5


def test_fp8_weights_scale_rows_exactly():
    codes = np.array([[[0x38, 0x40], [0xb8, 0x00]]], np.uint8)   # 1, 2 / -1, 0
    scale = np.array([[0.5, 3.0]], np.float32)
    np.testing.assert_array_equal(O.fp8_weights(codes, scale), [[[0.5, 1.0], [-3.0, 0.0]]])


# ------------------------------------------------------------- fp8 activations
def test_bf16_round_matches_torch_on_float32_values():
    rng = np.random.default_rng(30)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))
    x32 = x.astype(np.float32)
    # exact midpoints between neighbouring bf16 values (float32 holds them)
    b = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float32).numpy()
    mid = (b.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    for v in (x32, mid):
        ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
        np.testing.assert_array_equal(O.bf16_round(v.astype(np.float64)), ref)
    # by hand: a tie goes to the even significand; just above a tie rounds up;
    # a float64 just below the midpoint -2776 rounds to -2768 (a detour
    # through float32 would land on the midpoint and round to -2784)
    assert O.bf16_round(1 + 2.0 ** -8) == 1.0
    assert O.bf16_round(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6
    assert O.bf16_round(1 + 2.0 ** -8 + 2.0 ** -30) == 1 + 2.0 ** -7
    assert O.bf16_round(-2775.99990387) == -2768.0


def test_e4m3_encode_round_trips_every_code_and_matches_torch():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    np.testing.assert_array_equal(O.e4m3_encode(O.e4m3_value(codes)), codes)
    rng = np.random.default_rng(31)
    v = rng.uniform(-1, 1, 30000) * np.exp2(rng.integers(-12, 9, 30000))
    v = np.clip(v, -448, 448)
    vals = O.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[1:] + vals[:-1]) / 2
    for x in (v, mids, -mids):
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        np.testing.assert_array_equal(O.e4m3_encode(x), ref)


def test_e4m3_encode_is_the_nearest_value_ties_to_even():
    allc = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    allv = O.e4m3_value(allc)
    rng = np.random.default_rng(32)
    v = rng.uniform(-1, 1, 3000) * np.exp2(rng.integers(-11, 9, 3000))
    v = np.clip(v, -448, 448)
    got = O.e4m3_value(O.e4m3_encode(v))
    best = np.min(np.abs(v[:, None] - allv[None, :]), axis=1)   # brute force over all values
    np.testing.assert_array_equal(np.abs(v - got), best)
    vals = O.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[1:] + vals[:-1]) / 2
    c = O.e4m3_encode(mids)
    assert np.all(c % 2 == 0)                                     # even last mantissa bit
    assert np.all((O.e4m3_value(c) == vals[1:]) | (O.e4m3_value(c) == vals[:-1]))
    # saturation, zero signs, NaN
    np.testing.assert_array_equal(O.e4m3_encode([450.0, -1e6, 0.0, -0.0, np.nan]),
                                  [0x7E, 0xFE, 0x00, 0x80, 0x7F])


def test_quantize_rows_hand_examples():
    # scale exactly 1: 1.0625 is the tie between 1 (0x38) and 1.125 (0x39);
    # 2^-8 is the subnormal 2 * 2^-9
    c, a = O.quantize_rows_e4m3(np.array([[448.0, 1.0625, -2.0 ** -8, 0.0]]))
    assert a[0] == np.float32(1.0)
    np.testing.assert_array_equal(c[0], [0x7E, 0x38, 0x82, 0x00])
    # [3, 1]: a = float32(3/448); 1 * float32(1/a) = 149.33.. lies between 144 and 160
    c, a = O.quantize_rows_e4m3(np.array([[3.0, 1.0]]))
    assert a[0] == np.float32(3.0) / np.float32(448.0)
    np.testing.assert_array_equal(c[0], [0x7E, 0x71])
    assert O.e4m3_value([0x71])[0] == 144.0
    # a zero row: scale 0, codes 0
    c, a = O.quantize_rows_e4m3(np.zeros((2, 5)))
    assert np.all(a == 0) and np.all(c == 0)
    with pytest.raises(ValueError):
        O.quantize_rows_e4m3(np.array([[1.0 + 2.0 ** -40]]))


def test_quantize_rows_error_bound_and_scale_invariance():
    rng = np.random.default_rng(33)
    V = O.bf16_round(rng.standard_normal((64, 200)) * np.exp2(rng.integers(-6, 6, (64, 1))))
    V[3] = 0.0
    V[5, :7] = 0.0
    c, a = O.quantize_rows_e4m3(V)
    ok = a > 0
    # the largest |v| of each row lands on +-448
    arg = np.argmax(np.abs(V), axis=1)
    assert np.all(np.abs(O.e4m3_value(c[np.arange(64), arg]))[ok] == 448.0)
    assert np.all(a[ok] == (np.max(np.abs(V), axis=1)[ok] / 448.0).astype(np.float32))
    # every code is within half an E4M3 spacing of v / a (spacing 2^(E-3) for
    # |t| in [2^E, 2^(E+1)), E >= -6; 2^-9 below 2^-6), plus the float32
    # roundings of the reciprocal and of the product
    t = V[ok] / a[ok].astype(np.float64)[:, None]
    E = np.floor(np.log2(np.maximum(np.abs(t), 2.0 ** -6)))
    half = np.exp2(E - 3) / 2
    err = np.abs(O.e4m3_value(c[ok]) - t)
    assert np.all(err <= half + np.abs(t) * 2.0 ** -22)
    # the quotient is the float32 product with the float32 reciprocal
    r = (np.float32(1) / a[ok]).astype(np.float32)
    q = (V[ok].astype(np.float32) * r[:, None]).astype(np.float32)
    np.testing.assert_array_equal(c[ok], O.e4m3_encode(q.astype(np.float64)))
    # dequantised rows against the input: relative 2^-4 plus the subnormal floor
    D = O.dequantize_rows(c, a)
    assert np.all(np.abs(D - V) <= np.abs(V) * (2.0 ** -4 + 2.0 ** -22) + a[:, None] * 2.0 ** -10)
    # powers of two commute with the quantisation
    c2, a2 = O.quantize_rows_e4m3(V * 2.0 ** 5)
    np.testing.assert_array_equal(c2, c)
    np.testing.assert_array_equal(a2, a * np.float32(32.0))


def _silu_slope_max():
    x = np.linspace(-20, 20, 400001)
    s = scipy.special.expit(x)
    return float(np.max(np.abs(s * (1 + x * (1 - s)))))


def test_swiglu_fp8act_within_the_quantisation_bound():
    # the fp8-activation expert against the exact expert on the same bf16
    # input: every output differs by no more than the a-priori bound that the
    # two per-row quantisations (relative 2^-4 each, plus the subnormal floor)
    # and the bf16 rounding of the intermediate (2^-9) allow; a dropped scale,
    # a transposed operand or a missing quantisation step breaks it
    rng = np.random.default_rng(34)
    d, F, R = 64, 96, 40
    Wg = rng.standard_normal((F, d)) / 8
    Wu = rng.standard_normal((F, d)) / 8
    Wd = rng.standard_normal((d, F)) / 10
    U = O.bf16_round(rng.standard_normal((R, d)))
    Y8 = O.swiglu_expert_fp8act(Wg, Wu, Wd, U)
    G, V = U @ Wg.T, U @ Wu.T
    sg = scipy.special.expit(G) * G
    M = sg * V
    Y = M @ Wd.T
    ax = np.max(np.abs(U), axis=1, keepdims=True) / 448 * (1 + 2.0 ** -22)
    ex = np.abs(U) * (2.0 ** -4 + 2.0 ** -22) + ax * 2.0 ** -10
    dG, dV = ex @ np.abs(Wg).T, ex @ np.abs(Wu).T
    L = _silu_slope_max()
    dM1 = L * dG * (np.abs(V) + dV) + np.abs(sg) * dV          # SiLU(G~) V~ - SiLU(G) V
    Mb = (np.abs(M) + dM1) * (1 + 2.0 ** -9)                   # bound on |bf16(M~)|
    am = np.max(Mb, axis=1, keepdims=True) / 448 * (1 + 2.0 ** -22)
    dM = dM1 + (np.abs(M) + dM1) * 2.0 ** -9 + Mb * (2.0 ** -4 + 2.0 ** -22) + am * 2.0 ** -10
    bound = dM @ np.abs(Wd).T + 1e-12 * (np.abs(M) @ np.abs(Wd).T)
    err = np.abs(Y8 - Y)
    assert np.all(err <= bound)
    # and the quantisation is really there: errors of the order of 2^-5
    rel = np.max(err) / np.max(np.abs(Y))
    assert 1e-3 < rel < 0.1


def test_fp8act_layer_with_one_expert_is_the_dense_fp8act_ffn():
    rng = np.random.default_rng(35)
    T, d, F = 24, 32, 64
    vals = _rand_layer(rng, T, d, 1, F)
    r = O.oracle_forward(vals, k=1, eps=1e-6, fp8_act=True)
    x = O.rmsnorm(vals["hidden"], vals["gain"], 1e-6)
    want = O.swiglu_expert_fp8act(vals["w_gate"][0], vals["w_up"][0], vals["w_down"][0], x)
    np.testing.assert_array_equal(r["gate"], 1.0)
    np.testing.assert_allclose(r["out"], want, rtol=0, atol=0)
    # a planted mistake in the plain path would not pass for this one: the
    # fp8 path differs from it by the quantisation
    plain = O.oracle_forward(vals, k=1, eps=1e-6)
    assert np.max(np.abs(plain["out"] - r["out"])) > 1e-4 * np.max(np.abs(want))


def test_swiglu_fp8act_on_exact_fp8_inputs_quantises_the_intermediate():
    # rows that are E4M3 values times 2^j with a +-448 * 2^j entry quantise
    # exactly (scale 2^j), so the whole difference to the exact expert comes
    # from the bf16 rounding and the quantisation of SiLU(G) * V: it is of
    # the order of 2^-5 relative and within that step's bound
    rng = np.random.default_rng(36)
    d, F, R = 64, 96, 32
    Wg = rng.standard_normal((F, d)) / 8
    Wu = rng.standard_normal((F, d)) / 8
    Wd = rng.standard_normal((d, F)) / 10
    codes = rng.integers(0, 0x7F, (R, d)).astype(np.uint8) | (rng.integers(0, 2, (R, d)) << 7).astype(np.uint8)
    codes[:, 0] = 0x7E
    U = O.e4m3_value(codes) * np.exp2(rng.integers(-12, -6, (R, 1)))
    c, a = O.quantize_rows_e4m3(U)
    np.testing.assert_array_equal(O.dequantize_rows(c, a), U)
    M = scipy.special.expit(U @ Wg.T) * (U @ Wg.T) * (U @ Wu.T)
    Y8 = O.swiglu_expert_fp8act(Wg, Wu, Wd, U)
    Mb = np.abs(M) * (1 + 2.0 ** -9)
    am = np.max(Mb, axis=1, keepdims=True) / 448 * (1 + 2.0 ** -22)
    dM = np.abs(M) * 2.0 ** -9 + Mb * (2.0 ** -4 + 2.0 ** -22) + am * 2.0 ** -10
    err = np.abs(Y8 - M @ Wd.T)
    assert np.all(err <= dM @ np.abs(Wd).T + 1e-12 * (np.abs(M) @ np.abs(Wd).T))
    assert np.max(err) > 4e-3 * np.max(np.abs(M @ Wd.T))   # bf16 alone would give ~2^-9


def test_fp8_activation_quantises_the_bf16_value():
    # 1.0625 + 2^-20 rounds to the bf16 value 1.0625, the tie between the
    # E4M3 values 1 and 1.125, which goes to 1 (even); quantising the float64
    # value directly would give 1.125
    X = O.fp8_activation(np.array([[448.0, 1.0625 + 2.0 ** -20, -3.0 - 2.0 ** -12]]))
    np.testing.assert_array_equal(X, [[448.0, 1.0, -3.0]])
    # a scaled row: amax 3 -> scale float32(3/448); 1 -> 144 * scale
    X = O.fp8_activation(np.array([[3.0, 1.0]]))
    a = np.float64(np.float32(3.0) / np.float32(448.0))
    np.testing.assert_array_equal(X, [[448.0 * a, 144.0 * a]])


def test_scale_undecided_marks_rows_near_a_bf16_rounding_boundary():
    # amax 1 + 2^-8 (+-) is the midpoint between the bf16 values 1 and
    # 1 + 2^-7: any perturbation decides it; 1.25 is a bf16 value far from
    # every boundary; a row's other elements do not matter
    V = np.array([[1 + 2.0 ** -8, 0.5], [1.25, -1.0], [-(1 + 2.0 ** -8 + 2.0 ** -20), 0.0],
                  [0.0, 0.0]])
    np.testing.assert_array_equal(O.scale_undecided(V, 1e-4), [True, False, True, False])
    np.testing.assert_array_equal(O.scale_undecided(V, 1e-8), [True, False, False, False])
    # the flag is the only difference the perturbation can make to the scale
    rng = np.random.default_rng(37)
    M = rng.standard_normal((400, 50))
    und = O.scale_undecided(M, 1e-3)
    a0 = O.quantize_rows_e4m3(O.bf16_round(M))[1]
    for f in (1 - 1e-3, 1 + 1e-3):
        a1 = O.quantize_rows_e4m3(O.bf16_round(M * f))[1]
        assert np.all(a1[~und] == a0[~und])
    assert 0 < und.sum() < 400


def test_stack_with_fp8_activations_composes_the_fp8_layers():
    # a two-layer stack (dense, then MoE top-1) with fp8 activations is the
    # residual composition of the fp8-activation layers
    rng = np.random.default_rng(38)
    T, d, F = 12, 32, 64
    dense = _rand_layer(rng, T, d, 1, F)
    moe = _rand_layer(rng, T, d, 3, F)
    H = rng.standard_normal((T, d))
    st = O.stack_forward([dense, moe], H, [1, 1], 1e-6, fp8_act=True)
    h1 = H + O.oracle_forward(dict(dense, hidden=H), k=1, eps=1e-6, fp8_act=True)["out"]
    h2 = h1 + O.oracle_forward(dict(moe, hidden=h1), k=1, eps=1e-6, fp8_act=True)["out"]
    np.testing.assert_array_equal(st["out"], h2)
    plain = O.stack_forward([dense, moe], H, [1, 1], 1e-6)["out"]
    assert np.max(np.abs(plain - st["out"])) > 0
