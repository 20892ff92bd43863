"""fp64 CPU oracle of one ZONOS2 MoE feed-forward layer (plain NumPy).

TEST INFRASTRUCTURE ONLY: imported by tests, by the smoke check and by the
bench's CPU-baseline leg; never by the library.

What the layer computes (sources: the ZONOS2 Technical Report as summarised
on the audio-paper-digest page, section "Method overview and architecture",
item 5 (MoE backbone: RMSNorm-normalised input, 16 experts, top-1 routing,
top-2 in the last MoE layer) and item 6 (a per-expert bias vector b_l kept
for load balancing); the mlsanity index page of the report, "Builds on"
list (RMSNorm, GLU variants, auxiliary-loss-free load balancing); the
telknet.cc article, section 2.1 (a router scores experts from the hidden
state and TopK keeps a few of them)):

  O1  x_t   = g * h_t / sqrt(mean_i h_{t,i}^2 + eps)              RMSNorm
  O2  z_t   = W_r x_t ;  s_t = z_t + b                          router, biased scores
  O3  sel_t = the k experts with the largest s_t, in descending order of s,
              an exact tie going to the lower expert index
  O4  gate  : k = 1  -> softmax(z_t)[sel]   (full softmax of the unbiased logits)
              k >= 2 -> softmax of z_t restricted to the selected experts
  O5  c_e   = #{(t, j) : sel_{t,j} = e};  offsets = exclusive prefix sum of c
  O6  assignments a = t*k + j sorted stably by expert:
              gather[p] = token of slot p, scatter[a] = slot of assignment a
  O7  y_p   = W_down[e] (SiLU(W_gate[e] u) * (W_up[e] u)),  u = x_{gather[p]}
  O8  out_t = sum_{j<k} gate_{t,j} * y_{scatter[t*k+j]}       (no residual)
  O9  balancing step: b_e <- b_e + rate * sign(mean_load - c_e)  (between forwards)
  O10 FFN stack: h_{l+1} = h_l + FFN_l(h_l) over the backbone's layers
  O11 depth averaging of the router logits over a stack's MoE layers:
              z~_l = alpha * z~_{l-1} + (1 - alpha) * z_l   (optional)
  O12 fp8 activations (optional): O7 with its two GEMM inputs, u and
              SiLU(W_gate u) * (W_up u), quantised to E4M3 per row with the
              dynamic scale max|row| / 448 (fp8_activation)

Readings where the pages are silent:
the bias only steers selection and never enters a gate; the layer returns
the FFN output without the residual; no capacity limit and no dropped
tokens; no shared expert; a linear router, whose logits a stack may
depth-average across its MoE layers (O11: the state averaged and the rate
are readings, the rate the caller's); "fp8" read as fp8 weights and fp8
activations with per-row dynamic scales (O12, a reading of the cookbook
page's "fp8").

Every floating-point step runs in float64 on the exact values of the inputs
(bf16 inputs are widened exactly).  Nothing is rounded, except where O12
quantises: there the bf16 value of a row is quantised in float32, the
precision in which the device takes that integer decision.
"""

from __future__ import annotations

import numpy as np

# Tokens whose top-k decision has a margin below this (absolute, on the biased
# scores) may legitimately route either way in finite precision.
MARGIN_TOL = 1e-3
# fp8 activations (O12): a row's quantisation scale is a discrete decision
# (the bf16 value of the row's largest element).  Rows whose scale changes
# when every element moves by this much (relative) may legitimately be scaled
# either way: the expert input carries the RMSNorm's float32 rounding; the
# SwiGLU intermediate carries that of the fp8 dot products, which gfx950's
# fp8 MFMA forms to about 5e-5 relative (rms) rather than to float32.
FP8_SCALE_REL_U = 1e-5
FP8_SCALE_REL_M = 3e-4


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# O1 -------------------------------------------------------------------------
def rmsnorm(H, g, eps: float) -> np.ndarray:
    """RMSNorm of each row of H (the normalisation the digest's item 5 applies
    to the backbone input; defined in the RMSNorm paper of the index page's
    "Builds on" list): x = g * h / sqrt(mean(h^2) + eps)."""
    H = _f64(H)
    g = _f64(g)
    ms = np.mean(H * H, axis=-1, keepdims=True)
    return (H / np.sqrt(ms + float(eps))) * g


# O2 -------------------------------------------------------------------------
def router_scores(X, Wr, b):
    """Linear router: logits z = X W_r^T and selection scores s = z + b
    (digest item 6: the per-expert bias b_l; index page: auxiliary-loss-free
    balancing, where the bias shifts which experts are chosen)."""
    z = _f64(X) @ _f64(Wr).T
    s = z + _f64(b)[None, :]
    return z, s


# O3 -------------------------------------------------------------------------
def select_topk(s, k: int):
    """Top-k experts per row of s (digest item 5: top-1, or top-2 in the last
    MoE layer), in descending score order; exact ties go to the lower index.

    Returns (sel [T,k] int32, margin [T] float64) where margin is the smallest
    gap between consecutive sorted scores s_(i) - s_(i+1) for i = 1..min(k, E-1):
    the amount by which the decision (set and order) could flip.
    """
    s = _f64(s)
    T, E = s.shape
    if not 1 <= k <= E:
        raise ValueError("top-k needs 1 <= k <= E")
    # argsort of -s with a stable sort keeps equal scores in index order.
    order = np.argsort(-s, axis=1, kind="stable")
    sel = order[:, :k].astype(np.int32)
    ranked = np.take_along_axis(s, order, axis=1)
    m = min(k, E - 1)
    if m == 0:
        margin = np.full(T, np.inf)
    else:
        margin = np.min(ranked[:, :m] - ranked[:, 1:m + 1], axis=1)
    return sel, margin


# O4 -------------------------------------------------------------------------
def gates(z, sel) -> np.ndarray:
    """Gate weights from the unbiased logits z.

    k = 1: the softmax probability of the chosen expert over all E experts.
    k >= 2: softmax over the chosen experts only (the pair is renormalised).
    """
    z = _f64(z)
    sel = np.asarray(sel)
    k = sel.shape[1]
    if k == 1:
        zmax = np.max(z, axis=1, keepdims=True)
        ez = np.exp(z - zmax)
        p = ez / np.sum(ez, axis=1, keepdims=True)
        return np.take_along_axis(p, sel.astype(np.int64), axis=1)
    zs = np.take_along_axis(z, sel.astype(np.int64), axis=1)
    zmax = np.max(zs, axis=1, keepdims=True)
    ez = np.exp(zs - zmax)
    return ez / np.sum(ez, axis=1, keepdims=True)


# O5 -------------------------------------------------------------------------
def histogram(sel, E: int):
    """Assignments per expert and their exclusive prefix sum (offsets[E] = T*k)."""
    flat = np.asarray(sel).reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    return counts, offsets


# O6 -------------------------------------------------------------------------
def permutation(sel):
    """Stable counting sort of the assignments a = t*k + j by expert.

    gather[p]  = token whose row fills expert-ordered slot p;
    scatter[a] = slot that holds assignment a.
    Within one expert, slots follow increasing a (hence increasing token).
    """
    sel = np.asarray(sel)
    k = sel.shape[1]
    flat = sel.reshape(-1)
    perm = np.argsort(flat, kind="stable")
    gather = (perm // k).astype(np.int32)
    scatter = np.empty_like(perm)
    scatter[perm] = np.arange(perm.size)
    return gather, scatter.astype(np.int32)


# O7 -------------------------------------------------------------------------
def silu(v):
    """SiLU(v) = v / (1 + exp(-v))."""
    v = _f64(v)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def swiglu_expert(Wg, Wu, Wd, U) -> np.ndarray:
    """SwiGLU expert on the rows of U (GLU-variants paper, index page's
    "Builds on" list): y = W_down (SiLU(W_gate u) * (W_up u))."""
    U = _f64(U)
    G = U @ _f64(Wg).T
    V = U @ _f64(Wu).T
    return (silu(G) * V) @ _f64(Wd).T


# O8 -------------------------------------------------------------------------
def combine(Y, gate, scatter, k: int) -> np.ndarray:
    """out_t = sum over j of gate[t, j] * Y[scatter[t*k + j]], in j order."""
    gate = _f64(gate)
    T = gate.shape[0]
    Y = _f64(Y)
    out = np.zeros((T, Y.shape[1]))
    sc = np.asarray(scatter).reshape(T, k)
    for j in range(k):
        out += gate[:, j:j + 1] * Y[sc[:, j]]
    return out


# O9 -------------------------------------------------------------------------
def bias_update(b, counts, rate: float) -> np.ndarray:
    """One step of auxiliary-loss-free load balancing on the router bias.

    The ZONOS2 report keeps a per-expert bias b_l that pushes expert usage
    toward uniform (digest item 6) and builds on the auxiliary-loss-free
    load-balancing paper (title on the index page's "Builds on" list), whose
    step moves each bias by a fixed rate toward balance:

        b_e <- b_e + rate * sign(mean_load - c_e),   mean_load = sum(c) / E

    The sign is the sign of the integer sum(c) - E * c_e (exact, no division);
    sign(0) = 0 leaves a perfectly loaded expert alone.  The bias is stored
    in float32 (the layer's bias type): the exact sum b_e + rate * s_e is
    rounded once to float32.
    """
    c = np.asarray(counts, np.int64)
    E = c.size
    s = np.sign(c.sum() - E * c)
    b32 = np.asarray(b, np.float32)
    r32 = np.float32(rate)
    return (b32.astype(np.float64) + np.float64(r32) * s).astype(np.float32)


# whole layer ----------------------------------------------------------------
def oracle_forward(vals: dict, k: int | None = None, forced_sel=None, tokens=None,
                   eps: float | None = None, z_prev=None, eda_alpha: float | None = None,
                   fp8_act: bool = False) -> dict:
    """Run O1-O8 on exact input values (a dict as from ``synth.values_f32``).

    forced_sel : optional [T,k] expert ids that replace O3's choice (so the
                 expert path can be checked on the device's own routing).
    tokens     : optional token indices; the output is then computed for
                 those rows only (routing and permutation are always full).
    eda_alpha  : optional depth averaging of the logits (O11) with the
                 previous MoE layer's averaged logits z_prev (None: this is
                 the first MoE layer); selection and gates then use them.
    fp8_act    : the experts quantise their activations to E4M3 per row
                 (swiglu_expert_fp8act); the weights in vals are then the
                 dequantised fp8 weights (fp8_weights).
    Returns a dict with x, z, s, sel, margin, gate, counts, offsets, gather,
    scatter and out (float64; rows of ``tokens`` when given).
    """
    cfg = vals.get("cfg")
    if k is None:
        k = cfg.k
    if eps is None:
        eps = cfg.eps
    H = vals["hidden"]
    E = np.asarray(vals["w_router"]).shape[0]
    x = rmsnorm(H, vals["gain"], eps)
    z, s = router_scores(x, vals["w_router"], vals["bias"])
    if eda_alpha is not None:
        z = depth_average(z_prev, z, eda_alpha)
        s = z + _f64(vals["bias"])[None, :]
    sel_o, margin = select_topk(s, k)
    sel = sel_o if forced_sel is None else np.asarray(forced_sel, np.int32).reshape(-1, k)
    gate = gates(z, sel)
    counts, offsets = histogram(sel, E)
    gather, scatter = permutation(sel)

    T = x.shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    need = np.zeros(T * k, bool)
    for j in range(k):
        need[tok * k + j] = True
    slots_needed = np.sort(scatter[need])
    Y = np.zeros((T * k, x.shape[1]))
    undecided = np.zeros(T * k, bool)   # fp8_act: slots whose quantisation scales are undecided
    Wg, Wu, Wd = vals["w_gate"], vals["w_up"], vals["w_down"]
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        ps = slots_needed[(slots_needed >= lo) & (slots_needed < hi)]
        if ps.size == 0:
            continue
        if fp8_act:
            Y[ps], M = swiglu_expert_fp8act(Wg[e], Wu[e], Wd[e], x[gather[ps]], inner=True)
            undecided[ps] = (scale_undecided(x[gather[ps]], FP8_SCALE_REL_U)
                             | scale_undecided(M, FP8_SCALE_REL_M))
        else:
            Y[ps] = swiglu_expert(Wg[e], Wu[e], Wd[e], x[gather[ps]])
    if tokens is None:
        out = combine(Y, gate, scatter, k)
    else:
        sc = scatter.reshape(T, k)[tok]
        out = np.zeros((tok.size, x.shape[1]))
        for j in range(k):
            out += gate[tok, j:j + 1] * Y[sc[:, j]]
    # a token is undecided when one of its assignments is
    scale_tie = undecided[scatter.reshape(T, k)].any(axis=1)[tok]
    return {"x": x, "z": z, "s": s, "sel": sel, "sel_oracle": sel_o, "margin": margin,
            "gate": gate, "counts": counts, "offsets": offsets, "gather": gather,
            "scatter": scatter, "out": out, "tokens": tok, "scale_tie": scale_tie}


# O11 ------------------------------------------------------------------------
def depth_average(z_prev, z, alpha: float) -> np.ndarray:
    """Exponential depth averaging of the router state across layers.

    The ZONOS2 digest (item 5) says the router follows ZAYA1 in smoothing its
    state between layers by exponential depth averaging, and defines neither
    the state nor the rate.  Reading: the state is the router's logits z (the
    only state a linear router has), averaged over the stack's MoE layers in
    order, z~_l = alpha * z~_{l-1} + (1 - alpha) * z_l, with z~ = z at the
    first MoE layer; alpha in [0, 1) is the caller's (alpha = 0: no
    smoothing).  The layer's bias b_l is added after the averaging (it steers
    the choice only), and the gates come from z~.  The average runs per
    (token, expert), so it is defined only between layers with the same
    experts: logits of different widths raise ValueError."""
    if z_prev is None:
        return _f64(z)
    if np.shape(z_prev) != np.shape(z):
        raise ValueError(f"depth averaging needs logits of one shape, got {np.shape(z_prev)} "
                         f"and {np.shape(z)}")
    return alpha * _f64(z_prev) + (1.0 - alpha) * _f64(z)


# O10 ------------------------------------------------------------------------
def stack_forward(layer_vals: list, H, ks: list, eps: float, forced_sels=None,
                  eda_alpha: float | None = None, fp8_act: bool = False) -> dict:
    """The FFN half of a stack of backbone layers with residual adds (digest
    item 5: a 28-layer stack whose first three and last layers are dense and
    whose middle layers are MoE, the last MoE layer top-2):

        h_0 = H;   h_{l+1} = h_l + FFN_l(h_l)

    FFN_l is the layer of O1-O8 (a dense layer is its one-expert case).
    Everything stays in float64; forced_sels[l] optionally replaces layer l's
    routing choice.  eda_alpha: the MoE layers' (more than one expert) logits
    are depth-averaged (O11) in stack order; dense layers carry no router
    state.  fp8_act: every layer quantises its expert activations (O12).
    Returns the final h and every layer's routing (the forced one
    where given), the oracle's own choice and the top-k margins.
    """
    h = _f64(H)
    sels, own, margins = [], [], []
    if eda_alpha is not None:
        widths = {np.asarray(v["w_router"]).shape[0] for v in layer_vals}
        if len(widths - {1}) > 1:
            raise ValueError(f"depth averaging needs one expert count over the MoE layers, "
                             f"got {sorted(widths - {1})}")
    zp = None
    for l, vals in enumerate(layer_vals):
        v = dict(vals, hidden=h)
        fs = None if forced_sels is None else forced_sels[l]
        moe = np.asarray(vals["w_router"]).shape[0] > 1
        if eda_alpha is not None and moe:
            r = oracle_forward(v, k=ks[l], forced_sel=fs, eps=eps, z_prev=zp, eda_alpha=eda_alpha,
                               fp8_act=fp8_act)
            zp = r["z"]
        else:
            r = oracle_forward(v, k=ks[l], forced_sel=fs, eps=eps, fp8_act=fp8_act)
        h = h + r["out"]
        sels.append(r["sel"])
        own.append(r["sel_oracle"])
        margins.append(r["margin"])
    return {"out": h, "sel": sels, "sel_oracle": own, "margin": margins}


# fp8 expert weights ------------------------------------------------------------
def e4m3_value(codes) -> np.ndarray:
    """Values of OCP FP8 E4M3 byte codes (sign, 4 exponent bits with bias 7,
    3 mantissa bits; exponent 0 is subnormal, m * 2^-9; S.1111.111 is NaN; no
    infinities), as float64."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


def fp8_weights(codes, scale) -> np.ndarray:
    """Expert weights stored as E4M3 codes with one float32 scale per output
    row: W[e, r, :] = value(codes[e, r, :]) * scale[e, r] (exact in float64)."""
    return e4m3_value(codes) * np.asarray(scale, np.float64)[..., None]


# fp8 activations ----------------------------------------------------------------
# The SGLang-Omni cookbook page ("Benchmark Results") serves ZONOS2 with "fp8"
# and says nothing more.  Read as fp8 weights AND fp8 activations (both
# operands of the expert GEMMs in E4M3): the expert input of each routed row
# and the SwiGLU intermediate of each row are quantised on the fly with one
# float32 scale per row, scale = max|row| / 448 (dynamic per-token scales);
# the weights keep their per-output-row scales (fp8_weights).  The device
# stores both quantised vectors in bf16 before quantising them (the expert
# input as bf16 rows, the intermediate as bf16 SwiGLU outputs), and a
# quantisation decides integer codes, so this reading quantises the bf16
# value of each vector and takes the scale, its reciprocal and the product
# in float32, as the device does.  Everything else stays in float64.

def bf16_round(v) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (8 significant bits,
    float32's exponent range), ties to even; returned as float64.  Zeros,
    infinities and NaN pass through."""
    v = _f64(v)
    e = np.maximum(np.frexp(v)[1], -125)  # |v| in [2^(e-1), 2^e); bf16 subnormals below 2^-126
    r = np.ldexp(np.rint(np.ldexp(v, 8 - e)), e - 8)   # 8 significant bits, spacing 2^(e-8)
    return np.where(np.isfinite(v), r, v)


_E4M3_POS = None


def _e4m3_table():
    """The 127 finite non-negative E4M3 values in increasing order with their
    codes (code 0x00 .. 0x7e: the order of the codes is the order of the
    values)."""
    global _E4M3_POS
    if _E4M3_POS is None:
        codes = np.arange(0x7F, dtype=np.uint8)
        _E4M3_POS = (e4m3_value(codes), codes)
    return _E4M3_POS


def e4m3_encode(v) -> np.ndarray:
    """E4M3 code of the nearest E4M3 value to each float64 v, ties to the even
    code (the one whose last mantissa bit is 0), saturating at +-448 (the
    largest finite value); the sign bit follows v's sign (-0.0 -> 0x80).
    NaN gives 0x7f."""
    v = _f64(v)
    vals, codes = _e4m3_table()
    a = np.minimum(np.abs(v), 448.0)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 1, vals.size - 1)
    lo = hi - 1                            # vals[lo] <= a <= vals[hi]
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (codes[hi] % 2 == 0))
    c = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    c = np.where(a == 0.0, 0, c).astype(np.uint8)
    c = np.where(np.signbit(v), c | 0x80, c).astype(np.uint8)
    return np.where(np.isnan(v), 0x7F, c).astype(np.uint8)


def quantize_rows_e4m3(V):
    """Dynamic per-row E4M3 quantisation of V [R, K] (values that float32
    holds exactly; the layer passes bf16 values): with amax the largest |v| of
    a row, the row's scale is a = float32(amax / 448), its reciprocal
    r = float32(1 / a) (both correctly rounded divisions in float32), and its
    codes are e4m3_encode(float32(v * r)).  A row of zeros gets a = 0 and all
    codes 0.  Returns (codes uint8 [R, K], a float32 [R]); the row's values
    are then a * e4m3_value(codes)."""
    V32 = np.asarray(V, np.float64).astype(np.float32)
    if not np.array_equal(V32.astype(np.float64), _f64(V)):
        raise ValueError("quantize_rows_e4m3 takes values that float32 holds exactly")
    amax = np.max(np.abs(V32), axis=-1)
    a = (amax / np.float32(448.0)).astype(np.float32)
    safe = np.where(a > 0, a, np.float32(1.0)).astype(np.float32)
    r = (np.float32(1.0) / safe).astype(np.float32)
    q = (V32 * r[..., None]).astype(np.float32)
    codes = e4m3_encode(q.astype(np.float64))
    codes = np.where((a > 0)[..., None], codes, 0).astype(np.uint8)
    return codes, a


def dequantize_rows(codes, a) -> np.ndarray:
    """a[r] * value(codes[r, :]) in float64 (exact)."""
    return e4m3_value(codes) * np.asarray(a, np.float64)[..., None]


def fp8_activation(U) -> np.ndarray:
    """What an expert GEMM multiplies under fp8 activations: each row of U
    rounded to bf16, quantised per row (quantize_rows_e4m3) and dequantised,
    in float64."""
    return dequantize_rows(*quantize_rows_e4m3(bf16_round(U)))


def swiglu_expert_fp8act(Wg, Wu, Wd, U, inner: bool = False):
    """O7 with fp8 activations (the reading above): G and V are the exact
    products of fp8_activation(u) with the (dequantised fp8) weights, and
    y = W_down fp8_activation(SiLU(G) * V).  Float64 throughout, apart from
    the bf16 roundings and the float32 quantisation steps the reading names.
    inner=True also returns the intermediate SiLU(G) * V before its rounding."""
    X = fp8_activation(U)
    G = X @ _f64(Wg).T
    V = X @ _f64(Wu).T
    M = silu(G) * V
    Y = fp8_activation(M) @ _f64(Wd).T
    return (Y, M) if inner else Y


def scale_undecided(V, rel: float) -> np.ndarray:
    """Rows of V whose fp8 quantisation scale is not fixed under a relative
    change of at most `rel` in each element: the scale is amax / 448 with
    amax the largest |bf16(v)|, and bf16 rounding is monotone, so the row is
    undecided when bf16(max|v| (1 - rel)) != bf16(max|v| (1 + rel))."""
    amax = np.max(np.abs(_f64(V)), axis=-1)
    return bf16_round(amax * (1.0 - rel)) != bf16_round(amax * (1.0 + rel))
