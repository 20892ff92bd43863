"""Write the router bias of the skewed-load workload (T=16384, 16 experts).

TEST INFRASTRUCTURE: runs the oracle's RMSNorm and router (O1-O2) on the
workload's seeded hidden states and router weights, then searches for a bias b
such that top-1 selection on s = z + b gives expert shares that follow
Zipf(1.2) over 15 ranks (37% on the hottest expert), with the remaining expert
held at a bias of -1e4 so that it receives no token.  Ranks are assigned to
expert ids by a seeded permutation.

The bias steers selection only (digest of the ZONOS2 Technical Report, item 6:
a per-expert bias b_l for balancing; index page: auxiliary-loss-free
balancing), so this is exactly how a trained b_l shapes the load.

Search: repeated multiplicative correction of the shares in log space,
b_e += lr * (log target_e - log share_e), until every non-empty share is
within 0.5% (relative) of its target.  The result is written as exact float32
hex values to synth/zipf_bias_T16384_d2048_E16.txt.

Usage: python -m oracle.calibrate_zipf_bias
"""

from __future__ import annotations

import os
import sys

import numpy as np

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

from oracle.moe_oracle import rmsnorm, router_scores  # noqa: E402
from synth.configs import WORKLOADS, ZIPF_S, ZIPF_RANKS, ZIPF_EMPTY_BIAS  # noqa: E402
from synth import gen  # noqa: E402


def zipf_targets(E: int) -> np.ndarray:
    """Target share per expert id: Zipf(s) over ZIPF_RANKS ranks, 0 for the rest."""
    ranks = np.arange(1, ZIPF_RANKS + 1, dtype=np.float64)
    w = ranks ** (-ZIPF_S)
    w /= w.sum()
    perm = gen.zipf_rank_permutation(E)
    tgt = np.zeros(E)
    tgt[perm[:ZIPF_RANKS]] = w
    return tgt


def top1_shares(s: np.ndarray) -> np.ndarray:
    sel = np.argmax(s, axis=1)  # first maximum = lower index on ties
    return np.bincount(sel, minlength=s.shape[1]) / s.shape[0]


def calibrate(z: np.ndarray, tgt: np.ndarray, tol: float = 0.005, iters: int = 5000):
    E = z.shape[1]
    live = tgt > 0
    b = np.zeros(E)
    b[~live] = ZIPF_EMPTY_BIAS
    b[live] = np.log(tgt[live])  # a good first guess when logits are exchangeable
    lr = 0.5
    best = None
    for it in range(iters):
        b32 = b.astype(np.float32).astype(np.float64)
        sh = top1_shares(z + b32[None, :])
        rel = np.abs(sh[live] - tgt[live]) / tgt[live]
        if best is None or rel.max() < best[0]:
            best = (rel.max(), b32.copy(), sh.copy(), it)
        if rel.max() < tol:
            break
        b[live] += lr * (np.log(tgt[live]) - np.log(np.maximum(sh[live], 0.25 / z.shape[0])))
        if it % 200 == 199:
            lr *= 0.7
    return best


def main():
    cfg = WORKLOADS[4]
    E = cfg.E
    inp = gen.make_inputs(cfg.cid) if os.path.exists(gen.ZIPF_BIAS_FILE) else None
    # The bias file may not exist yet: build the other inputs directly.
    w = gen.family_weights(cfg)
    fam = gen._FAMILY_KEY[cfg.family]
    hid = gen._store(gen._normal((fam, gen._TENSOR_KEY["hidden"], cfg.cid, cfg.T, 0),
                                 (cfg.T, cfg.d), 1.0), cfg.dtype)
    if inp is not None:
        assert np.array_equal(inp["hidden"], hid)
    H = gen.bf16_bits_to_f32(hid)
    g = gen.bf16_bits_to_f32(w["gain"])
    Wr = gen.bf16_bits_to_f32(w["w_router"])
    x = rmsnorm(H, g, cfg.eps)
    z, _ = router_scores(x, Wr, np.zeros(E))
    tgt = zipf_targets(E)
    err, b32, sh, it = calibrate(z, tgt)
    print(f"calibrated in {it} iterations, max relative share error {err:.4%}")
    for e in range(E):
        print(f"  expert {e:2d}: target {tgt[e]:.4f} share {sh[e]:.4f} bias {b32[e]:+.6f}")
    if err > 0.02:
        raise SystemExit("calibration did not reach 2% relative share error")
    with open(gen.ZIPF_BIAS_FILE, "w") as f:
        f.write("# Router bias of the skewed-load workload (T=16384, d=2048, 16 experts, top-1).\n")
        f.write("# Written by oracle/calibrate_zipf_bias.py; float32 values as hex, one per expert.\n")
        f.write(f"# Zipf({ZIPF_S}) over {ZIPF_RANKS} ranks; max relative share error {err:.5f}.\n")
        for e in range(E):
            f.write(f"{float(np.float32(b32[e])).hex()}  # expert {e}: target share "
                    f"{tgt[e]:.6f}, oracle share {sh[e]:.6f}\n")
    print("wrote", gen.ZIPF_BIAS_FILE)


if __name__ == "__main__":
    main()
