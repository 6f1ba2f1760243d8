"""Write zipf_bias_k25.txt: the router correction bias of the skewed-routing
exact-mode workload (T=4096, 384 experts, top-8, Zipf(1.1) popularity over the
live experts, 20% of the experts dead).

Only the oracle's router is called.  Steps:
  1. a seeded permutation of the experts; its first round(0.2 E) are dead and
     get bias -4 (a live biased score is above -2 > -3, so a dead expert is
     never selected);
  2. the live experts get ranks r = 1..E_live in permutation order; the target
     count of rank r is the expected number of tokens choosing it when each
     token draws k distinct live experts without replacement with probability
     proportional to r^-1.1 (Monte Carlo, Gumbel top-k);
  3. the live biases start at 0 and are refit 300 times on a separate
     calibration batch: b_r <- b_r + clip(0.5 ln((c_r + 0.5) / (c^_r + 0.5)), +-0.05), c^ being
     the counts the oracle's selection gives with the current bias; after each
     step the live biases are re-centred on mean 0 (only differences matter,
     the total count is fixed at T k) and clipped to [-2, 2].
The sigmoid scores do not depend on the bias, so they are computed once.

Usage: python tests/golden/make_zipf_bias.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from int4_routed_expert_moe_amd import synthetic  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_bias_k25.txt")
ZIPF_S = 1.1
DEAD_FRAC = 0.2
ITERS = 300


def main():
    cfg = dict(synthetic.WORKLOADS[4])
    E, k, T = cfg["E"], cfg["k"], cfg["T"]
    w, _ = synthetic.gen_router(cfg)
    x_cal = synthetic.calibration_x(cfg, T)
    _, _, _, scores = oracle.route(x_cal, w, np.zeros(E, np.float32), k, True, return_scores=True)

    g = synthetic.rng(cfg["layer_seed"], synthetic.T_ZIPF_CAL, 1)
    perm = g.permutation(E)
    n_dead = int(round(DEAD_FRAC * E))
    dead, live = perm[:n_dead], perm[n_dead:]
    n_live = len(live)
    p = np.arange(1, n_live + 1, dtype=np.float64) ** -ZIPF_S
    p /= p.sum()

    # expected counts per live rank under k draws without replacement
    counts = np.zeros(n_live)
    reps = 25
    for rep in range(reps):
        gum = g.gumbel(size=(T, n_live))
        pick = np.argpartition(-(np.log(p)[None, :] + gum), k, axis=1)[:, :k]
        counts += np.bincount(pick.ravel(), minlength=n_live)
    target = counts / reps

    bias = np.zeros(E, np.float32)
    bias[dead] = -4.0
    for it in range(ITERS):
        idx, _ = oracle.topk_from_scores(scores, bias, k, True)
        got = np.bincount(idx.ravel(), minlength=E)[live].astype(np.float64)
        step = np.clip(0.5 * np.log((target + 0.5) / (got + 0.5)), -0.05, 0.05)
        b = bias[live].astype(np.float64) + step
        bias[live] = np.clip(b - b.mean(), -2.0, 2.0).astype(np.float32)

    idx, _ = oracle.topk_from_scores(scores, bias, k, True)
    got = np.bincount(idx.ravel(), minlength=E)
    assert got[dead].sum() == 0
    r = np.arange(1, n_live + 1)
    live_got = got[live]
    m = live_got > 0
    slope = np.polyfit(np.log(r[m]), np.log(live_got[m]), 1)[0]
    with open(OUT, "w") as f:
        f.write("# router correction bias (float32, one hex float per expert) of the skewed-routing\n")
        f.write("# exact-mode workload; written by make_zipf_bias.py using only the oracle router\n")
        f.write(f"# dead experts: {n_dead} (bias -4); live: {n_live}; target Zipf s={ZIPF_S}, "
                f"k={k} draws without replacement\n")
        f.write(f"# calibration batch T={T}: max count {int(live_got.max())}, min live count "
                f"{int(live_got.min())}, fitted log-log slope {slope:.3f}\n")
        for v in bias:
            f.write(float(v).hex() + "\n")
    print(f"wrote {OUT}: slope {slope:.3f}, max {live_got.max()}, head {live_got[:8].tolist()}")


if __name__ == "__main__":
    main()
