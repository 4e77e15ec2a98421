"""Writes skewed_afmoe_T8192.json: the parameters of the skewed-routing workload.

The workload asks for 10% of the experts to receive about 60% of the routed
assignments, plus a few percent of tokens with exactly tied selection keys.
The lever used is the one the routing rule provides for this purpose, the
selection-only expert bias (mlxcel issue #845 "Routing detail"): the hot
experts' bias is raised by delta, found by bisection on the oracle's routing so
that the hot share is 60% (+-1%). Returned weights are unaffected, since they
come from the unbiased scores. The tie: expert c gets expert a's router row
and bias, so both keys are equal for every token; the cold pair whose tie
straddles the top-k boundary for the fraction of tokens closest to 5% is used.

Only the oracle and the seeded generator are called here. Run:
    python tests/golden/make_skew_fixture.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import moe_oracle as O  # noqa: E402
from workloads import synth  # noqa: E402

NAME = "skewed_afmoe_T8192"
TARGET_SHARE = 0.60


def hot_share(idx, hot):
    return float(np.isin(idx, hot).mean())


def main():
    cfg = synth.config(NAME)
    inp = synth.generate(cfg, experts=False, apply_skew=False)
    E, k = cfg["num_experts"], cfg["num_experts_per_tok"]
    L = O.router_logits(inp.x, inp.w_router)
    s = O.scores(L, "sigmoid")
    hot = synth.hot_set(cfg)
    b0 = inp.expert_bias.astype(np.float32)

    def biased(delta, pair=None):
        b = b0.copy()
        b[hot] = (b[hot] + np.float32(delta)).astype(np.float32)
        if pair is not None:
            b[pair[1]] = b[pair[0]]
        return b

    def tied_scores(pair):
        if pair is None:
            return s
        st = s.copy()
        st[:, pair[1]] = st[:, pair[0]]
        return st

    def bisect(pair):
        st = tied_scores(pair)
        lo, hi = 0.0, 4.0
        for _ in range(60):
            mid = 0.5 * (lo + hi)
            if hot_share(O.select_topk(O.selection_keys(st, biased(mid, pair)), k), hot) < TARGET_SHARE:
                lo = mid
            else:
                hi = mid
        return float(np.float32(hi))

    delta = bisect(None)
    b = biased(delta)

    # tie pair among the cold experts
    cold = [e for e in range(E) if e not in set(hot.tolist())]
    best = None
    for ai, a in enumerate(cold):
        for c in cold[ai + 1:]:
            key = O.selection_keys(s, b)
            key[:, c] = key[:, a]
            idx = O.select_topk(key, k)
            has_a = (idx == a).any(1)
            has_c = (idx == c).any(1)
            rate = float((has_a ^ has_c).mean())
            if best is None or abs(rate - 0.05) < abs(best[2] - 0.05):
                best = (a, c, rate)
    a, c, _ = best
    # the tie moves a little load between cold experts: bisect again with it
    delta = bisect((a, c))

    # final statistics with both modifications applied
    bf = biased(delta, (a, c))
    Lf = L.copy()
    Lf[:, c] = Lf[:, a]
    idx = O.select_topk(O.selection_keys(O.scores(Lf, "sigmoid"), bf), k)
    rate = float(((idx == a).any(1) ^ (idx == c).any(1)).mean())
    counts = np.bincount(idx.reshape(-1), minlength=E)
    out = dict(
        workload=NAME,
        written_by="tests/golden/make_skew_fixture.py (oracle routing only)",
        hot_experts=hot.tolist(),
        delta=delta,
        tie_pair=[int(a), int(c)],
        tie_straddle_rate=rate,
        hot_share=hot_share(idx, hot),
        empty_experts=int((counts == 0).sum()),
        max_load=int(counts.max()),
        mean_load=float(counts.mean()),
    )
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), NAME + ".json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
