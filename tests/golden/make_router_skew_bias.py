"""Writes router_skew_bias.json: the router bias beta for the skewed-routing layer.

Reading taken for "router logits biased so that 20% of experts take 80% of
picks": the hot set is the first ceil(0.2 E) experts of a seeded permutation
(synth.recipe.router_bias); every hot expert gets the same logit bias beta and
the others none.  beta is found by bisection (to 1e-4) so that, over 4096
seeded tokens whose post-attention hidden state is N(0, 1), the hot set takes
0.80 of all top-k picks.  Logits come from the CPU oracle's router (the layer's
own RMSNorm-2 gain and W_R); only the constant bias is added here.

Run: python tests/golden/make_router_skew_bias.py
"""
import json
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402
from synth import recipe  # noqa: E402
from synth.configs import C4, HOT_FRACTION, HOT_SHARE_TARGET  # noqa: E402

N_TOKENS = 4096
SEED = 0
LAYER = 0


def hot_share(logits, hot_mask, beta, k):
    lg = logits + np.float32(beta) * hot_mask.astype(np.float32)
    # top-k by value, ties to the lower index (stable sort of the negated logits)
    sel = np.argsort(-lg, axis=1, kind="stable")[:, :k]
    return hot_mask[sel].mean()


def main():
    s = C4
    w = recipe.layer_weights_host(s.with_(routing="uniform"), SEED, LAYER, experts=[])
    Hp = synth.normal_f32((N_TOKENS, s.d), SEED, synth.stream_id("H", 0xFFFF, 0), 1.0)
    _, logits, _, _ = oracle.router(s, w, Hp)
    hot = synth.permutation(s.E, SEED, synth.stream_id("hot_perm", LAYER))[: int(math.ceil(HOT_FRACTION * s.E))]
    mask = np.zeros(s.E, bool)
    mask[hot] = True
    lo, hi = 0.0, 16.0
    while hi - lo > 1e-4:
        mid = 0.5 * (lo + hi)
        if hot_share(logits, mask, mid, s.top_k) < HOT_SHARE_TARGET:
            lo = mid
        else:
            hi = mid
    beta = float(np.float32(hi))
    share = float(hot_share(logits, mask, beta, s.top_k))
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "router_skew_bias.json")
    table = json.load(open(path)) if os.path.exists(path) else {}
    table["E%d_k%d_d%d" % (s.E, s.top_k, s.d)] = {
        "beta": beta, "realized_hot_share": share, "hot_experts": int(mask.sum()),
        "tokens": N_TOKENS, "seed": SEED, "layer": LAYER,
        "written_by": "tests/golden/make_router_skew_bias.py (CPU oracle router)",
    }
    json.dump(table, open(path, "w"), indent=2, sort_keys=True)
    print("beta=%.6f hot share=%.4f" % (beta, share))


if __name__ == "__main__":
    main()
