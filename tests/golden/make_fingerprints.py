"""Writes fingerprints.json: sha256 prefixes of the seeded inputs (seed 0) of the
small workloads.  Calls only the input generator; rerun only when the
generator's recipe changes on purpose."""
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import workloads as wl  # noqa: E402


def fingerprints():
    out = {}
    w = wl.CONFIGS["tiny_ag"]["make"](0)
    out["tiny_ag"] = {"B": wl.fingerprint(w.B), "order": w.order.tolist(),
                      "shards": [wl.fingerprint(s) for s in w.shards]}
    r = wl.make_rs(64, 32, 48, 4, seed=0)
    out["rs_small"] = {"A": wl.fingerprint(r.A), "B": wl.fingerprint(r.B),
                       "P": [wl.fingerprint(p) for p in r.partials]}
    m = wl.make_moe(64, 16, 32, 4, 8, 8, seed=0, block_tokens=16)
    out["moe_small"] = {"X": wl.fingerprint(m.X), "logits": wl.fingerprint(m.logits),
                        "W0": wl.fingerprint(m.W[0]), "order": m.order.tolist()}
    g = wl.make_ring(2, 16, 128, 3, seed=0)
    out["ring_small"] = {"Q": wl.fingerprint(g.Q), "K": [wl.fingerprint(k) for k in g.K],
                         "V": [wl.fingerprint(v) for v in g.V], "order": g.order.tolist()}
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fingerprints.json")
    with open(path, "w") as f:
        json.dump(fingerprints(), f, indent=1, sort_keys=True)
    print("wrote", path)
