"""Write tiny_layer_oracle.json: the oracle's result for the tiny layer, one
seeded token (a regression record of the oracle, not a pin).  Calls only the
oracle and the seeded input generator."""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import moe_inputs as mi  # noqa: E402
import oracle  # noqa: E402


def record():
    cfg = mi.TINY
    w = mi.gen_layer_weights(cfg, 0)
    x, resid = mi.gen_tokens(cfg, 0, 1)
    r = oracle.layer(cfg, w, x, resid)
    return {
        "workload": cfg.name, "layer": 0, "token": 0,
        "ids": r["route"]["ids"][0].tolist(),
        "scores": [float(v) for v in r["route"]["scores"][0]],
        "logits": [float(v) for v in r["route"]["logits"][0]],
        "out_first16": [float(v) for v in r["out"][0][:16]],
        "out_sum": float(r["out"][0].sum()),
        "act_sum": float(r["ffn"]["act"][0].sum()),
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_layer_oracle.json"), "w") as f:
        json.dump(record(), f, indent=1)
        f.write("\n")
