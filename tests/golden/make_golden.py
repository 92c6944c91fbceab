"""Writes the regression fixtures in this folder from the seeded generators and
the CPU oracle only (nothing here comes from the HIP path):

  input_manifest.json   SHA-256 of a fixed cut of every configured layer's
                        inputs (64 tokens x all columns of X, 32 rows of W),
                        freezing the generator recipe
  oracle_config1.json   the oracle's saliency digest, 20 losses and chosen
                        index for the 128x512->512 configuration

Run from the repository root: python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import awq_oracle as O  # noqa: E402

MANIFEST_CUT = dict(n_tokens=64, out_features=32)


def manifest():
    out = {}
    for key, cfg in synth.CONFIGS.items():
        for li, spec in enumerate(cfg.layers):
            _, X, W = synth.make_layer(key, li, **MANIFEST_CUT)
            out[f"{key}:{spec.name}"] = synth.digest(X, W)
    return out


def oracle_config1():
    _, X, W = synth.make_layer(1, 0)
    sal = O.act_stats(X)
    res = O.search_layer(X, W, sal)
    return {"sal_digest": synth.digest(sal), "losses": [float(v) for v in res.losses],
            "best": int(res.best)}


if __name__ == "__main__":
    json.dump({"cut": MANIFEST_CUT, "digests": manifest()},
              open(os.path.join(HERE, "input_manifest.json"), "w"), indent=1)
    json.dump(oracle_config1(), open(os.path.join(HERE, "oracle_config1.json"), "w"), indent=1)
    print("written")
