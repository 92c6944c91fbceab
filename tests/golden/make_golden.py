"""Writes the regression fixtures in this folder from the seeded generators and
the CPU oracle only (nothing here comes from the HIP path):

  input_manifest.json     SHA-256 of a fixed cut of every configured layer's
                          inputs (64 tokens x all columns of X, 32 rows of W),
                          freezing the generator recipe
  oracle_config1.json     the oracle's saliency digest, 20 losses and chosen
                          index for the 128x512->512 configuration
  oracle_full_layers.json (with --full) the oracle's 20 losses and chosen
                          index for every full-size layer of the 512-token
                          and larger configurations, with the digests of the
                          layer's X, W and saliency

Run from the repository root:
    python tests/golden/make_golden.py            # the small fixtures
    python tests/golden/make_golden.py --full     # the full-size layers (tens
                                                  # of minutes on 8 cores)
"""
import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

MANIFEST_CUT = dict(n_tokens=64, out_features=32)
FULL_CONFIGS = (2, 3, 4, 5)
FULL_FILE = os.path.join(HERE, "oracle_full_layers.json")
ROW_CHUNK = 2048


def manifest():
    import synth
    out = {}
    for key, cfg in synth.CONFIGS.items():
        for li, spec in enumerate(cfg.layers):
            _, X, W = synth.make_layer(key, li, **MANIFEST_CUT)
            out[f"{key}:{spec.name}"] = synth.digest(X, W)
    return out


def oracle_config1():
    import synth
    from oracle import awq_oracle as O
    _, X, W = synth.make_layer(1, 0)
    sal = O.act_stats(X)
    res = O.search_layer(X, W, sal)
    return {"sal_digest": synth.digest(sal), "losses": [float(v) for v in res.losses],
            "best": int(res.best)}


def full_layer(job):
    """One full-size layer: the oracle's saliency, then its whole 20-point search
    (output rows in blocks of ROW_CHUNK)."""
    key, li = job
    import synth
    from oracle import awq_oracle as O
    t0 = time.time()
    spec, X, W = synth.make_layer(key, li)
    sal = O.act_stats(X)
    res = O.search_layer(X, W, sal, row_chunk=ROW_CHUNK)
    rec = {
        "config": key, "layer": li, "name": spec.name,
        "shape": [spec.n_tokens, spec.in_features, spec.out_features],
        "x_digest": synth.digest(X), "w_digest": synth.digest(W),
        "sal_digest": synth.digest(sal),
        "losses": [float(v) for v in res.losses], "best": int(res.best),
    }
    print(f"  {key}:{spec.name} {spec.n_tokens}x{spec.in_features}->{spec.out_features} "
          f"best {res.best} in {time.time() - t0:.0f} s", flush=True)
    return f"{key}:{li}", rec


def full_layers(workers: int):
    import multiprocessing as mp
    import synth
    done = json.load(open(FULL_FILE)) if os.path.exists(FULL_FILE) else {"layers": {}}
    jobs = [(k, li) for k in FULL_CONFIGS for li in range(len(synth.CONFIGS[k].layers))
            if f"{k}:{li}" not in done["layers"]]
    # the largest layers first, so the pool's tail is short
    jobs.sort(key=lambda j: -synth.CONFIGS[j[0]].layers[j[1]].out_features *
              synth.CONFIGS[j[0]].layers[j[1]].in_features * synth.CONFIGS[j[0]].layers[j[1]].n_tokens)
    done["row_chunk"] = ROW_CHUNK
    done["note"] = ("oracle losses (binary64 mean squared output error per grid point) and "
                    "first-minimum index for each full-size configured layer")
    with mp.get_context("spawn").Pool(workers) as pool:
        for name, rec in pool.imap_unordered(full_layer, jobs):
            done["layers"][name] = rec
            json.dump(done, open(FULL_FILE, "w"), indent=1, sort_keys=True)
    return done


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--full", action="store_true", help="write oracle_full_layers.json")
    ap.add_argument("--workers", type=int, default=3)
    a = ap.parse_args()
    if a.full:
        full_layers(a.workers)
    else:
        json.dump({"cut": MANIFEST_CUT, "digests": manifest()},
                  open(os.path.join(HERE, "input_manifest.json"), "w"), indent=1)
        json.dump(oracle_config1(), open(os.path.join(HERE, "oracle_config1.json"), "w"),
                  indent=1)
    print("written")
