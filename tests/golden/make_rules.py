"""Write tests/golden/rules.json (the seeded per-head (alpha, beta) rule sets)
and tests/golden/model_rules.json (a seeded rule set for every layer of a
32-layer, 32-head model, in the per-layer rules file format).

The rule sets are inputs of the synthetic workloads, drawn from the discrete
candidate grids the workloads define and rejection-sampled to a target mean
density (mean S_h / N).  Spans are computed by the oracle only; nothing here
touches the HIP path.  Run from the repository root:

    python tests/golden/make_rules.py            # rewrite both files
    python tests/golden/make_rules.py --check    # verify the committed files

Sampling procedure (a reading; the density target has no stated tolerance or
draw order): with numpy's PCG64 seeded by `seed`, each attempt draws every
head in order (alpha index, then beta index) uniformly from its grid, and the
attempt is accepted iff |mean(S) / N - target| <= tol.  The 25 %-density
workload first draws a permutation of its heads; the first half of it are
local heads (beta = 0, alpha from the local grid), the rest elastic heads.
"""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402

ALPHA_GRID = [512 * i for i in range(9)]             # 0, 512, ..., 4096
BETA_GRID = [0.0, 0.25, 0.5, 0.75, 1.0]
LOCAL_ALPHA = [512, 1024, 1536, 2048]                 # fixed-local heads, beta = 0
ELASTIC_BETA = [0.25, 0.5, 0.75, 1.0]

# name -> (seed, n_kv_heads, N, target density, local/elastic split?)
SPECS = {
    "c1": (1001, 32, 8192, 0.50, False),
    "c2": (1002, 32, 16384, 0.50, False),
    "c3": (1003, 40, 32768, 0.25, True),
    "c4": (1004, 8, 65536, 0.50, False),
}
TOL = 0.01
MAX_ATTEMPTS = 2_000_000
# per-layer file: layer l drawn like "c1" (50 % grid at N = 8192) with seed
# MODEL_SEED + l
MODEL_SEED, MODEL_LAYERS, MODEL_HEADS, MODEL_N, MODEL_TARGET = 1100, 32, 32, 8192, 0.50


def draw(seed, heads, n, target, split):
    rng = np.random.Generator(np.random.PCG64(seed))
    for attempt in range(1, MAX_ATTEMPTS + 1):
        local = set()
        if split:
            local = set(int(x) for x in rng.permutation(heads)[: heads // 2])
        alpha, beta = [], []
        for h in range(heads):
            if h in local:
                alpha.append(LOCAL_ALPHA[int(rng.integers(len(LOCAL_ALPHA)))])
                beta.append(0.0)
            elif split:
                alpha.append(ALPHA_GRID[int(rng.integers(len(ALPHA_GRID)))])
                beta.append(ELASTIC_BETA[int(rng.integers(len(ELASTIC_BETA)))])
            else:
                alpha.append(ALPHA_GRID[int(rng.integers(len(ALPHA_GRID)))])
                beta.append(BETA_GRID[int(rng.integers(len(BETA_GRID)))])
        dens = float(oracle.spans(alpha, beta, n).mean()) / n
        if abs(dens - target) <= TOL:
            return {
                "seed": seed, "n_prompt": n, "target_density": target, "tol": TOL,
                "attempts": attempt, "density": dens,
                "local_heads": sorted(local), "alpha": alpha, "beta": beta,
            }
    raise RuntimeError(f"no rule set accepted for seed {seed}")


def build():
    return {name: draw(*spec) for name, spec in SPECS.items()}


def build_model():
    """The per-layer rules document ({"format": "moa-rules", "version": 1, ...})."""
    layers = []
    for layer in range(MODEL_LAYERS):
        r = draw(MODEL_SEED + layer, MODEL_HEADS, MODEL_N, MODEL_TARGET, False)
        layers.append({"alpha": r["alpha"], "beta": r["beta"]})
    return {"format": "moa-rules", "version": 1, "n_kv_heads": MODEL_HEADS, "layers": layers}


def main():
    outputs = {"rules.json": build(), "model_rules.json": build_model()}
    if "--check" in sys.argv:
        bad = False
        for name, doc in outputs.items():
            with open(os.path.join(HERE, name)) as f:
                stored = json.load(f)
            if stored != doc:
                print(f"{name} differs from a fresh draw")
                bad = True
            else:
                print(f"{name} matches")
        sys.exit(1 if bad else 0)
    for name, doc in outputs.items():
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(doc, f, indent=1)
            f.write("\n")
    for name, r in outputs["rules.json"].items():
        print(name, "attempts", r["attempts"], "density", round(r["density"], 4))
    print("model_rules.json:", MODEL_LAYERS, "layers")


if __name__ == "__main__":
    main()
