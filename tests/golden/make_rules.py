"""Write tests/golden/rules.json: the seeded per-head (alpha, beta) rule sets.

The rule sets are inputs of the synthetic workloads, drawn from the discrete
candidate grids the workloads define and rejection-sampled to a target mean
density (mean S_h / N).  Spans are computed by the oracle only; nothing here
touches the HIP path.  Run from the repository root:

    python tests/golden/make_rules.py            # rewrite rules.json
    python tests/golden/make_rules.py --check    # verify the committed file

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


def main():
    path = os.path.join(HERE, "rules.json")
    rules = build()
    if "--check" in sys.argv:
        with open(path) as f:
            stored = json.load(f)
        if stored != rules:
            print("rules.json differs from a fresh draw")
            sys.exit(1)
        print("rules.json matches")
        return
    with open(path, "w") as f:
        json.dump(rules, f, indent=1)
        f.write("\n")
    for name, r in rules.items():
        print(name, "attempts", r["attempts"], "density", round(r["density"], 4))


if __name__ == "__main__":
    main()
