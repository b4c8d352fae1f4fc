"""Write oracle_regression.json from the oracle alone (fixed dyadic inputs)."""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
import oracle  # noqa: E402


def inputs():
    r = np.arange
    q = ((r(1 * 4 * 1 * 3) % 7) - 3).reshape(1, 4, 1, 3) / 4.0
    k = ((r(1 * 4 * 1 * 3) * 5 % 9) - 4).reshape(1, 4, 1, 3) / 8.0
    v = ((r(1 * 4 * 2 * 2) * 3 % 11) - 5).reshape(1, 4, 2, 2) / 2.0
    alpha = np.array([[[0.5, 0.75], [1.0, 0.25], [0.875, 0.5], [0.625, 1.0]]])
    beta = np.array([[[0.25, 0.5], [0.75, 1.0], [0.5, 0.125], [1.0, 0.375]]])
    s0 = ((r(1 * 2 * 2 * 3) % 5) - 2).reshape(1, 2, 2, 3) / 4.0
    return q, k, v, alpha, beta, s0


def main():
    q, k, v, alpha, beta, s0 = inputs()
    ch = oracle.chain(q[:, :3], k[:, :3], v[:, :3], alpha[:, :3], beta[:, :3], s0, nthreads=1)
    parent = [-1, 0, 0, 1]
    tr = oracle.tree(q, k, v, alpha, beta, s0, parent, nthreads=1)
    out = {"inputs": {n: a.tolist() for n, a in zip(("q", "k", "v", "alpha", "beta", "state0"), inputs())},
           "parent": parent,
           "chain": {"out": ch["out"].tolist(), "final": ch["final"].tolist()},
           "tree": {"out": tr["out"].tolist(), "nodes": tr["nodes"].tolist()}}
    with open(os.path.join(HERE, "oracle_regression.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
