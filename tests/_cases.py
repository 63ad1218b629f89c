"""Shared test inputs: the golden NN fixture and small adversarial clouds.

Holds no method arithmetic: only parsing and seeded point generation.
"""

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_nn_cases(path=os.path.join(GOLDEN, "nn_cases.txt")):
    """Parse the hand-derived NN fixture into [(target, queries, idx, d2)]."""
    sets, T, Q, I, D = [], [], [], [], []

    def flush():
        if T:
            sets.append((np.array(T, np.float32), np.array(Q, np.float32).reshape(-1, 3),
                         np.array(I, np.int32), np.array(D, np.float32)))

    def num(s):
        s = s.strip()
        return float.fromhex(s) if "0x" in s.lower() else float(s)

    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        tok = line.split()
        if tok[0] == "RESET":
            flush()
            T, Q, I, D = [], [], [], []
        elif tok[0] == "T":
            T.append([num(x) for x in tok[1:4]])
        elif tok[0] == "Q":
            Q.append([num(x) for x in tok[1:4]])
            I.append(int(tok[4]))
            D.append(num(tok[5]))
    flush()
    return sets


def adversarial_clouds(seed=7):
    """(name, target, queries) triples that stress ties, duplicates and degeneracy."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    # integer grid: exact ties everywhere; queries on half-integers and on grid points
    g = np.stack(np.meshgrid(np.arange(6), np.arange(5), np.arange(4), indexing="ij"), -1).reshape(-1, 3)
    qg = np.concatenate([g[rng.permutation(len(g))[:40]],
                         rng.integers(-1, 8, (200, 3)) * 0.5])
    out.append(("grid", g.astype(np.float32), qg.astype(np.float32)))
    # heavy duplication: 300 points drawn from 12 distinct locations
    base = rng.random((12, 3)).astype(np.float32)
    dup = base[rng.integers(0, 12, 300)]
    out.append(("dups", dup, np.concatenate([base, rng.random((100, 3)).astype(np.float32)])))
    # all points identical
    same = np.tile(np.array([[0.25, -1.5, 3.0]], np.float32), (50, 1))
    out.append(("same", same, rng.normal(size=(30, 3)).astype(np.float32)))
    # collinear and coplanar sets
    tline = rng.random(200)
    out.append(("line", np.stack([tline, 2 * tline, -tline], 1).astype(np.float32),
                rng.random((100, 3)).astype(np.float32)))
    plane = np.concatenate([rng.random((300, 2)), np.zeros((300, 1))], 1).astype(np.float32)
    out.append(("plane", plane, (rng.random((100, 3)) - [0, 0, 0.5]).astype(np.float32)))
    # tight clusters + far outliers among the queries
    cl = (rng.integers(0, 4, (400, 1)) * 10.0 + rng.normal(scale=0.01, size=(400, 3))).astype(np.float32)
    qo = rng.normal(size=(60, 3))
    qo = 1000.0 * qo / np.linalg.norm(qo, axis=1, keepdims=True)
    out.append(("clusters", cl, np.concatenate([cl[:40], qo]).astype(np.float32)))
    # single point and two points
    out.append(("one", np.array([[1.0, 2.0, 3.0]], np.float32), rng.normal(size=(20, 3)).astype(np.float32)))
    out.append(("two", np.array([[0, 0, 0], [1, 1, 1]], np.float32),
                np.array([[0.5, 0.5, 0.5], [2, 2, 2], [-1, 0, 0]], np.float32)))
    # queries exactly on split-like coordinates (shared coordinate values)
    sv = rng.integers(0, 5, (500, 3)).astype(np.float32) * 0.125
    out.append(("coarse", sv, (rng.integers(0, 41, (150, 3)) * 0.015625).astype(np.float32)))
    # uniform random
    out.append(("uniform", rng.random((3000, 3)).astype(np.float32), rng.random((500, 3)).astype(np.float32)))
    return out
