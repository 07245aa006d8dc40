"""Writes tests/golden/*.json from the CPU oracle only.

The Vortex pages print no worked numeric example, so no fixture here holds a
value from the pages. ``hand_example.json`` is the hand-chosen case of
tests/test_oracle_pins.py::test_hand_worked_example (its closed forms are
derived there); ``seeded_small.json`` is a small seeded GQA case. Both store
the oracle's outputs so that an accidental change to the oracle's arithmetic
shows up as a diff. Run: python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
from oracle import vx_oracle as O  # noqa: E402


def hand_case():
    k = np.zeros((3, 1, 2, 2)); v = np.zeros((3, 1, 2, 2))
    keys = [(1, 0), (3, 0), (0, 2), (0, 4), (-2, -2)]
    vals = [(9, 9), (9, 9), (1, 0), (-1, 0), (0, 5)]
    for t in range(5):
        k[t // 2, 0, t % 2] = keys[t]
        v[t // 2, 0, t % 2] = vals[t]
    k[2, 0, 1] = (50, 50)
    return {"q": [[1.0, 0.0], [0.0, 1.0]], "k": k.tolist(), "v": v.tolist(),
            "seq_len": 5, "params": dict(page_size=2, num_kv_heads=1, k=1, n_sink=0,
                                         n_local=1, score_scale=1.0, sm_scale=1.0)}


def seeded_case():
    rng = np.random.default_rng(2024)
    P, L, Hq, Hkv, D = 4, 23, 4, 2, 4
    cap = -(-L // P) + 1
    return {"q": rng.standard_normal((Hq, D)).round(4).tolist(),
            "k": rng.standard_normal((cap, Hkv, P, D)).round(4).tolist(),
            "v": rng.standard_normal((cap, Hkv, P, D)).round(4).tolist(),
            "seq_len": L, "params": dict(page_size=P, num_kv_heads=Hkv, k=2, n_sink=1,
                                         n_local=1, score_scale=0.5, sm_scale=0.5)}


def run(case):
    seq = {"q": np.array(case["q"]), "k": np.array(case["k"]), "v": np.array(case["v"]),
           "seq_len": case["seq_len"], "rand_u32": np.zeros(case["params"]["num_kv_heads"], np.uint32)}
    r = O.decode_sequence(seq, **case["params"])
    case["expect"] = {key: np.asarray(r[key]).tolist() for key in ("centroids", "scores", "sel", "out", "lse")}
    return case


if __name__ == "__main__":
    for name, fn in (("hand_example", hand_case), ("seeded_small", seeded_case)):
        with open(os.path.join(HERE, name + ".json"), "w") as f:
            json.dump(run(fn()), f, indent=1)
        print("wrote", name)
