"""Writes oracle_tiny.json: oracle outputs on a tiny seeded workload (calls only oracle/).

The fixture guards the oracle against unnoticed drift: a change to its arithmetic must
come with a regenerated fixture and a commit message naming the passage that justifies it.
Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402

DIMS = 8

CASES = [
    dict(cfg="c1", T=24, flags=3, train_len=2048),
    dict(cfg="c2", B=1, T=10, Hq=8, Hkv=2, flags=3, train_len=4),  # temperature, floor on
]


def build():
    out = []
    for case in CASES:
        kw = {k: case[k] for k in ("B", "T", "Hq", "Hkv") if k in case}
        p = synth.prefill_inputs(case["cfg"], flags=case["flags"], train_len=case["train_len"],
                                 **kw)
        o = oracle.polar_prefill(p.as_f32("q"), p.as_f32("k"), p.as_f32("v"), p.beta,
                                 p.null_bias, p.count_vec, p.train_len, p.flags)
        # vectors are stored for their first DIMS components to keep the fixture small
        o = {k: (v[..., :DIMS] if v.ndim == 4 else v) for k, v in o.items()}
        out.append(dict(case=case, **{k: np.round(v, 14).tolist() for k, v in o.items()}))
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json")
    with open(path, "w") as f:
        json.dump(dict(source="tests/golden/make_golden.py (oracle/ only)", cases=build()), f)
    print("wrote", path)
