"""Regression guard: the oracle still reproduces its committed tiny-case outputs."""
import json
import os

import numpy as np

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_committed_fixture():
    with open(os.path.join(HERE, "golden", "oracle_tiny.json")) as f:
        data = json.load(f)
    for entry in data["cases"]:
        case = entry["case"]
        kw = {k: case[k] for k in ("B", "T", "Hq", "Hkv") if k in case}
        p = synth.prefill_inputs(case["cfg"], flags=case["flags"], train_len=case["train_len"],
                                 **kw)
        o = oracle.polar_prefill(p.as_f32("q"), p.as_f32("k"), p.as_f32("v"), p.beta,
                                 p.null_bias, p.count_vec, p.train_len, p.flags)
        for key in ("dir", "count", "n_eff", "gate", "lse"):
            val = o[key]
            if val.ndim == 4:
                val = val[..., :8]
            assert np.abs(val - np.array(entry[key])).max() < 1e-12, (case, key)
