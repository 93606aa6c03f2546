"""The oracle still reproduces its stored snapshot for the tiny block."""
import json
import os

import numpy as np

import oracle
from workload import CONFIGS, make_inputs

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_tiny_snapshot():
    gold = json.load(open(os.path.join(HERE, "tiny_oracle_rows.json")))
    cfg = CONFIGS[gold["config"]]
    inp = make_inputs(cfg, seed=gold["seed"])
    y = oracle.block_forward(inp.x, inp.gamma, inp.beta, inp.w_in, inp.w_out, cfg.H, cfg.hd, cfg.W,
                             eps=cfg.ln_eps, add_residual=bool(cfg.add_residual))
    np.testing.assert_allclose(y[0, gold["rows"]], np.array(gold["y"]), rtol=1e-12, atol=1e-12)
    assert abs(y.sum() - gold["checksum_sum"]) < 1e-8
    assert abs(np.abs(y).sum() - gold["checksum_abs"]) < 1e-8
