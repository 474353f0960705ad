"""The library's computation-budget allocator (prox_budget_s2 /
prox_budget_effective, host arithmetic behind the C ABI) against the page's
worked example and the pinned oracle formula ([blog] computation-budget
section).  Runs without a GPU."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from free_ffn_activation_amd import prox as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_values.json")


def _golden():
    with open(GOLDEN) as fh:
        return json.load(fh)


def test_page_operating_point():
    op = _golden()["budget_operating_point"]
    s2 = P.prox_budget_s2(op["e"], op["s1"], op["alpha"])
    assert abs(s2 - op["s2"]) <= op["printed_precision"]
    assert abs(P.prox_budget_effective(op["s1"], s2, op["alpha"]) - op["e"]) < 1e-6


def test_anchor_needs_full_input_sparsity():
    an = _golden()["budget_s2_anchor_forces_full_input_sparsity"]
    # e = s2 is reached only with s1 = 1
    assert abs(P.prox_budget_s2(an["e"], an["s1"], an["alpha"]) - an["s2"]) < 1e-7
    assert P.prox_budget_s2(an["e"], 0.99, an["alpha"]) > an["s2"]


def test_matches_oracle_formula_on_a_grid():
    rng = np.random.default_rng(5)
    for _ in range(200):
        s1, s2 = (float(np.float32(v)) for v in rng.uniform(0, 1, 2))
        alpha = float(np.float32(rng.uniform(0.05, 1.5)))
        e = P.prox_budget_effective(s1, s2, alpha)
        assert abs(e - oracle.effective_sparsity(s1, s2, alpha)) < 1e-6
        et = float(np.float32(rng.uniform(0, 0.6)))
        ref = oracle.stage2_sparsity_for_target(et, s1, alpha)
        if ref <= 1.0:
            got = P.prox_budget_s2(et, s1, alpha)
            assert abs(got - ref) < 1e-6
            # round trip: the returned s2 reaches the target
            assert abs(P.prox_budget_effective(s1, got, alpha) - et) < 2e-6


@pytest.mark.parametrize("args,status", [
    ((0.9, 0.0, 1.0), P.PROX_ERR_UNSUPPORTED),     # needs s2 = 1.567
    ((0.7, 1.5, 0.3), P.PROX_ERR_INVALID_ARG),     # s1 out of range
    ((-0.1, 0.5, 0.3), P.PROX_ERR_INVALID_ARG),    # e out of range
    ((0.7, 0.5, 0.0), P.PROX_ERR_INVALID_ARG),     # alpha must be > 0
    ((0.7, 0.5, math.nan), P.PROX_ERR_INVALID_ARG),
    ((0.7, 0.5, math.inf), P.PROX_ERR_INVALID_ARG),
])
def test_rejected_arguments(args, status):
    with pytest.raises(P.ProxError) as ei:
        P.prox_budget_s2(*args)
    assert ei.value.status == status
    assert P.prox_last_error() != ""
