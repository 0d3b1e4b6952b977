"""Oracle against the hand-derived closed-form fixtures under tests/golden/.

Each fixture states the passage it follows and how its values were derived by
hand (transcendentals from Python's math module, not from the oracle).
"""

import json
import math
import os

import numpy as np
import pytest

import oracle


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_qmem_two_turns(golden_dir):
    g = _load(golden_dir, "qmem_two_turns.json")
    t0, t1 = (np.array(t, dtype=np.float64) for t in g["turns"])
    M0 = oracle.qmem_update(t0, g["lambda"], None)
    np.testing.assert_allclose(M0, g["M_after_turn0"], rtol=0, atol=1e-14)
    M1 = oracle.qmem_update(t1, g["lambda"], M0)
    np.testing.assert_allclose(M1, g["M_after_turn1"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("case", range(2))
def test_rule_closed_form(golden_dir, case):
    c = _load(golden_dir, "rule_closed_form.json")["cases"][case]
    rule = oracle.rule_score(np.array(c["K"]), np.array(c["M"]), c["pi"], c["q_s"], c["q_e"])
    np.testing.assert_allclose(rule, c["rule"], rtol=0, atol=1e-14)


def test_topk_ties(golden_dir):
    g = _load(golden_dir, "topk_ties.json")
    for c in g["cases"]:
        keep, idx, n = oracle.topk_select(np.array(g["score"]), tuple(g["f0"]), tuple(g["f1"]), c["C"])
        assert idx.tolist() == c["keep_idx"], c["why"]
        assert n == len(c["keep_idx"])
        assert keep.sum() == n


def test_meank_closed_form(golden_dir):
    g = _load(golden_dir, "meank_closed_form.json")
    index, _ = oracle.meank_build(np.array(g["K"], dtype=np.float64), block=g["block"])
    np.testing.assert_array_equal(index, np.array(g["index"], dtype=np.float64))
    R = oracle.meank_score(np.array(g["Q"], dtype=np.float64), index, g["n_sink"], g["n_recent"])
    np.testing.assert_allclose(R, g["R"], rtol=0, atol=1e-14)


def test_rerope_closed_form(golden_dir):
    g = _load(golden_dir, "rerope_closed_form.json")
    k_src = np.array(g["k_src"], dtype=np.float64)
    v_src = np.array(g["v_src"], dtype=np.float32)
    P = g["pool_pages"] * g["block"]
    k_pool = np.full((1, 1, P, 4), -7.0)
    v_pool = np.full((1, 1, P, 4), -7.0, dtype=np.float32)
    ko, vo = oracle.rerope_scatter(k_src, v_src, np.array(g["src_block"]), np.array(g["page_table"]),
                                   g["pos_base"], g["theta"], k_pool, v_pool, block=g["block"])
    np.testing.assert_allclose(ko[0, 0, 5], g["k_pool_row5"], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(ko[0, 0, 4], np.zeros(4))
    np.testing.assert_array_equal(vo[0, 0, 4], g["v_pool_row4"])
    np.testing.assert_array_equal(vo[0, 0, 5], g["v_pool_row5"])
    # pages 0 and 1 receive nothing and keep their contents
    np.testing.assert_array_equal(ko[0, 0, :4], -7.0)
    np.testing.assert_array_equal(vo[0, 0, :4], -7.0)


def test_rope_closed_form_d2():
    # D = 2: omega_0 = 1, position pi/2 ... use an integer position p and compare with math.cos/sin.
    for p in (0, 1, 7, 123456):
        y = oracle.rope_rotate(np.array([[1.0, 0.0]]), np.array([p]), 1e6)
        np.testing.assert_allclose(y[0], [math.cos(p), math.sin(p)], rtol=0, atol=1e-12)
        y = oracle.rope_rotate(np.array([[0.0, 1.0]]), np.array([p]), 1e6)
        np.testing.assert_allclose(y[0], [-math.sin(p), math.cos(p)], rtol=0, atol=1e-12)
