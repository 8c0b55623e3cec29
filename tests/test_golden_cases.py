"""Hand-worked verify cases from tests/golden/hand_cases.json against the oracle (CPU)."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(HERE, "golden", "hand_cases.json")) as f:
    CASES = json.load(f)


@pytest.mark.parametrize("case", CASES["chain"], ids=[c["name"] for c in CASES["chain"]])
def test_chain_hand_case(case):
    lg = np.array([case["logits"]], np.float32)
    r = oracle.verify_chain(lg, "f32", np.array([case["q"]], np.float32),
                            np.array([case["x"]], np.int32), np.array([case["coins"]], np.float32),
                            np.array([case["T"]], np.float32))
    assert r["accept_len"][0] == case["accept_len"]
    assert list(r["out_tokens"][0]) == case["out_tokens"]
    np.testing.assert_allclose(r["probs"][0], case["probs"], rtol=1e-6, atol=1e-12)
    if case.get("edge"):
        assert r["margin"][0] == 0.0
    else:
        assert r["margin"][0] > 1e-3


@pytest.mark.parametrize("case", CASES["greedy"], ids=[c["name"] for c in CASES["greedy"]])
def test_greedy_hand_case(case):
    acc, out = oracle.verify_greedy(np.array([case["logits"]], np.float32), "f32",
                                    np.array([case["x"]], np.int32))
    assert acc[0] == case["accept_len"]
    assert list(out[0]) == case["out_tokens"]


@pytest.mark.parametrize("case", CASES["tree"], ids=[c["name"] for c in CASES["tree"]])
def test_tree_hand_case(case):
    sampling = case["mode"] == "sampling"
    r = oracle.verify_tree(np.array([case["logits"]], np.float32), "f32",
                           np.array([case["tokens"]], np.int32), np.array([case["parents"]], np.int32),
                           np.array([case["coins"]], np.float32) if sampling else None,
                           np.array([case["T"]], np.float32) if sampling else None, case["D"],
                           oracle.TREE_SAMPLING if sampling else oracle.TREE_GREEDY)
    assert r["accept_len"][0] == case["accept_len"]
    assert list(r["out_tokens"][0]) == case["out_tokens"]
    assert list(r["accepted_nodes"][0]) == case["accepted_nodes"]
    if sampling:
        np.testing.assert_allclose(r["probs"][0], case["probs"], rtol=1e-6, atol=1e-12)
        assert r["margin"][0] > 1e-3
