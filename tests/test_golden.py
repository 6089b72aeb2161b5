"""Stored fixtures: the oracle's smoke-workload answer and the page limits."""

import hashlib
import json
import os

import numpy as np

from workloads import make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_oracle_c1_regression(oracle_mod):
    doc = json.load(open(os.path.join(GOLDEN, "oracle_c1.json")))
    w = make_workload("C1")
    assert hashlib.sha256(w.raw.tobytes()).hexdigest() == doc["input_sha256"], "generator drifted"
    st, idx, val = oracle_mod.topk(w.raw, w.dtype, w.n, w.k, True, True)
    assert st == 0
    assert idx.tolist() == doc["indices"]
    assert val.astype(np.uint16).tolist() == doc["values_bits"]


def test_page_limits_fixture_shapes():
    doc = json.load(open(os.path.join(GOLDEN, "page_limits.json")))
    assert doc["k_max"]["value"] == 4096
    assert set(doc["dtypes"]["value"]) == {"bf16", "f32"}
    ex = doc["usage_example_shape"]["value"]
    w = make_workload("C2")
    assert (w.dtype, w.batch, w.n, w.k) == (ex["dtype"], ex["batch"], ex["vocab"], ex["topk"])
    w3 = make_workload("C3", batch=1)
    sampler = doc["perf_groups"]["value"][1]
    assert (w3.dtype, w3.n, w3.k) == (sampler["dtype"], sampler["vocab"], sampler["topk"])
