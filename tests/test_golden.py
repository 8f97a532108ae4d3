"""Fixtures under tests/golden/: figures the pages print, and a regression
record of the oracle on the tiny workload."""

import json
import os

import numpy as np

import oracle
from workloads import (HEAD_DIM_V, PAGE_SIZE, algorithmic_bytes, make_workload_inputs)
from workloads.roofline import kv_read_bytes

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_page_cache_read_figures():
    doc = _load("page_figures.json")
    for case in doc["cache_reads"]:
        got = kv_read_bytes(case["seq_len"], case["elems_per_token"], case["bytes_per_elem"], case["reads"])
        assert got == case["expected_bytes"], case["what"]
        assert got == int(case["page_value"].split()[0]) * 2**20
    mha, mla = (c["expected_bytes"] for c in doc["cache_reads"])
    assert mha // mla == doc["mla_over_mha_read_ratio"]["value"]


def test_algorithmic_bytes_reads_each_row_once():
    """The benchmark's byte count charges one read of each cache row (the
    MLA page's decode figure), never a second pass for the values."""
    n, h_q = 32768, 16
    rows = h_q
    other = 1152 * rows + 1024 * rows + 4 * rows + 4 * (n // 64) + 4
    assert algorithmic_bytes([n], 1, h_q) - other == kv_read_bytes(n, 576)
    # with the page's 512-wide latent row the cache term is the page's 32 MB
    assert kv_read_bytes(n, 512) == _load("page_figures.json")["cache_reads"][1]["expected_bytes"]


def test_problem_constants():
    c = _load("page_figures.json")["problem_constants"]
    assert PAGE_SIZE == c["page_size"] and HEAD_DIM_V == c["latent_dim"]


def test_tiny_oracle_regression():
    import importlib.util
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(GOLDEN, "make_golden.py"))
    mg = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mg)
    doc = _load("tiny_oracle.json")
    inp = make_workload_inputs("tiny")
    assert mg.input_digest(inp) == doc["input_sha256"], "input generator changed"
    out, lse = oracle.mla_decode_ref(inp.q_bits, inp.kv_bits, inp.block_table, inp.seqlens,
                                     inp.scale, inp.causal)
    np.testing.assert_allclose(lse, np.array(doc["lse"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(out[..., :8], np.array(doc["out_first8"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(out.sum(axis=-1), np.array(doc["out_row_sums"]), rtol=0, atol=1e-10)
