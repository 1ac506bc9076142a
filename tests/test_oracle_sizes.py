"""Pins the byte accounting against the size figures the pages print."""
import json
import os

import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "model_sizes.json")


def load():
    with open(GOLDEN) as f:
        return json.load(f)


def test_mistral_sizes_scale_with_bits():
    g = load()["mistral_7b"]
    params = g["fp16_GB"] * 1e9 * 8 / 16
    assert oracle.model_bytes(params, 16) / 1e9 == pytest.approx(g["fp16_GB"], abs=5e-3)
    assert oracle.model_bytes(params, 8) / 1e9 == pytest.approx(g["q8_GB"], abs=5e-3)
    assert oracle.model_bytes(params, 4) / 1e9 == pytest.approx(g["q4_GB"], abs=5e-3)


def test_bf16_estimates():
    g = load()
    # the parameter counts are the ones the page names (70B, 400B), not
    # values derived from the sizes they are checked against
    for key in ("llama3_70b_bf16", "llama3_400b_bf16"):
        est = oracle.model_bytes(g[key]["params_B"] * 1e9, 16) / 1e9
        assert est == pytest.approx(g[key]["GB"], rel=g[key]["rel_tol"])
    # and a rule with the wrong bits per weight misses the 70B figure
    assert oracle.model_bytes(70e9, 8) / 1e9 != pytest.approx(141.2, rel=0.01)


def test_codes_are_half_a_byte_and_group_overhead():
    # 4-bit codes: K*N/2 bytes; with one group spanning all of K the per-group
    # metadata is negligible and the set tends to 4 bits per weight.
    K, N = 8192, 4096
    assert oracle.weight_set_bytes(K, N, K) == K * N // 2 + 2 * N + N // 2
    bits = 8 * oracle.weight_set_bytes(4096, 4096, 128) / (4096 * 4096)
    assert bits == pytest.approx(4.15625)
    bits64 = 8 * oracle.weight_set_bytes(4096, 4096, 64) / (4096 * 4096)
    assert bits64 == pytest.approx(4.3125)


def test_falcon_sizes():
    g = load()
    # a 40B model at 4 bits is about 20 GB: the page's 22 GB with overhead fits 24 GB
    f40 = oracle.model_bytes(g["falcon_40b_4bit"]["params_B"] * 1e9, 4) / 1e9
    assert f40 <= g["falcon_40b_4bit"]["GB"] <= g["falcon_40b_4bit"]["fits_GB"]
    # the Falcon-180B-shaped 80-layer stack fits the 141 GB GPU the news page names
    w = synth.FALCON_180B_STACK
    total = w.layers * sum(oracle.weight_set_bytes(s.K, s.N, w.G) for s in w.shapes)
    assert 85e9 < total < g["falcon_180b_int4_fits_h200"]["gpu_GB"] * 1e9
