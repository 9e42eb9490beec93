"""The oracle against the pages' worked examples, closed forms, invariants,
textbook reductions and dense brute force (see oracle_pins.py)."""
import numpy as np
import pytest

import oracle_pins
from workloads import WORKLOADS


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


# Edge totals of the five workloads from the degree closed form
# (window + globals outside the window + min(R, pool), full global rows).
EXPECTED_NNZ = {
    "small_f32": 38154,
    "batch_bf16": 112144,
    "mlm4096_bf16": 1294208,
    "long16k_bf16": 10387712,
    "sweep8192_f32": 2612256,
}


@pytest.mark.parametrize("name", list(EXPECTED_NNZ))
def test_workload_nnz(orc, name):
    w = WORKLOADS[name]
    rp, _ = orc.graph(w.n, w.radius, w.global_idx, w.num_random, w.num_graphs, w.causal,
                      w.graph_seed)
    assert [int(x) for x in rp[:, -1]] == [EXPECTED_NNZ[name]] * w.num_graphs


@pytest.mark.parametrize("R,causal,nnz", [(0, False, 1567776), (32, False, 1828896),
                                          (128, False, 2612256), (0, True, 787984)])
def test_sweep_nnz(orc, R, causal, nnz):
    w = WORKLOADS["sweep8192_f32"]
    rp, _ = orc.graph(w.n, w.radius, w.global_idx, R, 1, causal, w.graph_seed)
    assert int(rp[0, -1]) == nnz


def test_degree_formula_headline(orc):
    w = WORKLOADS["mlm4096_bf16"]
    oracle_pins.pin_degrees(orc, [(w.n, w.radius, list(w.global_idx), w.num_random, 2)])


def test_thread_count_invariance(orc):
    rng = np.random.default_rng(0)
    n, d = 500, 16
    rp, cols = orc.graph(n, 8, [0, 250], 8, 1, False, 1)
    Q, K, V = (rng.normal(size=(n, d)) for _ in range(3))
    z1 = orc.attn(Q, K, V, rp[0], cols[0], 5, 0.1, threads=1)
    z8 = orc.attn(Q, K, V, rp[0], cols[0], 5, 0.1, threads=7)
    assert np.array_equal(z1, z8)


def test_invalid_arguments(orc):
    from oracle import OracleError
    with pytest.raises(OracleError):
        orc.graph(10, -1, [], 0)
    with pytest.raises(OracleError):
        orc.graph(10, 1, [3, 3], 0)
    with pytest.raises(OracleError):
        orc.graph(10, 1, [10], 0)
